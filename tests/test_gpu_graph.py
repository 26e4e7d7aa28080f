"""The C-ABI calls captured in a HIP graph (torch.cuda.CUDAGraph) replay to
the eager results: several replays, with eager work and synchronisation in
between, each checked against the eager outputs."""
import pytest
import torch

from depthwise_causal_conv1d_02_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_graph_replay_matches_eager():
    inp = synth.random_inputs(800, 2, 1024, 200, layout="cl", bias=False, init=True)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    x, w, init, dy = g["x"], g["weight"], g["initial_states"], g["dy"]
    y = torch.empty_like(x)
    fin = torch.empty(2, 1024, 3, dtype=x.dtype, device=DEV)
    dx = torch.empty_like(x)
    dw = torch.zeros(1024, 4, dtype=torch.float32, device=DEV)
    dinit = torch.empty_like(init)
    ws = torch.empty(1 << 24, dtype=torch.uint8, device=DEV)
    xt = x[:, :, -1].contiguous()
    yt = torch.empty_like(xt)

    def step():
        dw.zero_()
        ops.fwd(x, w, None, None, init, "silu", final_states_out=fin, y=y)
        ops.bwd(x, w, dy, None, None, init, None, "silu", True, False, dx=dx, dweight=dw,
                dinit=dinit, workspace=ws)
        ops.update(xt, fin, w, None, "silu", y=yt)

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in dict(y=y, fin=fin, dx=dx, dw=dw, dinit=dinit, yt=yt).items()}

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    outs = dict(y=y, fin=fin, dx=dx, dw=dw, dinit=dinit, yt=yt)
    for rep in range(4):
        for v in outs.values():
            v.fill_(7)                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(_bits(v), _bits(ref[k])), (rep, k)


# (8, 512): the per-lane update kernel; (192, 4096): the coalesced one
# (786,432 (row, channel) pairs).
@pytest.mark.parametrize("B,D", [(8, 512), (192, 4096)])
def test_graph_decode_loop(B, D):
    print("graph decode loop", B, D, flush=True)
    gen = torch.Generator().manual_seed(801)
    state0 = synth.state_tensor(gen, B, D).to(DEV)
    w = synth.weight_tensor(gen, D).to(DEV)
    b = synth.bias_tensor(gen, D).to(DEV)
    xs = torch.randn(16, B, D, generator=gen).to(torch.bfloat16).to(DEV)
    ys = torch.empty_like(xs)
    state = state0.clone()
    for s in range(16):
        ops.update(xs[s], state, w, b, "silu", y=ys[s])
    torch.cuda.synchronize()
    ref_y, ref_state = ys.clone(), state.clone()

    state.copy_(state0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(16):
            ops.update(xs[s], state, w, b, "silu", y=ys[s])
    for rep in range(3):
        state.copy_(state0)
        ys.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(ys), _bits(ref_y)), rep
        assert torch.equal(_bits(state), _bits(ref_state)), rep


def _padded_tc(t):
    """A [B,D,T] device copy whose rows start on 16-byte boundaries."""
    B, D, T = t.shape
    st = torch.zeros(B, D, (T + 7) // 8 * 8 + 8, dtype=t.dtype, device=DEV)
    st[:, :, :T].copy_(t.to(DEV))
    return st[:, :, :T]


def _case(kind):
    """(step, outputs) of one call sequence of the named kind."""
    if kind == "decode_tokens":
        gen = torch.Generator().manual_seed(810)
        state = synth.state_tensor(gen, 64, 1024).to(DEV)
        w = synth.weight_tensor(gen, 1024).to(DEV)
        b = synth.bias_tensor(gen, 1024).to(DEV)
        x = synth.activation_tensor(gen, 64, 1024, 8, "cl").to(DEV)
        st = state.clone()
        y = torch.empty_like(x)

        def step():
            st.copy_(state)
            ops.update(x, st, w, b, "silu", y=y)
        return step, dict(y=y, st=st)
    cu = None
    if kind in ("packed_cl", "packed_tc"):
        cu = synth.cu_from_lengths([5, 1, 40, 3, 700, 2, 90])
        B, D, T = 1, 256, int(cu[-1])
    else:
        B, D, T = 2, 256, 2047 if kind == "odd_tc" else 1536
    layout = "cl" if kind == "packed_cl" else "tc"
    inp = synth.random_inputs(820, B, D, T, layout=layout, bias=False,
                              init=kind != "seq_tc", cu_seqlens=cu)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    x, dy = g["x"], g["dy"]
    if kind in ("packed_tc", "seq_tc"):
        x, dy = _padded_tc(inp["x"]), _padded_tc(inp["dy"])
    seq = None
    if kind == "seq_tc":
        seq = synth.seq_idx_tensor(torch.Generator().manual_seed(821), B, T, "runs").to(DEV)
    w, init = g["weight"], g["initial_states"]
    y, dx = torch.empty_like(x), torch.empty_like(x)
    R = B if cu is None else cu.numel() - 1
    fin = torch.empty(R, D, 3, dtype=x.dtype, device=DEV) if init is not None else None
    dinit = torch.empty_like(init) if init is not None else None
    dw = torch.zeros(D, 4, dtype=torch.float32, device=DEV)
    ws = torch.empty(1 << 24, dtype=torch.uint8, device=DEV)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    gcu = None if cu is None else cu.to(DEV)

    def step():
        dw.zero_()
        ops.fwd(x, w, None, gcu, init, "silu", final_states_out=fin, y=y, err_flag=flag,
                seq_idx=seq)
        ops.bwd(x, w, dy, None, gcu, init, None, "silu", True, False, dx=dx, dweight=dw,
                dinit=dinit, workspace=ws, err_flag=flag, seq_idx=seq)
    outs = dict(y=y, dx=dx, dw=dw, flag=flag)
    if fin is not None:
        outs.update(fin=fin, dinit=dinit)
    return step, outs


@pytest.mark.parametrize("kind", ["packed_cl", "packed_tc", "seq_tc", "odd_tc",
                                  "decode_tokens"])
def test_graph_replay_other_paths(kind):
    """Packed rows (channel-last, and time lanes with their repair launches),
    seq_idx time lanes, rows with 2-byte-aligned starts, and the multi-token
    update, each captured and replayed four times against its eager bits
    (deterministic dweight)."""
    step, outs = _case(kind)
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    assert "flag" not in ref or int(ref["flag"].item()) == 0
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for k, v in outs.items():
            if k != "flag":
                v.fill_(7)                  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(_bits(v), _bits(ref[k])), (kind, rep, k)
