"""Full-size parity of the named workloads, in the launch configuration the
benchmark times (the same calls, the same shapes and layouts, and the
[B,D,T]-contiguous variants of the dense, packed, large and seq_idx ones).

* Every output buffer starts filled with a sentinel (a BF16 NaN pattern no
  finite input produces), so an element no launch wrote is caught anywhere
  in the tensor, not only where the oracle is consulted.
* The dense and packed workloads are compared with the oracle on every
  channel: channels are independent, so the oracle runs over channel slices
  in a thread pool (ctypes and numpy release the GIL).
* The large workload is compared on a channel sample holding at least one
  channel of every 256-channel group (the backward's channel groups; the
  forward's are 512 wide), at an offset that changes from group to group,
  plus both sides of the group edges at the ends and the middle.
* The decode workload is compared in full, every one of its 64 steps.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from depthwise_causal_conv1d_02_amd import _abi, ops, synth
from parity import SENTINEL, check_bf16, check_exact_bf16, check_f32_rel

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def sample_channels(D, group=256):
    cand = {0, 1, 7, 8, 255, 256, 511, 512, 513, D // 2 - 1, D // 2, D - 513, D - 512, D - 257,
            D - 256, D - 9, D - 8, D - 1}
    for gi in range((D + group - 1) // group):
        cand.add(gi * group + (gi * 37 + 3) % group)
    return sorted(c for c in cand if 0 <= c < D)


def test_sample_reaches_every_channel_group():
    for D in (4096, 5120, 8192):
        sel = sample_channels(D)
        for group in (256, 512):
            assert {c // group for c in sel} == set(range(D // group)), (D, group)


def f(t):
    return None if t is None else t.detach().cpu().double().numpy()


def sub(t, sel):
    if t is None:
        return None
    return t[:, sel] if t.dim() == 3 else t[sel]


def n_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 4
    return max(1, min(16, n))


def sentinel_like(t):
    """An uninitialised-looking output with t's strides, every element the sentinel."""
    out = torch.empty_like(t)
    assert out.stride() == t.stride()
    out.view(torch.int16).fill_(np.int16(SENTINEL))
    return out


def no_sentinel(name, t):
    left = int((t.view(torch.int16) == np.int16(SENTINEL)).sum().item())
    assert left == 0, "%s: %d elements never written" % (name, left)


def run_workload(idx, tc=False):
    """tc: the workload's activations in [B,D,T] time-contiguous storage (the
    benchmark's *_tc workloads) instead of its own layout."""
    w = synth.workload(idx)
    if tc:
        w = dict(w, x=w["x"].contiguous(),
                 dy=None if w["dy"] is None else w["dy"].contiguous())
    return run_inputs(w, "workload %d" % idx)


def run_inputs(w, label, options=0):
    """One forward (and backward) call on a workload's inputs, as the
    benchmark makes it, into sentinel-filled outputs."""
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}
    x = g["x"]
    assert x.stride() == w["x"].stride()
    B, D, T = x.shape
    R = B if w["cu_seqlens"] is None else w["cu_seqlens"].numel() - 1
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    seq = g.get("seq_idx")
    y = sentinel_like(x)
    fin = None
    if w["return_final_states"]:
        fin = torch.empty(R, D, w["weight"].shape[1] - 1, dtype=x.dtype, device=DEV)
        fin.view(torch.int16).fill_(np.int16(SENTINEL))
    print("%s: forward" % label, flush=True)
    ops.fwd(x, g["weight"], g["bias"], g["cu_seqlens"], g["initial_states"], g["activation"],
            final_states_out=fin, y=y, err_flag=flag, seq_idx=seq, options=options)
    out = {"y": y, "fin": fin}
    if g["dy"] is not None:
        dx = sentinel_like(x)
        dinit = None
        if g["initial_states"] is not None:
            dinit = sentinel_like(g["initial_states"])
        print("%s: backward" % label, flush=True)
        _, dw, db, _ = ops.bwd(x, g["weight"], g["dy"], g["bias"], g["cu_seqlens"],
                               g["initial_states"], None, g["activation"], g["deterministic"],
                               False, dx=dx, err_flag=flag, seq_idx=seq, dinit=dinit,
                               options=options)
        out.update(dx=dx, dw=dw, db=db, dinit=dinit)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    for name in ("y", "fin", "dx", "dinit"):
        if out.get(name) is not None:
            no_sentinel(name, out[name])
    return w, g, out


def check_sample(w, out):
    D = w["x"].shape[1]
    sel = sample_channels(D)
    print("sampled channels (%d)" % len(sel), sel, flush=True)
    cu = None if w["cu_seqlens"] is None else w["cu_seqlens"].numpy()
    xs, ws, bs = f(sub(w["x"], sel)), f(sub(w["weight"], sel)), f(sub(w["bias"], sel))
    init = f(sub(w["initial_states"], sel))
    oy, ofin = oracle.fwd(xs, ws, bs, cu, init, w["activation"])
    check_bf16("y", out["y"][:, sel], oy)
    if out["fin"] is not None:
        check_exact_bf16("final_states", out["fin"][:, sel], ofin)
    if w["dy"] is not None:
        odx, odw, odb, odinit = oracle.bwd(xs, ws, f(sub(w["dy"], sel)), bs, cu, init, None,
                                           w["activation"])
        check_bf16("dx", out["dx"][:, sel], odx)
        check_f32_rel("dweight", out["dw"][sel], odw)
        if odb is not None:
            check_f32_rel("dbias", out["db"][sel], odb)
        if odinit is not None:
            check_bf16("dinitial_states", out["dinit"][:, sel], odinit)


def check_full(w, out, step):
    """Every channel against the oracle, `step` channels per worker task."""
    D = w["x"].shape[1]
    cu = None if w["cu_seqlens"] is None else w["cu_seqlens"].numpy()
    host = {k: (None if v is None else v.cpu()) for k, v in out.items()}
    has_bwd = w["dy"] is not None
    odw = np.zeros((D, w["weight"].shape[1])) if has_bwd else None
    odb = np.zeros(D) if has_bwd and w["bias"] is not None else None

    def job(c0):
        sel = slice(c0, min(D, c0 + step))
        xs, ws, bs = f(sub(w["x"], sel)), f(sub(w["weight"], sel)), f(sub(w["bias"], sel))
        init = f(sub(w["initial_states"], sel))
        oy, ofin = oracle.fwd(xs, ws, bs, cu, init, w["activation"])
        check_bf16("y[:, %d:%d]" % (sel.start, sel.stop), host["y"][:, sel], oy)
        if host["fin"] is not None:
            check_exact_bf16("final_states", host["fin"][:, sel], ofin)
        if not has_bwd:
            return c0, None, None
        gdx, gw, gb, gi = oracle.bwd(xs, ws, f(sub(w["dy"], sel)), bs, cu, init, None,
                                     w["activation"])
        check_bf16("dx[:, %d:%d]" % (sel.start, sel.stop), host["dx"][:, sel], gdx)
        if gi is not None:
            check_bf16("dinitial_states", host["dinit"][:, sel], gi)
        return c0, gw, gb

    with ThreadPoolExecutor(n_workers()) as ex:
        for c0, gw, gb in ex.map(job, range(0, D, step)):
            if gw is not None:
                odw[c0:c0 + gw.shape[0]] = gw
            if gb is not None:
                odb[c0:c0 + gb.shape[0]] = gb
    if has_bwd:
        check_f32_rel("dweight", host["dw"], odw)
        if odb is not None:
            check_f32_rel("dbias", host["db"], odb)


def test_workload_1_tiny_dense_fwd_full():
    w, g, out = run_workload(1)
    oy, ofin = oracle.fwd(f(w["x"]), f(w["weight"]), f(w["bias"]), None, None, "silu")
    check_bf16("y", out["y"], oy)
    check_exact_bf16("final_states", out["fin"], ofin)
    assert out["fin"].shape == (1, 64, 3)


def test_workload_2_dense_fwd_bwd_update_full():
    w, g, out = run_workload(2)
    check_full(w, out, 256)
    # decode one token from the returned final states, as a decode loop would
    state = out["fin"].clone()
    xt = g["x"][:, :, -1].contiguous()
    yt = ops.update(xt, state, g["weight"], g["bias"], "silu")
    torch.cuda.synchronize()
    oyt, ost = oracle.update(f(w["x"][:, :, -1]), f(out["fin"]), f(w["weight"]), f(w["bias"]),
                             "silu")
    check_bf16("update y", yt, oyt)
    check_exact_bf16("update state", state, ost)


def test_workload_3_packed_fwd_bwd_full():
    w, g, out = run_workload(3)
    assert w["cu_seqlens"].numel() == 17 and int(w["cu_seqlens"][-1]) == 33280
    check_full(w, out, 64)


def test_workload_4_decode_64_steps_full():
    w = synth.workload(4)
    state = w["conv_state"].to(DEV)
    wt, bt = w["weight"].to(DEV), w["bias"].to(DEV)
    xs = w["x_steps"].to(DEV)
    ys = torch.empty_like(xs)
    ys.view(torch.int16).fill_(np.int16(SENTINEL))
    for s in range(xs.shape[0]):
        ops.update(xs[s], state, wt, bt, "silu", y=ys[s])
    torch.cuda.synchronize()
    no_sentinel("y (64 steps)", ys)
    host = ys.cpu()
    ost = f(w["conv_state"])
    wf, bf = f(w["weight"]), f(w["bias"])
    for s in range(xs.shape[0]):
        oy, ost = oracle.update(f(w["x_steps"][s]), ost, wf, bf, "silu")
        check_bf16("update y step %d" % s, host[s], oy)
    check_exact_bf16("conv_state after 64 steps", state, ost)


def test_workload_5_large_deterministic():
    w, g, out = run_workload(5)
    check_sample(w, out)
    # deterministic dweight: bit-identical over repeated runs
    ref = out["dw"].view(torch.int32).clone()
    dx = torch.empty_like(g["x"])
    for _ in range(10):
        _, dw, _, _ = ops.bwd(g["x"], g["weight"], g["dy"], None, None, None, None, "silu",
                              True, False, dx=dx)
        torch.cuda.synchronize()
        assert torch.equal(dw.view(torch.int32), ref)
    assert torch.equal(dx.view(torch.int16), out["dx"].view(torch.int16))


def check_seq_sample(w, out):
    D = w["x"].shape[1]
    sel = sample_channels(D)
    seq = w["seq_idx"].numpy()
    xs, ws, bs = f(sub(w["x"], sel)), f(sub(w["weight"], sel)), f(sub(w["bias"], sel))
    oy = oracle.fwd_seq(xs, ws, seq, bs, "silu")
    check_bf16("y", out["y"][:, sel], oy)
    odx, odw, odb = oracle.bwd_seq(xs, ws, f(sub(w["dy"], sel)), seq, bs, "silu")
    check_bf16("dx", out["dx"][:, sel], odx)
    check_f32_rel("dweight", out["dw"][sel], odw)
    check_f32_rel("dbias", out["db"][sel], odb)


def test_workload_6_seq_idx_fwd_bwd():
    w, g, out = run_workload(6)
    check_seq_sample(w, out)


@pytest.mark.parametrize("name", ["dense_w2", "dense_w3", "dense_noact", "dense_f32bias"])
def test_variant_workload_full(name):
    """The benchmark's variants of the dense workload (filter widths 2 and 3,
    no activation, FP32 weight with FP32 bias and the deterministic dweight
    and dbias), every channel against the oracle."""
    w = synth.variant(name)
    opts = ops._options(w["fp32_weight_bias"], w["deterministic_dbias"])
    w, g, out = run_inputs(w, name, opts)
    check_full(w, out, 256)
    if w["deterministic"]:
        dx = torch.empty_like(g["x"])
        for _ in range(3):
            _, dw, db, _ = ops.bwd(g["x"], g["weight"], g["dy"], g["bias"], None,
                                   g["initial_states"], None, g["activation"], True, False,
                                   dx=dx, options=opts)
            torch.cuda.synchronize()
            assert torch.equal(dw.view(torch.int32), out["dw"].view(torch.int32))
            assert torch.equal(db.view(torch.int32), out["db"].view(torch.int32))


def test_variant_decode_tokens_full():
    """The benchmark's multi-token decode: 64 tokens as 8 calls of 8 on the
    decode shape, against the oracle's calls in the same order."""
    w = synth.variant("decode_tokens")
    state = w["conv_state"].to(DEV)
    wt, bt = w["weight"].to(DEV), w["bias"].to(DEV)
    xs = w["x_calls"].to(DEV)
    assert xs.stride() == w["x_calls"].stride() and xs.stride(2) == 1
    ys = torch.empty_like(xs)
    ys.view(torch.int16).fill_(np.int16(SENTINEL))
    for c in range(xs.shape[0]):
        ops.update(xs[c], state, wt, bt, "silu", y=ys[c])
    torch.cuda.synchronize()
    no_sentinel("y (8 calls)", ys)
    host = ys.cpu()
    ost = f(w["conv_state"])
    wf, bf = f(w["weight"]), f(w["bias"])
    for c in range(xs.shape[0]):
        oy, ost = oracle.update_tokens(f(w["x_calls"][c]), ost, wf, bf, "silu")
        check_bf16("update y call %d" % c, host[c], oy)
    check_exact_bf16("conv_state after 8 calls", state, ost)


@pytest.mark.parametrize("idx", [2, 3, 5, 6])
def test_workload_time_contiguous(idx):
    """The dense, packed, large and seq_idx workloads with [B,D,T]-contiguous
    activations, which run on the time-lane kernels."""
    w, g, out = run_workload(idx, tc=True)
    assert w["x"].stride(2) == 1
    if idx == 6:
        check_seq_sample(w, out)
    elif idx == 5:
        check_sample(w, out)
    else:
        check_full(w, out, 256 if idx == 2 else 64)


def test_more_than_2_pow_31_elements():
    """64-bit indexing: x [1, 8, 2^28 + 37] (2.1 G elements, 4.3 GB) in
    channel-last storage, forward with final states, checked on sampled
    positions (each from its own 4-token window through the oracle) across
    the 2^31-element boundary and at both ends; then backward dx on samples
    with dy zero except at the sampled tokens."""
    T = (1 << 28) + 37
    D = 8
    gen = torch.Generator(device=DEV).manual_seed(31)
    x = torch.randn(1, T, D, generator=gen, device=DEV).to(torch.bfloat16).transpose(1, 2)
    w = (torch.rand(D, 4, generator=gen, device=DEV) - 0.5).to(torch.bfloat16)
    b = (torch.randn(D, generator=gen, device=DEV) * 0.1).to(torch.bfloat16)
    y, fin = ops.fwd(x, w, b, None, None, "silu", return_final_states=True)
    torch.cuda.synchronize()
    wf, bf = f(w), f(b)
    edge = (1 << 31) // D          # first token whose element index passes 2^31
    for t in (0, 1, 2, 3, edge - 2, edge - 1, edge, edge + 1, T // 2, T - 2, T - 1):
        lo = max(0, t - 3)
        win = f(x[:, :, lo:t + 1])
        oy, _ = oracle.fwd(win, wf, bf, None, None, "silu")
        check_bf16("y[%d]" % t, y[:, :, t:t + 1], oy[:, :, -1:])
    check_exact_bf16("final_states", fin, f(x[:, :, T - 3:]))
    # backward: dy nonzero only at a few tokens, so dx there has a local closed
    # window in the oracle
    dy = torch.zeros_like(x)
    picks = (edge, T - 1)
    for t in picks:
        dy[:, :, t] = 1.0
    dx, dwt, dbt, _ = ops.bwd(x, w, dy, b, None, None, None, "silu")
    torch.cuda.synchronize()
    for t in picks:
        lo, hi = t - 6, min(T, t + 4)
        xs, dys = f(x[:, :, lo:hi]), f(dy[:, :, lo:hi])
        # the window's leading tokens act as its past: use them as initial state
        odx, odw, odb, _ = oracle.bwd(xs[:, :, 3:], wf, dys[:, :, 3:], bf, None, xs[:, :, :3],
                                      None, "silu")
        check_bf16("dx near %d" % t, dx[:, :, lo + 3:hi], odx)
    # dW/dB: only the picked tokens contribute
    ow, ob = np.zeros((D, 4)), np.zeros(D)
    for t in picks:
        xs = f(x[:, :, t - 3:t + 1])
        _, odw, odb, _ = oracle.bwd(xs[:, :, 3:], wf, f(dy[:, :, t:t + 1]), bf, None,
                                    xs[:, :, :3], None, "silu")
        ow += odw
        ob += odb
    check_f32_rel("dweight", dwt, ow)
    check_f32_rel("dbias", dbt, ob)


def _window_y(x, wf, bf, init, s, t):
    """Oracle y at token t of a sequence that starts at s (init: its initial
    state [1,D,W-1] or None), from the shortest window that determines it."""
    lo = max(s, t - 3)
    win = f(x[:, :, lo:t + 1])
    oy, _ = oracle.fwd(win, wf, bf, None, init if lo == s else None, "silu")
    return oy[:, :, -1:]


def test_more_than_2_pow_31_elements_time_lanes():
    """64-bit indexing on the time-lane kernels: [1, 10, 286,331,149] in
    [B,D,T]-contiguous storage whose rows start on 16-byte boundaries (2.9 G
    elements; rows 8 and 9 start past element 2^31, row 7 crosses it half
    way along).
    Dense rows with initial states and final-state gradients (deterministic
    backward), packed rows with a sequence starting one token before the
    crossing and a last sequence of two tokens, and seq_idx rows split at the
    same place.  Outputs are checked on sampled tokens, each from its own
    window through the oracle; the backward takes dy zero except at a few
    tokens, so that dx, dW, dB and the state gradients have closed windows."""
    D, T = 10, 286_331_149                      # T % 8 = 5, T % 2048 = 269: ragged tails
    Tp = T + 3                                  # multiple of 8: aligned row starts
    edge = (1 << 31) - 7 * Tp                   # row 7's token at element 2^31
    assert 1000 < edge < T - 1000 and 8 * Tp > (1 << 31)
    check_time_lanes_sampled(D, T, Tp, edge)


def check_time_lanes_sampled(D, T, Tp, edge):
    """The body of the test above for any [1, D, T] shape with row stride Tp
    and a token `edge` (a sequence starts at edge - 1) well inside the row."""
    gen = torch.Generator(device=DEV).manual_seed(2031)

    def tc_buffer(fill=None):
        st = torch.empty(1, D, Tp, dtype=torch.bfloat16, device=DEV)
        if fill is None:
            st.view(torch.int16).fill_(np.int16(SENTINEL))
        else:
            st.normal_(generator=gen)
        return st[:, :, :T]

    x = tc_buffer(fill="randn")
    w = (torch.rand(D, 4, generator=gen, device=DEV) - 0.5).to(torch.bfloat16)
    b = (torch.randn(D, generator=gen, device=DEV) * 0.1).to(torch.bfloat16)
    wf, bf = f(w), f(b)
    samples = sorted({0, 1, 2, 3, 7, 8, 511, 512, 1023, 1024, 1025, edge - 2, edge - 1, edge,
                      edge + 1, edge + 4, T // 2, T - 38, T - 37, T - 36, T - 6, T - 2, T - 1})

    # dense rows, initial and final states
    init = torch.randn(1, D, 3, generator=gen, device=DEV).to(torch.bfloat16)
    y = tc_buffer()
    y, fin = ops.fwd(x, w, b, None, init, "silu", return_final_states=True, y=y)
    torch.cuda.synchronize()
    for t in samples:
        check_bf16("dense y[%d]" % t, y[:, :, t:t + 1], _window_y(x, wf, bf, f(init), 0, t))
    check_exact_bf16("dense final_states", fin, f(x[:, :, T - 3:]))
    del y
    dy = tc_buffer(fill="randn")
    picks = (0, 1, edge, T - 1)
    keep = {t: dy[:, :, t].clone() for t in picks}
    dy.zero_()
    for t, v in keep.items():
        dy[:, :, t] = v
    dfin = torch.randn(1, D, 3, generator=gen, device=DEV).to(torch.bfloat16)
    dx = tc_buffer()
    dx, dwt, dbt, dinit = ops.bwd(x, w, dy, b, None, init, dfin, "silu", deterministic=True,
                                  dx=dx, options=_abi.CCV_OPT_DETERMINISTIC_DBIAS)
    torch.cuda.synchronize()
    # the row's head (picks 0, 1 and the initial state) and tail (pick T-1 and
    # dfinal) through the oracle with the row's own states
    hx, hdy = f(x[:, :, :8]), f(dy[:, :, :8])
    # a window's final state sits at its end: zero dfinal for the head window
    odx, odw_h, odb_h, odinit = oracle.bwd(hx, wf, hdy, bf, None, f(init), None, "silu")
    check_bf16("dense dx head", dx[:, :, :5], odx[:, :, :5])
    check_bf16("dense dinit", dinit, odinit)
    tx, tdy = f(x[:, :, T - 11:]), f(dy[:, :, T - 8:])
    odx, odw_t, odb_t, _ = oracle.bwd(tx[:, :, 3:], wf, tdy, bf, None, tx[:, :, :3], f(dfin),
                                      "silu")
    check_bf16("dense dx tail", dx[:, :, T - 8:], odx)
    ex, edy = f(x[:, :, edge - 6:edge + 4]), f(dy[:, :, edge - 3:edge + 4])
    odx, odw_e, odb_e, _ = oracle.bwd(ex[:, :, 3:], wf, edy, bf, None, ex[:, :, :3], None, "silu")
    check_bf16("dense dx at the 2^31 crossing", dx[:, :, edge - 3:edge + 4], odx)
    for t in (T // 2, edge - 700, edge + 700):
        check_bf16("dense dx[%d] (dy zero nearby)" % t, dx[:, :, t:t + 1], np.zeros((1, D, 1)))
    check_f32_rel("dense dweight", dwt, odw_h + odw_t + odw_e)
    check_f32_rel("dense dbias", dbt, odb_h + odb_t + odb_e)
    del dx

    # packed rows: a sequence starts one token before row 7's crossing, the
    # last one holds two tokens
    s1, s2 = edge - 1, T - 2
    cu = torch.tensor([0, s1, s2, T], dtype=torch.int32, device=DEV)
    pinit = torch.randn(3, D, 3, generator=gen, device=DEV).to(torch.bfloat16)
    starts = (0, s1, s2)
    ops.reset_flag(DEV)
    y = tc_buffer()
    y, fin = ops.fwd(x, w, b, cu, pinit, "silu", return_final_states=True, y=y)
    torch.cuda.synchronize()
    for t in samples + [s1 + 1, s1 + 2, s1 + 3]:
        s = max(v for v in starts if v <= t)
        i = starts.index(s)
        check_bf16("packed y[%d]" % t, y[:, :, t:t + 1],
                   _window_y(x, wf, bf, f(pinit[i:i + 1]), s, t))
    check_exact_bf16("packed final_states[0]", fin[0:1], f(x[:, :, s1 - 3:s1]))
    check_exact_bf16("packed final_states[1]", fin[1:2], f(x[:, :, s2 - 3:s2]))
    check_exact_bf16("packed final_states[2]", fin[2:3],
                     np.concatenate([f(pinit[2:3])[:, :, 2:], f(x[:, :, s2:])], axis=2))
    del y
    picks = (s1, s1 + 2, T - 1)
    dy.zero_()
    for t in picks:
        dy[:, :, t] = 1.0
    dx = tc_buffer()
    dx, dwt, dbt, dinit = ops.bwd(x, w, dy, b, cu, pinit, None, "silu", dx=dx)
    torch.cuda.synchronize()
    ops.check_flag(DEV)
    check_bf16("packed dx before the start", dx[:, :, s1 - 3:s1], np.zeros((1, D, 3)))
    odx1, odw1, odb1, odi1 = oracle.bwd(f(x[:, :, s1:s1 + 6]), wf, f(dy[:, :, s1:s1 + 6]), bf,
                                        None, f(pinit[1:2]), None, "silu")
    check_bf16("packed dx after the start", dx[:, :, s1:s1 + 6], odx1)
    check_bf16("packed dinit[1]", dinit[1:2], odi1)
    odx2, odw2, odb2, odi2 = oracle.bwd(f(x[:, :, s2:]), wf, f(dy[:, :, s2:]), bf, None,
                                        f(pinit[2:3]), None, "silu")
    check_bf16("packed dx, last sequence", dx[:, :, s2:], odx2)
    check_bf16("packed dinit[2]", dinit[2:3], odi2)
    check_bf16("packed dinit[0]", dinit[0:1], np.zeros((1, D, 3)))
    check_f32_rel("packed dweight", dwt, odw1 + odw2)
    check_f32_rel("packed dbias", dbt, odb1 + odb2)
    del dx, dy

    # seq_idx rows: ids 4 before s1, 9 from s1 on, 2 on the last two tokens
    seq = torch.full((1, T), 4, dtype=torch.int32, device=DEV)
    seq[:, s1:] = 9
    seq[:, s2:] = 2
    y = tc_buffer()
    ops.fwd(x, w, b, None, None, "silu", y=y, seq_idx=seq)
    torch.cuda.synchronize()
    for t in samples + [s1 + 1, s1 + 2, s1 + 3]:
        s = max(v for v in starts if v <= t)
        check_bf16("seq_idx y[%d]" % t, y[:, :, t:t + 1], _window_y(x, wf, bf, None, s, t))
