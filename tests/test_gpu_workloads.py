"""Full-size parity of the five named workloads, in the launch configuration
the benchmark times (the same calls, the same shapes and layouts).

Channels are independent, so the oracle runs on a sample of channels (all
rows and tokens of each); the sample covers both ends of every channel
group boundary that the kernels use (groups of 512 channels).  The decode
workload is compared in full, step by step.
"""
import numpy as np
import pytest
import torch

import oracle
from depthwise_causal_conv1d_02_amd import ops, synth
from parity import check_bf16, check_exact_bf16, check_f32_rel

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def sample_channels(D):
    cand = [0, 1, 7, 8, 511, 512, 513, D // 2, D - 513, D - 512, D - 9, D - 8, D - 1]
    return sorted({c for c in cand if 0 <= c < D})


def f(t):
    return None if t is None else t.detach().cpu().double().numpy()


def sub(t, sel):
    if t is None:
        return None
    return t[:, sel] if t.dim() == 3 else t[sel]


def run_workload(idx):
    w = synth.workload(idx)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}
    x = g["x"]
    assert x.stride() == w["x"].stride()
    B, D, T = x.shape
    R = B if w["cu_seqlens"] is None else w["cu_seqlens"].numel() - 1
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    seq = g.get("seq_idx")
    y, fin = ops.fwd(x, g["weight"], g["bias"], g["cu_seqlens"], g["initial_states"],
                     g["activation"], return_final_states=w["return_final_states"], err_flag=flag,
                     seq_idx=seq)
    out = {"y": y, "fin": fin}
    if g["dy"] is not None:
        dx, dw, db, dinit = ops.bwd(x, g["weight"], g["dy"], g["bias"], g["cu_seqlens"],
                                    g["initial_states"], None, g["activation"], g["deterministic"],
                                    False, err_flag=flag, seq_idx=seq)
        out.update(dx=dx, dw=dw, db=db, dinit=dinit)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    return w, g, out


def check_sample(w, out):
    D = w["x"].shape[1]
    sel = sample_channels(D)
    print("sampled channels", sel, flush=True)
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
    return oy


def test_workload_1_tiny_dense_fwd_full():
    w, g, out = run_workload(1)
    oy, ofin = oracle.fwd(f(w["x"]), f(w["weight"]), f(w["bias"]), None, None, "silu")
    check_bf16("y", out["y"], oy)
    check_exact_bf16("final_states", out["fin"], ofin)
    assert out["fin"].shape == (1, 64, 3)


def test_workload_2_dense_fwd_bwd_update():
    w, g, out = run_workload(2)
    check_sample(w, out)
    # decode one token from the returned final states, as the benchmark does
    state = out["fin"].clone()
    xt = g["x"][:, :, -1].contiguous()
    yt = ops.update(xt, state, g["weight"], g["bias"], "silu")
    torch.cuda.synchronize()
    oyt, ost = oracle.update(f(w["x"][:, :, -1]), f(out["fin"]), f(w["weight"]), f(w["bias"]),
                             "silu")
    check_bf16("update y", yt, oyt)
    check_exact_bf16("update state", state, ost)


def test_workload_3_packed_fwd_bwd():
    w, g, out = run_workload(3)
    assert w["cu_seqlens"].numel() == 17 and int(w["cu_seqlens"][-1]) == 33280
    check_sample(w, out)


def test_workload_4_decode_64_steps_full():
    w = synth.workload(4)
    state = w["conv_state"].to(DEV)
    wt, bt = w["weight"].to(DEV), w["bias"].to(DEV)
    xs = w["x_steps"].to(DEV)
    ost = f(w["conv_state"])
    wf, bf = f(w["weight"]), f(w["bias"])
    y = torch.empty_like(xs[0])
    for s in range(xs.shape[0]):
        ops.update(xs[s], state, wt, bt, "silu", y=y)
        oy, ost = oracle.update(f(w["x_steps"][s]), ost, wf, bf, "silu")
        if s % 16 == 0 or s == xs.shape[0] - 1:
            torch.cuda.synchronize()
            check_bf16("update y step %d" % s, y, oy)
    torch.cuda.synchronize()
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


def test_workload_6_seq_idx_fwd_bwd():
    w, g, out = run_workload(6)
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
