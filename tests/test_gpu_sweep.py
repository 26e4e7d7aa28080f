"""GPU parity over a seeded sweep of the call surface: each case draws a row
mode (dense, packed, seq_idx), a layout (channel-last or [B,D,T]
contiguous), the filter width, channel count and length (lengths cluster at
the lane, tile and chunk edges of every kernel), the filter dtype, bias,
states, the final-state gradient, the activation and the determinism route,
then checks forward and backward against the fp64 oracle with every output
inside a sentinel-filled guard band.  A second sweep does the same for the
single- and multi-token update.  The draws are fixed by the case index, and
each case prints itself before it runs (512 forward+backward cases, 128 updates)."""
import random

import pytest
import torch

import oracle
from depthwise_causal_conv1d_02_amd import _abi, ops, synth
from parity import check_bf16, check_exact_bf16, check_f32_rel, f64, guarded_act
from test_gpu_parity import check_bwd, check_fwd, dev, inputs, padded_tc, run_bwd, run_fwd

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
BF16, F32 = torch.bfloat16, torch.float32
OPT_F32 = _abi.CCV_OPT_F32_FILTER_BIAS
OPT_DETDB = _abi.CCV_OPT_DETERMINISTIC_DBIAS

# lengths at and around the edges the kernels split at: lanes of 8 tokens,
# 16- and 32-step batches and chunks, 512-token tiles, 1024/2048-token chunks
EDGE_T = [1, 2, 3, 4, 7, 8, 9, 15, 16, 17, 31, 33, 63, 64, 65, 127, 129, 511, 512, 513,
          1023, 1024, 1025, 2047, 2048, 2049, 2050, 4099]
CHANNELS = [8, 16, 24, 40, 64, 72, 200, 256, 264, 512, 520, 1032, 1536, 2056]
MAX_ELEMS = 2_500_000
N_CASES = 512


def draw_case(i):
    r = random.Random(9100 + i)
    mode = r.choice(["dense", "dense", "packed", "seq"])
    c = {"i": i, "mode": mode, "W": r.choice([2, 3, 4, 4]),
         "layout": r.choice(["cl", "cl", "tc"]), "wdt": r.choice([BF16, BF16, F32]),
         "bias": r.random() < 0.6, "act": r.choice(["silu", "silu", None]),
         "det": r.random() < 0.35}
    c["D"] = r.choice(CHANNELS)
    if mode == "packed":
        n = r.randint(1, 12)
        c["lengths"] = [r.choice([1, 2, 3, r.randint(1, 40), r.randint(1, 700)]) for _ in range(n)]
        c["B"], c["T"] = 1, sum(c["lengths"])
    else:
        c["B"] = r.randint(1, 3)
        c["T"] = r.choice(EDGE_T) if r.random() < 0.7 else r.randint(1, 3000)
    while c["B"] * c["D"] * c["T"] > MAX_ELEMS and c["D"] > 8:
        c["D"] = max(8, c["D"] // 2)
    states = mode != "seq"
    c["init"] = states and r.random() < 0.6
    c["final"] = states and r.random() < 0.7
    c["dfinal"] = states and r.random() < 0.5
    c["padded"] = c["layout"] == "tc" and r.random() < 0.5
    return c


def options_for(c):
    opts = 0
    if c["bias"] and c["wdt"] == F32:
        opts |= OPT_F32
    if c["bias"] and c["det"]:
        opts |= OPT_DETDB
    return opts


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_fwd_bwd(i):
    c = draw_case(i)
    print("sweep case", {k: (str(v) if k == "wdt" else v) for k, v in c.items()}, flush=True)
    B, D, T, W, layout, act = c["B"], c["D"], c["T"], c["W"], c["layout"], c["act"]
    opts = options_for(c)
    cu = synth.cu_from_lengths(c["lengths"]) if c["mode"] == "packed" else None
    inp, g = inputs(9200 + i, B, D, T, layout, c["bias"], c["init"], c["wdt"], c["dfinal"],
                    cu=cu, W=W)
    if c["padded"]:
        g["x"], g["dy"] = padded_tc(inp["x"]), padded_tc(inp["dy"])
    if c["mode"] == "seq":
        seq = synth.seq_idx_tensor(torch.Generator().manual_seed(9300 + i), B, T,
                                   random.Random(9400 + i).choice(["runs", "random", "periodic"]))
        gseq = dev(seq)
        y = guarded_act(B, D, T, layout, DEV)
        ops.fwd(g["x"], g["weight"], g["bias"], None, None, act, y=y.view, seq_idx=gseq,
                options=opts)
        torch.cuda.synchronize()
        oy = oracle.fwd_seq(f64(inp["x"]), f64(inp["weight"]), seq.numpy(), f64(inp["bias"]), act)
        check_bf16("y", y.view, oy)
        assert y.intact(), "write outside y"
        dx = guarded_act(B, D, T, layout, DEV)
        _, dw, db, _ = ops.bwd(g["x"], g["weight"], g["dy"], g["bias"], None, None, None, act,
                               c["det"], False, dx=dx.view, seq_idx=gseq, options=opts)
        torch.cuda.synchronize()
        odx, odw, odb = oracle.bwd_seq(f64(inp["x"]), f64(inp["weight"]), f64(inp["dy"]),
                                       seq.numpy(), f64(inp["bias"]), act)
        check_bf16("dx", dx.view, odx)
        assert dx.intact(), "write outside dx"
        check_f32_rel("dweight", dw, odw)
        if odb is not None:
            check_f32_rel("dbias", db, odb)
        return
    if cu is not None:
        ops.reset_flag(DEV)
    y, fin = run_fwd(g, layout, act, c["final"], cu, options=opts)
    check_fwd(inp, y, fin, act)
    dx, dw, db, dinit = run_bwd(g, layout, act, c["det"], cu, options=opts)
    check_bwd(inp, dx, dw, db, dinit, act)
    if c["det"]:
        _, dw2, db2, _ = run_bwd(g, layout, act, True, cu, options=opts)
        assert torch.equal(dw2.view(torch.int32), dw.view(torch.int32))
        if db is not None:
            assert torch.equal(db2.view(torch.int32), db.view(torch.int32))
    if cu is not None:
        ops.check_flag(DEV)


N_UPDATE = 128


def draw_update(i):
    r = random.Random(9500 + i)
    return {"i": i, "B": r.randint(1, 40), "D": r.choice(CHANNELS), "W": r.choice([2, 3, 4]),
            "L": r.choice([1, 1, 2, 3, 5, 9]), "bias": r.random() < 0.6,
            "wdt": r.choice([BF16, BF16, F32]), "act": r.choice(["silu", None]),
            "layout": r.choice(["cl", "tc"])}


@pytest.mark.parametrize("i", range(N_UPDATE))
def test_sweep_update(i):
    c = draw_update(i)
    print("update sweep case", {k: (str(v) if k == "wdt" else v) for k, v in c.items()},
          flush=True)
    B, D, W, L = c["B"], c["D"], c["W"], c["L"]
    gen = torch.Generator().manual_seed(9600 + i)
    state = synth.state_tensor(gen, B, D, W)
    w = synth.weight_tensor(gen, D, W, dtype=c["wdt"])
    b = synth.bias_tensor(gen, D, c["wdt"]) if c["bias"] else None
    x = synth.activation_tensor(gen, B, D, L, c["layout"])
    opts = OPT_F32 if (c["bias"] and c["wdt"] == F32) else 0
    g_state = dev(state)
    if L == 1:
        xt = x[:, :, 0].contiguous()
        y = ops.update(dev(xt), g_state, dev(w), dev(b), c["act"], options=opts)
        torch.cuda.synchronize()
        oy, ost = oracle.update(f64(xt), f64(state), f64(w), f64(b), c["act"])
    else:
        yg = guarded_act(B, D, L, c["layout"], DEV)
        ops.update(dev(x), g_state, dev(w), dev(b), c["act"], y=yg.view, options=opts)
        torch.cuda.synchronize()
        oy, ost = oracle.update_tokens(f64(x), f64(state), f64(w), f64(b), c["act"])
        assert yg.intact(), "write outside y"
        y = yg.view
    check_bf16("y", y, oy)
    check_exact_bf16("conv_state", g_state, ost)
