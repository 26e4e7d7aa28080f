"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle on the
same seeded inputs, element by element, at sizes that span several tiles and
end in ragged tails; every output sits inside a sentinel-filled guard band
that must come back untouched."""
import numpy as np
import pytest
import torch

import oracle
from depthwise_causal_conv1d_02_amd import _abi, ops, synth
from parity import (SENTINEL, Guarded, check_bf16, check_cast_bf16, check_exact_bf16, check_f32_rel,
                    f64, guarded_act, guarded_flat)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
BF16, F32 = torch.bfloat16, torch.float32
OPT_F32 = _abi.CCV_OPT_F32_FILTER_BIAS
OPT_DETDB = _abi.CCV_OPT_DETERMINISTIC_DBIAS


def dev(t):
    if t is None:
        return None
    d = t.to(DEV)
    assert d.stride() == t.stride()
    return d


def inputs(seed, B, D, T, layout, bias=True, init=False, wdtype=BF16, dfinal=False, cu=None, W=4):
    inp = synth.random_inputs(seed, B, D, T, layout=layout, W=W, bias=bias, init=init,
                              dfinal=dfinal, weight_dtype=wdtype, cu_seqlens=cu)
    return inp, {k: dev(v) for k, v in inp.items()}


def run_fwd(g, layout, act, ret_final, cu=None, options=0):
    B, D, T = g["x"].shape
    R = B if cu is None else cu.numel() - 1
    W = g["weight"].shape[1]
    y = guarded_act(B, D, T, layout, DEV)
    fin = guarded_flat((R, D, W - 1), DEV) if ret_final else None
    ops.fwd(g["x"], g["weight"], g["bias"], g["cu_seqlens"], g["initial_states"], act,
            final_states_out=None if fin is None else fin.view, y=y.view, options=options)
    torch.cuda.synchronize()
    return y, fin


def check_fwd(inp, y, fin, act):
    oy, ofin = oracle.fwd(f64(inp["x"]), f64(inp["weight"]), f64(inp["bias"]),
                          None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy(),
                          f64(inp["initial_states"]), act)
    check_bf16("y", y.view, oy)
    assert y.intact(), "write outside y"
    if fin is not None:
        check_exact_bf16("final_states", fin.view, ofin)
        assert fin.intact(), "write outside final_states"


FWD_CASES = [
    # B, D, T, layout, bias, init, act, weight dtype
    (2, 1536, 300, "cl", True, True, "silu", BF16),
    (2, 1536, 300, "cl", False, False, None, BF16),
    (1, 1024, 77, "cl", False, True, "silu", F32),
    (1, 64, 128, "tc", True, False, "silu", BF16),
    (3, 40, 77, "cl", True, True, "silu", BF16),
    (2, 48, 50, "tc", True, True, None, BF16),
    (1, 512, 1, "cl", True, True, "silu", BF16),
    (2, 520, 2, "cl", True, False, "silu", BF16),
    (1, 8, 4100, "cl", True, True, "silu", BF16),
    (2, 24, 3, "tc", False, True, "silu", F32),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "B%d-D%d-T%d-%s-b%d-i%d-%s-%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "f32" if c[7] == F32 else "bf16"))
def test_fwd_parity(case):
    B, D, T, layout, bias, init, act, wdt = case
    print("fwd case", case, flush=True)
    inp, g = inputs(100 + D + T, B, D, T, layout, bias, init, wdt)
    y, fin = run_fwd(g, layout, act, True)
    check_fwd(inp, y, fin, act)
    # without the final state
    y2, _ = run_fwd(g, layout, act, False)
    assert torch.equal(y2.view, y.view)


BWD_CASES = [
    # B, D, T, layout, bias, init, dfinal, act, weight dtype, deterministic
    (2, 1536, 300, "cl", True, True, True, "silu", BF16, False),
    (2, 1536, 300, "cl", False, True, False, "silu", BF16, True),
    (2, 1024, 133, "cl", False, False, False, None, BF16, False),
    (1, 1024, 77, "cl", False, True, True, "silu", F32, True),
    (1, 64, 128, "tc", True, False, False, "silu", BF16, False),
    (3, 40, 77, "cl", True, True, True, "silu", BF16, False),
    (2, 48, 50, "tc", False, True, True, "silu", BF16, True),
    (1, 512, 1, "cl", True, True, True, "silu", BF16, False),
    (2, 520, 2, "cl", False, True, True, "silu", BF16, True),
    (1, 8, 4100, "cl", True, True, True, "silu", BF16, False),
]


def run_bwd(g, layout, act, det, cu=None, options=0, dweight=None, dbias=None):
    B, D, T = g["x"].shape
    R = B if cu is None else cu.numel() - 1
    dx = guarded_act(B, D, T, layout, DEV)
    dinit = None
    # dinit goes to a guarded buffer through the raw call
    _, dw, db, dinit_t = ops.bwd(g["x"], g["weight"], g["dy"], g["bias"], g["cu_seqlens"],
                                 g["initial_states"], g["dfinal_states"], act, det, False,
                                 dx=dx.view, options=options, dweight=dweight, dbias=dbias)
    torch.cuda.synchronize()
    return dx, dw, db, dinit_t


def check_bwd(inp, dx, dw, db, dinit, act, dw0=None, db0=None):
    """dw0/db0: the starting values the gradients were accumulated into."""
    odx, odw, odb, odinit = oracle.bwd(
        f64(inp["x"]), f64(inp["weight"]), f64(inp["dy"]), f64(inp["bias"]),
        None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy(),
        f64(inp["initial_states"]), f64(inp["dfinal_states"]), act)
    check_bf16("dx", dx.view, odx)
    assert dx.intact(), "write outside dx"
    if dw0 is not None:
        odw = odw + f64(dw0)
    check_f32_rel("dweight", dw, odw)
    if odb is not None:
        if db0 is not None:
            odb = odb + f64(db0)
        check_f32_rel("dbias", db, odb)
    else:
        assert db is None
    if odinit is not None:
        check_bf16("dinitial_states", dinit, odinit)


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B%d-D%d-T%d-%s-b%d-i%d-f%d-%s-%s-det%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], "f32" if c[8] == F32 else "bf16", c[9]))
def test_bwd_parity(case):
    B, D, T, layout, bias, init, dfinal, act, wdt, det = case
    print("bwd case", case, flush=True)
    inp, g = inputs(200 + D + T, B, D, T, layout, bias, init, wdt, dfinal)
    dx, dw, db, dinit = run_bwd(g, layout, act, det)
    check_bwd(inp, dx, dw, db, dinit, act)
    if det:
        dx2, dw2, _, _ = run_bwd(g, layout, act, det)
        assert torch.equal(dw2.view(torch.int32), dw.view(torch.int32))


PACKED = [
    ([1, 2, 3, 100, 17, 400, 5], 512, True),
    ([1, 2, 3, 100, 17, 400, 5], 40, False),
    ([64], 136, True),
    ([1] * 20 + [2] * 5 + [3, 3], 520, True),
    ([700, 1, 350, 2], 1024, False),
]


@pytest.mark.parametrize("lengths,D,init", PACKED)
@pytest.mark.parametrize("det", [False, True])
def test_packed_parity(lengths, D, init, det):
    print("packed case", lengths, D, init, det, flush=True)
    cu = synth.cu_from_lengths(lengths)
    T = int(cu[-1])
    inp, g = inputs(300 + D + T, 1, D, T, "cl", bias=not det, init=init, dfinal=True, cu=cu)
    ops.reset_flag(DEV)
    y, fin = run_fwd(g, "cl", "silu", True, cu)
    check_fwd(inp, y, fin, "silu")
    dx, dw, db, dinit = run_bwd(g, "cl", "silu", det, cu)
    check_bwd(inp, dx, dw, db, dinit, "silu")
    ops.check_flag(DEV)


def test_packed_many_sequences_global_offsets():
    """More offsets than fit in LDS: the separate validation kernel and the
    global-memory search."""
    rng = np.random.default_rng(5)
    lengths = rng.integers(1, 4, size=5000).tolist()
    cu = synth.cu_from_lengths(lengths)
    T = int(cu[-1])
    inp, g = inputs(401, 1, 64, T, "cl", bias=True, init=True, dfinal=True, cu=cu)
    ops.reset_flag(DEV)
    y, fin = run_fwd(g, "cl", "silu", True, cu)
    check_fwd(inp, y, fin, "silu")
    dx, dw, db, dinit = run_bwd(g, "cl", "silu", False, cu)
    check_bwd(inp, dx, dw, db, dinit, "silu")
    ops.check_flag(DEV)


@pytest.mark.parametrize("n_extra", [0, 5000])
def test_malformed_offsets_write_nothing_and_stick(n_extra):
    good = [0] + list(np.cumsum([3] * n_extra + [5, 7])) if n_extra else [0, 5, 12]
    T = good[-1]
    bad = list(good)
    bad[-2], bad[-3] = bad[-3], bad[-2]          # a decrease
    inp, g = inputs(402, 1, 64, T, "cl", bias=True, init=True,
                    cu=torch.tensor(good, dtype=torch.int32))
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    cu_bad = torch.tensor(bad, dtype=torch.int32, device=DEV)
    y = guarded_act(1, 64, T, "cl", DEV)
    fin = guarded_flat((len(bad) - 1, 64, 3), DEV)
    bits = lambda t: t.view(torch.int16)
    before_y, before_f = bits(y.storage).clone(), bits(fin.storage).clone()
    ops.fwd(g["x"], g["weight"], g["bias"], cu_bad, g["initial_states"], "silu",
            final_states_out=fin.view, y=y.view, err_flag=flag)
    torch.cuda.synchronize()
    want = oracle.validate_cu_seqlens(bad, T)
    assert want & 0x4 and int(flag.item()) == want
    assert torch.equal(bits(y.storage), before_y) and torch.equal(bits(fin.storage), before_f)
    # the flag is sticky: valid offsets still write nothing until it is cleared
    cu_good = g["cu_seqlens"]
    ops.fwd(g["x"], g["weight"], g["bias"], cu_good, g["initial_states"], "silu",
            final_states_out=fin.view, y=y.view, err_flag=flag)
    torch.cuda.synchronize()
    assert torch.equal(bits(y.storage), before_y)
    dx = guarded_act(1, 64, T, "cl", DEV)
    before_dx = bits(dx.storage).clone()
    dw = torch.full((64, 4), 0.5, dtype=F32, device=DEV)
    db = torch.full((64,), -1.0, dtype=F32, device=DEV)
    ops.bwd(g["x"], g["weight"], g["x"], g["bias"], cu_bad, g["initial_states"], None, "silu",
            dx=dx.view, err_flag=flag, dweight=dw, dbias=db)
    torch.cuda.synchronize()
    assert torch.equal(bits(dx.storage), before_dx)
    assert bool((dw == 0.5).all()) and bool((db == -1.0).all())
    assert int(flag.item()) == want
    flag.zero_()
    ops.fwd(g["x"], g["weight"], g["bias"], cu_good, g["initial_states"], "silu",
            final_states_out=fin.view, y=y.view, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    check_fwd(inp, y, fin, "silu")


def _flag_predicate(cu, total):
    bits = 0
    if cu[0] != 0:
        bits |= 1
    if cu[-1] != total:
        bits |= 2
    d = np.diff(np.asarray(cu))
    if (d < 0).any():
        bits |= 4
    if (d == 0).any():
        bits |= 8
    return bits


def test_validate_brute_force():
    import itertools
    from depthwise_causal_conv1d_02_amd import _abi
    cases = []
    for N in (1, 2, 3):
        for cu in itertools.product(range(-1, 6), repeat=N + 1):
            for total in range(1, 6):
                cases.append((cu, total))
    flat = torch.tensor([v for cu, _ in cases for v in cu], dtype=torch.int32, device=DEV)
    flags = torch.full((len(cases),), -1, dtype=torch.int32, device=DEV)
    L = _abi.lib()
    stream = torch.cuda.current_stream(DEV).cuda_stream
    off = 0
    base, fbase = flat.data_ptr(), flags.data_ptr()
    for i, (cu, total) in enumerate(cases):
        rc = L.ccv_validate_cu_seqlens(base + 4 * off, len(cu) - 1, total, fbase + 4 * i, stream)
        assert rc == 0
        off += len(cu)
    got = flags.cpu().numpy()
    want = np.array([oracle.validate_cu_seqlens(list(cu), total) for cu, total in cases])
    assert np.array_equal(got, want)
    assert all(want[i] == _flag_predicate(cu, t) for i, (cu, t) in enumerate(cases[:2000]))


UPDATE_CASES = [(4, 512, True, BF16, 4), (3, 40, True, BF16, 4), (2, 1024, False, F32, 4),
                (5, 24, False, BF16, 4), (3, 512, True, BF16, 3), (4, 64, True, BF16, 2),
                (1, 1024, False, F32, 3), (2, 40, True, BF16, 2)]


UPDATE_CASES += [(4, 512, True, F32, 4), (3, 40, True, F32, 3), (2, 64, True, F32, 2)]
UPDATE_CASES += [(5, 1536, True, BF16, 4), (7, 512, False, BF16, 4), (3, 1024, True, F32, 2),
                 (1, 2048, True, BF16, 3), (9, 512, False, F32, 3), (2, 512, True, BF16, 2)]
# Channel counts that are multiples of 512 with at least 786,432 (row,
# channel) pairs take the coalesced (LDS-staged) kernel: several waves per
# row group, odd batches (a half-empty last row group), a single row, the
# size threshold itself, every width and filter kind.
UPDATE_CASES += [(385, 2048, True, BF16, 4), (97, 8192, False, BF16, 4), (193, 4096, True, F32, 2),
                 (1, 786432, True, BF16, 3), (257, 3072, False, F32, 3), (768, 1024, True, BF16, 2)]


@pytest.mark.parametrize("B,D,bias,wdt,W", UPDATE_CASES)
def test_update_parity(B, D, bias, wdt, W):
    print("update case", B, D, bias, wdt, W, flush=True)
    gen = torch.Generator().manual_seed(500 + D)
    state = synth.state_tensor(gen, B, D, W)
    w = synth.weight_tensor(gen, D, W, dtype=wdt)
    b = synth.bias_tensor(gen, D, wdt) if bias else None
    opts = OPT_F32 if (bias and wdt == F32) else 0
    xs = [synth.activation_tensor(gen, B, D, 1, "tc")[:, :, 0].contiguous() for _ in range(6)]
    g_state = dev(state)
    st = f64(state)
    for x in xs:
        y = guarded_flat((B, D), DEV)
        ops.update(dev(x), g_state, dev(w), dev(b), "silu", y=y.view, options=opts)
        torch.cuda.synchronize()
        oy, st = oracle.update(f64(x), st, f64(w), f64(b), "silu")
        check_bf16("update y", y.view, oy)
        assert y.intact()
        check_exact_bf16("conv_state", g_state, st)


@pytest.mark.parametrize("B,D", [(3, 512), (513, 1536)])
def test_update_no_activation(B, D):
    print("update case act=none", B, D, flush=True)
    gen = torch.Generator().manual_seed(900 + D)
    state = synth.state_tensor(gen, B, D, 4)
    w = synth.weight_tensor(gen, D, 4, dtype=BF16)
    b = synth.bias_tensor(gen, D, BF16)
    g_state = dev(state)
    st = f64(state)
    for _ in range(3):
        x = synth.activation_tensor(gen, B, D, 1, "tc")[:, :, 0].contiguous()
        y = ops.update(dev(x), g_state, dev(w), dev(b), None)
        torch.cuda.synchronize()
        oy, st = oracle.update(f64(x), st, f64(w), f64(b), None)
        check_bf16("update y", y, oy)
        check_exact_bf16("conv_state", g_state, st)


def test_update_strided_state():
    """A state that is a slice of a wider buffer (generic lanes)."""
    gen = torch.Generator().manual_seed(77)
    big = synth.state_tensor(gen, 3, 64, W=6)         # [3,64,5]
    g_big = dev(big)
    g_state = g_big[:, :, 1:4]                          # [3,64,3], stride (320,5,1)
    w = synth.weight_tensor(gen, 64)
    x = synth.activation_tensor(gen, 3, 64, 1, "tc")[:, :, 0].contiguous()
    y = ops.update(dev(x), g_state, dev(w), None, None)
    torch.cuda.synchronize()
    oy, st = oracle.update(f64(x), f64(big[:, :, 1:4]), f64(w), None, None)
    check_bf16("y", y, oy)
    check_exact_bf16("state", g_state, st)
    check_exact_bf16("untouched", g_big[:, :, 0], f64(big[:, :, 0]))
    check_exact_bf16("untouched", g_big[:, :, 4], f64(big[:, :, 4]))


def test_update_staged_row_strided_views():
    """The coalesced update (D % 512 == 0, above its size threshold) on
    x, y and state that are row slices of wider buffers: row strides larger
    than the row, and nothing outside the views written."""
    gen = torch.Generator().manual_seed(78)
    B, D, DW = 193, 4096, 4608
    big_state = synth.state_tensor(gen, B, DW, 4)              # [B,4608,3]
    w = synth.weight_tensor(gen, D)
    b = synth.bias_tensor(gen, D, BF16)
    g_big = dev(big_state)
    g_state = g_big[:, :D, :]                                   # stride (13824, 3, 1)
    st = f64(big_state[:, :D, :])
    for step in range(3):
        print("staged update on row-strided views, token", step, flush=True)
        xbig = synth.activation_tensor(gen, B, DW, 1, "tc")[:, :, 0].contiguous()
        g_xbig = dev(xbig)
        x = g_xbig[:, :D]                                       # stride (4608, 1)
        ybig = guarded_flat((B, DW), DEV)
        y = ybig.view[:, :D]
        ops.update(x, g_state, dev(w), dev(b), "silu", y=y)
        torch.cuda.synchronize()
        oy, st = oracle.update(f64(xbig[:, :D]), st, f64(w), f64(b), "silu")
        check_bf16("update y", y, oy)
        check_exact_bf16("conv_state", g_state, st)
        check_exact_bf16("state outside the view", g_big[:, D:, :], f64(big_state[:, D:, :]))
        # y's columns past D keep the sentinel
        outside = ybig.view[:, D:].contiguous().view(torch.int16)
        assert bool((outside == SENTINEL).all())
        assert ybig.intact()


def test_autograd_wrapper():
    inp, g = inputs(600, 2, 512, 64, "cl", bias=True, init=True, dfinal=True)
    x = g["x"].detach().requires_grad_(True)
    w = g["weight"].detach().requires_grad_(True)
    b = g["bias"].detach().requires_grad_(True)
    init = g["initial_states"].detach().requires_grad_(True)
    y, fin = ops.causal_conv1d(x, w, b, initial_states=init, return_final_states=True,
                               activation="silu")
    (y.float() * g["dy"].float()).sum().backward(retain_graph=True)
    odx, odw, odb, _ = oracle.bwd(f64(inp["x"]), f64(inp["weight"]), f64(inp["dy"]),
                                  f64(inp["bias"]), None, f64(inp["initial_states"]), None,
                                  "silu")
    check_cast_bf16("dweight", w.grad, odw)  # cast to the BF16 parameter
    check_cast_bf16("dbias", b.grad, odb)
    oy, ofin = oracle.fwd(f64(inp["x"]), f64(inp["weight"]), f64(inp["bias"]), None,
                          f64(inp["initial_states"]), "silu")
    check_bf16("y", y, oy)
    check_exact_bf16("final", fin, ofin)
    assert x.grad.stride() == x.stride()
    check_bf16("dx", x.grad, odx)


def test_deterministic_flag_policy():
    inp, g = inputs(700, 1, 512, 40, "cl", bias=True)
    with pytest.raises(RuntimeError):
        ops.bwd(g["x"], g["weight"], g["dy"], g["bias"], deterministic=True)
    with pytest.warns(UserWarning):
        dx, dw, db, _ = ops.bwd(g["x"], g["weight"], g["dy"], g["bias"], deterministic=True,
                                warn_only=True)
    torch.cuda.synchronize()
    odx, odw, odb, _ = oracle.bwd(f64(inp["x"]), f64(inp["weight"]), f64(inp["dy"]),
                                  f64(inp["bias"]), None, None, None, "silu")
    check_f32_rel("dweight", dw, odw)
    check_f32_rel("dbias", db, odb)


def test_fp32_weight_rounding_is_single_rne():
    """y = x * w3 in FP32, rounded once to BF16 (no activation, one tap)."""
    gen = torch.Generator().manual_seed(9)
    x = synth.activation_tensor(gen, 1, 512, 256, "cl")
    w = torch.zeros(512, 4, dtype=F32)
    w[:, 3] = torch.rand(512, generator=gen) + 0.1
    y, _ = ops.fwd(dev(x), dev(w), None, None, None, None)
    torch.cuda.synchronize()
    want = (x.float() * w[:, 3][None, :, None]).to(BF16)
    assert torch.equal(y.cpu(), want)


WIDTH_CASES = [
    # W, B, D, T, layout, bias, init, dfinal, weight dtype, deterministic, packed lengths
    (2, 2, 1024, 150, "cl", True, True, True, BF16, False, None),
    (3, 2, 1024, 150, "cl", False, True, True, BF16, True, None),
    (3, 1, 520, 77, "cl", True, False, False, BF16, False, None),
    (2, 2, 40, 33, "tc", False, True, True, F32, False, None),
    (3, 1, 512, None, "cl", True, True, True, BF16, False, [1, 2, 3, 60, 1, 100]),
    (2, 1, 136, None, "cl", False, True, True, F32, True, [2, 1, 40, 1]),
]


@pytest.mark.parametrize("case", WIDTH_CASES, ids=lambda c: "W%d-B%d-D%d-%s-%s" % (
    c[0], c[1], c[2], c[4], "packed" if c[10] else "dense"))
def test_other_widths(case):
    W, B, D, T, layout, bias, init, dfinal, wdt, det, lengths = case
    print("width case", case, flush=True)
    cu = None
    if lengths is not None:
        cu = synth.cu_from_lengths(lengths)
        T = int(cu[-1])
    inp, g = inputs(900 + W + D, B, D, T, layout, bias, init, wdt, dfinal, cu, W=W)
    ops.reset_flag(DEV)
    y, fin = run_fwd(g, layout, "silu", True, cu)
    check_fwd(inp, y, fin, "silu")
    dx, dw, db, dinit = run_bwd(g, layout, "silu", det, cu)
    check_bwd(inp, dx, dw, db, dinit, "silu")
    ops.check_flag(DEV)


# ---- opt-ins beyond the pages' route -------------------------------------------

F32_BIAS_CASES = [
    # W, B, D, T, layout, init, dfinal, deterministic, packed lengths, misaligned bias
    (4, 2, 1536, 300, "cl", True, True, False, None, False),
    (4, 3, 40, 77, "cl", True, True, True, None, False),
    (4, 2, 1024, 64, "cl", False, False, False, None, True),
    (3, 2, 48, 50, "tc", True, False, False, None, False),
    (2, 1, 512, None, "cl", True, True, True, [1, 2, 3, 60, 1, 100], False),
]


@pytest.mark.parametrize("case", F32_BIAS_CASES, ids=lambda c: "W%d-B%d-D%d-%s-det%d-%s%s" % (
    c[0], c[1], c[2], c[4], c[7], "packed" if c[8] else "dense", "-misaligned" if c[9] else ""))
def test_fp32_weight_with_bias(case):
    """An FP32 filter with an FP32 bias (declined by default) under the
    opt-in: fwd and bwd against the oracle, on 8-, 4- and 1-channel lanes."""
    W, B, D, T, layout, init, dfinal, det, lengths, misaligned = case
    print("fp32 filter+bias case", case, flush=True)
    cu = None
    if lengths is not None:
        cu = synth.cu_from_lengths(lengths)
        T = int(cu[-1])
    inp, g = inputs(1100 + W + D, B, D, T, layout, True, init, F32, dfinal, cu, W=W)
    assert g["bias"].dtype == F32
    if misaligned:
        # a bias view 4 bytes into a buffer: not 16-byte aligned
        holder = torch.zeros(D + 1, dtype=F32, device=DEV)
        holder[1:].copy_(g["bias"])
        g["bias"] = holder[1:]
    with pytest.raises(NotImplementedError):
        ops.fwd(g["x"], g["weight"], g["bias"], g["cu_seqlens"], g["initial_states"], "silu")
    ops.reset_flag(DEV)
    y, fin = run_fwd(g, layout, "silu", True, cu, options=OPT_F32)
    check_fwd(inp, y, fin, "silu")
    opts = OPT_F32 | (OPT_DETDB if det else 0)
    dx, dw, db, dinit = run_bwd(g, layout, "silu", det, cu, options=opts)
    assert db.dtype == F32
    check_bwd(inp, dx, dw, db, dinit, "silu")
    if det:
        _, dw2, db2, _ = run_bwd(g, layout, "silu", det, cu, options=opts)
        assert torch.equal(dw2.view(torch.int32), dw.view(torch.int32))
        assert torch.equal(db2.view(torch.int32), db.view(torch.int32))
    ops.check_flag(DEV)


DET_DBIAS_CASES = [
    # W, B, D, T, layout, packed lengths
    (4, 2, 1536, 300, "cl", None),
    (4, 1, 520, 2100, "cl", None),
    (3, 3, 40, 77, "cl", None),
    (4, 2, 48, 50, "tc", None),
    (4, 1, 512, None, "cl", [1, 2, 3, 100, 17, 400, 5]),
    # the reduction's paths: 625 partials per element on 16-byte lanes, and
    # (D * (W+1) not a multiple of 4) single-element lanes with 282 partials
    # and with a few partials of packed rows
    (4, 1, 64, 40000, "cl", None),
    (4, 2, 37, 9000, "cl", None),
    (2, 1, 41, None, "cl", [5, 100, 2, 33]),
]


@pytest.mark.parametrize("case", DET_DBIAS_CASES, ids=lambda c: "W%d-B%d-D%d-%s-%s" % (
    c[0], c[1], c[2], c[4], "packed" if c[5] else "dense"))
def test_deterministic_dbias(case):
    """Deterministic dweight and dbias with a BF16 bias under the opt-in:
    accumulated into non-zero gradients, equal to start + the oracle's, and
    bit-identical over repeated runs."""
    W, B, D, T, layout, lengths = case
    print("deterministic dbias case", case, flush=True)
    cu = None
    if lengths is not None:
        cu = synth.cu_from_lengths(lengths)
        T = int(cu[-1])
    inp, g = inputs(1200 + W + D, B, D, T, layout, True, True, BF16, True, cu, W=W)
    gen = torch.Generator().manual_seed(1201)
    dw0 = torch.randn(D, W, generator=gen)
    db0 = torch.randn(D, generator=gen)
    ops.reset_flag(DEV)
    runs = []
    for _ in range(3):
        dw, db = dev(dw0.clone()), dev(db0.clone())
        dx, dw, db, dinit = run_bwd(g, layout, "silu", True, cu, options=OPT_DETDB,
                                    dweight=dw, dbias=db)
        runs.append((dw.view(torch.int32).clone(), db.view(torch.int32).clone()))
    check_bwd(inp, dx, dw, db, dinit, "silu", dw0=dw0, db0=db0)
    for rw, rb in runs[1:]:
        assert torch.equal(rw, runs[0][0]) and torch.equal(rb, runs[0][1])
    ops.check_flag(DEV)


def _grad_run(g, bias):
    """One autograd forward + backward with no per-call determinism flag;
    returns (dx, dweight, dbias) in the parameters' dtype."""
    x = g["x"].detach().requires_grad_(True)
    w = g["weight"].detach().requires_grad_(True)
    b = g["bias"].detach().requires_grad_(True) if bias else None
    y = ops.causal_conv1d(x, w, b, activation="silu")
    y.backward(g["dy"])
    return x.grad, w.grad, None if b is None else b.grad


def test_torch_deterministic_algorithms_switch():
    """cuDNN FE "Causal Conv1d", the determinism paragraph: the backward
    follows torch.use_deterministic_algorithms.  Enabled, bias-free calls take
    the fixed-order route (bit-identical to an explicit deterministic call,
    run to run); calls with a bias raise RuntimeError, or warn and use
    atomics under warn_only; disabled, every call uses atomics silently."""
    inp, g = inputs(1700, 2, 512, 200, "cl", bias=False)
    inpb, gb = inputs(1701, 2, 512, 200, "cl", bias=True)
    was, was_warn = (torch.are_deterministic_algorithms_enabled(),
                     torch.is_deterministic_algorithms_warn_only_enabled())
    try:
        torch.use_deterministic_algorithms(True)
        runs = [_grad_run(g, False) for _ in range(3)]
        _, dw_det, _, _ = ops.bwd(g["x"], g["weight"], g["dy"], None, deterministic=True)
        torch.cuda.synchronize()
        ref = dw_det.to(torch.bfloat16).view(torch.int16)
        for dx, dw, _ in runs:
            assert torch.equal(dw.view(torch.int16), ref)
            assert torch.equal(dx.view(torch.int16), runs[0][0].view(torch.int16))
        odx, odw, _, _ = oracle.bwd(f64(inp["x"]), f64(inp["weight"]), f64(inp["dy"]), None,
                                    None, None, None, "silu")
        check_bf16("dx", runs[0][0], odx)
        check_cast_bf16("dweight", runs[0][1], odw)

        with pytest.raises(RuntimeError):
            _grad_run(gb, True)

        torch.use_deterministic_algorithms(True, warn_only=True)
        with pytest.warns(UserWarning, match="atomics"):
            dx, dw, db = _grad_run(gb, True)
        odx, odw, odb, _ = oracle.bwd(f64(inpb["x"]), f64(inpb["weight"]), f64(inpb["dy"]),
                                      f64(inpb["bias"]), None, None, None, "silu")
        check_bf16("dx", dx, odx)
        check_cast_bf16("dweight", dw, odw)
        check_cast_bf16("dbias", db, odb)

        torch.use_deterministic_algorithms(False)
        import warnings
        with warnings.catch_warnings():
            warnings.simplefilter("error")
            dx, dw, db = _grad_run(gb, True)
        check_cast_bf16("dweight", dw, odw)
        check_cast_bf16("dbias", db, odb)
    finally:
        torch.use_deterministic_algorithms(was, warn_only=was_warn)


def test_deterministic_dbias_autograd():
    """The autograd surface: deterministic=True with a bias fails by default
    and runs the fixed-order reduction under deterministic_dbias."""
    inp, g = inputs(1300, 2, 512, 96, "cl", bias=True)
    x = g["x"].detach().requires_grad_(True)
    w = g["weight"].detach().requires_grad_(True)
    b = g["bias"].detach().requires_grad_(True)
    y = ops.causal_conv1d(x, w, b, activation="silu", deterministic=True)
    with pytest.raises(RuntimeError):
        (y.float() * g["dy"].float()).sum().backward()
    grads = []
    for _ in range(2):
        x.grad = w.grad = b.grad = None
        y = ops.causal_conv1d(x, w, b, activation="silu", deterministic=True,
                              deterministic_dbias=True)
        y.backward(g["dy"])
        grads.append((w.grad.clone(), b.grad.clone()))
    assert torch.equal(grads[0][0], grads[1][0]) and torch.equal(grads[0][1], grads[1][1])
    _, odw, odb, _ = oracle.bwd(f64(inp["x"]), f64(inp["weight"]), f64(inp["dy"]),
                                f64(inp["bias"]), None, None, None, "silu")
    check_cast_bf16("dweight", w.grad, odw)
    check_cast_bf16("dbias", b.grad, odb)


# ---- seq_idx rows (per-token sequence ids) ------------------------------------

SEQ_CASES = [
    # W, B, D, T, layout, bias, act, id kind, weight dtype, deterministic
    (4, 2, 1536, 300, "cl", True, "silu", "runs", BF16, False),
    (4, 2, 1024, 257, "cl", False, "silu", "random", BF16, True),
    (4, 3, 40, 77, "cl", True, None, "periodic", BF16, False),
    (4, 2, 48, 50, "tc", True, "silu", "random", BF16, False),
    (4, 1, 512, 4100, "cl", True, "silu", "runs", BF16, False),
    (3, 2, 520, 130, "cl", True, "silu", "random", BF16, False),
    (2, 2, 1024, 99, "cl", False, "silu", "runs", F32, True),
    (4, 2, 512, 64, "cl", False, "silu", "constant", F32, False),
    # time lanes, a block per four channels of one chunk: channel counts that
    # leave waves without a row, several 2048-token chunks with ragged tails
    (4, 2, 5, 4100, "tc", True, "silu", "random", BF16, True),
    (3, 3, 7, 2049, "tc", False, None, "runs", F32, False),
    (2, 1, 1, 600, "tc", True, "silu", "periodic", BF16, True),
    (4, 2, 66, 1030, "tc", True, "silu", "runs", BF16, False),
    (4, 1, 3, 513, "tc", False, "silu", "constant", BF16, True),
    (4, 2, 6, 2048, "tc", False, None, "periodic", F32, True),
]


@pytest.mark.parametrize("case", SEQ_CASES, ids=lambda c: "W%d-B%d-D%d-T%d-%s-%s-%s%s" % (
    c[0], c[1], c[2], c[3], c[4], c[7], "f32" if c[8] == F32 else "bf16",
    "-det" if c[9] else ""))
def test_seq_idx_parity(case):
    W, B, D, T, layout, bias, act, kind, wdt, det = case
    print("seq_idx case", case, flush=True)
    inp, g = inputs(1400 + W + D + T, B, D, T, layout, bias, False, wdt, W=W)
    gen = torch.Generator().manual_seed(1401 + T)
    seq = synth.seq_idx_tensor(gen, B, T, kind)
    gseq = dev(seq)
    y = guarded_act(B, D, T, layout, DEV)
    ops.fwd(g["x"], g["weight"], g["bias"], None, None, act, y=y.view, seq_idx=gseq)
    torch.cuda.synchronize()
    oy = oracle.fwd_seq(f64(inp["x"]), f64(inp["weight"]), seq.numpy(), f64(inp["bias"]), act)
    check_bf16("y", y.view, oy)
    assert y.intact(), "write outside y"
    dx = guarded_act(B, D, T, layout, DEV)
    opts = OPT_DETDB if (bias and det) else 0
    _, dw, db, _ = ops.bwd(g["x"], g["weight"], g["dy"], g["bias"], None, None, None, act, det,
                           False, dx=dx.view, seq_idx=gseq, options=opts)
    torch.cuda.synchronize()
    odx, odw, odb = oracle.bwd_seq(f64(inp["x"]), f64(inp["weight"]), f64(inp["dy"]),
                                   seq.numpy(), f64(inp["bias"]), act)
    check_bf16("dx", dx.view, odx)
    assert dx.intact(), "write outside dx"
    check_f32_rel("dweight", dw, odw)
    if odb is not None:
        check_f32_rel("dbias", db, odb)
    if det:
        _, dw2, db2, _ = ops.bwd(g["x"], g["weight"], g["dy"], g["bias"], None, None, None, act,
                                 det, False, seq_idx=gseq, options=opts)
        torch.cuda.synchronize()
        assert torch.equal(dw2.view(torch.int32), dw.view(torch.int32))
        if bias:
            assert torch.equal(db2.view(torch.int32), db.view(torch.int32))


def test_seq_idx_strided_ids_and_runs_equal_packed():
    """Ids read through a strided view ([T,B] storage transposed); ids that
    form contiguous runs give exactly the packed route's y (same kernels'
    arithmetic per token), checked against the oracle too."""
    B, D, T = 1, 512, 333
    inp, g = inputs(1500, B, D, T, "cl", True, False, BF16)
    lengths = [5, 1, 100, 2, 77, 148]
    cu = synth.cu_from_lengths(lengths)
    ids = torch.repeat_interleave(torch.arange(len(lengths), dtype=torch.int32),
                                  torch.tensor(lengths))[None, :]
    store = torch.zeros(T, 3, dtype=torch.int32)
    store[:, 1] = ids[0]
    gseq = dev(store).t()[1:2]                        # [1,T], stride (1, 3)
    assert gseq.stride() == (1, 3)
    y_seq, _ = ops.fwd(g["x"], g["weight"], g["bias"], None, None, "silu", seq_idx=gseq)
    ops.reset_flag(DEV)
    y_pk, _ = ops.fwd(g["x"], g["weight"], g["bias"], dev(cu), None, "silu")
    torch.cuda.synchronize()
    ops.check_flag(DEV)
    oy = oracle.fwd_seq(f64(inp["x"]), f64(inp["weight"]), ids.numpy(), f64(inp["bias"]),
                        "silu")
    check_bf16("y", y_seq, oy)
    assert torch.equal(y_seq, y_pk)


def test_seq_idx_autograd_and_declines():
    B, D, T = 2, 512, 96
    inp, g = inputs(1600, B, D, T, "cl", True, True, BF16)
    seq = synth.seq_idx_tensor(torch.Generator().manual_seed(1601), B, T, "runs", max_run=20)
    gseq = dev(seq)
    x = g["x"].detach().requires_grad_(True)
    w = g["weight"].detach().requires_grad_(True)
    b = g["bias"].detach().requires_grad_(True)
    y = ops.causal_conv1d(x, w, b, seq_idx=gseq, activation="silu")
    y.backward(g["dy"])
    odx, odw, odb = oracle.bwd_seq(f64(inp["x"]), f64(inp["weight"]), f64(inp["dy"]),
                                   seq.numpy(), f64(inp["bias"]), "silu")
    check_bf16("dx", x.grad, odx)
    check_cast_bf16("dweight", w.grad, odw)
    check_cast_bf16("dbias", b.grad, odb)
    with pytest.raises(NotImplementedError):
        ops.causal_conv1d(g["x"], g["weight"], g["bias"], seq_idx=gseq,
                          initial_states=g["initial_states"])
    with pytest.raises(NotImplementedError):
        ops.causal_conv1d(g["x"], g["weight"], g["bias"], seq_idx=gseq, return_final_states=True)


# ---- time-contiguous rows (time lanes) ----------------------------------------

def padded_tc(t, pad_to=8):
    """A [B,D,T] copy whose rows start on 16-byte boundaries (row stride
    rounded up to a multiple of 8 elements), on the device."""
    B, D, T = t.shape
    Tp = (T + pad_to - 1) // pad_to * pad_to + pad_to
    st = torch.zeros(B, D, Tp, dtype=t.dtype, device=DEV)
    view = st[:, :, :T]
    view.copy_(t.to(DEV))
    return view


TC_CASES = [
    # W, B, D, T, bias, init, dfinal, act, weight dtype, deterministic, padded rows
    (4, 2, 64, 4616, True, True, True, "silu", BF16, False, False),   # 3 chunks, last partial
    (4, 3, 40, 2048, True, False, False, "silu", BF16, True, False),  # exactly one chunk
    (4, 2, 24, 512, False, True, True, None, BF16, False, False),     # one tile
    (4, 1, 16, 8, True, True, True, "silu", BF16, False, False),      # one lane
    (4, 2, 16, 77, True, True, True, "silu", BF16, False, True),      # partial lanes
    (4, 2, 16, 2, True, True, True, "silu", BF16, False, True),       # T < W-1
    (3, 2, 32, 2600, True, True, True, "silu", BF16, True, False),
    (2, 2, 32, 1000, False, True, True, "silu", F32, False, True),
    (4, 2, 32, 2056, True, True, False, "silu", F32, True, False),    # FP32 filter + bias
    (4, 2, 16, 2049, True, True, True, "silu", BF16, False, False),   # right halo 1 token
    (4, 1, 24, 2050, False, True, True, "silu", BF16, True, False),   # dfinal across chunks
    (3, 2, 16, 1025, True, True, True, None, BF16, False, True),      # fwd chunk of 1 token
]


@pytest.mark.parametrize("case", TC_CASES, ids=lambda c: "W%d-B%d-D%d-T%d-%s%s%s" % (
    c[0], c[1], c[2], c[3], "f32" if c[8] == F32 else "bf16", "-det" if c[9] else "",
    "-padded" if c[10] else ""))
def test_time_lanes_parity(case):
    """Unit-stride time rows go to the time-lane kernels: forward (with the
    final state), backward (dx, dinit with dfinal, dW/dB atomics or
    deterministic partials) against the oracle, inside guard bands."""
    W, B, D, T, bias, init, dfinal, act, wdt, det, padded = case
    print("time-lane case", case, flush=True)
    inp, g = inputs(1700 + W + D + T, B, D, T, "tc", bias, init, wdt, dfinal, W=W)
    if padded:
        g["x"], g["dy"] = padded_tc(inp["x"]), padded_tc(inp["dy"])
    opts = (OPT_F32 if (bias and wdt == F32) else 0) | (OPT_DETDB if (bias and det) else 0)
    y, fin = run_fwd(g, "tc", act, True, options=opts)
    check_fwd(inp, y, fin, act)
    dx, dw, db, dinit = run_bwd(g, "tc", act, det, options=opts)
    check_bwd(inp, dx, dw, db, dinit, act)
    if det:
        _, dw2, db2, _ = run_bwd(g, "tc", act, det, options=opts)
        assert torch.equal(dw2.view(torch.int32), dw.view(torch.int32))
        if bias:
            assert torch.equal(db2.view(torch.int32), db.view(torch.int32))


def test_time_lanes_match_channel_lanes():
    """The same data in both layouts: time lanes and channel lanes agree to
    the rounding of their (identical) per-token arithmetic."""
    B, D, T = 2, 512, 3000
    inp, g = inputs(1800, B, D, T, "tc", True, True, BF16, True)
    y_tc, fin_tc = ops.fwd(g["x"], g["weight"], g["bias"], None, g["initial_states"], "silu",
                           return_final_states=True)
    x_cl = g["x"].transpose(1, 2).contiguous().transpose(1, 2)
    y_cl, fin_cl = ops.fwd(x_cl, g["weight"], g["bias"], None, g["initial_states"], "silu",
                           return_final_states=True)
    torch.cuda.synchronize()
    assert torch.equal(y_tc, y_cl) and torch.equal(fin_tc, fin_cl)


# ---- multi-token update ---------------------------------------------------------

MULTI_CASES = [
    # B, D, L, W, bias, weight dtype, layout of x/y
    (4, 512, 5, 4, True, BF16, "cl"),
    (3, 1024, 16, 4, False, BF16, "cl"),
    (2, 64, 2, 3, True, BF16, "cl"),
    (2, 64, 9, 2, True, F32, "cl"),
    (3, 40, 6, 4, True, BF16, "cl"),       # D % 8 != 0: one-channel lanes
    (2, 64, 7, 4, True, BF16, "tc"),       # [B,D,L] contiguous (unit token stride): one-channel lanes
    (5, 256, 1, 4, True, BF16, "cl"),      # L = 1 through the [B,D,L] form
    # token batches of 8 on 8-channel lanes: exactly one, two and a token,
    # three with other widths and filters
    (3, 512, 8, 4, True, BF16, "cl"),
    (2, 256, 17, 4, True, BF16, "cl"),
    (2, 128, 24, 3, False, F32, "cl"),
    (4, 64, 8, 2, False, BF16, "cl"),
]


@pytest.mark.parametrize("B,D,L,W,bias,wdt,layout", MULTI_CASES)
def test_update_several_tokens(B, D, L, W, bias, wdt, layout):
    """L tokens in one call == L single-token steps of the oracle; then a
    single-token call continues from the state it left."""
    print("multi-token update case", B, D, L, W, bias, wdt, layout, flush=True)
    gen = torch.Generator().manual_seed(1900 + D + L)
    state = synth.state_tensor(gen, B, D, W)
    w = synth.weight_tensor(gen, D, W, dtype=wdt)
    b = synth.bias_tensor(gen, D, wdt) if bias else None
    x = synth.activation_tensor(gen, B, D, L, layout)
    opts = OPT_F32 if (bias and wdt == F32) else 0
    g_state = dev(state)
    y = guarded_act(B, D, L, layout, DEV)
    ops.update(dev(x), g_state, dev(w), dev(b), "silu", y=y.view, options=opts)
    torch.cuda.synchronize()
    oy, ost = oracle.update_tokens(f64(x), f64(state), f64(w), f64(b), "silu")
    check_bf16("y", y.view, oy)
    assert y.intact()
    check_exact_bf16("conv_state", g_state, ost)
    xt = synth.activation_tensor(gen, B, D, 1, "tc")[:, :, 0].contiguous()
    yt = ops.update(dev(xt), g_state, dev(w), dev(b), "silu", options=opts)
    torch.cuda.synchronize()
    oyt, ost = oracle.update(f64(xt), ost, f64(w), f64(b), "silu")
    check_bf16("next token y", yt, oyt)
    check_exact_bf16("conv_state after", g_state, ost)


@pytest.mark.parametrize("T,D", [(93, 24), (126, 16), (100, 40), (2049, 8), (1030, 16)],
                         ids=["align2", "align4", "align8", "align2-long", "align4-long"])
def test_time_lanes_unaligned_rows(T, D):
    """[B,D,T]-contiguous activations whose rows start on 2-, 4- or 8-byte
    boundaries (T odd, T = 2 mod 4, T = 4 mod 8), outputs in unpadded
    storage too: the time lanes move a lane's 8 tokens in pieces of that
    width.  Forward with initial and final states, backward with dfinal and
    dinit, on both dW routes."""
    for det in (False, True):
        inp, g = inputs(2400 + T + det, 2, D, T, "tc", True, True, BF16, True)
        assert g["x"].stride() == (D * T, T, 1)
        opts = OPT_DETDB if det else 0
        y = guarded_act(2, D, T, "tc", DEV, aligned=False)
        fin = guarded_flat((2, D, 3), DEV)
        ops.fwd(g["x"], g["weight"], g["bias"], None, g["initial_states"], "silu",
                final_states_out=fin.view, y=y.view, options=opts)
        torch.cuda.synchronize()
        check_fwd(inp, y, fin, "silu")
        dx = guarded_act(2, D, T, "tc", DEV, aligned=False)
        _, dw, db, dinit = ops.bwd(g["x"], g["weight"], g["dy"], g["bias"], None,
                                   g["initial_states"], g["dfinal_states"], "silu", det, False,
                                   dx=dx.view, options=opts)
        torch.cuda.synchronize()
        check_bwd(inp, dx, dw, db, dinit, "silu")


def test_one_channel_lanes_packed_and_seq_idx():
    """Channel-last inputs with an odd channel count take the one-channel
    lanes: packed rows and seq_idx rows, forward and backward."""
    lengths = [5, 1, 40, 3, 77]
    cu = synth.cu_from_lengths(lengths)
    T = int(cu[-1])
    inp, g = inputs(2300, 1, 13, T, "cl", True, True, BF16, True, cu)
    ops.reset_flag(DEV)
    y, fin = run_fwd(g, "cl", "silu", True, cu)
    check_fwd(inp, y, fin, "silu")
    dx, dw, db, dinit = run_bwd(g, "cl", "silu", False, cu)
    check_bwd(inp, dx, dw, db, dinit, "silu")
    ops.check_flag(DEV)
    inp, g = inputs(2301, 2, 13, 93, "cl", True, False, BF16)
    seq = synth.seq_idx_tensor(torch.Generator().manual_seed(2302), 2, 93, "random")
    y = guarded_act(2, 13, 93, "cl", DEV)
    ops.fwd(g["x"], g["weight"], g["bias"], None, None, "silu", y=y.view, seq_idx=dev(seq))
    dx = guarded_act(2, 13, 93, "cl", DEV)
    _, dw, db, _ = ops.bwd(g["x"], g["weight"], g["dy"], g["bias"], None, None, None, "silu",
                           False, False, dx=dx.view, seq_idx=dev(seq))
    torch.cuda.synchronize()
    oy = oracle.fwd_seq(f64(inp["x"]), f64(inp["weight"]), seq.numpy(), f64(inp["bias"]), "silu")
    odx, odw, odb = oracle.bwd_seq(f64(inp["x"]), f64(inp["weight"]), f64(inp["dy"]),
                                   seq.numpy(), f64(inp["bias"]), "silu")
    check_bf16("y", y.view, oy)
    check_bf16("dx", dx.view, odx)
    check_f32_rel("dweight", dw, odw)
    check_f32_rel("dbias", db, odb)
    assert y.intact() and dx.intact()


@pytest.mark.parametrize("padded", [False, True], ids=["unaligned-rows", "aligned-rows"])
def test_packed_and_seq_idx_time_contiguous_layout(padded):
    """Packed offsets and seq_idx ids on a [B,D,T]-contiguous input: rows
    that start on 4- or 2-byte boundaries (T = 126, T = 93) and rows padded
    to 16-byte boundaries, on the time lanes.  Forward and backward against
    the oracle."""
    lengths = [5, 1, 40, 3, 77]
    cu = synth.cu_from_lengths(lengths)
    T = int(cu[-1])
    inp, g = inputs(2000, 1, 48, T, "tc", True, True, BF16, True, cu)
    if padded:
        g["x"], g["dy"] = padded_tc(inp["x"]), padded_tc(inp["dy"])
    ops.reset_flag(DEV)
    y, fin = run_fwd(g, "tc", "silu", True, cu)
    check_fwd(inp, y, fin, "silu")
    dx, dw, db, dinit = run_bwd(g, "tc", "silu", False, cu)
    check_bwd(inp, dx, dw, db, dinit, "silu")
    ops.check_flag(DEV)

    inp, g = inputs(2001, 2, 40, 93, "tc", True, False, BF16)
    if padded:
        g["x"], g["dy"] = padded_tc(inp["x"]), padded_tc(inp["dy"])
    seq = synth.seq_idx_tensor(torch.Generator().manual_seed(2002), 2, 93, "random")
    y = guarded_act(2, 40, 93, "tc", DEV)
    ops.fwd(g["x"], g["weight"], g["bias"], None, None, "silu", y=y.view, seq_idx=dev(seq))
    dx = guarded_act(2, 40, 93, "tc", DEV)
    _, dw, db, _ = ops.bwd(g["x"], g["weight"], g["dy"], g["bias"], None, None, None, "silu",
                           False, False, dx=dx.view, seq_idx=dev(seq))
    torch.cuda.synchronize()
    oy = oracle.fwd_seq(f64(inp["x"]), f64(inp["weight"]), seq.numpy(), f64(inp["bias"]), "silu")
    odx, odw, odb = oracle.bwd_seq(f64(inp["x"]), f64(inp["weight"]), f64(inp["dy"]),
                                   seq.numpy(), f64(inp["bias"]), "silu")
    check_bf16("y", y.view, oy)
    check_bf16("dx", dx.view, odx)
    check_f32_rel("dweight", dw, odw)
    check_f32_rel("dbias", db, odb)
    assert y.intact() and dx.intact()


TC_PACKED_CASES = [
    # lengths, D, W, bias, init, dfinal, deterministic
    ([1, 2, 3, 1, 1, 2, 3, 3, 2, 1] * 30 + [700, 1, 2], 24, 4, True, True, True, False),
    ([2049, 1, 2, 1100, 7], 16, 4, False, True, True, True),
    ([5, 1, 40, 3, 77, 513, 1, 1], 40, 3, True, True, False, False),
    ([1000, 30, 1], 8, 2, False, False, True, True),
    # few sequences, the forward chunk [1024, 2048) meets sequences 10..13
    ([700, 1, 1, 2, 3, 5, 8, 13, 21, 34, 400, 2, 2, 900, 1], 16, 4, True, True, True, False),
    # channel counts that leave part of the repair launches' last lane group idle
    ([300, 1, 2, 77, 3, 640], 13, 4, True, True, True, True),
    ([5, 1, 40, 3, 77, 513, 1, 1] * 9, 100, 3, False, True, True, False),
    ([3] * 1500, 8, 4, True, True, True, False),
    ([1, 2] * 2100, 8, 4, True, True, True, True),          # 4201 offsets: global path
]


@pytest.mark.parametrize("case", TC_PACKED_CASES, ids=lambda c: "N%d-D%d-W%d%s" % (
    len(c[0]), c[1], c[2], "-det" if c[6] else ""))
def test_packed_time_lanes(case):
    """Packed rows on time lanes (rows aligned to 16 bytes): sequence starts
    and ends inside a lane, several per lane, at tile and chunk edges, with
    initial states, dfinal, dinit and both dW routes."""
    lengths, D, W, bias, init, dfinal, det = case
    print("packed time-lane case", len(lengths), D, W, bias, init, dfinal, det, flush=True)
    cu = synth.cu_from_lengths(lengths)
    T = int(cu[-1])
    inp, g = inputs(2100 + len(lengths) + D, 1, D, T, "tc", bias, init, BF16, dfinal, cu, W=W)
    g["x"], g["dy"] = padded_tc(inp["x"]), padded_tc(inp["dy"])
    opts = OPT_DETDB if (bias and det) else 0
    ops.reset_flag(DEV)
    y, fin = run_fwd(g, "tc", "silu", True, cu, options=opts)
    check_fwd(inp, y, fin, "silu")
    dx, dw, db, dinit = run_bwd(g, "tc", "silu", det, cu, options=opts)
    check_bwd(inp, dx, dw, db, dinit, "silu")
    ops.check_flag(DEV)


@pytest.mark.parametrize("layout", ["cl", "tc"])
def test_large_magnitudes_saturate_like_the_oracle(layout):
    """Activations and states scaled by 64 (exact in BF16), so that the
    pre-activation spreads to |z| > 100: SiLU and its slope saturate (exp(-z)
    overflows and its reciprocal flushes to zero, or exp(-z) underflows) and
    must still match the oracle, forward, backward and update, with and
    without the activation."""
    B, D, T = 2, 64, 600
    inp = synth.random_inputs(4100 + (layout == "tc"), B, D, T, layout=layout, bias=True,
                              init=True, dfinal=True)
    for k in ("x", "initial_states"):
        inp[k] = inp[k] * 64
    assert inp["x"].stride() == synth.random_inputs(1, B, D, T, layout=layout)["x"].stride()
    g = {k: dev(v) for k, v in inp.items()}
    z = oracle.fwd(f64(inp["x"]), f64(inp["weight"]), f64(inp["bias"]), None,
                   f64(inp["initial_states"]), None)[0]
    assert np.abs(z).max() > 100  # the case the test is for
    for act in ("silu", None):
        print("large magnitudes", layout, act, flush=True)
        y, fin = run_fwd(g, layout, act, True)
        check_fwd(inp, y, fin, act)
        dx, dw, db, dinit = run_bwd(g, layout, act, False)
        check_bwd(inp, dx, dw, db, dinit, act)
    # the decode step from the same scaled states
    state = inp["initial_states"].contiguous()
    xt = inp["x"][:, :, 0].contiguous()
    g_state = dev(state)
    yt = ops.update(dev(xt), g_state, g["weight"], g["bias"], "silu")
    torch.cuda.synchronize()
    oyt, ost = oracle.update(f64(xt), f64(state), f64(inp["weight"]), f64(inp["bias"]), "silu")
    check_bf16("update y", yt, oyt)
    check_exact_bf16("conv_state", g_state, ost)


@pytest.mark.parametrize("k", [1, 2, 3, 5, 7])
def test_time_lanes_sliced_view_rows(k):
    """x and dy as [B,D,T] views that drop the first k tokens of wider rows:
    every row, the first included, starts k tokens past a 16-byte boundary
    and the tokens before it hold data.  Outputs match the oracle on the
    view alone, so nothing before a row's start is read into it."""
    B, D, T = 2, 12, 1500
    gen = torch.Generator().manual_seed(2600 + k)
    xw = synth.activation_tensor(gen, B, D, T + k, "tc")
    dyw = synth.activation_tensor(gen, B, D, T + k, "tc")
    w = synth.weight_tensor(gen, D, 4, dtype=BF16)
    b = synth.bias_tensor(gen, D, BF16)
    gx, gdy = dev(xw)[:, :, k:], dev(dyw)[:, :, k:]
    assert gx.stride() == (D * (T + k), T + k, 1)
    y = guarded_act(B, D, T, "tc", DEV, aligned=False)
    ops.fwd(gx, dev(w), dev(b), None, None, "silu", y=y.view)
    dx = guarded_act(B, D, T, "tc", DEV, aligned=False)
    _, dw, db, _ = ops.bwd(gx, dev(w), gdy, dev(b), None, None, None, "silu", False, False,
                           dx=dx.view)
    torch.cuda.synchronize()
    x, dy = f64(xw)[:, :, k:], f64(dyw)[:, :, k:]
    oy, _ = oracle.fwd(x, f64(w), f64(b), None, None, "silu", False)
    odx, odw, odb, _ = oracle.bwd(x, f64(w), dy, f64(b), None, None, None, "silu")
    check_bf16("y", y.view, oy)
    check_bf16("dx", dx.view, odx)
    check_f32_rel("dweight", dw, odw)
    check_f32_rel("dbias", db, odb)
    assert y.intact() and dx.intact()
