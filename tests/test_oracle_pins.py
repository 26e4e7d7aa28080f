"""Pins of the fp64 CPU oracle against things other than itself.

Each pin is one of: a value worked by hand (tests/golden), a library routine
(torch.nn.functional.conv1d / silu in float64 with torch autograd,
numpy.convolve), the pages' own general formula for a dilated causal conv1d
(POPCORNBENCH trace) specialised to a block-diagonal weight, an invariant of
the method (state chaining, packing, decode update, causality, adjoint),
closed forms, finite differences, and brute force over tiny metadata.

The last test plants mistakes in copies of the oracle source and checks that
the pins catch every one.
"""
import itertools
import json
import os
import tempfile

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_problem(seed, B, D, T, W=4, bias=True, init=True, dfinal=True, cu=None):
    r = _rng(seed)
    R = B if cu is None else len(cu) - 1
    p = dict(x=r.standard_normal((B, D, T)), w=r.uniform(-0.5, 0.5, (D, W)),
             bias=r.standard_normal(D) * 0.1 if bias else None,
             init=r.standard_normal((R, D, W - 1)) if init else None,
             dy=r.standard_normal((B, D, T)),
             dfinal=r.standard_normal((R, D, W - 1)) if dfinal else None, cu=cu)
    return p


def _fwd(p, act="silu"):
    return oracle.fwd(p["x"], p["w"], p["bias"], p["cu"], p["init"], act)


def _bwd(p, act="silu"):
    return oracle.bwd(p["x"], p["w"], p["dy"], p["bias"], p["cu"], p["init"], p["dfinal"], act)


# ---------------------------------------------------------------------------
# Worked examples (tests/golden/worked_example.json, derived by hand)
# ---------------------------------------------------------------------------

def test_golden_worked_example_dense():
    g = json.load(open(GOLDEN))["dense_no_activation"]
    x = np.array(g["x"], float)[None, None, :]
    w = np.array(g["weight"], float)[None, :]
    b = np.array([g["bias"]], float)
    init = np.array(g["initial_states"], float)[None, None, :]
    y, fin = oracle.fwd(x, w, b, None, init, None)
    assert y.ravel().tolist() == g["y"]
    assert fin.ravel().tolist() == g["final_states"]
    dy = np.array(g["dy"], float)[None, None, :]
    dfin = np.array(g["dfinal_states"], float)[None, None, :]
    dx, dw, db, dinit = oracle.bwd(x, w, dy, b, None, init, dfin, None)
    assert dx.ravel().tolist() == g["dx"]
    assert dinit.ravel().tolist() == g["dinitial_states"]
    assert dw.ravel().tolist() == g["dweight"]
    assert db.ravel().tolist() == [g["dbias"]]


def test_golden_worked_example_packed():
    g = json.load(open(GOLDEN))["packed_no_activation"]
    x = np.array(g["x"], float)[None, None, :]
    w = np.array(g["weight"], float)[None, :]
    y, fin = oracle.fwd(x, w, None, g["cu_seqlens"], None, None)
    assert y.ravel().tolist() == g["y"]
    assert fin[:, 0, :].tolist() == g["final_states"]


def test_golden_worked_example_update():
    g = json.load(open(GOLDEN))["update_no_activation"]
    y, st = oracle.update(np.array([[g["x"]]], float), np.array(g["state"], float)[None, None, :],
                          np.array(g["weight"], float)[None, :], np.array([g["bias"]], float), None)
    assert y.ravel().tolist() == [g["y"]]
    assert st.ravel().tolist() == g["new_state"]


# ---------------------------------------------------------------------------
# O1 single-tap weights reproduce a shifted copy of x
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_O1_single_tap_is_shift(W):
    p = _rand_problem(1, 2, 3, 9, W=W, bias=False)
    ext = np.concatenate([p["init"], p["x"]], axis=-1)      # [B, D, W-1+T]
    for j in range(W):
        w = np.zeros((3, W))
        w[:, j] = 1.0
        y, fin = oracle.fwd(p["x"], w, None, None, p["init"], None)
        # tap j meets x_ext[t - (W-1) + j]  ->  ext index t + j
        assert np.array_equal(y, ext[:, :, j:j + 9])
        assert np.array_equal(fin, ext[:, :, 9:])
    # without initial state the left pad is zeros
    w = np.zeros((3, W))
    w[:, 0] = 1.0
    y, _ = oracle.fwd(p["x"], w, None, None, None, None)
    assert np.all(y[:, :, :W - 1] == 0.0)
    assert np.array_equal(y[:, :, W - 1:], p["x"][:, :, :9 - (W - 1)])


# ---------------------------------------------------------------------------
# O6 library routines: F.conv1d (+ F.silu) in float64, torch autograd, np.convolve
# ---------------------------------------------------------------------------

def _torch_reference(p, act):
    """F.conv1d over the left-extended rows, grouped per channel."""
    x = torch.tensor(p["x"], requires_grad=True)
    w = torch.tensor(p["w"], requires_grad=True)
    b = torch.tensor(p["bias"], requires_grad=True) if p["bias"] is not None else None
    B, D, T = x.shape
    W = w.shape[1]
    init = (torch.tensor(p["init"], requires_grad=True) if p["init"] is not None
            else torch.zeros(B, D, W - 1, dtype=torch.float64))
    ext = torch.cat([init, x], dim=-1)
    z = F.conv1d(ext, w[:, None, :], b, groups=D)
    y = F.silu(z) if act == "silu" else z
    fin = ext[:, :, T:]
    loss = (y * torch.tensor(p["dy"])).sum()
    if p["dfinal"] is not None:
        loss = loss + (fin * torch.tensor(p["dfinal"])).sum()
    loss.backward()
    return dict(y=y.detach().numpy(), fin=fin.detach().numpy(), dx=x.grad.numpy(),
                dw=w.grad.numpy(), db=None if b is None else b.grad.numpy(),
                dinit=None if p["init"] is None else init.grad.numpy())


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("act", ["silu", None])
@pytest.mark.parametrize("bias,init,dfinal", [(True, True, True), (False, False, False),
                                              (True, False, True), (False, True, False)])
def test_O6_conv1d_library(W, act, bias, init, dfinal):
    p = _rand_problem(6, 2, 5, 11, W=W, bias=bias, init=init, dfinal=dfinal)
    ref = _torch_reference(p, act)
    y, fin = _fwd(p, act)
    dx, dw, db, dinit = _bwd(p, act)
    tol = dict(rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(y, ref["y"], **tol)
    np.testing.assert_array_equal(fin, ref["fin"])
    np.testing.assert_allclose(dx, ref["dx"], **tol)
    np.testing.assert_allclose(dw, ref["dw"], **tol)
    if bias:
        np.testing.assert_allclose(db, ref["db"], **tol)
    if init:
        np.testing.assert_allclose(dinit, ref["dinit"], **tol)


def test_O6_numpy_convolve():
    p = _rand_problem(7, 1, 4, 13, bias=True, init=True)
    y, _ = _fwd(p, None)
    for d in range(4):
        ext = np.concatenate([p["init"][0, d], p["x"][0, d]])
        # np.convolve flips its kernel: convolving with the reversed taps is
        # the cross-correlation; the 'valid' part is the causal output.
        z = np.convolve(ext, p["w"][d][::-1], mode="valid") + p["bias"][d]
        np.testing.assert_allclose(y[0, d], z, rtol=1e-13, atol=1e-14)


def test_O6_silu_library_closed_forms():
    z = np.linspace(-30, 30, 601)
    x = z[None, None, :]
    w = np.array([[0.0, 0.0, 0.0, 1.0]])
    y, _ = oracle.fwd(x, w, None, None, None, "silu")
    np.testing.assert_allclose(y.ravel(), F.silu(torch.tensor(z)).numpy(), rtol=1e-15, atol=1e-300)
    # silu(0) = 0, silu(-z) = silu(z) - z, silu(z) -> z for large z
    assert y[0, 0, 300] == 0.0
    np.testing.assert_allclose(y.ravel()[::-1], y.ravel() - z, rtol=0, atol=1e-13)
    assert abs(y.ravel()[-1] - 30.0) < 1e-11
    # silu'(0) = 1/2: d/dx of y at a zero pre-activation
    dx, dw, _, _ = oracle.bwd(np.zeros((1, 1, 1)), w, np.ones((1, 1, 1)), None, None, None, None, "silu")
    assert dx.ravel()[0] == 0.5


# ---------------------------------------------------------------------------
# O7 the pages' general dilated causal conv1d formula, block-diagonal weight
# ---------------------------------------------------------------------------

def test_O7_general_formula_block_diagonal():
    """POPCORNBENCH trace: out[b,oc,t] = sum_ic sum_k Wf[oc,ic,k] * in[b,ic,t+k*dil-P]
    with P = (K-1)*dil and zero for negative positions; dil = 1 and
    Wf[o,i,k] = w[o,k] * [i == o] is the depthwise special case."""
    p = _rand_problem(8, 2, 4, 10, bias=True, init=False)
    B, D, T = p["x"].shape
    K = 4
    Wf = np.zeros((D, D, K))
    for o in range(D):
        Wf[o, o, :] = p["w"][o]
    out = np.zeros((B, D, T))
    for b, oc, t in itertools.product(range(B), range(D), range(T)):
        s = 0.0
        for ic in range(D):
            for k in range(K):
                pos = t + k - (K - 1)
                if pos >= 0:
                    s += Wf[oc, ic, k] * p["x"][b, ic, pos]
        out[b, oc, t] = s + p["bias"][oc]
    y, _ = _fwd(p, None)
    np.testing.assert_allclose(y, out, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# O2 chaining through final_states, forward and backward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("split", [1, 2, 3, 6, 11])
def test_O2_chaining(split):
    T = 12
    p = _rand_problem(2, 2, 3, T, bias=True, init=True, dfinal=True)
    y, fin = _fwd(p)
    p1 = dict(p, x=p["x"][:, :, :split], dy=p["dy"][:, :, :split])
    y1, f1 = _fwd(p1)
    p2 = dict(p, x=p["x"][:, :, split:], dy=p["dy"][:, :, split:], init=f1)
    y2, f2 = _fwd(p2)
    assert np.array_equal(np.concatenate([y1, y2], -1), y)
    assert np.array_equal(f2, fin)
    # backward: the second chunk's dinit is the first chunk's dfinal
    dx, dw, db, dinit = _bwd(p)
    dx2, dw2, db2, dinit2 = _bwd(p2)
    dx1, dw1, db1, dinit1 = _bwd(dict(p1, dfinal=dinit2))
    np.testing.assert_allclose(np.concatenate([dx1, dx2], -1), dx, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dinit1, dinit, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dw1 + dw2, dw, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(db1 + db2, db, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# O3 packed == per-sequence dense runs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lengths", [[1, 2, 3, 5, 8], [4], [1, 1, 1], [7, 2], [3, 1, 6, 2]])
@pytest.mark.parametrize("init", [True, False])
def test_O3_packed_equals_dense(lengths, init):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    p = _rand_problem(3, 1, 3, T, bias=True, init=init, dfinal=True, cu=cu)
    y, fin = _fwd(p)
    dx, dw, db, dinit = _bwd(p)
    dw_sum = np.zeros_like(dw)
    db_sum = np.zeros_like(db)
    for i, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        q = dict(p, x=p["x"][:, :, s:e], dy=p["dy"][:, :, s:e], cu=None,
                 init=None if p["init"] is None else p["init"][i:i + 1],
                 dfinal=p["dfinal"][i:i + 1])
        yi, fi = _fwd(q)
        assert np.array_equal(y[:, :, s:e], yi)
        assert np.array_equal(fin[i:i + 1], fi)
        dxi, dwi, dbi, dii = _bwd(q)
        np.testing.assert_allclose(dx[:, :, s:e], dxi, rtol=1e-13, atol=1e-14)
        if init:
            np.testing.assert_allclose(dinit[i:i + 1], dii, rtol=1e-13, atol=1e-14)
        dw_sum += dwi
        db_sum += dbi
    np.testing.assert_allclose(dw, dw_sum, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(db, db_sum, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# O4 prefix forward then single-token updates == the full forward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T0", [1, 2, 3, 5])
@pytest.mark.parametrize("bias", [True, False])
def test_O4_update_steps_reproduce_forward(T0, bias):
    T = 9
    p = _rand_problem(4, 3, 5, T, bias=bias, init=True)
    y_full, fin_full = _fwd(p)
    _, state = _fwd(dict(p, x=p["x"][:, :, :T0]))
    for t in range(T0, T):
        yt, state = oracle.update(p["x"][:, :, t], state, p["w"], p["bias"], "silu")
        assert np.array_equal(yt, y_full[:, :, t])
    assert np.array_equal(state, fin_full)


@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("L", [1, 2, 7])
def test_O4_multi_token_update_is_forward_from_the_state(W, L):
    """L tokens at once == the forward over those tokens with the state as
    its initial state (outputs and final state, exactly), and == the
    library conv1d of the state followed by the tokens."""
    p = _rand_problem(14, 3, 4, L, W=W, bias=True, init=True)
    y, st = oracle.update_tokens(p["x"], p["init"], p["w"], p["bias"], "silu")
    yf, ff = oracle.fwd(p["x"], p["w"], p["bias"], None, p["init"], "silu")
    assert np.array_equal(y, yf) and np.array_equal(st, ff)
    full = torch.tensor(np.concatenate([p["init"], p["x"]], axis=2))
    ref = F.silu(F.conv1d(F.pad(full, (W - 1, 0)), torch.tensor(p["w"])[:, None, :],
                          torch.tensor(p["bias"]), groups=4))[:, :, W - 1:]
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(st, np.concatenate([p["init"], p["x"]], axis=2)[:, :, -(W - 1):])


# ---------------------------------------------------------------------------
# O5 central finite differences on tiny inputs
# ---------------------------------------------------------------------------

def _loss(p, act):
    y, fin = _fwd(p, act)
    return float(np.sum(p["dy"] * y) + np.sum(p["dfinal"] * fin))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("act", ["silu", None])
def test_O5_finite_differences(packed, act):
    if packed:
        cu = np.array([0, 1, 3, 8], np.int32)
        p = _rand_problem(5, 1, 3, 8, bias=True, init=True, dfinal=True, cu=cu)
    else:
        p = _rand_problem(5, 2, 3, 7, bias=True, init=True, dfinal=True)
    dx, dw, db, dinit = _bwd(p, act)
    h = 1e-6
    for name, grad in (("x", dx), ("w", dw), ("bias", db), ("init", dinit)):
        base = p[name]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += h
            minus[idx] -= h
            num[idx] = (_loss(dict(p, **{name: plus}), act) - _loss(dict(p, **{name: minus}), act)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-7, atol=1e-7, err_msg=name)


# ---------------------------------------------------------------------------
# O8 adjoint and Euler identities
# ---------------------------------------------------------------------------

def test_O8_adjoint_and_euler():
    p = _rand_problem(9, 2, 4, 10, bias=True, init=True, dfinal=False)
    y_lin, _ = _fwd(p, None)
    z_minus_b = y_lin - p["bias"][None, :, None]
    # with no activation g = dy, and the map (x_ext) -> z - b is linear:
    # <g, z - b> = <dx_ext, x_ext> summed over the whole extended rows
    dx, dw, db, dinit = _bwd(p, None)
    lhs = np.sum(p["dy"] * z_minus_b)
    rhs = np.sum(dx * p["x"]) + np.sum(dinit * p["init"])
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    # Euler: z - b is linear in w, so sum w * dW = <g, z - b>; dB = sum g
    assert abs(np.sum(p["w"] * dw) - lhs) <= 1e-12 * max(1.0, abs(lhs))
    np.testing.assert_allclose(db, p["dy"].sum(axis=(0, 2)), rtol=1e-13)


# ---------------------------------------------------------------------------
# O9 causality and sequence isolation
# ---------------------------------------------------------------------------

def test_O9_causality_and_isolation():
    p = _rand_problem(10, 1, 3, 12, bias=True, init=True)
    y, _ = _fwd(p)
    for t0 in (0, 4, 11):
        q = dict(p, x=p["x"].copy())
        q["x"][:, :, t0] += 1.0
        yq, _ = _fwd(q)
        assert np.array_equal(yq[:, :, :t0], y[:, :, :t0])
        assert not np.array_equal(yq[:, :, t0], y[:, :, t0])
    cu = np.array([0, 4, 5, 12], np.int32)
    p = _rand_problem(11, 1, 3, 12, bias=True, init=True, cu=cu)
    y, fin = _fwd(p)
    q = dict(p, x=p["x"].copy(), init=p["init"].copy())
    q["x"][:, :, 4] += 1.0          # sequence 1 is the single token at t = 4
    q["init"][1] += 1.0
    yq, finq = _fwd(q)
    keep = np.r_[0:4, 5:12]
    assert np.array_equal(yq[:, :, keep], y[:, :, keep])
    assert np.array_equal(finq[[0, 2]], fin[[0, 2]])


# ---------------------------------------------------------------------------
# O10 closed forms of the epilogue
# ---------------------------------------------------------------------------

def test_O10_closed_forms():
    p = _rand_problem(12, 2, 3, 6, bias=True, init=True)
    y, _ = oracle.fwd(p["x"], np.zeros((3, 4)), p["bias"], None, p["init"], "silu")
    b = p["bias"]
    expect = b / (1 + np.exp(-b))
    np.testing.assert_allclose(y, np.broadcast_to(expect[None, :, None], y.shape), rtol=1e-15)
    c = 0.75
    x = np.full((2, 3, 6), c)
    init = np.full((2, 3, 3), c)
    y, fin = oracle.fwd(x, p["w"], p["bias"], None, init, None)
    z = b + c * p["w"].sum(axis=1)
    np.testing.assert_allclose(y, np.broadcast_to(z[None, :, None], y.shape), rtol=1e-14)
    assert np.all(fin == c)


# ---------------------------------------------------------------------------
# O11 cu_seqlens flags by brute force
# ---------------------------------------------------------------------------

def _predicate(cu, total):
    """An independent reading of the four conditions (cuDNN FE 'Causal
    Conv1d', device-side validation paragraph)."""
    bits = 0
    if cu[0] != 0:
        bits |= oracle.CU_FIRST_NONZERO
    if cu[-1] != total:
        bits |= oracle.CU_LAST_MISMATCH
    diffs = [b - a for a, b in zip(cu[:-1], cu[1:])]
    if any(d < 0 for d in diffs):
        bits |= oracle.CU_DECREASING
    if any(d == 0 for d in diffs):
        bits |= oracle.CU_EMPTY
    return bits


def test_O11_flags_brute_force():
    n = 0
    for N in (1, 2, 3):
        for cu in itertools.product(range(-1, 6), repeat=N + 1):
            for total in range(1, 6):
                assert oracle.validate_cu_seqlens(list(cu), total) == _predicate(cu, total), (cu, total)
                n += 1
    assert n == 5 * (7 ** 2 + 7 ** 3 + 7 ** 4)


FLAG_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cu_seqlens_flags.json")


def test_O11_flags_hand_worked_table():
    """The oracle's flag word against a table worked by hand from the four
    malformed-metadata conditions of the cuDNN FE 'Causal Conv1d' page's
    device-side validation paragraph (tests/golden/cu_seqlens_flags.json):
    each condition alone, on several positions, and in combination."""
    table = json.load(open(FLAG_GOLDEN))["cases"]
    seen = 0
    for row in table:
        got = oracle.validate_cu_seqlens(row["cu"], row["total"])
        assert got == row["flags"], (row, got)
        seen |= row["flags"]
    # every bit is exercised alone and the table holds the all-bits case
    singles = {row["flags"] for row in table}
    assert {1, 2, 4, 8, 15} <= singles and seen == 15


# ---------------------------------------------------------------------------
# O12 per-token sequence ids (seq_idx)
# ---------------------------------------------------------------------------

def _seq_problem(seed, B, D, T, W=4, bias=True):
    r = _rng(seed)
    return dict(x=r.standard_normal((B, D, T)), w=r.uniform(-0.5, 0.5, (D, W)),
                bias=r.standard_normal(D) * 0.1 if bias else None,
                dy=r.standard_normal((B, D, T)))


def _runs_to_ids(lengths, first_id=0):
    return np.concatenate([np.full(n, first_id + i, np.int32) for i, n in enumerate(lengths)])


@pytest.mark.parametrize("W", [2, 3, 4])
def test_O12_constant_ids_are_the_dense_route(W):
    """One id per row: the library conv1d (float64, autograd) exactly as the
    dense route with zero initial state."""
    p = _seq_problem(21, 2, 3, 9, W)
    seq = np.array([[5] * 9, [-2] * 9], np.int32)
    y = oracle.fwd_seq(p["x"], p["w"], seq, p["bias"], "silu")
    dx, dw, db = oracle.bwd_seq(p["x"], p["w"], p["dy"], seq, p["bias"], "silu")
    xt = torch.tensor(p["x"], requires_grad=True)
    wt = torch.tensor(p["w"], requires_grad=True)
    bt = torch.tensor(p["bias"], requires_grad=True)
    yt = F.silu(F.conv1d(F.pad(xt, (W - 1, 0)), wt[:, None, :], bt, groups=3))
    (yt * torch.tensor(p["dy"])).sum().backward()
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("lengths", [[1, 2, 3, 5, 8], [4, 1, 1, 13], [19]])
def test_O12_contiguous_runs_are_the_packed_route(lengths):
    """Ids constant over contiguous runs: every run is an independent
    sequence, i.e. the packed route (cu_seqlens from the runs, no states), and
    per-run library conv1d."""
    T = sum(lengths)
    p = _seq_problem(22, 1, 3, T)
    seq = _runs_to_ids(lengths, first_id=7)[None, :]
    y = oracle.fwd_seq(p["x"], p["w"], seq, p["bias"], "silu")
    dx, dw, db = oracle.bwd_seq(p["x"], p["w"], p["dy"], seq, p["bias"], "silu")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    yp, _ = oracle.fwd(p["x"], p["w"], p["bias"], cu, None, "silu")
    dxp, dwp, dbp, _ = oracle.bwd(p["x"], p["w"], p["dy"], p["bias"], cu, None, None, "silu")
    assert np.array_equal(y, yp)
    np.testing.assert_allclose(dx, dxp, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dw, dwp, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(db, dbp, rtol=1e-12, atol=1e-13)
    for s, e in zip(cu[:-1], cu[1:]):
        xt = torch.tensor(p["x"][:, :, s:e])
        ref = F.silu(F.conv1d(F.pad(xt, (3, 0)), torch.tensor(p["w"])[:, None, :],
                              torch.tensor(p["bias"]), groups=3))
        np.testing.assert_allclose(y[:, :, s:e], ref.numpy(), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("m", [2, 3])
@pytest.mark.parametrize("W", [3, 4])
def test_O12_periodic_ids_reduce_to_a_sparse_filter(m, W):
    """ids[t] = t mod m: output t sees only positions t - j with j a multiple
    of m, so the route equals the dense library conv1d with the other taps
    zeroed (their dW is exactly zero); two rows, both activations."""
    T = 11
    p = _seq_problem(23, 2, 3, T, W)
    seq = np.tile((np.arange(T) % m).astype(np.int32), (2, 1))
    keep = np.array([(W - 1 - k) % m == 0 for k in range(W)])
    for act in ("silu", None):
        y = oracle.fwd_seq(p["x"], p["w"], seq, p["bias"], act)
        dx, dw, db = oracle.bwd_seq(p["x"], p["w"], p["dy"], seq, p["bias"], act)
        xt = torch.tensor(p["x"], requires_grad=True)
        wt = torch.tensor(p["w"] * keep, requires_grad=True)
        bt = torch.tensor(p["bias"], requires_grad=True)
        z = F.conv1d(F.pad(xt, (W - 1, 0)), wt[:, None, :], bt, groups=3)
        yt = F.silu(z) if act else z
        (yt * torch.tensor(p["dy"])).sum().backward()
        np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dw[:, keep], wt.grad.numpy()[:, keep], rtol=1e-12,
                                   atol=1e-13)
        assert np.all(dw[:, ~keep] == 0.0)
        np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-12, atol=1e-13)


def _seq_loss(p, seq, act):
    return float(np.sum(p["dy"] * oracle.fwd_seq(p["x"], p["w"], seq, p["bias"], act)))


@pytest.mark.parametrize("act", ["silu", None])
def test_O12_finite_differences_recurring_ids(act):
    """Ids that recur within the window (no run structure): the backward is
    the gradient of the forward, by central differences."""
    p = _seq_problem(24, 2, 2, 9)
    seq = np.array([[0, 1, 0, 0, 2, 1, 1, 2, 2], [3, 3, 4, 3, 4, 4, 3, 3, 3]], np.int32)
    dx, dw, db = oracle.bwd_seq(p["x"], p["w"], p["dy"], seq, p["bias"], act)
    h = 1e-6
    for name, grad in (("x", dx), ("w", dw), ("bias", db)):
        base = p[name]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += h
            minus[idx] -= h
            num[idx] = (_seq_loss(dict(p, **{name: plus}), seq, act) -
                        _seq_loss(dict(p, **{name: minus}), seq, act)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-7, atol=1e-7, err_msg=name)


def test_O12_relabelling_and_row_isolation():
    """Only equality of ids matters (a bijective relabelling changes nothing,
    bit for bit), and rows never see each other."""
    p = _seq_problem(25, 2, 3, 10)
    seq = np.array([[0, 0, 1, 1, 1, 0, 2, 2, 1, 1], [4, 4, 4, 5, 5, 4, 4, 6, 6, 6]], np.int32)
    relabel = {0: 100, 1: -3, 2: 7, 4: 0, 5: 2**31 - 1, 6: -2**31}
    seq2 = np.vectorize(relabel.get)(seq).astype(np.int32)
    y = oracle.fwd_seq(p["x"], p["w"], seq, p["bias"], "silu")
    assert np.array_equal(y, oracle.fwd_seq(p["x"], p["w"], seq2, p["bias"], "silu"))
    g1 = oracle.bwd_seq(p["x"], p["w"], p["dy"], seq, p["bias"], "silu")
    g2 = oracle.bwd_seq(p["x"], p["w"], p["dy"], seq2, p["bias"], "silu")
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)
    x2 = p["x"].copy()
    x2[1] += 5.0
    y2 = oracle.fwd_seq(x2, p["w"], seq, p["bias"], "silu")
    assert np.array_equal(y[0], y2[0]) and not np.array_equal(y[1], y2[1])


# ---------------------------------------------------------------------------
# The pins catch planted mistakes
# ---------------------------------------------------------------------------

MUTANTS = [
    ("tap order reversed",
     "acc += w[d * W + k] * x_ext(x, init, b, d, t - (W - 1) + k, row, D, T, W);",
     "acc += w[d * W + (W - 1 - k)] * x_ext(x, init, b, d, t - (W - 1) + k, row, D, T, W);"),
    ("initial state read newest-first",
     "int64_t j = p - row.s + (W - 1);", "int64_t j = row.s - 1 - p;"),
    ("SiLU slope sign",
     "return s * (1.0 + z * (1.0 - s));", "return s * (1.0 - z * (1.0 - s));"),
    ("bias dropped",
     "row, D, T, W);\n    if (bias)\n        acc += bias[d];", "row, D, T, W);"),
    ("seq_idx bias dropped",
     "t, D, T);\n    if (bias)\n        acc += bias[d];", "t, D, T);"),
    ("dfinal slot off by one",
     "int64_t j = tau - (row.e - (W - 1));", "int64_t j = tau - (row.e - W);"),
    ("packed row lookup off by one",
     "(int64_t)cu[i + 1] <= t", "(int64_t)cu[i + 1] < t"),
    ("update keeps the oldest token", "s[k] = v[k + 1];", "s[k] = v[k];"),
    ("equal offsets counted as decreasing",
     "if (cu[i + 1] < cu[i])", "if (cu[i + 1] <= cu[i])"),
    ("first offset checked for negatives only", "if (cu[0] != 0)", "if (cu[0] < 0)"),
    ("last offset read one early",
     "if ((int64_t)cu[N] != total)", "if ((int64_t)cu[N - 1] != total)"),
    ("empty sequences missed", "if (cu[i + 1] == cu[i])", "if (0)"),
    ("first offset pair skipped",
     "for (int64_t i = 0; i < N; ++i) {\n        if (cu[i + 1] < cu[i])",
     "for (int64_t i = 1; i < N; ++i) {\n        if (cu[i + 1] < cu[i])"),
    ("dW uses the wrong tap",
     "dw[d * W + k] += g * x_ext(x, init, b, d, t - (W - 1) + k, row, D, T, W);",
     "dw[d * W + k] += g * x_ext(x, init, b, d, t - k, row, D, T, W);"),
    ("final state shifted",
     "x_ext(x, init, b, d, row.e - (W - 1) + j, row, D, T, W);",
     "x_ext(x, init, b, d, row.e - W + j, row, D, T, W);"),
    ("dx misses the in-row bound", "if (t >= row.s && t < row.e)", "if (t >= row.s)"),
    ("dinit taken at the wrong place",
     "row.s - (W - 1) + j, row, D, T, W);", "row.s - W + j, row, D, T, W);"),
    ("seq_idx mask ignored",
     "if (p < 0 || seq[b * T + p] != seq[b * T + t])", "if (p < 0)"),
    ("seq_idx dx ignores the ids",
     "if (t < T && seq[b * T + t] == seq[b * T + p]) {", "if (t < T) {"),
    ("seq_idx dW unmasked",
     "dw[d * W + k] += g * x_seen(x, seq, b, d, t - (W - 1) + k, t, D, T);",
     "dw[d * W + k] += g * x_seen(x, seq, b, d, t - (W - 1) + k, t - (W - 1) + k, D, T);"),
    ("seq_idx tap order reversed",
     "acc += w[d * W + k] * x_seen(x, seq, b, d, t - (W - 1) + k, t, D, T);",
     "acc += w[d * W + (W - 1 - k)] * x_seen(x, seq, b, d, t - (W - 1) + k, t, D, T);"),
]

PIN_BATTERY = [
    test_golden_worked_example_dense,
    test_golden_worked_example_packed,
    test_golden_worked_example_update,
    lambda: test_O1_single_tap_is_shift(4),
    lambda: test_O6_conv1d_library(4, "silu", True, True, True),
    lambda: test_O3_packed_equals_dense([1, 2, 3, 5, 8], True),
    lambda: test_O4_update_steps_reproduce_forward(2, True),
    test_O11_flags_brute_force,
    test_O11_flags_hand_worked_table,
    lambda: test_O12_contiguous_runs_are_the_packed_route([1, 2, 3, 5, 8]),
    lambda: test_O12_periodic_ids_reduce_to_a_sparse_filter(2, 4),
    lambda: test_O12_finite_differences_recurring_ids("silu"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = oracle.source_text()
    assert src.count(old) == 1, "mutation site not unique: %s" % name
    lib = oracle.compile_variant(src.replace(old, new), str(tmp_path))
    caught = False
    with oracle.use_library(lib):
        for pin in PIN_BATTERY:
            try:
                pin()
            except (AssertionError, ValueError):
                caught = True
                break
    assert caught, "no pin caught the planted mistake: %s" % name
