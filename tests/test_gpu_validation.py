"""Device-side validation of packed offsets, as the packed forward and
backward run it (cuDNN FE "Causal Conv1d", the paragraph on device-side
validation): every malformed-metadata condition alone and in combination,
with the offsets staged and checked inside every block (N+1 <= 4096), with
the separate validation kernel ahead of the blocks (N+1 > 4096), and on
[B,D,T]-contiguous rows, whose time-lane chunk launch validates up to 64
offsets in every wave and otherwise follows the validation kernel.

For each call, on a freshly cleared flag word:
  * the word equals the oracle's flag bits, bit for bit;
  * nothing was written: y, final_states, dx and dinitial_states keep their
    sentinel fill, guard bands included, and dweight/dbias (accumulated into
    by the backward) keep their starting bits.  The deterministic backward is
    given a workspace full of non-zero garbage, so a reduction that ran
    anyway would show in dweight.
"""
import numpy as np
import pytest
import torch

import oracle
from depthwise_causal_conv1d_02_amd import _abi, ops, synth
from parity import check_bf16, check_exact_bf16, check_f32_rel, f64, guarded_act, guarded_flat

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
BF16, F32 = torch.bfloat16, torch.float32
D = 64


def _cu(lengths):
    return synth.cu_from_lengths(lengths).tolist()


def _set(cu, i, v):
    cu = list(cu)
    cu[i] = v
    return cu


def _lds_cases(lengths=(5, 7, 9, 4, 6)):
    good = _cu(list(lengths))                              # [0,5,12,21,25,31]
    T = good[-1]
    swap = list(good)
    swap[2], swap[3] = swap[3], swap[2]
    return T, [
        ("first_nonzero", _set(good, 0, 2)),
        ("first_negative", _set(good, 0, -3)),
        ("last_short", _set(good, -1, T - 1)),
        ("last_past_total", _set(good, -1, T + 9)),
        ("decreasing", swap),
        ("decreasing_negative", _set(good, 1, -4)),
        ("empty_first", _set(good, 1, 0)),
        ("empty_middle", _set(good, 3, good[2])),
        ("empty_last", _set(good, -2, T)),
        ("first_and_last", _set(_set(good, 0, 1), -1, T - 2)),
        ("decreasing_and_empty", [0, 5, 5, 3, 25, 31]),
        ("all_four", [4, 4, 2, 21, 25, 30]),
    ]


def _global_cases(lengths=None):
    good = _cu(lengths or [3] * 5000 + [5, 7])             # N = 5002 > 4095
    T = good[-1]
    n = len(good)
    swap = list(good)
    swap[4500], swap[4501] = swap[4501], swap[4500]
    return T, [
        ("first_nonzero", _set(good, 0, 1)),
        ("last_short", _set(good, -1, T - 1)),
        ("last_past_total", _set(good, -1, T + 100)),
        ("decreasing_late", swap),
        ("empty_late", _set(good, 4500, good[4499])),
        ("empty_early", _set(good, 10, good[9])),
        ("all_four", _set(_set(_set(swap, 0, 2), n - 1, T + 1), 20, good[19])),
    ]


# time lanes: [B,D,T]-contiguous rows whose length is a multiple of 8, so
# that every row starts on a 16-byte boundary; 5 sequences (the chunk
# launch validates them in every wave) and 5002 (the validation launch)
TIME_LENGTHS = (5, 7, 9, 4, 7)
TIME_MANY_LENGTHS = [3] * 5000 + [5, 11]
PATHS = ["lds", "global", "time", "time_many"]


def _cases(path):
    if path == "global":
        return _global_cases()
    if path == "time_many":
        return _global_cases(TIME_MANY_LENGTHS)
    return _lds_cases(TIME_LENGTHS if path == "time" else (5, 7, 9, 4, 6))


def _layout(path):
    return "tc" if path.startswith("time") else "cl"


def _inputs(T, seed, bias, layout):
    inp = synth.random_inputs(seed, 1, D, T, layout=layout, bias=bias, init=False)
    return {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}


def _bits(t):
    return t.view(torch.int16).clone() if t.dtype == BF16 else t.view(torch.int32).clone()


class _Call:
    """One packed call kind.  alloc() makes fresh output buffers (sentinel-
    filled activations and states inside guard bands, pattern-filled
    dweight/dbias, a garbage workspace) and returns every tensor the call
    may write; run(cu, flag) launches it on those buffers."""

    def __init__(self, name, T, R, g, init, dfin, kind, layout):
        self.name, self.T, self.R, self.g, self.init, self.dfin = name, T, R, g, init, dfin
        self.kind, self.layout = kind, layout

    def alloc(self):
        T, R = self.T, self.R
        bias = self.g["bias"] is not None
        if self.kind == "fwd":
            self.y = guarded_act(1, D, T, self.layout, DEV)
            self.fin = guarded_flat((R, D, 3), DEV)
            return [self.y.storage, self.fin.storage]
        self.dx = guarded_act(1, D, T, self.layout, DEV)
        self.dinit = guarded_flat((R, D, 3), DEV)
        self.dw = torch.full((D, 4), 1.5, dtype=F32, device=DEV)
        self.db = torch.full((D,), -2.25, dtype=F32, device=DEV) if bias else None
        self.ws = torch.full((1 << 18,), 7.0, dtype=F32, device=DEV)   # garbage partials
        out = [self.dx.storage, self.dinit.storage, self.dw, self.ws]
        return out + ([self.db] if bias else [])

    def run(self, cu, flag):
        g = self.g
        if self.kind == "fwd":
            ops.fwd(g["x"], g["weight"], g["bias"], cu, self.init, "silu",
                    final_states_out=self.fin.view, y=self.y.view, err_flag=flag)
            return
        det = self.kind != "bwd_atomic"
        opts = _abi.CCV_OPT_DETERMINISTIC_DBIAS if self.kind == "bwd_deterministic_dbias" else 0
        ops.bwd(g["x"], g["weight"], g["dy"], g["bias"], cu, self.init, self.dfin, "silu",
                deterministic=det, dx=self.dx.view, err_flag=flag, dweight=self.dw,
                dbias=self.db, dinit=self.dinit.view, workspace=self.ws.view(torch.uint8),
                options=opts)


def _calls(T, cu_len, layout):
    """fwd, atomic bwd, deterministic bwd (bias-free), and deterministic bwd
    with a bias whose dbias goes through the partials too."""
    R = cu_len - 1
    gb = _inputs(T, 900 + T, True, layout)
    gn = _inputs(T, 901 + T, False, layout)
    init = synth.state_tensor(torch.Generator().manual_seed(T), R, D, 4).to(DEV)
    dfin = synth.state_tensor(torch.Generator().manual_seed(T + 1), R, D, 4).to(DEV)
    kinds = ("fwd", "bwd_atomic", "bwd_deterministic", "bwd_deterministic_dbias")
    return [_Call(k, T, R, gn if k == "bwd_deterministic" else gb, init, dfin, k, layout)
            for k in kinds]


def _check_call(label, cu, T, call, flag_start=0, want=None):
    """Run one call with the flag word at `flag_start`; the word must come back
    as `want` (default: the oracle's bits) and nothing may have been written."""
    if want is None:
        want = oracle.validate_cu_seqlens(cu, T)
        assert want != 0, label
    flag = torch.full((1,), flag_start, dtype=torch.int32, device=DEV)
    bufs = call.alloc()
    before = [_bits(b) for b in bufs]
    call.run(torch.tensor(cu, dtype=torch.int32, device=DEV), flag)
    torch.cuda.synchronize()
    got = int(flag.item()) & 0xffffffff
    assert got == want, "%s: flag %#x, expected %#x" % (label, got, want)
    for i, (b, s) in enumerate(zip(bufs, before)):
        assert torch.equal(_bits(b), s), "%s: buffer %d was written" % (label, i)


@pytest.mark.parametrize("path", PATHS)
def test_malformed_offsets_flag_is_the_oracles_and_nothing_is_written(path):
    T, cases = _cases(path)
    calls = _calls(T, len(cases[0][1]), _layout(path))
    for label, cu in cases:
        for call in calls:
            print("validation case", path, label, call.name, flush=True)
            _check_call("%s/%s/%s" % (path, label, call.name), cu, T, call)
    # the standalone export agrees on the same arrays (it overwrites its word)
    for label, cu in cases:
        got = int(ops.validate_cu_seqlens(torch.tensor(cu, dtype=torch.int32, device=DEV),
                                          T).item())
        assert got == oracle.validate_cu_seqlens(cu, T), label


def _good(path):
    return _cu({"lds": [5, 7, 9, 4, 6], "global": [3] * 5000 + [5, 7],
                "time": list(TIME_LENGTHS), "time_many": TIME_MANY_LENGTHS}[path])


@pytest.mark.parametrize("path", PATHS)
def test_sticky_flag_blocks_every_call_and_keeps_its_bits(path):
    """A word already non-zero (here a bit no validation produces) stops
    well-formed calls too and comes back unchanged."""
    good = _good(path)
    T = good[-1]
    assert oracle.validate_cu_seqlens(good, T) == 0
    for call in _calls(T, len(good), _layout(path)):
        print("sticky case", path, call.name, flush=True)
        _check_call("sticky/%s/%s" % (path, call.name), good, T, call, flag_start=0x40,
                    want=0x40)


@pytest.mark.parametrize("path", PATHS)
def test_after_clearing_the_flag_packed_results_match_the_oracle(path):
    good = _good(path)
    T = good[-1]
    cu_cpu = torch.tensor(good, dtype=torch.int32)
    inp = synth.random_inputs(950 + T, 1, D, T, layout=_layout(path), bias=False, init=True,
                              dfinal=True, cu_seqlens=cu_cpu)
    g = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    # a malformed call first sets the word ...
    bad = list(good)
    bad[1] = 0
    ops.fwd(g["x"], g["weight"], None, torch.tensor(bad, dtype=torch.int32, device=DEV),
            g["initial_states"], "silu", return_final_states=True, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == oracle.validate_cu_seqlens(bad, T)
    flag.zero_()
    # ... and once it is cleared the deterministic route runs and is exact
    y, fin = ops.fwd(g["x"], g["weight"], None, g["cu_seqlens"], g["initial_states"], "silu",
                     return_final_states=True, err_flag=flag)
    dx, dw, _, dinit = ops.bwd(g["x"], g["weight"], g["dy"], None, g["cu_seqlens"],
                               g["initial_states"], g["dfinal_states"], "silu",
                               deterministic=True, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    oy, ofin = oracle.fwd(f64(inp["x"]), f64(inp["weight"]), None, good,
                          f64(inp["initial_states"]), "silu")
    odx, odw, _, odinit = oracle.bwd(f64(inp["x"]), f64(inp["weight"]), f64(inp["dy"]), None,
                                     good, f64(inp["initial_states"]),
                                     f64(inp["dfinal_states"]), "silu")
    check_bf16("y", y, oy)
    check_exact_bf16("final_states", fin, ofin)
    check_bf16("dx", dx, odx)
    check_bf16("dinitial_states", dinit, odinit)
    check_f32_rel("dweight", dw, odw)
