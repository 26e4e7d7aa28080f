"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Tolerances:
* BF16 outputs: let o be the fp64 oracle value and r its BF16 rounding
  (nearest, ties to even, done exactly here in float64).  The GPU value g
  passes if its BF16 bit pattern is within one step of r's in the monotonic
  ordering of BF16 values, or if |g - o| <= 1e-3.
* FP32 dweight/dbias: |g - o| <= 2e-3 * max(|o|, rms(o)).
* Copies (final states, the shifted decode state) and flags: exact.
"""
import numpy as np
import torch

BF16_ABS = 1e-3
F32_REL = 2e-3


def bf16_rne(o):
    """Round float64 values to the nearest BF16 value (ties to even), exactly."""
    o = np.asarray(o, dtype=np.float64)
    out = o.copy()
    fin = np.isfinite(o) & (o != 0)
    v = o[fin]
    _, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)              # quantum: 8 significant bits, or subnormal step
    r = np.ldexp(np.round(np.ldexp(v, -q)), q)
    maxv = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > maxv, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def bf16_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().astype(np.uint16)


def bf16_ord(bits):
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_bf16(name, g, o, abs_tol=BF16_ABS):
    """g: BF16 tensor (any device/layout), o: float64 array of the same shape."""
    o = np.asarray(o, dtype=np.float64)
    assert tuple(g.shape) == o.shape, (name, tuple(g.shape), o.shape)
    gb = bf16_bits(g)
    gv = g.detach().cpu().double().numpy()
    r = bf16_rne(o)
    rb = bf16_bits(torch.from_numpy(r).to(torch.bfloat16))
    near = np.abs(bf16_ord(gb) - bf16_ord(rb)) <= 1
    close = np.abs(gv - o) <= abs_tol
    nan_ok = np.isnan(o) & np.isnan(gv)
    ok = near | close | nan_ok
    if not ok.all():
        bad = np.argwhere(~ok)
        idx = tuple(bad[0])
        raise AssertionError(
            "%s: %d of %d BF16 values out of tolerance; first at %s: gpu=%r oracle=%r rne=%r"
            % (name, len(bad), ok.size, idx, gv[idx], o[idx], r[idx]))


def check_exact_bf16(name, g, o):
    """Copies of BF16 inputs: bit-exact (o holds exactly representable values)."""
    o = np.asarray(o, dtype=np.float64)
    gv = g.detach().cpu().double().numpy()
    if not np.array_equal(gv, o):
        bad = np.argwhere(gv != o)
        idx = tuple(bad[0])
        raise AssertionError("%s: %d values differ; first at %s: gpu=%r expected=%r"
                             % (name, len(bad), idx, gv[idx], o[idx]))


def check_f32_rel(name, g, o, rel=F32_REL):
    o = np.asarray(o, dtype=np.float64)
    gv = g.detach().cpu().double().numpy()
    assert gv.shape == o.shape, (name, gv.shape, o.shape)
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    scale = np.maximum(np.abs(o), rms)
    err = np.abs(gv - o)
    ok = err <= rel * scale
    if not ok.all():
        bad = np.argwhere(~ok)
        idx = tuple(bad[0])
        raise AssertionError("%s: %d of %d values out of rel %g; first at %s: gpu=%r oracle=%r"
                             % (name, len(bad), ok.size, rel, idx, gv[idx], o[idx]))


def check_cast_bf16(name, g, o, rel=F32_REL):
    """Parameter gradients handed back in BF16: the FP32 result (held to
    check_f32_rel's bound) rounded to nearest even.  A value passes if it is
    within one BF16 step of RNE(o) in ordinal order, or if it is within the
    FP32 bound plus the cast's own rounding (half a BF16 step at g), which is
    what entries much smaller than rms(o) can need."""
    o = np.asarray(o, dtype=np.float64)
    assert tuple(g.shape) == o.shape, (name, tuple(g.shape), o.shape)
    assert g.dtype == torch.bfloat16, (name, g.dtype)
    gv = g.detach().cpu().double().numpy()
    rb = bf16_bits(torch.from_numpy(bf16_rne(o)).to(torch.bfloat16))
    near = np.abs(bf16_ord(bf16_bits(g)) - bf16_ord(rb)) <= 1
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    half_step = np.ldexp(1.0, np.frexp(np.abs(gv))[1] - 9)
    close = np.abs(gv - o) <= rel * np.maximum(np.abs(o), rms) + half_step
    ok = near | close
    if not ok.all():
        bad = np.argwhere(~ok)
        idx = tuple(bad[0])
        raise AssertionError("%s: %d of %d BF16 gradients out of tolerance; first at %s: "
                             "gpu=%r oracle=%r" % (name, len(bad), ok.size, idx, gv[idx], o[idx]))


def f64(t):
    return None if t is None else t.detach().cpu().double().numpy()


# ---- guard-banded device buffers --------------------------------------------

SENTINEL = 0x7FA5  # a BF16 NaN pattern no kernel output produces


class Guarded:
    """A device view inside a larger sentinel-filled buffer; `intact()` checks
    that nothing outside the view was written."""

    def __init__(self, storage, view):
        self.storage = storage
        self.view = view
        mask = torch.zeros(storage.shape, dtype=torch.bool, device=storage.device)
        mv = mask.as_strided(view.shape, view.stride(),
                             view.storage_offset() - storage.storage_offset())
        mv.fill_(True)
        self.mask = mask

    def intact(self):
        s = self.storage.view(torch.int16)
        outside = s[~self.mask]
        return bool((outside == np.int16(SENTINEL)).all())


def _fill(storage):
    storage.view(torch.int16).fill_(np.int16(SENTINEL))
    return storage


def guarded_act(B, D, T, layout, device, dtype=torch.bfloat16, aligned=True):
    """[B,D,T] output with the given layout ('cl' = [B,T,D] storage viewed
    through transpose, 'tc' = [B,D,T]); pads keep 16-byte alignment, unless
    `aligned` is false ('tc' only: rows then start T + 16 tokens apart)."""
    if layout == "cl":
        st = _fill(torch.empty(B, T + 2, D + 16, dtype=dtype, device=device))
        view = st[:, 1:1 + T, 8:8 + D].transpose(1, 2)
    else:
        # rows padded to a multiple of 8 tokens, so that every row starts on
        # a 16-byte boundary (the widest pieces the time lanes move)
        Tp = (T + 7) // 8 * 8 if aligned else T
        st = _fill(torch.empty(B, D + 2, Tp + 16, dtype=dtype, device=device))
        view = st[:, 1:1 + D, 8:8 + T]
    return Guarded(st, view)


def guarded_flat(shape, device, dtype=torch.bfloat16):
    n = int(np.prod(shape))
    st = _fill(torch.empty(n + 64, dtype=dtype, device=device))
    view = st[32:32 + n].view(*shape)
    return Guarded(st, view)
