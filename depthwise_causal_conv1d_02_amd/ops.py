"""Python surface of the depthwise causal conv1d (cuDNN FE "Causal Conv1d":
``causal_conv1d`` and ``causal_conv1d_update``), over the C-ABI of libccv.

PyTorch supplies device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  Tensors must live on a ROCm
device: there is no CPU path.
"""
import ctypes
import warnings

import torch

from . import _abi

__all__ = ["causal_conv1d", "causal_conv1d_update", "validate_cu_seqlens", "check_flag",
           "reset_flag", "flag_tensor", "fwd", "bwd", "bwd_noalloc", "update", "CcvError"]

_DTYPES = {torch.bfloat16: _abi.CCV_DTYPE_BF16, torch.float32: _abi.CCV_DTYPE_F32,
           torch.int32: _abi.CCV_DTYPE_I32}


class CcvError(RuntimeError):
    pass


def _desc(t):
    """ccv_tensor for a device tensor, or None for an absent one."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor, got %r" % type(t))
    if t.device.type != "cuda":
        raise ValueError("libccv runs on the GPU only; got a tensor on %s" % t.device)
    if t.dtype not in _DTYPES:
        raise ValueError("unsupported dtype %s" % t.dtype)
    if t.dim() > 3 or t.dim() < 1:
        raise ValueError("tensors of rank 1..3 only")
    d = _abi.CcvTensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ref(d):
    return None if d is None else ctypes.byref(d)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _act(activation):
    if activation is None or activation == "none":
        return _abi.CCV_ACT_NONE
    if activation == "silu":
        return _abi.CCV_ACT_SILU
    raise NotImplementedError("activation must be None or 'silu'")


def _check(rc, what):
    if rc == _abi.CCV_OK:
        return
    if rc == _abi.CCV_WARN_NONDETERMINISTIC:
        warnings.warn("%s: no deterministic dbias route; ran with FP32 atomics" % what,
                      UserWarning, stacklevel=3)
        return
    name = _abi.status_name(rc)
    if rc in (_abi.CCV_ERR_INVALID_ARG, _abi.CCV_ERR_ALIAS):
        raise ValueError("%s: %s" % (what, name))
    if rc == _abi.CCV_ERR_TOO_LARGE:
        raise ValueError("%s: %s: the deterministic partials of this call exceed the library's "
                         "%d-byte device scratch; use the workspace form"
                         % (what, name, _abi.NOALLOC_SCRATCH_BYTES))
    if rc == _abi.CCV_ERR_UNSUPPORTED:
        raise NotImplementedError("%s: %s (declined)" % (what, name))
    if rc == _abi.CCV_ERR_NONDETERMINISTIC:
        raise RuntimeError("%s: %s: deterministic algorithms are enabled and this call has a "
                           "bias, which has no deterministic dbias route" % (what, name))
    raise CcvError("%s: %s" % (what, name))


# ---- the sticky cu_seqlens flag word (one per device) ----------------------

_flags = {}


def flag_tensor(device=None):
    """The device's flag word that packed calls OR their violation bits into."""
    dev = torch.device("cuda", torch.cuda.current_device() if device is None
                       else torch.device(device).index or 0)
    t = _flags.get(dev.index)
    if t is None:
        t = torch.zeros(1, dtype=torch.int32, device=dev)
        _flags[dev.index] = t
    return t


def check_flag(device=None):
    """Synchronise and raise ValueError if malformed cu_seqlens were seen on
    this device.  The flag stays set (packed calls then write nothing) until
    reset_flag()."""
    v = int(flag_tensor(device).item()) & 0xffffffff
    if v:
        names = [n for b, n in _abi.CU_BIT_NAMES.items() if v & b]
        raise ValueError("malformed cu_seqlens: " + ", ".join(names))


def reset_flag(device=None):
    flag_tensor(device).zero_()


def validate_cu_seqlens(cu_seqlens, total_tokens):
    """Device-side check; returns a device int32 tensor [1] holding the bits."""
    out = torch.empty(1, dtype=torch.int32, device=cu_seqlens.device)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector")
    rc = _abi.lib().ccv_validate_cu_seqlens(cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                                            int(total_tokens), out.data_ptr(), _stream(out))
    _check(rc, "validate_cu_seqlens")
    return out


# ---- raw calls (no autograd) ------------------------------------------------

def _rows(x, cu_seqlens):
    return x.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1


def _options(fp32_weight_bias=False, deterministic_dbias=False):
    return ((_abi.CCV_OPT_F32_FILTER_BIAS if fp32_weight_bias else 0) |
            (_abi.CCV_OPT_DETERMINISTIC_DBIAS if deterministic_dbias else 0))


def fwd(x, weight, bias=None, cu_seqlens=None, initial_states=None, activation="silu",
        return_final_states=False, final_states_out=None, y=None, err_flag=None, seq_idx=None,
        options=0):
    """One ccv_fwd call.  Returns (y, final_states or None)."""
    if y is None:
        y = torch.empty_like(x)
    fin = final_states_out
    if fin is None and return_final_states:
        fin = torch.empty(_rows(x, cu_seqlens), x.shape[1], weight.shape[1] - 1, dtype=x.dtype,
                          device=x.device)
    flag = None
    if cu_seqlens is not None:
        flag = err_flag if err_flag is not None else flag_tensor(x.device)
    rc = _abi.lib().ccv_fwd(_ref(_desc(x)), _ref(_desc(weight)), _ref(_desc(bias)),
                            _ref(_desc(cu_seqlens)), _ref(_desc(seq_idx)),
                            _ref(_desc(initial_states)), _ref(_desc(y)), _ref(_desc(fin)),
                            _act(activation), int(options),
                            None if flag is None else flag.data_ptr(), _stream(x))
    _check(rc, "causal_conv1d")
    return y, fin


def bwd(x, weight, dy, bias=None, cu_seqlens=None, initial_states=None, dfinal_states=None,
        activation="silu", deterministic=False, warn_only=False, dx=None, err_flag=None,
        want_dinit=True, seq_idx=None, workspace=None, dweight=None, dbias=None, dinit=None,
        options=0):
    """One ccv_bwd call.  Returns (dx, dweight_f32, dbias_f32 or None,
    dinitial_states or None).  ``dweight``/``dbias`` (FP32) are accumulated
    into when given, else freshly zeroed ones are used."""
    if dx is None:
        dx = torch.empty_like(x)
    D, W = weight.shape
    dw = dweight if dweight is not None else torch.zeros(D, W, dtype=torch.float32,
                                                          device=x.device)
    db = None
    if bias is not None:
        db = dbias if dbias is not None else torch.zeros(D, dtype=torch.float32, device=x.device)
    if dinit is None and initial_states is not None and want_dinit:
        dinit = torch.empty_like(initial_states)
    flag = None
    if cu_seqlens is not None:
        flag = err_flag if err_flag is not None else flag_tensor(x.device)
    L = _abi.lib()
    args_head = (_ref(_desc(x)), _ref(_desc(weight)), _ref(_desc(bias)), _ref(_desc(cu_seqlens)),
                 _ref(_desc(seq_idx)), _ref(_desc(initial_states)), _ref(_desc(dy)),
                 _ref(_desc(dfinal_states)), _ref(_desc(dx)), _ref(_desc(dw)), _ref(_desc(db)),
                 _ref(_desc(dinit)), _act(activation), int(bool(deterministic)),
                 int(bool(warn_only)), int(options))
    flag_ptr = None if flag is None else flag.data_ptr()
    need = ctypes.c_size_t(0)
    rc = L.ccv_bwd(*args_head, None, ctypes.byref(need), flag_ptr, _stream(x))
    _check(rc, "causal_conv1d backward")
    ws = None
    if need.value:
        ws = workspace if (workspace is not None and workspace.numel() >= need.value) else \
            torch.empty(need.value, dtype=torch.uint8, device=x.device)
    size = ctypes.c_size_t(0 if ws is None else ws.numel())
    rc = L.ccv_bwd(*args_head, None if ws is None else ws.data_ptr(),
                   None if ws is None else ctypes.byref(size), flag_ptr, _stream(x))
    _check(rc, "causal_conv1d backward")
    return dx, dw, db, dinit


def bwd_noalloc(x, weight, dy, bias=None, cu_seqlens=None, initial_states=None,
                dfinal_states=None, activation="silu", deterministic=False, warn_only=False, *,
                dx, dweight, dbias=None, dinit=None, err_flag=None, seq_idx=None, options=0):
    """One ccv_bwd_noalloc call: ccv_bwd with the deterministic partials in the
    library's fixed device scratch, so nothing is allocated here or in the
    library.  Every output is the caller's: dx, dweight (FP32, accumulated
    into), dbias when a bias is given, dinit when wanted; packed calls need
    ``err_flag``.  Calls that overlap on one device race (shared scratch)."""
    if cu_seqlens is not None and err_flag is None:
        raise ValueError("packed calls need err_flag (no flag word is allocated here)")
    rc = _abi.lib().ccv_bwd_noalloc(
        _ref(_desc(x)), _ref(_desc(weight)), _ref(_desc(bias)), _ref(_desc(cu_seqlens)),
        _ref(_desc(seq_idx)), _ref(_desc(initial_states)), _ref(_desc(dy)),
        _ref(_desc(dfinal_states)), _ref(_desc(dx)), _ref(_desc(dweight)), _ref(_desc(dbias)),
        _ref(_desc(dinit)), _act(activation), int(bool(deterministic)), int(bool(warn_only)),
        int(options), None if err_flag is None else err_flag.data_ptr(), _stream(x))
    _check(rc, "causal_conv1d backward (no allocation)")
    return dx, dweight, dbias, dinit


def update(x, conv_state, weight, bias=None, activation="silu", y=None, options=0):
    """One ccv_update call (conv_state is mutated in place).  x is [B,D] (one
    token) or [B,D,L] (L tokens in order).  Returns y (x's shape)."""
    if y is None:
        y = torch.empty_like(x)
    rc = _abi.lib().ccv_update(_ref(_desc(x)), _ref(_desc(conv_state)), _ref(_desc(weight)),
                               _ref(_desc(bias)), _ref(_desc(y)), _act(activation), int(options),
                               _stream(x))
    _check(rc, "causal_conv1d_update")
    return y


# ---- autograd ----------------------------------------------------------------

class _CausalConv1dFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, bias, seq_idx, cu_seqlens, initial_states, final_states_out,
                activation, return_final_states, deterministic, options):
        y, fin = fwd(x, weight, bias, cu_seqlens, initial_states, activation,
                     return_final_states, final_states_out, seq_idx=seq_idx, options=options)
        # Inputs are saved for backward; the final state is written after the
        # forward (cuDNN FE "Causal Conv1d", the aliasing paragraph).
        ctx.save_for_backward(x, weight, bias, seq_idx, cu_seqlens, initial_states)
        ctx.activation = activation
        ctx.deterministic = deterministic
        ctx.options = options
        ctx.has_fin = fin is not None
        if final_states_out is not None:
            ctx.mark_dirty(final_states_out)
        return y, fin

    @staticmethod
    def backward(ctx, dy, dfin):
        x, weight, bias, seq_idx, cu_seqlens, init = ctx.saved_tensors
        if dy is None:
            dy = torch.zeros_like(x)
        elif dy.stride() != x.stride():
            # The kernels read any layout, but match x's for the fast path.
            dy = torch.empty_like(x).copy_(dy)
        det = ctx.deterministic
        if det is None:
            det = torch.are_deterministic_algorithms_enabled()
        warn_only = torch.is_deterministic_algorithms_warn_only_enabled()
        need_dinit = init is not None and ctx.needs_input_grad[5]
        dx, dw, db, dinit = bwd(x, weight, dy, bias, cu_seqlens, init,
                                dfin if ctx.has_fin else None, ctx.activation, det, warn_only,
                                want_dinit=need_dinit, seq_idx=seq_idx, options=ctx.options)
        return (dx, dw.to(weight.dtype), None if db is None else db.to(bias.dtype), None, None,
                dinit, None, None, None, None, None)


def causal_conv1d(x, weight, bias=None, seq_idx=None, cu_seqlens=None, initial_states=None,
                  return_final_states=False, final_states_out=None, activation=None,
                  deterministic=None, fp32_weight_bias=False, deterministic_dbias=False):
    """y = act(bias + depthwise causal conv of x with weight), x [B,D,T].

    ``x`` may be a [B,T,D] storage seen through ``transpose(1, 2)``; it is
    consumed as is.  ``cu_seqlens`` packs N sequences along T of a B == 1
    input; their metadata is validated on the device and malformed offsets
    set the device flag (see :func:`check_flag`) instead of trapping.
    Returns ``y`` or ``(y, final_states)``.

    ``seq_idx`` [B,T] (int32) gives each token the id of its sequence: a tap
    contributes only when its token has the output token's id.  It excludes
    ``cu_seqlens`` and the state tensors.

    Two opt-ins widen what the pages' route declines: ``fp32_weight_bias``
    admits an FP32 weight with an FP32 bias, and ``deterministic_dbias``
    lets a deterministic backward with a bias reduce dbias in a fixed order
    instead of failing (or warning and using atomics).
    """
    if seq_idx is not None and cu_seqlens is not None:
        raise ValueError("seq_idx and cu_seqlens are mutually exclusive")
    if final_states_out is not None:
        return_final_states = True
    needs_grad = torch.is_grad_enabled() and any(
        t is not None and t.requires_grad for t in (x, weight, bias, initial_states))
    opts = _options(fp32_weight_bias, deterministic_dbias)
    if needs_grad:
        y, fin = _CausalConv1dFn.apply(x, weight, bias, seq_idx, cu_seqlens, initial_states,
                                       final_states_out, activation, return_final_states,
                                       deterministic, opts)
    else:
        y, fin = fwd(x, weight, bias, cu_seqlens, initial_states, activation,
                     return_final_states, final_states_out, seq_idx=seq_idx, options=opts)
    return (y, fin) if return_final_states else y


def causal_conv1d_update(x, conv_state, weight, bias=None, activation=None,
                         fp32_weight_bias=False):
    """Decode: x [B,D] (one token) or [B,D,L] (L tokens in order);
    conv_state [B,D,W-1] is mutated in place (it becomes the last W-1
    tokens).  Returns y with x's shape."""
    return update(x, conv_state, weight, bias, activation,
                  options=_options(fp32_weight_bias))
