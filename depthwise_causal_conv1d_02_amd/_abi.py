"""ctypes view of libccv.so (include/ccv.h): descriptors, prototypes, status codes.

Argument marshalling only.  The library must be built (python -m
depthwise_causal_conv1d_02_amd.build); there is no fallback of any kind.
"""
import ctypes
import os
import threading

ABI_VERSION = 3  # CCV_ABI_VERSION of include/ccv.h
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libccv.so")

CCV_DTYPE_BF16, CCV_DTYPE_F32, CCV_DTYPE_I32 = 0, 1, 2
CCV_ACT_NONE, CCV_ACT_SILU = 0, 1

CCV_OK = 0
CCV_WARN_NONDETERMINISTIC = 1
CCV_ERR_INVALID_ARG = -1
CCV_ERR_ALIAS = -2
CCV_ERR_UNSUPPORTED = -3
CCV_ERR_NONDETERMINISTIC = -4
CCV_ERR_HIP = -5
CCV_ERR_TOO_LARGE = -6

NOALLOC_SCRATCH_BYTES = 32 << 20   # CCV_NOALLOC_SCRATCH_BYTES

# option bits of ccv_fwd / ccv_bwd / ccv_update
CCV_OPT_F32_FILTER_BIAS, CCV_OPT_DETERMINISTIC_DBIAS = 0x1, 0x2

CU_FIRST_NONZERO, CU_LAST_MISMATCH, CU_DECREASING, CU_EMPTY = 0x1, 0x2, 0x4, 0x8
CU_BIT_NAMES = {CU_FIRST_NONZERO: "first offset is not zero",
                CU_LAST_MISMATCH: "last offset is not the token total",
                CU_DECREASING: "offsets decrease",
                CU_EMPTY: "empty sequence"}

EXPORTS = ("ccv_fwd", "ccv_bwd", "ccv_bwd_noalloc", "ccv_update", "ccv_validate_cu_seqlens",
           "ccv_abi_version", "ccv_status_string")


class CcvTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 3), ("stride", ctypes.c_int64 * 3)]


P = ctypes.POINTER(CcvTensor)
_vp = ctypes.c_void_p
_lock = threading.Lock()
_lib = None


class LibraryMissing(RuntimeError):
    pass


def _declare(lib):
    i, u32, sz = ctypes.c_int, ctypes.c_uint32, ctypes.POINTER(ctypes.c_size_t)
    lib.ccv_fwd.argtypes = [P, P, P, P, P, P, P, P, i, u32, _vp, _vp]
    lib.ccv_fwd.restype = i
    lib.ccv_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, i, i, i, u32, _vp, sz, _vp, _vp]
    lib.ccv_bwd.restype = i
    lib.ccv_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, i, i, i, u32, _vp, _vp]
    lib.ccv_bwd_noalloc.restype = i
    lib.ccv_update.argtypes = [P, P, P, P, P, i, u32, _vp]
    lib.ccv_update.restype = i
    lib.ccv_validate_cu_seqlens.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64, _vp, _vp]
    lib.ccv_validate_cu_seqlens.restype = i
    lib.ccv_abi_version.argtypes = []
    lib.ccv_abi_version.restype = i
    lib.ccv_status_string.argtypes = [i]
    lib.ccv_status_string.restype = ctypes.c_char_p


def lib(path=None):
    """The loaded library; raises LibraryMissing when it was never built."""
    global _lib
    if path is not None:
        l = ctypes.CDLL(path)
        _declare(l)
        return l
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise LibraryMissing(
                    "libccv.so is not built (%s); run `python -m depthwise_causal_conv1d_02_amd.build`"
                    % LIB_PATH)
            l = ctypes.CDLL(LIB_PATH)
            _declare(l)
            if l.ccv_abi_version() != ABI_VERSION:
                raise LibraryMissing("libccv.so ABI version mismatch")
            _lib = l
    return _lib


def status_name(rc):
    return lib().ccv_status_string(int(rc)).decode()
