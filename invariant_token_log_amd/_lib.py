"""ctypes loader of the in-tree HIP library (libinvariant_logp.so).

The product path has no fallback: if the library is missing or fails to load,
every call raises.  Build it with ``python -m invariant_token_log_amd.build``.
"""

import ctypes
import os

from .build import LIB_PATH

LOGP_OK = 0
LOGP_ERR_NULL = 1
LOGP_ERR_SHAPE = 2
LOGP_ERR_DTYPE = 3
LOGP_ERR_TILE = 4
LOGP_ERR_ALIGN = 5
LOGP_ERR_SHARDS = 6
LOGP_ERR_WORKSPACE = 7
LOGP_ERR_TARGET = 8
LOGP_ERR_HIP = 9
LOGP_ERR_VALUE = 10
LOGP_ERR_SCRATCH = 11
NOALLOC_SCRATCH_BYTES = 64 << 20  # LOGP_NOALLOC_SCRATCH_BYTES

LOGP_F32 = 0
LOGP_BF16 = 1
LOGP_F16 = 2

LOGP_I64 = 0
LOGP_I32 = 1
LOGP_ROUND_NONE = 0
LOGP_ROUND_BF16 = 1

LOGP_BWD_DHIDDEN = 1
LOGP_BWD_DWEIGHT = 2
LOGP_BWD_PREPARED = 4
LOGP_BWD_SAVED_LOGITS = 8
LOGP_BWD_BF16_OUT = 16

_i32, _i64, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
_f32 = ctypes.c_float

_SIGNATURES = {
    "logp_fwd_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32, _i32]),
    "logp_fwd": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _i32, _i64, _i32, _i32, _i32,
                        _vp, _vp, _vp, _vp, _sz, _vp]),
    "logp_bwd": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _i32, _i64, _i32, _vp, _vp,
                        _vp, _vp, _vp, _i64, _vp]),
    "linear_logp_fwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "linear_logp_fwd": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _i32, _i64,
                               _i32, _f32, _i32, _vp, _vp, _vp, _vp, _i32, _i64, _vp, _sz,
                               _vp, _sz, _vp]),
    "linear_logp_fwd_noalloc": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _i32, _i64,
                                       _i32, _f32, _i32, _vp, _vp, _vp, _vp, _i32, _i64, _vp,
                                       _sz, _vp]),
    "linear_logp_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32, _i64]),
    "linear_logp_bwd": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _i32, _i64,
                               _i32, _f32, _i32, _vp, _i32, _i64, _vp, _sz, _vp, _vp, _vp, _vp,
                               _i32, _vp, _i64, _vp, _i64, _i64, _vp, _sz, _vp]),
    "linear_logp_prepared_bytes": (_sz, [_i64, _i64]),
    "linear_logp_prepare_weight": (_i32, [_vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "logp_status_str": (ctypes.c_char_p, [_i32]),
    "logp_contract_id": (ctypes.c_char_p, []),
}

_lib = None


class LogpError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {status_str(status)} (status {status})")


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m invariant_token_log_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status):
    return lib().logp_status_str(int(status)).decode()


def contract_id():
    return lib().logp_contract_id().decode()


def check(fn, status):
    if status != LOGP_OK:
        raise LogpError(fn, status)
