"""ctypes view of the C ABI in include/ssm.h (libssm_mi355x.so).

Argument marshalling only.  If the shared library is missing this module
raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssm_mi355x.so")

SSM_F32 = 0
SSM_BF16 = 1
FLAG_DELTA_SOFTPLUS = 1
FLAG_ZOH = 2

STATUS = {
    0: "SSM_OK", 1: "SSM_ERR_NULL_ARG", 2: "SSM_ERR_BAD_SHAPE", 3: "SSM_ERR_BAD_DTYPE",
    4: "SSM_ERR_UNSUPPORTED", 5: "SSM_ERR_MISALIGNED", 6: "SSM_ERR_WORKSPACE",
    7: "SSM_ERR_HIP",
}

# exported symbol -> (restype, argtypes)
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_u = ctypes.c_uint
_i = ctypes.c_int
SIGNATURES = {
    "ssm_abi_version": (_i, []),
    "ssm_status_string": (ctypes.c_char_p, [_i]),
    "ssm_selective_scan_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i]),
    "ssm_selective_scan_segments": (_i, [_i64, _i64, _i64, _i64]),
    "ssm_selective_scan_lanes": (_i, [_i64, _i64, _i64, _i64]),
    "ssm_selective_scan_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _u, _vp, _vp, _vp,
                                    _i64, _i64, _i64, _i64, _i, _vp, _sz, _vp]),
    "ssm_selective_scan_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _u, _vp, _vp,
                                           _vp, _vp, _i64, _i64, _i64, _i64, _i, _vp, _sz, _vp]),
    "ssm_selective_scan_fwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _u, _vp, _vp,
                                            _vp, _i64, _i64, _i64, _i64, _i, _vp]),
    "ssm_selective_scan_fwd_timed": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _u, _vp, _vp, _vp,
                                          _i64, _i64, _i64, _i64, _i, _vp, _sz, _vp, _vp]),
    "ssm_selective_scan_conv_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _vp, _vp, _u, _vp, _vp, _vp, _i64, _i64, _i64,
                                         _i64, _i, _vp, _sz, _vp]),
    "ssm_ssd_chunk_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64, _i64, _i]),
    "ssm_ssd_chunk_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _u, _vp, _vp, _vp,
                               _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i, _vp, _sz, _vp]),
    "ssm_ssd_chunk_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _u, _vp, _vp, _vp,
                                      _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i, _vp,
                                      _sz, _vp]),
    "ssm_selective_scan_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i]),
    "ssm_selective_scan_bwd": (_i, [_vp] * 21 + [_i64, _i64, _i64, _i64, _i, _vp, _sz, _vp]),
    "ssm_selective_scan_bwd_segments": (_i, [_i64, _i64, _i64, _i64]),
    "ssm_selective_scan_bwd_varlen": (_i, [_vp] * 8 + [_u] + [_vp] * 13 +
                                      [_i64, _i64, _i64, _i64, _i, _vp, _sz, _vp]),
    "ssm_selective_scan_ckpt_bytes": (_sz, [_i64, _i64, _i64, _i64, _i]),
    "ssm_selective_scan_fwd_ckpt": (_i, [_vp] * 8 + [_u] + [_vp] * 4 +
                                    [_i64, _i64, _i64, _i64, _i, _vp, _sz, _vp]),
    "ssm_selective_scan_bwd_ckpt_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i]),
    "ssm_selective_scan_bwd_ckpt": (_i, [_vp] * 8 + [_u] + [_vp] * 13 +
                                    [_i64, _i64, _i64, _i64, _i, _vp, _sz, _vp]),
    "ssm_causal_conv1d_silu": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _vp, _i64, _i64, _i64, _i64,
                                    _i, _vp]),
    "ssm_selective_state_update": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _u, _vp,
                                        _i64, _i64, _i64, _i, _vp]),
}

_lock = threading.Lock()
_lib = None


class SSMError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


def load():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m selective_state_space_21_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().ssm_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != 0:
        raise SSMError(status, what)
