"""ctypes view of libbd.so, the C ABI declared in include/bd.h.

Loading fails loudly: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# BD_LIBRARY may name another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("BD_LIBRARY") or os.path.join(_HERE, "libbd.so")

BD_OK, BD_ERR_NULL, BD_ERR_SHAPE, BD_ERR_UNSUPPORTED, BD_ERR_WORKSPACE, BD_ERR_VALUE, BD_ERR_HIP, \
    BD_ERR_ALIGNMENT, BD_ERR_SCRATCH = range(9)
BD_NOALLOC_SCRATCH_BYTES = 4 << 20   # include/bd.h
BD_F32, BD_BF16 = 0, 1
BD_FALLBACK_NONE, BD_FALLBACK_TOP1 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m block_diffusion_decoding_amd.build` "
                      "(the HIP library is required; there is no fallback path)")

lib = ctypes.CDLL(LIB_PATH)

_p, _i, _f, _sz, _i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_int64
_u64 = ctypes.c_uint64

_SIGS = {
    "bd_status_string": (ctypes.c_char_p, [_i]),
    "bd_last_hip_error": (_i, []),
    "bd_version": (_i, []),
    "bd_attn_fwd": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p]),
    "bd_attn_bwd_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "bd_attn_bwd": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _i, _i, _i, _i, _i, _i, _f, _i, _p]),
    "bd_attn_decode_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "bd_attn_decode_block": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p, _sz,
                                  _p]),
    "bd_confidence_commit_workspace_size": (_sz, [_i, _i, _i]),
    "bd_confidence_commit": (_i, [_p, _i64, _i, _i, _i, _i, _f, _i, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "bd_confidence_commit_noalloc": (_i, [_p, _i64, _i, _i, _i, _i, _f, _i, _p, _p, _p, _p, _p, _p, _p]),
    "bd_confidence_commit_rowwise": (_i, [_p, _i64, _i, _i, _i, _i, _p, _i, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "bd_attn_decode_block_paged": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _p, _i, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p,
                                        _sz, _p]),
    "bd_kv_append_block": (_i, [_p, _p, _p, _p, _p, _i, _i, _p, _p, _i, _i, _i, _i, _i, _p]),
    "bd_confidence_commit_sampled_workspace_size": (_sz, [_i, _i, _i]),
    "bd_confidence_commit_sampled": (_i, [_p, _i64, _i, _i, _i, _i, _f, _u64, _u64, _i, _f, _f, _i, _p, _p, _p, _p,
                                         _p, _p, _p, _sz, _p]),
    "bd_lmhead_commit_workspace_size": (_sz, [_i, _i, _i]),
    "bd_lmhead_commit": (_i, [_p, _i64, _p, _i64, _i, _i, _i, _i, _f, _i, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
}

EXPORTS = tuple(_SIGS)

for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class BdError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.bd_status_string(status).decode()
        if status == BD_ERR_HIP:
            msg += f" (hipError_t {lib.bd_last_hip_error()})"
        super().__init__(f"{where}: {msg} [status {status}]")
        self.status = status


def check(status: int, where: str) -> None:
    if status != BD_OK:
        raise BdError(status, where)
