"""ctypes loader for the in-tree HIP library (``lib/libmoe_mi355x.so``).

Fails loudly when the library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmoe_mi355x.so")

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/moe.h and include/moe_calib.h
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_INT]),
    "moe_version": (_INT, []),
    "moe_capacity": (_INT, [_I64, _I64, _I32, _I64, _I32, ctypes.POINTER(_I64)]),
    "moe_workspace_bytes": (_INT, [_INT, _I64, _I32, _I32, _I32, _I32, _I64, ctypes.POINTER(_SZ)]),
    "moe_router_topk": (_INT, [_P, _INT, _I64, _I32, _P, _P, _P, _I32, _I32, _P, _F32, _F32, _P, _P, _P,
                               _P, _P, _SZ, _P]),
    "moe_mlp_router_topk": (_INT, [_P, _INT, _I64, _I32, _P, _P, _I32, _P, _P, _P, _I32, _I32, _P, _F32,
                                   _F32, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_dispatch": (_INT, [_P, _I64, _I32, _I32, _I64, _P, _INT, _I32, _P, _P, _P, _P, _P, _P, _P,
                            _SZ, _P]),
    "moe_route": (_INT, [_P, _INT, _I64, _I32, _P, _P, _P, _I32, _I32, _P, _F32, _F32, _I64, _F32, _F32]
                  + [_P] * 12 + [_P, _SZ, _P]),
    "moe_route_noalloc": (_INT, [_P, _INT, _I64, _I32, _P, _P, _P, _I32, _I32, _P, _F32, _F32, _I64, _F32, _F32]
                          + [_P] * 12 + [_P]),
    "moe_grouped_ffn": (_INT, [_P, _P, _P, _I32, _I64, _I32, _I32, _I32, _INT, _INT, _P, _P, _P, _P,
                               _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_up": (_INT, [_P, _P, _P, _I32, _I64, _I32, _I32, _INT, _INT, _P, _P, _P, _P, _P, _SZ,
                             _P]),
    "moe_expert_down": (_INT, [_P, _P, _I32, _I64, _I32, _I32, _INT, _P, _P, _P, _P]),
    "moe_shared_ffn": (_INT, [_P, _I64, _I32, _I32, _I32, _I32, _INT, _INT, _P, _P, _P, _P, _P, _P,
                              _P]),
    "moe_combine": (_INT, [_P, _P, _P, _P, _I64, _I32, _I32, _INT, _P, _P]),
    "moe_route_stats": (_INT, [_P, _P, _P, _P, _P, _I64, _I32, _I32, _F32, _F32, _P, _P, _P, _P, _P,
                               _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_balance_losses": (_INT, [_P, _P, _P, _P, _I64, _I32, _I32, _F32, _F32, _P, _P, _P, _SZ, _P]),
    "moe_selection_bias_update": (_INT, [_P, _I32, _I32, _I64, _F32, _P, _P]),
    "moe_dro_update": (_INT, [_P, _I32, _F32, _F32, _P, _P, _P, _P]),
    # measurement support (include/moe_calib.h)
    "moe_calib_copy": (_INT, [_P, _P, _SZ, _P]),
    "moe_calib_read": (_INT, [_P, _SZ, _P, _P]),
    "moe_calib_mfma": (_INT, [_I32, _I32, _P, ctypes.POINTER(ctypes.c_double), _P]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not found at {LIB_PATH}; build it with "
                "`python -m sparse_mixture_experts_10_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
