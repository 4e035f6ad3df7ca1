"""ctypes loader for libattnfwd.so.

The binding never falls back to anything else: if the library is missing or
fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattnfwd.so")

c_void_p = ctypes.c_void_p
c_int32 = ctypes.c_int32
c_int64 = ctypes.c_int64
c_float = ctypes.c_float

# name -> (restype, argtypes); mirrors include/attn_fwd.h
SIGNATURES = {
    "attn_fwd_varlen": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                  c_int32, c_float, c_int32, c_void_p, c_void_p, c_void_p]),
    "attn_fwd_dense": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                 c_int32, c_int32, c_int32, c_void_p, c_float, c_int32,
                                 c_void_p, c_void_p, c_void_p]),
    "attn_fwd_varlen_ws": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                     c_int32, c_float, c_int32, c_void_p, c_void_p, c_void_p,
                                     c_int64, c_void_p]),
    "attn_fwd_dense_ws": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                    c_int32, c_int32, c_int32, c_void_p, c_float, c_int32,
                                    c_void_p, c_void_p, c_void_p, c_int64, c_void_p]),
    "attn_fwd_workspace_bytes": (c_int64, [c_int32, c_int32, c_int32, c_int32, c_int32]),
    "attn_fwd_padded": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                  c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                  c_float, c_int32, c_void_p, c_void_p, c_void_p]),
    "attn_unpad_gather": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_int32,
                                    c_int64, c_void_p]),
    "attn_pad_scatter": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int64,
                                   c_void_p]),
    "attn_bwd_varlen": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                  c_int32, c_int32, c_int32, c_int32, c_float, c_int32,
                                  c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_void_p]),
    "attn_bwd_dense": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_float,
                                 c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                 c_void_p]),
    "attn_bwd_workspace_bytes": (c_int64, [c_int64, c_int32]),
    "attn_fwd_paged": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                 c_int32, c_int32, c_int32, c_float, c_int32, c_void_p, c_void_p,
                                 c_void_p, c_int64, c_void_p]),
    "attn_fwd_paged_fp8kv": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                       c_int32, c_int32, c_int32, c_int32, c_int32, c_float,
                                       c_float, c_float, c_int32, c_void_p, c_void_p, c_void_p,
                                       c_int64, c_void_p]),
    "attn_fwd_paged_noalloc": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                         c_int32, c_int32, c_int32, c_int32, c_int32, c_float,
                                         c_int32, c_void_p, c_void_p, c_void_p]),
    "attn_fwd_paged_workspace_bytes": (c_int64, [c_int32, c_int32, c_int32, c_int32, c_int32,
                                                 c_int32]),
    "attn_mask_to_varlen": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                      c_void_p]),
    "attn_fwd_fp8_varlen": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                      c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                      c_float, c_float, c_float, c_float, c_int32, c_void_p,
                                      c_void_p, c_void_p]),
    "attn_fwd_fp8_dense": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                     c_int32, c_int32, c_int32, c_float, c_float, c_float, c_float,
                                     c_int32, c_void_p, c_void_p, c_void_p]),
    "attn_fwd_launch_plan": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                       c_int32, c_int64, c_void_p]),
    "attn_fwd_tile_policy_compiled": (c_int32, [c_int32, c_int32]),
    "attn_status_str": (ctypes.c_char_p, [c_int32]),
    "attn_abi_version": (c_int32, []),
}

STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
          4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_HIP", 6: "ATTN_ERR_SCRATCH"}

_lib = None


def load() -> ctypes.CDLL:
    """Loads the library once and declares every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m tiled_attention_fwd_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load()
        text = lib.attn_status_str(status).decode()
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != 0:
        raise AttnError(fn, status)
