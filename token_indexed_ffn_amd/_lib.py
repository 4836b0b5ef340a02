"""ctypes loader of libstaple.so.

torch is imported first on purpose: libstaple.so then binds to the HIP runtime
torch has already loaded, so torch's streams and device pointers are valid in
the library.  There is no fallback: when the library is missing every call
fails with a RuntimeError that says how to build it.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libstaple.so")

c_i32, c_i64, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
c_f32 = ctypes.c_float

# name -> (restype, argtypes)
_SIGS = {
    "staple_status_string": (ctypes.c_char_p, [c_i32]),
    "staple_version": (ctypes.c_char_p, []),
    "staple_get_device_error": (c_i32, [c_vp]),
    "staple_dedup_workspace_bytes": (c_sz, [c_i64]),
    "staple_dedup": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "staple_cache_count": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_vp]),
    "staple_cache_build_workspace_bytes": (c_sz, [c_i64]),
    "staple_cache_build": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "staple_cache_fill": (c_i32, [c_vp, c_i64, c_i64, c_i32, c_vp, c_i64, c_vp, c_vp]),
    "staple_cache_lookup": (c_i32, [c_vp, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "staple_split_tokens": (c_i32, [c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "staple_stage_misses": (c_i32, [c_vp, c_i64, c_i64, c_i32, c_vp, c_i32, c_vp, c_vp, c_vp]),
    "staple_stage_misses_dma": (c_i32, [c_i64, c_vp, c_i64, c_i64, c_i64, c_i32, c_vp, c_i32, c_vp,
                                        c_vp]),
    "staple_assemble_rows": (c_i32, [c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_i64, c_i32,
                                     c_vp, c_vp]),
    "staple_assemble_rows_from_table": (c_i32, [c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp, c_i64,
                                                c_i64, c_i32, c_vp, c_vp]),
    "staple_gather_rows": (c_i32, [c_vp, c_i64, c_vp, c_vp, c_i64, c_i64, c_i32, c_vp, c_vp]),
    "staple_ffn_fwd_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i32]),
    "staple_ffn_fwd": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                               c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "staple_ffn_gate_up": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp,
                                   c_vp, c_vp, c_vp, c_vp]),
    "staple_ffn_gate_up_tokens": (c_i32, [c_i64, c_vp, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp,
                                          c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "staple_ffn_down_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i32]),
    "staple_ffn_down": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz,
                                c_vp]),
    "staple_decode_pack_weights": (c_i32, [c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "staple_ffn_gate_up_packed": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_i32, c_vp,
                                          c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "staple_ffn_down_packed": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp,
                                       c_sz, c_vp]),
    "staple_ffn_fwd_packed": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp, c_i32, c_vp,
                                      c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                                      c_vp]),
    "staple_ffn_fwd_packed_noalloc": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp, c_i32,
                                              c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                              c_vp]),
    "staple_decode_step_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64]),
    "staple_decode_step_cached": (c_i32, [c_i64, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_vp,
                                          c_i64, c_vp, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                          c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "staple_group_tables_host": (c_i32, [c_vp, c_i64, c_i64, c_i64, c_i32, c_vp]),
    "staple_prefill_rows_workspace_bytes": (c_sz, [c_i64]),
    "staple_prefill_rows_cached": (c_i32, [c_i64, c_vp, c_i64, c_i64, c_i32, c_vp, c_i64, c_vp,
                                           c_i64, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                           c_vp, c_vp, c_vp, c_sz, c_vp]),
    "staple_lowrank_expand": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp]),
    "staple_lowrank_bwd_workspace_bytes": (c_sz, [c_i64, c_i64, c_i32]),
    "staple_lowrank_bwd": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp,
                                   c_vp, c_sz, c_vp]),
    "staple_adamw_rows": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i32, c_vp, c_vp, c_i64, c_vp,
                                  c_f32, c_f32, c_f32, c_f32, c_f32, c_i64, c_vp]),
    "staple_adamw_rows_host": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i32, c_vp, c_i64, c_vp,
                                       c_f32, c_f32, c_f32, c_f32, c_f32, c_i64, c_i32]),
    "staple_cache_refresh": (c_i32, [c_vp, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_i64, c_vp, c_i64,
                                     c_vp]),
    "staple_ffn_bwd_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i32]),
    "staple_ffn_bwd_table_grad": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp, c_vp,
                                          c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                          c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_sz,
                                          c_vp, c_vp]),
    "staple_host_adamw_create": (c_i32, [c_i64, c_i64, c_vp]),
    "staple_host_adamw_event": (c_vp, [c_vp]),
    "staple_host_adamw_start": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_vp, c_vp, c_vp,
                                        c_f32, c_f32, c_f32, c_f32, c_f32, c_i64, c_i32, c_vp,
                                        c_vp, c_i64, c_vp]),
    "staple_host_adamw_finish": (c_i32, [c_vp, c_vp]),
    "staple_host_adamw_destroy": (None, [c_vp]),
}

EXPORTED = tuple(_SIGS)

_lib = None


def load(path: str = LIB_PATH):
    """Loads and types libstaple.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libstaple.so not found at {path}; build it with "
            "`python -m token_indexed_ffn_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
