"""ctypes loader for libmla.so (the C ABI declared in include/mla.h).

There is no fallback: if the library is missing the import fails with an
error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MLA_LIB_PATH", os.path.join(_HERE, "libmla.so"))

c_void_p = ctypes.c_void_p
c_int = ctypes.c_int
c_int64 = ctypes.c_int64
c_float = ctypes.c_float
c_size_t = ctypes.c_size_t
c_char_p = ctypes.c_char_p

# name -> (restype, argtypes), mirroring include/mla.h
SIGNATURES = {
    "mla_status_string": (c_char_p, [c_int]),
    "mla_last_error": (c_char_p, []),
    "mla_absorb_q": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int, c_void_p]),
    "mla_decode_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
    "mla_recommended_splits": (c_int, [c_int, c_int, c_int, c_int]),
    "mla_plan_splits": (c_int, [c_void_p, c_int, c_int, c_int, c_int]),
    "mla_validate_block_table": (c_int, [c_void_p, c_int, c_void_p, c_int, c_int64, c_void_p, c_void_p]),
    "mla_decode_paged": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int, c_void_p, c_int, c_int,
                                 c_int, c_float, c_int, c_void_p, c_void_p, c_void_p]),
    "mla_combine_splits": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "mla_up_proj": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int, c_void_p]),
    "mla_combine_up_proj": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                    c_void_p]),
    "mla_debug_gather": (c_int, [c_void_p, c_int64, c_void_p, c_int, c_void_p, c_int, c_int, c_void_p, c_void_p]),
    "mla_bench_stream_read": (c_int, [c_void_p, c_int64, c_void_p, c_void_p]),
    "mla_bench_mfma": (c_int, [c_int64, c_void_p, c_void_p]),
    "mla_rope_table": (c_int, [ctypes.c_double, c_int, c_void_p]),
    "mla_append_latent": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_int64, c_void_p, c_int, c_void_p,
                                  c_int, c_int, c_void_p]),
    "mla_rope_q": (c_int, [c_void_p, c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_void_p]),
    "mla_prefill_uses_absorption": (c_int, [c_int]),
    "mla_decompressed_kv_bytes": (c_size_t, [c_int, c_int]),
    "mla_decompress_kv": (c_int, [c_void_p, c_int64, c_void_p, c_int, c_void_p, c_int, c_int, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p]),
    "mla_quantize_cache_fp8": (c_int, [c_void_p, c_int64, c_void_p, c_void_p]),
    "mla_append_latent_fp8": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_int64, c_void_p, c_int,
                                      c_void_p, c_int, c_int, c_void_p]),
    "mla_decode_paged_fp8": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int, c_void_p, c_int, c_int,
                                     c_int, c_float, c_int, c_void_p, c_void_p, c_void_p]),
    "mla_quantize_cache_mxfp4": (c_int, [c_void_p, c_int64, c_void_p, c_void_p]),
    "mla_append_latent_mxfp4": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_int64, c_void_p, c_int,
                                        c_void_p, c_int, c_int, c_void_p]),
    "mla_decode_paged_mxfp4": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int, c_void_p, c_int, c_int,
                                       c_int, c_float, c_int, c_void_p, c_void_p, c_void_p]),
    "mla_decode_step": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int, c_void_p, c_int, c_int, c_int,
                                c_void_p, c_void_p, c_float, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p]),
    "mla_decode_step_fp8": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int, c_void_p, c_int, c_int,
                                    c_int, c_void_p, c_void_p, c_float, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p]),
    "mla_decode_step_mxfp4": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int, c_void_p, c_int, c_int,
                                    c_int, c_void_p, c_void_p, c_float, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p]),
    "mla_decode_step_static": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int, c_void_p, c_int, c_int,
                                       c_int, c_void_p, c_void_p, c_float, c_int, c_void_p, c_void_p, c_void_p]),
    "mla_prefill_mha": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_int64, c_void_p, c_int,
                                c_void_p, c_int, c_int, c_int, c_float, c_void_p, c_void_p, c_void_p]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"libmla.so not found at {path}; build it with `python mla_latent_kv_06_amd/build.py` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = load()
