"""ctypes loader for libmla_nvfp4.so (built in-tree by ``build.py``).

Loading fails loudly: there is no fallback path of any kind.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_nvfp4.so")

# every symbol include/mla_nvfp4.h declares, with its ctypes signature
c_i64, c_i32, c_int, c_f32, c_vp, c_size = (ctypes.c_int64, ctypes.c_int32, ctypes.c_int,
                                            ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t)
SIGNATURES = {
    "mla_nvfp4_quantize_append": (c_int, [c_vp, c_i64, c_vp, c_i64, c_int, c_i64, c_vp, c_vp, c_i64, c_vp]),
    "mla_nvfp4_quantize_append_2level": (c_int, [c_vp, c_i64, c_vp, c_i64, c_int, c_i64, c_vp, c_vp, c_i64,
                                                 c_f32, c_vp]),
    "mla_fp8_quantize_append": (c_int, [c_vp, c_i64, c_vp, c_i64, c_int, c_i64, c_vp, c_vp, c_i64, c_f32, c_vp]),
    "mla_sparse_decode_num_splits": (c_i32, [c_i64, c_i32, c_i32]),
    "mla_sparse_decode_workspace_size": (c_size, [c_i64, c_i32, c_i32, c_i32]),
    "mla_sparse_decode_set_merge_polls": (c_i32, [c_i32]),
    "mla_sparse_decode": (c_int, [c_vp, c_int, c_i64, c_i32, c_i64, c_i64,
                                  c_vp, c_int, c_i64, c_f32,
                                  c_vp, c_i32, c_i64,
                                  c_vp, c_i32, c_i64, c_i32, c_i32, c_vp,
                                  c_f32, c_vp, c_vp, c_vp, c_size, c_i32, c_vp]),
    "mla_sparse_decode_noalloc": (c_int, [c_vp, c_int, c_i64, c_i32, c_i64, c_i64,
                                          c_vp, c_int, c_i64, c_f32,
                                          c_vp, c_i32, c_i64,
                                          c_vp, c_i32, c_i64, c_i32, c_i32, c_vp,
                                          c_f32, c_vp, c_vp, c_i32, c_vp]),
    "mla_nvfp4_gather_dequant_fp8": (c_int, [c_vp, c_i64, c_vp, c_i64, c_i32, c_i64,
                                             c_vp, c_i32, c_i64, c_i32, c_i32, c_vp,
                                             c_f32, c_vp, c_vp, c_vp]),
    "mla_indexer_workspace_size": (c_size, [c_i64, c_i32]),
    "mla_indexer_topk": (c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_vp, c_i32, c_vp,
                                 c_vp, c_i32, c_i64, c_i32, c_i32, c_vp,
                                 c_i32, c_vp, c_i64, c_vp, c_size, c_vp]),
    "mla_pool_capacity_blocks": (c_i64, [c_i64, c_i32, c_i32, c_i32, c_i32]),
    "mla_pool_create": (c_int, [c_i64, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_vp)]),
    "mla_pool_destroy": (None, [c_vp]),
    "mla_pool_num_blocks": (c_i64, [c_vp]),
    "mla_pool_free_blocks": (c_i64, [c_vp]),
    "mla_pool_reserve": (c_int, [c_vp, c_i32, c_i64]),
    "mla_pool_release": (c_int, [c_vp, c_i32]),
    "mla_pool_block_table": (c_int, [c_vp, c_vp, c_i64]),
    "mla_pool_slots": (c_int, [c_vp, c_i32, c_i64, c_i64, c_vp]),
    "mla_pool_descriptors": (c_int, [c_vp, c_i32, c_i32, ctypes.POINTER(c_i64), ctypes.POINTER(c_i64)]),
    "mla_kv_pack_blocks": (c_int, [c_vp, c_i32, c_i64, c_i32, c_i32, c_i32, c_vp, c_i64, c_vp, c_vp]),
    "mla_kv_unpack_blocks": (c_int, [c_vp, c_i64, c_vp, c_vp, c_i32, c_i64, c_i32, c_i32, c_i32, c_vp]),
    "mla_kernel_timing": (c_int, [c_int]),
    "mla_gather_probe": (c_int, [c_vp, c_i64, c_i32, c_vp, c_i64, c_vp, c_vp]),
    "mla_last_kernel_ms": (c_int, [ctypes.POINTER(ctypes.c_float)]),
    "mla_status_string": (ctypes.c_char_p, [c_int]),
}

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library not built: {LIB_PATH} is missing. Run "
            "`python -m nvfp4_compressed_sparse_mla_amd.build` (needs ROCm hipcc) first.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MlaError(RuntimeError):
    pass


def check(status: int, what: str) -> None:
    if status != 0:
        msg = load().mla_status_string(status).decode()
        raise MlaError(f"{what} failed: status {status} ({msg})")
