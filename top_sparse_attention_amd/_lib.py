"""ctypes declarations of libtsa's C ABI (include/tsa.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtsa.so")

i32, i64, f32, vp, sz = C.c_int32, C.c_int64, C.c_float, C.c_void_p, C.c_size_t
P_i32, P_i64, P_f32, P_sz = C.POINTER(i32), C.POINTER(i64), C.POINTER(f32), C.POINTER(sz)

TSA_OK = 0
TSA_ERR_INVALID = -1
TSA_ERR_OUT_OF_PAGES = -2
TSA_ERR_SHARED_PAGE_WRITE = -3
TSA_ERR_HIP = -4
TSA_ERR_CAPACITY = -5
TSA_ERR_UNSUPPORTED = -6
STATUS_NAMES = {
    0: "TSA_OK", -1: "TSA_ERR_INVALID", -2: "TSA_ERR_OUT_OF_PAGES", -3: "TSA_ERR_SHARED_PAGE_WRITE",
    -4: "TSA_ERR_HIP", -5: "TSA_ERR_CAPACITY", -6: "TSA_ERR_UNSUPPORTED",
}


class PoolDesc(C.Structure):
    _fields_ = [("num_pages", i32), ("page_size", i32), ("num_layers", i32), ("num_kv_heads", i32),
                ("head_dim_k", i32), ("head_dim_v", i32), ("v_from_k", i32), ("index_dim", i32)]


class DecodeParams(C.Structure):
    _fields_ = [("batch", i32), ("num_q_heads", i32), ("index_heads", i32), ("top_k", i32),
                ("max_len", i32), ("sm_scale", f32)]


class AppendArgs(C.Structure):
    _fields_ = [("n_tok", i32), ("req_dev", vp), ("pos_dev", vp), ("k_src", vp), ("v_src", vp),
                ("idx_src", vp), ("bad_dev", vp)]


# name -> (restype, argtypes)
SIGNATURES = {
    "tsa_last_error": (C.c_char_p, []),
    "tsa_abi_version": (i32, []),
    "tsa_kv_pool_bytes": (i32, [C.POINTER(PoolDesc), P_sz, P_sz, P_sz]),
    "tsa_kv_pool_create": (i32, [C.POINTER(PoolDesc), vp, vp, vp, P_i32, C.POINTER(vp)]),
    "tsa_kv_pool_destroy": (i32, [vp]),
    "tsa_kv_pool_usage": (i32, [vp, P_i32, P_i32]),
    "tsa_kv_pool_refcount": (i32, [vp, i32, P_i32]),
    "tsa_page_table_build": (i32, [vp, i32, P_i32, P_i32, P_i32, i32, i32, P_i32, P_i32, P_i64]),
    "tsa_page_table_grow": (i32, [vp, i32, P_i32, i32, P_i32, P_i32]),
    "tsa_page_table_release": (i32, [vp, i32, P_i32, P_i32, i32]),
    "tsa_kv_append_check": (i32, [vp, i32, P_i32, P_i32, i32, P_i32, P_i32, i32]),
    "tsa_kv_append": (i32, [vp, i32, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]),
    "tsa_sparse_decode_workspace": (i32, [vp, C.POINTER(DecodeParams), P_sz]),
    "tsa_indexer_scores": (i32, [vp, i32, C.POINTER(DecodeParams), vp, vp, vp, i32, vp, vp, i32, vp]),
    "tsa_topk": (i32, [C.POINTER(DecodeParams), vp, i32, vp, vp, vp]),
    "tsa_indexer_topk": (i32, [vp, i32, C.POINTER(DecodeParams), vp, vp, vp, i32, vp, vp, vp, sz, vp]),
    "tsa_sparse_attn_gather": (i32, [vp, i32, C.POINTER(DecodeParams), vp, vp, vp, i32, vp, vp, vp, sz, vp]),
    "tsa_sparse_decode_attn": (i32, [vp, i32, C.POINTER(DecodeParams), vp, vp, vp, vp, i32, vp, vp, vp,
                                     vp, sz, vp]),
    "tsa_decode_step": (i32, [vp, i32, C.POINTER(DecodeParams), vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                              vp, vp, vp, sz, vp]),
    "tsa_decode_step_noalloc": (i32, [vp, i32, C.POINTER(DecodeParams), vp, vp, vp, vp, vp, vp, vp, vp,
                                      i32, vp, vp, vp, vp]),
    "tsa_decode_step_fused": (i32, [vp, i32, C.POINTER(DecodeParams), vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                    vp, vp, vp, vp]),
    "tsa_step_graph_create": (i32, [vp, i32, C.POINTER(DecodeParams), C.POINTER(AppendArgs), vp, vp, vp,
                                    vp, i32, vp, vp, vp, vp, sz, C.POINTER(vp)]),
    "tsa_step_graph_launch": (i32, [vp, vp]),
    "tsa_step_graph_destroy": (i32, [vp]),
    "tsa_lru_create": (i32, [vp, i32, i32, i32, vp, vp, C.POINTER(vp)]),
    "tsa_lru_destroy": (i32, [vp]),
    "tsa_lru_preload": (i32, [vp, i64, P_i64]),
    "tsa_lru_plan": (i32, [vp, i32, i64, i32, P_i32, i32, P_i32, P_i64]),
    "tsa_lru_workspace_bytes": (i32, [vp, i32, P_sz]),
    "tsa_lru_fetch": (i32, [vp, i32, P_i32, vp, vp, sz, vp]),
    "tsa_lru_release": (i32, [vp, i64]),
    "tsa_lru_release_layer": (i32, [vp, i64, vp]),
    "tsa_lru_prefetch": (i32, [vp, i32, i64, i32, P_i32, i32, vp, vp, sz, vp, vp]),
    "tsa_lru_stats": (i32, [vp, P_i64, P_i64, P_i64, P_i64]),
}

_lib = None


class TsaError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def load() -> C.CDLL:
    """Load libtsa.so from the package directory; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m top_sparse_attention_amd.build`")
    # torch brings its own HIP runtime (SONAME libamdhip64.so.7).  Load it first so that
    # libtsa's dependency resolves to that same copy: one process, one HIP runtime, and device
    # pointers and streams from torch are valid inside the library.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def call(name: str, *args) -> None:
    """Call a status-returning entry point; raise TsaError on failure."""
    lib = load()
    st = getattr(lib, name)(*args)
    if st != TSA_OK:
        raise TsaError(st, name, lib.tsa_last_error().decode(errors="replace"))
