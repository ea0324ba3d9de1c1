"""ctypes view of libgr.so (the C ABI declared in include/gr.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libgr.so.  Loading fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgr.so")

GR_OK, GR_E_INVALID, GR_E_UNSUPPORTED, GR_E_NOMEM, GR_E_WORKSPACE, GR_E_HIP = 0, -1, -2, -3, -4, -5
GR_F32, GR_BF16 = 0, 1

P = ctypes.c_void_p
i32, i64, u64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t

EXPORTS = [
    "gr_last_error", "gr_version", "gr_bloom_probes",
    "gr_trie_builder_create", "gr_trie_builder_add_ads", "gr_trie_builder_finish",
    "gr_trie_builder_destroy", "gr_trie_create", "gr_trie_host_view", "gr_trie_info",
    "gr_trie_destroy", "gr_cross_attn", "gr_cross_attn_workspace", "gr_cross_attn_ws",
    "gr_self_attn_paged", "gr_joint_attn",
    "gr_constrain_topk_workspace", "gr_constrain_topk_shape", "gr_constrain_topk",
    "gr_constrain_topk_noalloc",
    "gr_constrain", "gr_topk_reorder",
    "gr_decode_step", "gr_decode_graph_create", "gr_decode_graph_launch",
    "gr_decode_graph_destroy", "gr_ad_index_create", "gr_ad_index_add_ads",
    "gr_ad_index_finish", "gr_post_filter", "gr_ad_index_destroy",
]


class GrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libgr status {status}: {msg}")
        self.status = status


class TrieParams(ctypes.Structure):
    _fields_ = [("sid_length", i32), ("vocab_size", i32), ("w_bm", i32),
                ("bloom_bits", i32), ("bloom_k", i32), ("n_threads", i32),
                ("keep_host", i32), ("host_only", i32), ("bloom_slice_min", i32),
                ("kway_mode", i32), ("kway_k", i32 * 16), ("kway_kmax", i32),
                ("kway_target_fill", ctypes.c_float)]


class TrieView(ctypes.Structure):
    _fields_ = [("vocab_size", i32), ("sid_length", i32), ("w_bm", i32),
                ("bloom_bits", i32), ("bloom_k", i32),
                ("num_nodes", i64), ("num_entries", i64), ("bm_rows", i64), ("bl_rows", i64),
                ("node_offsets", P), ("child_nodes", P), ("tokens", P),
                ("bitmask_index", P), ("bloom_index", P),
                ("bitmask_table", P), ("bloom_table", P),
                ("node_depth", P), ("node_parent", P), ("node_token", P),
                ("slice_words", i64), ("kway_offsets", P), ("kway_bitmask_index", P),
                ("kway_bloom_index", P), ("kway_rows", i64)]


class TailArgs(ctypes.Structure):
    _fields_ = [("B", i32), ("M_in", i32), ("V", i32), ("k_out", i32), ("t", i32),
                ("L", i32), ("n_loc", i32), ("dtype", ctypes.c_int),
                ("user_bm", P), ("user_probes", P), ("logits", P), ("node_in", P),
                ("acc_in", P), ("tokens_in", P), ("table_in", P),
                ("parent_out", P), ("token_out", P), ("node_out", P), ("acc_out", P),
                ("tokens_out", P), ("table_out", P), ("dbg_mask", P), ("dbg_scores", P),
                ("ws", P), ("ws_bytes", sz)]


class StepArgs(ctypes.Structure):
    _fields_ = [("H", i32), ("d_h", i32), ("T_ctx", i32),
                ("k_ctx", P), ("v_ctx", P), ("qx", P), ("q", P), ("k_new", P), ("v_new", P),
                ("k_pool", P), ("v_pool", P), ("pool_blocks", i64), ("fresh_base", i64),
                ("cross_out", P), ("self_out", P), ("tail", TailArgs),
                ("attn_ws", P), ("attn_ws_bytes", sz)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgr.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    L.gr_last_error.restype = ctypes.c_char_p
    L.gr_version.restype = ctypes.c_char_p
    L.gr_bloom_probes.argtypes = [P, i64, i32, i32, P]
    L.gr_trie_builder_create.argtypes = [ctypes.POINTER(TrieParams), P, i64, ctypes.POINTER(P)]
    L.gr_trie_builder_add_ads.argtypes = [P, i64, P, P, P, P]
    L.gr_trie_builder_finish.argtypes = [P, ctypes.POINTER(P)]
    L.gr_trie_builder_destroy.argtypes = [P]
    L.gr_trie_builder_destroy.restype = None
    L.gr_trie_create.argtypes = [ctypes.POINTER(TrieView), ctypes.POINTER(P)]
    L.gr_trie_host_view.argtypes = [P, ctypes.POINTER(TrieView)]
    L.gr_trie_info.argtypes = [P, ctypes.POINTER(TrieView)]
    L.gr_trie_destroy.argtypes = [P]
    L.gr_trie_destroy.restype = None
    L.gr_cross_attn.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_int, P]
    L.gr_cross_attn_workspace.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    L.gr_cross_attn_workspace.restype = sz
    L.gr_cross_attn_ws.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_int, P, sz, P]
    L.gr_self_attn_paged.argtypes = [P, P, P, P, P, i64, P, i64, i32, i32, i32, i32, i32,
                                     ctypes.c_int, P, P]
    L.gr_joint_attn.argtypes = [P, P, P, P, P, P, P, i64, P, i64, i32, i32, i32, i32, i32, i32,
                                i32, ctypes.c_int, P, P]
    L.gr_constrain_topk_workspace.argtypes = [i32, i32, i32, i32]
    L.gr_constrain_topk_workspace.restype = sz
    L.gr_constrain_topk_shape.argtypes = [i32, i32, i32, P, P, P]
    L.gr_constrain_topk.argtypes = [P, ctypes.POINTER(TailArgs), P]
    L.gr_constrain_topk_noalloc.argtypes = [P, ctypes.POINTER(TailArgs), P]
    L.gr_constrain.argtypes = [P, ctypes.POINTER(TailArgs), P]
    L.gr_topk_reorder.argtypes = [P, ctypes.POINTER(TailArgs), P]
    L.gr_decode_step.argtypes = [P, ctypes.POINTER(StepArgs), P]
    L.gr_decode_graph_create.argtypes = [P, ctypes.POINTER(StepArgs), i32, P, ctypes.POINTER(P)]
    L.gr_decode_graph_launch.argtypes = [P, P]
    L.gr_decode_graph_destroy.argtypes = [P]
    L.gr_decode_graph_destroy.restype = None
    L.gr_ad_index_create.argtypes = [P, i64, i32, i32, i32, ctypes.POINTER(P)]
    L.gr_ad_index_add_ads.argtypes = [P, i64, P, P, P, P]
    L.gr_ad_index_finish.argtypes = [P]
    L.gr_post_filter.argtypes = [P, P, i64, i64, P, P, i32, P, P, i64, i32]
    L.gr_ad_index_destroy.argtypes = [P]
    L.gr_ad_index_destroy.restype = None
    for name in EXPORTS:
        if name not in ("gr_last_error", "gr_version", "gr_trie_builder_destroy",
                        "gr_trie_destroy", "gr_constrain_topk_workspace",
                        "gr_cross_attn_workspace",
                        "gr_decode_graph_destroy", "gr_ad_index_destroy"):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def check(status: int) -> None:
    if status != GR_OK:
        raise GrError(status, lib().gr_last_error().decode())
