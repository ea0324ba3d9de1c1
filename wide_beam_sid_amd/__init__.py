"""wide_beam_sid_amd: the wide-beam SID decode step on AMD MI355X (gfx950).

Thin Python binding over libgr.so (C ABI in include/gr.h).  Functions carry
the C names without the ``gr_`` prefix and only marshal arguments: torch
tensors provide device memory and the current HIP stream; every step of the
path runs in the library's HIP kernels.  Importing this package does not
need a GPU; calling into the library needs the built libgr.so and fails
loudly without it.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import _lib
from ._lib import GR_BF16, GR_F32, GrError, StepArgs, TailArgs, TrieParams, TrieView, check

__all__ = [
    "GrError", "Trie", "bloom_probes", "cross_attn", "self_attn_paged", "joint_attn",
    "constrain_topk_workspace", "constrain_topk_shape", "constrain_topk", "constrain",
    "topk_reorder", "decode_step",
    "DecodeGraph", "AdIndex", "version",
]


def version() -> str:
    return _lib.lib().gr_version().decode()


def _ptr(x) -> Optional[int]:
    """Device (torch) or host (numpy) buffer address; None for a missing one."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        assert x.flags["C_CONTIGUOUS"]
        return x.ctypes.data
    assert x.is_contiguous(), "tensors passed to libgr must be contiguous"
    return x.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GR_BF16
    if t.dtype == torch.float32:
        return GR_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def bloom_probes(ids: np.ndarray, bloom_bits: int, bloom_k: int) -> np.ndarray:
    """Bloom probe positions [n, bloom_k] of geo ids (host)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    out = np.zeros((ids.size, bloom_k), dtype=np.uint32)
    check(_lib.lib().gr_bloom_probes(_ptr(ids) if ids.size else None, ids.size,
                                     bloom_bits, bloom_k, _ptr(out)))
    return out


class Trie:
    """A GTM SID trie resident on the current HIP device."""

    def __init__(self, handle: int):
        self.h = ctypes.c_void_p(handle)

    @classmethod
    def build(cls, sids: np.ndarray, vocab_size: int, w_bm: int, bloom_bits: int,
              bloom_k: int, ad_chunks, keep_host: bool = False, n_threads: int = 0,
              host_only: bool = False, bloom_slice_min: int = 0, kway_mode: int = 0,
              kway_k=(), kway_kmax: int = 0, kway_target_fill: float = 0.0) -> "Trie":
        """Build from the catalog and an iterable of ad chunks (objects with
        ad_sid, rules, geo_offsets, geo_ids).  kway_mode 1 (static, kway_k per
        decoding position) or 2 (dynamic, kway_kmax, kway_target_fill) keeps
        k-way partitioned matchers (see gr_trie_params)."""
        L = _lib.lib()
        sids = np.ascontiguousarray(sids, dtype=np.int32)
        p = TrieParams(sid_length=sids.shape[1], vocab_size=vocab_size, w_bm=w_bm,
                       bloom_bits=bloom_bits, bloom_k=bloom_k, n_threads=n_threads,
                       keep_host=int(keep_host), host_only=int(host_only),
                       bloom_slice_min=bloom_slice_min, kway_mode=kway_mode,
                       kway_kmax=kway_kmax, kway_target_fill=kway_target_fill)
        for i, k in enumerate(kway_k):
            p.kway_k[i] = k
        b = ctypes.c_void_p()
        check(L.gr_trie_builder_create(ctypes.byref(p), _ptr(sids), sids.shape[0], ctypes.byref(b)))
        try:
            for ch in ad_chunks:
                ad_sid = np.ascontiguousarray(ch.ad_sid, dtype=np.int64)
                rules = np.ascontiguousarray(ch.rules, dtype=np.uint64)
                go = np.ascontiguousarray(ch.geo_offsets, dtype=np.int64)
                gi = np.ascontiguousarray(ch.geo_ids, dtype=np.int32)
                check(L.gr_trie_builder_add_ads(b, ad_sid.size, _ptr(ad_sid), _ptr(rules),
                                                _ptr(go), _ptr(gi) if gi.size else None))
        except Exception:
            L.gr_trie_builder_destroy(b)
            raise
        t = ctypes.c_void_p()
        check(L.gr_trie_builder_finish(b, ctypes.byref(t)))
        return cls(t.value)

    @classmethod
    def create(cls, arrays: dict, vocab_size: int, sid_length: int, w_bm: int,
               bloom_bits: int = 0, bloom_k: int = 0) -> "Trie":
        """Upload caller-built Appendix A arrays (numpy, host)."""
        a = {k: np.ascontiguousarray(v) for k, v in arrays.items()}
        v = TrieView()
        v.vocab_size, v.sid_length, v.w_bm = vocab_size, sid_length, w_bm
        v.bloom_bits, v.bloom_k = bloom_bits, bloom_k
        v.num_nodes = a["node_offsets"].size - 1
        v.num_entries = a["child_nodes"].size
        v.bm_rows = a["bitmask_table"].shape[0]
        v.bl_rows = a["bloom_table"].shape[0] if "bloom_table" in a else 0
        for name in ("node_offsets", "child_nodes", "tokens", "bitmask_index",
                     "bloom_index", "bitmask_table", "bloom_table"):
            if name in a:
                setattr(v, name, _ptr(a[name]))
        t = ctypes.c_void_p()
        check(_lib.lib().gr_trie_create(ctypes.byref(v), ctypes.byref(t)))
        return cls(t.value)

    def info(self) -> dict:
        v = TrieView()
        check(_lib.lib().gr_trie_info(self.h, ctypes.byref(v)))
        return {k: getattr(v, k) for k in ("vocab_size", "sid_length", "w_bm", "bloom_bits",
                                           "bloom_k", "num_nodes", "num_entries", "bm_rows",
                                           "bl_rows", "slice_words", "kway_rows")}

    def host_view(self, copy: bool = True) -> dict:
        """The host arrays (trie built with keep_host=True): copies, or with
        copy=False read-only views of the trie's own arrays, valid while the
        trie lives."""
        v = TrieView()
        check(_lib.lib().gr_trie_host_view(self.h, ctypes.byref(v)))
        n, e = v.num_nodes, v.num_entries
        w_bl = v.bloom_bits // 64

        def arr(ptr, ctype, count, np_dtype):
            if not ptr or count == 0:
                return np.zeros(0, np_dtype)
            buf = (ctype * count).from_address(ptr)
            a = np.frombuffer(buf, dtype=np_dtype, count=count)
            if copy:
                return a.copy()
            a.flags.writeable = False
            return a

        out = {
            "node_offsets": arr(v.node_offsets, ctypes.c_int32, n + 1, np.int32),
            "child_nodes": arr(v.child_nodes, ctypes.c_int32, e, np.int32),
            "tokens": arr(v.tokens, ctypes.c_int16, e, np.int16),
            "bitmask_index": arr(v.bitmask_index, ctypes.c_int32, e, np.int32),
            "bloom_index": arr(v.bloom_index, ctypes.c_int32, e, np.int32),
            "bitmask_table": arr(v.bitmask_table, ctypes.c_uint64, v.bm_rows * v.w_bm,
                                 np.uint64).reshape(v.bm_rows, v.w_bm),
            "bloom_table": arr(v.bloom_table, ctypes.c_uint64, v.bl_rows * w_bl,
                               np.uint64).reshape(v.bl_rows, w_bl),
            "node_depth": arr(v.node_depth, ctypes.c_int32, n, np.int32),
            "node_parent": arr(v.node_parent, ctypes.c_int32, n, np.int32),
            "node_token": arr(v.node_token, ctypes.c_int16, n, np.int16),
        }
        if v.kway_offsets:
            kr = arr(v.kway_offsets, ctypes.c_int32, e + 1, np.int32)
            out["kway_offsets"] = kr
            out["kway_bitmask_index"] = arr(v.kway_bitmask_index, ctypes.c_int32, int(kr[-1]), np.int32)
            out["kway_bloom_index"] = arr(v.kway_bloom_index, ctypes.c_int32, int(kr[-1]), np.int32)
        out.update({k: getattr(v, k) for k in ("vocab_size", "sid_length", "w_bm", "bloom_bits",
                                                "bloom_k", "num_nodes", "num_entries",
                                                "bm_rows", "bl_rows")})
        return out

    def close(self):
        if self.h and self.h.value:
            _lib.lib().gr_trie_destroy(self.h)
            self.h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cross_attn(q, k_ctx, v_ctx, out, B: int, M: int, stream=None, ws=None) -> None:
    """A1 on torch tensors: q/out [B*M, H, d_h], k_ctx/v_ctx [B, H, T_ctx, d_h].
    With ws (a device buffer of cross_attn_workspace bytes) a long context
    is split across workgroups when the launch has few tiles."""
    H, T, d = k_ctx.shape[1], k_ctx.shape[2], k_ctx.shape[3]
    if ws is None:
        check(_lib.lib().gr_cross_attn(_ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(out), B, M, H, T,
                                       d, _dtype(q), _stream(stream)))
    else:
        check(_lib.lib().gr_cross_attn_ws(_ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(out), B, M, H,
                                          T, d, _dtype(q), _ptr(ws), ws.numel() * ws.element_size(),
                                          _stream(stream)))


def cross_attn_workspace(B: int, M: int, H: int, T_ctx: int, d_h: int, dtype: str) -> int:
    """Bytes of the split cross-attention workspace for these shapes (0: no split)."""
    return int(_lib.lib().gr_cross_attn_workspace(B, M, H, T_ctx, d_h,
                                                  GR_BF16 if dtype == "bf16" else GR_F32))


def self_attn_paged(q, k_new, v_new, k_pool, v_pool, table, fresh_base: int, t: int, out,
                    stream=None) -> None:
    """A2 on torch tensors: q/k_new/v_new/out [R, H, d_h], pools [N, H, d_h],
    table int32 [R, L]."""
    R, H, d = q.shape
    L = table.shape[1]
    check(_lib.lib().gr_self_attn_paged(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                        _ptr(v_pool), k_pool.shape[0], _ptr(table), fresh_base,
                                        R, t, L, H, d, _dtype(q), _ptr(out), _stream(stream)))


def joint_attn(q, k_ctx, v_ctx, k_new, v_new, k_pool, v_pool, table, fresh_base: int, t: int,
               B: int, M: int, out, stream=None) -> None:
    """Joint context + beam-prefix attention on torch tensors (see
    gr_joint_attn): q/k_new/v_new/out [B*M, H, d_h], k_ctx/v_ctx
    [B, H, T_ctx, d_h], pools [N, H, d_h], table int32 [B*M, L]."""
    R, H, d = q.shape
    T = k_ctx.shape[2]
    L = table.shape[1]
    check(_lib.lib().gr_joint_attn(_ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(k_new), _ptr(v_new),
                                   _ptr(k_pool), _ptr(v_pool), k_pool.shape[0], _ptr(table),
                                   fresh_base, B, M, H, T, d, t, L, _dtype(q), _ptr(out),
                                   _stream(stream)))


def constrain_topk_workspace(B: int, M_in: int, V: int, k_out: int) -> int:
    return int(_lib.lib().gr_constrain_topk_workspace(B, M_in, V, k_out))


def constrain_topk_shape(B: int, M_in: int, V: int):
    """(rows_wg, gx, seg_cap): the tail's expand workgroups per request, the
    beam rows each takes and its survivor segment size."""
    rw, gx, sc = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _lib.check(_lib.lib().gr_constrain_topk_shape(B, M_in, V, ctypes.byref(rw), ctypes.byref(gx),
                                                  ctypes.byref(sc)))
    return rw.value, gx.value, sc.value


def tail_args(**kw) -> TailArgs:
    """TailArgs from keyword arguments (tensors become device pointers)."""
    a = TailArgs()
    for k, v in kw.items():
        if k == "dtype":
            a.dtype = v
        elif isinstance(v, (int, np.integer)) and k in ("B", "M_in", "V", "k_out", "t", "L",
                                                        "n_loc", "ws_bytes"):
            setattr(a, k, int(v))
        else:
            setattr(a, k, _ptr(v))
    return a


def constrain_topk(trie: Trie, args: TailArgs, stream=None) -> None:
    """A3-A6 (see gr_constrain_topk).  The workspace must start zero-filled."""
    check(_lib.lib().gr_constrain_topk(trie.h, ctypes.byref(args), _stream(stream)))


def constrain(trie: Trie, args: TailArgs, stream=None) -> None:
    """A3-A4, the first stage of gr_constrain_topk (see gr_constrain)."""
    check(_lib.lib().gr_constrain(trie.h, ctypes.byref(args), _stream(stream)))


def topk_reorder(trie: Trie, args: TailArgs, stream=None) -> None:
    """A5-A6, the second stage of gr_constrain_topk (see gr_topk_reorder)."""
    check(_lib.lib().gr_topk_reorder(trie.h, ctypes.byref(args), _stream(stream)))


def decode_step(trie: Trie, args: StepArgs, stream=None) -> None:
    """A1 -> A2 -> A3..A6 for one step (see gr_decode_step)."""
    check(_lib.lib().gr_decode_step(trie.h, ctypes.byref(args), _stream(stream)))


class DecodeGraph:
    """A whole decode (consecutive gr_decode_step calls) captured once as a
    HIP graph (see gr_decode_graph_create); launch() replays it on a stream.
    The step arguments' buffers are baked in and must stay alive."""

    def __init__(self, trie: Trie, steps, stream):
        arr = (StepArgs * len(steps))(*steps)
        h = ctypes.c_void_p()
        check(_lib.lib().gr_decode_graph_create(trie.h, arr, len(steps), _stream(stream),
                                                ctypes.byref(h)))
        self.h = h
        self.trie = trie      # the graph reads the trie's device arrays

    def launch(self, stream=None) -> None:
        check(_lib.lib().gr_decode_graph_launch(self.h, _stream(stream)))

    def close(self) -> None:
        h = getattr(self, "h", None)
        if h is not None and h.value:
            _lib.lib().gr_decode_graph_destroy(h)
        self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class AdIndex:
    """SID-to-ad index plus the ads' targeting (host), for the post stage
    (see gr_ad_index_create / gr_post_filter)."""

    def __init__(self, sids: np.ndarray, vocab_size: int, w_bm: int, ad_chunks):
        L = _lib.lib()
        sids = np.ascontiguousarray(sids, dtype=np.int32)
        h = ctypes.c_void_p()
        check(L.gr_ad_index_create(_ptr(sids), sids.shape[0], sids.shape[1], vocab_size, w_bm,
                                   ctypes.byref(h)))
        self.h = h
        self.sid_length = sids.shape[1]
        try:
            for ch in ad_chunks:
                ad_sid = np.ascontiguousarray(ch.ad_sid, dtype=np.int64)
                rules = np.ascontiguousarray(ch.rules, dtype=np.uint64)
                go = np.ascontiguousarray(ch.geo_offsets, dtype=np.int64)
                gi = np.ascontiguousarray(ch.geo_ids, dtype=np.int32)
                check(L.gr_ad_index_add_ads(h, ad_sid.size, _ptr(ad_sid), _ptr(rules), _ptr(go),
                                            _ptr(gi) if gi.size else None))
            check(L.gr_ad_index_finish(h))
        except Exception:
            self.close()
            raise

    def post_filter(self, tokens: np.ndarray, rows_per_request: int, user_bm: np.ndarray,
                    user_locs: Optional[np.ndarray], n_threads: int = 0):
        """Per row [ads, bitmask passes, location passes, passes] (int64
        [n, 4]) and the passing ad ids row by row."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1, self.sid_length)
        ubm = np.ascontiguousarray(user_bm, dtype=np.uint64)
        n_loc = 0 if user_locs is None else int(user_locs.shape[1])
        locs = None if not n_loc else np.ascontiguousarray(user_locs, dtype=np.int32)
        counts = np.zeros((tokens.shape[0], 4), np.int64)
        L = _lib.lib()
        check(L.gr_post_filter(self.h, _ptr(tokens), tokens.shape[0], rows_per_request, _ptr(ubm),
                               _ptr(locs), n_loc, _ptr(counts), None, 0, n_threads))
        total = int(counts[:, 3].sum())
        ids = np.zeros(max(total, 1), np.int64)
        check(L.gr_post_filter(self.h, _ptr(tokens), tokens.shape[0], rows_per_request, _ptr(ubm),
                               _ptr(locs), n_loc, _ptr(counts), _ptr(ids), ids.size, n_threads))
        return counts, ids[:total]

    def close(self) -> None:
        h = getattr(self, "h", None)
        if h is not None and h.value:
            _lib.lib().gr_ad_index_destroy(h)
        self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
