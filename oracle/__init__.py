"""CPU oracle for the wide-beam SID decode step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the GPU
library (``wide_beam_sid_amd``) and never imports it; both read the same
seeded inputs from ``synth``.

The arithmetic lives in ``oracle.c`` (plain C, fp64, compiled with gcc into
``_oracle.so``); this module only marshals numpy arrays and walks the decode
loop of GRACE Section 3.1 step by step (``decode.py``).

Parity status per function (pins live in tests/test_oracle_*.py):
  bloom_positions   pinned: SplitMix64 published test vector, eq 8 property
  mask_row          pinned: toy example of eqs 6-7, brute force on tiny
                    catalogs (catalog validity, no false negatives)
  log_softmax       pinned: closed forms (uniform logits, normalisation)
  topk              pinned: brute-force rank counting, two-level lemma
  cross_attn        pinned: torch SDPA fp64 (Appendix B per-row broadcast),
                    T_ctx = 1, q = 0, identical keys
  self_attn         pinned: T_self = 1, coalesced block-diagonal tile of
                    Section 5.2, torch SDPA fp64 per row
  post.post_filter  pinned: hand-worked example, brute-force properties
                    (tests/test_oracle_post.py)
  decode.step       pinned: the dense K/V history reorder against each beam's
                    parent chain rebuilt independently, with brute-force
                    self-attention per row (dead slots included); final
                    scores = sum of per-step log-probs; finished SIDs in the
                    catalog (tests/test_oracle_pins.py)
  SampledUnions     pinned: equals the prefix tables' rows (themselves pinned
                    by brute force) on every sampled prefix of small catalogs
  TrieAsData        pinned: masks equal mask_row's on every (prefix, request)
                    of small catalogs, for a trie whose rows equal the prefix
                    tables'; no false negatives by brute force
  joint_attn        pinned: no beam positions = cross_attn; the log-sum-exp
                    merge of the pinned cross_attn and self_attn results;
                    identical keys (mean of every value); q = 0
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "_oracle.so")


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, u64 = ctypes.c_int64, ctypes.c_int, ctypes.c_uint64
        L.orc_splitmix64_first.restype = u64
        L.orc_splitmix64_first.argtypes = [u64]
        L.orc_bloom_positions.argtypes = [i64, i32, i32, P]
        L.orc_bloom_row.argtypes = [i64, i32, i32, P]
        L.orc_bloom_contains.argtypes = [P, P, i32]
        L.orc_bloom_contains.restype = i32
        L.orc_bitmask_match.argtypes = [P, P, i32]
        L.orc_bitmask_match.restype = i32
        L.orc_index_create.restype = P
        L.orc_index_create.argtypes = [i32, i32, i64, P, i32, i32, i32]
        L.orc_index_add_ads.argtypes = [P, i64, P, P, P, P]
        L.orc_index_finish.argtypes = [P]
        L.orc_index_destroy.argtypes = [P]
        L.orc_index_count.restype = i64
        L.orc_index_count.argtypes = [P, i32]
        L.orc_index_find.restype = i64
        L.orc_index_find.argtypes = [P, P, i32]
        L.orc_index_rows.argtypes = [P, i32, P, P, P]
        L.orc_mask_row.restype = i32
        L.orc_mask_row.argtypes = [P, P, i32, P, P, i32, P]
        L.orc_log_softmax.argtypes = [P, i32, P]
        L.orc_topk.restype = i64
        L.orc_topk.argtypes = [P, i64, i64, P, P]
        L.orc_cross_attn.argtypes = [P, P, P, i32, i32, i32, i32, i32, P]
        L.orc_self_attn.argtypes = [P, P, P, P, i64, i32, i32, i32, P]
        L.orc_joint_attn.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, P]
        L.orc_usample_create.restype = P
        L.orc_usample_create.argtypes = [i32, i32, i32, i32, i32, P, i64]
        L.orc_usample_destroy.argtypes = [P]
        L.orc_usample_destroy.restype = None
        L.orc_usample_set_level.argtypes = [P, i32, P, i64]
        L.orc_usample_set_level.restype = None
        L.orc_usample_add_ads.argtypes = [P, i64, P, P, P, P]
        L.orc_usample_add_ads.restype = None
        L.orc_usample_rows.argtypes = [P, i32, P, P]
        L.orc_usample_rows.restype = None
        L.orc_mask_row_csr.restype = i32
        L.orc_mask_row_csr.argtypes = [P, P, P, P, P, P, i32, P, i32, i32, P, i32, P, P, i32, P]
        L.orc_set_threads.argtypes = [i32]
        L.orc_set_threads.restype = None
        L.orc_get_threads.restype = i32
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops over rows (timing only)."""
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------
# O1: Bloom hashing
# ---------------------------------------------------------------------------

def splitmix64_first(state: int) -> int:
    return int(lib().orc_splitmix64_first(ctypes.c_uint64(state & (2**64 - 1))))


def bloom_positions(geo_id: int, w_bits: int, k: int) -> np.ndarray:
    out = np.zeros(k, dtype=np.uint32)
    lib().orc_bloom_positions(int(geo_id), w_bits, k, _p(out))
    return out


def bloom_row(geo_id: int, w_bits: int, k: int) -> np.ndarray:
    out = np.zeros(w_bits // 64, dtype=np.uint64)
    lib().orc_bloom_row(int(geo_id), w_bits, k, _p(out))
    return out


def bloom_contains(B: np.ndarray, bloom_l: np.ndarray) -> bool:
    B = _c(B, np.uint64)
    bl = _c(bloom_l, np.uint64)
    return bool(lib().orc_bloom_contains(_p(B), _p(bl), B.size))


def bitmask_match(node_bm: np.ndarray, user_bm: np.ndarray) -> bool:
    a = _c(node_bm, np.uint64)
    u = _c(user_bm, np.uint64)
    return bool(lib().orc_bitmask_match(_p(a), _p(u), a.size))


# ---------------------------------------------------------------------------
# O2-O5: prefix tables and masks
# ---------------------------------------------------------------------------

class Index:
    """Per-level prefix tables with OR-union matchers (eqs 4, 9)."""

    def __init__(self, L: int, V: int, sids: np.ndarray, w_bm: int,
                 bloom_bits: int, bloom_k: int):
        self.L, self.V, self.w_bm = L, V, w_bm
        self.bloom_bits, self.bloom_k = bloom_bits, bloom_k
        self.w_bl = bloom_bits // 64
        s = _c(sids, np.int32)
        self._keep = s
        self.h = lib().orc_index_create(L, V, s.shape[0], _p(s), w_bm, bloom_bits, bloom_k)
        if not self.h:
            raise ValueError("bad index parameters")

    def add_ads(self, ad_sid, rules, geo_off, geo_ids):
        a = _c(ad_sid, np.int64)
        r = _c(rules, np.uint64)
        go = _c(geo_off, np.int64)
        gi = _c(geo_ids, np.int32) if len(geo_ids) else np.zeros(1, np.int32)
        lib().orc_index_add_ads(self.h, a.size, _p(a), _p(r), _p(go), _p(gi))

    def finish(self):
        lib().orc_index_finish(self.h)
        return self

    def count(self, level: int) -> int:
        return int(lib().orc_index_count(self.h, level))

    def find(self, prefix) -> int:
        p = _c(prefix, np.int32)
        if p.size == 0:
            p = np.zeros(1, np.int32)
            return int(lib().orc_index_find(self.h, _p(p), 0))
        return int(lib().orc_index_find(self.h, _p(p), len(prefix)))

    def rows(self, level: int):
        n = self.count(level)
        pfx = np.zeros((n, level), np.int32)
        bm = np.zeros((n, max(self.w_bm, 1)), np.uint64)
        bl = np.zeros((n, max(self.w_bl, 1)), np.uint64)
        lib().orc_index_rows(self.h, level, _p(pfx), _p(bm), _p(bl))
        return pfx, bm[:, : self.w_bm], bl[:, : self.w_bl]

    def user_blooms(self, user_locs) -> np.ndarray:
        """bloom(l) rows [n_loc, w_bl] of a request's locations (eq 8 operand)."""
        rows = np.zeros((max(len(user_locs), 1), max(self.w_bl, 1)), np.uint64)
        if self.w_bl:
            for j, g in enumerate(user_locs):
                lib().orc_bloom_row(int(g), self.bloom_bits, self.bloom_k, _p(rows[j]))
        return rows

    def mask_row(self, prefix, t: int, user_bm, user_locs, blooms=None) -> np.ndarray:
        """Mask words of one row; t < 0 marks a dead row.  ``blooms`` may hold
        the request's precomputed user_blooms(user_locs)."""
        words = (self.V + 63) // 64
        out = np.zeros(words, dtype=np.uint64)
        p = _c(prefix if t > 0 else [0], np.int32)
        ub = _c(user_bm, np.uint64)
        bl = self.user_blooms(user_locs) if blooms is None else _c(blooms, np.uint64)
        lib().orc_mask_row(self.h, _p(p), t, _p(ub), _p(bl), len(user_locs), _p(out))
        return out

    def __del__(self):
        try:
            if getattr(self, "h", None):
                lib().orc_index_destroy(self.h)
                self.h = None
        except Exception:
            pass


def build_index(w, sids, ads) -> Index:
    ix = Index(w.L, w.V, sids, w.w_bm, w.bloom_bits, w.bloom_k)
    ix.add_ads(ads.ad_sid, ads.rules, ads.geo_offsets, ads.geo_ids)
    return ix.finish()


def mask_bits_to_bool(words: np.ndarray, V: int) -> np.ndarray:
    w = np.asarray(words, dtype=np.uint64)
    bits = (w[..., :, None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)
    return bits.reshape(*w.shape[:-1], -1)[..., :V].astype(bool)


# ---------------------------------------------------------------------------
# O6, O8, O10
# ---------------------------------------------------------------------------

def log_softmax(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib().orc_log_softmax(_p(x), x.size, _p(out))
    return out


def topk(scores: np.ndarray, k: int):
    """Top-k over flat candidates: (score desc, index asc), -inf excluded."""
    s = _c(scores, np.float32)
    f = np.zeros(max(k, 1), np.uint32)
    v = np.zeros(max(k, 1), np.float32)
    n = lib().orc_topk(_p(s), s.size, k, _p(f), _p(v))
    return f[:n].copy(), v[:n].copy()


def cross_attn(q, K, Vv, B: int, M: int) -> np.ndarray:
    q = _c(q, np.float64)
    K = _c(K, np.float64)
    Vv = _c(Vv, np.float64)
    R, H, d = q.shape
    T = K.shape[2]
    assert R == B * M and K.shape == (B, H, T, d) and Vv.shape == K.shape
    out = np.empty_like(q)
    lib().orc_cross_attn(_p(q), _p(K), _p(Vv), B, M, H, T, d, _p(out))
    return out


def self_attn(q, hk, hv, valid) -> np.ndarray:
    q = _c(q, np.float64)
    hk = _c(hk, np.float64)
    hv = _c(hv, np.float64)
    va = _c(valid, np.uint8)
    R, H, d = q.shape
    T = hk.shape[1]
    assert hk.shape == (R, T, H, d) and va.shape == (R, T) and T <= 64
    out = np.empty_like(q)
    lib().orc_self_attn(_p(q), _p(hk), _p(hv), _p(va), R, T, H, d, _p(out))
    return out


def joint_attn(q, K, Vv, hk, hv, valid, B: int, M: int) -> np.ndarray:
    """One softmax over request b's context keys followed by row r's own beam
    prefix positions (hk/hv [R, Tb, H, d], valid [R, Tb])."""
    q = _c(q, np.float64)
    K = _c(K, np.float64)
    Vv = _c(Vv, np.float64)
    hk = _c(hk, np.float64)
    hv = _c(hv, np.float64)
    va = _c(valid, np.uint8)
    R, H, d = q.shape
    T, Tb = K.shape[2], hk.shape[1]
    assert R == B * M and K.shape == (B, H, T, d) and Vv.shape == K.shape
    assert hk.shape == (R, Tb, H, d) and hv.shape == hk.shape and va.shape == (R, Tb)
    out = np.empty_like(q)
    lib().orc_joint_attn(_p(q), _p(K), _p(Vv), _p(hk), _p(hv), _p(va), B, M, H, T, Tb, d, _p(out))
    return out


# ---------------------------------------------------------------------------
# Large catalogs (too big for the prefix tables above): matcher unions of
# sampled prefixes from the catalog and the ad stream, and the mask logic
# applied to an Appendix A trie given as data.
# ---------------------------------------------------------------------------

def prefix_codes(sids: np.ndarray, level: int, V: int) -> np.ndarray:
    """Base-V code t_1 V^(l-1) + ... + t_l of each SID's length-l prefix."""
    code = np.zeros(sids.shape[0], np.int64)
    for j in range(level):
        code = code * V + sids[:, j].astype(np.int64)
    return code


class SampledUnions:
    """bitmask(p) and bloom(p) (eqs 4 and 9) of chosen prefixes p, each the
    OR over the ads of every catalog SID that starts with p."""

    def __init__(self, w, sids: np.ndarray, samples: dict):
        """samples: {level: sorted int64 prefix codes}."""
        self._sids = _c(sids, np.int32)
        self.w, self.samples = w, samples
        self.h = lib().orc_usample_create(w.L, w.V, w.w_bm, w.bloom_bits, w.bloom_k,
                                          _p(self._sids), self._sids.shape[0])
        for level, codes in samples.items():
            c = _c(codes, np.int64)
            assert (np.diff(c) > 0).all()
            lib().orc_usample_set_level(self.h, level, _p(c), c.size)

    def add_ads(self, ad_sid, rules, geo_off, geo_ids):
        a = _c(ad_sid, np.int64)
        r = _c(rules, np.uint64)
        go = _c(geo_off, np.int64)
        gi = _c(geo_ids, np.int32) if len(geo_ids) else np.zeros(1, np.int32)
        lib().orc_usample_add_ads(self.h, a.size, _p(a), _p(r), _p(go), _p(gi))

    def rows(self, level: int):
        n = self.samples[level].size
        bm = np.zeros((max(n, 1), self.w.w_bm), np.uint64)
        bl = np.zeros((max(n, 1), max(self.w.w_bl, 1)), np.uint64)
        lib().orc_usample_rows(self.h, level, _p(bm), _p(bl))
        return bm[:n], bl[:n, : self.w.w_bl]

    def __del__(self):
        try:
            if getattr(self, "h", None):
                lib().orc_usample_destroy(self.h)
                self.h = None
        except Exception:
            pass


class TrieAsData:
    """The oracle's mask logic (Appendix A Lookup, eqs 5 and 8) over an
    Appendix A trie given as arrays; the same mask_row / user_blooms
    interface as Index, so the decode walk can use either."""

    def __init__(self, w, arrays: dict):
        self.w, self.V, self.L = w, w.V, w.L
        self.w_bm, self.w_bl = w.w_bm, w.w_bl
        self.bloom_bits, self.bloom_k = w.bloom_bits, w.bloom_k
        self.a = {k: np.ascontiguousarray(arrays[k]) for k in
                  ("node_offsets", "child_nodes", "tokens", "bitmask_index", "bitmask_table")}
        if self.w_bl:
            for k in ("bloom_index", "bloom_table"):
                self.a[k] = np.ascontiguousarray(arrays[k])
        assert self.a["tokens"].dtype == np.int16 and self.a["node_offsets"].dtype == np.int32

    def user_blooms(self, user_locs) -> np.ndarray:
        rows = np.zeros((max(len(user_locs), 1), max(self.w_bl, 1)), np.uint64)
        if self.w_bl:
            for j, g in enumerate(user_locs):
                lib().orc_bloom_row(int(g), self.bloom_bits, self.bloom_k, _p(rows[j]))
        return rows

    def mask_row(self, prefix, t: int, user_bm, user_locs, blooms=None) -> np.ndarray:
        a = self.a
        out = np.zeros((self.V + 63) // 64, np.uint64)
        p = _c(prefix if t > 0 else [0], np.int32)
        ub = _c(user_bm, np.uint64)
        bl = self.user_blooms(user_locs) if blooms is None else _c(blooms, np.uint64)
        z = np.zeros(1, np.uint64)
        lib().orc_mask_row_csr(_p(a["node_offsets"]), _p(a["child_nodes"]), _p(a["tokens"]),
                               _p(a["bitmask_index"]),
                               _p(a["bloom_index"]) if self.w_bl else None,
                               _p(a["bitmask_table"]), self.w_bm,
                               _p(a["bloom_table"]) if self.w_bl else _p(z), self.w_bl, self.V,
                               _p(p), t, _p(ub), _p(bl), len(user_locs), _p(out))
        return out
