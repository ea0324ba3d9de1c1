"""Seeded synthetic workloads for the wide-beam SID decode step.

This module only draws random data: the SID catalog, the ads with their
targeting rules, the requests, and the per-step dense tensors.  It holds none
of the decode method's arithmetic (no matcher unions, no hashing into Bloom
filters, no attention, no scoring); the product library and the CPU oracle
each implement those on their own and both read the arrays made here.

Shapes follow the pages' workloads: GRACE (arXiv 2608.00938), Section 3.2
(encoder-decoder model), Section 3.3 (dynamic per-step beam sizes), Section 4
(bitmask and Bloom matchers, Table 1) and Section 6 (64 synthetic locations per
user), plus GR-Inference's long-context / 20->300->900-beam shape.

Sub-streams: every array family has its own stream id, and the generator for
(seed, stream, chunk) is numpy's PCG64 seeded through SeedSequence
([seed, stream, chunk]), so any chunk can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Iterator, Optional, Tuple

import numpy as np

# Stream ids: one per array family.
S_CATALOG = 1
S_AD_COUNT = 2
S_AD_RULES = 3
S_AD_GEO = 4
S_REQUEST = 5
S_CONTEXT = 6
S_STEP = 7


@dataclass(frozen=True)
class Workload:
    """One synthetic decode workload (all sizes explicit)."""

    name: str
    dtype: str                 # "f32" or "bf16": dtype of Q/K/V/logits
    B: int                     # requests per batch
    L: int                     # SID length (decode steps)
    V: int                     # codebook size per SID level
    schedule: Tuple[int, ...]  # per-step top-k width k_t (M_{t+1} = k_t)
    T_ctx: int                 # encoder context tokens per request
    H: int                     # attention heads
    d_h: int                   # head dim
    n_sids: int                # distinct catalog SIDs
    zipf_s: Optional[float]    # first-level Zipf exponent (None: uniform)
    ads_per_sid: Tuple[int, int]
    bm_segments: Tuple[int, ...]   # bit widths of the low-cardinality attributes
    bm_p: float                    # per-bit probability an ad allows a value
    bloom_bits: int                # Bloom width w (0: bitmask-only GTM)
    bloom_k: int                   # hash probes per id
    geo_pool: int                  # number of distinct geo ids
    geo_per_ad: Tuple[int, int]
    n_loc: int                     # user-side locations per request

    @property
    def w_bm(self) -> int:
        return (sum(self.bm_segments) + 63) // 64

    @property
    def w_bl(self) -> int:
        return self.bloom_bits // 64

    def rows(self, t: int) -> int:
        """Beam rows R_t entering step t (M_0 = 1, M_{t+1} = k_t)."""
        return self.B * (1 if t == 0 else self.schedule[t - 1])

    @property
    def total_rows(self) -> int:
        return sum(self.rows(t) for t in range(self.L))

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_BM64 = (48, 12, 4)  # country | age | gender

WORKLOADS = {
    # B=1, M=8, L=3, V=16, T_ctx=16, 2x32 heads, fp32, 200 SIDs, 1-3 ads,
    # 8-bit rule, 256-bit Bloom k=3, geo lists of 1-4 ids from 64.
    "tiny_fp32": Workload(
        name="tiny_fp32", dtype="f32", B=1, L=3, V=16, schedule=(8, 8, 8),
        T_ctx=16, H=2, d_h=32, n_sids=200, zipf_s=None, ads_per_sid=(1, 3),
        bm_segments=(4, 2, 2), bm_p=0.5, bloom_bits=256, bloom_k=3,
        geo_pool=64, geo_per_ad=(1, 4), n_loc=1),
    # GRACE's main shape: B=16, M=1024, L=4, V=256, T_ctx=64, 4x64 heads.
    "main_b16_m1024": Workload(
        name="main_b16_m1024", dtype="bf16", B=16, L=4, V=256,
        schedule=(1024, 1024, 1024, 1024), T_ctx=64, H=4, d_h=64,
        n_sids=1_000_000, zipf_s=1.1, ads_per_sid=(1, 8), bm_segments=_BM64,
        bm_p=0.3, bloom_bits=4096, bloom_k=4, geo_pool=100_000,
        geo_per_ad=(1, 32), n_loc=64),
    # Dynamic per-step widths 64->256->1024->1024.
    "dynamic_b32": Workload(
        name="dynamic_b32", dtype="bf16", B=32, L=4, V=256,
        schedule=(64, 256, 1024, 1024), T_ctx=256, H=8, d_h=64,
        n_sids=4_000_000, zipf_s=1.1, ads_per_sid=(1, 8), bm_segments=_BM64,
        bm_p=0.2, bloom_bits=4096, bloom_k=4, geo_pool=100_000,
        geo_per_ad=(1, 32), n_loc=64),
    # Long shared context: T_ctx=2048, 16x128 heads, widths 20->300->900,
    # bitmask-only GTM.
    "longctx_b8": Workload(
        name="longctx_b8", dtype="bf16", B=8, L=3, V=1024,
        schedule=(20, 300, 900), T_ctx=2048, H=16, d_h=128,
        n_sids=2_000_000, zipf_s=1.1, ads_per_sid=(1, 8), bm_segments=_BM64,
        bm_p=0.3, bloom_bits=0, bloom_k=0, geo_pool=0, geo_per_ad=(0, 0),
        n_loc=0),
    # Stress: B=64, M=1024, V=1024, 8192-bit Bloom k=5, geo 1-256 of 1M.
    "stress_b64": Workload(
        name="stress_b64", dtype="bf16", B=64, L=4, V=1024,
        schedule=(1024, 1024, 1024, 1024), T_ctx=512, H=8, d_h=64,
        n_sids=16_000_000, zipf_s=1.2, ads_per_sid=(1, 8), bm_segments=_BM64,
        bm_p=0.1, bloom_bits=8192, bloom_k=5, geo_pool=1_000_000,
        geo_per_ad=(1, 256), n_loc=64),
}


def rng(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, chunk])))


# ----------------------------------------------------------------------------
# bf16 storage helpers (data encoding only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_tensor(w: Workload, g: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) draws; bf16 workloads return uint16 bf16 bits, fp32 ones float32."""
    x = g.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if w.dtype == "bf16" else x


def as_float(w: Workload, a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(a) if w.dtype == "bf16" else np.asarray(a, dtype=np.float32)


# ----------------------------------------------------------------------------
# Catalog
# ----------------------------------------------------------------------------

def _first_level(w: Workload, g: np.random.Generator, n: int) -> np.ndarray:
    if w.zipf_s is None:
        return g.integers(0, w.V, size=n, dtype=np.int64)
    ranks = np.arange(1, w.V + 1, dtype=np.float64)
    p = ranks ** (-w.zipf_s)
    p /= p.sum()
    return g.choice(w.V, size=n, p=p).astype(np.int64)


def make_catalog(w: Workload, seed: int) -> np.ndarray:
    """n_sids distinct SIDs, int32 [n_sids, L], in draw order.

    First level Zipf(s) over V ranks (token = rank - 1), deeper levels
    uniform; duplicates are rejected until n_sids are distinct.
    """
    g = rng(seed, S_CATALOG)
    V, L = w.V, w.L
    assert V ** L >= 2 * w.n_sids, "codebook too small for the catalog"
    keys = np.empty(0, dtype=np.int64)
    need = w.n_sids
    while need > 0:
        n = need + need // 8 + 16
        first = _first_level(w, g, n)
        code = first
        for _ in range(1, L):
            code = code * V + g.integers(0, V, size=n, dtype=np.int64)
        cat = np.concatenate([keys, code])
        _, idx = np.unique(cat, return_index=True)
        idx.sort()
        keys = cat[idx][: w.n_sids]
        need = w.n_sids - keys.size
    sids = np.empty((w.n_sids, L), dtype=np.int32)
    code = keys.copy()
    for lvl in range(L - 1, -1, -1):
        sids[:, lvl] = (code % V).astype(np.int32)
        code //= V
    return sids


# ----------------------------------------------------------------------------
# Ads: targeting rules (bitmask) and geo allow-lists
# ----------------------------------------------------------------------------

def ad_counts(w: Workload, seed: int) -> np.ndarray:
    """Ads per SID, uniform on ads_per_sid (int32 [n_sids])."""
    lo, hi = w.ads_per_sid
    return rng(seed, S_AD_COUNT).integers(lo, hi + 1, size=w.n_sids, dtype=np.int32)


def _rules(w: Workload, g: np.random.Generator, n: int) -> np.ndarray:
    """Per-ad rule words u64 [n, w_bm]: each attribute segment's bits are
    Bernoulli(bm_p); an empty segment is redrawn so every ad is satisfiable.
    Bit b of the rule (segments laid out in order) is bit b % 64 of word
    b // 64."""
    bits = np.zeros((n, 64 * w.w_bm), dtype=bool)
    base = 0
    for width in w.bm_segments:
        seg = g.random((n, width)) < w.bm_p
        empty = ~seg.any(axis=1)
        while empty.any():
            seg[empty] = g.random((int(empty.sum()), width)) < w.bm_p
            empty = ~seg.any(axis=1)
        bits[:, base:base + width] = seg
        base += width
    packed = np.packbits(bits, axis=1, bitorder="little")      # byte j holds bits 8j..8j+7
    return np.ascontiguousarray(packed).view("<u8").astype(np.uint64, copy=False)


@dataclass
class AdChunk:
    """Ads [first_ad, first_ad + n) in global ad order (grouped by SID index)."""

    first_ad: int
    ad_sid: np.ndarray        # int64 [n]: catalog row of each ad
    rules: np.ndarray         # uint64 [n, w_bm]
    geo_offsets: np.ndarray   # int64 [n + 1], local to this chunk
    geo_ids: np.ndarray       # int32 [geo_offsets[-1]]


def _ad_chunk(w: Workload, seed: int, counts: np.ndarray, c: int, s0: int, s1: int,
              first_ad: int) -> AdChunk:
    cnt = counts[s0:s1]
    n = int(cnt.sum())
    ad_sid = np.repeat(np.arange(s0, s1, dtype=np.int64), cnt)
    rules = _rules(w, rng(seed, S_AD_RULES, c), n)
    if w.bloom_bits:
        g = rng(seed, S_AD_GEO, c)
        lo, hi = w.geo_per_ad
        ng = g.integers(lo, hi + 1, size=n, dtype=np.int64)
        offs = np.zeros(n + 1, dtype=np.int64)
        np.cumsum(ng, out=offs[1:])
        geo = g.integers(0, w.geo_pool, size=int(offs[-1]), dtype=np.int32)
    else:
        offs = np.zeros(n + 1, dtype=np.int64)
        geo = np.zeros(0, dtype=np.int32)
    return AdChunk(first_ad, ad_sid, rules, offs, geo)


def iter_ads(w: Workload, seed: int, counts: np.ndarray,
             sids_per_chunk: int = 1 << 18, workers: int = 1) -> Iterator[AdChunk]:
    """Stream the ads of SIDs in catalog order, chunk by chunk.

    Chunk c covers SIDs [c*sids_per_chunk, (c+1)*sids_per_chunk); its rules and
    geo lists come from sub-streams keyed by c, so it can be regenerated alone
    (and ``workers`` threads draw the next chunks while the caller consumes
    one; the chunks and their order do not depend on it).  Geo ids are drawn
    with replacement from the pool (a list with a repeated id is the same
    allow-set).
    """
    n_sids = counts.size
    starts = list(range(0, n_sids, sids_per_chunk))
    firsts = np.concatenate([[0], np.cumsum([int(counts[s0:s0 + sids_per_chunk].sum())
                                              for s0 in starts])])
    jobs = [(c, s0, min(n_sids, s0 + sids_per_chunk), int(firsts[c]))
            for c, s0 in enumerate(starts)]
    if workers <= 1:
        for c, s0, s1, fa in jobs:
            yield _ad_chunk(w, seed, counts, c, s0, s1, fa)
        return
    from collections import deque
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=workers) as ex:
        pending = deque()
        it = iter(jobs)
        for job in it:
            pending.append(ex.submit(_ad_chunk, w, seed, counts, *job))
            if len(pending) >= workers:
                break
        while pending:
            ch = pending.popleft().result()
            for job in it:
                pending.append(ex.submit(_ad_chunk, w, seed, counts, *job))
                break
            yield ch


def make_ads(w: Workload, seed: int, counts: np.ndarray) -> AdChunk:
    """All ads in one chunk (small and medium catalogs)."""
    chunks = list(iter_ads(w, seed, counts))
    if len(chunks) == 1:
        return chunks[0]
    offs = [np.zeros(1, dtype=np.int64)]
    base = 0
    for ch in chunks:
        offs.append(ch.geo_offsets[1:] + base)
        base += int(ch.geo_offsets[-1])
    return AdChunk(0, np.concatenate([c.ad_sid for c in chunks]),
                   np.concatenate([c.rules for c in chunks]),
                   np.concatenate(offs),
                   np.concatenate([c.geo_ids for c in chunks]))


# ----------------------------------------------------------------------------
# Requests
# ----------------------------------------------------------------------------

@dataclass
class Requests:
    attrs: np.ndarray      # int32 [B, n_attr]: chosen value per attribute
    user_bm: np.ndarray    # uint64 [B, w_bm]: one bit set per attribute
    locs: np.ndarray       # int32 [B, n_loc]: distinct user geo ids


def make_requests(w: Workload, seed: int) -> Requests:
    g = rng(seed, S_REQUEST)
    n_attr = len(w.bm_segments)
    attrs = np.zeros((w.B, n_attr), dtype=np.int32)
    user_bm = np.zeros((w.B, w.w_bm), dtype=np.uint64)
    base = 0
    for a, width in enumerate(w.bm_segments):
        val = g.integers(0, width, size=w.B)
        attrs[:, a] = val
        bit = base + val
        for b in range(w.B):
            user_bm[b, bit[b] // 64] |= np.uint64(1) << np.uint64(bit[b] % 64)
        base += width
    locs = np.zeros((w.B, w.n_loc), dtype=np.int32)
    for b in range(w.B):
        if w.n_loc:
            locs[b] = g.choice(w.geo_pool, size=w.n_loc, replace=False)
    return Requests(attrs, user_bm, locs)


# ----------------------------------------------------------------------------
# Dense per-request / per-step tensors
# ----------------------------------------------------------------------------

def make_context(w: Workload, seed: int):
    """Cross-attention K, V [B, H, T_ctx, d_h] (one per request)."""
    g = rng(seed, S_CONTEXT)
    shape = (w.B, w.H, w.T_ctx, w.d_h)
    return normal_tensor(w, g, shape), normal_tensor(w, g, shape)


def make_step(w: Workload, seed: int, t: int, rows: Optional[int] = None):
    """Per-step decoder outputs for R_t rows: cross-attention queries qx,
    self-attention q, k, v (each [R_t, H, d_h]) and logits [R_t, V]."""
    R = w.rows(t) if rows is None else rows
    g = rng(seed, S_STEP, t)
    shape = (R, w.H, w.d_h)
    return {
        "qx": normal_tensor(w, g, shape),
        "q": normal_tensor(w, g, shape),
        "k": normal_tensor(w, g, shape),
        "v": normal_tensor(w, g, shape),
        "logits": normal_tensor(w, g, (R, w.V)),
    }
