"""Oracle for k-way partitioned matchers (GRACE Section 4.2 and Figure 3; the
decoding modes of Section 6).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Plain Python from the
catalog and the ads; shares nothing with the library.

The pages: k-way partitioning splits the descendants of a trie node into k
groups, each with its own union matcher, and a prefix is kept when at least
one group matches every attribute.  Static k-way fixes k per decoding
position and assigns each SID to the partition with the smallest fill after
adding the SID's matcher; dynamic k-way grows k per node until the union fill
reaches a target or k_max.  Readings where the pages leave a step open (the
library takes the same ones):
  * a node's descendants are its SIDs in ascending token order; a SID's rows
    are the OR of its ads' rows (eqs 4 and 9 at a leaf);
  * "fill" counts the set bits of the bitmask and Bloom rows together; on a
    tie the lowest partition index wins; empty partitions are dropped;
  * k never exceeds the node's SID count; dynamic k grows 1, 2, 4, ... and
    stops at the first k whose partitions' mean fill is <= the target, or at
    k_max.
Parity status: pinned (tests/test_oracle_kway.py).
"""
from __future__ import annotations

import numpy as np

from . import bloom_row


def _popcount_rows(rows: np.ndarray) -> np.ndarray:
    """Set bits per row of a uint64 matrix."""
    b = rows.view(np.uint8).reshape(rows.shape[0], -1)
    return np.unpackbits(b, axis=1).sum(axis=1).astype(np.int64)


def leaf_rows(sids: np.ndarray, ads, w_bm: int, bloom_bits: int, bloom_k: int) -> dict:
    """SID tuple -> its rows: the OR of its ads' rule words, then (if there
    is a Bloom matcher) the OR of its ads' Bloom rows."""
    w_bl = bloom_bits // 64
    out = {}
    cache = {}
    for a, s in enumerate(ads.ad_sid.tolist()):
        key = tuple(sids[s].tolist())
        row = out.setdefault(key, np.zeros(w_bm + w_bl, np.uint64))
        row[:w_bm] |= ads.rules[a]
        if w_bl:
            for g in ads.geo_ids[ads.geo_offsets[a]:ads.geo_offsets[a + 1]].tolist():
                if g not in cache:
                    cache[g] = bloom_row(g, bloom_bits, bloom_k)
                row[w_bm:] |= cache[g]
    return out


def greedy(rows: np.ndarray, k: int) -> list:
    """Assign the rows (in order) to k partitions: each to the one whose union
    gets the fewest set bits; returns the non-empty unions, by index."""
    W = rows.shape[1]
    P = np.zeros((k, W), np.uint64)
    used = np.zeros(k, bool)
    for r in rows:
        cost = _popcount_rows(P | r)
        j = int(np.argmin(cost))            # the first minimum: lowest index
        P[j] |= r
        used[j] = True
    return [P[j].copy() for j in range(k) if used[j]]


def partitions(desc_rows: np.ndarray, depth: int, mode: int, k_static=(), k_max: int = 0,
               target: float = 0.0) -> list:
    """Partition unions of a node at `depth` (1-based decoding position)
    whose descendant SIDs have rows desc_rows (ascending SID order)."""
    n = desc_rows.shape[0]
    if mode == 1:
        return greedy(desc_rows, min(k_static[depth - 1], n))
    cap = min(k_max, n)
    k = 1
    while True:
        parts = greedy(desc_rows, k)
        bits = 64 * desc_rows.shape[1]
        fill = sum(int(_popcount_rows(p[None])[0]) for p in parts) / (len(parts) * bits)
        if fill <= target or k >= cap:
            return parts
        k = min(2 * k, cap)


def node_partitions(rows_by_sid: dict, prefix: tuple, mode: int, **kw) -> list:
    """Partitions of the trie node for `prefix` (a tuple of tokens)."""
    l = len(prefix)
    desc = sorted(s for s in rows_by_sid if s[:l] == prefix)
    return partitions(np.array([rows_by_sid[s] for s in desc]), l, mode, **kw)


def passes(parts: list, user_bm: np.ndarray, user_blooms: list, w_bm: int) -> bool:
    """Kept if one partition passes eq 5 and (with a Bloom matcher) eq 8 for
    ANY of the user's location rows."""
    for p in parts:
        bm = p[:w_bm]
        if not np.array_equal(bm & user_bm, user_bm):
            continue
        if p.size == w_bm:
            return True
        bl = p[w_bm:]
        if any(np.array_equal(bl & u, u) for u in user_blooms):
            return True
    return False
