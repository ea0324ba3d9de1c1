"""Oracle for the post stage after decoding (GRACE Section 2.1 steps 3-4 and
Section 2.2): every finished SID is expanded into its ads through the
SID-to-ad index, and each ad goes through the exact ad-level target matcher.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Plain Python over the
synthetic catalog arrays; it shares nothing with the library.

Reading of the pages: the ad-level matcher applies the same targeting as the
trie matchers, at single-ad granularity and exactly: the bitmask part passes
when every bit the user sets is set in the ad's rule words (the eq 5 test on
one ad's rules instead of a union), the location part when one of the user's
locations is in the ad's geo list (set membership, no Bloom filter); an ad
passes when both do.  With no user locations (a bitmask-only setting) the
location part passes.  Parity status: pinned (tests/test_oracle_post.py).
"""
from __future__ import annotations

import numpy as np


def sid_to_ads(sids: np.ndarray, ad_sid: np.ndarray) -> dict:
    """SID tuple -> list of ad ids (ads in id order)."""
    rows = {}
    for a, s in enumerate(ad_sid.tolist()):
        rows.setdefault(s, []).append(a)
    return {tuple(sids[s].tolist()): ads for s, ads in rows.items()}


def ad_passes(a: int, rules: np.ndarray, geo_offsets: np.ndarray, geo_ids: np.ndarray,
              user_bm: np.ndarray, user_locs) -> tuple:
    """(bitmask part, location part) of the exact matcher for ad a."""
    bm_ok = all((int(rules[a, w]) & int(u)) == int(u) for w, u in enumerate(user_bm.tolist()))
    if len(user_locs) == 0:
        geo_ok = True
    else:
        geo = set(geo_ids[geo_offsets[a]:geo_offsets[a + 1]].tolist())
        geo_ok = any(int(l) in geo for l in user_locs)
    return bm_ok, geo_ok


def post_filter(index: dict, rules, geo_offsets, geo_ids, tokens: np.ndarray,
                rows_per_request: int, user_bm: np.ndarray, user_locs: np.ndarray):
    """Per finished row: [ads expanded, bitmask passes, location passes, both]
    (int64 [n, 4]) and the ids of the ads that pass, row by row.  A row with a
    token -1 (a dead slot) expands to nothing."""
    n = tokens.shape[0]
    counts = np.zeros((n, 4), np.int64)
    passing = []
    for r in range(n):
        b = r // rows_per_request
        row = tokens[r]
        if (row < 0).any():
            continue
        locs = user_locs[b].tolist() if user_locs is not None and user_locs.size else []
        for a in index.get(tuple(row.tolist()), []):
            bm_ok, geo_ok = ad_passes(a, rules, geo_offsets, geo_ids, user_bm[b], locs)
            counts[r] += (1, bm_ok, geo_ok, bm_ok and geo_ok)
            if bm_ok and geo_ok:
                passing.append(a)
    return counts, np.array(passing, np.int64)
