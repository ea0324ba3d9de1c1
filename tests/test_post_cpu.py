"""The library's post stage (gr_post_filter: SID -> ad expansion and the exact
ad-level matcher, host C++) against the post-stage oracle, on synthetic
catalogs: counts and passing ad ids bit-exact."""
import numpy as np
import pytest

import wide_beam_sid_amd as gr
from oracle import post
from synth import workload as W
from wide_beam_sid_amd import _lib

CASES = {
    "main": (W.WORKLOADS["main_b16_m1024"].scaled(n_sids=4000, B=4), 3),
    "dense_rules": (W.WORKLOADS["main_b16_m1024"].scaled(n_sids=2000, B=2, bm_p=0.8,
                                                          geo_pool=300), 5),
    "bitmask_only": (W.WORKLOADS["longctx_b8"].scaled(n_sids=3000, B=3, V=64), 6),
    "tiny": (W.WORKLOADS["tiny_fp32"], 1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_post_filter_matches_oracle(name):
    w, seed = CASES[name]
    sids = W.make_catalog(w, seed)
    ads = W.make_ads(w, seed, W.ad_counts(w, seed))
    req = W.make_requests(w, seed)
    ix = gr.AdIndex(sids, w.V, w.w_bm, [ads])
    r = np.random.default_rng(seed)
    per = 40
    rows = sids[r.integers(0, sids.shape[0], size=w.B * per)].copy()
    rows[r.random(rows.shape[0]) < 0.1] = -1                    # dead slots
    off = r.random(rows.shape[0]) < 0.05                         # SIDs not in the catalog
    rows[off, -1] = (rows[off, -1] + 1) % w.V
    locs = req.locs if w.n_loc else None
    got, gids = ix.post_filter(rows, per, req.user_bm, locs, n_threads=3)
    oi = post.sid_to_ads(sids, ads.ad_sid)
    want, wids = post.post_filter(oi, ads.rules, ads.geo_offsets, ads.geo_ids, rows, per,
                                  req.user_bm, locs if locs is not None else np.zeros((w.B, 0)))
    assert np.array_equal(got, want), name
    assert np.array_equal(gids, wids), name
    assert got[:, 0].sum() > 0


def test_post_filter_chunked_ads_and_errors():
    w, seed = W.WORKLOADS["main_b16_m1024"].scaled(n_sids=3000, B=2), 9
    sids = W.make_catalog(w, seed)
    counts = W.ad_counts(w, seed)
    chunks = list(W.iter_ads(w, seed, counts, sids_per_chunk=700))   # several chunks
    assert len(chunks) > 1
    req = W.make_requests(w, seed)
    ix = gr.AdIndex(sids, w.V, w.w_bm, chunks)
    # the same ads as one set for the oracle (chunk-local geo offsets rebased)
    ad_sid = np.concatenate([c.ad_sid for c in chunks])
    rules = np.concatenate([c.rules for c in chunks])
    geo_ids = np.concatenate([c.geo_ids for c in chunks])
    offs, base = [np.zeros(1, np.int64)], 0
    for c in chunks:
        offs.append(c.geo_offsets[1:] + base)
        base += int(c.geo_offsets[-1])
    geo_offsets = np.concatenate(offs)
    oi = post.sid_to_ads(sids, ad_sid)
    rows = sids[:100]
    got, gids = ix.post_filter(rows, 50, req.user_bm, req.locs)
    want, wids = post.post_filter(oi, rules, geo_offsets, geo_ids, rows, 50, req.user_bm, req.locs)
    assert np.array_equal(got, want) and np.array_equal(gids, wids)
    L = _lib.lib()
    import ctypes
    out = ctypes.c_void_p()
    dup = np.ascontiguousarray(np.vstack([sids[:3], sids[:1]]), dtype=np.int32)
    assert L.gr_ad_index_create(dup.ctypes.data, 4, dup.shape[1], w.V, 1, ctypes.byref(out)) \
        == _lib.GR_E_INVALID
    assert b"repeat" in L.gr_last_error()
    # too small a pass_cap: counts are still written, the ids are refused
    tok = np.ascontiguousarray(rows, dtype=np.int32)
    ubm = np.ascontiguousarray(req.user_bm)
    locs = np.ascontiguousarray(req.locs)
    c = np.zeros((100, 4), np.int64)
    ids = np.zeros(1, np.int64)
    st = L.gr_post_filter(ix.h, tok.ctypes.data, 100, 50, ubm.ctypes.data, locs.ctypes.data,
                          locs.shape[1], c.ctypes.data, ids.ctypes.data, 0, 1)
    assert st == (_lib.GR_E_WORKSPACE if want[:, 3].sum() > 0 else _lib.GR_OK)
    assert np.array_equal(c, want)
