"""Pins of the post-stage oracle (SID -> ad expansion and the exact ad-level
matcher, GRACE Sections 2.1-2.2): a hand-worked example and brute-force
properties on a synthetic catalog."""
import numpy as np

from oracle import post
from synth import workload as W


def test_hand_worked_example():
    # 3 SIDs of length 2; ads: SID 0 -> ads 0, 1; SID 2 -> ad 2; SID 1 none
    sids = np.array([[0, 1], [1, 1], [2, 0]], np.int32)
    ad_sid = np.array([0, 0, 2], np.int64)
    # one rule word: bit 0 | bit 1 = attribute values the ad allows
    rules = np.array([[0b011], [0b010], [0b111]], np.uint64)
    geo_offsets = np.array([0, 2, 3, 5], np.int64)
    geo_ids = np.array([10, 11, 12, 10, 13], np.int32)
    ix = post.sid_to_ads(sids, ad_sid)
    assert ix == {(0, 1): [0, 1], (2, 0): [2]}
    tokens = np.array([[0, 1], [2, 0], [1, 1], [-1, -1]], np.int32)
    user_bm = np.array([[0b001], [0b010]], np.uint64)     # request 0 then 1
    locs = np.array([[11, 99], [13, 98]], np.int32)
    counts, passing = post.post_filter(ix, rules, geo_offsets, geo_ids, tokens, 2, user_bm, locs)
    # row 0 (request 0, SID 0): ad 0 bm 011&001 ok, geo {10,11} has 11 -> pass;
    #                           ad 1 bm 010&001 fails, geo {12} fails
    # row 1 (request 0, SID 2): ad 2 bm ok, geo {10,13} misses 11, 99
    # row 2 (request 1, SID 1): no ads; row 3: dead slot
    assert counts.tolist() == [[2, 1, 1, 1], [1, 1, 0, 0], [0, 0, 0, 0], [0, 0, 0, 0]]
    assert passing.tolist() == [0]
    # no locations: the location part passes
    counts, _ = post.post_filter(ix, rules, geo_offsets, geo_ids, tokens, 2, user_bm,
                                 np.zeros((2, 0), np.int32))
    assert counts[0].tolist() == [2, 1, 2, 1]


def test_brute_force_properties():
    w = W.WORKLOADS["main_b16_m1024"].scaled(n_sids=3000, B=3)
    sids = W.make_catalog(w, 7)
    ads = W.make_ads(w, 7, W.ad_counts(w, 7))
    req = W.make_requests(w, 7)
    ix = post.sid_to_ads(sids, ads.ad_sid)
    per_sid = np.bincount(ads.ad_sid, minlength=sids.shape[0])
    r = np.random.default_rng(1)
    pick = r.choice(sids.shape[0], size=60, replace=False)
    tokens = sids[pick]
    counts, passing = post.post_filter(ix, ads.rules, ads.geo_offsets, ads.geo_ids, tokens, 20,
                                       req.user_bm, req.locs)
    assert np.array_equal(counts[:, 0], per_sid[pick])            # every ad expanded once
    assert (counts[:, 3] <= counts[:, 1]).all() and (counts[:, 3] <= counts[:, 2]).all()
    assert (counts[:, 1] + counts[:, 2] - counts[:, 3] <= counts[:, 0]).all()
    assert passing.size == counts[:, 3].sum()
    # every passing ad really is eligible, checked against numpy set logic
    for a in passing.tolist():
        b = None
        for rr in range(tokens.shape[0]):
            if a in ix[tuple(tokens[rr].tolist())]:
                b = rr // 20
        assert b is not None
        geo = ads.geo_ids[ads.geo_offsets[a]:ads.geo_offsets[a + 1]]
        assert np.intersect1d(geo, req.locs[b]).size > 0
        assert ((ads.rules[a] & req.user_bm[b]) == req.user_bm[b]).all()
