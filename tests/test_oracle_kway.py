"""Pins of the k-way partition oracle (GRACE Section 4.2, Figure 3), and the
library's partitions (host copies of a built trie) against it."""
import numpy as np
import pytest

import oracle
from oracle import kway
from synth import workload as W


def _case(n_sids=600, seed=3, **over):
    w = W.WORKLOADS["main_b16_m1024"].scaled(n_sids=n_sids, B=2, V=16, **over)
    sids = W.make_catalog(w, seed)
    ads = W.make_ads(w, seed, W.ad_counts(w, seed))
    return w, sids, ads


def test_greedy_hand_example():
    # rows (one word), k = 2: the first goes to partition 0; the second
    # costs 2 bits in partition 0 but 1 bit alone in the empty partition 1;
    # the third costs 4 bits with 0011 and 3 bits with 0001, so it joins 1
    rows = np.array([[0b0011], [0b0001], [0b1100]], np.uint64)
    parts = kway.greedy(rows, 2)
    assert [int(p[0]) for p in parts] == [0b0011, 0b1101]
    # a row that adds no bit to a partition that already has the same bits
    # ties with an empty one and takes the lower index
    rows3 = np.array([[0b0110], [0b0110], [0b1000]], np.uint64)
    assert [int(p[0]) for p in kway.greedy(rows3, 3)] == [0b0110, 0b1000]
    # one partition: the union; as many partitions as distinct single bits:
    # each row alone
    assert [int(p[0]) for p in kway.greedy(rows, 1)] == [0b1111]
    rows2 = np.array([[0b01], [0b10], [0b100]], np.uint64)
    assert [int(p[0]) for p in kway.greedy(rows2, 3)] == [0b01, 0b10, 0b100]


def test_partition_properties():
    w, sids, ads = _case()
    rows = kway.leaf_rows(sids, ads, w.w_bm, w.bloom_bits, w.bloom_k)
    for prefix in [(int(sids[0, 0]),), tuple(sids[5, :2].tolist()), tuple(sids[9, :3].tolist())]:
        desc = sorted(s for s in rows if s[:len(prefix)] == prefix)
        union = np.bitwise_or.reduce(np.array([rows[s] for s in desc]), axis=0)
        for mode, kw in [(1, dict(k_static=(4, 4, 4, 2))), (1, dict(k_static=(1, 1, 1, 1))),
                         (2, dict(k_max=8, target=0.05))]:
            parts = kway.node_partitions(rows, prefix, mode, **kw)
            # the partitions cover the subtree union exactly and are no more than k
            assert np.array_equal(np.bitwise_or.reduce(np.array(parts), axis=0), union)
            if mode == 1:
                assert len(parts) <= kw["k_static"][len(prefix) - 1]
                if kw["k_static"][0] == 1:
                    assert len(parts) == 1
            else:
                assert 1 <= len(parts) <= 8


def test_kway_masks_between_exact_and_one_union():
    """A k-way decision keeps every prefix with an exactly eligible ad (no
    false negatives) and keeps no prefix the one-union matcher drops."""
    w, sids, ads = _case(n_sids=400, seed=5)
    req = W.make_requests(w.scaled(B=2), 5)
    rows = kway.leaf_rows(sids, ads, w.w_bm, w.bloom_bits, w.bloom_k)
    blooms = [oracle.bloom_row(int(l), w.bloom_bits, w.bloom_k) for l in req.locs[0]]
    ubm = req.user_bm[0]
    geo = {a: set(ads.geo_ids[ads.geo_offsets[a]:ads.geo_offsets[a + 1]].tolist())
           for a in range(ads.ad_sid.size)}
    ad_of = {}
    for a, s in enumerate(ads.ad_sid.tolist()):
        ad_of.setdefault(tuple(sids[s].tolist()), []).append(a)
    locs = set(req.locs[0].tolist())
    prefixes = sorted({tuple(s[:l]) for s in rows for l in (1, 2, 3)})
    for p in prefixes:
        desc = [s for s in rows if s[:len(p)] == p]
        exact = any(((ads.rules[a] & ubm) == ubm).all() and geo[a] & locs
                    for s in desc for a in ad_of[s])
        one = kway.passes([np.bitwise_or.reduce(np.array([rows[s] for s in desc]), axis=0)],
                          ubm, blooms, w.w_bm)
        kk = kway.passes(kway.node_partitions(rows, p, 1, k_static=(4, 4, 4, 2)), ubm, blooms,
                         w.w_bm)
        assert (not exact) or kk, p
        assert (not kk) or one, p


@pytest.mark.parametrize("mode,kw", [(1, dict(kway_k=(8, 4, 3, 2))),
                                     (2, dict(kway_kmax=8, kway_target_fill=0.1))])
def test_library_partitions_match_oracle(mode, kw):
    import wide_beam_sid_amd as gr
    w, sids, ads = _case(n_sids=500, seed=7)
    t = gr.Trie.build(sids, w.V, w.w_bm, w.bloom_bits, w.bloom_k, [ads], keep_host=True,
                      host_only=True, kway_mode=mode, **kw)
    v = t.host_view()
    rows = kway.leaf_rows(sids, ads, w.w_bm, w.bloom_bits, w.bloom_k)
    okw = (dict(k_static=kw["kway_k"]) if mode == 1
           else dict(k_max=kw["kway_kmax"], target=kw["kway_target_fill"]))
    off, kb, kl = v["kway_offsets"], v["kway_bitmask_index"], v["kway_bloom_index"]
    bm, bl = v["bitmask_table"], v["bloom_table"]
    npar, ntok, depth = v["node_parent"], v["node_token"], v["node_depth"]
    checked = 0
    for node in range(1, v["num_nodes"]):
        # the node's prefix, from the parent chain
        pre, n = [], node
        while n > 0:
            pre.append(int(ntok[n]))
            n = int(npar[n])
        prefix = tuple(reversed(pre))
        e = node - 1
        got = [np.concatenate([bm[kb[q]], bl[kl[q]]]) for q in range(off[e], off[e + 1])]
        want = kway.node_partitions(rows, prefix, mode, **okw)
        assert len(got) == len(want), prefix
        for a, b in zip(got, want):
            assert np.array_equal(a, b), prefix
        checked += 1
    assert checked == v["num_nodes"] - 1
