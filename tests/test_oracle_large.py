"""Pins of the oracle parts for catalogs too large for its prefix tables:
the sampled-prefix unions (eqs 4 and 9 from the catalog and the ad stream)
and the mask logic applied to an Appendix A trie given as data.  Both are
checked on small catalogs against the prefix tables, which the brute-force
tests pin."""
import numpy as np
import pytest

import oracle
from synth import workload as W

CASES = {
    "tiny": (W.WORKLOADS["tiny_fp32"], 0),
    "deep": (W.WORKLOADS["tiny_fp32"].scaled(L=4, V=6, n_sids=400), 1),
    "main_20k": (W.WORKLOADS["main_b16_m1024"].scaled(n_sids=20_000), 1),
    "long_20k": (W.WORKLOADS["longctx_b8"].scaled(n_sids=20_000), 3),
    "stress_5k": (W.WORKLOADS["stress_b64"].scaled(n_sids=5_000, geo_per_ad=(1, 40)), 4),
}


def _setup(name):
    w, seed = CASES[name]
    sids = W.make_catalog(w, seed)
    counts = W.ad_counts(w, seed)
    # several chunks (each chunk's ads come from its own sub-streams, so the
    # prefix tables are built from the same chunks, concatenated)
    chunks = list(W.iter_ads(w, seed, counts, sids_per_chunk=max(1, w.n_sids // 5)))
    base = np.concatenate([[0], np.cumsum([int(c.geo_offsets[-1]) for c in chunks])])
    ads = W.AdChunk(0, np.concatenate([c.ad_sid for c in chunks]),
                    np.concatenate([c.rules for c in chunks]),
                    np.concatenate([[0]] + [c.geo_offsets[1:] + base[i]
                                            for i, c in enumerate(chunks)]).astype(np.int64),
                    np.concatenate([c.geo_ids for c in chunks]))
    ix = oracle.build_index(w, sids, ads)
    return w, seed, sids, chunks, ix


@pytest.mark.parametrize("name", list(CASES))
def test_sampled_unions_equal_prefix_tables(name):
    """Each sampled prefix's rows equal the prefix tables' rows, with the ads
    fed in several chunks (about half the prefixes of each level sampled)."""
    w, seed, sids, chunks, ix = _setup(name)
    rng = np.random.default_rng(seed)
    samples, want = {}, {}
    for l in range(1, w.L + 1):
        pf, bm, bl = ix.rows(l)
        codes = oracle.prefix_codes(pf, l, w.V)
        pick = np.sort(rng.choice(codes.size, size=max(1, codes.size // 2), replace=False))
        order = np.argsort(codes[pick])
        samples[l] = codes[pick][order]
        want[l] = (bm[pick][order], bl[pick][order])
    su = oracle.SampledUnions(w, sids, samples)
    assert len(chunks) > 1
    for ch in chunks:
        su.add_ads(ch.ad_sid, ch.rules, ch.geo_offsets, ch.geo_ids)
    for l in range(1, w.L + 1):
        bm, bl = su.rows(l)
        assert np.array_equal(bm, want[l][0]), l
        assert np.array_equal(bl, want[l][1]), l


def _csr_from_prefix_tables(w, ix):
    """Appendix A arrays built here from the prefix tables: nodes numbered
    level by level in sorted prefix order, a node's child entries sorted by
    token, every entry's rows those of its child's prefix."""
    codes = {0: np.zeros(1, np.int64)}
    rows = {}
    for l in range(1, w.L + 1):
        pf, bm, bl = ix.rows(l)
        codes[l] = oracle.prefix_codes(pf, l, w.V)
        assert (np.diff(codes[l]) > 0).all()
        rows[l] = (bm, bl)
    base = {0: 0}
    for l in range(1, w.L + 1):
        base[l] = base[l - 1] + codes[l - 1].size
    n_nodes = base[w.L] + codes[w.L].size
    off = np.zeros(n_nodes + 1, np.int32)
    child, tok, bmi, bli = [], [], [], []
    bm_tab, bl_tab = [], []
    for l in range(0, w.L + 1):
        for i, c in enumerate(codes[l]):
            node = base[l] + i
            off[node] = len(child)
            if l == w.L:
                continue
            lo = np.searchsorted(codes[l + 1] // w.V, c, "left")
            hi = np.searchsorted(codes[l + 1] // w.V, c, "right")
            for j in range(lo, hi):
                child.append(base[l + 1] + j)
                tok.append(int(codes[l + 1][j] % w.V))
                bmi.append(len(bm_tab))
                bm_tab.append(rows[l + 1][0][j])
                bli.append(len(bl_tab))
                bl_tab.append(rows[l + 1][1][j])
    off[n_nodes] = len(child)
    return {"node_offsets": off, "child_nodes": np.array(child, np.int32),
            "tokens": np.array(tok, np.int16), "bitmask_index": np.array(bmi, np.int32),
            "bloom_index": np.array(bli, np.int32),
            "bitmask_table": np.array(bm_tab, np.uint64).reshape(-1, w.w_bm),
            "bloom_table": np.array(bl_tab, np.uint64).reshape(-1, max(w.w_bl, 1))[:, :w.w_bl]}


@pytest.mark.parametrize("name", list(CASES))
def test_mask_over_trie_data_equals_prefix_table_masks(name):
    """The Appendix A Lookup over a trie given as arrays gives the prefix
    tables' mask on every prefix of every depth (and on a prefix the catalog
    does not hold, and on a dead row), for several requests."""
    w, seed, sids, chunks, ix = _setup(name)
    td = oracle.TrieAsData(w, _csr_from_prefix_tables(w, ix))
    req = W.make_requests(w.scaled(B=3), seed)
    rng = np.random.default_rng(seed)
    prefixes = [[]]
    for l in range(1, w.L):
        pf = ix.rows(l)[0]
        take = pf if pf.shape[0] <= 300 else pf[rng.choice(pf.shape[0], 300, replace=False)]
        prefixes += [list(p) for p in take]
    missing = [int(v) for v in range(w.V)]
    root_tokens = set(int(x) for x in ix.rows(1)[0][:, 0])
    absent = [v for v in missing if v not in root_tokens]
    if absent:
        prefixes.append([absent[0]])
    n_kept = 0
    for b in range(3):
        blooms = ix.user_blooms(req.locs[b])
        for p in prefixes:
            t = len(p)
            got = td.mask_row(p, t, req.user_bm[b], req.locs[b], blooms)
            want = ix.mask_row(p, t, req.user_bm[b], req.locs[b], blooms)
            assert np.array_equal(got, want), (b, p)
            n_kept += int(np.unpackbits(got.view(np.uint8)).sum())
        assert not td.mask_row([], -1, req.user_bm[b], req.locs[b], blooms).any()
    assert n_kept > 0


@pytest.mark.parametrize("name", ["main_20k", "stress_5k", "long_20k"])
def test_mask_over_library_trie_equals_prefix_table_masks(name):
    """The library builder's Appendix A arrays, read as data by the oracle's
    mask logic, give the prefix tables' masks."""
    import wide_beam_sid_amd as gr
    w, seed, sids, chunks, ix = _setup(name)
    trie = gr.Trie.build(sids, w.V, w.w_bm, w.bloom_bits, w.bloom_k, chunks, host_only=True)
    td = oracle.TrieAsData(w, trie.host_view())
    req = W.make_requests(w.scaled(B=2), seed)
    rng = np.random.default_rng(seed + 1)
    for l in range(0, w.L):
        pf = ix.rows(l)[0] if l else np.zeros((1, 0), np.int32)
        take = pf if pf.shape[0] <= 200 else pf[rng.choice(pf.shape[0], 200, replace=False)]
        for b in range(2):
            blooms = ix.user_blooms(req.locs[b])
            for p in take:
                p = list(p)
                assert np.array_equal(td.mask_row(p, l, req.user_bm[b], req.locs[b], blooms),
                                      ix.mask_row(p, l, req.user_bm[b], req.locs[b], blooms))


def test_large_index_sampled_verification():
    """The large-catalog path end to end on a host-only trie: the library's
    rows of every sampled prefix (all of level 1, 3000 per deeper level)
    equal the oracle's unions accumulated from the same streamed ad chunks,
    children equal the catalog's next tokens, and the trie-as-data masks
    equal the prefix tables' on sampled rows."""
    from tests.large import build_verified_trie
    w = W.WORKLOADS["stress_b64"].scaled(n_sids=300_000, geo_per_ad=(1, 32))
    r = build_verified_trie(w, 4, n_sample=3000, host_only=True, workers=4)
    assert r["checked"] >= 3 * 3000 + 1
    sids = r["sids"]
    ads = W.make_ads(w, 4, W.ad_counts(w, 4))
    ix = oracle.build_index(w, sids, ads)
    req = W.make_requests(w.scaled(B=2), 4)
    rng = np.random.default_rng(0)
    for l in range(0, w.L):
        pf = ix.rows(l)[0] if l else np.zeros((1, 0), np.int32)
        for p in pf[rng.choice(pf.shape[0], min(50, pf.shape[0]), replace=False)]:
            p = list(p)
            blooms = ix.user_blooms(req.locs[0])
            assert np.array_equal(r["ix"].mask_row(p, l, req.user_bm[0], req.locs[0], blooms),
                                  ix.mask_row(p, l, req.user_bm[0], req.locs[0], blooms))
