"""Index of a large catalog (too large for the oracle's prefix tables), built
by the library from the streamed ads while the oracle accumulates, from the
same ad chunks, the matcher unions of sampled prefixes (eqs 4 and 9); then
every sampled prefix is found in the library's trie by walking its CSR from
the root, and its bitmask and Bloom rows and its child tokens (eq 1, from
the catalog) are compared.  The decode tests then read the verified trie as
data with the oracle's mask logic (oracle.TrieAsData)."""
import os
import time

import numpy as np

import oracle
from synth import workload as W


def progress(msg: str) -> None:
    """A progress line on stdout and, since test output is captured, also
    appended to the file that GR_PROGRESS_LOG names, when it is set (a long
    test then shows that it is alive while pytest holds its output)."""
    print(msg, flush=True)
    path = os.environ.get("GR_PROGRESS_LOG")
    if not path:
        return
    try:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "a") as f:
            f.write(f"{time.strftime('%H:%M:%S')} {msg}\n")
    except OSError:
        pass


def build_verified_trie(w, seed, n_sample=10_000, host_only=False, workers=8, log=progress):
    import wide_beam_sid_amd as gr
    t0 = time.time()
    sids = W.make_catalog(w, seed)
    counts = W.ad_counts(w, seed)
    log(f"[large] {w.name}: catalog of {w.n_sids} SIDs, {int(counts.sum())} ads "
        f"({time.time() - t0:.0f} s)")
    rng = np.random.default_rng(seed + 12345)
    codes, samples = {}, {}
    for l in range(1, w.L + 1):
        c = np.unique(oracle.prefix_codes(sids, l, w.V))
        codes[l] = c
        samples[l] = c if (l == 1 or c.size <= n_sample) else \
            np.sort(rng.choice(c, n_sample, replace=False))
    log(f"[large] sampled prefixes per level: {[int(samples[l].size) for l in samples]} of "
        f"{[int(codes[l].size) for l in codes]}")
    su = oracle.SampledUnions(w, sids, samples)
    stats = dict(chunks=0, geo=0)

    def feed():
        for i, ch in enumerate(W.iter_ads(w, seed, counts, workers=workers)):
            su.add_ads(ch.ad_sid, ch.rules, ch.geo_offsets, ch.geo_ids)
            stats["chunks"] += 1
            stats["geo"] += int(ch.geo_offsets[-1])
            if i % 8 == 0:
                log(f"[large] ad chunk {i}: {stats['geo']} geo ids so far "
                    f"({time.time() - t0:.0f} s)")
            yield ch

    trie = gr.Trie.build(sids, w.V, w.w_bm, w.bloom_bits, w.bloom_k, feed(), keep_host=True,
                         host_only=host_only)
    info = trie.info()
    log(f"[large] trie built: {info} ({time.time() - t0:.0f} s)")
    view = trie.host_view(copy=False)
    off, child, tok = view["node_offsets"], view["child_nodes"], view["tokens"]
    bmi, bm_tab = view["bitmask_index"], view["bitmask_table"]
    bli, bl_tab = view["bloom_index"], view["bloom_table"]
    # the root's children are the catalog's first tokens (eq 1)
    assert np.array_equal(np.sort(tok[off[0]:off[1]]), codes[1])
    checked = 0
    for l in range(1, w.L + 1):
        bm_want, bl_want = su.rows(l)
        nxt = codes.get(l + 1)
        for i, code in enumerate(samples[l]):
            toks = [(int(code) // w.V ** (l - 1 - j)) % w.V for j in range(l)]
            node, e = 0, -1
            for tk in toks:                       # Appendix A: follow the child entries
                s0, s1 = int(off[node]), int(off[node + 1])
                hit = np.nonzero(tok[s0:s1] == tk)[0]
                assert hit.size == 1, (l, toks)
                e = s0 + int(hit[0])
                node = int(child[e])
            assert np.array_equal(bm_tab[bmi[e]], bm_want[i]), ("bitmask", l, toks)
            if w.bloom_bits:
                assert np.array_equal(bl_tab[bli[e]], bl_want[i]), ("bloom", l, toks)
            if nxt is not None:                   # eq 1: the catalog's next tokens
                lo = np.searchsorted(nxt, int(code) * w.V, "left")
                hi = np.searchsorted(nxt, int(code) * w.V + w.V, "left")
                want = (nxt[lo:hi] % w.V).astype(np.int64)
                got = np.sort(tok[off[node]:off[node + 1]].astype(np.int64))
                assert np.array_equal(got, want), ("children", l, toks)
            else:
                assert off[node] == off[node + 1]  # a full SID is a leaf
            checked += 1
    log(f"[large] {checked} sampled nodes verified against catalog-derived unions "
        f"({time.time() - t0:.0f} s)")
    return dict(trie=trie, view=view, sids=sids, samples=samples, checked=checked,
                ix=oracle.TrieAsData(w, view))
