"""Step-by-step comparison of a chained GPU decode with the CPU oracle's walk
of the same decode loop (shared by the eager-chain and HIP-graph tests).

Per step: masks, selected parents / tokens / scores and child nodes are
bit-exact (top-k compared on the GPU's own fp32 scores), scores and attention
outputs within tolerance, block table and KV pool checked structurally.  The
oracle continues from its own selection, which the bit-exact checks have
just shown to be the GPU's, so a near-tie cannot cascade.
"""
import numpy as np

import oracle
from oracle.decode import initial_state, step as oracle_step
from synth import workload as W
from tests.helpers import attn_close, to_np64


class ChainCheck:
    """The oracle's side of one decode of workload ``w`` (seed ``seed``)."""

    def __init__(self, w, seed, sids, ads, req, ctx, view, sample_rows=None, mask_sample=None,
                 ix=None):
        """``ix``: the oracle's mask source (default: its prefix tables built
        from ``sids`` and ``ads``; for large catalogs, ``oracle.TrieAsData``
        over a trie whose rows were verified on sampled prefixes)."""
        self.w, self.seed, self.req, self.ctx = w, seed, req, ctx
        self.view = view
        self.ix = oracle.build_index(w, sids, ads) if ix is None else ix
        self.sids = sids
        self.st = initial_state(w)
        self.rng = np.random.default_rng(seed)
        self.sample_rows, self.mask_sample = sample_rows, mask_sample

    def check(self, dec, t, inp, later_steps_ran=False):
        """Compare step t of decoder ``dec`` (a debug decoder) with the
        oracle.  ``later_steps_ran``: the decode went on past step t before
        this check (a replayed graph), so step t + 1 has already written its
        own column of the block table it received."""
        import torch
        w, view = self.w, self.view
        npar, ntok, depth = view["node_parent"], view["node_token"], view["node_depth"]
        R = w.rows(t)
        as_f = lambda a: W.as_float(w, a)
        scores = dec.dbg_scores[t].cpu().numpy()
        rows = None
        if self.sample_rows is not None and R > self.sample_rows:
            rows = np.sort(self.rng.choice(R, size=self.sample_rows, replace=False))
        gmask = dec.dbg_mask[t].cpu().numpy().view(np.uint64)
        mrows = None
        if self.mask_sample is not None and R > self.mask_sample:
            mrows = np.sort(self.rng.choice(R, size=self.mask_sample, replace=False))
        ref = oracle_step(w, self.ix, self.req, self.ctx, t, self.st, inp, as_f,
                          gpu_scores=scores, rows_subset=rows, mask_rows=mrows, given_mask=gmask)
        # A3 mask (bit-exact on every row, or on the sampled rows), A4 scores
        assert np.array_equal(gmask, ref.mask), f"mask t={t}"
        fin = np.isfinite(ref.cand)
        assert np.array_equal(np.isfinite(scores), fin), f"finite t={t}"
        if fin.any():
            err = np.abs(scores[fin] - ref.cand[fin])
            assert (err <= 2e-5 + 2e-7 * np.abs(ref.cand[fin])).all(), f"scores t={t}: {err.max()}"
        # A5 selection
        parent = dec.parent[t].cpu().numpy()
        token = dec.token[t].cpu().numpy()
        assert np.array_equal(parent, ref.parent), f"parent t={t}"
        assert np.array_equal(token, ref.token), f"token t={t}"
        acc_out = dec.acc[t + 1].cpu().numpy()
        k = w.schedule[t]
        for b in range(w.B):
            n = ref.sel_s[b].size
            assert np.array_equal(acc_out[b * k:b * k + n].view(np.uint32), ref.sel_s[b].view(np.uint32))
            assert np.isneginf(acc_out[b * k + n:(b + 1) * k]).all()
        # A6 reorder: child nodes, token history, block table
        live = parent >= 0
        node_prev = dec.node[t].cpu().numpy()
        node_out = dec.node[t + 1].cpu().numpy()
        assert np.array_equal(npar[node_out[live]], node_prev[parent[live]])
        assert np.array_equal(ntok[node_out[live]], token[live])
        assert (depth[node_out[live]] == t + 1).all() and (node_out[~live] == -1).all()
        tokens = dec.tokens[t + 1].cpu().numpy()
        assert np.array_equal(tokens, ref.next_state.tokens), f"tokens t={t}"
        tab_prev = dec.table[t].cpu().numpy()
        tab = dec.table[t + 1].cpu().numpy()
        assert np.array_equal(tab_prev[:, t], dec.fresh[t] + np.arange(R))
        assert np.array_equal(tab[live, :t + 1], tab_prev[parent[live], :t + 1])
        if later_steps_ran and t + 1 < w.L:
            # step t + 1 wrote its fresh blocks into column t + 1 of every row
            assert np.array_equal(tab[:, t + 1], dec.fresh[t + 1] + np.arange(tab.shape[0]))
            assert (tab[live, t + 2:] == -1).all() and (tab[~live, :t + 1] == -1).all()
            assert (tab[~live, t + 2:] == -1).all()
        else:
            assert (tab[live, t + 1:] == -1).all() and (tab[~live] == -1).all()
        # A2 pool write, A1/A2 outputs
        kp = dec.k_pool[dec.fresh[t]:dec.fresh[t] + R].view(
            torch.int16 if w.dtype == "bf16" else torch.int32)
        kin = inp["k"].view(np.int16) if w.dtype == "bf16" else inp["k"].view(np.int32)
        assert np.array_equal(kp.cpu().numpy(), kin)
        sel = slice(None) if rows is None else rows
        attn_close(to_np64(dec.cross_out[t])[sel], ref.cross_out[sel], w.dtype, f"cross t={t}")
        attn_close(to_np64(dec.self_out[t])[sel], ref.self_out[sel], w.dtype, f"self t={t}")
        from tests.large import progress
        progress(f"[chain] {w.name} t={t} R={R} live_out={int(live.sum())} ok")
        self.st = ref.next_state

    def check_final(self, dec):
        """Every finished SID of a live beam is a catalog SID."""
        w = self.w
        final = dec.tokens[w.L].cpu().numpy()
        live = dec.node[w.L].cpu().numpy() >= 0
        cat = np.sort(oracle.prefix_codes(self.sids, w.L, w.V))
        got = oracle.prefix_codes(final[live], w.L, w.V)
        pos = np.minimum(np.searchsorted(cat, got), cat.size - 1)
        assert (cat[pos] == got).all()
