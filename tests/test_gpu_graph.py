"""A whole decode captured as one HIP graph (gr_decode_graph_create) and
replayed: every replay must reproduce the eager gr_decode_step chain on the
same inputs bit for bit.  Replays are interleaved with eager library and
torch work, and each replay's outputs are overwritten beforehand, so a node
that only worked on the first replay, or read stale state, is caught.
"""
import numpy as np
import pytest

from synth import workload as W
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


CASES = {
    "tiny": (W.WORKLOADS["tiny_fp32"], 0),
    "main_small": (W.WORKLOADS["main_b16_m1024"].scaled(n_sids=50_000, B=2,
                                                        schedule=(200, 300, 300, 300)), 1),
    "long_small": (W.WORKLOADS["longctx_b8"].scaled(n_sids=50_000, B=2, T_ctx=300,
                                                    schedule=(20, 300, 900)), 3),
    # a 1024-token context over few tiles: every step's cross-attention runs
    # split over the context (its workspace is part of the step arguments)
    "long_split": (W.WORKLOADS["longctx_b8"].scaled(n_sids=50_000, B=2, T_ctx=1024,
                                                    schedule=(20, 300, 900)), 3),
}


def _outputs(dec):
    res = {}
    for t in range(dec.L):
        res[f"parent{t}"] = dec.parent[t].cpu().numpy().copy()
        res[f"token{t}"] = dec.token[t].cpu().numpy().copy()
        res[f"cross{t}"] = dec.cross_out[t].float().cpu().numpy().copy()
        res[f"self{t}"] = dec.self_out[t].float().cpu().numpy().copy()
    for t in range(dec.L + 1):
        res[f"node{t}"] = dec.node[t].cpu().numpy().copy()
        res[f"acc{t}"] = dec.acc[t].cpu().numpy().view(np.uint32).copy()
        res[f"tokens{t}"] = dec.tokens[t].cpu().numpy().copy()
        res[f"table{t}"] = dec.table[t].cpu().numpy().copy()
    res["k_pool"] = dec.k_pool.float().cpu().numpy().copy()
    return res


def _scribble(dec):
    for t in range(dec.L):
        dec.parent[t].fill_(7)
        dec.token[t].fill_(7)
        dec.cross_out[t].fill_(3.0)
        dec.self_out[t].fill_(3.0)
        dec.node[t + 1].fill_(5)
        dec.acc[t + 1].fill_(1.0)
        dec.tokens[t + 1].fill_(9)
        dec.table[t + 1].fill_(9)
    dec.k_pool.fill_(2.0)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_graph_replays_match_eager(name):
    import wide_beam_sid_amd as gr
    from wide_beam_sid_amd.runner import Decoder
    w, seed = CASES[name]
    print(f"[graph] {name} seed={seed}", flush=True)
    sids = W.make_catalog(w, seed)
    ads = W.make_ads(w, seed, W.ad_counts(w, seed))
    req = W.make_requests(w, seed)
    kc, vc = W.make_context(w, seed)
    trie = gr.Trie.build(sids, w.V, w.w_bm, w.bloom_bits, w.bloom_k, [ads])
    probes = (gr.bloom_probes(req.locs.reshape(-1), w.bloom_bits, w.bloom_k)
              if w.bloom_bits else np.zeros((1, 1), np.uint32))
    ubm, upr = to_dev(req.user_bm), to_dev(probes)
    kct, vct = to_dev(kc, w.dtype), to_dev(vc, w.dtype)
    inputs = [{k: to_dev(v, w.dtype) for k, v in W.make_step(w, seed, t).items()}
              for t in range(w.L)]
    other = [{k: to_dev(v, w.dtype) for k, v in W.make_step(w, seed + 100, t).items()}
             for t in range(w.L)]
    args = (ubm, upr if w.bloom_bits else None, w.n_loc, kct, vct)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        eager = Decoder(trie, w.B, w.V, w.schedule, w.H, w.d_h, w.T_ctx, w.dtype)
        eager.run(*args, inputs)
        torch.cuda.synchronize()
        want = _outputs(eager)

        dec = Decoder(trie, w.B, w.V, w.schedule, w.H, w.d_h, w.T_ctx, w.dtype)
        g = dec.graph(*args, inputs, stream)
        torch.cuda.synchronize()
        for rep in range(3):
            _scribble(dec)
            g.launch(stream)
            torch.cuda.synchronize()
            got = _outputs(dec)
            for key, ref in want.items():
                assert np.array_equal(got[key], ref), f"{name} replay {rep}: {key}"
            # eager library and torch work between replays
            eager.run(*args, other)
            _ = (inputs[0]["logits"].float() * 2.0).sum()
            torch.cuda.synchronize()
            print(f"[graph] {name} replay {rep} ok", flush=True)
        g.close()


@pytest.mark.parametrize("name", ["tiny", "main_small", "long_split"])
def test_decode_graph_replay_matches_oracle(name):
    """The replayed graph itself against the CPU oracle, step by step (masks,
    scores, selection, reorder, block table, pool, attention), on two
    replays with eager work and scribbled outputs between them.  The split
    case runs every step's cross-attention split over the 1024-token
    context inside the graph."""
    import wide_beam_sid_amd as gr
    from wide_beam_sid_amd.runner import Decoder
    from tests.chain import ChainCheck
    w, seed = CASES[name]
    print(f"[graph-oracle] {name} seed={seed} T_ctx={w.T_ctx}", flush=True)
    sids = W.make_catalog(w, seed)
    ads = W.make_ads(w, seed, W.ad_counts(w, seed))
    req = W.make_requests(w, seed)
    kc, vc = W.make_context(w, seed)
    trie = gr.Trie.build(sids, w.V, w.w_bm, w.bloom_bits, w.bloom_k, [ads], keep_host=True)
    view = trie.host_view()
    probes = (gr.bloom_probes(req.locs.reshape(-1), w.bloom_bits, w.bloom_k)
              if w.bloom_bits else np.zeros((1, 1), np.uint32))
    ubm, upr = to_dev(req.user_bm), to_dev(probes)
    kct, vct = to_dev(kc, w.dtype), to_dev(vc, w.dtype)
    inp_np = [W.make_step(w, seed, t) for t in range(w.L)]
    inputs = [{k: to_dev(v, w.dtype) for k, v in x.items()} for x in inp_np]
    other = [{k: to_dev(v, w.dtype) for k, v in W.make_step(w, seed + 100, t).items()}
             for t in range(w.L)]
    args = (ubm, upr if w.bloom_bits else None, w.n_loc, kct, vct)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        dec = Decoder(trie, w.B, w.V, w.schedule, w.H, w.d_h, w.T_ctx, w.dtype, debug=True)
        if name == "long_split":
            assert dec.attn_ws is not None   # the split path is part of the graph
        g = dec.graph(*args, inputs, stream)
        eager = Decoder(trie, w.B, w.V, w.schedule, w.H, w.d_h, w.T_ctx, w.dtype)
        for rep in range(2):
            _scribble(dec)
            for t in range(dec.L):
                dec.dbg_mask[t].fill_(-1)
                dec.dbg_scores[t].fill_(5.0)
            torch.cuda.synchronize()
            g.launch(stream)
            torch.cuda.synchronize()
            chk = ChainCheck(w, seed, sids, ads, req, (kc, vc), view)
            for t in range(w.L):
                chk.check(dec, t, inp_np[t], later_steps_ran=True)
            chk.check_final(dec)
            eager.run(*args, other)
            torch.cuda.synchronize()
            print(f"[graph-oracle] {name} replay {rep} ok", flush=True)
        g.close()
