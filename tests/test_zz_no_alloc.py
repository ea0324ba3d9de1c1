"""gr_constrain_topk_noalloc (the tail with the library's own scratch, for
callers that cannot allocate) against gr_constrain_topk with a caller
workspace: the same outputs bit for bit, on two calls in a row, the second
smaller than the first (the scratch still holds the first call's data)."""
import ctypes

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


_OUT = ("parent_out", "token_out", "node_out", "acc_out", "tokens_out", "table_out",
        "dbg_mask", "dbg_scores")


def _call(lib, trie, w, view, B, M_in, k_out, t, seed, noalloc):
    import wide_beam_sid_amd as gr
    from wide_beam_sid_amd import _lib
    print(f"[noalloc] B={B} M_in={M_in} k={k_out} t={t} noalloc={noalloc}", flush=True)
    rng = np.random.default_rng(seed)
    R, L = B * M_in, w.L
    depth_nodes = np.nonzero(view["node_depth"] == t)[0]
    node_in = rng.choice(depth_nodes, size=R).astype(np.int32)
    node_in[rng.random(R) < 0.1] = -1
    acc_in = (-rng.random(R) * 4).astype(np.float32)
    acc_in[node_in < 0] = -np.inf
    logits = W.normal_tensor(w, rng, (R, w.V))
    req = W.make_requests(w.scaled(B=B), seed)
    probes = gr.bloom_probes(req.locs.reshape(-1), w.bloom_bits, w.bloom_k)
    tokens_in = rng.integers(0, w.V, size=(R, L)).astype(np.int32)
    table_in = rng.integers(0, 10**6, size=(R, L)).astype(np.int32)
    dev = {k: to_dev(v) for k, v in dict(node_in=node_in, acc_in=acc_in, tokens_in=tokens_in,
                                         table_in=table_in, user_bm=req.user_bm,
                                         user_probes=probes).items()}
    dev["logits"] = to_dev(logits, w.dtype)
    Rn = B * k_out
    i32, cu = torch.int32, "cuda"
    # outputs start as garbage so that every element must be written
    out = dict(parent_out=torch.full((Rn,), 7, dtype=i32, device=cu),
               token_out=torch.full((Rn,), 7, dtype=i32, device=cu),
               node_out=torch.full((Rn,), 7, dtype=i32, device=cu),
               acc_out=torch.full((Rn,), 7.0, dtype=torch.float32, device=cu),
               tokens_out=torch.full((Rn, L), 7, dtype=i32, device=cu),
               table_out=torch.full((Rn, L), 7, dtype=i32, device=cu),
               dbg_mask=torch.full((R, (w.V + 63) // 64), 7, dtype=torch.int64, device=cu),
               dbg_scores=torch.full((R, w.V), 7.0, dtype=torch.float32, device=cu))
    ws_bytes = gr.constrain_topk_workspace(B, M_in, w.V, k_out)
    ws = None if noalloc else torch.zeros(ws_bytes, dtype=torch.uint8, device=cu)
    args = gr.tail_args(B=B, M_in=M_in, V=w.V, k_out=k_out, t=t, L=L, n_loc=w.n_loc,
                        dtype=gr.GR_BF16, user_bm=dev["user_bm"], user_probes=dev["user_probes"],
                        logits=dev["logits"], node_in=dev["node_in"], acc_in=dev["acc_in"],
                        tokens_in=dev["tokens_in"], table_in=dev["table_in"],
                        ws=ws, ws_bytes=0 if noalloc else ws_bytes, **out)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    fn = lib.gr_constrain_topk_noalloc if noalloc else lib.gr_constrain_topk
    st = fn(trie.h, ctypes.byref(args), stream)
    assert st == _lib.GR_OK, lib.gr_last_error()
    return out


def _bits(x):
    if x.dtype == torch.float32:
        x = x.view(torch.int32)
    return x.cpu().numpy()


def test_noalloc_tail_equals_workspace_tail_on_consecutive_calls():
    import wide_beam_sid_amd as gr
    from wide_beam_sid_amd import _lib
    lib = _lib.lib()
    w = W.WORKLOADS["main_b16_m1024"].scaled(n_sids=50_000)
    seed = 1
    sids = W.make_catalog(w, seed)
    ads = W.make_ads(w, seed, W.ad_counts(w, seed))
    trie = gr.Trie.build(sids, w.V, w.w_bm, w.bloom_bits, w.bloom_k, [ads], keep_host=True)
    view = trie.host_view()
    calls = [(8, 1024, 1024, 1, 11),   # the larger call first
             (3, 200, 500, 2, 12)]     # then a smaller one over the same scratch
    got = [_call(lib, trie, w, view, *c, noalloc=True) for c in calls]
    torch.cuda.synchronize()
    got = [{k: _bits(v) for k, v in o.items()} for o in got]
    for c, g in zip(calls, got):
        ref = _call(lib, trie, w, view, *c, noalloc=False)
        torch.cuda.synchronize()
        for k in _OUT:
            assert np.array_equal(g[k], _bits(ref[k])), (c, k)
        assert (g["parent_out"] >= 0).any()
    # a third call repeats the first: the smaller call in between left
    # nothing behind that changes it
    again = _call(lib, trie, w, view, *calls[0], noalloc=True)
    torch.cuda.synchronize()
    for k in _OUT:
        assert np.array_equal(_bits(again[k]), got[0][k]), k


def test_noalloc_tail_refuses_shapes_beyond_its_scratch():
    import wide_beam_sid_amd as gr
    from wide_beam_sid_amd import _lib
    lib = _lib.lib()
    # 64 x 1024 x 1024 candidates need far more than the 128 MiB scratch
    assert gr.constrain_topk_workspace(64, 1024, 1024, 1024) > (128 << 20)
    w = W.WORKLOADS["tiny_fp32"]
    sids = W.make_catalog(w, 0)
    trie = gr.Trie.build(sids, w.V, w.w_bm, w.bloom_bits, w.bloom_k,
                         [W.make_ads(w, 0, W.ad_counts(w, 0))])
    buf = torch.zeros(64, dtype=torch.uint8, device="cuda")
    a = gr.tail_args(B=64, M_in=1024, V=1024, k_out=1024, t=1, L=w.L, n_loc=1, dtype=gr.GR_F32,
                     user_bm=buf, user_probes=buf, logits=buf, node_in=buf, acc_in=buf,
                     parent_out=buf, token_out=buf, node_out=buf, acc_out=buf)
    assert lib.gr_constrain_topk_noalloc(trie.h, ctypes.byref(a), None) == _lib.GR_E_UNSUPPORTED
    assert b"scratch" in lib.gr_last_error()
