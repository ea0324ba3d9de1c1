"""CPU-side checks of libgr.so: exports, argument validation, the host index
builder and the request-side Bloom encoding (no kernel is launched here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import wide_beam_sid_amd as gr
from synth import workload as W
from wide_beam_sid_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "gr.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gr_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), f"{n} declared in gr.h but not exported"
    assert set(names) == set(_lib.EXPORTS)


def test_bloom_probes_equal_oracle():
    r = np.random.default_rng(0)
    ids = r.integers(0, 2**31 - 1, size=500).astype(np.int32)
    for w_bits, k in [(256, 3), (4096, 4), (8192, 5), (64, 1)]:
        got = gr.bloom_probes(ids, w_bits, k)
        for i in range(0, ids.size, 7):
            assert got[i].tolist() == oracle.bloom_positions(int(ids[i]), w_bits, k).tolist()


def _status(fn, *args):
    return fn(*args)


def test_argument_errors_return_codes_without_launch():
    L = _lib.lib()
    # null pointers / bad shapes are rejected before any HIP call
    assert L.gr_cross_attn(None, None, None, None, 1, 1, 1, 1, 64, 1, None) == _lib.GR_E_INVALID
    buf = ctypes.c_void_p(16)
    assert L.gr_cross_attn(buf, buf, buf, buf, 1, 1, 1, 1, 48, 1, None) == _lib.GR_E_UNSUPPORTED
    assert L.gr_cross_attn(buf, buf, buf, buf, 0, 1, 1, 1, 64, 1, None) == _lib.GR_E_INVALID
    assert L.gr_cross_attn(buf, buf, buf, buf, 1, 1, 1, 1, 64, 7, None) == _lib.GR_E_INVALID
    assert b"dtype" in L.gr_last_error()
    # pool too small for the fresh blocks
    assert L.gr_self_attn_paged(buf, buf, buf, buf, buf, 10, buf, 8, 4, 0, 4, 2, 64, 1, buf,
                                None) == _lib.GR_E_INVALID
    assert b"pool" in L.gr_last_error()
    # t outside [0, L)
    assert L.gr_self_attn_paged(buf, buf, buf, buf, buf, 100, buf, 0, 4, 4, 4, 2, 64, 1, buf,
                                None) == _lib.GR_E_INVALID
    # split cross-attention: a workspace smaller than the plan, or not
    # 16-byte aligned, is refused before any launch
    need = L.gr_cross_attn_workspace(8, 1, 16, 2048, 128, 1)
    assert need > 0
    ws = ctypes.c_void_p(256)
    assert L.gr_cross_attn_ws(buf, buf, buf, buf, 8, 1, 16, 2048, 128, 1, ws, need - 16,
                              None) == _lib.GR_E_WORKSPACE
    assert L.gr_cross_attn_ws(buf, buf, buf, buf, 8, 1, 16, 2048, 128, 1, ctypes.c_void_p(264),
                              need, None) == _lib.GR_E_WORKSPACE
    assert L.gr_cross_attn_ws(None, buf, buf, buf, 8, 1, 16, 2048, 128, 1, ws, need,
                              None) == _lib.GR_E_INVALID
    assert L.gr_bloom_probes(None, 3, 4096, 4, None) == _lib.GR_E_INVALID
    assert L.gr_bloom_probes(None, 0, 1000, 4, None) == _lib.GR_E_INVALID
    assert gr.constrain_topk_workspace(16, 1024, 256, 1024) > 16 * 1024 * 256 * 12


def test_builder_rejects_bad_input():
    with pytest.raises(gr.GrError) as e:
        gr.Trie.build(np.array([[0, 5]], np.int32), 4, 1, 0, 0, [], host_only=True)
    assert e.value.status == _lib.GR_E_INVALID
    ch = W.AdChunk(0, np.array([3]), np.zeros((1, 1), np.uint64), np.zeros(2, np.int64),
                   np.zeros(0, np.int32))
    with pytest.raises(gr.GrError) as e:
        gr.Trie.build(np.array([[0, 1]], np.int32), 4, 1, 0, 0, [ch], host_only=True)
    assert "ad_sid" in str(e.value)


def test_host_only_trie_is_rejected_by_hot_path():
    t = gr.Trie.build(np.array([[0, 1]], np.int32), 4, 1, 0, 0, [], host_only=True)
    a = gr.tail_args(B=1, M_in=1, V=4, k_out=1, t=0, L=2, n_loc=0, dtype=0)
    st = _lib.lib().gr_constrain_topk(t.h, ctypes.byref(a), None)
    assert st == _lib.GR_E_INVALID


def _check_trie_against_oracle(w, seed):
    sids = W.make_catalog(w, seed)
    counts = W.ad_counts(w, seed)
    ads = W.make_ads(w, seed, counts)
    trie = gr.Trie.build(sids, w.V, w.w_bm, w.bloom_bits, w.bloom_k, [ads], host_only=True)
    v = trie.host_view()
    ix = oracle.build_index(w, sids, ads)
    n = v["num_nodes"]
    assert n == 1 + sum(ix.count(l) for l in range(1, w.L + 1))
    assert v["num_entries"] == n - 1
    depth, par, ntok = v["node_depth"], v["node_parent"], v["node_token"]
    off, child, tok = v["node_offsets"], v["child_nodes"], v["tokens"]
    # prefix of every node from the parent / token chain
    prefix = [()] * n
    for node in range(1, n):
        assert par[node] < node
        prefix[node] = prefix[par[node]] + (int(ntok[node]),)
        assert len(prefix[node]) == depth[node]
    for l in range(1, w.L + 1):
        pf, bm, bl = ix.rows(l)
        lookup = {tuple(p): i for i, p in enumerate(pf.tolist())}
        nodes = np.nonzero(depth == l)[0]
        assert len(nodes) == len(lookup)
        for node in nodes:
            i = lookup[prefix[node]]
            j = node - 1                          # the entry leading into the node
            assert child[j] == node and tok[j] == ntok[node]
            assert np.array_equal(v["bitmask_table"][v["bitmask_index"][j]], bm[i])
            if w.bloom_bits:
                assert np.array_equal(v["bloom_table"][v["bloom_index"][j]], bl[i])
    # CSR: children of a node are exactly the catalog's next tokens, sorted
    expect = {(): []}
    for l in range(1, w.L + 1):
        for p in ix.rows(l)[0].tolist():
            expect.setdefault(tuple(p[:-1]), []).append(p[-1])
    for node in range(n):
        toks = tok[off[node]:off[node + 1]].tolist()
        assert toks == sorted(expect.get(prefix[node], []))
    # deduplicated tables hold distinct rows
    for name in ("bitmask_table", "bloom_table"):
        tab = v[name]
        if tab.size:
            assert len({r.tobytes() for r in tab}) == tab.shape[0]
    return v


@pytest.mark.parametrize("name,w,seed", [
    ("tiny", W.WORKLOADS["tiny_fp32"], 0),
    ("tiny_s3", W.WORKLOADS["tiny_fp32"], 3),
    ("deep", W.WORKLOADS["tiny_fp32"].scaled(L=4, V=6, n_sids=400), 1),
    ("main_20k", W.WORKLOADS["main_b16_m1024"].scaled(n_sids=20_000), 1),
    ("longctx_20k", W.WORKLOADS["longctx_b8"].scaled(n_sids=20_000), 3),
    ("stress_5k", W.WORKLOADS["stress_b64"].scaled(n_sids=5_000, geo_per_ad=(1, 40)), 4),
], ids=lambda x: x if isinstance(x, str) else "")
def test_trie_builder_matches_oracle_unions(name, w, seed):
    v = _check_trie_against_oracle(w, seed)
    if name == "main_20k":
        # single-child chains share rows: fewer rows than non-root nodes
        assert v["bl_rows"] < v["num_entries"]


def test_decode_graph_argument_errors_without_capture():
    L = _lib.lib()
    out = ctypes.c_void_p(123)
    # no steps, no trie, no out: rejected before any stream or capture call
    assert L.gr_decode_graph_create(None, None, 0, ctypes.c_void_p(16), ctypes.byref(out)) \
        == _lib.GR_E_INVALID
    assert out.value is None
    assert L.gr_decode_graph_create(None, None, 1, ctypes.c_void_p(16), None) == _lib.GR_E_INVALID
    assert L.gr_decode_graph_launch(None, None) == _lib.GR_E_INVALID
    L.gr_decode_graph_destroy(None)   # no-op


def test_cross_attn_workspace_plan():
    """The split cross-attention is planned only for bf16 launches with few
    tiles and a long context; its workspace holds S * rows * heads * (d + 2)
    floats."""
    import wide_beam_sid_amd as gr
    assert gr.cross_attn_workspace(16, 1024, 4, 64, 64, "bf16") == 0      # short context
    assert gr.cross_attn_workspace(32, 64, 8, 256, 64, "bf16") == 0       # four key tiles
    assert gr.cross_attn_workspace(64, 1024, 8, 512, 64, "bf16") == 0     # many tiles
    assert gr.cross_attn_workspace(8, 1, 16, 2048, 128, "f32") == 0       # fp32 path
    n = gr.cross_attn_workspace(8, 1, 16, 2048, 128, "bf16")
    per_split = 8 * 1 * 16 * (128 + 2) * 4
    assert n > 0 and n % per_split == 0 and 2 <= n // per_split <= 16


def test_tail_shape_prefix_covers_every_segment_near_the_row_limit():
    """The select's prefix sums over a request's segment counts are written
    two per thread (1024 threads): entries 2 tid and 2 tid + 1 while they are
    <= gx, plus entry gx by the last thread when gx = 2048.  Every entry the
    select reads (0..gx) must have been written, for every row count up to
    the documented M_in limit of 65536, and gx never exceeds 2048."""
    threads = 1024
    for B in (1, 2, 16, 64):
        for M_in in list(range(65000, 65537)) + [1, 2, 31, 1024, 2048, 4096, 32768]:
            rw, gx, seg_cap = gr.constrain_topk_shape(B, M_in, 1024)
            assert 1 <= gx <= 2 * threads and 1 <= rw <= 32, (B, M_in, rw, gx)
            assert rw * gx >= M_in and (gx - 1) * rw < M_in   # every row, no empty workgroup
            assert seg_cap >= rw * 1024 and seg_cap % 8 == 0
            written = np.zeros(2 * threads + 1, bool)
            for tid in range(threads):
                if 2 * tid <= gx:
                    written[2 * tid] = True
                if 2 * tid + 1 <= gx:
                    written[2 * tid + 1] = True
                if gx == 2 * threads and tid == threads - 1:
                    written[gx] = True
            assert written[:gx + 1].all(), (B, M_in, gx)
    with pytest.raises(gr.GrError):
        gr.constrain_topk_shape(0, 1, 16)


def _step_args(H, d_h, T_ctx, dtype, B=1, M_in=1, V=4, L=2, pool=16):
    buf = 4096
    a = _lib.StepArgs()
    a.H, a.d_h, a.T_ctx = H, d_h, T_ctx
    for f in ("k_ctx", "v_ctx", "qx", "q", "k_new", "v_new", "k_pool", "v_pool", "cross_out",
              "self_out"):
        setattr(a, f, buf)
    a.pool_blocks, a.fresh_base = pool, 0
    a.tail = gr.tail_args(B=B, M_in=M_in, V=V, k_out=1, t=0, L=L, n_loc=0, dtype=dtype)
    for f in ("user_bm", "logits", "node_in", "acc_in", "tokens_in", "table_in", "parent_out",
              "token_out", "node_out", "acc_out", "ws"):
        setattr(a.tail, f, buf)
    return a


def test_decode_step_rejects_head_groups_the_self_attention_cannot_sum():
    """An fp32 head of d_h = 6, 12, 24 or 48 values spans 3, 6, 12 or 24
    lanes, which the self-attention's butterfly over a power-of-two lane group
    cannot sum: the decode step refuses it before any launch, as
    gr_self_attn_paged does.  A supported shape gets past the attention checks
    and is then refused for the host-only trie."""
    L = _lib.lib()
    t = gr.Trie.build(np.array([[0, 1]], np.int32), 4, 1, 0, 0, [], host_only=True)
    for d in (6, 12, 24, 48):
        a = _step_args(2, d, 8, _lib.GR_F32)
        assert L.gr_decode_step(t.h, ctypes.byref(a), None) == _lib.GR_E_UNSUPPORTED, d
        assert b"self-attention" in L.gr_last_error()
        buf = ctypes.c_void_p(4096)
        assert L.gr_self_attn_paged(buf, buf, buf, buf, buf, 16, buf, 0, 1, 0, 2, 2, d,
                                    _lib.GR_F32, buf, None) == _lib.GR_E_UNSUPPORTED
    for d in (2, 8, 32, 64):
        a = _step_args(2, d, 8, _lib.GR_F32)
        assert L.gr_decode_step(t.h, ctypes.byref(a), None) == _lib.GR_E_INVALID, d
        assert b"host_only" in L.gr_last_error()


def test_bf16_attention_refuses_extents_past_32_bits():
    """The bf16 cross-attention reads a request's queries and a head's context
    through 32-bit buffer extents: M*H*d_h*2 or T_ctx*d_h*2 of 2^32 bytes or
    more is refused (it would wrap and read zeros), below that it is not."""
    L = _lib.lib()
    b = ctypes.c_void_p(4096)
    bf = _lib.GR_BF16
    assert L.gr_cross_attn(b, b, b, b, 1, 1 << 20, 16, 64, 128, bf, None) == _lib.GR_E_UNSUPPORTED
    assert b"2^32" in L.gr_last_error()
    assert L.gr_cross_attn(b, b, b, b, 1, 1, 1, 1 << 24, 128, bf, None) == _lib.GR_E_UNSUPPORTED
    assert L.gr_joint_attn(b, b, b, b, b, b, b, 1 << 30, b, 0, 1, 1 << 20, 16, 64, 128, 0, 2,
                           bf, b, None) == _lib.GR_E_UNSUPPORTED
    need = L.gr_cross_attn_workspace(1, 1, 1, 1 << 24, 128, bf)
    assert L.gr_cross_attn_ws(b, b, b, b, 1, 1, 1, 1 << 24, 128, bf, ctypes.c_void_p(256),
                              max(need, 16), None) == _lib.GR_E_UNSUPPORTED
    t = gr.Trie.build(np.array([[0, 1]], np.int32), 4, 1, 0, 0, [], host_only=True)
    a = _step_args(1, 128, 1 << 24, bf)
    assert L.gr_decode_step(t.h, ctypes.byref(a), None) == _lib.GR_E_UNSUPPORTED
    # the fp32 path reads through plain pointers: no such limit
    a = _step_args(2, 32, 1 << 24, _lib.GR_F32)
    assert L.gr_decode_step(t.h, ctypes.byref(a), None) == _lib.GR_E_INVALID   # host-only trie


def _appendix_a_arrays(w, seed):
    sids = W.make_catalog(w, seed)
    ads = W.make_ads(w, seed, W.ad_counts(w, seed))
    t = gr.Trie.build(sids, w.V, w.w_bm, w.bloom_bits, w.bloom_k, [ads], host_only=True)
    v = t.host_view()
    keys = ("node_offsets", "child_nodes", "tokens", "bitmask_index", "bloom_index",
            "bitmask_table", "bloom_table")
    return {k: v[k].copy() for k in keys}, v


def test_trie_create_validates_every_appendix_a_field():
    """gr_trie_create (GRACE Appendix A layout from the caller) refuses each
    broken field with GR_E_INVALID and a message naming it, before anything
    is uploaded; the arrays of a built trie pass validation (without a GPU
    the upload then fails with GR_E_HIP, never GR_E_INVALID)."""
    w = W.WORKLOADS["tiny_fp32"]
    base, v = _appendix_a_arrays(w, 0)
    kw = dict(vocab_size=w.V, sid_length=w.L, w_bm=w.w_bm, bloom_bits=w.bloom_bits,
              bloom_k=w.bloom_k)
    off = base["node_offsets"]
    n_nodes, n_ent = off.size - 1, base["child_nodes"].size
    wide = int(np.argmax(np.diff(off)))          # a node with several children
    j0 = int(off[wide])

    def broken(name, fn):
        a = {k: x.copy() for k, x in base.items()}
        fn(a)
        return a

    cases = [
        ("child id past the last node", "child_nodes",
         broken("c", lambda a: a["child_nodes"].__setitem__(3, n_nodes))),
        ("child id of the root", "child_nodes",
         broken("c0", lambda a: a["child_nodes"].__setitem__(3, 0))),
        ("token outside the codebook", "tokens",
         broken("tv", lambda a: a["tokens"].__setitem__(5, w.V))),
        ("tokens of a node not increasing", "not strictly increasing",
         broken("ti", lambda a: a["tokens"].__setitem__(j0 + 1, a["tokens"][j0]))),
        ("first offset not zero", "node_offsets[0]",
         broken("o0", lambda a: a["node_offsets"].__setitem__(0, 1))),
        ("offsets decreasing", "decreases",
         broken("od", lambda a: a["node_offsets"].__setitem__(wide + 1, a["node_offsets"][wide] - 1))),
        ("last offset not the entry count", "node_offsets[num_nodes]",
         broken("ol", lambda a: a["node_offsets"].__setitem__(n_nodes, n_ent - 1))),
        ("bitmask row out of range", "bitmask_index",
         broken("bm", lambda a: a["bitmask_index"].__setitem__(7, a["bitmask_table"].shape[0]))),
        ("negative bitmask row", "bitmask_index",
         broken("bmn", lambda a: a["bitmask_index"].__setitem__(7, -1))),
        ("Bloom row out of range", "bloom_index",
         broken("bl", lambda a: a["bloom_index"].__setitem__(9, a["bloom_table"].shape[0]))),
    ]
    for what, needle, arrays in cases:
        with pytest.raises(gr.GrError) as e:
            gr.Trie.create(arrays, **kw)
        assert e.value.status == _lib.GR_E_INVALID, what
        assert needle in str(e.value), (what, str(e.value))
    # bad parameters
    for over in (dict(vocab_size=1), dict(sid_length=0), dict(w_bm=0),
                 dict(bloom_bits=100), dict(bloom_k=0)):
        with pytest.raises(gr.GrError) as e:
            gr.Trie.create(base, **{**kw, **over})
        assert e.value.status == _lib.GR_E_INVALID, over
    # the built trie's own arrays are valid
    try:
        gr.Trie.create(base, **kw).close()
    except gr.GrError as e:
        assert e.status in (_lib.GR_E_HIP, _lib.GR_E_NOMEM), str(e)


def test_noalloc_tail_refuses_shapes_beyond_its_scratch_before_any_launch():
    """gr_constrain_topk_noalloc holds 128 MiB of scratch per device: larger
    shapes are refused with GR_E_UNSUPPORTED before the trie or any device
    state is touched; a fitting shape reaches the trie checks."""
    L = _lib.lib()
    t = gr.Trie.build(np.array([[0, 1]], np.int32), 4, 1, 0, 0, [], host_only=True)
    big = gr.tail_args(B=64, M_in=1024, V=1024, k_out=1024, t=0, L=2, n_loc=0, dtype=0)
    assert gr.constrain_topk_workspace(64, 1024, 1024, 1024) > (128 << 20)
    assert L.gr_constrain_topk_noalloc(t.h, ctypes.byref(big), None) == _lib.GR_E_UNSUPPORTED
    assert b"128" in L.gr_last_error() or b"scratch" in L.gr_last_error()
    fits = gr.tail_args(B=32, M_in=1024, V=4, k_out=1024, t=0, L=2, n_loc=0, dtype=0)
    assert L.gr_constrain_topk_noalloc(t.h, ctypes.byref(fits), None) == _lib.GR_E_INVALID
    assert b"host_only" in L.gr_last_error()
    assert L.gr_constrain_topk_noalloc(None, ctypes.byref(fits), None) == _lib.GR_E_INVALID
