"""GPU parity of each hot-path kernel against the CPU oracle, through the C ABI.

Sizes span several tiles with ragged tails; edge cases cover dead rows, ties,
k larger than the survivors, the large-threshold-bin fallback of the top-k and
single-row requests.
"""
import numpy as np
import pytest

import oracle
from synth import workload as W
from tests.helpers import attn_close, to_dev, to_np64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import wide_beam_sid_amd  # noqa: F401
    yield


def _gr():
    import wide_beam_sid_amd as gr
    return gr


def _rand(shape, dtype, rng):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return W.f32_to_bf16_bits(x) if dtype == "bf16" else x


def _as_f(a, dtype):
    return W.bf16_bits_to_f32(a).astype(np.float64) if dtype == "bf16" else a.astype(np.float64)


# ---------------------------------------------------------------------------
# A1: cross-attention
# ---------------------------------------------------------------------------

CROSS_CASES = [
    # B, M, H, T, d, dtype
    (1, 8, 2, 16, 32, "f32"),
    (3, 5, 2, 7, 64, "f32"),
    (2, 37, 2, 70, 64, "bf16"),      # ragged beams and keys
    (3, 129, 4, 64, 32, "bf16"),     # two row tiles + 1
    (1, 300, 2, 2048, 128, "bf16"),  # long context tiles
    (16, 256, 4, 64, 64, "bf16"),
    (2, 1, 8, 256, 64, "bf16"),      # one beam per request
    (1, 20, 16, 1, 128, "bf16"),     # T_ctx = 1: output = V
    (2, 200, 2, 333, 64, "bf16"),    # 128-row workgroups, ragged last key tile
    (1, 150, 2, 200, 32, "bf16"),    # 128-row workgroups at d_h = 32
    (2, 300, 2, 333, 64, "bf16"),    # 256-row workgroups, ragged rows and last key tile
    (1, 512, 2, 256, 32, "bf16"),    # 256-row workgroups at d_h = 32
    (2, 1024, 2, 512, 64, "bf16"),   # the stress shape's per-request rows and context
]


@pytest.mark.parametrize("B,M,H,T,d,dt", CROSS_CASES)
def test_cross_attn_parity(B, M, H, T, d, dt):
    gr = _gr()
    rng = np.random.default_rng(B * 1000 + M + T)
    q = _rand((B * M, H, d), dt, rng)
    K = _rand((B, H, T, d), dt, rng)
    Vv = _rand((B, H, T, d), dt, rng)
    out = torch.empty(to_dev(q, dt).shape, dtype=torch.bfloat16 if dt == "bf16" else torch.float32,
                      device="cuda")
    gr.cross_attn(to_dev(q, dt), to_dev(K, dt), to_dev(Vv, dt), out, B, M)
    torch.cuda.synchronize()
    ref = oracle.cross_attn(_as_f(q, dt), _as_f(K, dt), _as_f(Vv, dt), B, M)
    attn_close(to_np64(out), ref, dt, f"cross {B}x{M}x{H}x{T}x{d}")
    if T == 1:
        got = to_np64(out)
        assert np.array_equal(got, np.repeat(_as_f(Vv, dt)[:, :, 0], M, axis=0))


@pytest.mark.parametrize("B,M,H,T,d", [(2, 300, 2, 512, 64), (1, 100, 2, 384, 64),
                                       (1, 70, 2, 640, 32)])
def test_cross_attn_growing_scores(B, M, H, T, d):
    """Keys whose scale grows along the context, so that every key tile's
    max lies far above the running max of the tiles before it: the path
    that rescales the output and normaliser after the first tile."""
    gr = _gr()
    rng = np.random.default_rng(7 * T + M)
    q = _rand((B * M, H, d), "bf16", rng)
    K = _rand((B, H, T, d), "bf16", rng)
    Vv = _rand((B, H, T, d), "bf16", rng)
    # the tile maxima climb by well over 8 (log2 units) from one 64-key
    # tile to the next
    grow = np.linspace(0.05, 30.0, T).astype(np.float32)[None, None, :, None]
    K = W.f32_to_bf16_bits((_as_f(K, "bf16") * grow).astype(np.float32))
    out = torch.empty((B * M, H, d), dtype=torch.bfloat16, device="cuda")
    gr.cross_attn(to_dev(q, "bf16"), to_dev(K, "bf16"), to_dev(Vv, "bf16"), out, B, M)
    torch.cuda.synchronize()
    ref = oracle.cross_attn(_as_f(q, "bf16"), _as_f(K, "bf16"), _as_f(Vv, "bf16"), B, M)
    attn_close(to_np64(out), ref, "bf16", f"growing {B}x{M}x{H}x{T}x{d}")


@pytest.mark.parametrize("B,M,H,T,d", [(2, 300, 2, 512, 64), (1, 100, 2, 384, 64)])
def test_cross_attn_single_key_spikes(B, M, H, T, d):
    """One key per 64-key tile scaled up, at a random place in the tile,
    with the scale climbing from tile to tile: a row's tile max then sits
    in one of the four lanes that hold the row's scores, and only that
    lane's own max passes the running max by more than 8 (log2 units)."""
    gr = _gr()
    rng = np.random.default_rng(11 * T + M)
    q = _rand((B * M, H, d), "bf16", rng)
    K = _as_f(_rand((B, H, T, d), "bf16", rng), "bf16")
    Vv = _rand((B, H, T, d), "bf16", rng)
    for t0 in range(0, T, 64):
        j = t0 + int(rng.integers(0, min(64, T - t0)))
        K[:, :, j, :] *= 2.0 + 6.0 * t0 / 64
    K = W.f32_to_bf16_bits(K.astype(np.float32))
    out = torch.empty((B * M, H, d), dtype=torch.bfloat16, device="cuda")
    gr.cross_attn(to_dev(q, "bf16"), to_dev(K, "bf16"), to_dev(Vv, "bf16"), out, B, M)
    torch.cuda.synchronize()
    ref = oracle.cross_attn(_as_f(q, "bf16"), _as_f(K, "bf16"), _as_f(Vv, "bf16"), B, M)
    attn_close(to_np64(out), ref, "bf16", f"spiky {B}x{M}x{H}x{T}x{d}")


# Few tiles over a long context: the split path (key ranges over several
# workgroups, merged with a log-sum-exp) against the oracle, and the same
# inputs without a workspace.
SPLIT_CASES = [
    # B, M, H, T, d
    (8, 1, 16, 2048, 128),   # the long-context workload's first step
    (8, 20, 16, 2048, 128),  # its second step
    (32, 1, 8, 1024, 64),    # 32 requests, one beam each
    (2, 3, 2, 700, 64),      # ragged last key tile, uneven splits
    (1, 70, 2, 1000, 32),    # two row tiles, ragged keys, d_h = 32
]


@pytest.mark.parametrize("B,M,H,T,d", SPLIT_CASES)
def test_cross_attn_split_parity(B, M, H, T, d):
    gr = _gr()
    nbytes = gr.cross_attn_workspace(B, M, H, T, d, "bf16")
    assert nbytes > 0, "these shapes take the split path"
    rng = np.random.default_rng(B * 31 + M * 7 + T + d)
    q = _rand((B * M, H, d), "bf16", rng)
    K = _rand((B, H, T, d), "bf16", rng)
    Vv = _rand((B, H, T, d), "bf16", rng)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(0xFF)   # no state needed
    out = torch.empty(to_dev(q, "bf16").shape, dtype=torch.bfloat16, device="cuda")
    plain = torch.empty_like(out)
    print(f"[split] {B}x{M}x{H}x{T}x{d} ws={nbytes}", flush=True)
    gr.cross_attn(to_dev(q, "bf16"), to_dev(K, "bf16"), to_dev(Vv, "bf16"), out, B, M, ws=ws)
    gr.cross_attn(to_dev(q, "bf16"), to_dev(K, "bf16"), to_dev(Vv, "bf16"), plain, B, M)
    torch.cuda.synchronize()
    ref = oracle.cross_attn(_as_f(q, "bf16"), _as_f(K, "bf16"), _as_f(Vv, "bf16"), B, M)
    attn_close(to_np64(out), ref, "bf16", f"split cross {B}x{M}x{H}x{T}x{d}")
    attn_close(to_np64(plain), ref, "bf16", f"plain cross {B}x{M}x{H}x{T}x{d}")


def test_cross_attn_split_workspace_error():
    gr = _gr()
    B, M, H, T, d = 8, 1, 16, 2048, 128
    nbytes = gr.cross_attn_workspace(B, M, H, T, d, "bf16")
    small = torch.empty(nbytes - 256, dtype=torch.uint8, device="cuda")
    x = torch.zeros((B * M, H, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, H, T, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gr.GrError):
        gr.cross_attn(x, kv, kv, torch.empty_like(x), B, M, ws=small)


# ---------------------------------------------------------------------------
# Joint attention: context + the row's beam prefix in one softmax
# ---------------------------------------------------------------------------

JOINT_CASES = [
    # B, M, H, T, d, L, t, dtype
    (1, 8, 2, 16, 32, 3, 0, "f32"),
    (2, 5, 2, 7, 64, 4, 3, "f32"),
    (2, 37, 2, 70, 64, 4, 2, "bf16"),     # ragged beams and keys
    (3, 129, 4, 64, 32, 4, 3, "bf16"),    # two row tiles + 1
    (1, 300, 2, 2048, 128, 3, 2, "bf16"), # long context
    (4, 256, 4, 64, 64, 4, 1, "bf16"),
    (2, 200, 2, 333, 64, 4, 3, "bf16"),   # 128-row workgroups, ragged last tile
    (1, 20, 16, 1, 128, 3, 0, "bf16"),    # T_ctx = 1, no prefix
]


@pytest.mark.parametrize("B,M,H,T,d,L,t,dt", JOINT_CASES)
def test_joint_attn_parity(B, M, H, T, d, L, t, dt):
    gr = _gr()
    rng = np.random.default_rng(B * 7 + M + T + t)
    R = B * M
    q = _rand((R, H, d), dt, rng)
    K = _rand((B, H, T, d), dt, rng)
    Vv = _rand((B, H, T, d), dt, rng)
    kn = _rand((R, H, d), dt, rng)
    vn = _rand((R, H, d), dt, rng)
    old = 2 * R + 3
    pool_blocks = old + R
    kp = _rand((pool_blocks, H, d), dt, rng)
    vp = _rand((pool_blocks, H, d), dt, rng)
    table = rng.integers(0, old, size=(R, L)).astype(np.int32)
    table[rng.random((R, L)) < 0.15] = -1          # missing past (dead rows)
    table[:, t:] = -1
    dkp, dvp, dtab = to_dev(kp, dt), to_dev(vp, dt), to_dev(table)
    out = torch.empty(to_dev(q, dt).shape, dtype=dkp.dtype, device="cuda")
    gr.joint_attn(to_dev(q, dt), to_dev(K, dt), to_dev(Vv, dt), to_dev(kn, dt), to_dev(vn, dt),
                  dkp, dvp, dtab, old, t, B, M, out)
    torch.cuda.synchronize()
    # oracle: the row's history gathered from the (input) pool, then the current token
    hk = np.zeros((R, t + 1, H, d))
    hv = np.zeros((R, t + 1, H, d))
    valid = np.zeros((R, t + 1), np.uint8)
    kpf, vpf = _as_f(kp, dt), _as_f(vp, dt)
    for j in range(t):
        ok = table[:, j] >= 0
        hk[ok, j] = kpf[table[ok, j]]
        hv[ok, j] = vpf[table[ok, j]]
        valid[ok, j] = 1
    hk[:, t], hv[:, t], valid[:, t] = _as_f(kn, dt), _as_f(vn, dt), 1
    ref = oracle.joint_attn(_as_f(q, dt), _as_f(K, dt), _as_f(Vv, dt), hk, hv, valid, B, M)
    attn_close(to_np64(out), ref, dt, f"joint {B}x{M}x{H}x{T}x{d} t={t}")
    # the current token went to its fresh block, the table names it
    got_tab = dtab.cpu().numpy()
    assert np.array_equal(got_tab[:, t], old + np.arange(R))
    assert np.array_equal(got_tab[:, :t], table[:, :t])
    kview = dkp[old:].view(torch.int16 if dt == "bf16" else torch.int32).cpu().numpy()
    kin = kn.view(np.int16) if dt == "bf16" else kn.view(np.int32)
    assert np.array_equal(kview, kin)
    vview = dvp[old:].view(torch.int16 if dt == "bf16" else torch.int32).cpu().numpy()
    vin = vn.view(np.int16) if dt == "bf16" else vn.view(np.int32)
    assert np.array_equal(vview, vin)


# ---------------------------------------------------------------------------
# A2: paged self-attention
# ---------------------------------------------------------------------------

SELF_CASES = [
    # R, H, d, L, t, dtype
    (8, 2, 32, 3, 0, "f32"),
    (8, 2, 32, 3, 2, "f32"),
    (37, 4, 64, 4, 3, "bf16"),
    (1000, 4, 64, 4, 1, "bf16"),
    (301, 16, 128, 3, 2, "bf16"),
    (130, 8, 64, 4, 3, "bf16"),
    # 16 lanes per row (16 rows per workgroup), ragged
    (29, 2, 64, 4, 2, "bf16"),
    # 24 pieces per row on 32 lanes (8 lanes idle), ragged
    (45, 3, 64, 4, 3, "bf16"),
    # heads narrower than 16 bytes: 8-byte pieces
    (19, 4, 4, 3, 2, "bf16"),
    (11, 3, 2, 3, 2, "f32"),
]


@pytest.mark.parametrize("R,H,d,L,t,dt", SELF_CASES)
def test_self_attn_paged_parity(R, H, d, L, t, dt):
    gr = _gr()
    rng = np.random.default_rng(R + 7 * t)
    old = 3 * R + 5                      # blocks already in the pool
    pool_blocks = old + R
    kp = _rand((pool_blocks, H, d), dt, rng)
    vp = _rand((pool_blocks, H, d), dt, rng)
    q, kn, vn = (_rand((R, H, d), dt, rng) for _ in range(3))
    table = rng.integers(0, old, size=(R, L)).astype(np.int32)
    table[rng.random((R, L)) < 0.15] = -1          # missing past (dead rows)
    table[:, t:] = -1
    fresh = old
    dkp, dvp, dtab = to_dev(kp, dt), to_dev(vp, dt), to_dev(table)
    out = torch.empty(to_dev(q, dt).shape, dtype=dkp.dtype, device="cuda")
    gr.self_attn_paged(to_dev(q, dt), to_dev(kn, dt), to_dev(vn, dt), dkp, dvp, dtab, fresh, t, out)
    torch.cuda.synchronize()
    # oracle: dense per-row history gathered from the same (input) pool
    hk = np.zeros((R, t + 1, H, d))
    hv = np.zeros((R, t + 1, H, d))
    ok = np.zeros((R, t + 1), np.uint8)
    kpf, vpf = _as_f(kp, dt), _as_f(vp, dt)
    for j in range(t):
        live = table[:, j] >= 0
        hk[live, j] = kpf[table[live, j]]
        hv[live, j] = vpf[table[live, j]]
        ok[live, j] = 1
    hk[:, t], hv[:, t], ok[:, t] = _as_f(kn, dt), _as_f(vn, dt), 1
    ref = oracle.self_attn(_as_f(q, dt), hk, hv, ok)
    attn_close(to_np64(out), ref, dt, f"self R={R} t={t}")
    # the current token went to block fresh + i and the table column t
    gk = to_np64(dkp)
    assert np.array_equal(gk[fresh:fresh + R], _as_f(kn, dt))
    assert np.array_equal(to_np64(dvp)[fresh:fresh + R], _as_f(vn, dt))
    assert np.array_equal(gk[:old], kpf[:old])
    tab = dtab.cpu().numpy()
    assert np.array_equal(tab[:, t], fresh + np.arange(R))
    assert np.array_equal(np.delete(tab, t, axis=1), np.delete(table, t, axis=1))
    if t == 0:   # one position: the softmax weight is exactly 1
        assert np.array_equal(to_np64(out), _as_f(vn, dt))


# ---------------------------------------------------------------------------
# A3-A6: constrain / log-softmax / top-k / reorder
# ---------------------------------------------------------------------------

_TRIES = {}
_WS = {}


def _workspace(nbytes):
    """One zero-filled workspace reused by every tail call of the session
    (each call leaves it zero-filled), grown when a call needs more."""
    if _WS.get("ws") is None or _WS["ws"].numel() < nbytes:
        _WS["ws"] = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    return _WS["ws"]


def _trie_case(w, seed, slice_min=0, kway=None):
    key = (w, seed, slice_min, None if kway is None else repr(kway))
    if key not in _TRIES:
        gr = _gr()
        sids = W.make_catalog(w, seed)
        ads = W.make_ads(w, seed, W.ad_counts(w, seed))
        trie = gr.Trie.build(sids, w.V, w.w_bm, w.bloom_bits, w.bloom_k, [ads], keep_host=True,
                             bloom_slice_min=slice_min, **(kway or {}))
        view = trie.host_view()
        ix = oracle.build_index(w, sids, ads)
        n = view["num_nodes"]
        prefix = [()] * n
        for node in range(1, n):
            prefix[node] = prefix[view["node_parent"][node]] + (int(view["node_token"][node]),)
        _TRIES[key] = (trie, view, ix, prefix)
    return _TRIES[key]


def run_tail(w, seed, M_in, k_out, t, dead_frac=0.1, logit_mode="normal", acc_mode="normal",
             B=None, slice_min=0, staged=False, kway=None, trie=None, between=None,
             node_in=None, acc_in=None):
    """Run gr_constrain_topk on synthetic beam rows at depth t and check every
    output against the oracle.  ``trie`` replaces the built trie of the
    workload for the GPU call (the same index, made another way)."""
    gr = _gr()
    B = B or w.B
    print(f"[tail] {w.name} seed={seed} B={B} M_in={M_in} k={k_out} t={t}", flush=True)
    built, view, ix, prefix = _trie_case(w, seed, slice_min, kway)
    trie = built if trie is None else trie
    rng = np.random.default_rng(seed * 31 + M_in + t)
    R = B * M_in
    if node_in is None:   # random rows at depth t (a few dead)
        depth_nodes = np.nonzero(view["node_depth"] == t)[0]
        node_in = rng.choice(depth_nodes, size=R).astype(np.int32)
        dead = rng.random(R) < dead_frac
        node_in[dead] = -1
        if acc_mode == "normal":
            acc_in = (-rng.random(R) * 4).astype(np.float32)
        else:
            acc_in = np.full(R, -1.5, np.float32)
        acc_in[dead] = -np.inf
    else:                 # the given beam rows (e.g. a previous step's outputs)
        node_in = np.ascontiguousarray(node_in, np.int32)
        acc_in = np.ascontiguousarray(acc_in, np.float32)
        rng.random(R)
    if logit_mode == "normal":
        logits = _rand((R, w.V), w.dtype, rng)
    else:  # every logit equal: ties everywhere
        logits = _rand((1, 1), w.dtype, rng).repeat(R * w.V).reshape(R, w.V)
    req = W.make_requests(w.scaled(B=B), seed)
    probes = gr.bloom_probes(req.locs.reshape(-1), w.bloom_bits, w.bloom_k) if w.bloom_bits else \
        np.zeros((1, 1), np.uint32)
    L = w.L
    tokens_in = rng.integers(0, w.V, size=(R, L)).astype(np.int32)
    table_in = rng.integers(0, 10**6, size=(R, L)).astype(np.int32)
    dev = {k: to_dev(v) for k, v in dict(node_in=node_in, acc_in=acc_in, tokens_in=tokens_in,
                                         table_in=table_in, user_bm=req.user_bm,
                                         user_probes=probes).items()}
    dev["logits"] = to_dev(logits, w.dtype)
    Rn = B * k_out
    out = dict(parent_out=torch.empty(Rn, dtype=torch.int32, device="cuda"),
               token_out=torch.empty(Rn, dtype=torch.int32, device="cuda"),
               node_out=torch.empty(Rn, dtype=torch.int32, device="cuda"),
               acc_out=torch.empty(Rn, dtype=torch.float32, device="cuda"),
               tokens_out=torch.empty((Rn, L), dtype=torch.int32, device="cuda"),
               table_out=torch.empty((Rn, L), dtype=torch.int32, device="cuda"),
               dbg_mask=torch.empty((R, (w.V + 63) // 64), dtype=torch.int64, device="cuda"),
               dbg_scores=torch.empty((R, w.V), dtype=torch.float32, device="cuda"))
    ws_bytes = gr.constrain_topk_workspace(B, M_in, w.V, k_out)
    ws = _workspace(ws_bytes)
    args = gr.tail_args(B=B, M_in=M_in, V=w.V, k_out=k_out, t=t, L=L, n_loc=w.n_loc,
                        dtype=gr.GR_BF16 if w.dtype == "bf16" else gr.GR_F32,
                        user_bm=dev["user_bm"], user_probes=dev["user_probes"] if w.bloom_bits else None,
                        logits=dev["logits"], node_in=dev["node_in"], acc_in=dev["acc_in"],
                        tokens_in=dev["tokens_in"], table_in=dev["table_in"], ws=ws,
                        ws_bytes=ws_bytes, **out)
    if staged:
        gr.constrain(trie, args)
        if between is not None:   # sees the workspace between the two stages
            torch.cuda.synchronize()
            between(ws)
        gr.topk_reorder(trie, args)
    else:
        gr.constrain_topk(trie, args)
    torch.cuda.synchronize()
    o = {k: v.cpu().numpy() for k, v in out.items()}
    exp_mask = None
    if kway is not None:   # k-way decisions from the partition oracle
        from oracle import kway as okway
        sids = W.make_catalog(w, seed)
        ads = W.make_ads(w, seed, W.ad_counts(w, seed))
        rows = okway.leaf_rows(sids, ads, w.w_bm, w.bloom_bits, w.bloom_k)
        okw = (dict(k_static=kway["kway_k"]) if kway["kway_mode"] == 1
               else dict(k_max=kway["kway_kmax"], target=kway["kway_target_fill"]))
        blooms = [[oracle.bloom_row(int(l), w.bloom_bits, w.bloom_k) for l in req.locs[b]]
                  for b in range(B)] if w.bloom_bits else [[] for _ in range(B)]
        children = {}
        for sid in rows:
            children.setdefault(sid[:t], set()).add(sid[t])
        memo = {}
        exp_mask = np.zeros((R, (w.V + 63) // 64), np.uint64)
        for r in range(R):
            if node_in[r] < 0:
                continue
            b = r // M_in
            pre = tuple(prefix[node_in[r]])
            for v in sorted(children.get(pre, ())):
                key = (b, pre + (v,))
                if key not in memo:
                    parts = okway.node_partitions(rows, pre + (v,), kway["kway_mode"], **okw)
                    memo[key] = okway.passes(parts, req.user_bm[b], blooms[b], w.w_bm)
                if memo[key]:
                    exp_mask[r, v // 64] |= np.uint64(1) << np.uint64(v % 64)
        exp_mask = exp_mask.view(np.uint64)
    check_tail(w, ix, view, prefix, req, node_in, acc_in, W.as_float(w, logits).astype(np.float64),
               M_in, k_out, t, o, tokens_in, table_in, B, exp_mask=exp_mask)
    return o


def check_tail(w, ix, view, prefix, req, node_in, acc_in, logits64, M_in, k_out, t, o,
               tokens_in=None, table_in=None, B=None, exp_mask=None):
    B = B or w.B
    V, L = w.V, w.L
    R = B * M_in
    mask = o["dbg_mask"].view(np.uint64)
    scores = o["dbg_scores"]
    # A3: masks bit-exact
    if exp_mask is None:
        blooms = [ix.user_blooms(req.locs[b]) for b in range(B)]
        exp_mask = np.zeros_like(mask)
        for r in range(R):
            b = r // M_in
            live = node_in[r] >= 0
            exp_mask[r] = ix.mask_row(list(prefix[node_in[r]]) if live else [], t if live else -1,
                                      req.user_bm[b], req.locs[b], blooms[b])
    assert np.array_equal(mask, exp_mask), "mask mismatch"
    # A4: scores within tolerance of acc + fp64 log-softmax
    keep = oracle.mask_bits_to_bool(mask, V)
    assert np.array_equal(np.isfinite(scores), keep)
    lp = np.stack([oracle.log_softmax(x) for x in logits64]) if R else np.zeros((0, V))
    cand = np.where(keep, acc_in.astype(np.float64)[:, None] + lp, -np.inf)
    if keep.any():
        err = np.abs(scores[keep] - cand[keep])
        bound = 2e-5 + 2e-7 * np.abs(cand[keep])
        assert (err <= bound).all(), f"score err {err.max():.3g}"
    # A5: top-k on the GPU's own scores, bit-exact
    for b in range(B):
        f, s = oracle.topk(scores[b * M_in:(b + 1) * M_in].reshape(-1), k_out)
        n = f.size
        sl = slice(b * k_out, b * k_out + n)
        assert np.array_equal(o["parent_out"][sl], b * M_in + (f // V).astype(np.int32)), f"parent b={b}"
        assert np.array_equal(o["token_out"][sl], (f % V).astype(np.int32)), f"token b={b}"
        assert np.array_equal(o["acc_out"][sl].view(np.uint32), s.view(np.uint32))
        dead = slice(b * k_out + n, (b + 1) * k_out)
        assert (o["parent_out"][dead] == -1).all() and (o["node_out"][dead] == -1).all()
        assert (o["token_out"][dead] == -1).all() and np.isneginf(o["acc_out"][dead]).all()
    # A6: child node of (parent, token); token / table rows reordered
    live = o["parent_out"] >= 0
    par = o["parent_out"][live]
    nodes = o["node_out"][live]
    assert np.array_equal(view["node_parent"][nodes], node_in[par])
    assert np.array_equal(view["node_token"][nodes], o["token_out"][live])
    if tokens_in is not None:
        tk = o["tokens_out"]
        assert np.array_equal(tk[live, :t], tokens_in[par, :t])
        assert np.array_equal(tk[live, t], o["token_out"][live])
        assert (tk[live, t + 1:] == -1).all() and (tk[~live] == -1).all()
        tb = o["table_out"]
        assert np.array_equal(tb[live, :t + 1], table_in[par, :t + 1])
        assert (tb[live, t + 1:] == -1).all() and (tb[~live] == -1).all()


# 70 two-valued attributes (3 bitmask words, 70 user bits set), 9 Bloom
# probes per id and 100 user locations: the paths past 64 user bits, past 8
# probes per location and past 64 locations.
_WIDE_ATTR = W.Workload(
    name="wide_attr", dtype="bf16", B=2, L=3, V=64, schedule=(64, 256, 256), T_ctx=40, H=2,
    d_h=32, n_sids=20_000, zipf_s=1.1, ads_per_sid=(1, 8), bm_segments=(2,) * 70, bm_p=0.97,
    bloom_bits=1024, bloom_k=9, geo_pool=2000, geo_per_ad=(1, 16), n_loc=100)

TAIL_WORKLOADS = {
    "wide_attr": _WIDE_ATTR,
    "tiny": W.WORKLOADS["tiny_fp32"],
    "main_50k": W.WORKLOADS["main_b16_m1024"].scaled(n_sids=50_000),
    "long_50k": W.WORKLOADS["longctx_b8"].scaled(n_sids=50_000),
    "stress_20k": W.WORKLOADS["stress_b64"].scaled(n_sids=20_000, geo_per_ad=(1, 64)),
}

TAIL_CASES = [
    # workload, seed, B, M_in, k_out, t, dead, logits, acc
    ("tiny", 0, 1, 1, 8, 0, 0.0, "normal", "normal"),
    ("tiny", 0, 1, 8, 8, 1, 0.2, "normal", "normal"),
    ("tiny", 1, 1, 8, 8, 2, 0.0, "normal", "normal"),
    ("main_50k", 1, 4, 1, 1024, 0, 0.0, "normal", "normal"),    # k > survivors: dead slots
    ("main_50k", 1, 4, 300, 1000, 1, 0.1, "normal", "normal"),
    ("main_50k", 1, 3, 1024, 1024, 2, 0.05, "normal", "normal"),
    ("main_50k", 1, 2, 1024, 1024, 3, 0.0, "normal", "normal"),
    ("main_50k", 1, 2, 700, 1024, 1, 0.0, "equal", "equal"),    # ties: huge threshold bin
    ("main_50k", 1, 2, 64, 37, 1, 0.0, "equal", "normal"),
    ("main_50k", 1, 2, 16, 5, 1, 1.0, "normal", "normal"),      # every row dead
    ("long_50k", 3, 3, 300, 900, 1, 0.1, "normal", "normal"),
    ("stress_20k", 4, 2, 1024, 1024, 1, 0.1, "normal", "normal"),
    ("stress_20k", 4, 2, 1024, 1024, 2, 0.1, "normal", "normal"),
    ("wide_attr", 5, 2, 64, 256, 1, 0.1, "normal", "normal"),
    ("wide_attr", 5, 2, 256, 256, 2, 0.1, "normal", "normal"),
]


@pytest.mark.parametrize("name,seed,B,M_in,k_out,t,dead,lmode,amode", TAIL_CASES)
def test_constrain_topk_parity(name, seed, B, M_in, k_out, t, dead, lmode, amode):
    w = TAIL_WORKLOADS[name]
    run_tail(w, seed, M_in, k_out, t, dead, lmode, amode, B=B)


ROOT_CASES = [
    # workload, seed, B, k_out, t, dead, logits, acc -- one beam row per request
    ("main_50k", 1, 4, 37, 0, 0.0, "normal", "normal"),       # fewer slots than candidates
    ("main_50k", 2, 6, 1024, 1, 0.3, "normal", "normal"),     # rows at depth-1 nodes, some dead
    ("main_50k", 3, 4, 200, 2, 0.0, "normal", "normal"),      # deeper nodes, most without a block
    ("main_50k", 1, 3, 1000, 0, 0.0, "equal", "normal"),      # every candidate in one score bin
    ("stress_20k", 4, 3, 1024, 0, 0.0, "normal", "normal"),   # V = 1024 at the root
    ("stress_20k", 5, 4, 300, 1, 0.25, "normal", "normal"),
    ("long_50k", 3, 2, 900, 0, 0.0, "normal", "normal"),      # bitmask-only matcher
    ("tiny", 1, 2, 8, 1, 0.0, "normal", "normal"),            # fp32, nodes without blocks
    ("wide_attr", 5, 2, 64, 0, 0.0, "normal", "normal"),      # three attribute words: two launches
]


@pytest.mark.parametrize("name,seed,B,k_out,t,dead,lmode,amode", ROOT_CASES)
def test_one_row_per_request_tail(name, seed, B, k_out, t, dead, lmode, amode):
    """One beam row per request, as at the root: the tail runs as one launch
    that places the candidates in order in LDS.  Checked against the oracle
    as the two-launch tail is, with dead rows, nodes with and without a
    bit-sliced block, ties in one score bin and more candidates than slots."""
    run_tail(TAIL_WORKLOADS[name], seed, 1, k_out, t, dead, lmode, amode, B=B)


def test_constrain_topk_workspace_error():
    gr = _gr()
    w = TAIL_WORKLOADS["tiny"]
    trie = _trie_case(w, 0)[0]
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    args = gr.tail_args(B=1, M_in=8, V=w.V, k_out=8, t=1, L=w.L, n_loc=1, dtype=gr.GR_F32,
                        user_bm=small, user_probes=small, logits=small, node_in=small,
                        acc_in=small, parent_out=small, token_out=small, node_out=small,
                        acc_out=small, ws=small, ws_bytes=64)
    with pytest.raises(gr.GrError) as e:
        gr.constrain_topk(trie, args)
    assert e.value.status == -4


@pytest.mark.parametrize("name,seed,M_in,t", [("tiny", 0, 8, 1), ("main_50k", 1, 64, 2),
                                              ("stress_20k", 4, 200, 1), ("long_50k", 3, 300, 2)])
def test_constrain_topk_k_at_survivor_count(name, seed, M_in, t):
    """k equal to the number of finite candidates, and one either side: the
    boundary between 'every survivor is selected' and a threshold bin."""
    w = TAIL_WORKLOADS[name]
    o = run_tail(w, seed, M_in, 1024, t, 0.0, B=1)
    n = int((o["parent_out"] >= 0).sum())
    assert 2 <= n < 1024, n
    for k in (n, n - 1, n + 1):
        run_tail(w, seed, M_in, k, t, 0.0, B=1)


_KWAY_W = W.WORKLOADS["main_b16_m1024"].scaled(n_sids=600, B=2, V=16)


@pytest.mark.parametrize("kw,t", [
    (dict(kway_mode=1, kway_k=(8, 4, 3, 2)), 1),
    (dict(kway_mode=1, kway_k=(8, 4, 3, 2)), 2),
    (dict(kway_mode=2, kway_kmax=8, kway_target_fill=0.1), 1),
    (dict(kway_mode=2, kway_kmax=8, kway_target_fill=0.1), 3),
])
def test_constrain_topk_kway(kw, t):
    """k-way partitioned matchers: the GPU's masks equal the partition
    oracle's decisions; scores, top-k and reorder as for one-union tries."""
    run_tail(_KWAY_W, 11, 40, 30, t, 0.1, B=2, kway=kw)


@pytest.mark.parametrize("slice_min", [-1, 1])
@pytest.mark.parametrize("name,seed,M_in,k_out,t", [("tiny", 1, 8, 8, 1), ("main_50k", 1, 300, 1000, 1),
                                                   ("wide_attr", 5, 64, 256, 1),
                                                   ("main_50k", 1, 700, 1024, 2),
                                                   ("stress_20k", 4, 512, 1024, 1)])
def test_constrain_topk_bloom_layouts(slice_min, name, seed, M_in, k_out, t):
    """The Bloom test through staged rows only (no bit-sliced blocks) and
    through bit-sliced blocks for every node with a child: same oracle."""
    w = TAIL_WORKLOADS[name]
    trie = _trie_case(w, seed, slice_min)[0]
    info = trie.info()
    assert (info["slice_words"] == 0) == (slice_min == -1)
    run_tail(w, seed, M_in, k_out, t, 0.1, B=2, slice_min=slice_min)


@pytest.mark.parametrize("name,seed,M_in,k_out,t", [("main_50k", 1, 300, 1000, 1),
                                                   ("stress_20k", 4, 512, 1024, 2)])
def test_constrain_then_topk_reorder(name, seed, M_in, k_out, t):
    """The two stages called one by one give the outputs of the fused call
    (the oracle checks both), and leave the shared workspace reusable."""
    w = TAIL_WORKLOADS[name]
    a = run_tail(w, seed, M_in, k_out, t, 0.1, B=2, staged=True)
    b = run_tail(w, seed, M_in, k_out, t, 0.1, B=2)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    ws = _WS["ws"]
    lay_hist = 2048 * 1024 * 4
    assert int(ws[:lay_hist].count_nonzero()) == 0   # histograms left zero-filled


@pytest.mark.parametrize("name,seed,M_in,k_out,t", [
    ("tiny", 0, 65536, 1024, 1),      # gx = 2048 expand workgroups, the select's last prefix entry
    ("tiny", 1, 65505, 1000, 2),      # gx = 2048 with a short last row block
    ("tiny", 1, 65504, 1024, 1),      # gx = 2047
    ("main_50k", 1, 65536, 1024, 1),  # many survivors per request at the row limit
])
def test_constrain_topk_at_the_row_limit(name, seed, M_in, k_out, t):
    """One request with the documented maximum of 65536 beam rows (and just
    below it): every survivor segment enters the select's prefix sums."""
    run_tail(TAIL_WORKLOADS[name], seed, M_in, k_out, t, 0.05, B=1)


@pytest.mark.parametrize("name,seed,M_in,k_out,t", [("main_50k", 1, 300, 1000, 1),
                                                   ("stress_20k", 4, 512, 1024, 2),
                                                   ("tiny", 0, 8, 8, 2)])
def test_trie_create_from_arrays_runs_the_same_tail(name, seed, M_in, k_out, t):
    """A trie uploaded with gr_trie_create from a built trie's Appendix A
    arrays answers the tail exactly as the built one: the oracle checks the
    created trie's masks, scores, top-k and reorder."""
    gr = _gr()
    w = TAIL_WORKLOADS[name]
    view = _trie_case(w, seed)[1]
    keys = ("node_offsets", "child_nodes", "tokens", "bitmask_index", "bloom_index",
            "bitmask_table", "bloom_table")
    arrays = {k: view[k] for k in keys if view[k].size or k in ("bitmask_table",)}
    made = gr.Trie.create(arrays, w.V, w.L, w.w_bm, w.bloom_bits, w.bloom_k)
    assert made.info()["num_nodes"] == view["num_nodes"]
    a = run_tail(w, seed, M_in, k_out, t, 0.1, B=2, trie=made)
    b = run_tail(w, seed, M_in, k_out, t, 0.1, B=2)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_node_major_step_after_map_writes_of_other_batch_sizes():
    """The step after the root takes the rows named by the inverse map that
    the previous step's select leaves in the workspace.  Calls of different
    batch sizes share the workspace here (B = 1 then 2 then 4 at the root, each
    followed by the step after the root at another B): whatever the map and
    the other calls left, every output matches the oracle."""
    w = TAIL_WORKLOADS["stress_20k"]   # V = 1024: the node-major pass runs
    seen = []

    def back_counts(ws):
        # the segments' back counts (node-major survivors) follow the
        # 2048-bin histograms of up to 1024 requests in the workspace
        off = 4 * 2048 * 1024
        seen.append(int(ws[off:off + 4 * 1024 * 4].view(torch.int32).count_nonzero()))

    # the workspace sized for the largest call first: a workspace that grows
    # between the root step and the next would start the next with no map
    _workspace(_gr().constrain_topk_workspace(4, 1024, w.V, 1024))
    for B1, B0 in ((2, 1), (3, 2), (4, 1), (4, 3)):
        root = run_tail(w, 4, 1, 1024, 0, 0.0, B=B1)   # root step: writes the map
        run_tail(w, 4, 1, 1024, 0, 0.0, B=B0)          # another B overwrites part of it
        # the step after the root on the first call's outputs: rows of the
        # requests b >= B0 are named by the map, the others are not
        run_tail(w, 4, 1024, 1000, 1, B=B1, staged=True, between=back_counts,
                 node_in=root["node_out"], acc_in=root["acc_out"])
    assert all(n > 0 for n in seen), seen         # the pass took rows every time


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_node_major_pass_logit_dtypes(dtype):
    """The node-major pass keeps its row's logits in LDS as they are in
    memory: bf16 bits (16-byte pieces) or fp32 values, at different LDS
    pitches.  The step after the root with fp32 and with bf16 logits,
    against the oracle; the back counts show the pass took rows."""
    w = TAIL_WORKLOADS["stress_20k"].scaled(dtype=dtype)
    seen = []

    def back_counts(ws):
        off = 4 * 2048 * 1024
        seen.append(int(ws[off:off + 4 * 1024 * 4].view(torch.int32).count_nonzero()))

    _workspace(_gr().constrain_topk_workspace(2, 1024, w.V, 1024))   # kept by both calls
    root = run_tail(w, 5, 1, 1024, 0, 0.0, B=2)
    run_tail(w, 5, 1024, 1000, 1, B=2, staged=True, between=back_counts,
             node_in=root["node_out"], acc_in=root["acc_out"])
    assert seen and seen[0] > 0, seen


@pytest.mark.parametrize("geo", [(1, 64), (200, 256)])
def test_node_major_pass_sparse_and_dense_bloom_rows(geo):
    """The node-major pass stops testing a row's locations once every child
    that passes eq 5 has a location with all its probe bits.  With long geo
    lists (dense Bloom rows) that happens after the first group of
    locations; with shorter ones most rows test every location.  Both
    against the oracle, on the step after the root."""
    w = TAIL_WORKLOADS["stress_20k"].scaled(geo_per_ad=geo)
    seen = []

    def back_counts(ws):
        off = 4 * 2048 * 1024
        seen.append(int(ws[off:off + 4 * 1024 * 4].view(torch.int32).count_nonzero()))

    _workspace(_gr().constrain_topk_workspace(2, 1024, w.V, 1024))   # kept by both calls
    root = run_tail(w, 4, 1, 1024, 0, 0.0, B=2)
    run_tail(w, 4, 1024, 1000, 1, B=2, staged=True, between=back_counts,
             node_in=root["node_out"], acc_in=root["acc_out"])
    assert seen and seen[0] > 0, seen


def _cutoff_preset(cuts, k_out):
    """The 32 cutoff counters of each request (bytes): k_out at the first of
    the 25 cutoffs whose count in cuts reaches k_out, zero elsewhere."""
    cnt = torch.zeros((cuts.shape[0], 32), dtype=torch.int32)
    for b in range(cuts.shape[0]):
        full = np.nonzero(cuts[b] >= k_out)[0]
        if full.size:
            cnt[b, int(full[0])] = k_out
    return cnt.reshape(-1).view(torch.uint8)


def test_node_major_pass_drops_candidates_past_a_full_cutoff():
    """A node-major wavefront drops the candidates past the first cutoff bin
    that already holds k counted survivors of its request (on large launches
    the workgroups that run later see such counts).  Here the counter of the
    first cutoff that an identical run's histogram fills to k is preset to k
    (those survivors exist, so k of them will be counted there; presetting
    every final count would count them twice), so every wavefront drops
    past it, and every output still matches the oracle."""
    w = TAIL_WORKLOADS["stress_20k"]
    gr = _gr()
    ws = _workspace(gr.constrain_topk_workspace(2, 1024, w.V, 1024))
    root = run_tail(w, 4, 1, 1024, 0, 0.0, B=2)
    hists = []

    def grab(wsv):   # after gr_constrain: the requests' histograms
        hists.append(wsv[:2 * 2048 * 4].view(torch.int32).cpu().numpy().reshape(2, 2048).copy())

    # a narrow top-k (5 of a few hundred survivors per request), so that a
    # tight cutoff holds k
    kw = dict(B=2, staged=True, node_in=root["node_out"], acc_in=root["acc_out"])
    first = run_tail(w, 4, 1024, 5, 1, between=grab, **kw)
    # the cutoff bins: 15, 18, 21, 26, 31, ..., 863, 1023 (about 2^(1/4) apart)
    bins = [(16 << (j >> 2)) * (64, 76, 91, 108)[j & 3] // 64 - 1 for j in range(25)]
    cuts = np.stack([hists[0][:, :b + 1].sum(axis=1) for b in bins], axis=1)
    assert ((cuts >= 5) & (cuts < cuts[:, -1:])).any(), cuts   # some are past it somewhere
    # the 32 counters of each request sit after the histograms (8 MiB) and
    # the back counts (4 MiB)
    off = 4 * 2048 * 1024 + 4 * 1024 * 1024
    ws[off:off + 2 * 32 * 4].copy_(_cutoff_preset(cuts, 5).to("cuda"))
    second = run_tail(w, 4, 1024, 5, 1, between=grab, **kw)
    assert hists[1].sum() < hists[0].sum()   # candidates were dropped
    for k in ("parent_out", "token_out", "node_out", "acc_out"):
        assert np.array_equal(first[k], second[k]), k
