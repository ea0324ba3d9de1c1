"""The decode loop of GRACE Section 3.1 / 3.3, walked step by step on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Per step t (rows R_t = B * M_t, request-major: row r = b * M_t + m):
  A1  cross-attention of every row against its request's context (Section 5.1)
  A2  self-attention over the row's own prefix positions 0..t, kept as a dense
      per-row history that is copied from the parent on reorder -- the dense
      baseline of Section 3.3 that the paged block table replaces
  A3  CD and TM masks of every row (eqs 1-5, 8)
  A4  full-vocabulary log-softmax (fp64), masked tokens set to -inf (eq 3),
      candidate score = accumulated log-prob of the prefix + new log-prob
  A5  per-request top-k_t over flat index f = m * V + v, score descending then
      f ascending; -inf is never selected; missing slots are dead
  A6  reorder: parent row, token, accumulated score, token history and the
      dense KV history follow the selection

Readings where the pages are silent (the same ones the GPU library takes):
  * M_0 = 1; M_{t+1} = k_t; dead slots have parent = token = -1, score -inf,
    history -1 and produce no candidates later.
  * A position whose history is missing (a dead row's past) is excluded from
    self-attention; the current position is always present.
  * Log-softmax is taken over all V logits, then the mask is applied.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import cross_attn, log_softmax, mask_bits_to_bool, self_attn, topk


@dataclass
class OracleState:
    """Beam state entering a step (rows R_t)."""

    tokens: np.ndarray         # int32 [R, L]; -1 where not yet chosen or dead
    live: np.ndarray           # bool [R]
    acc: np.ndarray            # float64 [R]
    hist_k: np.ndarray         # float64 [R, L, H, d]
    hist_v: np.ndarray         # float64 [R, L, H, d]
    hist_ok: np.ndarray        # uint8 [R, L]


def initial_state(w) -> OracleState:
    R = w.B
    return OracleState(
        tokens=np.full((R, w.L), -1, np.int32),
        live=np.ones(R, bool),
        acc=np.zeros(R, np.float64),
        hist_k=np.zeros((R, w.L, w.H, w.d_h)),
        hist_v=np.zeros((R, w.L, w.H, w.d_h)),
        hist_ok=np.zeros((R, w.L), np.uint8),
    )


@dataclass
class OracleStepOut:
    cross_out: Optional[np.ndarray]
    self_out: Optional[np.ndarray]
    mask: np.ndarray           # uint64 [R, ceil(V/64)]
    lp: np.ndarray             # float64 [R, V] full log-softmax
    cand: np.ndarray           # float64 [R, V] (-inf where masked)
    sel_f: list                # per request: uint32 flat indices (sorted)
    sel_s: list                # per request: float32 scores used for the sort
    parent: np.ndarray         # int32 [B*k]
    token: np.ndarray          # int32 [B*k]
    next_state: OracleState = field(repr=False)


def step(w, ix, req, ctx, t: int, st: OracleState, inp: dict, as_float,
         gpu_scores: Optional[np.ndarray] = None, attention: bool = True,
         rows_subset: Optional[np.ndarray] = None,
         mask_rows: Optional[np.ndarray] = None,
         given_mask: Optional[np.ndarray] = None) -> OracleStepOut:
    """One decode step.

    ``gpu_scores`` (float32 [R, V]) are the GPU's own candidate scores; when
    given, top-k sorts them (so that the selection can be compared bit for
    bit), otherwise it sorts float32(oracle fp64 score).
    ``rows_subset`` restricts attention to some rows (others stay NaN).
    ``mask_rows`` restricts the CD/TM masks to some rows (for catalogs too
    large to enumerate every row); the other rows take ``given_mask``.
    """
    B, V, L = w.B, w.V, w.L
    R = st.tokens.shape[0]
    M = R // B
    k_t = w.schedule[t]

    # A1 / A2
    cross_out = self_out = None
    if attention:
        q = as_float(inp["q"]).astype(np.float64)
        st.hist_k[:, t] = as_float(inp["k"]).astype(np.float64)
        st.hist_v[:, t] = as_float(inp["v"]).astype(np.float64)
        st.hist_ok[:, t] = 1
        qx = as_float(inp["qx"]).astype(np.float64)
        K = as_float(ctx[0]).astype(np.float64)
        Vc = as_float(ctx[1]).astype(np.float64)
        if rows_subset is None:
            cross_out = cross_attn(qx, K, Vc, B, M)
            self_out = self_attn(q, st.hist_k[:, : t + 1], st.hist_v[:, : t + 1],
                                 st.hist_ok[:, : t + 1])
        else:
            cross_out = np.full(qx.shape, np.nan)
            self_out = np.full(q.shape, np.nan)
            for r in rows_subset:
                b = r // M
                cross_out[r:r + 1] = cross_attn(qx[r:r + 1], K[b:b + 1], Vc[b:b + 1], 1, 1)
                self_out[r:r + 1] = self_attn(q[r:r + 1], st.hist_k[r:r + 1, : t + 1],
                                              st.hist_v[r:r + 1, : t + 1],
                                              st.hist_ok[r:r + 1, : t + 1])

    # A3 / A4
    words = (V + 63) // 64
    mask = np.zeros((R, words), np.uint64)
    logits = as_float(inp["logits"]).astype(np.float64)
    lp = np.empty((R, V))
    blooms = [ix.user_blooms(req.locs[b]) for b in range(B)]
    if mask_rows is not None:
        mask[:] = given_mask
    for r in (range(R) if mask_rows is None else mask_rows):
        b = r // M
        mask[r] = ix.mask_row(st.tokens[r, :t], t if st.live[r] else -1,
                              req.user_bm[b], req.locs[b], blooms[b])
    for r in range(R):
        lp[r] = log_softmax(logits[r])
    keep = mask_bits_to_bool(mask, V)
    cand = np.where(keep, st.acc[:, None] + lp, -np.inf)

    # A5
    scores = gpu_scores if gpu_scores is not None else cand.astype(np.float32)
    sel_f, sel_s = [], []
    parent = np.full(B * k_t, -1, np.int32)
    token = np.full(B * k_t, -1, np.int32)
    for b in range(B):
        f, s = topk(np.ascontiguousarray(scores[b * M:(b + 1) * M]).reshape(-1), k_t)
        sel_f.append(f)
        sel_s.append(s)
        n = f.size
        parent[b * k_t: b * k_t + n] = b * M + (f // V).astype(np.int32)
        token[b * k_t: b * k_t + n] = (f % V).astype(np.int32)

    # A6
    Rn = B * k_t
    live = parent >= 0
    src = np.where(live, parent, 0)
    tokens = np.full((Rn, L), -1, np.int32)
    tokens[live] = st.tokens[src[live]]
    tokens[live, t] = token[live]
    acc = np.full(Rn, -np.inf)
    acc[live] = cand[src[live], token[live]]
    hk = np.zeros((Rn, L, w.H, w.d_h))
    hv = np.zeros((Rn, L, w.H, w.d_h))
    ok = np.zeros((Rn, L), np.uint8)
    if attention:
        hk[live] = st.hist_k[src[live]]
        hv[live] = st.hist_v[src[live]]
        ok[live] = st.hist_ok[src[live]]
    nxt = OracleState(tokens, live, acc, hk, hv, ok)
    return OracleStepOut(cross_out, self_out, mask, lp, cand, sel_f, sel_s,
                         parent, token, nxt)
