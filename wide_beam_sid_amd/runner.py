"""Device buffers for a batch of L decode steps and the gr_decode_step chain.

Plumbing only: torch allocates the beam-state buffers, the paged KV pool and
the workspace; each step is one gr_decode_step call (GRACE Section 3.1 decode
loop with the dynamic per-step widths of Section 3.3: M_0 = 1, M_{t+1} = k_t,
and the block ids of step t starting at sum_{s<t} R_s).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from . import (DecodeGraph, StepArgs, Trie, _ptr, constrain_topk_workspace, cross_attn_workspace,
               decode_step, tail_args)
from ._lib import GR_BF16, GR_F32


class Decoder:
    """Buffers for B requests decoded over L = len(schedule) steps."""

    def __init__(self, trie: Trie, B: int, V: int, schedule: Sequence[int], H: int, d_h: int,
                 T_ctx: int, dtype: str, debug: bool = False, device: str = "cuda"):
        import torch
        self.torch = torch
        self.trie = trie
        self.B, self.V, self.H, self.d_h, self.T_ctx = B, V, H, d_h, T_ctx
        self.schedule = list(schedule)
        self.L = len(schedule)
        self.dtype = dtype
        self.gr_dtype = GR_BF16 if dtype == "bf16" else GR_F32
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        L = self.L
        self.M = [1] + self.schedule[:-1]                  # rows per request entering step t
        self.rows = [B * m for m in self.M]
        self.fresh = [int(x) for x in np.concatenate([[0], np.cumsum(self.rows)[:-1]])]
        self.pool_blocks = int(sum(self.rows))
        dev = device
        self.k_pool = torch.zeros((self.pool_blocks, H, d_h), dtype=tdt, device=dev)
        self.v_pool = torch.zeros_like(self.k_pool)
        n_state = [*self.rows, B * self.schedule[-1]]
        i32 = torch.int32
        self.node = [torch.empty(n, dtype=i32, device=dev) for n in n_state]
        self.acc = [torch.empty(n, dtype=torch.float32, device=dev) for n in n_state]
        self.tokens = [torch.full((n, L), -1, dtype=i32, device=dev) for n in n_state]
        self.table = [torch.full((n, L), -1, dtype=i32, device=dev) for n in n_state]
        self.parent = [torch.empty(B * k, dtype=i32, device=dev) for k in self.schedule]
        self.token = [torch.empty(B * k, dtype=i32, device=dev) for k in self.schedule]
        self.cross_out = [torch.empty((r, H, d_h), dtype=tdt, device=dev) for r in self.rows]
        self.self_out = [torch.empty((r, H, d_h), dtype=tdt, device=dev) for r in self.rows]
        self.ws_bytes = max(constrain_topk_workspace(B, self.M[t], V, self.schedule[t])
                            for t in range(L))
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)  # zero-filled once
        # split cross-attention partials (steps with few tiles over a long
        # context); no state between calls
        self.attn_ws_bytes = max(cross_attn_workspace(B, self.M[t], H, T_ctx, d_h, dtype)
                                 for t in range(L))
        self.attn_ws = (torch.empty(self.attn_ws_bytes, dtype=torch.uint8, device=dev)
                        if self.attn_ws_bytes else None)
        self.debug = debug
        words = (V + 63) // 64
        if debug:
            self.dbg_mask = [torch.empty((r, words), dtype=torch.int64, device=dev) for r in self.rows]
            self.dbg_scores = [torch.empty((r, V), dtype=torch.float32, device=dev) for r in self.rows]
        # initial state: every request at the trie root with score 0
        self.node[0].fill_(0)
        self.acc[0].fill_(0.0)

    def step_args(self, t: int, user_bm, user_probes, n_loc: int, k_ctx, v_ctx,
                  inp: Dict) -> StepArgs:
        a = StepArgs()
        a.H, a.d_h, a.T_ctx = self.H, self.d_h, self.T_ctx
        a.k_ctx, a.v_ctx = _ptr(k_ctx), _ptr(v_ctx)
        a.qx, a.q, a.k_new, a.v_new = (_ptr(inp[k]) for k in ("qx", "q", "k", "v"))
        a.k_pool, a.v_pool = _ptr(self.k_pool), _ptr(self.v_pool)
        a.pool_blocks, a.fresh_base = self.pool_blocks, self.fresh[t]
        a.cross_out, a.self_out = _ptr(self.cross_out[t]), _ptr(self.self_out[t])
        a.tail = tail_args(
            B=self.B, M_in=self.M[t], V=self.V, k_out=self.schedule[t], t=t, L=self.L,
            n_loc=n_loc, dtype=self.gr_dtype, user_bm=user_bm, user_probes=user_probes,
            logits=inp["logits"], node_in=self.node[t], acc_in=self.acc[t],
            tokens_in=self.tokens[t], table_in=self.table[t], parent_out=self.parent[t],
            token_out=self.token[t], node_out=self.node[t + 1], acc_out=self.acc[t + 1],
            tokens_out=self.tokens[t + 1], table_out=self.table[t + 1],
            dbg_mask=self.dbg_mask[t] if self.debug else None,
            dbg_scores=self.dbg_scores[t] if self.debug else None,
            ws=self.ws, ws_bytes=self.ws_bytes)
        if self.attn_ws is not None:
            a.attn_ws, a.attn_ws_bytes = _ptr(self.attn_ws), self.attn_ws_bytes
        return a

    def step(self, t: int, user_bm, user_probes, n_loc: int, k_ctx, v_ctx, inp: Dict,
             stream=None) -> None:
        decode_step(self.trie, self.step_args(t, user_bm, user_probes, n_loc, k_ctx, v_ctx, inp),
                    stream)

    def run(self, user_bm, user_probes, n_loc: int, k_ctx, v_ctx, inputs: List[Dict],
            stream=None) -> None:
        for t in range(self.L):
            self.step(t, user_bm, user_probes, n_loc, k_ctx, v_ctx, inputs[t], stream)

    def graph(self, user_bm, user_probes, n_loc: int, k_ctx, v_ctx, inputs: List[Dict],
              stream) -> DecodeGraph:
        """The L steps of run() captured as one HIP graph on `stream` (a
        created stream); each launch() replays the whole decode on the same
        buffers."""
        steps = [self.step_args(t, user_bm, user_probes, n_loc, k_ctx, v_ctx, inputs[t])
                 for t in range(self.L)]
        return DecodeGraph(self.trie, steps, stream)
