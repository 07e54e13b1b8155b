"""Per-layer driver of the routing + sparse-attention path.

One routed layer runs route score -> top-k -> context assembly -> sparse
attention on one stream (README, Inference Pipeline: Online Routing & Context
Assembly, then Sparse Generation; routing happens in every upper-half layer,
each with its own routing-key store).  ``LayerRunner`` owns the per-layer
outputs and workspaces so a loop over layers allocates nothing.

With ``indexed=True`` (a device-resident K/V store) the context is not copied:
assembly writes each context entry's store row and attention reads the rows in
place; the result is bit-identical to the gathered path.
"""
from __future__ import annotations

import math

import torch

from . import _binding as B


class LayerRunner:
    def __init__(self, *, batch, tokens, q_heads, kv_heads, head_dim, n_docs, n_chunks, k, max_doc_chunks,
                 local_len, dtype, device, q_pos_offset=None, rope_base=1e6, sm_scale=None,
                 src_mode=B.MSA_SRC_DEVICE, chunk_off_h=None, kr_layout=B.MSA_LAYOUT_ROWS, indexed=False,
                 rounds=1):
        if indexed and src_mode != B.MSA_SRC_DEVICE:
            raise ValueError("indexed assembly reads the K/V store in place: it must be in device memory")
        if rounds > 1 and not indexed:
            raise ValueError("Memory Interleave rounds grow an indexed context (K/V store in device memory)")
        self.rounds = rounds
        self.B, self.T, self.Hq, self.Hkv, self.d = batch, tokens, q_heads, kv_heads, head_dim
        self.n_docs, self.n_chunks, self.k = n_docs, n_chunks, k
        self.max_doc_chunks = max_doc_chunks
        self.max_ctx = rounds * k * max_doc_chunks
        self.L_loc = local_len
        # "offset by k": the number of documents in the context (rounds x k)
        self.q_pos_offset = rounds * k if q_pos_offset is None else q_pos_offset
        self.rope_base = rope_base
        self.sm_scale = 1.0 / math.sqrt(head_dim) if sm_scale is None else sm_scale
        self.src_mode = src_mode
        self.kr_layout = kr_layout
        self.chunk_off_h = chunk_off_h
        self.dtype = dtype
        dt = B.MSA_BF16 if dtype == torch.bfloat16 else B.MSA_F32
        dev = torch.device(device)
        f32, i32 = torch.float32, torch.int32
        self.doc_score = torch.empty((batch, n_docs), dtype=f32, device=dev)
        self.ids = torch.empty((batch, k), dtype=i32, device=dev)
        self.vals = torch.empty((batch, k), dtype=f32, device=dev)
        self.indexed = indexed
        if indexed:
            self.ctx_row = torch.empty((batch, self.max_ctx), dtype=i32, device=dev)
            self.k_ctx = self.v_ctx = None
        else:
            self.k_ctx = torch.empty((batch, self.max_ctx, kv_heads, head_dim), dtype=dtype, device=dev)
            self.v_ctx = torch.empty_like(self.k_ctx)
        self._store = None
        self.ctx_pos = torch.empty((batch, self.max_ctx), dtype=i32, device=dev)
        self.ctx_len = torch.empty((batch,), dtype=i32, device=dev)
        self._lens = [self.ctx_len, torch.empty_like(self.ctx_len)]   # round r writes _lens[r % 2]
        self.ids_rounds = torch.empty((rounds, batch, k), dtype=i32, device=dev) if rounds > 1 else None
        self.out = torch.empty((batch, tokens, q_heads, head_dim), dtype=f32, device=dev)

        def ws(n):
            return torch.empty(max(n, 1), dtype=torch.uint8, device=dev)

        self.rs_ws = ws(B.msa_route_score_workspace(dt, batch, tokens, kv_heads, head_dim, n_docs, n_chunks))
        self.tk_ws = ws(B.msa_topk_workspace(batch, n_docs, k))
        self.at_ws = ws(B.msa_sparse_attn_workspace(dt, batch, tokens, q_heads, kv_heads, head_dim, self.max_ctx,
                                                    local_len, self.q_pos_offset))
        # the RoPE (cos, sin) rows are the same for every layer: built once
        self.rope_table = B.msa_rope_table(B.msa_rope_table_rows(self.max_ctx, local_len, self.q_pos_offset),
                                           head_dim, rope_base, device=dev)
        self.ids_h = None
        self.copy_stream = None
        if src_mode == B.MSA_SRC_HOST_MEMCPY:
            self.ids_h = torch.empty((batch, k), dtype=i32, pin_memory=True)
            self.copy_stream = torch.cuda.Stream(device=dev)

    def route(self, q_r, kr_hat, chunk_doc, stream=None):
        B.msa_route_score(q_r, kr_hat, chunk_doc, self.n_docs, doc_score=self.doc_score, ws=self.rs_ws,
                          layout=self.kr_layout, stream=stream)
        return self.doc_score

    def select(self, stream=None):
        B.msa_topk(self.doc_score, self.k, ids=self.ids, vals=self.vals, ws=self.tk_ws, stream=stream)
        return self.ids, self.vals

    def select_assemble(self, chunk_off, k_bar, v_bar, stream=None):
        """select() then assemble(); on the HBM (indexed) path one fused call."""
        if not self.indexed:
            self.select(stream)
            self.assemble(chunk_off, k_bar, v_bar, stream)
            return
        B.msa_topk_context_index(self.doc_score, self.k, chunk_off, k_bar.shape[0], self.max_doc_chunks, self.max_ctx,
                                 ids=self.ids, vals=self.vals, ctx_row=self.ctx_row, ctx_pos=self.ctx_pos,
                                 ctx_len=self.ctx_len, ws=self.tk_ws, stream=stream)
        self._store = (k_bar, v_bar)

    def assemble(self, chunk_off, k_bar, v_bar, stream=None):
        if self.indexed:
            B.msa_context_index(self.ids, chunk_off, k_bar.shape[0], self.max_doc_chunks, self.max_ctx,
                                ctx_row=self.ctx_row, ctx_pos=self.ctx_pos, ctx_len=self.ctx_len, stream=stream)
            self._store = (k_bar, v_bar)
            return
        B.msa_gather_kv(self.ids, chunk_off, k_bar, v_bar, self.max_doc_chunks, self.max_ctx, self.src_mode,
                        chunk_off_h=self.chunk_off_h, k_ctx=self.k_ctx, v_ctx=self.v_ctx, ctx_pos=self.ctx_pos,
                        ctx_len=self.ctx_len, ids_h=self.ids_h, stream=stream, copy_stream=self.copy_stream)

    def attend(self, q, k_loc, v_loc, stream=None):
        if self.indexed:
            k_bar, v_bar = self._store
            B.msa_sparse_attn_indexed(q, k_bar, v_bar, self.ctx_row, self.ctx_pos, self.ctx_len, k_loc, v_loc,
                                      self.q_pos_offset, self.rope_base, self.sm_scale, out=self.out, ws=self.at_ws,
                                      rope_table=self.rope_table, stream=stream)
            return self.out
        B.msa_sparse_attn(q, self.k_ctx, self.v_ctx, self.ctx_pos, self.ctx_len, k_loc, v_loc, self.q_pos_offset,
                          self.rope_base, self.sm_scale, out=self.out, ws=self.at_ws, rope_table=self.rope_table,
                          stream=stream)
        return self.out

    def fetch_rounds(self, q_r_rounds, kr_hat, chunk_doc, chunk_off, k_bar, v_bar, stream=None, route_events=None):
        """The rounds of Memory Interleave: per round, route with that round's
        routing query, skip the documents fetched in earlier rounds, select k
        and append them to the context.  Round r's ids are ids_rounds[r].
        route_events: optional (start, end) events recorded around round 0's
        routing-score call."""
        R = len(q_r_rounds)
        if R > self.rounds:
            raise ValueError(f"built for {self.rounds} rounds")
        for r, q_r in enumerate(q_r_rounds):
            if r == 0 and route_events is not None:
                route_events[0].record(stream)
            self.route(q_r, kr_hat, chunk_doc, stream)
            if r == 0 and route_events is not None:
                route_events[1].record(stream)
            B.msa_exclude_docs(self.doc_score, self.ids_rounds[:r], stream)
            if r == 0:
                B.msa_topk_context_index(self.doc_score, self.k, chunk_off, k_bar.shape[0], self.max_doc_chunks,
                                         self.max_ctx, ids=self.ids_rounds[0], vals=self.vals, ctx_row=self.ctx_row,
                                         ctx_pos=self.ctx_pos, ctx_len=self._lens[0], ws=self.tk_ws, stream=stream)
            else:
                B.msa_topk(self.doc_score, self.k, ids=self.ids_rounds[r], vals=self.vals, ws=self.tk_ws,
                           stream=stream)
                B.msa_context_append(self.ids_rounds[r], chunk_off, k_bar.shape[0], self.max_doc_chunks, self.ctx_row,
                                     self.ctx_pos, self._lens[(r - 1) % 2], self._lens[r % 2], stream=stream)
        self.ctx_len = self._lens[(R - 1) % 2]
        self._store = (k_bar, v_bar)

    def interleave(self, q_r_rounds, kr_hat, chunk_doc, chunk_off, k_bar, v_bar, q, k_loc, v_loc, stream=None):
        """Memory Interleave: fetch_rounds, then attention over every fetched
        document and the local tokens (query offset rounds x k)."""
        self.fetch_rounds(q_r_rounds, kr_hat, chunk_doc, chunk_off, k_bar, v_bar, stream)
        return self.attend(q, k_loc, v_loc, stream)

    def run(self, q_r, kr_hat, chunk_doc, chunk_off, k_bar, v_bar, q, k_loc, v_loc, stream=None):
        self.route(q_r, kr_hat, chunk_doc, stream)
        self.select_assemble(chunk_off, k_bar, v_bar, stream)
        return self.attend(q, k_loc, v_loc, stream)
