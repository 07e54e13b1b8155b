"""Per-layer driver of the routing + sparse-attention path.

One routed layer runs route score -> top-k -> context assembly -> sparse
attention on one stream (README, Inference Pipeline: Online Routing & Context
Assembly, then Sparse Generation; routing happens in every upper-half layer,
each with its own routing-key store).  ``LayerRunner`` owns the per-layer
outputs and workspaces so a loop over layers allocates nothing.

With ``indexed=True`` the context is not copied: assembly writes each context
entry's store row and attention reads the rows in place, from device memory or
(src_mode MSA_SRC_HOST_MAPPED) from pinned host memory over the host link,
where the reads overlap the local-window keys' work in the same kernel; the
result is bit-identical to the gathered path.

With ``overlap_local=True`` the attention runs as its two parts
(msa_sparse_attn_part): the local-window part on a side stream once the top-k
is known, beside the context's fetch, which it does not need; the context
part, with the merge, after both.  At the 100M-token preset's host tier this
measured slower than one call after the fetch (the two streams' kernels slow
each other, and the fork and join cost more than the overlap saves), so it is
off by default; started earlier, beside the top-k, it was slower still.

With ``fill_in_topk=True`` the routing score's -inf fill (a launch of its own
per layer) moves into the top-k: its first pass writes -inf over the scores
once it has read them (MSA_TOPK_RESET_SCORES), and the next route() skips the
fill (MSA_ROUTE_PREFILLED).  ``doc_score`` then holds -inf after select(), not
the scores.  The runner tracks whether the buffer was left so; a route() that
follows anything else fills as usual.  A captured step (StepGraph) must start
where the last call on the runner was a select (as after any run()), and every
replay leaves it so.
"""
from __future__ import annotations

import math

import torch

from . import _binding as B


class LayerRunner:
    def __init__(self, *, batch, tokens, q_heads, kv_heads, head_dim, n_docs, n_chunks, k, max_doc_chunks,
                 local_len, dtype, device, q_pos_offset=None, rope_base=1e6, sm_scale=None,
                 src_mode=B.MSA_SRC_DEVICE, chunk_off_h=None, kr_layout=B.MSA_LAYOUT_ROWS, indexed=False,
                 rounds=1, overlap_local=False, fill_in_topk=False):
        if indexed and src_mode == B.MSA_SRC_HOST_MEMCPY:
            raise ValueError("indexed assembly reads the K/V store in place (device or mapped pinned host memory)")
        if rounds > 1 and not indexed:
            raise ValueError("Memory Interleave rounds grow an indexed context (K/V store in device memory)")
        if rounds > 1 and overlap_local:
            raise ValueError("Memory Interleave runs the attention in one call (overlap_local is for one round)")
        self.rounds = rounds
        self.fill_in_topk = fill_in_topk
        self._prefilled = False   # doc_score holds -inf, left so by the last select()
        self._selected = False    # ids hold a selection (route_fetch copies it)
        self.B, self.T, self.Hq, self.Hkv, self.d = batch, tokens, q_heads, kv_heads, head_dim
        self.n_docs, self.n_chunks, self.k = n_docs, n_chunks, k
        self.max_doc_chunks = max_doc_chunks
        self.max_ctx = rounds * k * max_doc_chunks
        self.L_loc = local_len
        # the query offset is the number of documents in the context (rounds x k)
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
        # route_fetch's workspace: the routing one and the fetch's counter
        self.rf_ws = None if indexed else ws(B.lib.msa_route_score_fetch_workspace(dt, batch, tokens, kv_heads,
                                                                                   head_dim, n_docs, n_chunks))
        self.tk_ws = ws(B.msa_topk_workspace(batch, n_docs, k))
        self.overlap_local = overlap_local
        at_ws = B.msa_sparse_attn_part_workspace if overlap_local else B.msa_sparse_attn_workspace
        self.at_ws = ws(at_ws(dt, batch, tokens, q_heads, kv_heads, head_dim, self.max_ctx, local_len,
                              self.q_pos_offset))
        # default priority, like every other stream here
        self.local_stream = torch.cuda.Stream(device=dev) if overlap_local else None
        self._local_queued = False
        # the RoPE (cos, sin) rows are the same for every layer: built once
        self.rope_table = B.msa_rope_table(B.msa_rope_table_rows(self.max_ctx, local_len, self.q_pos_offset),
                                           head_dim, rope_base, device=dev)
        self.ids_h = None
        self.copy_stream = None
        if src_mode == B.MSA_SRC_HOST_MEMCPY:
            self.ids_h = torch.empty((batch, k), dtype=i32, pin_memory=True)
            self.copy_stream = torch.cuda.Stream(device=dev)

    def balance(self, q_r, kr_hat, chunk_doc, rounds=4):
        """Setup-time: size the routing scan's chunk ranges per XCD for this
        device from timed launches on this layer's arguments
        (msa_route_balance; it synchronises, so never inside a captured step).
        Scores are unchanged; returns the 8 XCD shares."""
        self._prefilled = False   # the calibration writes scores into doc_score
        return B.msa_route_balance(q_r, kr_hat, chunk_doc, self.n_docs, rounds=rounds, doc_score=self.doc_score,
                                   ws=self.rs_ws, layout=self.kr_layout)

    def route(self, q_r, kr_hat, chunk_doc, stream=None):
        prefilled, self._prefilled = self._prefilled, False
        B.msa_route_score(q_r, kr_hat, chunk_doc, self.n_docs, doc_score=self.doc_score, ws=self.rs_ws,
                          layout=self.kr_layout, stream=stream, prefilled=prefilled)
        return self.doc_score

    def route_fetch(self, q_r, kr_hat, chunk_doc, chunk_off, k_bar, v_bar, stream=None):
        """route() of this layer and, in its scan's tail, assemble() of the
        last select(): that layer's documents copied from its content store
        k_bar / v_bar (device or pinned host memory) into the context, hidden
        behind this layer's routing (msa_route_score_fetch)."""
        if self.indexed or self.src_mode == B.MSA_SRC_HOST_MEMCPY:
            raise RuntimeError("route_fetch copies the context: a gathered runner over device or mapped memory")
        if not self._selected:
            raise RuntimeError("route_fetch copies the last select()'s documents: select() first")
        prefilled, self._prefilled = self._prefilled, False
        B.msa_route_score_fetch(q_r, kr_hat, chunk_doc, self.n_docs, self.ids, chunk_off, k_bar, v_bar,
                                self.max_doc_chunks, self.k_ctx, self.v_ctx, self.ctx_pos, self.ctx_len,
                                doc_score=self.doc_score, ws=self.rf_ws, layout=self.kr_layout, stream=stream,
                                prefilled=prefilled)
        return self.doc_score

    def run_layers(self, layers, stream=None, after_layer=None):
        """A sequence of independent routed layers with each one's context
        fetch hidden behind the next one's routing scan: route and select
        layer 0; then for each layer l, route_fetch(l + 1) (plain assemble()
        for the last layer), attend(l), select(l + 1).  The order is open only
        when a layer's routing query does not depend on the previous layer's
        output: independent queries served together, not the layers of one
        query.  layers: per-layer tuples (q_r, kr_hat, chunk_doc, chunk_off,
        k_bar, v_bar, q, k_loc, v_loc); after_layer(l): called once layer l's
        output is queued in self.out.  The results are those of run() layer
        by layer."""
        if self.overlap_local:
            raise RuntimeError("run_layers runs the attention in one call (overlap_local is for run())")
        L = len(layers)
        if L == 0:
            return self.out
        q_r, kr_hat, chunk_doc = layers[0][:3]
        self.route(q_r, kr_hat, chunk_doc, stream)
        self.select(stream)
        for l in range(L):
            _, _, _, chunk_off, k_bar, v_bar, q, k_loc, v_loc = layers[l]
            if l + 1 < L:
                nq_r, nkr, ncd = layers[l + 1][:3]
                self.route_fetch(nq_r, nkr, ncd, chunk_off, k_bar, v_bar, stream)
            else:
                self.assemble(chunk_off, k_bar, v_bar, stream)
            self.attend(q, k_loc, v_loc, stream)
            if after_layer is not None:
                after_layer(l)
            if l + 1 < L:
                self.select(stream)
        return self.out

    def select(self, stream=None):
        B.msa_topk(self.doc_score, self.k, ids=self.ids, vals=self.vals, ws=self.tk_ws, stream=stream,
                   reset=self.fill_in_topk)
        self._prefilled = self.fill_in_topk
        self._selected = True
        return self.ids, self.vals

    def select_assemble(self, chunk_off, k_bar, v_bar, stream=None):
        """select() then assemble(); on the HBM (indexed) path one fused call."""
        if not self.indexed:
            self.select(stream)
            self.assemble(chunk_off, k_bar, v_bar, stream)
            return
        B.msa_topk_context_index(self.doc_score, self.k, chunk_off, k_bar.shape[0], self.max_doc_chunks, self.max_ctx,
                                 ids=self.ids, vals=self.vals, ctx_row=self.ctx_row, ctx_pos=self.ctx_pos,
                                 ctx_len=self.ctx_len, ws=self.tk_ws, stream=stream, reset=self.fill_in_topk)
        self._prefilled = self.fill_in_topk
        self._selected = True
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

    def start_local(self, q, k_loc, v_loc, stream=None):
        """overlap_local: the local-window part of the attention, on the side
        stream, after the work already queued on `stream`.  q, k_loc and v_loc
        must stay alive until attend() has been queued."""
        if not self.overlap_local:
            raise RuntimeError("start_local needs LayerRunner(overlap_local=True)")
        cur = torch.cuda.current_stream() if stream is None else stream
        self.local_stream.wait_stream(cur)
        B.msa_sparse_attn_part(B.MSA_ATTN_PART_LOCAL, q, k_loc, v_loc, self.q_pos_offset, self.max_ctx,
                               rope_base=self.rope_base, sm_scale=self.sm_scale, ws=self.at_ws,
                               rope_table=self.rope_table, stream=self.local_stream)
        self._local_queued = True

    def attend(self, q, k_loc, v_loc, stream=None):
        """The layer's attention into out; with overlap_local, its context part
        and the merge, after start_local() has queued the local part."""
        if self.overlap_local:
            # the context part, after start_local's part: the two merge into out
            if not self._local_queued:
                raise RuntimeError("overlap_local: start_local() must queue the local part before attend()")
            self._local_queued = False
            cur = torch.cuda.current_stream() if stream is None else stream
            cur.wait_stream(self.local_stream)
            if self.indexed:
                k_bar, v_bar = self._store
                kw = dict(k_ctx=k_bar, v_ctx=v_bar, ctx_row=self.ctx_row)
            else:
                kw = dict(k_ctx=self.k_ctx, v_ctx=self.v_ctx)
            B.msa_sparse_attn_part(B.MSA_ATTN_PART_CONTEXT, q, k_loc, v_loc, self.q_pos_offset, self.max_ctx,
                                   ctx_pos=self.ctx_pos, ctx_len=self.ctx_len, rope_base=self.rope_base,
                                   sm_scale=self.sm_scale, out=self.out, ws=self.at_ws, rope_table=self.rope_table,
                                   stream=stream, **kw)
            return self.out
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
        self._prefilled = False   # the rounds keep their scores (no reset)

    def interleave(self, q_r_rounds, kr_hat, chunk_doc, chunk_off, k_bar, v_bar, q, k_loc, v_loc, stream=None):
        """Memory Interleave: fetch_rounds, then attention over every fetched
        document and the local tokens (query offset rounds x k)."""
        self.fetch_rounds(q_r_rounds, kr_hat, chunk_doc, chunk_off, k_bar, v_bar, stream)
        return self.attend(q, k_loc, v_loc, stream)

    def run(self, q_r, kr_hat, chunk_doc, chunk_off, k_bar, v_bar, q, k_loc, v_loc, stream=None):
        self.route(q_r, kr_hat, chunk_doc, stream)
        if not self.overlap_local:
            self.select_assemble(chunk_off, k_bar, v_bar, stream)
        elif self.indexed:
            # the context index comes out of the top-k call itself: nothing to overlap
            self.select_assemble(chunk_off, k_bar, v_bar, stream)
            self.start_local(q, k_loc, v_loc, stream)
        else:
            self.select(stream)
            self.start_local(q, k_loc, v_loc, stream)
            self.assemble(chunk_off, k_bar, v_bar, stream)
        return self.attend(q, k_loc, v_loc, stream)


class StepGraph:
    """A sequence of library calls (typically every routed layer of one step)
    captured once into a HIP graph and replayed.  Replay submits the whole
    sequence at once, so the host no longer issues (and validates) each call:
    for the smaller memories, where a layer's kernels take tens of
    microseconds, host-side launch cost would otherwise set the step time.

    ``fn`` must only enqueue work on the current stream with fixed buffers
    (LayerRunner with preallocated outputs and workspaces does); calls that
    synchronise with the host (msa_gather_kv in MSA_SRC_HOST_MEMCPY mode)
    cannot be captured.  The library's kernels clear their own buffers with
    fill kernels, never with memset nodes."""

    def __init__(self, fn, warmup=1):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            fn()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()
