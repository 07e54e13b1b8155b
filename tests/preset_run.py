"""Builds one routed layer of a workload preset on the GPU (device-generated
inputs, planted needles) and gives the oracle the same layer on the host, by
document, so full-size presets can be checked on sampled documents."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle as O
import synth
from synth import device as SD
import sparse_attention_long_msa_amd as M


def dev():
    return torch.device("cuda:0")


_STORE_CACHE: dict = {}


class HostLayer:
    """Host-side (oracle) view of layer l of preset p."""

    def __init__(self, p, l, device_gen=None):
        self.p, self.l = p, l
        self.dt = "bf16" if p.bf16 else "f32"
        H, d = p.H, p.d
        self.qr = synth.tensor(p.qseed, l, synth.T_QR, (p.B, p.T, H, d), bf16=p.bf16)
        self.q = synth.tensor(p.qseed, l, synth.T_Q, (p.B, p.T, p.Hq, d), bf16=p.bf16)
        self.needles = synth.needle_docs(p.seed, p.n_docs, p.n_needles)
        # needle i belongs to query i (one per query) or to query 0
        self.owner = {int(nd): (i if p.needle_per_query else 0) for i, nd in enumerate(self.needles)}
        # generated values come from the device copy of the generator when a
        # GPU is present (bit-identical to the host copy, and far faster for
        # the long documents and local windows of the full-size presets)
        self.device_gen = torch.cuda.is_available() if device_gen is None else device_gen

    def _normal(self, seed, stream, start, count, scale_pow2=0):
        """count generator values of (seed, stream) from start, float64."""
        p = self.p
        if not self.device_gen:
            return synth.normal(seed, stream, start, count, bf16=p.bf16, scale_pow2=scale_pow2)
        buf = torch.empty(count, dtype=torch.bfloat16 if p.bf16 else torch.float32, device=dev())
        SD.fill_stream(buf, seed, stream, start=start, scale_pow2=scale_pow2)
        return buf.float().cpu().numpy().astype(np.float64)

    def raw_rows(self, tensor, doc):
        """Raw rows (tokens, or pooled rows for pooled-level presets) of one document."""
        p = self.p
        off = p.chunk_off if p.pooled_level else p.tok_off
        lo, hi = int(off[doc]), int(off[doc + 1])
        if tensor == synth.T_KR and int(doc) in self.owner:
            b = self.owner[int(doc)]
            return synth.needle_rows(self.qr[b], p.seed, self.l, hi - lo, bf16=p.bf16, start=lo)
        scale = -3 if (p.pooled_level and tensor in (synth.T_K, synth.T_V)) else 0
        x = self._normal(p.seed, synth.stream_id(self.l, tensor), lo * p.H * p.d, (hi - lo) * p.H * p.d, scale)
        return x.reshape(hi - lo, p.H, p.d)

    def store(self, tensor, doc):
        """Oracle store entries of one document (pooled; routing keys normalised)."""
        p = self.p
        x = self.raw_rows(tensor, doc)
        chunk = 1 if p.pooled_level else p.chunk
        return O.pool_encode(x, np.array([0, len(x)]), chunk, tensor == synth.T_KR, self.dt)

    def doc_scores(self, docs):
        """Oracle routing scores [B, len(docs)] of the given documents."""
        out = np.empty((self.p.B, len(docs)))
        for j, doc in enumerate(docs):
            kr = self.store(synth.T_KR, doc)
            out[:, j] = O.route_scores(self.qr, kr, np.array([0, len(kr)]))[:, 0]
        return out

    def routing_store(self, gen_rows=None, blk_rows=1 << 19):
        """The oracle's pooled, normalised routing-key store [N, H, d] of the
        whole layer (every document), float32 (its values are store-dtype
        values, exact in float32).

        Built a block of documents at a time from the raw rows of the seeded
        generator: ``gen_rows(r0, r1)`` gives raw rows r0 .. r1-1 as float64;
        by default the device copy of the generator (bit-identical to the host
        copy) fills them, so that a 10M-token layer takes seconds.  Needle
        documents' rows are the host-side needle rows, as on the GPU.  The
        needle-free store of a (memory, layer) is cached: the 10M-token and
        batched-decode presets share their memory, and so do the two 100M
        tiers."""
        p = self.p
        key = (p.seed, self.l, p.chunk, p.bf16, p.pooled_level, p.n_chunks, p.n_docs)
        base = _STORE_CACHE.get(key)
        if base is None:
            _STORE_CACHE.clear()
            base = self._pooled_blocks(gen_rows or self._device_rows(blk_rows), blk_rows)
            _STORE_CACHE[key] = base
        store = base.copy() if self.owner else base
        for nd in self.owner:
            lo, hi = int(p.chunk_off[nd]), int(p.chunk_off[nd + 1])
            store[lo:hi] = self.store(synth.T_KR, nd)
        return store

    def _device_rows(self, blk_rows):
        p = self.p
        buf = torch.empty((blk_rows, p.H, p.d), dtype=torch.bfloat16 if p.bf16 else torch.float32, device=dev())

        def gen(r0, r1):
            out = np.empty((r1 - r0, p.H, p.d), dtype=np.float64)
            for a in range(r0, r1, blk_rows):
                b = min(r1, a + blk_rows)
                SD.fill(buf[: b - a], p.seed, self.l, synth.T_KR, start=a * p.H * p.d)
                out[a - r0:b - r0] = buf[: b - a].float().cpu().numpy()
            return out
        return gen

    def _pooled_blocks(self, gen_rows, blk_rows):
        """Pool + normalise + round every document, without needles."""
        p = self.p
        dt = self.dt
        off = p.chunk_off if p.pooled_level else p.tok_off      # raw-row offsets per document
        store = np.empty((p.n_chunks, p.H, p.d), dtype=np.float32)
        d0 = 0
        while d0 < p.n_docs:
            d1 = int(np.searchsorted(off, off[d0] + blk_rows, side="right") - 1)
            d1 = min(p.n_docs, max(d0 + 1, d1))
            r0, r1 = int(off[d0]), int(off[d1])
            raw = gen_rows(r0, r1)
            c0, c1 = int(p.chunk_off[d0]), int(p.chunk_off[d1])
            if p.pooled_level:
                # chunk = 1: the pool is the identity (pinned), so the store is the
                # normalised, rounded rows; the oracle's pool_encode is checked on
                # the block's first rows
                blk = O.round_to_store(O.l2_normalize(raw), dt)
                n = min(64, len(raw))
                assert np.array_equal(blk[:n], O.pool_encode(raw[:n], np.arange(n + 1), 1, True, dt))
            else:
                blk = O.pool_encode(raw, off[d0:d1 + 1] - r0, p.chunk, True, dt)
            assert blk.shape[0] == c1 - c0
            store[c0:c1] = blk
            d0 = d1
        return store

    def all_doc_scores(self, store=None, blk_docs=1 << 15):
        """Oracle routing scores [B, D] of every document of the layer."""
        p = self.p
        store = self.routing_store() if store is None else store
        out = np.empty((p.B, p.n_docs))
        for d0 in range(0, p.n_docs, blk_docs):
            d1 = min(p.n_docs, d0 + blk_docs)
            c0, c1 = int(p.chunk_off[d0]), int(p.chunk_off[d1])
            out[:, d0:d1] = O.route_scores(self.qr, store[c0:c1], p.chunk_off[d0:d1 + 1] - c0)
        return out

    def local(self, b):
        p = self.p
        n = p.L_loc * p.H * p.d
        kl = self._normal(p.qseed, synth.stream_id(self.l, synth.T_KLOC), b * n, n)
        vl = self._normal(p.qseed, synth.stream_id(self.l, synth.T_VLOC), b * n, n)
        return kl.reshape(p.L_loc, p.H, p.d), vl.reshape(p.L_loc, p.H, p.d)

    def attention(self, b, ids_b):
        """Oracle attention of query b over the documents ids_b (rank order)."""
        p = self.p
        ks, vs, ps = [], [], []
        for doc in ids_b:
            kb, vb = self.store(synth.T_K, doc), self.store(synth.T_V, doc)
            ks.append(kb)
            vs.append(vb)
            ps.append(np.arange(len(kb)))
        kl, vl = self.local(b)
        return O.attend_one(self.q[b], np.concatenate(ks), np.concatenate(vs), np.concatenate(ps), kl, vl,
                            p.qpo, p.rope_base, 1.0 / math.sqrt(p.d))


class GpuLayer:
    """Layer l of preset p built and run on the GPU through the C ABI."""

    def __init__(self, p, l, host: HostLayer, src_mode=M.MSA_SRC_DEVICE, indexed=False, overlap_local=False):
        self.p, self.l = p, l
        d0 = dev()
        bf = torch.bfloat16 if p.bf16 else torch.float32
        H, d = p.H, p.d
        co = p.chunk_off
        self.co_d = torch.from_numpy(co).to(d0)
        self.cd = M.msa_chunk_doc_map(self.co_d, p.n_chunks)
        if p.pooled_level:
            to_d, chunk, n_rows = self.co_d, 1, p.n_chunks
            row_off = co
        else:
            to_d, chunk, n_rows = torch.from_numpy(p.tok_off).to(d0), p.chunk, int(p.lengths.sum())
            row_off = p.tok_off
        raw = torch.empty((n_rows, H, d), dtype=bf, device=d0)
        self.store = {}
        for tid in (synth.T_KR, synth.T_K, synth.T_V):
            scale = -3 if (p.pooled_level and tid != synth.T_KR) else 0
            SD.fill(raw, p.seed, l, tid, scale_pow2=scale)
            if tid == synth.T_KR:
                for nd, b in host.owner.items():
                    lo, hi = int(row_off[nd]), int(row_off[nd + 1])
                    rows = synth.needle_rows(host.qr[b], p.seed, l, hi - lo, bf16=p.bf16, start=lo)
                    raw[lo:hi] = torch.from_numpy(rows).to(d0, bf)
            lay = M.MSA_LAYOUT_TILED if (tid == synth.T_KR and p.bf16) else M.MSA_LAYOUT_ROWS
            self.store[tid] = M.msa_pool_encode(raw, to_d, self.co_d, self.cd, chunk, tid == synth.T_KR,
                                                layout=lay)
        del raw
        self.qr = torch.from_numpy(host.qr).to(d0, bf)
        self.q = torch.from_numpy(host.q).to(d0, bf)
        self.kl = SD.fill(torch.empty((p.B, p.L_loc, H, d), dtype=bf, device=d0), p.qseed, l, synth.T_KLOC)
        self.vl = SD.fill(torch.empty((p.B, p.L_loc, H, d), dtype=bf, device=d0), p.qseed, l, synth.T_VLOC)
        kb, vb = self.store[synth.T_K], self.store[synth.T_V]
        if src_mode != M.MSA_SRC_DEVICE:
            kb, vb = kb.cpu().pin_memory(), vb.cpu().pin_memory()
        self.kb, self.vb = kb, vb
        self.runner = M.LayerRunner(batch=p.B, tokens=p.T, q_heads=p.Hq, kv_heads=H, head_dim=d, n_docs=p.n_docs,
                                    n_chunks=p.n_chunks, k=p.k, max_doc_chunks=p.max_doc_chunks,
                                    local_len=p.L_loc, dtype=bf, device=d0, q_pos_offset=p.qpo,
                                    rope_base=p.rope_base, src_mode=src_mode, chunk_off_h=co,
                                    kr_layout=M.MSA_LAYOUT_TILED if p.bf16 else M.MSA_LAYOUT_ROWS,
                                    indexed=indexed, overlap_local=overlap_local)

    def run(self):
        r = self.runner
        r.run(self.qr, self.store[synth.T_KR], self.cd, self.co_d, self.kb, self.vb, self.q, self.kl, self.vl)
        torch.cuda.synchronize()
        return dict(doc_score=r.doc_score.cpu().double().numpy(), ids=r.ids.cpu().numpy(),
                    vals=r.vals.cpu().double().numpy(), out=r.out.cpu().double().numpy(),
                    ctx_len=r.ctx_len.cpu().numpy())
