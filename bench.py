"""Benchmark of the MSA routing + sparse-attention hot path on one MI355X.

One step = one query through all routed layers: per layer, routing score over
that layer's whole pooled routing-key store -> top-k -> context assembly ->
sparse attention.  The default workload is the 100M-token memory (195,312
documents x 512 tokens, chunk 64 -> 1,562,496 pooled chunks per layer, 18
layers, 8 heads x 128, bf16; the routing-key store is 57.6 GB in HBM), query
of 64 tokens, 32 query heads, 4,096 local tokens, k = 16.  Inputs are seeded
synthetic data generated on the device before the timed region.

Timing: the K timed steps are measured by the wall clock between two device
synchronisations, once with the library calls launched one by one (inside
them only one pair of HIP events per step brackets a routing-score launch:
the roofline's launch duration) and once replaying the step captured as a
HIP graph; the line reports the faster of the two and both times.  The per-stage
breakdown comes from up to 3 further steps with events between all stages
(each event record idles the device for a few microseconds, so these steps
are not part of the timed region).

The default run prints one JSON line: the 100M-token step with every input
resident in HBM (the routing keys, and the content K/V read in place by the
attention) is the line's value; then, in the same line,
  ceiling      the streaming-read rate over the same bytes (msa_stream_read),
  memory_parallel  the calls one GPU of a 2-, 4- or 8-GPU Memory Parallel
               step makes (routing and top-k over its shard of the store) and
               the global reduce of the shards' lists (msa_topk_merge),
  host_tier    the pages' own tier for this workload, the content K/V in
               pinned host memory (the host pins as many layers' K/V as it
               can, 8 of 18 with ~270 GB of RAM, which the layers cycle
               over): the step with the attention reading the selected rows
               over the host link (in_place), with the rows first copied by
               the gather kernel (mapped) or by hipMemcpyAsync per document
               (memcpy), and with each copy in the next layer's routing scan
               (fetch_in_next_route: independent queries only),
  cpu_baseline the float64 oracle's routing on a bounded sample,
  per_config   warm and cold lines of the four smaller presets with the
               oracle's routing and attention times.
--gpus above 1 is not supported (one GPU per process, no collectives).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="cfg4")
    ap.add_argument("--hbm-assembly", choices=["index", "copy"], default="index",
                    help="attention reads the selected rows in place (index) or from a gathered copy")
    ap.add_argument("--no-host-tier", action="store_true",
                    help="skip the host-tier leg (content K/V in pinned host memory, fetched per layer)")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-config lines of the smaller presets (after the 100M-token line)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--no-balance", action="store_true",
                    help="keep the routing scan's chunk ranges equal over the XCDs (by default msa_route_balance "
                         "sizes them per XCD from timed launches before the timed region)")
    ap.add_argument("--overlap", action="store_true",
                    help="on the host tier, run each layer's attention as its two calls, the local-window part on "
                         "a side stream beside the fetch (measured slower than one call after the fetch)")
    ap.add_argument("--no-fill-in-topk", action="store_true",
                    help="fill the score buffer with -inf in a launch of its own before every routing call (by "
                         "default each layer's top-k leaves it at -inf for the next layer's routing call)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no HIP graph replay; for counter collection)")
    ap.add_argument("--layers", type=int, default=None, help="override the routed-layer count (profiling only)")
    ap.add_argument("--rounds", type=int, default=1,
                    help="Memory Interleave rounds per layer (> 1: route, skip the fetched documents, select and "
                         "append, rounds times, then attend; content K/V in HBM)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-memory-parallel", action="store_true",
                    help="skip the Memory Parallel leg (per-shard routing and top-k at 2, 4 and 8 shards, merge)")
    ap.add_argument("--cpu-sample-chunks", type=int, default=None,
                    help="routing-key chunks of the oracle's sample (default: 1048576 at pooled level, "
                         "262144 for token-level memories, whose sample the oracle also pools)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (the reference for the HBM byte counters)")
    ap.add_argument("--encode", action="store_true",
                    help="time Stage 1 from hidden states instead (msa_encode over a 1M-token memory, one layer per "
                         "call, hidden 2560)")
    ap.add_argument("--corpus", action="store_true",
                    help="with --encode: Stage 1 over the whole 100M-token memory (195,312 documents x 512 tokens) "
                         "for every routed layer, a block of 2,048 documents per call, into the full stores")
    ap.add_argument("--train", action="store_true",
                    help="time the training-time path instead (routing loss and attention backward per routed "
                         "layer; --config defaults to train64k)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: --gpus must be 1 "
                                   "(no sharding and no collectives)"}))
        sys.exit(2)
    import torch

    if args.copy_calibration:
        return copy_calibration(torch)
    if args.train:
        return train_main(args, torch)
    if args.encode and args.corpus:
        return encode_corpus_main(args, torch)
    if args.encode:
        return encode_main(args, torch)

    from synth import configs

    p = configs.PRESETS[args.config]()
    pb = PresetBench(torch, p, args.layers, rounds=args.rounds, graph=not args.no_graph,
                     overlap=args.overlap, fill_in_topk=not args.no_fill_in_topk)
    pb.build_stores()
    pb.build_content("hbm")
    assembly = args.hbm_assembly if args.rounds == 1 else "index"
    pb.make_runner("hbm", indexed=assembly == "index")
    shares = pb.balance(not args.no_balance)
    recall = pb.needle_recall()
    hbm = pb.headline(args.steps, args.warmup)
    hbm["config"]["gather"] = f"hbm-{assembly}"
    res = hbm
    # The line's value is the step with every input resident in HBM.  The
    # pages' own tier for the 100M-token workload keeps the content K/V in
    # pinned host memory; that step (the attention reads the selected rows
    # over the host link) is timed too and reported as host_tier.in_place.
    pinned = pb.pin_host() if p.name == "cfg4" and args.rounds == 1 and not args.no_host_tier else None
    host = None
    if pinned is not None:
        kv, desc = pinned
        pb.make_runner("host", indexed=True, src_mode=pb.M.MSA_SRC_HOST_MAPPED)
        host = pb.headline(args.steps, args.warmup, kv=kv,
                           tier=f"host-mapped ({desc['pinned_layers']} of {pb.layers} layers' K/V pinned, cycled)")
        pb.make_runner("hbm", indexed=assembly == "index")
    res["needle_recall_layer0"] = recall
    res["config"]["xcd_shares"] = shares
    if not args.no_ceiling:
        res["ceiling"] = pb.ceiling()
    if p.name == "cfg4" and args.rounds == 1 and not args.no_memory_parallel:
        res["memory_parallel"] = pb.memory_parallel()
    if pinned is not None:
        res["host_tier"] = pb.host_tier(args.steps, args.warmup, pinned,
                                        modes=("mapped", "memcpy", "fetch_in_next_route"))
        res["host_tier"]["in_place"] = {k: host[k] for k in ("value", "ms_per_step", "route_attn_us_per_query",
                                                             "ms_per_step_eager_launches", "ms_per_step_graph_replay",
                                                             "stage_ms_per_step", "attention_GBps")}
        res["host_tier"]["in_place"]["config"] = host["config"]
        res["host_tier"]["in_place"]["note"] = ("the pages' tier: the attention reads the selected rows over the host "
                                                "link (host-link-inclusive, so not the line's value)")
        pb.unpin_host()
    pb.release()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(p, pb.layers, args.cpu_sample_chunks)
    if p.name == "cfg4" and args.rounds == 1 and not args.no_per_config:
        res["per_config"] = {name: config_leg(torch, name, args) for name in ("cfg1", "cfg2", "cfg3", "cfg5")}
    print(json.dumps(res), flush=True)


class PresetBench:
    """One workload preset on the device: its stores (built by the offline
    stage before any timing), a LayerRunner and the whole-path step."""

    def __init__(self, torch, p, layers=None, rounds=1, graph=True, overlap=False, fill_in_topk=True,
                 fetch_in_route=False):
        import synth
        from synth import device as SD
        import sparse_attention_long_msa_amd as M
        self.torch, self.p, self.synth, self.SD, self.M = torch, p, synth, SD, M
        self.layers = p.layers if layers is None else layers
        self.rounds = rounds
        self.graph = graph
        self.overlap = overlap
        self.fill_in_topk = fill_in_topk and rounds == 1
        self.fetch_in_route = fetch_in_route and rounds == 1
        self.pipelined = False   # the current runner's step fetches layer l in layer l + 1's routing scan
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.bf = torch.bfloat16 if p.bf16 else torch.float32
        self.esz = 2 if p.bf16 else 4
        H, d, L = p.H, p.d, self.layers
        self.co_d = torch.from_numpy(p.chunk_off).to(self.dev)
        self.cd = M.msa_chunk_doc_map(self.co_d, p.n_chunks)
        fill = lambda shape, tid, l, seed=p.qseed: SD.fill(torch.empty(shape, dtype=self.bf, device=self.dev),  # noqa
                                                              seed, l, tid)
        self.qr = [fill((p.B, p.T, H, d), synth.T_QR, l) for l in range(L)]
        self.qq = [fill((p.B, p.T, p.Hq, d), synth.T_Q, l) for l in range(L)]
        self.kl = [fill((p.B, p.L_loc, H, d), synth.T_KLOC, l) for l in range(L)]
        self.vl = [fill((p.B, p.L_loc, H, d), synth.T_VLOC, l) for l in range(L)]
        # routing queries of the later Memory Interleave rounds: seeded like round 0's, seed + round
        self.qr_rounds = [[self.qr[l]] + [fill((p.B, p.T, H, d), synth.T_QR, l, p.qseed + r)
                                          for r in range(1, rounds)] for l in range(L)]
        self.kr_layout = M.MSA_LAYOUT_TILED if p.bf16 else M.MSA_LAYOUT_ROWS
        if p.pooled_level:
            self.rows_off, self.pool_chunk, self.n_rows, self.to_d = p.chunk_off, 1, p.n_chunks, self.co_d
        else:
            self.rows_off, self.pool_chunk, self.n_rows = p.tok_off, p.chunk, int(p.tok_off[-1])
            self.to_d = torch.from_numpy(p.tok_off).to(self.dev)
        self.needles = synth.needle_docs(p.seed, p.n_docs, p.n_needles)
        self.kbar, self.vbar, self.store = [], [], None
        self.encode_ms = []

    def _raw(self):
        if getattr(self, "raw", None) is None:
            self.raw = self.torch.empty((self.n_rows, self.p.H, self.p.d), dtype=self.bf, device=self.dev)
        return self.raw

    def build_stores(self):
        """The offline stage: every layer's routing-key store (pooled, normalised,
        in the MFMA-tiled layout), from seeded raw rows with planted needles."""
        torch, p, M, synth = self.torch, self.p, self.M, self.synth
        t0 = time.time()
        log(f"{p.name}: {p.n_docs} docs, {p.n_chunks} chunks/layer, {self.layers} layers, routing-key store "
            f"{p.n_chunks * p.H * p.d * self.esz * self.layers / 1e9:.1f} GB")
        self.store = torch.empty((self.layers, M.padded_chunks(p.n_chunks, self.kr_layout), p.H, p.d), dtype=self.bf,
                                 device=self.dev)
        raw = self._raw()
        for l in range(self.layers):
            self.SD.fill(raw, p.seed, l, synth.T_KR)
            for i, nd in enumerate(self.needles):
                b = i if p.needle_per_query else 0
                qh = self.qr[l][b].float().cpu().numpy()
                lo, hi = int(self.rows_off[nd]), int(self.rows_off[nd + 1])
                rows = synth.needle_rows(qh, p.seed, l, hi - lo, bf16=p.bf16, start=lo)
                raw[lo:hi] = torch.from_numpy(rows).to(self.dev, self.bf)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            M.msa_pool_encode(raw, self.to_d, self.co_d, self.cd, self.pool_chunk, True, out=self.store[l],
                              layout=self.kr_layout)
            e1.record()
            torch.cuda.synchronize()
            self.encode_ms.append(e0.elapsed_time(e1))
        log(f"routing-key store ready in {time.time() - t0:.1f} s")

    def content(self, l, tid, out):
        """pooled K or V of layer l into out (device)"""
        raw = self._raw()
        self.SD.fill(raw, self.p.seed, l, tid, scale_pow2=-3 if self.p.pooled_level else 0)
        return self.M.msa_pool_encode(raw, self.to_d, self.co_d, self.cd, self.pool_chunk, False, out=out)

    def build_content(self, tier):
        torch, p = self.torch, self.p
        t0 = time.time()
        self.kbar, self.vbar = [], []
        for l in range(self.layers):
            for lst, tid in ((self.kbar, self.synth.T_K), (self.vbar, self.synth.T_V)):
                lst.append(self.content(l, tid, torch.empty((p.n_chunks, p.H, p.d), dtype=self.bf, device=self.dev)))
        torch.cuda.synchronize()
        self.raw = None
        log(f"content K/V ({tier}) ready in {time.time() - t0:.1f} s")

    def balance(self, on=True):
        """msa_route_balance on layer 0's store and query before any timing (the
        shares hold for the device); off: equal ranges.  Returns the shares used."""
        r = self.runner
        shares = r.balance(self.qr[0], self.store[0], self.cd, rounds=4 if on else 0)
        self.torch.cuda.synchronize()
        log(f"routing scan split per XCD: {' '.join(f'{v:.4f}' for v in shares)}")
        return [round(float(v), 4) for v in shares]

    def make_runner(self, tier, indexed, src_mode=None, overlap=None):
        p, M = self.p, self.M
        self.tier = tier
        if overlap is None:
            # only a fetched context leaves something to overlap
            overlap = self.overlap and self.rounds == 1 and not indexed
        self.runner = M.LayerRunner(batch=p.B, tokens=p.T, q_heads=p.Hq, kv_heads=p.H, head_dim=p.d,
                                    n_docs=p.n_docs, n_chunks=p.n_chunks, k=p.k, max_doc_chunks=p.max_doc_chunks,
                                    local_len=p.L_loc, dtype=self.bf, device=self.dev,
                                    q_pos_offset=p.qpo if self.rounds == 1 else None, rope_base=p.rope_base,
                                    src_mode=M.MSA_SRC_DEVICE if src_mode is None else src_mode,
                                    chunk_off_h=p.chunk_off, kr_layout=self.kr_layout, indexed=indexed,
                                    rounds=self.rounds, overlap_local=overlap, fill_in_topk=self.fill_in_topk)
        # a fetched context from mapped host memory: each layer's fetch runs in the next layer's routing scan
        self.pipelined = (self.fetch_in_route and not indexed and not overlap
                          and src_mode == M.MSA_SRC_HOST_MAPPED)
        return self.runner

    def step(self, mark=None, route_ev=None, route_layer=-1, kv=None, flush=None):
        """One pass of the whole path over all routed layers.  mark(stage):
        called after each call of the step, stage 0 routing, 1 top-k (and the
        context index), 2 context assembly, 3 attention, and mark(None) where
        a stretch that belongs to no stage ends (stage timing); route_ev:
        events around the routing-score call of layer route_layer only (the
        timed steps); kv(l): the layer's content stores (default: its own, in
        HBM); flush(): run before each layer (cold-cache timing)."""
        runner, stream = self.runner, self.torch.cuda.current_stream()

        def done(stage):
            if mark is not None:
                mark(stage)

        def route(l, fn):
            if l == route_layer:
                route_ev[0].record(stream)
            fn()
            if l == route_layer:
                route_ev[1].record(stream)
            done(0)

        def kv_of(l):
            return (self.kbar[l], self.vbar[l]) if kv is None else kv(l)
        if self.pipelined:
            # layer l's context is fetched in layer l + 1's routing scan (LayerRunner.run_layers' order)
            for l in range(-1, self.layers):
                if flush is not None:
                    flush()
                    done(None)
                if l + 1 < self.layers:
                    nl = l + 1
                    if l < 0:
                        route(nl, lambda: runner.route(self.qr[nl], self.store[nl], self.cd))
                    else:
                        kb, vb = kv_of(l)
                        route(nl, lambda: runner.route_fetch(self.qr[nl], self.store[nl], self.cd, self.co_d, kb, vb))
                else:
                    kb, vb = kv_of(l)
                    runner.assemble(self.co_d, kb, vb)
                    done(2)
                if l >= 0:
                    runner.attend(self.qq[l], self.kl[l], self.vl[l])
                    done(3)
                if l + 1 < self.layers:
                    runner.select()
                    done(1)
            return
        for l in range(self.layers):
            kb, vb = kv_of(l)
            if flush is not None:
                flush()
                done(None)
            if self.rounds > 1:
                runner.fetch_rounds(self.qr_rounds[l], self.store[l], self.cd, self.co_d, kb, vb,
                                    route_events=route_ev if l == route_layer else None)
                done(0)
                runner.attend(self.qq[l], self.kl[l], self.vl[l])
                done(3)
                continue
            route(l, lambda: runner.route(self.qr[l], self.store[l], self.cd))
            if runner.indexed:
                # top-k and the context index in one call (the final selection pass writes the index)
                runner.select_assemble(self.co_d, kb, vb)
                done(1)
                if runner.overlap_local:
                    runner.start_local(self.qq[l], self.kl[l], self.vl[l])
            else:
                runner.select()
                done(1)
                if runner.overlap_local:
                    # the local-window half of the attention, beside the fetch
                    runner.start_local(self.qq[l], self.kl[l], self.vl[l])
                runner.assemble(self.co_d, kb, vb)
                done(2)
            runner.attend(self.qq[l], self.kl[l], self.vl[l])
            done(3)

    def needle_recall(self):
        """Planted-needle recall of layer 0 on one pass (a property of the data, not timed)."""
        p = self.p
        self.step()
        self.torch.cuda.synchronize()
        ids_all = (self.runner.ids if self.rounds == 1 else self.runner.ids_rounds[0]).cpu().numpy()
        return float(np.mean([int(nd) in set(ids_all[i if p.needle_per_query else 0].tolist())
                              for i, nd in enumerate(self.needles)]))

    def timed(self, steps, warmup, kv=None, route_events=True, graph=False):
        """Wall-clock ms per step over `steps` timed steps after `warmup`, and
        the event-timed routing-score launches (one per step).  With graph,
        the step is captured once into a HIP graph (StepGraph) and the timed
        steps are replays; the launch durations then come from as many eager
        steps after the timed region."""
        torch = self.torch
        if graph:
            g = self.M.StepGraph(lambda: self.step(kv=kv), warmup=1)
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            t_start = time.perf_counter()
            for _ in range(steps):
                g.replay()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t_start
            del g
            route_ms = self.route_launches(steps, kv) if route_events else []
            return wall * 1e3 / steps, route_ms
        for _ in range(warmup):
            self.step(kv=kv)
        torch.cuda.synchronize()
        route_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for s in range(steps):
            if route_events:
                self.step(route_ev=route_evs[s], route_layer=s % self.layers, kv=kv)
            else:
                self.step(kv=kv)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        route_ms = [e[0].elapsed_time(e[1]) for e in route_evs] if route_events else []
        return wall * 1e3 / steps, route_ms

    def route_launches(self, n, kv=None):
        """Event-timed routing-score calls: n eager steps, one layer's call each."""
        torch = self.torch
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for s in range(n):
            self.step(route_ev=evs[s], route_layer=s % self.layers, kv=kv)
        torch.cuda.synchronize()
        return [e[0].elapsed_time(e[1]) for e in evs]

    def stages(self, n_steps, kv=None, flush=None):
        """Per-stage ms per step: (route, top-k, assembly, attention), from
        extra steps with one event after every call (each stage is the time
        from the previous event)."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        spans, last = [], [None]

        def mark(stage):
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            if stage is not None and last[0] is not None:
                spans.append((stage, last[0], e))
            last[0] = e
        for s in range(n_steps):
            last[0] = None
            mark(None)
            self.step(mark, kv=kv, flush=flush)
        torch.cuda.synchronize()
        stage = np.zeros(4)
        for st, a, b in spans:
            stage[st] += a.elapsed_time(b)
        return stage / n_steps

    def attn_bytes(self):
        p = self.p
        ctx_len = self.runner.ctx_len.cpu().numpy().astype(np.int64)
        return int((ctx_len + p.L_loc).sum()) * p.H * p.d * 2 * self.esz + p.B * p.T * p.Hq * p.d * (self.esz + 4)

    def headline(self, steps, warmup, kv=None, tier="hbm"):
        """The JSON line: whole-step throughput of the routing-key scan, the
        stage breakdown and the roofline of the routing-score launch.  kv(l):
        the layer's content stores when they are not the HBM ones (tier names
        where they are)."""
        p, layers = self.p, self.layers
        ms_eager, route_ms = self.timed(steps, warmup, kv=kv)
        ms_graph = self.timed(steps, warmup, kv=kv, route_events=False, graph=True)[0] if self.graph else float("inf")
        launch = "hip-graph replay" if ms_graph < ms_eager else "eager launches"
        ms_per_step = min(ms_eager, ms_graph)
        stage = self.stages(min(steps, 3), kv=kv)
        H, d, N, D = p.H, p.d, p.n_chunks, p.n_docs
        store_bytes = N * H * d * self.esz                     # per layer
        step_bytes = store_bytes * layers * self.rounds        # every round scans the layer's store
        value = step_bytes / (ms_per_step * 1e-3) / 1e9
        routing_gbps = step_bytes / ((stage[0] + stage[1]) * 1e-3) / 1e9
        # algorithmic bytes of one msa_route_score call: the store, the chunk->doc map,
        # the routing query and the score row (the result, and the -inf fill when the
        # call launches it itself)
        fills = 1 if self.runner.fill_in_topk else 2
        alg_bytes = store_bytes + N * 4 + p.B * p.T * H * d * self.esz + fills * p.B * D * 4
        route_avg_ms = float(np.mean(route_ms))
        achieved = alg_bytes / (route_avg_ms * 1e-3) / 1e9
        attn_bytes = self.attn_bytes()
        attn_gbps = attn_bytes * layers / (stage[3] * 1e-3) / 1e9
        encode_gbps = (self.n_rows * H * d * self.esz + store_bytes) / (float(np.median(self.encode_ms)) * 1e-3) / 1e9
        workload = (f"{p.name}: {int(p.lengths.sum())}-token memory, {D} docs, chunk {p.chunk}, {N} chunks/layer, "
                    f"{layers} routed layers, H={H}, d={d}; {p.B} quer{'y' if p.B == 1 else 'ies'} x T={p.T}, "
                    f"Hq={p.Hq}, L_loc={p.L_loc}, k={p.k}")
        if self.rounds == 1:
            if self.runner.indexed:
                stages = {"route_score": round(stage[0], 4), "topk_and_context_index": round(stage[1], 4),
                          "attention": round(stage[3], 4)}
            elif self.pipelined:
                # the fetch of layers 0 .. L-2 runs inside the next layer's routing call
                stages = {"route_score_and_previous_fetch": round(stage[0], 4), "topk": round(stage[1], 4),
                          "fetch_last_layer": round(stage[2], 4), "attention": round(stage[3], 4)}
            else:
                stages = {"route_score": round(stage[0], 4), "topk": round(stage[1], 4),
                          ("fetch" if kv is not None else "gather"): round(stage[2], 4),
                          "attention": round(stage[3], 4)}
        else:
            stages = {"rounds_route_topk_append": round(stage[0] + stage[1] + stage[2], 4),
                      "attention": round(stage[3], 4)}
        self.route_avg_ms = route_avg_ms
        return {
            "metric": "routing-key (K_r) scan GB/s over the whole route+attn step",
            "value": round(value, 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": steps,
            "warmup": warmup,
            "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16" if p.bf16 else "f32",
            "data": "synthetic (seeded counter-based generator; planted needles)",
            "config": {"workload": workload, "global_batch": p.B, "seq_len": p.T, "parallelism": "single GPU",
                       "kv_tier": tier, "rounds": self.rounds, "step_launch": launch,
                       "score_fill": ("in the previous layer's top-k (MSA_TOPK_RESET_SCORES)"
                                      if self.runner.fill_in_topk else "a launch before each routing call"),
                       "attention_calls": ("two: the local-window part on a side stream beside the fetch, the "
                                           "context part and the merge after it")
                       if self.runner.overlap_local else "one, after the context is assembled"},
            "route_attn_us_per_query": round(ms_per_step * 1e3 / p.B, 1),
            "ms_per_step_eager_launches": round(ms_eager, 4),
            "ms_per_step_graph_replay": round(ms_graph, 4) if self.graph else None,
            "routing_GBps": round(routing_gbps, 1),
            "routing_frac_of_8TBps": round(routing_gbps / 8000, 4),
            "stage_ms_per_step": stages,
            "attention_GBps": round(attn_gbps, 1),
            "attention_frac_of_8TBps": round(attn_gbps / 8000, 4),
            "attention_bytes_per_layer": attn_bytes,
            "encode_GBps": round(encode_gbps, 1),
            "roofline": {"kernel": "msa_route_score (route_score_mfma_kernel" +
                                   (")" if self.runner.fill_in_topk else " + score fill)"), "bound": "hbm",
                         "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                         "frac": round(achieved / 8000.0, 4), "traffic": counted_traffic(p.name),
                         "avg_launch_ms": round(route_avg_ms, 4), "alg_bytes_per_launch": int(alg_bytes)},
        }

    def ceiling(self):
        """The achievable streaming-read rate over the same bytes as one
        routing launch: msa_stream_read over each layer's routing-key store
        (each read cold: the previous layer's read evicted it), event-timed."""
        torch, p = self.torch, self.p
        sink = torch.zeros(1, dtype=torch.int32, device=self.dev)
        nbytes = p.n_chunks * p.H * p.d * self.esz
        ms = []
        for rep in range(2):
            for l in range(self.layers):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                flat = self.store[l].view(-1)[: nbytes // self.esz]
                e0.record()
                self.M.msa_stream_read(flat, sink)
                e1.record()
                torch.cuda.synchronize()
                if rep:
                    ms.append(e0.elapsed_time(e1))
        t = float(np.mean(ms))
        gbps = nbytes / (t * 1e-3) / 1e9
        route_gbps = nbytes / (self.route_avg_ms * 1e-3) / 1e9
        return {"kernel": "msa_stream_read (1 KB-contiguous 16-byte non-temporal loads, no arithmetic)",
                "bytes_per_read": nbytes, "avg_read_ms": round(t, 4), "ceiling_GBps": round(gbps, 1),
                "ceiling_frac_of_8TBps": round(gbps / 8000, 4),
                "route_store_GBps_over_ceiling": round(route_gbps / gbps, 4)}

    def memory_parallel(self, shard_counts=(2, 4, 8)):
        """The pages' Memory Parallel as far as one GPU shows it: the store cut
        into G contiguous document shards, and the calls one GPU of G makes per
        layer at its real shape (routing score and top-k over its shard), then
        the global reduce of the G lists (msa_topk_merge).  Event-timed over
        the layers; the all-gather of the G * k keys between GPUs is not
        measured here (one GPU).  Each leg is captured once and replayed as a
        HIP graph."""
        torch, p, M = self.torch, self.p, self.M
        co = p.chunk_off
        ok = np.flatnonzero(co[:-1] % 16 == 0)   # shards start on 16-chunk groups of the tiled store
        k, B = p.k, p.B
        out = {"note": "per-GPU calls of a G-GPU Memory Parallel step, timed on one GPU; the all-gather of "
                       "G x k (score, id) keys per query between GPUs is not measured"}
        for G in shard_counts:
            cuts = [0] + [int(ok[np.searchsorted(ok, g * p.n_docs // G)]) for g in range(1, G)] + [p.n_docs]
            lo, hi = cuts[0], cuts[1]
            c0, c1 = int(co[lo]), int(co[hi])
            nc, nd = c1 - c0, hi - lo
            co_g = torch.from_numpy(co[lo:hi + 1] - c0).to(self.dev)
            cd_g = M.msa_chunk_doc_map(co_g, nc)
            score = torch.empty((B, nd), dtype=torch.float32, device=self.dev)
            ids = torch.empty((B, k), dtype=torch.int32, device=self.dev)
            vals = torch.empty((B, k), dtype=torch.float32, device=self.dev)
            tk_ws = torch.empty(max(M.msa_topk_workspace(B, nd, k), 1), dtype=torch.uint8, device=self.dev)
            lay = self.kr_layout
            shards = [self.store[l][c0:c0 + M.padded_chunks(nc, lay)] for l in range(self.layers)]

            def select():
                for l in range(self.layers):
                    M.msa_route_score(self.qr[l], shards[l], cd_g, nd, doc_score=score, layout=lay)
                    M.msa_topk(score, k, ids=ids, vals=vals, ws=tk_ws)
            # replayed as HIP graphs, so that the host's issue rate does not
            # bound the small per-shard launches
            g_sel = M.StepGraph(select)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g_sel.replay()
            e0.record()
            g_sel.replay()
            e1.record()
            torch.cuda.synchronize()
            sel_us = e0.elapsed_time(e1) * 1e3 / self.layers
            gv = vals.unsqueeze(0).expand(G, B, k).contiguous()
            gi = ids.unsqueeze(0).expand(G, B, k).contiguous()
            off = torch.tensor(cuts[:-1], dtype=torch.int64, device=self.dev)
            mi = torch.empty((B, k), dtype=torch.int32, device=self.dev)
            mv = torch.empty((B, k), dtype=torch.float32, device=self.dev)

            def merge():
                for _ in range(self.layers):
                    M.msa_topk_merge(gv, gi, off, k, ids_out=mi, vals_out=mv)
            g_m = M.StepGraph(merge)
            g_m.replay()
            e0.record()
            g_m.replay()
            e1.record()
            torch.cuda.synchronize()
            merge_us = e0.elapsed_time(e1) * 1e3 / self.layers
            shard_bytes = nc * p.H * p.d * self.esz
            out[f"G{G}"] = {"shard_docs": nd, "shard_chunks": nc, "shard_store_GB": round(shard_bytes / 1e9, 3),
                            "route_and_topk_us_per_layer": round(sel_us, 2),
                            "shard_routing_GBps": round(shard_bytes / (sel_us * 1e-6) / 1e9, 1),
                            "merge_us_per_layer": round(merge_us, 2),
                            "select_ms_per_step": round((sel_us + merge_us) * self.layers / 1e3, 4)}
            del shards, g_sel, g_m
        return out

    def pin_host(self):
        """The pages' tier: content K/V in pinned host memory.  A host pins
        only part of the 115 GB, so as many layers as fit are pinned and the
        18 layers cycle over them (the fetch cost does not depend on the
        values).  Returns kv(l) and a description, or None."""
        torch, p = self.torch, self.p
        t0 = time.time()
        hk, hv = [], []
        try:
            for l in range(self.layers):
                a = torch.empty((p.n_chunks, p.H, p.d), dtype=self.bf, pin_memory=True)
                b = torch.empty((p.n_chunks, p.H, p.d), dtype=self.bf, pin_memory=True)
                a.copy_(self.kbar[l])
                b.copy_(self.vbar[l])
                hk.append(a)
                hv.append(b)
        except (RuntimeError, torch.OutOfMemoryError) as e:   # pinned host memory exhausted
            log(f"host tier: pinned {len(hk)} layers ({str(e).splitlines()[0]})")
        torch.cuda.synchronize()
        n_pin = len(hk)
        if n_pin == 0:
            return None
        pinned_gb = 2 * n_pin * p.n_chunks * p.H * p.d * self.esz / 1e9
        log(f"host tier: {n_pin} layers pinned ({pinned_gb:.1f} GB) in {time.time() - t0:.1f} s")
        self.pinned = (hk, hv)
        desc = {"pinned_layers": n_pin, "pinned_GB": round(pinned_gb, 1), "layers_cycled": self.layers,
                "note": f"layer l reads pinned layer l % {n_pin}"}
        return (lambda l: (hk[l % n_pin], hv[l % n_pin])), desc

    def unpin_host(self):
        self.pinned = None
        if hasattr(self.torch._C, "_host_emptyCache"):
            self.torch._C._host_emptyCache()    # hand the pinned pages back

    def host_tier(self, steps, warmup, pinned, modes=("mapped", "memcpy")):
        """The step with the content K/V in pinned host memory (pin_host),
        timed for the zero-copy gather kernel (mapped), for hipMemcpyAsync per
        document on a side stream (memcpy), and with each layer's fetch done in
        the next layer's routing scan (fetch_in_next_route,
        msa_route_score_fetch)."""
        p, M = self.p, self.M
        kv, desc = pinned
        out = dict(desc)
        hbm_runner = self.runner
        srcs = {"mapped": M.MSA_SRC_HOST_MAPPED, "memcpy": M.MSA_SRC_HOST_MEMCPY,
                "fetch_in_next_route": M.MSA_SRC_HOST_MAPPED}
        for mode in modes:
            src = srcs[mode]
            self.fetch_in_route = mode == "fetch_in_next_route"
            self.make_runner("host", indexed=False, src_mode=src)
            ms, route_ms = self.timed(steps, warmup, kv=kv)
            if self.pipelined and self.graph:
                ms = min(ms, self.timed(steps, warmup, kv=kv, route_events=False, graph=True)[0])
            stage = self.stages(min(steps, 3), kv=kv)
            fetch_key = "fetch_last_layer" if self.pipelined else "fetch"
            out[mode] = {"route_attn_us_per_query": round(ms * 1e3 / p.B, 1), "ms_per_step": round(ms, 4),
                         "fetch_ms_per_step": round(stage[2], 4),
                         "stage_ms_per_step": {("route_score_and_previous_fetch" if self.pipelined else "route_score"):
                                               round(stage[0], 4), "topk": round(stage[1], 4),
                                               fetch_key: round(stage[2], 4), "attention": round(stage[3], 4)},
                         "fetched_bytes_per_step": int(self.runner.ctx_len.sum().item()) * p.H * p.d * 2 * self.esz
                         * self.layers}
            if self.pipelined:
                out[mode]["note"] = ("each layer's fetch runs in the next layer's routing launch; this order holds "
                                     "only when that routing call does not depend on the fetched layer's output, "
                                     "as between independent queries served together (the synthetic layers here "
                                     "are independent); one query's next-layer routing needs this layer's output")
            log(f"host tier {mode}: {ms:.3f} ms per step, fetch {stage[2]:.3f} ms")
        self.fetch_in_route = False
        self.pipelined = False
        self.runner = hbm_runner
        return out

    def cold(self, flush_buf):
        """Per-stage ms per step with the caches flushed before every layer (a
        1 GB buffer written), and the whole step as the sum of its stages."""
        stage = self.stages(2, flush=lambda: flush_buf.fill_(1))
        return stage

    def release(self):
        self.store = None
        self.kbar, self.vbar = [], []
        self.runner = None
        self.raw = None
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def config_leg(torch, name, args):
    """Per-config line for the smaller presets: warm and cold step times,
    routing and attention GB/s, and the oracle's routing and attention time
    on the host's cores (bounded samples)."""
    from synth import configs
    p = configs.PRESETS[name]()
    pb = PresetBench(torch, p, graph=not args.no_graph, overlap=args.overlap, fill_in_topk=not args.no_fill_in_topk)
    pb.build_stores()
    pb.build_content("hbm")
    pb.make_runner("hbm", indexed=True)
    recall = pb.needle_recall()
    steps, warmup = max(3, min(args.steps, 10)), max(1, min(args.warmup, 3))
    ms_eager, _ = pb.timed(steps, warmup, route_events=False)
    ms_graph = pb.timed(steps, warmup, route_events=False, graph=True)[0] if pb.graph else float("inf")
    ms = min(ms_eager, ms_graph)
    warm = pb.stages(2)
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=pb.dev)
    cold = pb.cold(flush_buf)
    del flush_buf
    store_bytes = p.n_chunks * p.H * p.d * pb.esz * pb.layers
    attn_bytes = pb.attn_bytes() * pb.layers

    def gbps(b, ms_):
        return round(b / (ms_ * 1e-3) / 1e9, 1)
    out = {
        "workload": f"{p.n_docs} docs, {int(p.lengths.sum())} tokens, {p.n_chunks} chunks/layer, {pb.layers} layers; "
                    f"B={p.B} x T={p.T}, L_loc={p.L_loc}, k={p.k}, {'bf16' if p.bf16 else 'f32'}",
        "ms_per_step": round(ms, 4), "us_per_query": round(ms * 1e3 / p.B, 1),
        "step_launch": "hip-graph replay" if ms_graph < ms_eager else "eager launches",
        "ms_per_step_eager_launches": round(ms_eager, 4),
        "ms_per_step_graph_replay": round(ms_graph, 4) if pb.graph else None,
        "routing_GBps": gbps(store_bytes, warm[0] + warm[1]),
        "attention_GBps": gbps(attn_bytes, warm[3]),
        "stage_ms_per_step": {"route_score": round(warm[0], 4), "topk_and_context_index": round(warm[1], 4),
                              "attention": round(warm[3], 4)},
        "cold": {"flush": "1 GB buffer written before every layer",
                 "ms_per_step_sum_of_stages": round(float(cold.sum()), 4),
                 "routing_GBps": gbps(store_bytes, cold[0] + cold[1]), "attention_GBps": gbps(attn_bytes, cold[3]),
                 "stage_ms_per_step": {"route_score": round(cold[0], 4), "topk_and_context_index": round(cold[1], 4),
                                       "attention": round(cold[3], 4)}},
        "needle_recall_layer0": recall,
    }
    ctx_len0 = int(pb.runner.ctx_len[0].item())
    pb.release()
    del pb
    if not args.no_cpu_baseline:
        out["oracle"] = oracle_leg(p, ctx_len0)
    log(f"{name}: {ms:.3f} ms per step (warm), {float(cold.sum()):.3f} ms (cold)")
    return out


def oracle_leg(p, ctx_len0):
    """The float64 oracle timed on the host cores: routing (score + top-k) of
    two routed layers' queries against a bounded sample of the memory,
    scaled to the whole memory, and the attention of query 0 over a context
    of the GPU's length plus the local tokens."""
    import oracle as O
    import synth
    cores = _oracle_threads()
    base = cpu_baseline(p, 2, n_sample_chunks=min(p.n_chunks, 1 << 16), quiet=True)
    route_ms = base["seconds"] * 1e3 / 2 * (p.n_chunks / base["sample_chunks"])
    bf = p.bf16
    H, d = p.H, p.d
    kc = synth.tensor(p.seed, 0, synth.T_K, (max(ctx_len0, 1), H, d), bf16=bf, scale_pow2=-3)
    vc = synth.tensor(p.seed, 0, synth.T_V, (max(ctx_len0, 1), H, d), bf16=bf, scale_pow2=-3)
    pos = np.arange(max(ctx_len0, 1)) % max(p.max_doc_chunks, 1)
    q = synth.tensor(p.qseed, 0, synth.T_Q, (1, p.T, p.Hq, d), bf16=bf)[0]
    kl = synth.tensor(p.qseed, 0, synth.T_KLOC, (p.L_loc, H, d), bf16=bf)
    vl = synth.tensor(p.qseed, 0, synth.T_VLOC, (p.L_loc, H, d), bf16=bf)
    t0 = time.perf_counter()
    O.attend_one(q, kc[:ctx_len0], vc[:ctx_len0], pos[:ctx_len0], kl, vl, p.qpo, p.rope_base, 1.0 / math.sqrt(d))
    attn_ms = (time.perf_counter() - t0) * 1e3
    return {"kind": "oracle", "cores": cores,
            "route_ms_per_query_layer": round(route_ms / p.B, 4),
            "attention_ms_per_query_layer": round(attn_ms, 4),
            "route_sample": f"{base['sample_chunks']} of {p.n_chunks} chunks, 2 layers' queries, scaled to the whole "
                            f"memory",
            "attention_sample": f"query 0: {ctx_len0} context entries + {p.L_loc} local tokens, {p.T} tokens x "
                                f"{p.Hq} heads"}


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def counted_traffic(preset_name):
    """HBM bytes per routing-score launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE scaled by a plain copy), or None when the
    kernel sources changed since the counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", "route_score_100M.txt")
    if preset_name != "cfg4" or not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("route_score.hip", "common.h"):
        h.update(open(os.path.join(here, "sparse_attention_long_msa_amd", "csrc", f), "rb").read())
    if fields.get("kernel_sources_sha256") != h.hexdigest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def train_main(args, torch):
    """Training-time path, one step = every routed layer of one sample:
    routing scores with their maximisers -> routing loss -> routing-score
    backward -> top-k -> context index -> attention backward (forward
    recomputed) -> pooling backward of the routing keys, K and V to the
    tokens.  Inputs are seeded synthetic tensors; the output gradient of the
    attention is a seeded synthetic tensor."""
    import synth
    from synth import configs
    from synth import device as SD
    import sparse_attention_long_msa_amd as M

    name = "train64k" if args.config == "cfg4" else args.config
    p = configs.TRAIN_PRESETS[name]()
    layers = p.layers if args.layers is None else args.layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = torch.bfloat16
    H, d, N, D, B, T, Hq, L, k = p.H, p.d, p.n_chunks, p.n_docs, p.B, p.T, p.Hq, p.L_loc, p.k
    tau = 0.1
    tok_off, chunk_off = p.tok_off, p.chunk_off
    n_tok = int(tok_off[-1])
    to_d = torch.from_numpy(tok_off).to(dev)
    co_d = torch.from_numpy(chunk_off).to(dev)
    cd = M.msa_chunk_doc_map(co_d, N)
    t0 = time.time()
    # token-level routing keys (kept: the pooling backward renormalises them), pooled stores
    xr = [SD.fill(torch.empty((n_tok, H, d), dtype=bf, device=dev), p.seed, l, synth.T_KR) for l in range(layers)]
    kr = [M.msa_pool_encode(xr[l], to_d, co_d, cd, p.chunk, True) for l in range(layers)]
    raw = torch.empty((n_tok, H, d), dtype=bf, device=dev)
    kbar, vbar = [], []
    for l in range(layers):
        kbar.append(M.msa_pool_encode(SD.fill(raw, p.seed, l, synth.T_K), to_d, co_d, cd, p.chunk, False))
        vbar.append(M.msa_pool_encode(SD.fill(raw, p.seed, l, synth.T_V), to_d, co_d, cd, p.chunk, False))
    del raw
    qr = [SD.fill(torch.empty((B, T, H, d), dtype=bf, device=dev), p.qseed, l, synth.T_QR) for l in range(layers)]
    qq = [SD.fill(torch.empty((B, T, Hq, d), dtype=bf, device=dev), p.qseed, l, synth.T_Q) for l in range(layers)]
    kl = [SD.fill(torch.empty((B, L, H, d), dtype=bf, device=dev), p.qseed, l, synth.T_KLOC) for l in range(layers)]
    vl = [SD.fill(torch.empty((B, L, H, d), dtype=bf, device=dev), p.qseed, l, synth.T_VLOC) for l in range(layers)]
    dout = [SD.fill(torch.empty((B, T, Hq, d), dtype=torch.float32, device=dev), p.qseed, l, synth.T_DOUT)
            for l in range(layers)]
    pos = torch.from_numpy(np.stack([synth.needle_docs(p.seed, D, p.n_needles, salt=b) for b in range(B)])
                           .astype(np.int32)).to(dev)
    max_doc = p.max_doc_chunks
    max_ctx = k * max_doc
    tab = M.msa_rope_table(M.msa_rope_table_rows(max_ctx, L, p.qpo), d, p.rope_base, device=dev)
    # outputs and scratch, reused by every layer
    f32 = dict(dtype=torch.float32, device=dev)
    score, ac, at = (torch.empty((B, D), **f32), torch.empty((B, D), dtype=torch.int32, device=dev),
                     torch.empty((B, D), dtype=torch.int32, device=dev))
    ax_ws = torch.empty(M.msa_route_argmax_workspace(M.MSA_BF16, B, T, H, d, D, N), dtype=torch.uint8, device=dev)
    loss = torch.empty((layers, B), **f32)
    grad = torch.empty((B, D), **f32)
    dqr = torch.empty((B, T, H, d), **f32)
    # the three accumulated store gradients share one buffer: one clearing launch per layer
    acc = torch.empty((3, N, H, d), **f32)
    dkr, dkb, dvb = acc[0], acc[1], acc[2]
    ids, vals = torch.empty((B, k), dtype=torch.int32, device=dev), torch.empty((B, k), **f32)
    tk_ws = torch.empty(max(M.msa_topk_workspace(B, D, k), 1), dtype=torch.uint8, device=dev)
    row, cpos, clen = (torch.empty((B, max_ctx), dtype=torch.int32, device=dev),
                       torch.empty((B, max_ctx), dtype=torch.int32, device=dev),
                       torch.empty((B,), dtype=torch.int32, device=dev))
    bw_ws = torch.empty(M.msa_sparse_attn_backward_workspace(M.MSA_BF16, B, T, Hq, H, d, max_ctx, L, p.qpo),
                        dtype=torch.uint8, device=dev)
    dq, dkl, dvl = (torch.empty((B, T, Hq, d), **f32), torch.empty((B, L, H, d), **f32),
                    torch.empty((B, L, H, d), **f32))
    dxr, dxk, dxv = (torch.empty((n_tok, H, d), **f32) for _ in range(3))
    torch.cuda.synchronize()
    log(f"{p.name}: {D} docs, {N} chunks/layer, {layers} layers, T={T}; inputs ready in {time.time() - t0:.1f} s")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        for l in range(layers):
            if ev is not None:
                ev[l][0].record(stream)
            M.msa_route_argmax(qr[l], kr[l], cd, D, doc_score=score, arg_chunk=ac, arg_tok=at, ws=ax_ws)
            M.msa_route_loss(score, pos, tau, loss=loss[l], grad=grad)
            acc.zero_()
            M.msa_route_score_backward(qr[l], kr[l], ac, at, grad, dkr, dq_r=dqr)
            M.msa_topk_context_index(score, k, co_d, N, max_doc, max_ctx, ids=ids, vals=vals, ctx_row=row, ctx_pos=cpos,
                                     ctx_len=clen, ws=tk_ws)
            if ev is not None:
                ev[l][1].record(stream)
            M.msa_sparse_attn_backward(qq[l], kbar[l], vbar[l], row, cpos, clen, kl[l], vl[l], p.qpo, dout[l], dkb,
                                       dvb, rope_base=p.rope_base, rope_table=tab, dq=dq, dk_loc=dkl, dv_loc=dvl,
                                       ws=bw_ws)
            if ev is not None:
                ev[l][2].record(stream)
            M.msa_pool_backward(dkr, to_d, co_d, cd, n_tok, p.chunk, x=xr[l], dx=dxr)
            M.msa_pool_backward(dkb, to_d, co_d, cd, n_tok, p.chunk, dtype=M.MSA_BF16, dx=dxk)
            M.msa_pool_backward(dvb, to_d, co_d, cd, n_tok, p.chunk, dtype=M.MSA_BF16, dx=dxv)
            if ev is not None:
                ev[l][3].record(stream)

    step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    n_stage = min(args.steps, 3)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(layers)] for _ in range(n_stage)]
    for s_ in range(n_stage):
        step(evs[s_])
    torch.cuda.synchronize()
    stage = np.zeros(3)
    for s_ in range(n_stage):
        for l in range(layers):
            e = evs[s_][l]
            stage += [e[i].elapsed_time(e[i + 1]) for i in range(3)]
    stage /= n_stage
    ms = wall * 1e3 / args.steps
    # attention backward, per layer: visible (row, key) pairs x (4 d forward + 10 d backward) flops
    ctx_len = int(clen.sum().item())
    horizon = L - T + np.arange(T)
    pairs = Hq * (B * T * (ctx_len // B) + B * int(np.minimum(horizon + 1, L).sum()))
    attn_flops = pairs * 14 * d
    attn_ms = stage[1] / layers
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    res = {
        "metric": "training-path query tokens/s (routing loss + attention backward, all routed layers)",
        "value": round(B * T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator)",
        "config": {"workload": f"{p.name}: {n_tok}-token memory, {D} docs, chunk {p.chunk}, {N} chunks/layer, "
                               f"{layers} routed layers, H={H}, d={d}; {B} x T={T} trained tokens, Hq={Hq}, "
                               f"L_loc={L}, k={k}, {p.n_needles} positives, tau={tau}",
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "stage_ms_per_step": {"routing_fwd_loss_bwd_topk_index": round(stage[0], 4),
                              "attention_fwd_recompute_and_bwd": round(stage[1], 4),
                              "pool_backward_kr_k_v": round(stage[2], 4)},
        "mean_routing_loss": round(float(loss.mean().item()), 5),
        "roofline": {"kernel": "msa_sparse_attn_backward (forward recompute + dK/dV + dQ)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(achieved / 2500.0, 4), "traffic": None,
                     "avg_call_ms": round(attn_ms, 4), "alg_flops_per_call": int(attn_flops)},
    }
    print(json.dumps(res), flush=True)


def encode_main(args, torch):
    """Stage 1 at corpus scale: one call = one routed layer's pooled stores
    (K, V, normalised K_r) of the 1M-token memory (2,048 documents x 512
    tokens, chunk 64) from the tokens' hidden states (hidden 2,560, the
    backbone's width) and synthetic projection weights."""
    import synth
    from synth import configs
    from synth import device as SD
    import sparse_attention_long_msa_amd as M

    p = configs.PRESETS["cfg2"]()
    hidden, H, d = 2560, p.H, p.d
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = torch.bfloat16
    tok_off, chunk_off = p.tok_off, p.chunk_off
    n_tok, N = int(tok_off[-1]), p.n_chunks
    to_d = torch.from_numpy(tok_off).to(dev)
    co_d = torch.from_numpy(chunk_off).to(dev)
    cd = M.msa_chunk_doc_map(co_d, N)
    x = SD.fill(torch.empty((n_tok, hidden), dtype=bf, device=dev), p.seed, 0, synth.T_K)
    w = SD.fill(torch.empty((3 * H * d, hidden), dtype=bf, device=dev), p.seed, 0, synth.T_V, scale_pow2=-6)
    kb = torch.empty((N, H, d), dtype=bf, device=dev)
    vb = torch.empty_like(kb)
    kr = torch.empty((M.padded_chunks(N, M.MSA_LAYOUT_TILED), H, d), dtype=bf, device=dev)
    ws = torch.empty(M.lib.msa_encode_workspace(M.MSA_BF16, N, hidden, H, d), dtype=torch.uint8, device=dev)

    def call():
        M.msa_encode(x, w, to_d, co_d, cd, p.chunk, H, d, kr_layout=M.MSA_LAYOUT_TILED, k_bar=kb, v_bar=vb,
                     kr_hat=kr, ws=ws)

    for _ in range(max(args.warmup, 1)):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record()
        call()
        e[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    x_bytes = n_tok * hidden * 2
    alg = x_bytes + 2 * N * hidden * 4 + 3 * H * d * hidden * 2 + 3 * N * H * d * 2
    gemm_flops = 2 * N * hidden * 3 * H * d
    res = {
        "metric": "Stage-1 encode: hidden-state GB/s (pool + projection to K, V, K_r)",
        "value": round(x_bytes / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; synthetic projection weights)",
        "config": {"workload": f"encode: {n_tok}-token memory (cfg2 documents), chunk {p.chunk}, {N} chunks, "
                               f"hidden {hidden}, H={H}, d={d}, one routed layer per call",
                   "global_batch": 1, "seq_len": n_tok, "parallelism": "single GPU"},
        "tokens_per_s": round(n_tok / (ms * 1e-3), 1),
        "projected_100M_tokens_18_layers_s": round(18 * 100e6 / (n_tok / (ms * 1e-3)), 1),
        "gemm_flops_per_call": gemm_flops,
        "roofline": {"kernel": "msa_encode (pool_hidden_kernel + encode_gemm_kernel)", "bound": "hbm",
                     "achieved": round(alg / (ms * 1e-3) / 1e9, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(alg / (ms * 1e-3) / 1e9 / 8000.0, 4), "traffic": None,
                     "avg_call_ms": round(ms, 4), "alg_bytes_per_call": int(alg)},
    }
    print(json.dumps(res), flush=True)


def encode_corpus_main(args, torch):
    """Stage 1 at corpus scale: the pooled stores of every routed layer of the
    100M-token memory (195,312 documents x 512 tokens, chunk 64: K, V and the
    normalised K_r, 1,562,496 chunks per layer, 173 GB in HBM) from the
    tokens' hidden states (width 2,560), 2,048 documents (1M tokens, 5.4 GB of
    hidden states) per block, 96 blocks per layer.  The hidden states of four
    blocks are generated once (seeded synthetic values) and the blocks cycle
    over them: the encode cost does not depend on the values, and the inputs
    of a 100M-token layer (512 GB) cannot be held at once.  Timed twice:
    msa_encode per block on one stream (serial), and msa_encode_pool /
    msa_encode_project on two streams with two workspaces, so that a block's
    pooling (HBM-bound) overlaps the previous block's projection (MFMA)."""
    import synth
    from synth import configs
    from synth import device as SD
    import sparse_attention_long_msa_amd as M

    p = configs.cfg4()
    layers = p.layers if args.layers is None else args.layers
    hidden, H, d, chunk = 2560, p.H, p.d, p.chunk
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = torch.bfloat16
    N = p.n_chunks
    blk_docs = 2048
    tok_per_doc = int(p.lengths[0])
    assert (p.lengths == tok_per_doc).all()
    kb = torch.empty((layers, N, H, d), dtype=bf, device=dev)
    vb = torch.empty((layers, N, H, d), dtype=bf, device=dev)
    kr = torch.empty((layers, M.padded_chunks(N, M.MSA_LAYOUT_TILED), H, d), dtype=bf, device=dev)
    NX = 4
    xs = [SD.fill(torch.empty((blk_docs * tok_per_doc, hidden), dtype=bf, device=dev), p.seed, 0, synth.T_K,
                  start=i * blk_docs * tok_per_doc * hidden) for i in range(NX)]
    ws_ = [SD.fill(torch.empty((3 * H * d, hidden), dtype=bf, device=dev), p.seed, l, synth.T_V, scale_pow2=-6)
           for l in range(layers)]
    cpb = blk_docs * tok_per_doc // chunk                     # chunks per full block
    wsb = M.lib.msa_encode_workspace(M.MSA_BF16, cpb, hidden, H, d)
    work = [torch.empty(wsb, dtype=torch.uint8, device=dev) for _ in range(2)]

    def index(n_docs):
        to = synth.offsets(np.full(n_docs, tok_per_doc, dtype=np.int64))
        co = synth.offsets(np.full(n_docs, tok_per_doc // chunk, dtype=np.int64))
        to_d, co_d = torch.from_numpy(to).to(dev), torch.from_numpy(co).to(dev)
        return to_d, co_d, M.msa_chunk_doc_map(co_d, int(co[-1]))
    n_blocks = (p.n_docs + blk_docs - 1) // blk_docs
    last_docs = p.n_docs - (n_blocks - 1) * blk_docs
    idx = {blk_docs: index(blk_docs), last_docs: index(last_docs)}
    log(f"encode corpus: {p.n_docs} docs, {N} chunks/layer, {layers} layers, {n_blocks} blocks per layer; stores "
        f"{3 * layers * N * H * d * 2 / 1e9:.1f} GB")

    def block(bi):
        nd = blk_docs if bi < n_blocks - 1 else last_docs
        n_tok, nc = nd * tok_per_doc, nd * tok_per_doc // chunk
        return idx[nd], n_tok, nc, bi * cpb

    def outs(l, c0, nc):
        return dict(k_bar=kb[l, c0:c0 + nc], v_bar=vb[l, c0:c0 + nc],
                    kr_hat=kr[l, c0:c0 + M.padded_chunks(nc, M.MSA_LAYOUT_TILED)])

    def serial():
        for l in range(layers):
            for bi in range(n_blocks):
                (to_d, co_d, cd), n_tok, nc, c0 = block(bi)
                M.msa_encode(xs[bi % NX][:n_tok], ws_[l], to_d, co_d, cd, chunk, H, d, kr_layout=M.MSA_LAYOUT_TILED,
                             ws=work[0], **outs(l, c0, nc))

    s_pool, s_proj = torch.cuda.Stream(), torch.cuda.Stream()

    def pipelined():
        s_pool.wait_stream(torch.cuda.current_stream())
        s_proj.wait_stream(torch.cuda.current_stream())
        done = [None, None]                  # the projection that last read each workspace
        i = 0
        for l in range(layers):
            for bi in range(n_blocks):
                (to_d, co_d, cd), n_tok, nc, c0 = block(bi)
                w = work[i % 2]
                if done[i % 2] is not None:
                    s_pool.wait_event(done[i % 2])
                with torch.cuda.stream(s_pool):
                    M.msa_encode_pool(xs[bi % NX][:n_tok], to_d, co_d, cd, chunk, H, d, ws=w)
                    pooled = torch.cuda.Event()
                    pooled.record(s_pool)
                s_proj.wait_event(pooled)
                with torch.cuda.stream(s_proj):
                    M.msa_encode_project(ws_[l], nc, H, d, w, kr_layout=M.MSA_LAYOUT_TILED, **outs(l, c0, nc))
                    done[i % 2] = torch.cuda.Event()
                    done[i % 2].record(s_proj)
                i += 1
        torch.cuda.current_stream().wait_stream(s_proj)

    res_t = {}
    for name, fn in (("serial", serial), ("pipelined", pipelined)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        res_t[name] = time.perf_counter() - t0
        log(f"encode corpus {name}: {res_t[name]:.3f} s for {layers} layers")
    n_tok_total = int(p.lengths.sum())
    x_bytes = n_tok_total * hidden * 2 * layers
    best = min(res_t, key=res_t.get)
    t = res_t[best]
    res = {
        "metric": "Stage-1 encode at corpus scale: hidden-state GB/s (pool + projection to K, V, K_r)",
        "value": round(x_bytes / t / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": 1,
        "warmup": 0,
        "ms_per_step": round(t * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; four input blocks cycled; synthetic projection weights)",
        "config": {"workload": f"encode corpus: {n_tok_total}-token memory ({p.n_docs} docs x {tok_per_doc}), "
                               f"chunk {chunk}, {N} chunks/layer, {layers} routed layers, hidden {hidden}, H={H}, "
                               f"d={d}; {n_blocks} blocks of {blk_docs} docs per layer",
                   "global_batch": 1, "seq_len": n_tok_total, "parallelism": "single GPU", "launch": best},
        "encode_s_all_layers": {k: round(v, 3) for k, v in res_t.items()},
        "tokens_per_s": round(n_tok_total * layers / t, 1),
        "ms_per_block": {k: round(v * 1e3 / (layers * n_blocks), 4) for k, v in res_t.items()},
        "stores_GB": round(3 * layers * N * H * d * 2 / 1e9, 1),
    }
    print(json.dumps(res), flush=True)


def copy_calibration(torch):
    """A plain device copy of 1 GiB, three times: the reference that scales the
    HBM byte counters (FETCH_SIZE / WRITE_SIZE) of the other kernels."""
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty(n, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)


def cpu_baseline(p, layers, n_sample_chunks=None, quiet=False):
    """The float64 oracle's routing (score + top-k) timed on a bounded sample
    of the same workload: every routed layer's query scored against the
    routing keys of layer 0's first documents.  The sample's keys come from
    the seeded generator (its device copy, bit-identical to the host one) and
    are pooled and normalised by the oracle before the timed region."""
    import torch

    import oracle as O
    import synth
    from synth import device as SD
    threads = _oracle_threads()
    if n_sample_chunks is None:
        n_sample_chunks = 1 << 20 if p.pooled_level else 1 << 18
    n_docs = int(np.searchsorted(p.chunk_off, n_sample_chunks, side="right") - 1)
    n_docs = max(1, min(n_docs, p.n_docs))
    co = p.chunk_off[: n_docs + 1]
    n = int(co[-1])
    dt_name = "bf16" if p.bf16 else "f32"
    t_prep = time.perf_counter()
    blk = 1 << 17
    buf = torch.empty((blk, p.H, p.d), dtype=torch.bfloat16 if p.bf16 else torch.float32, device="cuda")

    def gen_rows(r0, r1):
        """rows r0 .. r1-1 of layer 0's raw routing keys (float64, host)"""
        out = np.empty((r1 - r0, p.H, p.d), dtype=np.float64)
        for a in range(r0, r1, blk):
            b = min(r1, a + blk)
            SD.fill(buf[: b - a], p.seed, 0, synth.T_KR, start=a * p.H * p.d)
            out[a - r0:b - r0] = buf[: b - a].float().cpu().numpy()
        return out

    if p.pooled_level:
        # chunk = 1: pooling is the identity, the store is the normalised, rounded
        # keys (the oracle's pool_encode, checked here on a slice, without its
        # per-chunk loop)
        raw = gen_rows(0, n)
        store = O.round_to_store(O.l2_normalize(raw), dt_name)
        assert np.array_equal(store[:256], O.pool_encode(raw[:256], np.arange(257), 1, True, dt_name))
        del raw
    else:
        # the oracle pools the tokens of a few documents at a time
        parts, d0 = [], 0
        while d0 < n_docs:
            d1 = int(np.searchsorted(p.tok_off, p.tok_off[d0] + (1 << 20), side="right") - 1)
            d1 = min(n_docs, max(d0 + 1, d1))
            t0_, t1_ = int(p.tok_off[d0]), int(p.tok_off[d1])
            parts.append(O.pool_encode(gen_rows(t0_, t1_), p.tok_off[d0:d1 + 1] - t0_, p.chunk, True, dt_name))
            d0 = d1
        store = np.concatenate(parts)
        assert store.shape[0] == n
    del buf
    queries = [synth.tensor(p.qseed, l, synth.T_QR, (p.B, p.T, p.H, p.d), bf16=p.bf16) for l in range(layers)]
    t_prep = time.perf_counter() - t_prep
    t0 = time.perf_counter()
    for qr in queries:
        s = O.route_scores(qr, store, co)
        O.topk(s, p.k)
    dt = time.perf_counter() - t0
    gb = layers * n * p.H * p.d * (2 if p.bf16 else 4) / 1e9
    if not quiet:
        log(f"cpu baseline ({p.name}): sample prepared in {t_prep:.1f} s, oracle routing {dt:.1f} s")
    return {"value": round(gb / dt, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 4), "sample_chunks": n,
            "sample": f"layer 0, first {n_docs} documents ({n} pooled chunks, "
                      f"{n * p.H * p.d * (2 if p.bf16 else 4) / 1e9:.2f} GB of routing keys) scored against each of the "
                      f"{layers} routed layers' {p.B} x {p.T}-token queries: routing score + top-k, float64"}


if __name__ == "__main__":
    main()
