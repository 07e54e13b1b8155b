"""Benchmark of the MSA routing + sparse-attention hot path on one MI355X.

One step = one query through all routed layers: per layer, routing score over
that layer's whole pooled routing-key store -> top-k -> context assembly
(content K/V fetched from the host tier or HBM) -> sparse attention.  The
default workload is the 100M-token memory (195,312 documents x 512 tokens,
chunk 64 -> 1,562,496 pooled chunks per layer, 18 layers, 8 heads x 128,
bf16; the routing-key store is 57.6 GB in HBM), query of 64 tokens, 32 query
heads, 4,096 local tokens, k = 16.  Inputs are seeded synthetic data
generated on the device before the timed region.

Timing: the K timed steps are measured by the wall clock between two device
synchronisations; inside them only one pair of HIP events per step brackets a
routing-score launch (the roofline's launch duration).  The per-stage
breakdown comes from up to 3 further steps with events between all stages
(each event record idles the device for a few microseconds, so these steps
are not part of the timed region).

Prints one JSON line.  --gpus above 1 is not supported (one GPU per process,
no collectives in this build).
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
    ap.add_argument("--kv-tier", choices=["host", "hbm"], default="host")
    ap.add_argument("--gather", choices=["mapped", "memcpy"], default="mapped",
                    help="host tier: how the selected K/V cross the host link")
    ap.add_argument("--hbm-assembly", choices=["index", "copy"], default="index",
                    help="HBM tier: attention reads the selected rows in place (index) or from a gathered copy")
    ap.add_argument("--layers", type=int, default=None, help="override the routed-layer count (profiling only)")
    ap.add_argument("--rounds", type=int, default=1,
                    help="Memory Interleave rounds per layer (> 1: route, skip the fetched documents, select and "
                         "append, rounds times, then attend; content K/V in HBM)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-chunks", type=int, default=None,
                    help="routing-key chunks of the oracle's sample (default: 1048576 at pooled level, "
                         "262144 for token-level memories, whose sample the oracle also pools)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (the reference for the HBM byte counters)")
    ap.add_argument("--encode", action="store_true",
                    help="time Stage 1 from hidden states instead (msa_encode over a 1M-token memory, one layer per "
                         "call, hidden 2560)")
    ap.add_argument("--train", action="store_true",
                    help="time the training-time path instead (routing loss and attention backward per routed "
                         "layer; --config defaults to train64k)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: --gpus must be 1 "
                                   "(no sharding and no collectives)"}))
        sys.exit(2)
    import torch

    if args.copy_calibration:
        return copy_calibration(torch)
    if args.train:
        return train_main(args, torch)
    if args.encode:
        return encode_main(args, torch)

    import synth
    from synth import configs
    from synth import device as SD
    import sparse_attention_long_msa_amd as M

    p = configs.PRESETS[args.config]()
    layers = p.layers if args.layers is None else args.layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = torch.bfloat16 if p.bf16 else torch.float32
    esz = 2 if p.bf16 else 4
    H, d, N, D = p.H, p.d, p.n_chunks, p.n_docs
    log(f"{p.name}: {D} docs, {N} chunks/layer, {layers} layers, store {N * H * d * esz * layers / 1e9:.1f} GB")

    # ------------------------------------------------------------ document index
    chunk_off = p.chunk_off
    tok_off = p.tok_off
    co_d = torch.from_numpy(chunk_off).to(dev)
    cd = M.msa_chunk_doc_map(co_d, N)

    # ------------------------------------------------------------ query-side inputs (per layer)
    qr = [SD.fill(torch.empty((p.B, p.T, H, d), dtype=bf, device=dev), p.qseed, l, synth.T_QR) for l in range(layers)]
    qq = [SD.fill(torch.empty((p.B, p.T, p.Hq, d), dtype=bf, device=dev), p.qseed, l, synth.T_Q) for l in range(layers)]
    kl = [SD.fill(torch.empty((p.B, p.L_loc, H, d), dtype=bf, device=dev), p.qseed, l, synth.T_KLOC)
          for l in range(layers)]
    vl = [SD.fill(torch.empty((p.B, p.L_loc, H, d), dtype=bf, device=dev), p.qseed, l, synth.T_VLOC)
          for l in range(layers)]

    # ------------------------------------------------------------ routing-key store (HBM)
    # The offline stage (pooling) runs here, before the timed region.  The
    # 100M-token preset is synthesised at pooled level (chunk = 1 pooling,
    # which only normalises); the others pool raw per-token tensors.
    t0 = time.time()
    kr_layout = M.MSA_LAYOUT_TILED if p.bf16 else M.MSA_LAYOUT_ROWS
    store = torch.empty((layers, M.padded_chunks(N, kr_layout), H, d), dtype=bf, device=dev)
    if p.pooled_level:
        rows_off, pool_chunk, n_rows, to_d = chunk_off, 1, N, co_d
    else:
        rows_off, pool_chunk, n_rows = tok_off, p.chunk, int(tok_off[-1])
        to_d = torch.from_numpy(tok_off).to(dev)
    raw = torch.empty((n_rows, H, d), dtype=bf, device=dev)
    needles = synth.needle_docs(p.seed, D, p.n_needles)
    encode_ms = []
    for l in range(layers):
        SD.fill(raw, p.seed, l, synth.T_KR)
        for i, nd in enumerate(needles):
            b = i if p.needle_per_query else 0
            qh = qr[l][b].float().cpu().numpy()
            lo, hi = int(rows_off[nd]), int(rows_off[nd + 1])
            rows = synth.needle_rows(qh, p.seed, l, hi - lo, bf16=p.bf16, start=lo)
            raw[lo:hi] = torch.from_numpy(rows).to(dev, bf)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        M.msa_pool_encode(raw, to_d, co_d, cd, pool_chunk, True, out=store[l], layout=kr_layout)
        e1.record()
        torch.cuda.synchronize()
        encode_ms.append(e0.elapsed_time(e1))
    torch.cuda.synchronize()
    log(f"routing-key store ready in {time.time() - t0:.1f} s")

    # ------------------------------------------------------------ content K/V tier
    t0 = time.time()
    tier = args.kv_tier
    if args.rounds > 1 and tier != "hbm":
        log("Memory Interleave rounds read the content K/V in place: using the HBM tier")
        tier = "hbm"
    kbar, vbar = [], []
    kv_scale = -3 if p.pooled_level else 0

    def content(l, tid, out):
        """pooled K or V of layer l into out (device)"""
        SD.fill(raw, p.seed, l, tid, scale_pow2=kv_scale)
        return M.msa_pool_encode(raw, to_d, co_d, cd, pool_chunk, False, out=out)

    if tier == "host":
        try:
            tmp = torch.empty((N, H, d), dtype=bf, device=dev)
            for l in range(layers):
                for lst, tid in ((kbar, synth.T_K), (vbar, synth.T_V)):
                    content(l, tid, tmp)
                    h = torch.empty((N, H, d), dtype=bf, pin_memory=True)
                    h.copy_(tmp)
                    lst.append(h)
                log(f"host tier layer {l} ready ({time.time() - t0:.1f} s)")
            torch.cuda.synchronize()
        except (RuntimeError, torch.OutOfMemoryError) as e:  # pinned host memory exhausted
            log(f"pinned host tier unavailable ({str(e).splitlines()[0]}); falling back to the HBM tier")
            kbar.clear()
            vbar.clear()
            torch.cuda.synchronize()
            tier = "hbm"
    if tier == "hbm":
        for l in range(layers):
            kbar.append(content(l, synth.T_K, torch.empty((N, H, d), dtype=bf, device=dev)))
            vbar.append(content(l, synth.T_V, torch.empty((N, H, d), dtype=bf, device=dev)))
        torch.cuda.synchronize()
    del raw
    log(f"content K/V tier '{tier}' ready in {time.time() - t0:.1f} s")
    src_mode = M.MSA_SRC_DEVICE if tier == "hbm" else (
        M.MSA_SRC_HOST_MAPPED if args.gather == "mapped" else M.MSA_SRC_HOST_MEMCPY)

    runner = M.LayerRunner(batch=p.B, tokens=p.T, q_heads=p.Hq, kv_heads=H, head_dim=d, n_docs=D, n_chunks=N,
                           k=p.k, max_doc_chunks=p.max_doc_chunks, local_len=p.L_loc, dtype=bf, device=dev,
                           q_pos_offset=p.qpo if args.rounds == 1 else None, rope_base=p.rope_base,
                           src_mode=src_mode, chunk_off_h=chunk_off, kr_layout=kr_layout,
                           indexed=(tier == "hbm" and (args.hbm_assembly == "index" or args.rounds > 1)),
                           rounds=args.rounds)
    stream = torch.cuda.current_stream()
    # routing queries of the later rounds: seeded like round 0's, seed + round
    qr_rounds = [[qr[l]] + [SD.fill(torch.empty_like(qr[l]), p.qseed + r, l, synth.T_QR) for r in range(1, args.rounds)]
                 for l in range(layers)]

    def step(ev=None, route_ev=None, route_layer=-1):
        """One pass of the whole path over all routed layers.  ev: per-stage
        events of every layer (stage breakdown); route_ev: events around the
        routing-score call of layer route_layer only (the timed steps)."""
        for l in range(layers):
            if args.rounds > 1:
                if ev is not None:
                    ev[l][0].record(stream)
                runner.fetch_rounds(qr_rounds[l], store[l], cd, co_d, kbar[l], vbar[l],
                                    route_events=route_ev if l == route_layer else None)
                if ev is not None:
                    ev[l][3].record(stream)
                runner.attend(qq[l], kl[l], vl[l])
                if ev is not None:
                    ev[l][4].record(stream)
                continue
            if ev is not None:
                ev[l][0].record(stream)
            if l == route_layer:
                route_ev[0].record(stream)
            runner.route(qr[l], store[l], cd)
            if l == route_layer:
                route_ev[1].record(stream)
            if ev is not None:
                ev[l][1].record(stream)
            if runner.indexed:
                # top-k and the context index in one call (the final selection pass writes the index)
                runner.select_assemble(co_d, kbar[l], vbar[l])
                if ev is not None:
                    ev[l][2].record(stream)
                    ev[l][3].record(stream)
            else:
                runner.select()
                if ev is not None:
                    ev[l][2].record(stream)
                runner.assemble(co_d, kbar[l], vbar[l])
                if ev is not None:
                    ev[l][3].record(stream)
            runner.attend(qq[l], kl[l], vl[l])
            if ev is not None:
                ev[l][4].record(stream)

    # needle check on one pass (a property of the planted data, not timed)
    step()
    torch.cuda.synchronize()
    ids_all = (runner.ids if args.rounds == 1 else runner.ids_rounds[0]).cpu().numpy()
    recall = float(np.mean([int(nd) in set(ids_all[i if p.needle_per_query else 0].tolist())
                            for i, nd in enumerate(needles)]))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed steps: one pair of events per step, around one layer's routing-score
    # call (a different layer each step), so that the step is not slowed by
    # instrumentation; the whole-step time is the wall clock
    route_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        step(route_ev=route_evs[s], route_layer=s % layers)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    route_ms = [e[0].elapsed_time(e[1]) for e in route_evs]
    # stage breakdown: extra, untimed steps with events between all stages
    n_stage = min(args.steps, 3)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(layers)]
           for _ in range(n_stage)]
    for s in range(n_stage):
        step(evs[s])
    torch.cuda.synchronize()
    stage = np.zeros(4)
    for s in range(n_stage):
        for l in range(layers):
            e = evs[s][l]
            if args.rounds > 1:   # rounds (route, skip, select, append) | attention
                stage += [e[0].elapsed_time(e[3]), 0.0, 0.0, e[3].elapsed_time(e[4])]
            else:
                stage += [e[i].elapsed_time(e[i + 1]) for i in range(4)]
    stage /= n_stage
    ms_per_step = wall * 1e3 / args.steps
    store_bytes = N * H * d * esz                      # per layer
    step_bytes = store_bytes * layers * args.rounds   # every round scans the layer's store
    value = step_bytes / (ms_per_step * 1e-3) / 1e9   # GB/s over the whole step
    routing_gbps = step_bytes / ((stage[0] + stage[1]) * 1e-3) / 1e9
    # algorithmic bytes of one msa_route_score launch: the store, the chunk->doc map,
    # the routing query and the score row (initial fill + result)
    alg_bytes = store_bytes + N * 4 + p.B * p.T * H * d * esz + 2 * p.B * D * 4
    route_avg_ms = float(np.mean(route_ms))
    achieved = alg_bytes / (route_avg_ms * 1e-3) / 1e9
    # attention: K/V of the context and the local part, read once per KV head, plus Q and O
    ctx_len = runner.ctx_len.cpu().numpy().astype(np.int64)
    attn_bytes = int((ctx_len + p.L_loc).sum()) * H * d * 2 * esz + p.B * p.T * p.Hq * d * (esz + 4)
    attn_gbps = attn_bytes * layers / (stage[3] * 1e-3) / 1e9
    raw_bytes = n_rows * H * d * esz
    encode_gbps = (raw_bytes + store_bytes) / (float(np.median(encode_ms)) * 1e-3) / 1e9

    workload = (f"{p.name}: {int(p.lengths.sum())}-token memory, {D} docs, chunk {p.chunk}, {N} chunks/layer, "
                f"{layers} routed layers, H={H}, d={d}; {p.B} quer{'y' if p.B == 1 else 'ies'} x T={p.T}, "
                f"Hq={p.Hq}, L_loc={p.L_loc}, k={p.k}")
    res = {
        "metric": "routing-key (K_r) scan GB/s over the whole route+attn step",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if p.bf16 else "f32",
        "data": "synthetic (seeded counter-based generator; planted needles)",
        "config": {"workload": workload,
                   "global_batch": p.B, "seq_len": p.T, "parallelism": "single GPU",
                   "kv_tier": tier, "gather": args.gather if tier == "host" else
                   f"hbm-{args.hbm_assembly if args.rounds == 1 else 'index'}", "rounds": args.rounds},
        "route_attn_us_per_query": round(ms_per_step * 1e3 / p.B, 1),
        "routing_GBps": round(routing_gbps, 1),
        "routing_frac_of_8TBps": round(routing_gbps / 8000, 4),
        "stage_ms_per_step": (({"route_score": round(stage[0], 4), "topk_and_context_index": round(stage[1], 4),
                                "attention": round(stage[3], 4)} if runner.indexed else
                               {"route_score": round(stage[0], 4), "topk": round(stage[1], 4),
                                "gather": round(stage[2], 4), "attention": round(stage[3], 4)}) if args.rounds == 1 else
                              {"rounds_route_topk_append": round(stage[0], 4), "attention": round(stage[3], 4)}),
        "attention_GBps": round(attn_gbps, 1),
        "attention_frac_of_8TBps": round(attn_gbps / 8000, 4),
        "attention_bytes_per_layer": attn_bytes,
        "encode_GBps": round(encode_gbps, 1),
        "needle_recall_layer0": recall,
        "roofline": {"kernel": "msa_route_score (route_score_mfma_kernel + score fill)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(achieved / 8000.0, 4), "traffic": counted_traffic(p.name),
                     "avg_launch_ms": round(route_avg_ms, 4), "alg_bytes_per_launch": int(alg_bytes)},
    }

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(p, layers, args.cpu_sample_chunks)
    print(json.dumps(res), flush=True)


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


def cpu_baseline(p, layers, n_sample_chunks=None):
    """The float64 oracle's routing (score + top-k) timed on a bounded sample
    of the same workload: every routed layer's query scored against the
    routing keys of layer 0's first documents.  The sample's keys come from
    the seeded generator (its device copy, bit-identical to the host one) and
    are pooled and normalised by the oracle before the timed region."""
    import torch

    import oracle as O
    import synth
    from synth import device as SD
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
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
    log(f"cpu baseline: sample prepared in {t_prep:.1f} s, oracle routing {dt:.1f} s")
    return {"value": round(gb / dt, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"layer 0, first {n_docs} documents ({n} pooled chunks, "
                      f"{n * p.H * p.d * (2 if p.bf16 else 4) / 1e9:.2f} GB of routing keys) scored against each of the "
                      f"{layers} routed layers' {p.B} x {p.T}-token queries: routing score + top-k, float64"}


if __name__ == "__main__":
    main()
