"""The routed layers of one step captured into a HIP graph (StepGraph) and
replayed: every replay gives the eager path's outputs bit for bit (scores,
ids, context and attention), with eager work on the same buffers between
replays; and the eager outputs match the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.helpers import ATOL_ATTN, RTOL_SCORE, check_ids, check_scores, dev, gen, host, ragged_lengths, tile_np, \
    to_dev, to_dev_i64

pytestmark = pytest.mark.gpu

import sparse_attention_long_msa_amd as M  # noqa: E402  (a missing library fails loudly)


@pytest.mark.parametrize("B,T,L_loc,k,overlap,indexed", [(1, 64, 512, 8, False, True), (8, 1, 1024, 4, False, True),
                                                           (1, 64, 512, 8, True, True), (8, 1, 1024, 4, True, True),
                                                           (1, 64, 512, 8, True, False)])
def test_step_graph_replays_equal_the_eager_step(B, T, L_loc, k, overlap, indexed):
    """overlap: the attention's local part on a side stream (two streams in
    the captured graph); indexed: the context read in place, else gathered."""
    H, d, Hq, layers = 8, 128, 32, 3
    lens = ragged_lengths(90 + B, 700, 0, 900, n_empty=9)
    tok_off = synth.offsets(lens)
    chunk_off = O.chunk_offsets(tok_off, 64)
    n_chunks, D = int(chunk_off[-1]), len(lens)
    mdc = int(np.diff(chunk_off).max())
    co_d = to_dev_i64(chunk_off)
    cd = M.msa_chunk_doc_map(co_d, n_chunks)
    L = []
    for l in range(layers):
        store = O.round_to_bf16(O.l2_normalize(gen(71, l, synth.T_KR, (n_chunks, H, d), True).astype(np.float64)))
        x = dict(store=store,
                 kb=gen(71, l, synth.T_K, (n_chunks, H, d), True, scale_pow2=-3),
                 vb=gen(71, l, synth.T_V, (n_chunks, H, d), True, scale_pow2=-3),
                 qr=gen(72, l, synth.T_QR, (B, T, H, d), True), q=gen(72, l, synth.T_Q, (B, T, Hq, d), True),
                 kl=gen(72, l, synth.T_KLOC, (B, L_loc, H, d), True),
                 vl=gen(72, l, synth.T_VLOC, (B, L_loc, H, d), True))
        x["dev"] = [to_dev(tile_np(store), True)] + [to_dev(x[n], True) for n in ("kb", "vb", "qr", "q", "kl", "vl")]
        x["run"] = M.LayerRunner(batch=B, tokens=T, q_heads=Hq, kv_heads=H, head_dim=d, n_docs=D, n_chunks=n_chunks,
                                 k=k, max_doc_chunks=mdc, local_len=L_loc, dtype=torch.bfloat16, device=dev(),
                                 kr_layout=M.MSA_LAYOUT_TILED, indexed=indexed, overlap_local=overlap)
        L.append(x)

    def step():
        for x in L:
            kr, kb, vb, qr, q, kl, vl = x["dev"]
            x["run"].run(qr, kr, cd, co_d, kb, vb, q, kl, vl)

    names = ("doc_score", "ids", "vals", "ctx_row" if indexed else "k_ctx", "ctx_pos", "ctx_len", "out")
    step()
    torch.cuda.synchronize()
    eager = [{n: getattr(x["run"], n).clone() for n in names} for x in L]
    g = M.StepGraph(step)
    for rep in range(3):
        for x in L:                                   # eager work on the same buffers between replays
            for n in names:
                getattr(x["run"], n).fill_(-3 if getattr(x["run"], n).dtype == torch.int32 else float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, x in enumerate(L):
            r = x["run"]
            for n in ("doc_score", "ids", "vals", "ctx_len", "out"):
                assert torch.equal(getattr(r, n), eager[l][n]), f"replay {rep}, layer {l}: {n}"
            for b in range(B):                        # the context entries (rows past ctx_len are not written)
                n_b = int(eager[l]["ctx_len"][b])
                for n in (names[3], "ctx_pos"):
                    assert torch.equal(getattr(r, n)[b, :n_b], eager[l][n][b, :n_b]), f"replay {rep}, layer {l}: {n}"
    # the eager outputs against the oracle
    for l, x in enumerate(L):
        ref = O.layer(x["qr"], x["store"], chunk_off, x["kb"], x["vb"], k, x["q"], x["kl"], x["vl"],
                      ids_override=eager[l]["ids"].cpu().numpy())
        check_scores(host(eager[l]["doc_score"]), ref["doc_score"], RTOL_SCORE["bf16"], k)
        check_ids(eager[l]["ids"].cpu().numpy(), ref["doc_score"], k)
        assert np.abs(host(eager[l]["out"]) - ref["out"]).max() <= ATOL_ATTN["bf16"]


@pytest.mark.parametrize("name,overlap", [("cfg2", True), ("cfg5", True), ("cfg4", True), ("cfg4", False)])
def test_step_graph_full_size(name, overlap):
    """The bench's graph-replayed step at the full presets (two routed layers of
    the 1M-token, batched-decode and 100M-token workloads, context read in
    place, the attention as its two calls with the local part on a side stream, and the
    100M-token step with one attention call): every replay equals the eager
    step bit for bit.  The eager step is checked against the oracle by the
    preset parity tests."""
    from synth import configs
    from tests.preset_run import GpuLayer, HostLayer
    p = getattr(configs, name)()
    layers = [GpuLayer(p, l, HostLayer(p, l), indexed=True, overlap_local=overlap) for l in (0, 1)]

    def step():
        for gl in layers:
            gl.runner.run(gl.qr, gl.store[synth.T_KR], gl.cd, gl.co_d, gl.kb, gl.vb, gl.q, gl.kl, gl.vl)

    names = ("doc_score", "ids", "vals", "ctx_row", "ctx_pos", "ctx_len", "out")
    step()
    torch.cuda.synchronize()
    eager = [{n: getattr(gl.runner, n).clone() for n in names} for gl in layers]
    g = M.StepGraph(step)
    for rep in range(2):
        for gl in layers:
            for n in names:
                t = getattr(gl.runner, n)
                t.fill_(-3 if t.dtype == torch.int32 else float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, gl in enumerate(layers):
            r = gl.runner
            for n in ("doc_score", "ids", "vals", "ctx_len", "out"):
                assert torch.equal(getattr(r, n), eager[l][n]), f"{name} replay {rep}, layer {l}: {n}"
            for b in range(p.B):
                n_b = int(eager[l]["ctx_len"][b])
                for n in ("ctx_row", "ctx_pos"):
                    assert torch.equal(getattr(r, n)[b, :n_b], eager[l][n][b, :n_b]), f"{name} replay {rep}: {n}"
    del g, layers
    torch.cuda.empty_cache()


@pytest.mark.parametrize("indexed", [True, False])
def test_fill_in_topk_step_equals_the_filling_step(indexed):
    """LayerRunner(fill_in_topk=True): one runner over three layers, as the
    benchmark drives it, the score fill moved into the previous layer's top-k.
    Eager steps and graph replays give the selection, context and attention
    of a runner that fills before every routing call, bit for bit."""
    B, T, L_loc, k, H, d, Hq, layers = 1, 64, 512, 8, 8, 128, 32, 3
    lens = ragged_lengths(95, 700, 0, 900, n_empty=9)
    tok_off = synth.offsets(lens)
    chunk_off = O.chunk_offsets(tok_off, 64)
    n_chunks, D = int(chunk_off[-1]), len(lens)
    mdc = int(np.diff(chunk_off).max())
    co_d = to_dev_i64(chunk_off)
    cd = M.msa_chunk_doc_map(co_d, n_chunks)
    L = []
    for l in range(layers):
        store = O.round_to_bf16(O.l2_normalize(gen(75, l, synth.T_KR, (n_chunks, H, d), True).astype(np.float64)))
        L.append([to_dev(tile_np(store), True)] +
                 [to_dev(gen(75, l, t, (n_chunks, H, d), True, scale_pow2=-3), True) for t in (synth.T_K, synth.T_V)] +
                 [to_dev(gen(76, l, t, shp, True), True) for t, shp in ((synth.T_QR, (B, T, H, d)),
                                                                        (synth.T_Q, (B, T, Hq, d)),
                                                                        (synth.T_KLOC, (B, L_loc, H, d)),
                                                                        (synth.T_VLOC, (B, L_loc, H, d)))])

    def runner(fused):
        return M.LayerRunner(batch=B, tokens=T, q_heads=Hq, kv_heads=H, head_dim=d, n_docs=D, n_chunks=n_chunks,
                             k=k, max_doc_chunks=mdc, local_len=L_loc, dtype=torch.bfloat16, device=dev(),
                             kr_layout=M.MSA_LAYOUT_TILED, indexed=indexed, fill_in_topk=fused)

    names = ("ids", "vals", "ctx_len", "out")
    plain, fused = runner(False), runner(True)

    def step(r, keep=None):
        for l, (kr, kb, vb, qr, q, kl, vl) in enumerate(L):
            r.run(qr, kr, cd, co_d, kb, vb, q, kl, vl)
            if keep is not None:
                keep.append({n: getattr(r, n).clone() for n in names})

    want = []
    step(plain, want)
    for rep in range(2):                                  # eager steps
        got = []
        step(fused, got)
        torch.cuda.synchronize()
        for l in range(layers):
            for n in names:
                assert torch.equal(got[l][n], want[l][n]), f"eager step {rep}, layer {l}: {n}"
        assert bool((fused.doc_score == float("-inf")).all())
    g = M.StepGraph(lambda: step(fused))
    for rep in range(3):                                  # replays: the last layer's outputs
        fused.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(fused, n), want[-1][n]), f"replay {rep}: {n}"
        step(fused)                                       # eager work on the same runner between replays
        torch.cuda.synchronize()
    # a route() that does not follow a select fills the buffer itself
    kr, kb, vb, qr, q, kl, vl = L[0]
    fused.route(qr, kr, cd)
    fused.route(qr, kr, cd)
    ref = plain.route(qr, kr, cd)
    torch.cuda.synchronize()
    assert torch.equal(fused.doc_score.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("host_src", [True, False])
def test_run_layers_equals_run(host_src):
    """LayerRunner.run_layers (each layer's context fetched in the next
    layer's routing scan, msa_route_score_fetch) gives every layer the
    selection, context and attention output of run() layer by layer, bit for
    bit; eager and replayed as a HIP graph, from pinned host or device memory."""
    B, T, L_loc, k, H, d, Hq, layers = 1, 64, 512, 8, 8, 128, 32, 4
    lens = ragged_lengths(97, 700, 0, 900, n_empty=9)
    tok_off = synth.offsets(lens)
    chunk_off = O.chunk_offsets(tok_off, 64)
    n_chunks, D = int(chunk_off[-1]), len(lens)
    mdc = int(np.diff(chunk_off).max())
    co_d = to_dev_i64(chunk_off)
    cd = M.msa_chunk_doc_map(co_d, n_chunks)
    L = []
    for l in range(layers):
        store = O.round_to_bf16(O.l2_normalize(gen(77, l, synth.T_KR, (n_chunks, H, d), True).astype(np.float64)))
        kb, vb = (to_dev(gen(77, l, t, (n_chunks, H, d), True, scale_pow2=-3), True) for t in (synth.T_K, synth.T_V))
        if host_src:
            kb, vb = kb.cpu().pin_memory(), vb.cpu().pin_memory()
        qr, q, kl, vl = (to_dev(gen(78, l, t, shp, True), True) for t, shp in ((synth.T_QR, (B, T, H, d)),
                                                                             (synth.T_Q, (B, T, Hq, d)),
                                                                             (synth.T_KLOC, (B, L_loc, H, d)),
                                                                             (synth.T_VLOC, (B, L_loc, H, d))))
        L.append((qr, to_dev(tile_np(store), True), cd, co_d, kb, vb, q, kl, vl))
    src = M.MSA_SRC_HOST_MAPPED if host_src else M.MSA_SRC_DEVICE

    def runner(fill):
        return M.LayerRunner(batch=B, tokens=T, q_heads=Hq, kv_heads=H, head_dim=d, n_docs=D, n_chunks=n_chunks,
                             k=k, max_doc_chunks=mdc, local_len=L_loc, dtype=torch.bfloat16, device=dev(),
                             kr_layout=M.MSA_LAYOUT_TILED, src_mode=src, fill_in_topk=fill)

    names = ("ids", "vals", "ctx_len", "out")
    plain = runner(False)
    want = []
    for x in L:
        plain.run(*x)
        want.append({n: getattr(plain, n).clone() for n in names})
    piped = runner(True)
    got = []
    piped.run_layers(L, after_layer=lambda l: got.append({n: getattr(piped, n).clone() for n in names}))
    torch.cuda.synchronize()
    for l in range(layers):
        for n in names:
            assert torch.equal(got[l][n], want[l][n]), f"layer {l}: {n}"
    g = M.StepGraph(lambda: piped.run_layers(L))
    for rep in range(3):
        piped.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(piped, n), want[-1][n]), f"replay {rep}: {n}"


def test_indexed_runner_over_a_host_store():
    """LayerRunner(indexed=True, src_mode=MSA_SRC_HOST_MAPPED): the top-k
    writes the selected rows' index and the attention reads them from pinned
    host memory; every layer equals the runner over the same stores in device
    memory bit for bit, eager and graph-replayed."""
    B, T, L_loc, k, H, d, Hq, layers = 1, 64, 4096, 16, 8, 128, 32, 3
    lens = ragged_lengths(99, 900, 0, 900, n_empty=9)
    tok_off = synth.offsets(lens)
    chunk_off = O.chunk_offsets(tok_off, 64)
    n_chunks, D = int(chunk_off[-1]), len(lens)
    mdc = int(np.diff(chunk_off).max())
    co_d = to_dev_i64(chunk_off)
    cd = M.msa_chunk_doc_map(co_d, n_chunks)
    dev_layers, host_layers = [], []
    for l in range(layers):
        store = O.round_to_bf16(O.l2_normalize(gen(79, l, synth.T_KR, (n_chunks, H, d), True).astype(np.float64)))
        kb, vb = (to_dev(gen(79, l, t, (n_chunks, H, d), True, scale_pow2=-3), True) for t in (synth.T_K, synth.T_V))
        qr, q, kl, vl = (to_dev(gen(80, l, t, shp, True), True) for t, shp in ((synth.T_QR, (B, T, H, d)),
                                                                             (synth.T_Q, (B, T, Hq, d)),
                                                                             (synth.T_KLOC, (B, L_loc, H, d)),
                                                                             (synth.T_VLOC, (B, L_loc, H, d))))
        kr = to_dev(tile_np(store), True)
        dev_layers.append((qr, kr, cd, co_d, kb, vb, q, kl, vl))
        host_layers.append((qr, kr, cd, co_d, kb.cpu().pin_memory(), vb.cpu().pin_memory(), q, kl, vl))

    def runner(src):
        return M.LayerRunner(batch=B, tokens=T, q_heads=Hq, kv_heads=H, head_dim=d, n_docs=D, n_chunks=n_chunks,
                             k=k, max_doc_chunks=mdc, local_len=L_loc, dtype=torch.bfloat16, device=dev(),
                             kr_layout=M.MSA_LAYOUT_TILED, indexed=True, src_mode=src, fill_in_topk=True)

    names = ("ids", "vals", "ctx_len", "out")
    on_dev, on_host = runner(M.MSA_SRC_DEVICE), runner(M.MSA_SRC_HOST_MAPPED)
    want = []
    for x in dev_layers:
        on_dev.run(*x)
        want.append({n: getattr(on_dev, n).clone() for n in names})
    for l, x in enumerate(host_layers):
        on_host.run(*x)
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(on_host, n), want[l][n]), f"layer {l}: {n}"

    def step():
        for x in host_layers:
            on_host.run(*x)
    g = M.StepGraph(step)
    for rep in range(2):
        on_host.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(on_host, n), want[-1][n]), f"replay {rep}: {n}"
