"""Parity of the training-time path on the GPU against the oracle: routing
scores with their maximiser, the routing loss, the routing-score backward and
the pooling backward, on seeded inputs with ragged and empty documents,
partial chunks and several tiles."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.helpers import RTOL_SCORE, check_scores, dev, gen, host, ragged_lengths, to_dev, to_dev_i64

pytestmark = pytest.mark.gpu

import sparse_attention_long_msa_amd as M  # noqa: E402  (a missing library fails loudly)

ARG_BAND = 1e-4   # maximiser tie band on oracle candidate scores


def _index(lens, chunk):
    tok_off = synth.offsets(lens)
    chunk_off = O.chunk_offsets(tok_off, chunk)
    n_chunks = int(chunk_off[-1])
    co_d = to_dev_i64(chunk_off)
    return tok_off, chunk_off, n_chunks, co_d, M.msa_chunk_doc_map(co_d, n_chunks)


def _store(seed, n_chunks, H, d, bf16):
    kr = O.round_to_store(O.l2_normalize(gen(seed, 0, synth.T_KR, (n_chunks, H, d), bf16)), "bf16" if bf16 else "f32")
    return kr, to_dev(kr, bf16)


def check_argmax(q, kr, chunk_off, arg_c, arg_t, band=ARG_BAND):
    """The GPU's maximiser lies in the document and attains the oracle's best
    candidate within the band; it is the oracle's own (chunk, then token)
    choice whenever the best beats the runner-up by more than the band."""
    s = O.chunk_cosines(q, kr)                          # [B, T, N]
    B, T, _ = s.shape
    exact = 0
    for b in range(B):
        for i in range(len(chunk_off) - 1):
            lo, hi = int(chunk_off[i]), int(chunk_off[i + 1])
            c, t = int(arg_c[b, i]), int(arg_t[b, i])
            if lo == hi:
                assert (c, t) == (-1, -1)
                continue
            assert lo <= c < hi and 0 <= t < T, (b, i, c, t)
            block = s[b, :, lo:hi].T.ravel()            # chunk-major
            order = np.argsort(-block, kind="stable")
            best = block[order[0]]
            assert s[b, t, c] >= best - band, (b, i)
            if len(block) == 1 or best - block[order[1]] > band:
                assert (c - lo) * T + t == order[0], (b, i)
                exact += 1
    return exact


@pytest.mark.parametrize("bf16,T", [(True, 16), (True, 64), (True, 5), (False, 7)])
def test_route_argmax(bf16, T):
    H, d = 8, 128 if bf16 else 32
    B = 2
    lens = ragged_lengths(21, 300, 0, 600, n_empty=9)
    tok_off, chunk_off, n_chunks, co_d, cd = _index(lens, 64)
    kr, kr_d = _store(3, n_chunks, H, d, bf16)
    q = gen(4, 0, synth.T_QR, (B, T, H, d), bf16)
    score, ac, at = M.msa_route_argmax(to_dev(q, bf16), kr_d, cd, len(lens))
    ref = O.route_scores(q, kr, chunk_off)
    check_scores(host(score), ref, RTOL_SCORE["bf16" if bf16 else "f32"], 16)
    exact = check_argmax(q, kr, chunk_off, host(ac), host(at))
    assert exact > 0.9 * B * np.count_nonzero(lens)


def test_route_argmax_ties_take_the_smallest_chunk_then_token():
    """Exact ties (bit-identical candidates on both sides): a query token equal
    to a repeated chunk's key scores the maximum at every copy, and a repeated
    token ties with itself; the maximiser is the smallest chunk, then the
    smallest token."""
    H, d, T = 8, 128, 16
    lens = np.array([64 * 5, 64 * 3, 0, 64 * 7])
    tok_off, chunk_off, n_chunks, co_d, cd = _index(lens, 64)
    kr, _ = _store(5, n_chunks, H, d, True)
    kr[3] = kr[1]                      # document 0: chunks 1 and 3 equal
    kr[8] = kr[10]                     # document 3 (chunks 8..14): chunks 8, 9, 10 equal
    kr[9] = kr[10]
    q = gen(6, 0, synth.T_QR, (1, T, H, d), True)
    q[0, 2] = q[0, 9] = kr[1]          # tokens 2 and 9 point at chunk 1
    q[0, 5] = kr[10]                   # token 5 points at chunks 8..10
    score, ac, at = M.msa_route_argmax(to_dev(q, True), to_dev(kr, True), cd, len(lens))
    _, rac, rat = O.route_argmax(q, kr, chunk_off)
    got = list(zip(host(ac)[0].tolist(), host(at)[0].tolist()))
    assert got[0] == (1, 2) and (rac[0, 0], rat[0, 0]) == (1, 2)
    assert got[2] == (-1, -1)
    assert got[3] == (8, 5) and (rac[0, 3], rat[0, 3]) == (8, 5)


@pytest.mark.parametrize("B,D,P", [(1, 195, 1), (3, 5000, 4), (2, 40000, 8)])
def test_route_loss(B, D, P):
    r = np.random.default_rng(B * 7 + P)
    s = r.uniform(-0.3, 0.9, (B, D)).astype(np.float32)
    s[:, r.choice(D, size=D // 50 + 1, replace=False)] = -np.inf       # empty documents
    pos = np.full((B, P + 2), -1, dtype=np.int32)
    for b in range(B):
        fin = np.nonzero(np.isfinite(s[b]))[0]
        pos[b, :P] = r.choice(fin, size=P, replace=False)
        pos[b, P] = pos[b, 0]                                         # a repeated id
        pos[b, P + 1] = D + 5                                         # outside [0, D): ignored
    for tau in (0.05, 1.0):
        loss, grad = M.msa_route_loss(torch.from_numpy(s).to(dev()), torch.from_numpy(pos).to(dev()), tau)
        rl, rg = O.route_loss(s.astype(np.float64), pos, tau)
        np.testing.assert_allclose(host(loss), rl, rtol=2e-5, atol=2e-5)
        g = host(grad)
        scale = np.abs(rg).max(axis=1, keepdims=True)
        assert np.all(np.abs(g - rg) <= 2e-5 * scale + 1e-9)
        assert np.all(g[~np.isfinite(s)] == 0)


@pytest.mark.parametrize("bf16", [True, False])
def test_route_score_backward(bf16):
    H, d, T, B = 8, 128 if bf16 else 32, 16, 2
    lens = ragged_lengths(31, 400, 0, 500, n_empty=7)
    tok_off, chunk_off, n_chunks, co_d, cd = _index(lens, 64)
    kr, kr_d = _store(7, n_chunks, H, d, bf16)
    q = gen(8, 0, synth.T_QR, (B, T, H, d), bf16)
    q[0, 3, 2] = 0.0                                                   # a zero head: the 1/eps branch
    q_d = to_dev(q, bf16)
    _, ac, at = M.msa_route_argmax(q_d, kr_d, cd, len(lens))
    g = np.random.default_rng(9).normal(size=(B, len(lens))).astype(np.float32)
    dkr = torch.zeros((n_chunks, H, d), dtype=torch.float32, device=dev())
    dq, dkr = M.msa_route_score_backward(q_d, kr_d, ac, at, torch.from_numpy(g).to(dev()), dkr)
    rdq, rdk = O.route_score_backward(q, kr, host(ac), host(at), g.astype(np.float64))
    for got, ref in ((host(dq), rdq), (host(dkr), rdk)):
        finite = ref[np.abs(ref) < 1e6]
        scale = np.abs(finite).max()
        big = np.abs(ref) >= 1e6                                       # the 1/eps branch: relative
        assert np.all(np.abs(got[~big] - ref[~big]) <= 1e-5 * scale)
        if big.any():
            np.testing.assert_allclose(got[big], ref[big], rtol=1e-5)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("chunk", [64, 5, 1])
@pytest.mark.parametrize("normalized", [False, True])
@pytest.mark.parametrize("H,d", [(4, 64), (8, 128), (3, 40)])     # whole-row kernel, and the per-head one (3 x 40)
def test_pool_backward(bf16, chunk, normalized, H, d):
    lens = ragged_lengths(41, 60, 0, 300, n_empty=4)
    lens[0] = 130
    tok_off, chunk_off, n_chunks, co_d, cd = _index(lens, chunk)
    n_tok = int(lens.sum())
    x = gen(12, 0, synth.T_KR, (n_tok, H, d), bf16)
    dy = np.random.default_rng(13).normal(size=(n_chunks, H, d)).astype(np.float32)
    dx = M.msa_pool_backward(torch.from_numpy(dy).to(dev()), to_dev_i64(tok_off), co_d, cd, n_tok, chunk,
                             x=to_dev(x, bf16) if normalized else None,
                             dtype=M.MSA_BF16 if bf16 else M.MSA_F32)
    ref = O.pool_backward(dy.astype(np.float64), tok_off, chunk, x=x if normalized else None)
    scale = np.abs(ref).max()
    assert np.abs(host(dx) - ref).max() <= 2e-5 * scale


def test_routing_training_chain():
    """scores with maximiser -> loss -> routing backward -> token-level
    routing-key gradient, against the oracle's chain on the GPU's maximisers."""
    H, d, T, B, chunk = 8, 128, 32, 2, 64
    lens = ragged_lengths(51, 120, 1, 700)
    tok_off, chunk_off, n_chunks, co_d, cd = _index(lens, chunk)
    n_tok = int(lens.sum())
    x = gen(14, 0, synth.T_KR, (n_tok, H, d), True)
    kr_d = M.msa_pool_encode(to_dev(x, True), to_dev_i64(tok_off), co_d, cd, chunk, True)
    kr = host(kr_d)
    q = gen(15, 0, synth.T_QR, (B, T, H, d), True)
    q_d = to_dev(q, True)
    score, ac, at = M.msa_route_argmax(q_d, kr_d, cd, len(lens))
    pos = np.array([[3, 17, -1], [50, -1, -1]], dtype=np.int32)
    loss, grad = M.msa_route_loss(score, torch.from_numpy(pos).to(dev()), 0.1)
    dkr = torch.zeros((n_chunks, H, d), dtype=torch.float32, device=dev())
    dq, dkr = M.msa_route_score_backward(q_d, kr_d, ac, at, grad, dkr)
    dx = M.msa_pool_backward(dkr, to_dev_i64(tok_off), co_d, cd, n_tok, chunk, x=to_dev(x, True))
    rs = O.route_scores(q, kr, chunk_off)
    rl, rg = O.route_loss(rs, pos, 0.1)
    np.testing.assert_allclose(host(loss), rl, rtol=1e-4)
    rdq, rdk = O.route_score_backward(q, kr, host(ac), host(at), rg)
    rdx = O.pool_backward(rdk, tok_off, chunk, x=x)
    for got, ref in ((host(dq), rdq), (host(dx), rdx)):
        assert np.abs(got - ref).max() <= 1e-3 * np.abs(ref).max()


# ---------------------------------------------------------------- attention backward

def _bwd_case(seed, B, T, Hq, Hkv, d, L_loc, n_docs, k, bf16, shared_ids=False):
    r = np.random.default_rng(seed)
    lens = r.integers(1, 9, size=n_docs) * 64 - r.integers(0, 40, size=n_docs)   # 1..8 chunks, partial last
    chunk_off = O.chunk_offsets(synth.offsets(lens), 64)
    n_chunks = int(chunk_off[-1])
    kb = gen(seed, 0, synth.T_K, (n_chunks, Hkv, d), bf16, scale_pow2=-3)
    vb = gen(seed, 0, synth.T_V, (n_chunks, Hkv, d), bf16, scale_pow2=-3)
    q = gen(seed, 0, synth.T_Q, (B, T, Hq, d), bf16)
    kl = gen(seed, 0, synth.T_KLOC, (B, L_loc, Hkv, d), bf16)
    vl = gen(seed, 0, synth.T_VLOC, (B, L_loc, Hkv, d), bf16)
    ids = np.stack([r.choice(n_docs, size=k, replace=False) for _ in range(B)]).astype(np.int32)
    if shared_ids:
        ids[1:] = ids[0]                       # every query reads the same rows: the row sums meet
    dout = r.normal(size=(B, T, Hq, d)).astype(np.float32)
    return chunk_off, n_chunks, kb, vb, q, kl, vl, ids, dout


@pytest.mark.parametrize("bf16,B,T,Hq,Hkv,d,L_loc,k,shared", [
    (True, 1, 16, 32, 8, 128, 64, 4, False),
    (True, 2, 5, 32, 8, 128, 40, 3, True),       # 20 rows per head: a ragged row tile; shared rows
    (True, 1, 64, 32, 8, 128, 300, 8, False),
    (True, 3, 1, 16, 8, 128, 100, 5, True),      # decode-shaped rows, G = 2
    (False, 2, 3, 8, 2, 32, 20, 3, True),        # the float32 vector path
    (True, 1, 4, 6, 2, 64, 30, 2, False),        # bf16 vector path (d = 64, G = 3)
])
def test_sparse_attn_backward(bf16, B, T, Hq, Hkv, d, L_loc, k, shared):
    qpo = k
    chunk_off, n_chunks, kb, vb, q, kl, vl, ids, dout = _bwd_case(70 + T + B, B, T, Hq, Hkv, d, L_loc, 40, k, bf16,
                                                                  shared)
    max_doc = int(np.diff(chunk_off).max())
    max_ctx = k * max_doc
    co_d = to_dev_i64(chunk_off)
    row, pos, ln = M.msa_context_index(torch.from_numpy(ids).to(dev()), co_d, n_chunks, max_doc, max_ctx)
    dkb = torch.zeros((n_chunks, Hkv, d), dtype=torch.float32, device=dev())
    dvb = torch.zeros_like(dkb)
    dq, dkl, dvl, dkb, dvb = M.msa_sparse_attn_backward(
        to_dev(q, bf16), to_dev(kb, bf16), to_dev(vb, bf16), row, pos, ln, to_dev(kl, bf16), to_dev(vl, bf16), qpo,
        torch.from_numpy(dout).to(dev()), dkb, dvb)
    ctx = [O.gather(ids[b], chunk_off, kb, vb) for b in range(B)]
    rdq, cg, rdkl, rdvl = O.sparse_attention_backward(q, ctx, kl, vl, qpo, 1e6, dout.astype(np.float64))
    rdkb, rdvb = O.gather_backward(ids, chunk_off, cg, n_chunks)
    # bf16 operands (P, dS, dout, the rotated q and k) carry 2^-9 relative rounding each
    tol = 1.5e-2 if bf16 else 1e-4
    for name, got, ref in (("dq", dq, rdq), ("dk_loc", dkl, rdkl), ("dv_loc", dvl, rdvl), ("dk_bar", dkb, rdkb),
                           ("dv_bar", dvb, rdvb)):
        g = host(got)
        err = np.abs(g - ref).max() / np.abs(ref).max()
        print(f"{name}: normwise error {err:.3g}")
        assert err <= tol, f"{name}: normwise error {err:.3g} > {tol}"



def test_training_chain_at_the_bench_workload():
    """One routed layer of the training benchmark's launch (train64k: 1,024
    chunks, 1,024 trained tokens, 32 query heads, 1,024-token window, k = 16),
    inputs from the same seeded device generator, every output against the
    oracle on the GPU's own selection and maximisers."""
    from synth import configs
    from synth import device as SD
    p = configs.TRAIN_PRESETS["train64k"]()
    H, d, N, D, T, Hq, L, k = p.H, p.d, p.n_chunks, p.n_docs, p.T, p.Hq, p.L_loc, p.k
    bf = torch.bfloat16
    tok_off, chunk_off = p.tok_off, p.chunk_off
    n_tok = int(tok_off[-1])
    to_d, co_d = to_dev_i64(tok_off), to_dev_i64(chunk_off)
    cd = M.msa_chunk_doc_map(co_d, N)
    fill = lambda shape, seed, t, dt=bf, sp=0: SD.fill(torch.empty(shape, dtype=dt, device=dev()), seed, 0, t,
                                                       scale_pow2=sp)
    xr = fill((n_tok, H, d), p.seed, synth.T_KR)
    kr = M.msa_pool_encode(xr, to_d, co_d, cd, p.chunk, True)
    kbar = M.msa_pool_encode(fill((n_tok, H, d), p.seed, synth.T_K), to_d, co_d, cd, p.chunk, False)
    vbar = M.msa_pool_encode(fill((n_tok, H, d), p.seed, synth.T_V), to_d, co_d, cd, p.chunk, False)
    qr = fill((1, T, H, d), p.qseed, synth.T_QR)
    q = fill((1, T, Hq, d), p.qseed, synth.T_Q)
    kl = fill((1, L, H, d), p.qseed, synth.T_KLOC)
    vl = fill((1, L, H, d), p.qseed, synth.T_VLOC)
    dout = fill((1, T, Hq, d), p.qseed, synth.T_DOUT, torch.float32)
    pos = np.array([synth.needle_docs(p.seed, D, p.n_needles)], dtype=np.int32)
    score, ac, at = M.msa_route_argmax(qr, kr, cd, D)
    loss, grad = M.msa_route_loss(score, torch.from_numpy(pos).to(dev()), 0.1)
    dkr = torch.zeros((N, H, d), dtype=torch.float32, device=dev())
    dqr, dkr = M.msa_route_score_backward(qr, kr, ac, at, grad, dkr)
    ids, _ = M.msa_topk(score, k)
    row, cpos, clen = M.msa_context_index(ids, co_d, N, p.max_doc_chunks, k * p.max_doc_chunks)
    dkb = torch.zeros((N, H, d), dtype=torch.float32, device=dev())
    dvb = torch.zeros_like(dkb)
    dq, dkl, dvl, dkb, dvb = M.msa_sparse_attn_backward(q, kbar, vbar, row, cpos, clen, kl, vl, p.qpo, dout, dkb,
                                                        dvb)
    dxr = M.msa_pool_backward(dkr, to_d, co_d, cd, n_tok, p.chunk, x=xr)
    # routing side
    krh, qrh = host(kr), host(qr)
    rs = O.route_scores(qrh, krh, chunk_off)
    check_scores(host(score), rs, RTOL_SCORE["bf16"], k)
    check_argmax(qrh, krh, chunk_off, host(ac), host(at))
    rl, rg = O.route_loss(host(score), pos, 0.1)     # the loss on the GPU's own scores
    np.testing.assert_allclose(host(loss), rl, rtol=1e-4)
    rdq, rdk = O.route_score_backward(qrh, krh, host(ac), host(at), rg)
    rdx = O.pool_backward(rdk, tok_off, p.chunk, x=host(xr))
    for name, got, ref, tol in (("dq_r", dqr, rdq, 1e-4), ("dx_r", dxr, rdx, 1e-4)):
        err = np.abs(host(got) - ref).max() / np.abs(ref).max()
        assert err <= tol, f"{name}: normwise error {err:.3g}"
    # attention side, on the GPU's selection; KV heads are independent, so the
    # oracle runs one of them (its 4 query heads) at full length
    g, G = 3, Hq // H
    hs = slice(g * G, (g + 1) * G)
    ids_h = host(ids)
    kbh, vbh = host(kbar)[:, g:g + 1], host(vbar)[:, g:g + 1]
    ctx = [O.gather(ids_h[0], chunk_off, kbh, vbh)]
    rdq2, cg, rdkl, rdvl = O.sparse_attention_backward(host(q)[:, :, hs], ctx, host(kl)[:, :, g:g + 1],
                                                       host(vl)[:, :, g:g + 1], p.qpo, p.rope_base,
                                                       host(dout)[:, :, hs], sm_scale=1.0 / np.sqrt(d))
    rdkb, rdvb = O.gather_backward(ids_h, chunk_off, cg, N)
    for name, got, ref in (("dq", host(dq)[:, :, hs], rdq2), ("dk_loc", host(dkl)[:, :, g:g + 1], rdkl),
                           ("dv_loc", host(dvl)[:, :, g:g + 1], rdvl), ("dk_bar", host(dkb)[:, g:g + 1], rdkb),
                           ("dv_bar", host(dvb)[:, g:g + 1], rdvb)):
        err = np.abs(got - ref).max() / np.abs(ref).max()
        print(f"{name}: normwise error {err:.3g}")
        assert err <= 1.5e-2, f"{name}: normwise error {err:.3g}"
