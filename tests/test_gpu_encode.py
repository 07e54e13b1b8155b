"""Parity of msa_encode (Stage 1 from hidden states) against the oracle's
per-token projection and pool, on ragged documents with empty documents and
partial chunks, both store layouts, the MFMA path and the vector path."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.helpers import gen, host, ragged_lengths, to_dev, to_dev_i64, untile_np

pytestmark = pytest.mark.gpu

import sparse_attention_long_msa_amd as M  # noqa: E402  (a missing library fails loudly)


def _case(seed, n_docs, hidden, H, d, chunk, bf16):
    lens = ragged_lengths(seed, n_docs, 0, 300, n_empty=3)
    lens[0] = 2 * chunk + 5
    tok_off = synth.offsets(lens)
    chunk_off = O.chunk_offsets(tok_off, chunk)
    n_chunks = int(chunk_off[-1])
    co_d = to_dev_i64(chunk_off)
    cd = M.msa_chunk_doc_map(co_d, n_chunks)
    x = gen(seed, 0, synth.T_K, (int(lens.sum()), hidden), bf16)
    w = gen(seed, 0, synth.T_V, (3 * H * d, hidden), bf16, scale_pow2=-4)
    return tok_off, chunk_off, n_chunks, co_d, cd, x, w


def _check(got, ref, mag, min_exact):
    """At most one bf16 ulp of the oracle plus the projection's error: the
    pooled row is split into two bf16 parts (2^-17 relative), so 2^-16 of the
    magnitude sum |pooled x| . |w| of the element (outputs of cancelling sums
    are small next to that sum)."""
    ulp = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)
    err = np.abs(got - ref)
    bound = ulp + 2.0 ** -16 * mag
    assert np.all(err <= bound), (err / bound).max()
    assert np.mean(got == ref) >= min_exact, np.mean(got == ref)


def _magnitudes(x, w, tok_off, chunk, H, d):
    xa = O.pool(np.abs(x)[:, None, :], tok_off, chunk)[:, 0, :]
    mag = (xa @ np.abs(w).T).reshape(-1, 3, H, d)
    raw = (O.pool(x[:, None, :], tok_off, chunk)[:, 0, :] @ w[2 * H * d:].T).reshape(-1, H, d)
    norm = np.maximum(np.sqrt((raw * raw).sum(-1, keepdims=True)), 1e-8)
    return mag[:, 0], mag[:, 1], mag[:, 2] / norm


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("chunk", [64, 7])
@pytest.mark.parametrize("hidden", [320, 288])   # whole 64-wide k-stages, and a trailing 32-wide one
def test_encode_mfma(layout, chunk, hidden):
    H, d = 2, 128
    tok_off, chunk_off, n_chunks, co_d, cd, x, w = _case(31, 40, hidden, H, d, chunk, True)
    kb, vb, kr = M.msa_encode(to_dev(x, True), to_dev(w, True), to_dev_i64(tok_off), co_d, cd, chunk, H, d,
                              kr_layout=layout)
    rk, rv, rr = O.encode(x, w, tok_off, chunk, H, d, "bf16")
    got_r = host(kr)
    if layout == 1:
        assert np.all(untile_np(got_r, got_r.shape[0])[n_chunks:] == 0)
        got_r = untile_np(got_r, n_chunks)
    mk, mv, mr = _magnitudes(x, w, tok_off, chunk, H, d)
    _check(host(kb), rk, mk, 0.95)
    _check(host(vb), rv, mv, 0.95)
    _check(got_r, rr, mr, 0.95)


def test_encode_vector_path_float32():
    H, d, hidden = 2, 32, 48
    tok_off, chunk_off, n_chunks, co_d, cd, x, w = _case(32, 25, hidden, H, d, 5, False)
    kb, vb, kr = M.msa_encode(to_dev(x, False), to_dev(w, False), to_dev_i64(tok_off), co_d, cd, 5, H, d)
    rk, rv, rr = O.encode(x, w, tok_off, 5, H, d, "f32")
    for got, ref in ((kb, rk), (vb, rv), (kr, rr)):
        np.testing.assert_allclose(host(got), ref, rtol=2e-5, atol=2e-6 * np.abs(ref).max())


def test_encode_bench_workload_sampled_documents():
    """The benchmark's launch: the 1M-token memory (2,048 documents x 512
    tokens), hidden 2,560, tiled routing keys.  Documents are independent, so
    the oracle encodes a sample of them on their own tokens."""
    from synth import configs
    from synth import device as SD
    p = configs.PRESETS["cfg2"]()
    hidden, H, d = 2560, p.H, p.d
    tok_off, chunk_off = p.tok_off, p.chunk_off
    N = p.n_chunks
    co_d = to_dev_i64(chunk_off)
    cd = M.msa_chunk_doc_map(co_d, N)
    x = SD.fill(torch.empty((int(tok_off[-1]), hidden), dtype=torch.bfloat16, device="cuda"), p.seed, 0, synth.T_K)
    w = SD.fill(torch.empty((3 * H * d, hidden), dtype=torch.bfloat16, device="cuda"), p.seed, 0, synth.T_V,
                scale_pow2=-6)
    kb, vb, kr = M.msa_encode(x, w, to_dev_i64(tok_off), co_d, cd, p.chunk, H, d, kr_layout=M.MSA_LAYOUT_TILED)
    kr_rows = untile_np(host(kr), N)
    wh = host(w)
    for doc in (0, 777, 2047):
        lo, hi = int(tok_off[doc]), int(tok_off[doc + 1])
        xd = host(x[lo:hi])
        sub = np.array([0, hi - lo])
        rk, rv, rr = O.encode(xd, wh, sub, p.chunk, H, d, "bf16")
        c0, c1 = int(chunk_off[doc]), int(chunk_off[doc + 1])
        mk, mv, mr = _magnitudes(xd, wh, sub, p.chunk, H, d)
        _check(host(kb[c0:c1]), rk, mk, 0.95)
        _check(host(vb[c0:c1]), rv, mv, 0.95)
        _check(kr_rows[c0:c1], rr, mr, 0.95)


@pytest.mark.parametrize("bf16,d", [(True, 128), (False, 64)])
def test_encode_halves_compose_to_encode(bf16, d):
    """msa_encode_pool then msa_encode_project on two streams, two blocks in
    flight with one workspace each, give msa_encode's stores bit for bit."""
    H, chunk, hidden = 2, 64, 320
    blocks = [_case(40 + i, 30, hidden, H, d, chunk, bf16) for i in range(2)]
    s_pool, s_proj = torch.cuda.Stream(), torch.cuda.Stream()
    outs, refs, keep = [], [], []            # every tensor a side stream touches lives until the sync
    for tok_off, chunk_off, n_chunks, co_d, cd, x, w in blocks:
        xd, wd, to_d = to_dev(x, bf16), to_dev(w, bf16), to_dev_i64(tok_off)
        refs.append([host(t) for t in M.msa_encode(xd, wd, to_d, co_d, cd, chunk, H, d, kr_layout=int(bf16))])
        ws = torch.empty(M.lib.msa_encode_workspace(M.MSA_BF16 if bf16 else M.MSA_F32, n_chunks, hidden, H, d),
                         dtype=torch.uint8, device=xd.device)
        keep += [xd, wd, to_d, co_d, cd, ws]
        s_pool.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_pool):
            M.msa_encode_pool(xd, to_d, co_d, cd, chunk, H, d, ws=ws)
            ev = torch.cuda.Event()
            ev.record(s_pool)
        s_proj.wait_event(ev)
        with torch.cuda.stream(s_proj):
            kb = torch.empty((n_chunks, H, d), dtype=xd.dtype, device=xd.device)
            vb = torch.empty_like(kb)
            kr = torch.empty((M.padded_chunks(n_chunks, int(bf16)), H, d), dtype=xd.dtype, device=xd.device)
            outs.append(M.msa_encode_project(wd, n_chunks, H, d, ws, kr_layout=int(bf16), k_bar=kb, v_bar=vb,
                                             kr_hat=kr))
    torch.cuda.synchronize()
    for got, ref in zip(outs, refs):
        for g, r in zip(got, ref):
            np.testing.assert_array_equal(host(g), r)
