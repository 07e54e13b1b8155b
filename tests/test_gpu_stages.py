"""Stage parity on the GPU: every msa_* call against the oracle's same step,
fed the same seeded inputs, at sizes that span several tiles, ragged
documents, empty documents and partial chunks."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.helpers import (ATOL_ATTN, RTOL_SCORE, check_ids, check_scores, dev, gen, host, ragged_lengths,
                           tile_np, to_dev, to_dev_i64, untile_np)

pytestmark = pytest.mark.gpu

import sparse_attention_long_msa_amd as M  # noqa: E402  (a missing library fails loudly)


def _doc_index(lengths, chunk):
    tok_off = synth.offsets(lengths)
    chunk_off = O.chunk_offsets(tok_off, chunk)
    n_chunks = int(chunk_off[-1])
    co_d = to_dev_i64(chunk_off)
    cd = M.msa_chunk_doc_map(co_d, n_chunks)
    return tok_off, chunk_off, n_chunks, co_d, cd


def test_synth_device_matches_host():
    from synth import device as SD
    for bf16, start, n, sp in ((True, 0, 100003, 0), (False, 12345678901, 4099, 0), (True, 7, 5000, -3)):
        t = torch.empty(n, dtype=torch.bfloat16 if bf16 else torch.float32, device=dev())
        SD.fill(t, 1234, 3, synth.T_KR, start=start, scale_pow2=sp)
        want = synth.normal(1234, synth.stream_id(3, synth.T_KR), start, n, bf16=bf16, scale_pow2=sp)
        got = t.float().cpu().numpy()
        np.testing.assert_array_equal(got, want)


def test_chunk_doc_map():
    lens = ragged_lengths(1, 500, 0, 300, n_empty=40)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    want = np.repeat(np.arange(500), np.diff(chunk_off))
    np.testing.assert_array_equal(cd.cpu().numpy(), want)


def test_tile_routing_keys_is_the_documented_permutation():
    for N, H, d in ((37, 8, 128), (64, 2, 32), (1, 8, 128)):
        x = gen(5, 0, synth.T_KR, (N, H, d), True)
        t = M.msa_tile_routing_keys(to_dev(x, True))
        np.testing.assert_array_equal(host(t), tile_np(x))
        np.testing.assert_array_equal(untile_np(host(t), N), x)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("normalize", [False, True])
@pytest.mark.parametrize("chunk", [64, 1, 5])
@pytest.mark.parametrize("layout", [0, 1])
def test_pool_encode(bf16, normalize, chunk, layout):
    H, d = 8, 128
    lens = ragged_lengths(2, 37, 0, 400, n_empty=3)
    lens[0] = 130                                    # two full chunks and a partial one
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, chunk)
    x = gen(11, 0, synth.T_KR, (int(lens.sum()), H, d), bf16)
    out = M.msa_pool_encode(to_dev(x, bf16), to_dev_i64(tok_off), co_d, cd, chunk, normalize, layout=layout)
    ref = O.pool_encode(x, tok_off, chunk, normalize, "bf16" if bf16 else "f32")
    got = host(out)
    if layout == 1:
        assert got.shape[0] == (n_chunks + 15) // 16 * 16
        assert np.all(untile_np(got, got.shape[0])[n_chunks:] == 0)      # zero padding chunks
        got = untile_np(got, n_chunks)
    if bf16:
        # float32 accumulation may move the once-rounded result by one bf16 ulp
        ulp = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)
        assert np.all(np.abs(got - ref) <= ulp + 1e-30)
        assert np.mean(got == ref) > 0.99
    else:
        np.testing.assert_allclose(got, ref, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("H,d", [(2, 32), (4, 64), (12, 128), (8, 256), (1, 512), (20, 128), (28, 128)])
def test_pool_encode_head_shapes(bf16, layout, H, d):
    # rows of 1/8 to 14 waves of 16-byte vectors, heads of 4 to 128 vectors:
    # every instantiation of the wave-per-chunk kernel (1 to 8 vectors per
    # lane) and the workgroup-per-chunk kernel
    lens = ragged_lengths(3, 41, 0, 90, n_empty=2)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 5)
    x = gen(12, 0, synth.T_KR, (int(lens.sum()), H, d), bf16)
    out = M.msa_pool_encode(to_dev(x, bf16), to_dev_i64(tok_off), co_d, cd, 5, True, layout=layout)
    ref = O.pool_encode(x, tok_off, 5, True, "bf16" if bf16 else "f32")
    got = host(out)
    if layout == 1:
        assert np.all(untile_np(got, got.shape[0])[n_chunks:] == 0)
        got = untile_np(got, n_chunks)
    if bf16:
        ulp = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)
        assert np.all(np.abs(got - ref) <= ulp + 1e-30)
        assert np.mean(got == ref) > 0.99
    else:
        np.testing.assert_allclose(got, ref, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("bf16,layout", [(True, 1), (True, 0), (False, 0)])
@pytest.mark.parametrize("B,T", [(1, 64), (1, 16), (1, 1), (2, 32), (32, 1), (1, 128), (3, 7), (1, 80), (4, 64),
                                 (100, 1)])
def test_route_score(bf16, layout, B, T):
    H, d = 8, 128
    lens = ragged_lengths(3 + T, 180, 1, 1500, n_empty=5)
    while ((lens + 63) // 64).sum() % 32 == 0:
        lens[-1] += 64
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    assert n_chunks % 32 != 0 and n_chunks > 32 * 40            # many tiles and a ragged tail
    dt = "bf16" if bf16 else "f32"
    raw = gen(21, 0, synth.T_KR, (n_chunks, H, d), bf16)
    store = O.round_to_store(O.l2_normalize(raw.astype(np.float64)), dt)
    q = gen(22, 0, synth.T_QR, (B, T, H, d), bf16)
    # plant a needle: one chunk of document 17 is the first query token itself
    nd = 17
    store[chunk_off[nd]] = O.round_to_store(O.l2_normalize(q[0, 0].astype(np.float64)), dt)
    st = tile_np(store) if layout == 1 else store
    ds = M.msa_route_score(to_dev(q, bf16), to_dev(st, bf16), cd, len(lens), layout=layout)
    ref = O.route_scores(q, store, chunk_off)
    got = host(ds)
    err = check_scores(got, ref, RTOL_SCORE[dt], k=16)
    print(f"route_score {dt} layout={layout} B={B} T={T}: normwise err {err:.3g}")
    assert np.argmax(got[0]) == nd


@pytest.mark.parametrize("layout", [1, 0])
def test_route_balance_keeps_the_scores(layout):
    """msa_route_balance sizes the scan's chunk ranges per XCD: the shares stay
    in their band and sum to one, and the scores after it equal, bit for bit,
    those of equal ranges (one 64-token query, 32 single-token queries and two
    column-grouped shapes, over a 1.1 GB store whose ranges are long enough for
    the split).  Clearing restores 1/8 each."""
    from synth import device as SD
    H, d = 8, 128
    r = np.random.default_rng(40)
    chunks = r.integers(1, 31, size=36000).astype(np.int64)
    chunks[r.choice(36000, size=7, replace=False)] = 0               # empty documents
    chunk_off = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    n_chunks, D = int(chunk_off[-1]), len(chunks)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert n_chunks >= 128 * 16 * n_cu                                 # ranges of 128+ tiles
    co_d = to_dev_i64(chunk_off)
    cd = M.msa_chunk_doc_map(co_d, n_chunks)
    rows = torch.empty((n_chunks, H, d), dtype=torch.bfloat16, device=dev())
    SD.fill(rows, 41, 0, synth.T_KR)
    st = M.msa_tile_routing_keys(rows) if layout == 1 else rows
    shapes = ((1, 64), (32, 1), (1, 128), (2, 100), (3, 64))   # the last three: 2, 4 and 3 column groups
    qs = [SD.fill(torch.empty((B, T, H, d), dtype=torch.bfloat16, device=dev()), 42 + i, 0, synth.T_QR)
          for i, (B, T) in enumerate(shapes)]
    try:
        M.msa_route_balance(None, None, None, 0, rounds=0)
        refs = [M.msa_route_score(q, st, cd, D, layout=layout).clone() for q in qs]
        for q, (B, T) in zip(qs[:3], shapes[:3]):   # one and two column groups can be calibrated
            shares = M.msa_route_balance(q, st, cd, D, rounds=2, layout=layout)
            assert abs(float(shares.sum()) - 1.0) < 1e-5
            assert (shares >= 0.75 / 8 - 1e-6).all() and (shares <= 1.25 / 8 + 1e-6).all()
            print(f"balance B={B} T={T} layout={layout}: shares {np.round(shares, 4).tolist()}")
            for q2, ref, (B2, T2) in zip(qs, refs, shapes):
                got = M.msa_route_score(q2, st, cd, D, layout=layout)
                torch.cuda.synchronize()
                assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), f"B={B2} T={T2}"
        # three column groups do not divide the CUs into one round: no calibration, the shares stay
        kept = M.msa_route_balance(qs[4], st, cd, D, rounds=1, layout=layout)
        assert np.array_equal(kept, shares)
    finally:
        cleared = M.msa_route_balance(None, None, None, 0, rounds=0)
    assert np.allclose(cleared, 0.125)


@pytest.mark.parametrize("bf16,layout", [(True, 1), (True, 0), (False, 0)])
@pytest.mark.parametrize("B,T", [(1, 64), (32, 1), (1, 128), (3, 7)])
def test_route_score_unfused_equals_fused(bf16, layout, B, T):
    """The unfused routing score: per-chunk scores (the max over the query's
    tokens, compared with the oracle's chunk cosines) then the standalone
    segmented max by document, which equals the fused msa_route_score bit for
    bit (max is exact), empty documents included."""
    H, d = 8, 128
    lens = ragged_lengths(60 + T, 300, 1, 1500, n_empty=7)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    dt = "bf16" if bf16 else "f32"
    store = O.round_to_store(O.l2_normalize(gen(61, 0, synth.T_KR, (n_chunks, H, d), bf16).astype(np.float64)), dt)
    q = gen(62, 0, synth.T_QR, (B, T, H, d), bf16)
    st = to_dev(tile_np(store) if layout == 1 else store, bf16)
    qd = to_dev(q, bf16)
    cs = M.msa_chunk_scores(qd, st, n_chunks, layout=layout)
    ref_c = O.chunk_cosines(q, store).max(axis=1)                  # token max per chunk [B, N]
    err = check_scores(host(cs), ref_c, RTOL_SCORE[dt], k=16)
    fused = M.msa_route_score(qd, st, cd, len(lens), layout=layout)
    seg = M.msa_segment_max(cs, co_d)
    assert torch.equal(seg, fused)
    print(f"unfused route score {dt} layout={layout} B={B} T={T}: chunk-score normwise err {err:.3g}")


def test_segment_max_is_the_document_max():
    rng = np.random.default_rng(7)
    lens = rng.integers(0, 9, size=5000)
    lens[:3] = 0
    lens[-1] = 0
    chunk_off = synth.offsets(lens)
    n_chunks = int(chunk_off[-1])
    x = rng.standard_normal((3, n_chunks)).astype(np.float32)
    got = host(M.msa_segment_max(torch.from_numpy(x).to(dev()), to_dev_i64(chunk_off)))
    want = np.full((3, len(lens)), -np.inf)
    for i in range(len(lens)):
        if lens[i]:
            want[:, i] = x[:, chunk_off[i]:chunk_off[i + 1]].max(axis=1)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("bf16,H,d,B,T", [(True, 4, 64, 2, 9), (False, 16, 256, 1, 20), (False, 2, 16, 5, 4),
                                         (False, 8, 128, 40, 1)])
def test_route_score_vector_path(bf16, H, d, B, T):
    """The vector path (float32, or head shapes off the MFMA path): column
    blocks of 16, 8 and 4 (by the LDS the scaled query rows take), ragged and
    empty documents, several queries per block."""
    lens = ragged_lengths(80 + d, 150, 0, 900, n_empty=6)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    dt = "bf16" if bf16 else "f32"
    store = O.round_to_store(O.l2_normalize(gen(81, 0, synth.T_KR, (n_chunks, H, d), bf16).astype(np.float64)), dt)
    q = gen(82, 0, synth.T_QR, (B, T, H, d), bf16)
    got = host(M.msa_route_score(to_dev(q, bf16), to_dev(store, bf16), cd, len(lens)))
    ref = O.route_scores(q, store, chunk_off)
    err = check_scores(got, ref, RTOL_SCORE[dt], k=8)
    cs = M.msa_chunk_scores(to_dev(q, bf16), to_dev(store, bf16), n_chunks)
    fused = M.msa_route_score(to_dev(q, bf16), to_dev(store, bf16), cd, len(lens))
    assert torch.equal(M.msa_segment_max(cs, co_d), fused)
    print(f"route_score vector path {dt} H={H} d={d} B={B} T={T}: normwise err {err:.3g}")


def test_route_score_document_table_paths():
    """64 single-token queries over a memory mixing one-chunk documents (a
    workgroup's range holds more (document, query) pairs than its LDS table:
    one global atomic per run), long documents (the table path: interior
    documents stored once, boundary documents atomically), a document that
    spans several workgroup ranges, and empty documents."""
    H, d, B, T = 8, 128, 64, 1
    rng = np.random.default_rng(5)
    lens = np.concatenate([np.full(3000, 64), rng.integers(1500, 2600, 40), [100_000], [0, 0],
                           rng.integers(1, 200, 2000), [0]]).astype(np.int64)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    raw = gen(41, 0, synth.T_KR, (n_chunks, H, d), True)
    store = O.round_to_store(O.l2_normalize(raw.astype(np.float64)), "bf16")
    q = gen(42, 0, synth.T_QR, (B, T, H, d), True)
    ref = O.route_scores(q, store, chunk_off)
    for layout in (1, 0):
        st = tile_np(store) if layout == 1 else store
        got = host(M.msa_route_score(to_dev(q, True), to_dev(st, True), cd, len(lens), layout=layout))
        err = check_scores(got, ref, RTOL_SCORE["bf16"], k=16)
        print(f"route_score table paths layout={layout}: normwise err {err:.3g}")


@pytest.mark.parametrize("bf16,layout", [(True, 1), (False, 0)])
def test_route_score_single_chunk_is_the_cosine(bf16, layout):
    """A memory of one document of one chunk and a one-token query: the score
    is the head mean of the per-head cosines (the textbook cosine when the
    heads agree)."""
    H, d = 8, 128
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(np.array([40]), 64)
    assert n_chunks == 1
    dt = "bf16" if bf16 else "f32"
    store = O.round_to_store(O.l2_normalize(gen(51, 0, synth.T_KR, (1, H, d), bf16).astype(np.float64)), dt)
    q = gen(52, 0, synth.T_QR, (1, 1, H, d), bf16)
    st = tile_np(store) if layout == 1 else store
    got = host(M.msa_route_score(to_dev(q, bf16), to_dev(st, bf16), cd, 1, layout=layout))
    qd = q.astype(np.float64)[0, 0]
    want = np.mean([qd[h] @ store[0, h].astype(np.float64) / np.linalg.norm(qd[h]) for h in range(H)])
    assert got.shape == (1, 1)
    assert abs(got[0, 0] - want) <= RTOL_SCORE[dt] * max(abs(want), 1e-3)


def test_route_score_rescale_invariance():
    """Cosine is invariant to a positive rescale of the routing query."""
    H, d = 8, 128
    lens = ragged_lengths(5, 64, 64, 640)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    store = O.round_to_store(O.l2_normalize(gen(31, 0, synth.T_KR, (n_chunks, H, d), True)), "bf16")
    q = gen(32, 0, synth.T_QR, (1, 64, H, d), True)
    st = to_dev(tile_np(store), True)
    a = host(M.msa_route_score(to_dev(q, True), st, cd, len(lens), layout=1))
    b = host(M.msa_route_score(to_dev(q * 4.0, True), st, cd, len(lens), layout=1))
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("B,D,k", [(1, 64, 4), (1, 2048, 16), (1, 195312, 16), (32, 10518, 16), (2, 5000, 256),
                                   (3, 4096, 1), (1, 4097, 32), (1, 9000, 9000 // 40),
                                   # the 16-wave final pass at its capacity (k = 64: the largest LDS),
                                   # one past it, a second reducing pass, a reducing pass into it
                                   (2, 16384, 64), (1, 16385, 64), (2, 1_000_000, 64), (1, 300_000, 48),
                                   # degenerate: every document selected; a single document
                                   (2, 64, 64), (3, 1, 1), (1, 256, 256)])
def test_topk_exact(B, D, k):
    r = np.random.default_rng(B * 7 + D)
    s = np.round(r.normal(size=(B, D)), 3).astype(np.float32)       # many exact ties
    s[:, r.integers(0, D, size=D // 10)] = -np.inf
    ids, vals = M.msa_topk(torch.from_numpy(s).to(dev()), k)
    want_ids, want_vals = O.topk(s.astype(np.float64), k)
    np.testing.assert_array_equal(ids.cpu().numpy(), want_ids)
    np.testing.assert_array_equal(vals.cpu().numpy().astype(np.float64), want_vals)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_gather(bf16, mode):
    Hkv, d, B, k = 8, 128, 3, 5
    lens = ragged_lengths(6, 50, 0, 500, n_empty=2)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    kb = gen(41, 0, synth.T_K, (n_chunks, Hkv, d), bf16)
    vb = gen(42, 0, synth.T_V, (n_chunks, Hkv, d), bf16)
    r = np.random.default_rng(9)
    ids = np.stack([r.choice(50, size=k, replace=False) for _ in range(B)]).astype(np.int32)
    mdc = int(np.diff(chunk_off).max())
    max_ctx = k * mdc
    if mode == 0:
        kbar, vbar = to_dev(kb, bf16), to_dev(vb, bf16)
    else:
        kbar = to_dev(kb, bf16).cpu().pin_memory()
        vbar = to_dev(vb, bf16).cpu().pin_memory()
    kc, vc, cp, cl = M.msa_gather_kv(torch.from_numpy(ids).to(dev()), co_d, kbar, vbar, mdc, max_ctx, src_mode=mode,
                                     chunk_off_h=chunk_off if mode == 2 else None, device=dev())
    torch.cuda.synchronize()
    for b in range(B):
        rk, rv, rp = O.gather(ids[b], chunk_off, kb, vb)
        n = len(rp)
        assert int(cl[b]) == n
        np.testing.assert_array_equal(host(kc[b, :n]), rk)
        np.testing.assert_array_equal(host(vc[b, :n]), rv)
        np.testing.assert_array_equal(cp[b, :n].cpu().numpy(), rp)


@pytest.mark.parametrize("B,D,k,n_excl", [(1, 195312, 16, 0), (32, 10518, 16, 0), (2, 300, 64, 0), (3, 2000, 16, 1990),
                                          (2, 20000, 40, 0), (2, 5000, 100, 0)])
def test_topk_context_index_matches_the_two_calls(B, D, k, n_excl):
    """msa_topk_context_index writes exactly what msa_topk and then
    msa_context_index write: the final selection pass of the 4- and 16-wave
    kinds, after a reducing pass, with excluded documents (trailing ids -1),
    and the k > 64 fallback."""
    r = np.random.default_rng(D + k)
    lens = r.integers(1, 700, D)
    lens[r.integers(0, D, D // 20)] = 0                       # empty documents
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    s = np.round(r.normal(size=(B, D)), 3).astype(np.float32)  # exact ties
    s[:, np.flatnonzero(lens == 0)] = -np.inf
    if n_excl:
        s[:, r.choice(D, n_excl, replace=False)] = np.nan      # fewer than k documents left
    mdc = int(np.diff(chunk_off).max())
    max_ctx = k * mdc
    sd = torch.from_numpy(s).to(dev())
    ids, vals = M.msa_topk(sd, k)
    row, pos, ln = M.msa_context_index(ids, co_d, n_chunks, mdc, max_ctx)
    fill = torch.full((B, max_ctx), -7, dtype=torch.int32, device=dev())
    row2, pos2 = fill.clone(), fill.clone()
    row[:], pos[:] = -7, -7                                   # entries past ctx_len stay untouched in both
    M.msa_context_index(ids, co_d, n_chunks, mdc, max_ctx, ctx_row=row, ctx_pos=pos, ctx_len=ln)
    ids2, vals2, row2, pos2, ln2 = M.msa_topk_context_index(sd, k, co_d, n_chunks, mdc, max_ctx, ctx_row=row2,
                                                            ctx_pos=pos2)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(vals.view(torch.int32), vals2.view(torch.int32))
    assert torch.equal(ln, ln2) and torch.equal(row, row2) and torch.equal(pos, pos2)
    if n_excl:
        assert (ids2[:, D - n_excl:] == -1).all()


@pytest.mark.parametrize("B,D,k", [(1, 195312, 16), (32, 10518, 16), (2, 3000, 64), (3, 1, 1), (2, 20000, 100),
                                    (1, 4096, 200)])
def test_topk_reset_leaves_minus_inf(B, D, k):
    """MSA_TOPK_RESET_SCORES: the selection and the context index are those of
    the call without it, and every score reads -inf afterwards (a reducing
    pass of either kind, a single pass, the k > 64 slice passes, NaN-excluded
    documents)."""
    r = np.random.default_rng(D * 3 + k)
    lens = r.integers(1, 600, D)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    s = np.round(r.normal(size=(B, D)), 3).astype(np.float32)
    s[:, r.integers(0, D, size=max(1, D // 50))] = np.nan
    s[:, 0] = 5.0
    sd = torch.from_numpy(s).to(dev())
    ids, vals = M.msa_topk(sd, k)
    work = sd.clone()
    ids2, vals2 = M.msa_topk(work, k, reset=True)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(vals.view(torch.int32), vals2.view(torch.int32))
    assert bool((work == float("-inf")).all())
    mdc = int(np.diff(chunk_off).max())
    max_ctx = k * mdc
    row, pos, ln = M.msa_context_index(ids, co_d, n_chunks, mdc, max_ctx)
    work = sd.clone()
    ids3, vals3, row3, pos3, ln3 = M.msa_topk_context_index(work, k, co_d, n_chunks, mdc, max_ctx, reset=True)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids3) and torch.equal(vals.view(torch.int32), vals3.view(torch.int32))
    assert torch.equal(ln, ln3)
    for b in range(B):
        n = int(ln[b])
        assert torch.equal(row[b, :n], row3[b, :n]) and torch.equal(pos[b, :n], pos3[b, :n])
    assert bool((work == float("-inf")).all())


@pytest.mark.parametrize("bf16,layout,B,T", [(True, 1, 1, 64), (True, 0, 3, 16), (True, 1, 32, 1), (False, 0, 2, 5)])
def test_route_prefilled_after_reset(bf16, layout, B, T):
    """Route -> top-k with reset -> route with MSA_ROUTE_PREFILLED on the same
    buffer, three layers in a row: every layer's scores, ids and values equal
    those of the filling call bit for bit, and the buffer ends at -inf."""
    H, d = 8, 128
    lens = ragged_lengths(13, 700, 0, 900, n_empty=11)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    D, k = len(lens), 16
    buf = torch.full((B, D), float("-inf"), dtype=torch.float32, device=dev())
    for l in range(3):
        st = O.round_to_store(O.l2_normalize(gen(31, l, synth.T_KR, (n_chunks, H, d), bf16).astype(np.float64)),
                              "bf16" if bf16 else "f32")
        st_d = to_dev(tile_np(st) if layout == 1 else st, bf16)
        q = to_dev(gen(32, l, synth.T_QR, (B, T, H, d), bf16), bf16)
        ref = M.msa_route_score(q, st_d, cd, D, layout=layout)
        ids, vals = M.msa_topk(ref, k)
        M.msa_route_score(q, st_d, cd, D, doc_score=buf, layout=layout, prefilled=True)
        torch.cuda.synchronize()
        assert torch.equal(buf.view(torch.int32), ref.view(torch.int32)), f"layer {l}"
        ids2, vals2 = M.msa_topk(buf, k, reset=True)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids2) and torch.equal(vals.view(torch.int32), vals2.view(torch.int32))
        assert bool((buf == float("-inf")).all())


@pytest.mark.parametrize("bf16,layout,B,T,host_src", [(True, 1, 1, 64, True), (True, 0, 3, 16, False),
                                                      (True, 1, 32, 1, True), (False, 0, 2, 5, False)])
def test_route_score_fetch_equals_the_two_calls(bf16, layout, B, T, host_src):
    """msa_route_score_fetch: the scores of msa_route_score and the context of
    msa_gather_kv, bit for bit, from device memory or pinned host memory; two
    calls in a row on one workspace (the second finds the first's counter),
    the second with a prefilled score buffer and a smaller selection."""
    H, d, Hkv = 8, 128, 8
    lens = ragged_lengths(17, 900, 0, 900, n_empty=13)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    D = len(lens)
    mdc = int(np.diff(chunk_off).max())
    st = O.round_to_store(O.l2_normalize(gen(33, 0, synth.T_KR, (n_chunks, H, d), bf16).astype(np.float64)),
                          "bf16" if bf16 else "f32")
    st_d = to_dev(tile_np(st) if layout == 1 else st, bf16)
    q = to_dev(gen(34, 0, synth.T_QR, (B, T, H, d), bf16), bf16)
    kb = to_dev(gen(35, 0, synth.T_K, (n_chunks, Hkv, d), bf16), bf16)
    vb = to_dev(gen(35, 0, synth.T_V, (n_chunks, Hkv, d), bf16), bf16)
    if host_src:
        kb, vb = kb.cpu().pin_memory(), vb.cpu().pin_memory()
    ws = torch.empty(M.lib.msa_route_score_fetch_workspace(int(bf16), B, T, H, d, D, n_chunks), dtype=torch.uint8,
                     device=dev())
    buf = torch.empty((B, D), dtype=torch.float32, device=dev())
    r = np.random.default_rng(B + T)
    for call, (fB, k) in enumerate(((3, 16), (2, 5))):
        ids = np.stack([r.choice(D, size=k, replace=False) for _ in range(fB)]).astype(np.int32)
        ids[0, -1] = -1                                   # a rank left empty (fewer documents than k)
        ids_d = torch.from_numpy(ids).to(dev())
        max_ctx = k * mdc
        want = M.msa_gather_kv(ids_d, co_d, kb, vb, mdc, max_ctx,
                               src_mode=M.MSA_SRC_HOST_MAPPED if host_src else M.MSA_SRC_DEVICE, device=dev())
        ref = M.msa_route_score(q, st_d, cd, D, layout=layout)
        out = [torch.full_like(want[0], 7), torch.full_like(want[1], 7), torch.full_like(want[2], -5),
               torch.full_like(want[3], -5)]
        if call == 1:
            buf.fill_(float("-inf"))
        M.msa_route_score_fetch(q, st_d, cd, D, ids_d, co_d, kb, vb, mdc, *out, doc_score=buf, ws=ws, layout=layout,
                                prefilled=call == 1)
        torch.cuda.synchronize()
        assert torch.equal(buf.view(torch.int32), ref.view(torch.int32)), f"call {call}: scores"
        assert torch.equal(out[3], want[3]), f"call {call}: ctx_len"
        for b in range(fB):
            n = int(want[3][b])
            for i in range(3):
                assert torch.equal(out[i][b, :n], want[i][b, :n]), f"call {call}, query {b}: output {i}"


@pytest.mark.parametrize("B,k", [(3, 5), (1, 50), (4, 1)])
def test_context_index(B, k):
    lens = ragged_lengths(7, 50, 0, 500, n_empty=3)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    r = np.random.default_rng(10 + k)
    ids = np.stack([r.choice(50, size=k, replace=False) for _ in range(B)]).astype(np.int32)
    mdc = int(np.diff(chunk_off).max())
    max_ctx = k * mdc
    row, pos, ln = M.msa_context_index(torch.from_numpy(ids).to(dev()), co_d, n_chunks, mdc, max_ctx)
    torch.cuda.synchronize()
    # the oracle's concatenation of a store whose row c holds the value c gives the rows
    rowval = np.arange(n_chunks, dtype=np.float64)[:, None, None]
    for b in range(B):
        rk, _, rp = O.gather(ids[b], chunk_off, rowval, rowval)
        n = len(rp)
        assert int(ln[b]) == n
        np.testing.assert_array_equal(row[b, :n].cpu().numpy(), rk[:, 0, 0].astype(np.int32))
        np.testing.assert_array_equal(pos[b, :n].cpu().numpy(), rp)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("B,T,L_loc,ctx", [(1, 16, 16, [32]), (32, 1, 2048, None), (2, 64, 300, [0, 700]),
                                           (4, 1, 1, [5, 0, 31, 64]), (1, 128, 200, [1000]),
                                           (2, 1, 64, [4100, 2500]), (1, 64, 64, [5000])])
def test_sparse_attention_indexed(bf16, B, T, L_loc, ctx):
    """Attention reading the context rows in place equals the gathered path
    bit for bit and the oracle within tolerance."""
    Hq, Hkv, d, qpo, n_rows = 32, 8, 128, 16, 3000
    if ctx is None:
        ctx = list(np.random.default_rng(1).integers(100, 1500, size=B))
    max_ctx = max(max(ctx), 1)
    if not bf16 and B * (max_ctx + L_loc) > 200000:
        pytest.skip("float32 path is the small-case vector path")
    seed = 70 + T
    q = gen(seed, 0, synth.T_Q, (B, T, Hq, d), bf16)
    kl = gen(seed, 0, synth.T_KLOC, (B, L_loc, Hkv, d), bf16)
    vl = gen(seed, 0, synth.T_VLOC, (B, L_loc, Hkv, d), bf16)
    kst = gen(seed, 0, synth.T_K, (n_rows, Hkv, d), bf16, scale_pow2=-3)
    vst = gen(seed, 0, synth.T_V, (n_rows, Hkv, d), bf16, scale_pow2=-3)
    r = np.random.default_rng(seed)
    rows = r.integers(0, n_rows, size=(B, max_ctx)).astype(np.int32)
    cp = r.integers(0, min(128, max_ctx), size=(B, max_ctx)).astype(np.int32)   # positions < max_ctx
    cl = np.asarray(ctx, dtype=np.int32)
    d_rows, d_cp, d_cl = (torch.from_numpy(a).to(dev()) for a in (rows, cp, cl))
    kst_d, vst_d = to_dev(kst, bf16), to_dev(vst, bf16)
    qd, kld, vld = to_dev(q, bf16), to_dev(kl, bf16), to_dev(vl, bf16)
    got = M.msa_sparse_attn_indexed(qd, kst_d, vst_d, d_rows, d_cp, d_cl, kld, vld, qpo)
    gathered = M.msa_sparse_attn(qd, kst_d[d_rows.long()].contiguous(), vst_d[d_rows.long()].contiguous(), d_cp,
                                 d_cl, kld, vld, qpo)
    assert torch.equal(got, gathered)
    sm = 1.0 / math.sqrt(d)
    g = host(got)
    for b in (range(B) if B <= 4 else [0, 17, 31]):
        n = int(cl[b])
        ref = O.attend_one(q[b], kst[rows[b, :n]], vst[rows[b, :n]], cp[b, :n], kl[b], vl[b], qpo, 1e6, sm)
        e = np.abs(g[b] - ref).max()
        assert e <= ATOL_ATTN["bf16" if bf16 else "f32"], f"b={b}: max-abs {e}"


@pytest.mark.parametrize("B,T,L_loc,ctx", [(1, 64, 4096, [128]), (32, 1, 2048, None), (2, 64, 300, [0, 700]),
                                           (1, 128, 200, [1000])])
def test_sparse_attention_indexed_host_store(B, T, L_loc, ctx):
    """The indexed attention reading its context rows from a store in pinned
    host memory (over the host link) equals the same call on the store in
    device memory bit for bit: the prefill (with the context's own split at
    the 100M shape) and decode kernels, empty and long contexts."""
    Hq, Hkv, d, qpo, n_rows = 32, 8, 128, 16, 3000
    if ctx is None:
        ctx = list(np.random.default_rng(3).integers(100, 1500, size=B))
    max_ctx = max(max(ctx), 1)
    seed = 150 + T
    q, kl, vl = (to_dev(gen(seed, 0, t, shp, True), True) for t, shp in ((synth.T_Q, (B, T, Hq, d)),
                                                                       (synth.T_KLOC, (B, L_loc, Hkv, d)),
                                                                       (synth.T_VLOC, (B, L_loc, Hkv, d))))
    kst = to_dev(gen(seed, 0, synth.T_K, (n_rows, Hkv, d), True, scale_pow2=-3), True)
    vst = to_dev(gen(seed, 0, synth.T_V, (n_rows, Hkv, d), True, scale_pow2=-3), True)
    r = np.random.default_rng(seed)
    rows = torch.from_numpy(r.integers(0, n_rows, size=(B, max_ctx)).astype(np.int32)).to(dev())
    cp = torch.from_numpy(r.integers(0, min(128, max_ctx), size=(B, max_ctx)).astype(np.int32)).to(dev())
    cl = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).to(dev())
    want = M.msa_sparse_attn_indexed(q, kst, vst, rows, cp, cl, kl, vl, qpo)
    got = M.msa_sparse_attn_indexed(q, kst.cpu().pin_memory(), vst.cpu().pin_memory(), rows, cp, cl, kl, vl, qpo)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


@pytest.mark.parametrize("B,D,k,n_sets", [(3, 5000, 16, 2), (2, 300, 64, 4), (1, 40, 16, 2), (2, 2000, 100, 3),
                                          (4, 20000, 32, 1)])
def test_exclude_then_topk(B, D, k, n_sets):
    """Documents fetched in earlier rounds are skipped; ties keep the id order;
    when the documents run out the trailing ids are -1 (oracle topk_excluding)."""
    r = np.random.default_rng(D + k)
    s = np.round(r.standard_normal((B, D)), 2).astype(np.float32)   # many ties
    s[:, ::97] = -np.inf                                             # empty documents
    sets = np.stack([np.stack([r.choice(D, size=k, replace=False) for _ in range(B)]) for _ in range(n_sets)])
    sets = sets.astype(np.int32)
    sets[0, 0, 0] = -1                      # an exhausted round
    sets[-1, -1, -1] = D + 7                # out of range: ignored
    ds = torch.from_numpy(s).to(dev())
    M.msa_exclude_docs(ds, torch.from_numpy(sets).to(dev()))
    ids, vals = M.msa_topk(ds, k)
    torch.cuda.synchronize()
    want_ids, want_vals = O.topk_excluding(s.astype(np.float64), k, [sets[:, b].reshape(-1).tolist() for b in range(B)])
    np.testing.assert_array_equal(ids.cpu().numpy(), want_ids)
    got_v = vals.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(np.isnan(got_v), np.isnan(want_vals))
    np.testing.assert_array_equal(got_v[~np.isnan(got_v)], want_vals[~np.isnan(want_vals)])


def test_context_append_rounds():
    lens = ragged_lengths(17, 60, 0, 500, n_empty=4)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    B, k, R = 3, 5, 4
    mdc = int(np.diff(chunk_off).max())
    max_ctx = R * k * mdc
    r = np.random.default_rng(3)
    picks = np.stack([r.permutation(60)[:R * k] for _ in range(B)]).astype(np.int32).reshape(B, R, k)
    picks[1, 2, 3:] = -1                    # a round that ran out of documents
    row = torch.full((B, max_ctx), -7, dtype=torch.int32, device=dev())
    pos = torch.full((B, max_ctx), -7, dtype=torch.int32, device=dev())
    lens_d = [torch.empty(B, dtype=torch.int32, device=dev()) for _ in range(2)]
    for rd in range(R):
        ids = torch.from_numpy(np.ascontiguousarray(picks[:, rd])).to(dev())
        if rd == 0:
            M.msa_context_index(ids, co_d, n_chunks, mdc, max_ctx, ctx_row=row, ctx_pos=pos, ctx_len=lens_d[0])
        else:
            M.msa_context_append(ids, co_d, n_chunks, mdc, row, pos, lens_d[(rd - 1) % 2], lens_d[rd % 2])
    torch.cuda.synchronize()
    ln = lens_d[(R - 1) % 2].cpu().numpy()
    rowval = np.arange(n_chunks, dtype=np.float64)[:, None, None]
    for b in range(B):
        fetched = [int(x) for x in picks[b].reshape(-1) if x >= 0]
        rk, _, rp = O.gather(np.asarray(fetched), chunk_off, rowval, rowval)
        n = len(rp)
        assert ln[b] == n
        np.testing.assert_array_equal(row[b, :n].cpu().numpy(), rk[:, 0, 0].astype(np.int32))
        np.testing.assert_array_equal(pos[b, :n].cpu().numpy(), rp)
        assert (row[b, n:].cpu().numpy() == -7).all()      # nothing written past the context


def test_interleave_end_to_end():
    """Three rounds of route -> skip fetched -> top-k -> append, then attention
    over the grown context, against the oracle's rounds on the GPU's picks."""
    H, d, Hq, B, T, L_loc, k, R = 8, 128, 32, 2, 4, 300, 8, 3
    lens = ragged_lengths(23, 900, 0, 1200, n_empty=20)
    tok_off, chunk_off, n_chunks, co_d, cd = _doc_index(lens, 64)
    D = len(lens)
    mdc = int(np.diff(chunk_off).max())
    store = O.round_to_bf16(O.l2_normalize(gen(61, 0, synth.T_KR, (n_chunks, H, d), True).astype(np.float64)))
    kb = gen(61, 0, synth.T_K, (n_chunks, H, d), True, scale_pow2=-3)
    vb = gen(61, 0, synth.T_V, (n_chunks, H, d), True, scale_pow2=-3)
    qr = [gen(62, rd, synth.T_QR, (B, T, H, d), True) for rd in range(R)]
    q = gen(62, 0, synth.T_Q, (B, T, Hq, d), True)
    kl = gen(62, 0, synth.T_KLOC, (B, L_loc, H, d), True)
    vl = gen(62, 0, synth.T_VLOC, (B, L_loc, H, d), True)
    run = M.LayerRunner(batch=B, tokens=T, q_heads=Hq, kv_heads=H, head_dim=d, n_docs=D, n_chunks=n_chunks, k=k,
                        max_doc_chunks=mdc, local_len=L_loc, dtype=torch.bfloat16, device=dev(),
                        kr_layout=M.MSA_LAYOUT_TILED, indexed=True, rounds=R)
    out = run.interleave([to_dev(x, True) for x in qr], to_dev(tile_np(store), True), cd, co_d, to_dev(kb, True),
                         to_dev(vb, True), to_dev(q, True), to_dev(kl, True), to_dev(vl, True))
    torch.cuda.synchronize()
    gpu_ids = run.ids_rounds.cpu().numpy()
    ref = O.interleave(qr, store, chunk_off, kb, vb, k, q, kl, vl, ids_override=gpu_ids)
    fetched = [set() for _ in range(B)]
    for rd in range(R):
        s_ref = ref["rounds"][rd]["doc_score"].copy()
        for b in range(B):
            s_ref[b, list(fetched[b])] = -np.inf          # documents fetched earlier cannot be chosen
            fetched[b].update(int(x) for x in gpu_ids[rd, b])
        check_ids(gpu_ids[rd], s_ref, k)
    for b in range(B):
        assert len(fetched[b]) == R * k                   # no document fetched twice
    e = np.abs(host(out) - ref["out"]).max()
    assert e <= ATOL_ATTN["bf16"], e
    assert int(run.ctx_len.cpu()[0]) == sum(int(np.diff(chunk_off)[x]) for x in gpu_ids[:, 0].reshape(-1))


def _attn_case(seed, B, T, Hq, Hkv, d, L_loc, ctx_lens, bf16, max_ctx):
    q = gen(seed, 0, synth.T_Q, (B, T, Hq, d), bf16)
    kl = gen(seed, 0, synth.T_KLOC, (B, L_loc, Hkv, d), bf16)
    vl = gen(seed, 0, synth.T_VLOC, (B, L_loc, Hkv, d), bf16)
    kc = gen(seed, 0, synth.T_K, (B, max_ctx, Hkv, d), bf16, scale_pow2=-3)
    vc = gen(seed, 0, synth.T_V, (B, max_ctx, Hkv, d), bf16, scale_pow2=-3)
    r = np.random.default_rng(seed)
    cp = r.integers(0, min(128, max_ctx), size=(B, max_ctx)).astype(np.int32)
    cl = np.asarray(ctx_lens, dtype=np.int32)
    return q, kl, vl, kc, vc, cp, cl


@pytest.mark.parametrize("bf16,Hq,Hkv,d,B,T,L_loc,ctx", [
    (False, 4, 2, 2, 2, 3, 5, [0, 9]),              # smallest head, empty context
    (True, 6, 2, 64, 3, 2, 40, [17, 0, 130]),       # off the MFMA path: d = 64, group of 3
    (False, 8, 8, 96, 1, 16, 16, [700]),            # d = 96 (pairs not a multiple of 64)
    (True, 4, 1, 256, 2, 1, 300, [2100, 5]),        # largest head, two pairs per lane
    (False, 32, 8, 128, 1, 7, 7, [4000]),           # key count off the four-key step
])
def test_sparse_attention_vector_path(bf16, Hq, Hkv, d, B, T, L_loc, ctx):
    """The vector attention path (float32, or head shapes off the MFMA path)
    against the oracle, over head sizes from 2 to 256 and group sizes 1-4."""
    max_ctx = max(max(ctx), 1)
    qpo = 16
    q, kl, vl, kc, vc, cp, cl = _attn_case(90 + d, B, T, Hq, Hkv, d, L_loc, ctx, bf16, max_ctx)
    out = M.msa_sparse_attn(to_dev(q, bf16), to_dev(kc, bf16), to_dev(vc, bf16),
                            torch.from_numpy(cp).to(dev()), torch.from_numpy(cl).to(dev()), to_dev(kl, bf16),
                            to_dev(vl, bf16), qpo)
    got = host(out)
    sm = 1.0 / math.sqrt(d)
    for b in range(B):
        n = int(cl[b])
        ref = O.attend_one(q[b], kc[b, :n], vc[b, :n], cp[b, :n], kl[b], vl[b], qpo, 1e6, sm)
        e = np.abs(got[b] - ref).max()
        assert e <= ATOL_ATTN["bf16" if bf16 else "f32"], f"b={b}: max-abs {e}"


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("B,T,L_loc,ctx", [(1, 16, 16, [32]), (1, 64, 4096, [128]), (32, 1, 8192, None),
                                           (2, 3, 50, [0, 77]), (1, 128, 300, [1000]), (4, 1, 1, [5, 0, 31, 64])])
def test_sparse_attention(bf16, B, T, L_loc, ctx):
    Hq, Hkv, d, qpo = 32, 8, 128, 16
    if ctx is None:
        ctx = list(np.random.default_rng(0).integers(100, 2048, size=B))
    max_ctx = max(max(ctx), 1)
    q, kl, vl, kc, vc, cp, cl = _attn_case(50 + T, B, T, Hq, Hkv, d, L_loc, ctx, bf16, max_ctx)
    if not bf16 and B * (max_ctx + L_loc) > 200000:
        pytest.skip("float32 path is the small-case vector path")
    out = M.msa_sparse_attn(to_dev(q, bf16), to_dev(kc, bf16), to_dev(vc, bf16),
                            torch.from_numpy(cp).to(dev()), torch.from_numpy(cl).to(dev()), to_dev(kl, bf16),
                            to_dev(vl, bf16), qpo)
    got = host(out)
    sm = 1.0 / math.sqrt(d)
    worst = 0.0
    rows = range(B) if B <= 4 else [0, 7, 31]
    for b in rows:
        n = int(cl[b])
        ref = O.attend_one(q[b], kc[b, :n], vc[b, :n], cp[b, :n], kl[b], vl[b], qpo, 1e6, sm)
        e = np.abs(got[b] - ref).max()
        worst = max(worst, e)
        assert e <= ATOL_ATTN["bf16" if bf16 else "f32"], f"b={b}: max-abs {e}"
    print(f"attention bf16={bf16} B={B} T={T}: max-abs {worst:.3g}")


@pytest.mark.parametrize("B,T,L_loc,ctx,indexed", [
    (1, 64, 4096, [128], False),          # the 100M-token preset's shape, gathered (host-tier) context
    (1, 64, 4096, [128], True),           # the same, context read in place
    (32, 1, 8192, None, True),            # batched decode (decode kernel)
    (2, 3, 50, [0, 77], False),           # an empty context, ragged lengths
    (4, 1, 1, [5, 0, 31, 64], False),     # one local token
    (1, 128, 300, [1000], True),          # two row groups
    (2, 64, 64, [5000, 4100], True),      # context over the LDS index cache: several context splits
    (1, 16, 16, [0], False),              # no context at all: the context part only merges
])
def test_sparse_attention_two_calls(B, T, L_loc, ctx, indexed):
    """msa_sparse_attn_part: the local call on a side stream (it reads no
    context), the context call after it on the main stream; the oracle within
    the attention tolerance, and msa_sparse_attn within the same bound."""
    Hq, Hkv, d, qpo, n_rows = 32, 8, 128, 16, 6000
    if ctx is None:
        ctx = list(np.random.default_rng(2).integers(100, 2048, size=B))
    max_ctx = max(max(ctx), 1)
    seed = 110 + T
    q = gen(seed, 0, synth.T_Q, (B, T, Hq, d), True)
    kl = gen(seed, 0, synth.T_KLOC, (B, L_loc, Hkv, d), True)
    vl = gen(seed, 0, synth.T_VLOC, (B, L_loc, Hkv, d), True)
    kst = gen(seed, 0, synth.T_K, (n_rows, Hkv, d), True, scale_pow2=-3)
    vst = gen(seed, 0, synth.T_V, (n_rows, Hkv, d), True, scale_pow2=-3)
    r = np.random.default_rng(seed)
    rows = r.integers(0, n_rows, size=(B, max_ctx)).astype(np.int32)
    cp = r.integers(0, min(128, max_ctx), size=(B, max_ctx)).astype(np.int32)
    cl = np.asarray(ctx, dtype=np.int32)
    d_rows, d_cp, d_cl = (torch.from_numpy(a).to(dev()) for a in (rows, cp, cl))
    kst_d, vst_d = to_dev(kst, True), to_dev(vst, True)
    qd, kld, vld = to_dev(q, True), to_dev(kl, True), to_dev(vl, True)
    kc_d, vc_d = kst_d[d_rows.long()].contiguous(), vst_d[d_rows.long()].contiguous()
    ws = torch.empty(M.msa_sparse_attn_part_workspace(M.MSA_BF16, B, T, Hq, Hkv, d, max_ctx, L_loc, qpo),
                     dtype=torch.uint8, device=dev())
    side, main = torch.cuda.Stream(), torch.cuda.current_stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        M.msa_sparse_attn_part(M.MSA_ATTN_PART_LOCAL, qd, kld, vld, qpo, max_ctx, ws=ws, stream=side)
    main.wait_stream(side)
    if indexed:
        out = M.msa_sparse_attn_part(M.MSA_ATTN_PART_CONTEXT, qd, kld, vld, qpo, max_ctx, k_ctx=kst_d, v_ctx=vst_d,
                                     ctx_row=d_rows, ctx_pos=d_cp, ctx_len=d_cl, ws=ws)
    else:
        out = M.msa_sparse_attn_part(M.MSA_ATTN_PART_CONTEXT, qd, kld, vld, qpo, max_ctx, k_ctx=kc_d, v_ctx=vc_d,
                                     ctx_pos=d_cp, ctx_len=d_cl, ws=ws)
    whole = M.msa_sparse_attn(qd, kc_d, vc_d, d_cp, d_cl, kld, vld, qpo)
    got = host(out)
    assert np.isfinite(got).all()
    e_whole = np.abs(got - host(whole)).max()
    assert e_whole <= ATOL_ATTN["bf16"], f"against msa_sparse_attn: max-abs {e_whole}"
    sm = 1.0 / math.sqrt(d)
    for b in (range(B) if B <= 4 else [0, 13, 31]):
        n = int(cl[b])
        ref = O.attend_one(q[b], kst[rows[b, :n]], vst[rows[b, :n]], cp[b, :n], kl[b], vl[b], qpo, 1e6, sm)
        e = np.abs(got[b] - ref).max()
        assert e <= ATOL_ATTN["bf16"], f"b={b}: max-abs {e}"
    print(f"two-call attention B={B} T={T} indexed={indexed}: against msa_sparse_attn {e_whole:.3g}")


@pytest.mark.parametrize("Hq,B,T,L_loc,ctx", [
    (32, 1, 64, 4096, [128]),        # the 100M- and 1M-token presets' shape
    (32, 2, 64, 4096, [128, 0]),     # an empty context: its split sees no key
    (32, 3, 32, 2048, [100, 37, 1]),  # contexts shorter than max_ctx
    (16, 1, 16, 512, [40]),          # group of 2
    (64, 2, 64, 1024, [64, 20]),     # group of 8
])
def test_sparse_attention_context_split(Hq, B, T, L_loc, ctx):
    """Shapes whose context is no longer than one split's share of the keys:
    the one-call attention gives the context a split of its own and the local
    keys the others.  Against the oracle within the attention tolerance, the
    in-place and gathered contexts bit for bit, and the two-call form within
    the same tolerance."""
    Hkv, d, qpo, n_rows = 8, 128, 16, 4000
    max_ctx = max(ctx)
    seed = 130 + T + Hq
    q = gen(seed, 0, synth.T_Q, (B, T, Hq, d), True)
    kl = gen(seed, 0, synth.T_KLOC, (B, L_loc, Hkv, d), True)
    vl = gen(seed, 0, synth.T_VLOC, (B, L_loc, Hkv, d), True)
    kst = gen(seed, 0, synth.T_K, (n_rows, Hkv, d), True, scale_pow2=-3)
    vst = gen(seed, 0, synth.T_V, (n_rows, Hkv, d), True, scale_pow2=-3)
    r = np.random.default_rng(seed)
    rows = r.integers(0, n_rows, size=(B, max_ctx)).astype(np.int32)
    cp = r.integers(0, min(128, max_ctx), size=(B, max_ctx)).astype(np.int32)
    cl = np.asarray(ctx, dtype=np.int32)
    d_rows, d_cp, d_cl = (torch.from_numpy(a).to(dev()) for a in (rows, cp, cl))
    kst_d, vst_d = to_dev(kst, True), to_dev(vst, True)
    qd, kld, vld = to_dev(q, True), to_dev(kl, True), to_dev(vl, True)
    got = M.msa_sparse_attn_indexed(qd, kst_d, vst_d, d_rows, d_cp, d_cl, kld, vld, qpo)
    kc_d, vc_d = kst_d[d_rows.long()].contiguous(), vst_d[d_rows.long()].contiguous()
    gathered = M.msa_sparse_attn(qd, kc_d, vc_d, d_cp, d_cl, kld, vld, qpo)
    assert torch.equal(got, gathered)
    ws = torch.empty(M.msa_sparse_attn_part_workspace(M.MSA_BF16, B, T, Hq, Hkv, d, max_ctx, L_loc, qpo),
                     dtype=torch.uint8, device=dev())
    M.msa_sparse_attn_part(M.MSA_ATTN_PART_LOCAL, qd, kld, vld, qpo, max_ctx, ws=ws)
    two = M.msa_sparse_attn_part(M.MSA_ATTN_PART_CONTEXT, qd, kld, vld, qpo, max_ctx, k_ctx=kc_d, v_ctx=vc_d,
                                 ctx_pos=d_cp, ctx_len=d_cl, ws=ws)
    g = host(got)
    assert np.isfinite(g).all()
    assert np.abs(g - host(two)).max() <= ATOL_ATTN["bf16"]
    sm = 1.0 / math.sqrt(d)
    for b in range(B):
        n = int(cl[b])
        ref = O.attend_one(q[b], kst[rows[b, :n]], vst[rows[b, :n]], cp[b, :n], kl[b], vl[b], qpo, 1e6, sm)
        e = np.abs(g[b] - ref).max()
        assert e <= ATOL_ATTN["bf16"], f"b={b}: max-abs {e}"


def test_rope_table_values_and_reuse():
    rows, d, base = M.msa_rope_table_rows(2048, 8192, 16), 128, 1e6
    tab = M.msa_rope_table(rows, d, base, device=dev()).cpu().numpy().astype(np.float64)
    ang = O.rope_angles(np.arange(rows), d, base)               # float64 angles
    np.testing.assert_allclose(tab[..., 0], np.cos(ang), atol=1e-7, rtol=0)
    np.testing.assert_allclose(tab[..., 1], np.sin(ang), atol=1e-7, rtol=0)
    # a caller-built table gives the same bits as the per-call one
    B, T, Hq, Hkv, L_loc, qpo = 2, 1, 32, 8, 300, 16
    ctx = [77, 128]
    q, kl, vl, kc, vc, cp, cl = _attn_case(91, B, T, Hq, Hkv, d, L_loc, ctx, True, max(ctx))
    args = (to_dev(q, True), to_dev(kc, True), to_dev(vc, True), torch.from_numpy(cp).to(dev()),
            torch.from_numpy(cl).to(dev()), to_dev(kl, True), to_dev(vl, True), qpo)
    t2 = M.msa_rope_table(M.msa_rope_table_rows(max(ctx), L_loc, qpo), d, base, device=dev())
    a = M.msa_sparse_attn(*args)
    b = M.msa_sparse_attn(*args, rope_table=t2)
    assert torch.equal(a, b)
