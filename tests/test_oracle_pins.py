"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test pins the oracle to something other than itself: a hand-worked
example, a closed form, a special case that reduces to a textbook or
library routine (scipy cosine, heapq selection, torch's scaled-dot-product
attention, complex multiplication), an invariant, or brute force on a tiny
input.  Every check is chosen so that a plausible slip in the oracle (a
dropped 1/H, a max and a mean swapped, a wrong RoPE sign or pairing, a
causal off-by-one, a transposed operand) fails at least one of them.
"""
import heapq
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import synth
from synth import configs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- worked example

def test_route_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "route_worked_example.json")))
    tok = np.array(g["tokens"], dtype=np.float64)
    tok_off = np.array(g["tok_off"])
    co = O.chunk_offsets(tok_off, g["chunk"])
    assert co.tolist() == g["expected_chunk_off"]
    kr = O.pool_encode(tok, tok_off, g["chunk"], True, "f32")
    np.testing.assert_allclose(kr, np.array(g["expected_pooled_kr"]), atol=1e-7)
    # routing on the exact (unrounded) pooled keys
    kr64 = O.l2_normalize(O.pool(tok, tok_off, g["chunk"]))
    s = O.route_scores(np.array(g["q_r"], dtype=np.float64), kr64, co)
    np.testing.assert_allclose(s, np.array(g["expected_doc_score"]), atol=1e-15)
    ids, vals = O.topk(s, 3)
    assert ids.tolist() == g["expected_top3_ids"]


def test_store_size_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "store_size.json")))
    b = configs.store_bytes(g["tokens"], g["chunk"], g["routed_layers"], g["heads"],
                            g["head_dim"], g["elem_bytes"])
    assert b == 57_600_000_000
    assert abs(b / 1e9 - g["pages_value_gb"]) / g["pages_value_gb"] < g["tolerance_rel"]
    for other in (32, 128):
        b2 = configs.store_bytes(g["tokens"], other, 18, 8, 128, 2)
        assert abs(b2 / 1e9 - 56.0) / 56.0 > g["tolerance_rel"]


# ---------------------------------------------------------------- pooling (P1)

def test_pool_constant_document():
    x = np.broadcast_to(rng().normal(size=(1, 3, 4)), (150, 3, 4)).copy()
    off = np.array([0, 150])
    p = O.pool(x, off, 64)
    assert p.shape == (3, 3, 4)
    np.testing.assert_allclose(p, np.broadcast_to(x[:1], p.shape), rtol=1e-14, atol=0)


def test_pool_chunk1_identity():
    x = rng(1).normal(size=(37, 2, 6))
    off = np.array([0, 5, 5, 20, 37])          # includes an empty document
    np.testing.assert_array_equal(O.pool(x, off, 1), x)
    assert O.chunk_offsets(off, 1).tolist() == [0, 5, 5, 20, 37]


def test_pool_arithmetic_sequence_midpoint():
    # x[tau] = a + b*tau pools to a + b * (first + last)/2 of each chunk, exactly
    a, b = 0.25, 0.5
    n = 200
    tau = np.arange(n, dtype=np.float64)
    x = (a + b * tau)[:, None, None] * np.ones((1, 1, 2))
    off = np.array([0, n])
    p = O.pool(x, off, 64)
    starts = np.arange(0, n, 64)
    ends = np.minimum(starts + 64, n) - 1
    want = a + b * (starts + ends) / 2.0
    np.testing.assert_array_equal(p[:, 0, 0], want)


def test_pool_weighted_sum_and_partial_chunk():
    x = rng(2).normal(size=(130 + 7, 2, 3))
    off = np.array([0, 130, 137])
    p = O.pool(x, off, 64)
    co = O.chunk_offsets(off, 64)
    assert co.tolist() == [0, 3, 4]
    counts = np.array([64, 64, 2, 7])
    np.testing.assert_allclose((p * counts[:, None, None])[:3].sum(0), x[:130].sum(0), atol=1e-12)
    np.testing.assert_allclose(p[2], x[128:130].mean(0), atol=1e-15)   # partial last chunk
    np.testing.assert_allclose(p[3], x[130:137].mean(0), atol=1e-15)


def test_pool_matches_reshape_mean_uniform():
    x = rng(3).normal(size=(4 * 256, 3, 5))
    off = np.arange(0, 4 * 256 + 1, 256)
    p = O.pool(x, off, 64)
    np.testing.assert_allclose(p, x.reshape(16, 64, 3, 5).mean(axis=1), atol=1e-14)


# ---------------------------------------------------------------- normalisation (P2)

def test_normalize_unit_and_zero():
    x = rng(4).normal(size=(50, 8, 128))
    n = np.linalg.norm(O.l2_normalize(x), axis=-1)
    np.testing.assert_allclose(n, 1.0, atol=1e-15)
    z = O.l2_normalize(np.zeros((1, 1, 4)))
    assert np.all(z == 0)                       # R5: clamped norm, cosine 0


def test_cosine_rescale_invariance():
    r = rng(5)
    x = r.normal(size=(6 * 64, 4, 16))
    off = np.array([0, 64, 200, 384])
    q = r.normal(size=(2, 3, 4, 16))
    co = O.chunk_offsets(off, 64)
    base = O.route_scores(q, O.l2_normalize(O.pool(x, off, 64)), co)
    for alpha in (1e-3, 7.5, 1e4):
        s = O.route_scores(alpha * q, O.l2_normalize(O.pool(alpha * x, off, 64)), co)
        np.testing.assert_allclose(s, base, atol=1e-13)


# ---------------------------------------------------------------- scoring (P3-P6)

def test_score_single_head_is_textbook_cosine():
    from scipy.spatial.distance import cosine
    r = rng(6)
    keys = r.normal(size=(9, 1, 33))
    q = r.normal(size=(1, 1, 1, 33))
    co = np.arange(10)
    s = O.route_scores(q, O.l2_normalize(keys), co)
    want = [1.0 - cosine(q[0, 0, 0], keys[i, 0]) for i in range(9)]
    np.testing.assert_allclose(s[0], want, atol=1e-14)
    assert np.all(np.abs(s) <= 1 + 1e-15)


def test_score_identical_heads_equal_single_head():
    r = rng(7)
    k1 = r.normal(size=(12, 1, 16))
    q1 = r.normal(size=(1, 2, 1, 16))
    co = np.array([0, 5, 12])
    s1 = O.route_scores(q1, O.l2_normalize(k1), co)
    s8 = O.route_scores(np.repeat(q1, 8, axis=2), O.l2_normalize(np.repeat(k1, 8, axis=1)), co)
    np.testing.assert_allclose(s8, s1, atol=1e-14)


def test_score_brute_force_loop():
    r = rng(8)
    B, T, H, d, N = 2, 3, 2, 5, 7
    q = r.normal(size=(B, T, H, d))
    k = O.l2_normalize(r.normal(size=(N, H, d)))
    co = np.array([0, 3, 3, 7])                     # an empty document in the middle
    s = O.route_scores(q, k, co)
    for b in range(B):
        for i in range(3):
            best = -math.inf
            for c in range(co[i], co[i + 1]):
                for t in range(T):
                    acc = 0.0
                    for h in range(H):
                        qq = q[b, t, h]
                        acc += float(np.dot(qq, k[c, h]) / math.sqrt(float(np.dot(qq, qq))))
                    best = max(best, acc / H)
            assert s[b, i] == pytest.approx(best, abs=1e-14) if best > -math.inf else s[b, i] == -math.inf


def test_needle_identity_scores_one_and_ranks_first():
    r = rng(9)
    H, d = 8, 128
    q = r.normal(size=(1, 1, H, d))
    keys = O.l2_normalize(r.normal(size=(40, H, d)))
    keys[23] = O.l2_normalize(q[0, 0])
    co = np.arange(0, 41, 4)
    s = O.route_scores(q, keys, co)
    assert s[0, 5] == pytest.approx(1.0, abs=1e-15)
    ids, _ = O.topk(s, 3)
    assert ids[0, 0] == 5


def test_permutation_invariance():
    r = rng(10)
    q = r.normal(size=(1, 5, 4, 8))
    x = r.normal(size=(8 * 16, 4, 8))
    off = np.arange(0, 8 * 16 + 1, 16)
    co = O.chunk_offsets(off, 4)
    k = O.l2_normalize(O.pool(x, off, 4))
    base = O.route_scores(q, k, co)
    np.testing.assert_array_equal(O.route_scores(q[:, ::-1], k, co), base)
    kp = k.copy()
    for i in range(8):                             # reverse chunks inside each document
        kp[co[i]:co[i + 1]] = k[co[i]:co[i + 1]][::-1]
    np.testing.assert_array_equal(O.route_scores(q, kp, co), base)


# ---------------------------------------------------------------- top-k (P7)

def _heap_topk(scores, k):
    return [i for _, i in heapq.nlargest(k, ((s, -i) for i, s in enumerate(scores)))]


def test_topk_against_heapq_random_and_ties():
    r = rng(11)
    for trial in range(20):
        D = int(r.integers(1, 300))
        k = int(r.integers(1, D + 1))
        s = np.round(r.normal(size=(3, D)), 1)         # many exact ties
        s[0, r.integers(0, D, size=D // 3)] = -np.inf
        ids, vals = O.topk(s, k)
        for b in range(3):
            want = [-i for i in _heap_topk(s[b], k)]
            assert ids[b].tolist() == want
            np.testing.assert_array_equal(vals[b], s[b, want])


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        O.topk(np.zeros((1, 4)), 5)
    with pytest.raises(ValueError):
        O.topk(np.zeros((1, 4)), 0)



# ---------------------------------------------------------------- Memory Parallel merge

def _shard_bounds(r, D, G):
    """G contiguous document ranges covering [0, D) (some may be empty)."""
    cuts = np.sort(r.integers(0, D + 1, size=G - 1))
    return np.concatenate([[0], cuts, [D]]).astype(np.int64)


def test_topk_merge_of_shards_is_the_global_topk():
    """Per-shard top-k lists merged by (score desc, global id asc) give the
    top-k of the whole memory, ties included, whatever the shard boundaries;
    a shard with fewer than k documents pads with -1 / NaN."""
    r = rng(31)
    for trial in range(40):
        D = int(r.integers(1, 400))
        k = int(r.integers(1, min(D, 64) + 1))
        G = int(r.integers(1, 7))
        B = 2
        s = np.round(r.normal(size=(B, D)), 1)          # many exact ties, also across shards
        s[0, r.integers(0, D, size=D // 4)] = -np.inf
        bounds = _shard_bounds(r, D, G)
        vals = np.full((G, B, k), np.nan)
        ids = np.full((G, B, k), -1, dtype=np.int32)
        for g in range(G):
            lo, hi = int(bounds[g]), int(bounds[g + 1])
            if hi == lo:
                continue
            kk = min(k, hi - lo)
            gi, gv = O.topk(s[:, lo:hi], kk)
            ids[g, :, :kk], vals[g, :, :kk] = gi, gv
        mi, mv = O.topk_merge(vals, ids, bounds[:-1], k)
        wi, wv = O.topk(s, k)
        np.testing.assert_array_equal(mi, wi)
        np.testing.assert_array_equal(mv, wv)


def test_topk_merge_worked_cases():
    # equal scores in two shards: the smaller global id ranks first
    vals = np.array([[[0.5, 0.25]], [[0.5, 0.75]]])
    ids = np.array([[[3, 1]], [[0, 2]]], dtype=np.int32)
    mi, mv = O.topk_merge(vals, ids, np.array([0, 10]), 3)
    assert mi[0].tolist() == [12, 3, 10]
    assert mv[0].tolist() == [0.75, 0.5, 0.5]
    # empty slots (id -1 or NaN score) never rank; too few entries pad with -1 / NaN
    vals = np.array([[[1.0, np.nan]], [[2.0, 3.0]]])
    ids = np.array([[[0, 5]], [[-1, 4]]], dtype=np.int32)
    mi, mv = O.topk_merge(vals, ids, np.array([0, 100]), 3)
    assert mi[0].tolist() == [104, 0, -1]
    assert mv[0, :2].tolist() == [3.0, 1.0] and np.isnan(mv[0, 2])

# ---------------------------------------------------------------- gather (P9)

def test_gather_is_index_copy():
    r = rng(12)
    co = np.array([0, 3, 3, 8, 9])
    kb = r.normal(size=(9, 2, 4))
    vb = r.normal(size=(9, 2, 4))
    kc, vc, pc = O.gather(np.array([3, 0, 2]), co, kb, vb)
    idx = [8, 0, 1, 2, 3, 4, 5, 6, 7]
    np.testing.assert_array_equal(kc, kb[idx])
    np.testing.assert_array_equal(vc, vb[idx])
    assert pc.tolist() == [0, 0, 1, 2, 0, 1, 2, 3, 4]


# ---------------------------------------------------------------- RoPE (P10-P11)

def test_rope_zero_position_identity_and_norm():
    x = rng(13).normal(size=(5, 3, 16))
    np.testing.assert_array_equal(O.rope(x, np.zeros((5, 3)), 1e6), x)
    y = O.rope(x, np.arange(15).reshape(5, 3) * 97, 1e6)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)


def test_rope_d2_is_rotation_matrix():
    x = np.array([0.3, -1.7])
    for p in (0, 1, 5, 1234):
        c, s = math.cos(p), math.sin(p)                 # d=2: theta_0 = 1
        want = np.array([[c, -s], [s, c]]) @ x
        np.testing.assert_allclose(O.rope(x, np.array(p), 1e6), want, atol=1e-15)


def test_rope_matches_complex_rotation():
    r = rng(14)
    d, base = 128, 1e6
    x = r.normal(size=(7, d))
    pos = r.integers(0, 9000, size=7)
    z = x[:, : d // 2] + 1j * x[:, d // 2:]
    theta = base ** (-np.arange(d // 2) * 2.0 / d)
    w = z * np.exp(1j * pos[:, None] * theta)
    np.testing.assert_allclose(O.rope(x, pos, base), np.concatenate([w.real, w.imag], -1), atol=1e-12)


def test_rope_relative_position_identity():
    r = rng(15)
    q, k = r.normal(size=(2, 128))
    for m, n in ((0, 0), (3, 11), (8191, 5), (100, 4200)):
        lhs = np.dot(O.rope(q, np.array(m), 1e6), O.rope(k, np.array(n), 1e6))
        rhs = np.dot(q, O.rope(k, np.array(n - m), 1e6))
        assert lhs == pytest.approx(rhs, abs=1e-12)


# ---------------------------------------------------------------- attention (P12-P14)

def _case(seed, T=3, L=5, n_ctx=4, Hq=4, Hkv=2, d=8):
    r = rng(seed)
    return dict(q=r.normal(size=(T, Hq, d)), kc=r.normal(size=(n_ctx, Hkv, d)),
                vc=r.normal(size=(n_ctx, Hkv, d)), pc=r.integers(0, 3, size=n_ctx),
                kl=r.normal(size=(L, Hkv, d)), vl=r.normal(size=(L, Hkv, d)))


def test_attention_matches_torch_sdpa():
    import torch
    c = _case(16)
    T, Hq, d = c["q"].shape
    L, Hkv = c["kl"].shape[:2]
    n_ctx = c["kc"].shape[0]
    qpo, base = 4, 1e6
    out = O.attend_one(c["q"], c["kc"], c["vc"], c["pc"], c["kl"], c["vl"], qpo, base, 1 / math.sqrt(d))
    # library path: rotate with the complex form, expand GQA, boolean mask, torch SDPA in float64
    theta = base ** (-np.arange(d // 2) * 2.0 / d)

    def crot(x, p):
        z = x[..., : d // 2] + 1j * x[..., d // 2:]
        w = z * np.exp(1j * np.asarray(p)[..., None] * theta)
        return np.concatenate([w.real, w.imag], -1)

    pos_k = np.concatenate([c["pc"], qpo + np.arange(L)])
    k = crot(np.concatenate([c["kc"], c["kl"]]), pos_k[:, None])
    v = np.concatenate([c["vc"], c["vl"]])
    q = crot(c["q"], (qpo + L - T + np.arange(T))[:, None])
    G = Hq // Hkv
    kq = np.repeat(k, G, axis=1).transpose(1, 0, 2)
    vq = np.repeat(v, G, axis=1).transpose(1, 0, 2)
    mask = np.ones((T, n_ctx + L), dtype=bool)
    for t in range(T):
        mask[t, n_ctx + L - T + t + 1:] = False
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2).copy()), torch.from_numpy(kq.copy()),
        torch.from_numpy(vq.copy()), attn_mask=torch.from_numpy(mask))
    np.testing.assert_allclose(out, ref.numpy().transpose(1, 0, 2), atol=1e-12)


def test_attention_shift_invariance():
    c = _case(17)
    d = c["q"].shape[-1]
    a = O.attend_one(c["q"], c["kc"], c["vc"], c["pc"], c["kl"], c["vl"], 4, 1e6, 1 / math.sqrt(d))
    b = O.attend_one(c["q"], c["kc"], c["vc"], c["pc"] + 1000, c["kl"], c["vl"], 1004, 1e6, 1 / math.sqrt(d))
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_attention_single_visible_key_and_zero_query():
    r = rng(18)
    Hq, Hkv, d = 4, 2, 8
    kl = r.normal(size=(1, Hkv, d))
    vl = r.normal(size=(1, Hkv, d))
    empty = np.zeros((0, Hkv, d))
    q = r.normal(size=(1, Hq, d))
    out = O.attend_one(q, empty, empty, np.zeros(0, np.int64), kl, vl, 4, 1e6, 0.3)
    np.testing.assert_allclose(out, np.repeat(vl, 2, axis=1), atol=1e-15)
    # causal: with T = L = 3 and no context, token 0 sees only local 0
    kl3, vl3 = r.normal(size=(3, Hkv, d)), r.normal(size=(3, Hkv, d))
    out3 = O.attend_one(r.normal(size=(3, Hq, d)), empty, empty, np.zeros(0, np.int64),
                        kl3, vl3, 4, 1e6, 0.3)
    np.testing.assert_allclose(out3[0], np.repeat(vl3[:1], 2, axis=1)[0], atol=1e-15)
    # q = 0: every visible logit is 0 -> mean of the visible values
    c = _case(19)
    qz = np.zeros_like(c["q"])
    out = O.attend_one(qz, c["kc"], c["vc"], c["pc"], c["kl"], c["vl"], 4, 1e6, 0.3)
    T, L, n_ctx = qz.shape[0], c["kl"].shape[0], c["kc"].shape[0]
    for t in range(T):
        vis = np.concatenate([c["vc"], c["vl"][: L - T + t + 1]])
        np.testing.assert_allclose(out[t], np.repeat(vis.mean(0), 2, axis=0), atol=1e-14)


# ---------------------------------------------------------------- rounding (R18)

def test_round_to_bf16_matches_bit_rounding():
    r = rng(20)
    x = r.normal(size=10000).astype(np.float32)
    # reference: torch's float32 -> bfloat16 cast (round to nearest even)
    import torch
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_bf16(x.astype(np.float64)), want)
    # exact halfway cases go to even
    assert O.round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert O.round_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6


# ---------------------------------------------------------------- end to end (P8)

def test_planted_needle_is_rank_one_tiny():
    """The tiny preset's planted needle document (routing keys = query mean
    + 0.1 noise) must rank first, as the pages' NIAH retrieval implies."""
    p = configs.cfg1()
    H, d, T = p.H, p.d, p.T
    qr = synth.tensor(p.qseed, 0, synth.T_QR, (p.B, T, H, d), bf16=False)
    n_tok = int(p.lengths.sum())
    x = synth.tensor(p.seed, 0, synth.T_KR, (n_tok, H, d), bf16=False)
    nd = synth.needle_docs(p.seed, p.n_docs, p.n_needles)
    for doc in nd:
        lo, hi = p.tok_off[doc], p.tok_off[doc + 1]
        x[lo:hi] = synth.needle_rows(qr[0], p.seed, 0, hi - lo, bf16=False, start=lo)
    kr = O.pool_encode(x, p.tok_off, p.chunk, True, "f32")
    s = O.route_scores(qr, kr, p.chunk_off)
    ids, vals = O.topk(s, p.k)
    assert ids[0, 0] == nd[0]
    assert vals[0, 0] > vals[0, 1] + 0.1


# ---------------------------------------------------------------- Memory Interleave (R23-R26)

def _interleave_case(seed, n_docs=40, B=2, T=3, H=4, d=16, rounds=3, k=4):
    r = rng(seed)
    lens = r.integers(1, 6, size=n_docs)
    chunk_off = np.concatenate([[0], np.cumsum(lens)])
    N = int(chunk_off[-1])
    store = O.l2_normalize(r.standard_normal((N, H, d)))
    kb, vb = r.standard_normal((N, H, d)), r.standard_normal((N, H, d))
    qr = [r.standard_normal((B, T, H, d)) for _ in range(rounds)]
    q = r.standard_normal((B, T, 2 * H, d))
    kl, vl = r.standard_normal((B, 5, H, d)), r.standard_normal((B, 5, H, d))
    return qr, store, chunk_off, kb, vb, q, kl, vl


def test_interleave_same_query_each_round_equals_one_longer_ranking():
    """With one routing query reused in every round, the rounds' selections
    laid end to end are the top (rounds x k) of that query's ranking
    (heapq selection by (-score, id))."""
    qr, store, co, kb, vb, q, kl, vl = _interleave_case(1)
    rounds, k = 4, 5
    res = O.interleave([qr[0]] * rounds, store, co, kb, vb, k, q, kl, vl)
    s = O.route_scores(qr[0], store, co)
    for b in range(q.shape[0]):
        want = [i for _, i in heapq.nsmallest(rounds * k, [(-s[b, i], i) for i in range(s.shape[1])])]
        got = np.concatenate([rd["ids"][b] for rd in res["rounds"]]).tolist()
        assert got == want
        assert res["fetched"][b] == want


def test_interleave_rounds_match_iterative_argmax():
    """Each round picks, k times, the best document not yet fetched (a plain
    iterative argmax with the id tie-break); no document is fetched twice."""
    qr, store, co, kb, vb, q, kl, vl = _interleave_case(2)
    k = 4
    res = O.interleave(qr, store, co, kb, vb, k, q, kl, vl)
    for b in range(q.shape[0]):
        taken = set()
        for r, rd in enumerate(res["rounds"]):
            s = O.route_scores(qr[r], store, co)[b]
            for j in range(k):
                best = None
                for i in range(len(s)):
                    if i in taken:
                        continue
                    if best is None or s[i] > s[best]:
                        best = i
                assert rd["ids"][b, j] == best and rd["vals"][b, j] == s[best]
                taken.add(best)
        assert len(res["fetched"][b]) == len(set(res["fetched"][b])) == k * len(qr)


def test_interleave_pads_when_documents_run_out():
    s = np.array([[0.3, 0.9, -0.2, 0.5, 0.1]])
    ids, vals = O.topk_excluding(s, 3, [[1, 3, 0]])
    assert ids.tolist() == [[4, 2, -1]]
    assert vals[0, :2].tolist() == [0.1, -0.2] and np.isnan(vals[0, 2])
    # ties keep the id order; excluded ids outside [0, D) are ignored
    ids, _ = O.topk_excluding(np.array([[0.5, 0.5, 0.5, 0.7]]), 2, [[3, 99, -1]])
    assert ids.tolist() == [[0, 1]]


def test_interleave_context_is_round_then_rank_order_with_local_positions():
    """Document-wise positions restart at 0 for every fetched document, in
    the order the documents were fetched (worked by hand on a tiny index)."""
    co = np.array([0, 2, 5, 6, 9])                 # 4 documents of 2, 3, 1, 3 chunks
    N = 9
    kb = np.arange(N, dtype=np.float64).reshape(N, 1, 1).repeat(2, axis=2)
    out = O.gather(np.array([3, 0, 1]), co, kb, kb)
    assert out[0][:, 0, 0].tolist() == [6, 7, 8, 0, 1, 2, 3, 4]
    assert out[2].tolist() == [0, 1, 2, 0, 1, 0, 1, 2]


def test_interleave_one_round_is_the_single_layer():
    qr, store, co, kb, vb, q, kl, vl = _interleave_case(3)
    k = 6
    one = O.interleave(qr[:1], store, co, kb, vb, k, q, kl, vl)
    ref = O.layer(qr[0], store, co, kb, vb, k, q, kl, vl)
    assert np.array_equal(one["rounds"][0]["ids"], ref["ids"])
    assert np.abs(one["out"] - ref["out"]).max() < 1e-13


# ---------------------------------------------------------------- Stage 1 from hidden states (R32)

def test_encode_with_identity_projections_is_pool_encode():
    r = rng(21)
    H, d = 2, 3
    tok_off = np.array([0, 5, 5, 12])
    x = r.normal(size=(12, H * d))
    eye = np.eye(H * d)
    kb, vb, kr = O.encode(x, np.concatenate([eye, 2 * eye, eye]), tok_off, 4, H, d, "f32")
    xs = x.reshape(12, H, d)
    np.testing.assert_array_equal(kb, O.pool_encode(xs, tok_off, 4, False, "f32"))
    np.testing.assert_array_equal(vb, O.pool_encode(2 * xs, tok_off, 4, False, "f32"))
    np.testing.assert_array_equal(kr, O.pool_encode(xs, tok_off, 4, True, "f32"))


def test_encode_hand_worked():
    """One document of three tokens, chunk 2, hidden 2, one head of d = 2:
    W_k = [[1, 0], [1, 1]] (rows = features), W_v = 2 W_k, W_r = [[0, 1], [3, 0]]."""
    x = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    wk = np.array([[1.0, 0.0], [1.0, 1.0]])
    wt = np.concatenate([wk, 2 * wk, [[0.0, 1.0], [3.0, 0.0]]])
    kb, vb, kr = O.encode(x, wt, np.array([0, 3]), 2, 1, 2, "f32")
    # K per token: (1, 3), (3, 7), (5, 11); chunk means (2, 5) and (5, 11)
    np.testing.assert_array_equal(kb[:, 0], [[2.0, 5.0], [5.0, 11.0]])
    np.testing.assert_array_equal(vb[:, 0], [[4.0, 10.0], [10.0, 22.0]])
    # K_r per token: (2, 3), (4, 9), (6, 15); means (3, 6) -> /sqrt(45), (6, 15) -> /sqrt(261)
    np.testing.assert_allclose(kr[:, 0], [[3 / 45 ** 0.5, 6 / 45 ** 0.5], [6 / 261 ** 0.5, 15 / 261 ** 0.5]],
                               rtol=1e-7)


def test_encode_pool_commutes_with_the_projection():
    """The mean of projected tokens is the projection of the mean token: the
    identity the library's pool-then-project order rests on."""
    r = rng(22)
    H, d, hidden = 2, 4, 6
    tok_off = np.array([0, 7, 7, 20])
    x = r.normal(size=(20, hidden))
    w = r.normal(size=(3 * H * d, hidden))
    kb, vb, _ = O.encode(x, w, tok_off, 3, H, d, "f32")
    xb = O.pool(x[:, None, :], tok_off, 3)[:, 0, :]
    proj = xb @ w.T
    np.testing.assert_allclose(kb, O.round_to_f32(proj[:, :H * d].reshape(-1, H, d)), rtol=2e-7, atol=1e-12)
    np.testing.assert_allclose(vb, O.round_to_f32(proj[:, H * d:2 * H * d].reshape(-1, H, d)), rtol=2e-7,
                               atol=1e-12)
