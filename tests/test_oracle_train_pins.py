"""Pins of the oracle's training-time path (routing loss and backward).

Each function is pinned to something other than itself: central finite
differences of the oracle's own forward functions (which are pinned in
test_oracle_pins.py), library routines (torch's cross entropy with
probability targets, torch autograd through scaled-dot-product attention),
closed forms (the two-document loss is a softplus), adjoint identities of the
linear steps, and brute force on tiny inputs.
"""
import numpy as np
import pytest
import torch

import oracle as O


def rng(seed=0):
    return np.random.default_rng(seed)


def fd_grad(f, x, h=1e-6):
    """Central differences of the scalar function f at x (float64)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        x0 = x[i]
        x[i] = x0 + h
        fp = f(x)
        x[i] = x0 - h
        fm = f(x)
        x[i] = x0
        g[i] = (fp - fm) / (2 * h)
    return g


# ---------------------------------------------------------------- routing loss (R27)

def test_route_loss_is_cross_entropy_with_uniform_targets_on_the_positives():
    r = rng(1)
    B, D, tau = 3, 9, 0.07
    s = r.uniform(-1, 1, (B, D))
    pos = np.array([[2, -1, -1], [0, 5, 7], [8, 8, 1]])   # padding and a repeated id
    loss, grad = O.route_loss(s, pos, tau)
    target = np.zeros((B, D))
    for b, ps in enumerate(pos):
        ps = sorted({p for p in ps if p >= 0})
        target[b, ps] = 1.0 / len(ps)
    logits = torch.tensor(s / tau, dtype=torch.float64, requires_grad=True)
    ref = torch.nn.functional.cross_entropy(logits, torch.tensor(target), reduction="none")
    np.testing.assert_allclose(loss, ref.detach().numpy(), rtol=1e-13, atol=1e-13)
    ref.sum().backward()
    np.testing.assert_allclose(grad, logits.grad.numpy() / tau, rtol=1e-12, atol=1e-12)


def test_route_loss_two_documents_is_a_softplus():
    tau = 0.5
    for s0, s1 in [(0.3, -0.2), (-0.9, 0.95), (0.1, 0.1)]:
        loss, grad = O.route_loss(np.array([[s0, s1]]), np.array([[0]]), tau)
        z = (s1 - s0) / tau
        assert abs(loss[0] - math_softplus(z)) < 1e-14
        sig = 1.0 / (1.0 + np.exp(-z))
        np.testing.assert_allclose(grad[0], [-sig / tau, sig / tau], atol=1e-14)


def math_softplus(z):
    return float(np.log1p(np.exp(z)))


def test_route_loss_gradient_sums_to_zero_and_matches_finite_differences():
    r = rng(2)
    s = r.uniform(-1, 1, (2, 6))
    pos = np.array([[1, 4], [3, -1]])
    _, grad = O.route_loss(s, pos, 0.2)
    np.testing.assert_allclose(grad.sum(axis=1), 0.0, atol=1e-13)
    for b in range(2):
        fd = fd_grad(lambda x: O.route_loss(x[None], pos[b:b + 1], 0.2)[0][0], s[b].copy())
        np.testing.assert_allclose(grad[b], fd, atol=1e-8)


def test_route_loss_empty_documents_carry_no_weight():
    s = np.array([[0.4, -np.inf, 0.1, -np.inf, 0.7]])
    loss, grad = O.route_loss(s, np.array([[2]]), 0.3)
    loss2, grad2 = O.route_loss(s[:, [0, 2, 4]], np.array([[1]]), 0.3)
    assert abs(loss[0] - loss2[0]) < 1e-14
    assert grad[0, 1] == 0.0 and grad[0, 3] == 0.0
    np.testing.assert_allclose(grad[0, [0, 2, 4]], grad2[0], atol=1e-15)
    with pytest.raises(ValueError):
        O.route_loss(s, np.array([[-1]]), 0.3)


# ---------------------------------------------------------------- maximiser (R28)

def test_route_argmax_brute_force():
    r = rng(3)
    B, T, H, d = 2, 3, 2, 4
    co = np.array([0, 2, 2, 5, 6])                  # document 1 is empty
    N = 6
    q = r.normal(size=(B, T, H, d))
    kr = O.l2_normalize(r.normal(size=(N, H, d)))
    score, ac, at = O.route_argmax(q, kr, co)
    np.testing.assert_array_equal(score, O.route_scores(q, kr, co))
    for b in range(B):
        for i in range(4):
            lo, hi = co[i], co[i + 1]
            if lo == hi:
                assert ac[b, i] == -1 and at[b, i] == -1 and score[b, i] == -np.inf
                continue
            best, arg = -np.inf, None
            for c in range(lo, hi):
                for t in range(T):
                    v = 0.0
                    for h in range(H):
                        qq = q[b, t, h] / np.linalg.norm(q[b, t, h])
                        v += float(qq @ kr[c, h]) / H
                    if v > best:
                        best, arg = v, (c, t)
            assert (ac[b, i], at[b, i]) == arg
            assert abs(score[b, i] - best) < 1e-14


def test_route_argmax_ties_take_the_smallest_chunk_then_token():
    H, d = 1, 2
    kr = np.array([[[1.0, 0.0]], [[0.0, 1.0]], [[1.0, 0.0]]])       # chunks 0 and 2 equal
    q = np.array([[[[0.0, 1.0]], [[1.0, 0.0]], [[2.0, 0.0]]]])       # tokens 1 and 2 parallel
    score, ac, at = O.route_argmax(q, kr, np.array([0, 3]))
    assert score[0, 0] == 1.0 and (ac[0, 0], at[0, 0]) == (0, 1)
    score, ac, at = O.route_argmax(q, kr, np.array([0, 1, 3]))
    assert (ac[0, 1], at[0, 1]) == (1, 0)


# ---------------------------------------------------------------- normalisation (R29)

def test_normalize_backward_finite_differences_and_projection():
    r = rng(4)
    x = r.normal(size=(3, 5))
    dy = r.normal(size=(3, 5))
    dx = O.normalize_backward(x, dy)
    fd = fd_grad(lambda z: float((O.l2_normalize(z) * dy).sum()), x.copy())
    np.testing.assert_allclose(dx, fd, atol=1e-8)
    np.testing.assert_allclose((dx * x).sum(axis=1), 0.0, atol=1e-12)   # no radial part


def test_normalize_backward_below_eps_is_linear():
    x = np.array([[1e-9, -2e-9, 0.0]])
    dy = np.array([[0.5, 1.0, -2.0]])
    np.testing.assert_allclose(O.normalize_backward(x, dy), dy / 1e-8)


# ---------------------------------------------------------------- routing-score backward

def test_route_score_backward_matches_finite_differences():
    r = rng(5)
    B, T, H, d = 2, 3, 2, 4
    co = np.array([0, 2, 3, 3, 7])
    N = 7
    q = r.normal(size=(B, T, H, d))
    kr = O.l2_normalize(r.normal(size=(N, H, d)))
    g = r.normal(size=(B, 4))
    _, ac, at = O.route_argmax(q, kr, co)
    dq, dkr = O.route_score_backward(q, kr, ac, at, g)

    def f_q(x):
        s = O.route_scores(x, kr, co)
        return float(np.where(np.isfinite(s), g * s, 0.0).sum())

    def f_k(x):
        s = O.route_scores(q, x, co)
        return float(np.where(np.isfinite(s), g * s, 0.0).sum())

    np.testing.assert_allclose(dq, fd_grad(f_q, q.copy()), atol=1e-7)
    np.testing.assert_allclose(dkr, fd_grad(f_k, kr.copy()), atol=1e-7)


# ---------------------------------------------------------------- pooling adjoint

def test_pool_backward_is_the_adjoint_of_pool():
    r = rng(6)
    tok_off = np.array([0, 5, 5, 12, 13])
    chunk = 3
    x = r.normal(size=(13, 2, 3))
    n = len(O.pool(x, tok_off, chunk))
    y = r.normal(size=(n, 2, 3))
    lhs = float((O.pool(x, tok_off, chunk) * y).sum())
    rhs = float((x * O.pool_backward(y, tok_off, chunk)).sum())
    assert abs(lhs - rhs) < 1e-12


def test_pool_backward_through_the_normalisation_matches_finite_differences():
    r = rng(7)
    tok_off = np.array([0, 4, 9])
    chunk = 2
    x = r.normal(size=(9, 2, 3))
    n = len(O.pool(x, tok_off, chunk))
    y = r.normal(size=(n, 2, 3))
    dx = O.pool_backward(y, tok_off, chunk, x=x)
    fd = fd_grad(lambda z: float((O.l2_normalize(O.pool(z, tok_off, chunk)) * y).sum()), x.copy())
    np.testing.assert_allclose(dx, fd, atol=1e-8)


# ---------------------------------------------------------------- attention backward (R30)

def _attn_case(seed, T=3, Hq=4, Hkv=2, d=8, n_ctx=3, L_loc=5):
    r = rng(seed)
    return (r.normal(size=(T, Hq, d)), r.normal(size=(n_ctx, Hkv, d)), r.normal(size=(n_ctx, Hkv, d)),
            np.array([0, 1, 0][:n_ctx]), r.normal(size=(L_loc, Hkv, d)), r.normal(size=(L_loc, Hkv, d)),
            r.normal(size=(T, Hq, d)))


def test_attention_backward_matches_finite_differences():
    q, kc, vc, pc, kl, vl, dout = _attn_case(8)
    qpo, base, sc = 4, 100.0, 0.4
    grads = O.attend_one_backward(q, kc, vc, pc, kl, vl, qpo, base, sc, dout)
    args = [q, kc, vc, kl, vl]
    for which, gr in zip(range(5), [grads[0], grads[1], grads[2], grads[3], grads[4]]):
        def f(x, which=which):
            a = list(args)
            a[which] = x
            return float((O.attend_one(a[0], a[1], a[2], pc, a[3], a[4], qpo, base, sc) * dout).sum())
        np.testing.assert_allclose(gr, fd_grad(f, args[which].copy()), atol=1e-7)


def test_attention_backward_matches_torch_autograd_in_rotated_space():
    """The softmax part against torch's scaled-dot-product attention in float64:
    the oracle's gradients, rotated forward, are the gradients with respect to
    the rotated operands."""
    q, kc, vc, pc, kl, vl, dout = _attn_case(9, T=4, Hq=4, Hkv=2, d=8, n_ctx=2, L_loc=6)
    qpo, base = 2, 1e4
    T, Hq, d = q.shape
    L_loc, Hkv = kl.shape[:2]
    sc = 1.0 / np.sqrt(d)
    dq, dkc, dvc, dkl, dvl = O.attend_one_backward(q, kc, vc, pc, kl, vl, qpo, base, sc, dout)
    n_ctx = kc.shape[0]
    pos_all = np.concatenate([pc, qpo + np.arange(L_loc)])
    q_pos = qpo + L_loc - T + np.arange(T)
    k_rot = O.rope(np.concatenate([kc, kl]), pos_all[:, None], base)
    q_rot = O.rope(q, q_pos[:, None], base)
    v_all = np.concatenate([vc, vl])
    G = Hq // Hkv
    Q = torch.tensor(q_rot.transpose(1, 0, 2), requires_grad=True)                        # [Hq, T, d]
    K = torch.tensor(np.repeat(k_rot, G, axis=1).transpose(1, 0, 2), requires_grad=True)  # [Hq, n, d]
    V = torch.tensor(np.repeat(v_all, G, axis=1).transpose(1, 0, 2), requires_grad=True)
    mask = np.ones((T, n_ctx + L_loc), dtype=bool)
    for t in range(T):
        mask[t, n_ctx + L_loc - T + t + 1:] = False
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=torch.tensor(mask))
    (out * torch.tensor(dout.transpose(1, 0, 2))).sum().backward()
    np.testing.assert_allclose(O.rope(dq, q_pos[:, None], base), Q.grad.numpy().transpose(1, 0, 2), atol=1e-12)
    dk_rot = K.grad.numpy().reshape(Hkv, G, -1, d).sum(axis=1).transpose(1, 0, 2)
    dv = V.grad.numpy().reshape(Hkv, G, -1, d).sum(axis=1).transpose(1, 0, 2)
    np.testing.assert_allclose(O.rope(np.concatenate([dkc, dkl]), pos_all[:, None], base), dk_rot, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([dvc, dvl]), dv, atol=1e-12)


def test_gather_backward_is_the_adjoint_of_gather():
    r = rng(10)
    co = np.array([0, 2, 5, 6, 9])
    N = 9
    kb = r.normal(size=(N, 2, 3))
    vb = r.normal(size=(N, 2, 3))
    ids = np.array([[3, 0], [0, 2]])
    ctx = [O.gather(ids[b], co, kb, vb) for b in range(2)]
    ys = [(r.normal(size=c[0].shape), r.normal(size=c[1].shape)) for c in ctx]
    dkb, dvb = O.gather_backward(ids, co, ys, N)
    lhs = sum(float((c[0] * y[0]).sum() + (c[1] * y[1]).sum()) for c, y in zip(ctx, ys))
    rhs = float((kb * dkb).sum() + (vb * dvb).sum())
    assert abs(lhs - rhs) < 1e-12
