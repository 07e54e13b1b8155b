"""Shared helpers of the GPU parity tests: seeded inputs, uploads, and the
comparison rules (score tolerance, top-k tie band)."""
from __future__ import annotations

import numpy as np
import torch

import synth

BAND = 1e-4          # top-k tie band on oracle scores
RTOL_SCORE = {"f32": 1e-5, "bf16": 2e-3}
ATOL_ATTN = {"f32": 1e-3, "bf16": 1e-2}


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, bf16: bool) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return (t.to(torch.bfloat16) if bf16 else t).to(dev())


def to_dev_i64(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int64))).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy() if t.is_floating_point() else t.cpu().numpy()


def tile_np(x: np.ndarray) -> np.ndarray:
    """Row-major [N, H, d] -> the MSA_LAYOUT_TILED element order, padded with
    zero chunks to a multiple of 16; returned as [N_pad, H, d]-shaped storage."""
    N, H, d = x.shape
    n_pad = (N + 15) // 16 * 16
    xp = np.zeros((n_pad, H, d), dtype=x.dtype)
    xp[:N] = x
    t = xp.reshape(n_pad // 16, 16, H, d // 32, 4, 8).transpose(0, 2, 3, 4, 1, 5)
    return np.ascontiguousarray(t).reshape(n_pad, H, d)


def untile_np(t: np.ndarray, N: int) -> np.ndarray:
    n_pad, H, d = t.shape
    x = t.reshape(n_pad // 16, H, d // 32, 4, 16, 8).transpose(0, 4, 1, 2, 3, 5)
    return np.ascontiguousarray(x).reshape(n_pad, H, d)[:N]


def ragged_lengths(seed: int, n_docs: int, lo: int, hi: int, n_empty: int = 0) -> np.ndarray:
    r = np.random.default_rng(seed)
    lens = r.integers(lo, hi + 1, size=n_docs).astype(np.int64)
    if n_empty:
        lens[r.choice(n_docs, size=n_empty, replace=False)] = 0
    return lens


def gen(seed, layer, tensor, shape, bf16, scale_pow2=0):
    return synth.tensor(seed, layer, tensor, shape, bf16=bf16, scale_pow2=scale_pow2)


def check_scores(gpu: np.ndarray, ref: np.ndarray, rtol: float, k: int):
    """Normwise per query, and elementwise relative on the oracle's top 2k
    documents.  -inf (empty documents) must match exactly."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ref)), "empty-document pattern differs"
    fin = np.isfinite(ref)
    worst = 0.0
    for b in range(ref.shape[0]):
        f = fin[b]
        scale = np.abs(ref[b, f]).max()
        err = np.abs(gpu[b, f] - ref[b, f]).max() / scale
        worst = max(worst, err)
        assert err <= rtol, f"query {b}: normwise score error {err:.3g} > {rtol}"
        top = np.lexsort((np.arange(ref.shape[1]), -ref[b]))[: 2 * k]
        top = top[np.isfinite(ref[b, top])]
        rel = np.abs(gpu[b, top] - ref[b, top]) / np.maximum(np.abs(ref[b, top]), 1e-30)
        assert rel.max() <= rtol, f"query {b}: top-2k relative error {rel.max():.3g} > {rtol}"
    return worst


def check_ids(gpu_ids: np.ndarray, ref_scores: np.ndarray, k: int, band: float = BAND):
    """Top-k ids: exact outside the tie band; inside it, the GPU set holds
    every oracle id above the band and fills the rest from the band.  Returns
    True when the exact branch applied."""
    exact = True
    for b in range(ref_scores.shape[0]):
        s = np.asarray(ref_scores[b], np.float64)
        order = np.lexsort((np.arange(len(s)), -s))
        g = [int(x) for x in gpu_ids[b]]
        assert len(set(g)) == k, "duplicate ids"
        sk = s[order[k - 1]]
        sk1 = s[order[k]] if k < len(s) else -np.inf
        if sk - sk1 >= band:
            assert set(g) == set(order[:k].tolist()), f"query {b}: id set differs outside the tie band"
            # order: wherever adjacent oracle scores differ by >= band the ranks must agree
            for r in range(k - 1):
                assert s[g[r]] >= s[g[r + 1]] - band, f"query {b}: rank order differs at {r}"
            for r in range(k):
                if (r == 0 or s[order[r - 1]] - s[order[r]] >= band) and (
                        r == k - 1 or s[order[r]] - s[order[r + 1]] >= band):
                    assert g[r] == order[r], f"query {b}: rank {r} differs"
        else:
            exact = False
            above = set(np.nonzero(s >= sk + band)[0].tolist())
            in_band = set(np.nonzero(np.abs(s - sk) < band)[0].tolist())
            assert above <= set(g), f"query {b}: misses an id above the tie band"
            assert set(g) <= above | in_band, f"query {b}: id outside the tie band"
    return exact
