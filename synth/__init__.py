"""Seeded synthetic inputs for the MSA routing + sparse-attention path.

This module generates inputs only.  It holds none of the method's arithmetic
(no pooling, normalisation, scoring, selection, RoPE or attention): it turns
(seed, stream, element index) into a value, lays out document lengths and
builds the planted "needle" documents that stand in for the pages' NIAH and
QA memories (no dataset item is reproduced).  Tests, the benchmark and the
CPU oracle's timing leg all draw their inputs from here, so the HIP path and
the oracle see bit-identical data.

Generator definition (shared with the device copy in ``synth_device.hip``):

* SplitMix64 finaliser (Steele, Lea & Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014)::

      mix(z) = z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
               z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31

* counter-based stream: ``base = mix(seed * GAMMA + stream)`` and the i-th
  word is ``mix(base + (i + 1) * GAMMA)`` (all arithmetic mod 2**64,
  ``GAMMA = 0x9E3779B97F4A7C15``).
* value: the four 16-bit lanes of the word are summed (Irwin-Hall, n = 4),
  centred by 131070 and scaled by the float32 constant 1/sqrt((2**32 - 1)/3)
  with one IEEE float32 multiply, optionally multiplied by an exact power of
  two, then rounded to bfloat16 with round-to-nearest-even when asked.  This
  is a unit-variance stand-in for N(0, 1), bounded by +-3.46.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
# 1/sqrt(4 * (65536**2 - 1) / 12): unit variance for the sum of four u16 lanes
NORMAL_SCALE = np.float32(2.6428997921303014e-05)
NORMAL_CENTRE = 131070

# tensor ids inside a (seed, layer) pair; stream = layer * 16 + tensor id
T_KR, T_K, T_V, T_QR, T_Q, T_KLOC, T_VLOC, T_NEEDLE, T_DOUT = range(9)


def stream_id(layer: int, tensor: int) -> int:
    return layer * 16 + tensor


def _mix_int(z: int) -> int:
    z &= MASK64
    z ^= z >> 30
    z = (z * M1) & MASK64
    z ^= z >> 27
    z = (z * M2) & MASK64
    z ^= z >> 31
    return z


def stream_base(seed: int, stream: int) -> int:
    return _mix_int(seed * GAMMA + stream)


def _mix_np(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(M1)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(M2)
    z = z ^ (z >> np.uint64(31))
    return z


def words(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """uint64 words ``start .. start+count-1`` of stream (seed, stream)."""
    base = np.uint64(stream_base(seed, stream))
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix_np(base + idx * np.uint64(GAMMA))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest even (finite input)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(seed: int, stream: int, start: int, count: int, *, scale_pow2: int = 0,
           bf16: bool = False, chunk: int = 1 << 22) -> np.ndarray:
    """float32 values of the stream; bf16-representable when ``bf16``."""
    out = np.empty(count, dtype=np.float32)
    mul = np.float32(2.0 ** scale_pow2)
    for s in range(0, count, chunk):
        n = min(chunk, count - s)
        w = words(seed, stream, start + s, n)
        m = np.uint64(0xFFFF)
        tot = ((w & m) + ((w >> np.uint64(16)) & m) + ((w >> np.uint64(32)) & m)
               + (w >> np.uint64(48))).astype(np.int64) - NORMAL_CENTRE
        v = tot.astype(np.float32) * NORMAL_SCALE
        if scale_pow2:
            v = v * mul
        if bf16:
            v = bf16_bits_to_f32(f32_to_bf16_bits(v))
        out[s:s + n] = v
    return out


def tensor(seed: int, layer: int, tensor_id: int, shape, *, bf16: bool,
           scale_pow2: int = 0, start: int = 0) -> np.ndarray:
    """A whole tensor of the stream (row-major flat index = element index)."""
    n = int(np.prod(shape))
    return normal(seed, stream_id(layer, tensor_id), start, n, bf16=bf16,
                  scale_pow2=scale_pow2).reshape(shape)


# --------------------------------------------------------------------------
# document lengths and needles
# --------------------------------------------------------------------------

def uniform_lengths(n_docs: int, length: int) -> np.ndarray:
    return np.full(n_docs, length, dtype=np.int64)


def lognormal_lengths(total: int, median: float, sigma: float, lo: int, hi: int,
                      seed: int) -> np.ndarray:
    """Lengths drawn lognormal(median, sigma), clipped to [lo, hi], until they
    sum to ``total`` (the last one truncated).  Host-side only."""
    rng = np.random.default_rng(seed)
    out = []
    acc = 0
    while acc < total:
        draw = rng.lognormal(mean=np.log(median), sigma=sigma, size=4096)
        for v in np.clip(np.rint(draw), lo, hi).astype(np.int64):
            v = int(min(v, total - acc))
            out.append(v)
            acc += v
            if acc >= total:
                break
    return np.asarray(out, dtype=np.int64)


def offsets(lengths: np.ndarray) -> np.ndarray:
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


def needle_docs(seed: int, n_docs: int, count: int, salt: int = 0) -> np.ndarray:
    """``count`` distinct document ids chosen by the seed."""
    rng = np.random.default_rng([seed, 77, salt])
    return np.sort(rng.choice(n_docs, size=count, replace=False)).astype(np.int64)


def needle_rows(q_r: np.ndarray, seed: int, layer: int, n_rows: int, noise: float = 0.1,
                bf16: bool = True, start: int = 0) -> np.ndarray:
    """Raw routing-key rows of a planted needle: mean over the query tokens of
    Q_r plus ``noise`` times generator noise, per head.  q_r: [T, H, d]."""
    T, H, d = q_r.shape
    mean = q_r.astype(np.float64).mean(axis=0)                     # [H, d]
    n = normal(seed, stream_id(layer, T_NEEDLE), start * H * d, n_rows * H * d)
    rows = mean[None] + noise * n.reshape(n_rows, H, d).astype(np.float64)
    rows = rows.astype(np.float32)
    if bf16:
        rows = bf16_bits_to_f32(f32_to_bf16_bits(rows))
    return rows
