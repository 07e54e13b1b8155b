"""The five workload presets (documents, chunking, query shapes, seeds).

Shapes follow the pages' workloads: QA memories of 277K-10M tokens and NIAH
up to 1M (the pages' Table 1 "Tokens" column and the RULER setup), and the
100M-token memory served by the Memory Parallel engine.  None of those
datasets is used; every value comes from the seeded generator in
``synth``.  Readings where the presets are silent are marked "reading".
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import lognormal_lengths, offsets, uniform_lengths


@dataclass
class Preset:
    name: str
    seed: int
    bf16: bool
    layers: int
    lengths: np.ndarray           # tokens per document
    chunk: int
    H: int                        # routing heads == KV heads
    d: int
    Hq: int
    B: int
    T: int
    L_loc: int
    k: int
    n_needles: int                # total planted needle docs
    needle_per_query: bool = False
    pooled_level: bool = False    # memory synthesised directly at pooled level
    rope_base: float = 1e6
    q_pos_offset: int | None = None   # defaults to k
    query_seed: int | None = None     # seed of the query-side streams; defaults to seed
    extra: dict = field(default_factory=dict)

    @property
    def n_docs(self) -> int:
        return int(len(self.lengths))

    @property
    def tok_off(self) -> np.ndarray:
        return offsets(self.lengths)

    @property
    def chunk_counts(self) -> np.ndarray:
        return (self.lengths + self.chunk - 1) // self.chunk

    @property
    def chunk_off(self) -> np.ndarray:
        return offsets(self.chunk_counts)

    @property
    def n_chunks(self) -> int:
        return int(self.chunk_counts.sum())

    @property
    def max_doc_chunks(self) -> int:
        return int(self.chunk_counts.max())

    @property
    def qseed(self) -> int:
        return self.seed if self.query_seed is None else self.query_seed

    @property
    def qpo(self) -> int:
        return self.k if self.q_pos_offset is None else self.q_pos_offset


def cfg1() -> Preset:
    """Tiny: 64 docs x 512 tokens, chunk 64 -> 512 chunks, fp32, 1 layer,
    16 query tokens (also the local KV), 32 query heads, k=4, one needle."""
    return Preset("cfg1", 1001, False, 1, uniform_lengths(64, 512), 64, 8, 128, 32,
                  1, 16, 16, 4, 1)


def cfg2() -> Preset:
    """1M tokens: 2048 docs x 512 tokens -> 16,384 chunks per layer, bf16,
    18 routed layers, 64 query tokens, 4,096 local tokens, k=16, 8 needles."""
    return Preset("cfg2", 1002, True, 18, uniform_lengths(2048, 512), 64, 8, 128, 32,
                  1, 64, 4096, 16, 8)


def cfg3_lengths() -> np.ndarray:
    # reading: lognormal sigma = 1.0 (the preset gives only the median)
    return lognormal_lengths(10_000_000, 600.0, 1.0, 64, 8192, seed=1003)


def cfg3() -> Preset:
    """10M tokens, lognormal document lengths (median 600, clipped 64-8192),
    ragged chunk counts, bf16, 18 layers, 128 query tokens, k=32.
    Readings: 4,096 local tokens, 32 query heads and 8 needles as in the
    1M-token preset."""
    return Preset("cfg3", 1003, True, 18, cfg3_lengths(), 64, 8, 128, 32,
                  1, 128, 4096, 32, 8)


def cfg4() -> Preset:
    """100M tokens: 195,312 docs x 512 tokens -> 1,562,496 chunks per layer,
    bf16, 18 layers; the routing-key store is ~57.6 GB.  Synthesised at
    pooled level (chunk means drawn directly; the raw 100M-token tensors
    would be ~11 TB).  Readings: 4,096 local tokens, 32 query heads, 8 needles."""
    return Preset("cfg4", 1004, True, 18, uniform_lengths(195_312, 512), 64, 8, 128, 32,
                  1, 64, 4096, 16, 8, pooled_level=True)


def cfg5() -> Preset:
    """Batched decode against the 10M-token memory: 32 queries x 1 token,
    each with its own 8,192-token local KV, k=16, one needle per query."""
    return Preset("cfg5", 1003, True, 18, cfg3_lengths(), 64, 8, 128, 32,
                  32, 1, 8192, 16, 32, needle_per_query=True, query_seed=1005)


def train64k() -> Preset:
    """Training-time workload (the pages' 64K-context fine-tuning stage):
    128 documents x 512 tokens = 65,536 memory tokens, chunk 64 -> 1,024
    pooled chunks per layer, bf16, 18 routed layers; 1,024 trained query
    tokens that are their own causal local window, 32 query heads, k = 16.
    Readings: the query length, the window and the 4 positive documents per
    query (the routing loss's positive set) are not given by the pages."""
    return Preset("train64k", 1006, True, 18, uniform_lengths(128, 512), 64, 8, 128, 32,
                  1, 1024, 1024, 16, 4)


PRESETS = {"cfg1": cfg1, "cfg2": cfg2, "cfg3": cfg3, "cfg4": cfg4, "cfg5": cfg5}
TRAIN_PRESETS = {"train64k": train64k}


def store_bytes(n_tokens: int, chunk: int, layers: int, heads: int, d: int,
                elem_bytes: int) -> int:
    """Bytes of the pooled routing-key store: one [chunks, heads, d] tensor
    per routed layer."""
    return (n_tokens // chunk) * layers * heads * d * elem_bytes
