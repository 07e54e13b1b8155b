"""msa_sparse_attn_indexed_noalloc (the attention entry point that allocates
nothing: its workspace is the library's own device array) gives the same
result, bit for bit, as msa_sparse_attn_indexed with a caller workspace, on
consecutive calls of decreasing size that reuse the array, and the oracle's
result within the attention tolerance."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.helpers import ATOL_ATTN, dev, gen, host, to_dev

pytestmark = pytest.mark.gpu

import sparse_attention_long_msa_amd as M  # noqa: E402  (a missing library fails loudly)


def _case(bf16, B, T, L_loc, ctx, seed, n_rows=3000, Hq=32, Hkv=8, d=128, qpo=16):
    max_ctx = max(max(ctx), 1)
    q = gen(seed, 0, synth.T_Q, (B, T, Hq, d), bf16)
    kl = gen(seed, 0, synth.T_KLOC, (B, L_loc, Hkv, d), bf16)
    vl = gen(seed, 0, synth.T_VLOC, (B, L_loc, Hkv, d), bf16)
    kst = gen(seed, 0, synth.T_K, (n_rows, Hkv, d), bf16, scale_pow2=-3)
    vst = gen(seed, 0, synth.T_V, (n_rows, Hkv, d), bf16, scale_pow2=-3)
    r = np.random.default_rng(seed)
    rows = r.integers(0, n_rows, size=(B, max_ctx)).astype(np.int32)
    cp = r.integers(0, min(128, max_ctx), size=(B, max_ctx)).astype(np.int32)
    cl = np.asarray(ctx, dtype=np.int32)
    host_in = dict(q=q, kl=kl, vl=vl, kst=kst, vst=vst, rows=rows, cp=cp, cl=cl, qpo=qpo, d=d)
    args = (to_dev(q, bf16), to_dev(kst, bf16), to_dev(vst, bf16), *(torch.from_numpy(a).to(dev()) for a in (rows, cp, cl)),
            to_dev(kl, bf16), to_dev(vl, bf16), qpo)
    return host_in, args


def _oracle_check(h, got, bf16, queries):
    g = host(got)
    sm = 1.0 / math.sqrt(h["d"])
    for b in queries:
        n = int(h["cl"][b])
        ref = O.attend_one(h["q"][b], h["kst"][h["rows"][b, :n]], h["vst"][h["rows"][b, :n]], h["cp"][b, :n],
                           h["kl"][b], h["vl"][b], h["qpo"], 1e6, sm)
        assert np.abs(g[b] - ref).max() <= ATOL_ATTN["bf16" if bf16 else "f32"]


def test_noalloc_matches_workspace_entry_on_consecutive_calls():
    # 1: batched decode with long contexts (split partials fill much of the array)
    h1, a1 = _case(True, 32, 1, 8192, list(np.random.default_rng(3).integers(1000, 2048, size=32)), 91)
    ref1 = M.msa_sparse_attn_indexed(*a1)
    got1 = M.msa_sparse_attn_indexed_noalloc(*a1)
    torch.cuda.synchronize()
    need1 = M.msa_sparse_attn_workspace(M.MSA_BF16, 32, 1, 32, 8, 128, a1[3].shape[1], 8192, 16)
    print(f"[noalloc] call 1: batched decode, workspace {need1} of {M.MSA_NOALLOC_SCRATCH_BYTES} bytes", flush=True)
    assert need1 <= M.MSA_NOALLOC_SCRATCH_BYTES
    assert torch.equal(got1, ref1)
    _oracle_check(h1, got1, True, [0, 31])
    # 2: a smaller prefill-shaped call reusing the array (its stale contents must not matter),
    #    with a caller RoPE table
    h2, a2 = _case(True, 2, 64, 300, [0, 700], 92)
    tab = M.msa_rope_table(M.msa_rope_table_rows(a2[3].shape[1], 300, 16), 128, device=dev())
    ref2 = M.msa_sparse_attn_indexed(*a2, rope_table=tab)
    got2 = M.msa_sparse_attn_indexed_noalloc(*a2, rope_table=tab)
    torch.cuda.synchronize()
    print("[noalloc] call 2: two 64-token queries", flush=True)
    assert torch.equal(got2, ref2)
    _oracle_check(h2, got2, True, [0, 1])
    # 3: float32 vector path, smaller still
    h3, a3 = _case(False, 1, 4, 8, [37], 93, n_rows=200)
    ref3 = M.msa_sparse_attn_indexed(*a3)
    got3 = M.msa_sparse_attn_indexed_noalloc(*a3)
    torch.cuda.synchronize()
    print("[noalloc] call 3: float32", flush=True)
    assert torch.equal(got3, ref3)
    _oracle_check(h3, got3, False, [0])


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    # 64 queries x 64 tokens: the split partials exceed the array; rejected on the host
    B, T, L_loc, max_ctx = 64, 64, 4096, 2048
    need = M.msa_sparse_attn_workspace(M.MSA_BF16, B, T, 32, 8, 128, max_ctx, L_loc, 16)
    assert need > M.MSA_NOALLOC_SCRATCH_BYTES
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device=dev())   # noqa: E731
    with pytest.raises(M.MsaError) as e:
        M.msa_sparse_attn_indexed_noalloc(z(B, T, 32, 128), z(100, 8, 128), z(100, 8, 128),
                                          z(B, max_ctx, dt=torch.int32), z(B, max_ctx, dt=torch.int32),
                                          z(B, dt=torch.int32), z(B, L_loc, 8, 128), z(B, L_loc, 8, 128), 16)
    assert e.value.status == 2 and "no-alloc" in str(e.value)
