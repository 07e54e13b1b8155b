"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every symbol include/msa.h declares, and rejects invalid calls with the
documented status before touching the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_long_msa_amd as M
from sparse_attention_long_msa_amd import _binding as MB

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    txt = open(os.path.join(ROOT, "include", "msa.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert len(syms) >= 13
    h = ctypes.CDLL(M.lib_path)
    for s in syms:
        assert hasattr(h, s), s


def test_abi_version_and_status_strings():
    assert M.msa_abi_version() == 14
    assert M.lib.msa_status_string(0).decode() == "ok"
    assert "workspace" in M.lib.msa_status_string(3).decode()


def test_chunk_offsets_host_matches_oracle():
    r = np.random.default_rng(0)
    lens = r.integers(0, 700, size=300)
    lens[::17] = 0
    tok_off = np.concatenate([[0], np.cumsum(lens)])
    for chunk in (1, 7, 64):
        np.testing.assert_array_equal(M.msa_chunk_offsets(tok_off, chunk), O.chunk_offsets(tok_off, chunk))


@pytest.mark.parametrize("bad", [[1, 5], [0, 5, 3]])
def test_chunk_offsets_rejects_bad_offsets(bad):
    with pytest.raises(M.MsaError) as e:
        M.msa_chunk_offsets(bad, 64)
    assert e.value.status == 1


P = ctypes.c_void_p(16)   # a non-null dummy; validation fails before any dereference
Q = ctypes.c_void_p(48)   # a second one, for outputs that must not alias an input


def test_route_score_validation():
    L = M.lib
    assert L.msa_route_score(1, None, 1, 1, 8, 128, P, 0, P, 4, 4, P, None, 0, 0, None) == 1
    assert L.msa_route_score(1, P, 0, 1, 8, 128, P, 0, P, 4, 4, P, None, 0, 0, None) == 1
    assert L.msa_route_score(7, P, 1, 1, 8, 128, P, 0, P, 4, 4, P, None, 0, 0, None) == 1
    assert L.msa_route_score(1, P, 1, 1, 8, 260, P, 0, P, 4, 4, P, None, 0, 0, None) == 2
    assert L.msa_route_score(1, P, 1, 1, 8, 128, P, 5, P, 4, 4, P, None, 0, 0, None) == 1     # bad layout
    assert L.msa_route_score(1, P, 1, 1, 4, 128, P, 1, P, 4, 4, P, P, 1 << 20, 0, None) == 2  # tiled off the MFMA path
    # float32 needs a workspace for the column norms
    need = L.msa_route_score_workspace(0, 1, 16, 8, 128, 4, 4)
    assert need >= 16 * 8 * 4
    assert L.msa_route_score(0, P, 1, 16, 8, 128, P, 0, P, 4, 4, P, P, need - 1, 0, None) == 3
    assert L.msa_route_score(1, P, 1, 1, 8, 128, P, 0, P, 4, 4, P, None, 0, 2, None) == 1   # unknown flag


def test_route_score_fetch_validation():
    L = M.lib
    ws = L.msa_route_score_fetch_workspace(1, 1, 64, 8, 128, 4, 4)
    assert ws >= 256
    base = [1, P, 1, 64, 8, 128, P, 1, P, 4, 4, P, P, ws, 0]
    fetch = [P, 1, 4, P, 4, 8, P, P, 8, 128, 32, P, P, P, P, None]
    bad = list(fetch)
    bad[0] = None                                                 # NULL selection
    assert L.msa_route_score_fetch(*base, *bad) == 1
    bad = list(fetch)
    bad[2] = 5                                                    # f_k > f_n_docs
    assert L.msa_route_score_fetch(*base, *bad) == 1
    bad = list(fetch)
    bad[10] = 31                                                  # f_max_ctx < f_k * f_max_doc_chunks
    assert L.msa_route_score_fetch(*base, *bad) == 1
    bad = list(fetch)
    bad[8], bad[9] = 1, 2                                         # a row of 4 bytes
    assert L.msa_route_score_fetch(*base, *bad) == 2
    small = list(base)
    small[13] = ws - 1
    assert L.msa_route_score_fetch(*small, *fetch) == 3
    flags = list(base)
    flags[14] = 4
    assert L.msa_route_score_fetch(*flags, *fetch) == 1


def test_topk_validation():
    L = M.lib
    assert L.msa_topk(P, 1, 10, 0, P, P, P, 1 << 20, 0, None) == 1
    assert L.msa_topk(P, 1, 10, 11, P, P, P, 1 << 20, 0, None) == 1
    assert L.msa_topk(P, 1, 1000, 300, P, P, P, 1 << 30, 0, None) == 2
    need = L.msa_topk_workspace(1, 100000, 16)
    assert need > 0
    assert L.msa_topk(P, 1, 100000, 16, P, P, P, need - 1, 0, None) == 3
    assert L.msa_topk_workspace(1, 4096, 16) == 0      # one slice: no workspace
    assert L.msa_topk(P, 1, 10, 4, P, P, P, 1 << 20, 2, None) == 1     # unknown flag
    assert L.msa_topk_context_index(P, 1, 10, 4, P, P, P, 8, 40, 32, P, P, P, P, 1 << 20, 2, None) == 1



def test_topk_merge_validation():
    L = M.lib
    assert L.msa_topk_merge(P, P, P, 2, 1, 8, 0, P, P, None) == 1          # k < 1
    assert L.msa_topk_merge(P, P, P, 2, 1, 8, 17, P, P, None) == 1         # k > G * k_in
    assert L.msa_topk_merge(P, P, P, 0, 1, 8, 4, P, P, None) == 1          # no shard
    assert L.msa_topk_merge(None, P, P, 2, 1, 8, 4, P, P, None) == 1       # NULL
    assert L.msa_topk_merge(P, P, P, 4, 1, 32, 65, P, P, None) == 2        # k > 64
    with pytest.raises(ValueError, match="vals: must be in device memory"):
        M.msa_topk_merge(torch.zeros((2, 1, 4)), torch.zeros((2, 1, 4), dtype=torch.int32),
                         torch.zeros(2, dtype=torch.int64), 4)

def test_gather_rejects_small_context_and_bad_mode():
    L = M.lib
    # max_ctx (31) < k * max_doc_chunks (32)
    assert L.msa_gather_kv(1, P, 2, 4, P, None, 10, 8, P, P, 80, 8, 128, 0, 31, P, P, P, P, None, None, None) == 1
    assert L.msa_gather_kv(1, P, 2, 4, P, None, 10, 8, P, P, 80, 8, 128, 9, 32, P, P, P, P, None, None, None) == 2
    assert L.msa_gather_kv(1, P, 2, 11, P, None, 10, 8, P, P, 80, 8, 128, 0, 88, P, P, P, P, None, None, None) == 1
    # host-memcpy mode needs the host offsets and the pinned id staging
    assert L.msa_gather_kv(1, P, 2, 4, P, None, 10, 8, P, P, 80, 8, 128, 2, 32, P, P, P, P, None, None, None) == 1


def test_interleave_validation():
    L = M.lib
    assert L.msa_exclude_docs(None, 1, 10, P, 1, 4, None) == 1
    assert L.msa_exclude_docs(P, 1, 10, None, 1, 4, None) == 1
    assert L.msa_exclude_docs(P, 0, 10, P, 1, 4, None) == 1
    assert L.msa_exclude_docs(P, 1, 10, None, 0, 4, None) == 0      # nothing to exclude: no launch
    #                          ids B  k  co n_docs maxdc n_chunks max_ctx row pos len_in len_out
    assert L.msa_context_append(P, 2, 4, P, 10, 8, 80, 32, P, P, P, P, None) == 1            # aliased lengths
    assert L.msa_context_append(P, 2, 4, P, 10, 8, 80, 31, P, P, P, ctypes.c_void_p(32), None) == 1
    assert L.msa_context_append(P, 2, 4, P, 10, 8, 80, 32, P, P, None, P, None) == 1


def test_training_path_validation():
    L = M.lib
    F = ctypes.c_float
    #                      dt q  B  T  H  d   kr chunk_doc n_docs n_chunks score ac at ws wsb stream
    assert L.msa_route_argmax(1, None, 1, 4, 8, 128, P, P, 10, 80, P, P, P, P, 1 << 30, None) == 1
    assert L.msa_route_argmax(1, P, 1, 4, 8, 128, P, P, 10, 80, P, P, P, P, 0, None) == 3          # workspace
    assert L.msa_route_argmax(1, P, 1, 4, 8, 512, P, P, 10, 80, P, P, P, P, 1 << 30, None) == 2    # d > 256
    assert L.msa_route_argmax(1, P, 1, 1 << 12, 8, 128, P, P, 10, 1 << 21, P, P, P, P, 1 << 40, None) == 2
    #                    score B n_docs pos n_pos tau loss grad stream
    assert L.msa_route_loss(P, 1, 10, P, 2, F(0.0), P, P, None) == 1      # tau <= 0
    assert L.msa_route_loss(P, 1, 10, None, 2, F(0.1), P, P, None) == 1
    assert L.msa_route_loss(P, 1, 10, P, 300, F(0.1), P, P, None) == 2    # n_pos > 256
    #                             dt q  B  T  H  d   kr n_chunks ac at grad n_docs dq dkr stream
    assert L.msa_route_score_backward(1, P, 1, 4, 8, 128, P, 80, P, P, P, 0, P, P, None) == 1
    assert L.msa_route_score_backward(1, P, 1, 4, 8, 128, P, 1 << 31, P, P, P, 10, P, P, None) == 2
    assert L.msa_route_score_backward(1, P, 1, 4, 8, 128, P, 80, P, P, P, 10, P, None, None) == 1
    #                      dt dy tok chunk_off chunk_doc n_docs n_tok n_chunks H d chunk x dx stream
    assert L.msa_pool_backward(1, P, P, P, P, 4, 100, 8, 8, 512, 64, None, P, None) == 2
    assert L.msa_pool_backward(1, P, P, P, P, 4, 100, 8, 8, 128, 0, None, P, None) == 1
    assert L.msa_pool_backward(1, None, P, P, P, 4, 100, 8, 8, 128, 64, None, P, None) == 1


def test_sparse_attn_backward_validation():
    L = M.lib
    F = ctypes.c_float

    def call(dk_bar=P, n_chunks=80, wsb=1 << 30, Hkv=8):
        return L.msa_sparse_attn_backward(1, P, 1, 16, 32, Hkv, 128, P, P, n_chunks, P, P, P, 32, P, P, 64, 4,
                                          F(1e6), None, 0, F(0.088), P, P, P, P, dk_bar, P, P, wsb, None)
    assert call(dk_bar=None) == 1
    assert call(n_chunks=0) == 1
    assert call(Hkv=7) == 1                         # Hq % Hkv != 0
    assert call(wsb=16) == 3
    assert M.msa_sparse_attn_backward_workspace(1, 1, 16, 32, 8, 128, 32, 64, 4) > 0


def test_context_index_validation():
    L = M.lib
    #            ids B  k  chunk_off n_docs maxdc n_chunks max_ctx row pos len stream
    assert L.msa_context_index(P, 2, 4, P, 10, 8, 80, 31, P, P, P, None) == 1      # max_ctx < k * max_doc_chunks
    assert L.msa_context_index(P, 2, 11, P, 10, 8, 80, 88, P, P, P, None) == 1     # k > n_docs
    assert L.msa_context_index(P, 2, 4, P, 10, 8, 80, 32, None, P, P, None) == 1   # NULL ctx_row
    assert L.msa_context_index(P, 2, 4, P, 10, 8, 1 << 31, 32, P, P, P, None) == 2  # int32 rows
    assert L.msa_context_index(P, 0, 4, P, 10, 8, 80, 32, P, P, P, None) == 1


def test_sparse_attn_indexed_validation():
    L = M.lib

    def call(n_chunks=80, row=P, Hq=32, q=P, wsb=1 << 30):
        return L.msa_sparse_attn_indexed(1, q, 1, 4, Hq, 8, 128, P, P, n_chunks, row, P, P, 16, P, P, 8, 4, 1e6,
                                         None, 0, 0.088, P, P, wsb, None)
    assert call(row=None) == 1
    assert call(n_chunks=0) == 1
    assert call(n_chunks=1 << 31) == 1
    assert call(Hq=30) == 1
    assert call(q=None) == 1
    assert call(wsb=16) == 3
    assert "msa_sparse_attn_indexed" in L.msa_last_error().decode()


def test_route_balance_validation():
    L = M.lib
    out = (ctypes.c_float * 8)()
    # rounds out of range
    assert L.msa_route_balance(1, P, 1, 64, 8, 128, P, 1, P, 4, 64, P, None, 0, -1, out, None) == 1
    assert L.msa_route_balance(1, P, 1, 64, 8, 128, P, 1, P, 4, 64, P, None, 0, 65, out, None) == 1
    assert "msa_route_balance" in L.msa_last_error().decode()


def test_sparse_attn_part_validation():
    L = M.lib

    def call(part=1, dtype=1, kc=None, cl=None, row=None, rows=0, wsb=1 << 30, d=128, out=None):
        return L.msa_sparse_attn_part(part, dtype, P, 1, 4, 32, 8, d, kc, kc, rows, row, cl, cl, 16, P, P, 8, 4,
                                      1e6, None, 0, 0.088, out, P, wsb, None)
    assert call(part=0) == 1 and call(part=3) == 1
    # the local part takes no context arguments: a NULL context passes validation
    assert call(part=1, wsb=16) == 3
    assert call(part=2) == 1                                  # the context part needs them
    assert call(part=2, kc=P, cl=P, row=P, rows=0, out=P) == 1    # ctx_rows with ctx_row
    assert call(part=2, kc=P, cl=P, wsb=16) == 1                  # ... and out
    assert call(part=2, kc=P, cl=P, wsb=16, out=P) == 3
    assert call(dtype=0) == 2                                 # float32: off the MFMA path
    assert call(d=64) == 2
    assert L.msa_sparse_attn_part_workspace(1, 1, 64, 32, 8, 128, 128, 4096, 16) > 0
    assert "msa_sparse_attn_part" in L.msa_last_error().decode()


def test_sparse_attn_validation():
    L = M.lib
    base = dict(dtype=1, q=P, B=1, T=4, Hq=32, Hkv=8, d=128, kc=P, vc=P, cp=P, cl=P, max_ctx=16, kl=P, vl=P,
                L=8, qpo=4, base=1e6, scale=0.088, out=P, ws=P, wsb=1 << 30, s=None)

    def call(**kw):
        a = dict(base, **kw)
        return L.msa_sparse_attn(a["dtype"], a["q"], a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["kc"], a["vc"],
                                 a["cp"], a["cl"], a["max_ctx"], a["kl"], a["vl"], a["L"], a["qpo"], a["base"],
                                 a.get("tab"), a.get("rows", 0), a["scale"], a["out"], a["ws"], a["wsb"], a["s"])
    assert call(Hq=30) == 1          # Hq % Hkv
    assert call(L=3) == 1            # L_loc < T
    assert call(d=127) == 1          # odd head dim
    assert call(qpo=-1) == 1
    assert call(d=512) == 2
    assert call(q=None) == 1
    assert call(wsb=16) == 3
    assert call(tab=P, rows=5) == 1  # caller table shorter than msa_rope_table_rows()
    assert L.msa_sparse_attn_workspace(1, 1, 4, 32, 8, 128, 16, 8, 4) > 0
    assert L.msa_rope_table_rows(2048, 8192, 16) == 8208
    assert L.msa_rope_table_rows(64, 1, 4) == 64
    assert L.msa_rope_table(0, 128, 1e6, P, None) == 1
    assert L.msa_rope_table(10, 128, 1.0, P, None) == 1


def test_pool_and_docmap_validation():
    L = M.lib
    assert L.msa_pool_encode(1, P, P, P, P, 4, 100, 8, 8, 128, 0, 1, 0, Q, None) == 1     # chunk 0
    assert L.msa_pool_encode(1, P, P, P, P, 4, 100, 8, 8, 127, 64, 1, 0, Q, None) == 1    # odd d
    assert L.msa_pool_encode(1, P, P, P, P, 4, 100, 8, 64, 128, 64, 1, 0, Q, None) == 2   # H*d > 4096
    assert L.msa_pool_encode(1, P, P, P, P, 4, 100, 8, 8, 48, 64, 1, 1, Q, None) == 1     # tiled needs d % 32
    assert L.msa_pool_encode(1, P, P, P, P, 4, 100, 8, 8, 128, 1, 1, 0, Q, None) == 1     # chunk 1: a chunk per token
    assert L.msa_pool_encode(1, P, P, P, P, 4, 100, 100, 8, 128, 1, 1, 0, P, None) == 1   # out aliases x
    assert L.msa_pool_encode(1, P, P, P, P, 4, 100, 8, 3, 64, 64, 1, 0, Q, None) == 2     # 24 vectors per row
    assert L.msa_pool_encode(1, P, P, P, P, 4, 100, 8, 16, 96, 64, 1, 0, Q, None) == 2    # 12 vectors per head
    assert L.msa_pool_encode(1, ctypes.c_void_p(8), P, P, P, 4, 100, 8, 8, 128, 64, 1, 0, Q, None) == 1  # x align
    assert L.msa_tile_routing_keys(1, P, 10, 8, 48, ctypes.c_void_p(32), None) == 1
    assert L.msa_tile_routing_keys(1, P, 10, 8, 128, P, None) == 1                     # aliased
    assert L.msa_chunk_doc_map(None, 4, 8, P, None) == 1
    assert L.msa_chunk_doc_map(P, 0, 8, P, None) == 1
    assert M.lib.msa_last_error().decode() != ""


# ---------------------------------------------------------------- binding-side operand checks
# The Python binding rejects operands that a kernel could not read correctly
# (host memory where device memory is required, pageable memory where the
# host tier needs pinned memory, strided views, wrong dtypes or shapes) with
# ValueError, before any pointer reaches the library.  On a machine without a
# GPU every CPU tensor is such an operand, so these run here.

def _cpu(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_binding_rejects_host_tensor_as_device_operand():
    q_r = _cpu((1, 4, 8, 128))
    kr = _cpu((32, 8, 128))
    cd = torch.zeros(32, dtype=torch.int32)
    with pytest.raises(ValueError, match="q_r: must be in device memory"):
        M.msa_route_score(q_r, kr, cd, 4)
    with pytest.raises(ValueError, match="q_r: must be in device memory"):
        M.msa_route_balance(q_r, kr, cd, 4)
    with pytest.raises(ValueError, match="q: must be in device memory"):
        M.msa_sparse_attn_part(M.MSA_ATTN_PART_LOCAL, _cpu((1, 4, 32, 128)), _cpu((1, 8, 8, 128)),
                               _cpu((1, 8, 8, 128)), 4, 16)
    with pytest.raises(ValueError, match="doc_score: must be in device memory"):
        M.msa_topk(torch.zeros((1, 10)), 4)
    with pytest.raises(ValueError, match="chunk_off: must be in device memory"):
        M.msa_chunk_doc_map(torch.zeros(5, dtype=torch.int64), 8)
    with pytest.raises(ValueError, match="x: must be in device memory"):
        M.msa_pool_encode(_cpu((100, 8, 128)), torch.zeros(5, dtype=torch.int64), torch.zeros(5, dtype=torch.int64),
                          cd, 64, True)
    with pytest.raises(ValueError, match="q: must be in device memory"):
        M.msa_sparse_attn(_cpu((1, 4, 32, 128)), _cpu((1, 16, 8, 128)), _cpu((1, 16, 8, 128)),
                          torch.zeros((1, 16), dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                          _cpu((1, 8, 8, 128)), _cpu((1, 8, 8, 128)), 4)
    with pytest.raises(ValueError, match="x: expected a torch tensor"):
        M.msa_encode(np.zeros((64, 256), np.float32), None, None, None, None, 64, 8, 128)


def test_binding_rejects_pageable_host_tier():
    ids = _cpu((1, 4), torch.int32)
    co = torch.zeros(11, dtype=torch.int64)
    kb = _cpu((80, 8, 128))
    for mode in (M.MSA_SRC_HOST_MAPPED, M.MSA_SRC_HOST_MEMCPY):
        # the device operands are checked first; with device-resident ids the
        # host-tier check comes next, which a pageable tensor fails the same way
        with pytest.raises(ValueError, match="(ids: must be in device memory|k_bar: must be in pinned host memory)"):
            M.msa_gather_kv(ids, co, kb, kb, 8, 32, src_mode=mode)
    with pytest.raises(ValueError, match="k_bar: must be in pinned host memory"):
        MB._pinned(kb, "k_bar")


def test_binding_rejects_strided_wrong_dtype_and_shape():
    t = torch.zeros((8, 16))
    with pytest.raises(ValueError, match="contiguous"):
        MB._layout(t.t(), "x", None, None)
    with pytest.raises(ValueError, match="dtype torch.float32, expected torch.int32"):
        MB._layout(t, "ids", torch.int32, None)
    with pytest.raises(ValueError, match=r"shape \(8, 16\), expected \(8, 8\)"):
        MB._layout(t, "out", torch.float32, (8, 8))
    MB._layout(t, "out", torch.float32, (8, None))          # None matches any extent
    with pytest.raises(ValueError, match="required"):
        MB._dev(None, "q")
    MB._dev(None, "ws", optional=True)
    with pytest.raises(ValueError, match="chunk_off_h"):
        MB._host_i64(np.zeros(4, np.int32), "chunk_off_h")
    MB._host_i64(np.zeros(4, np.int64), "chunk_off_h", 4)


def test_unfused_routing_validation():
    L = M.lib
    #                     dt q  B  T  H  d   kr layout n_chunks score ws wsb stream
    assert L.msa_chunk_scores(1, None, 1, 1, 8, 128, P, 0, 10, Q, None, 0, None) == 1
    assert L.msa_chunk_scores(1, P, 1, 1, 8, 128, P, 0, 0, Q, None, 0, None) == 1
    assert L.msa_chunk_scores(1, P, 1, 1, 8, 128, P, 0, 1 << 31, Q, None, 0, None) == 2
    assert L.msa_chunk_scores(0, P, 1, 16, 8, 128, P, 0, 10, Q, P, 8, None) == 3      # float32 needs norms
    #                    score B n_chunks chunk_off n_docs doc_score stream
    assert L.msa_segment_max(None, 1, 10, P, 4, Q, None) == 1
    assert L.msa_segment_max(P, 0, 10, P, 4, Q, None) == 1
    assert L.msa_segment_max(P, 1, 10, None, 4, Q, None) == 1
