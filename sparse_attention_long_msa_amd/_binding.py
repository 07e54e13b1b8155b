"""ctypes binding of libmsa.so.  Same names as the C ABI; each function only
marshals torch tensors / numpy arrays into pointers and sizes, allocates
outputs and workspaces with torch when the caller passes none, and raises
MsaError on a non-OK status."""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmsa.so")

MSA_F32, MSA_BF16 = 0, 1
MSA_SRC_DEVICE, MSA_SRC_HOST_MAPPED, MSA_SRC_HOST_MEMCPY = 0, 1, 2
MSA_LAYOUT_ROWS, MSA_LAYOUT_TILED = 0, 1

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_F = ctypes.c_float
_S = ctypes.c_size_t

_SIGS = {
    "msa_abi_version": (_I, []),
    "msa_status_string": (ctypes.c_char_p, [_I]),
    "msa_last_error": (ctypes.c_char_p, []),
    "msa_chunk_offsets": (_I, [_P, _L, _I, _P]),
    "msa_chunk_doc_map": (_I, [_P, _L, _L, _P, _P]),
    "msa_tile_routing_keys": (_I, [_I, _P, _L, _I, _I, _P, _P]),
    "msa_pool_encode": (_I, [_I, _P, _P, _P, _P, _L, _L, _L, _I, _I, _I, _I, _I, _P, _P]),
    "msa_route_score_workspace": (_S, [_I, _I, _I, _I, _I, _L, _L]),
    "msa_route_score": (_I, [_I, _P, _I, _I, _I, _I, _P, _I, _P, _L, _L, _P, _P, _S, _P]),
    "msa_topk_workspace": (_S, [_I, _L, _I]),
    "msa_topk": (_I, [_P, _I, _L, _I, _P, _P, _P, _S, _P]),
    "msa_gather_kv": (_I, [_I, _P, _I, _I, _P, _P, _L, _I, _P, _P, _L, _I, _I, _I, _I,
                           _P, _P, _P, _P, _P, _P, _P]),
    "msa_context_index": (_I, [_P, _I, _I, _P, _L, _I, _L, _I, _P, _P, _P, _P]),
    "msa_topk_context_index": (_I, [_P, _I, _L, _I, _P, _P, _P, _I, _L, _I, _P, _P, _P, _P, _S, _P]),
    "msa_exclude_docs": (_I, [_P, _I, _L, _P, _I, _I, _P]),
    "msa_context_append": (_I, [_P, _I, _I, _P, _L, _I, _L, _I, _P, _P, _P, _P, _P]),
    "msa_sparse_attn_workspace": (_S, [_I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "msa_sparse_attn": (_I, [_I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _I, _I,
                             _F, _P, _I, _F, _P, _P, _S, _P]),
    "msa_sparse_attn_indexed": (_I, [_I, _P, _I, _I, _I, _I, _I, _P, _P, _L, _P, _P, _P, _I, _P, _P, _I, _I,
                                     _F, _P, _I, _F, _P, _P, _S, _P]),
    "msa_rope_table_rows": (_I, [_I, _I, _I]),
    "msa_rope_table": (_I, [_I, _I, _F, _P, _P]),
    "msa_route_argmax_workspace": (_S, [_I, _I, _I, _I, _I, _L, _L]),
    "msa_route_argmax": (_I, [_I, _P, _I, _I, _I, _I, _P, _P, _L, _L, _P, _P, _P, _P, _S, _P]),
    "msa_route_loss": (_I, [_P, _I, _L, _P, _I, _F, _P, _P, _P]),
    "msa_route_score_backward": (_I, [_I, _P, _I, _I, _I, _I, _P, _L, _P, _P, _P, _L, _P, _P, _P]),
    "msa_pool_backward": (_I, [_I, _P, _P, _P, _P, _L, _L, _L, _I, _I, _I, _P, _P, _P]),
    "msa_encode_workspace": (_S, [_I, _L, _I, _I, _I]),
    "msa_encode": (_I, [_I, _P, _P, _I, _I, _I, _P, _P, _P, _L, _L, _L, _I, _I, _P, _P, _P, _P, _S, _P]),
    "msa_sparse_attn_backward_workspace": (_S, [_I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "msa_sparse_attn_backward": (_I, [_I, _P, _I, _I, _I, _I, _I, _P, _P, _L, _P, _P, _P, _I, _P, _P, _I, _I,
                                      _F, _P, _I, _F, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
}


class MsaError(RuntimeError):
    def __init__(self, name, status, detail):
        super().__init__(f"{name} failed: status {status} ({_status_string(status)}): {detail}")
        self.status = status


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is not built: run `python sparse_attention_long_msa_amd/build.py`")
    h = ctypes.CDLL(lib_path)
    for name, (res, args) in _SIGS.items():
        try:
            f = getattr(h, name)
        except AttributeError as e:
            raise ImportError(f"{lib_path} lacks {name}: rebuild with `python sparse_attention_long_msa_amd/build.py`") from e
        f.restype = res
        f.argtypes = args
    return h


lib = _load()


def _status_string(s):
    return lib.msa_status_string(s).decode()


def _check(name, rc):
    if rc != 0:
        raise MsaError(name, rc, lib.msa_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return s.cuda_stream if hasattr(s, "cuda_stream") else s


def _dtype(t):
    if t.dtype == torch.float32:
        return MSA_F32
    if t.dtype == torch.bfloat16:
        return MSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ws(nbytes, device, ws):
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def msa_abi_version():
    return lib.msa_abi_version()


def msa_chunk_offsets(tok_off, chunk):
    tok_off = np.ascontiguousarray(np.asarray(tok_off, dtype=np.int64))
    out = np.empty_like(tok_off)
    _check("msa_chunk_offsets", lib.msa_chunk_offsets(_ptr(tok_off), len(tok_off) - 1, chunk, _ptr(out)))
    return out


def msa_chunk_doc_map(chunk_off, n_chunks, chunk_doc=None, stream=None):
    if chunk_doc is None:
        chunk_doc = torch.empty(n_chunks, dtype=torch.int32, device=chunk_off.device)
    _check("msa_chunk_doc_map", lib.msa_chunk_doc_map(_ptr(chunk_off), chunk_off.numel() - 1, n_chunks,
                                                      _ptr(chunk_doc), _stream(stream)))
    return chunk_doc


def padded_chunks(n_chunks, layout):
    """Rows a store of n_chunks chunks occupies in the given layout."""
    return (n_chunks + 15) // 16 * 16 if layout == MSA_LAYOUT_TILED else n_chunks


def msa_tile_routing_keys(src, out=None, stream=None):
    n_chunks, H, d = src.shape
    if out is None:
        out = torch.empty((padded_chunks(n_chunks, MSA_LAYOUT_TILED), H, d), dtype=src.dtype, device=src.device)
    _check("msa_tile_routing_keys", lib.msa_tile_routing_keys(_dtype(src), _ptr(src), n_chunks, H, d, _ptr(out),
                                                              _stream(stream)))
    return out


def msa_pool_encode(x, tok_off, chunk_off, chunk_doc, chunk, l2_normalize, out=None, layout=MSA_LAYOUT_ROWS,
                    stream=None):
    n_tok, H, d = x.shape
    n_chunks = chunk_doc.numel()
    if out is None:
        out = torch.empty((padded_chunks(n_chunks, layout), H, d), dtype=x.dtype, device=x.device)
    _check("msa_pool_encode", lib.msa_pool_encode(
        _dtype(x), _ptr(x), _ptr(tok_off), _ptr(chunk_off), _ptr(chunk_doc), tok_off.numel() - 1, n_tok,
        n_chunks, H, d, chunk, int(bool(l2_normalize)), layout, _ptr(out), _stream(stream)))
    return out


def msa_route_score_workspace(dtype, B, T, H, d, n_docs, n_chunks):
    return lib.msa_route_score_workspace(dtype, B, T, H, d, n_docs, n_chunks)


def msa_route_score(q_r, kr_hat, chunk_doc, n_docs, doc_score=None, ws=None, layout=MSA_LAYOUT_ROWS, stream=None):
    B, T, H, d = q_r.shape
    n_chunks = chunk_doc.numel()
    if kr_hat.shape[0] < padded_chunks(n_chunks, layout):
        raise ValueError("kr_hat holds fewer chunks than chunk_doc names")
    dt = _dtype(q_r)
    if doc_score is None:
        doc_score = torch.empty((B, n_docs), dtype=torch.float32, device=q_r.device)
    ws, wsb = _ws(msa_route_score_workspace(dt, B, T, H, d, n_docs, n_chunks), q_r.device, ws)
    _check("msa_route_score", lib.msa_route_score(
        dt, _ptr(q_r), B, T, H, d, _ptr(kr_hat), layout, _ptr(chunk_doc), n_docs, n_chunks, _ptr(doc_score),
        _ptr(ws), wsb, _stream(stream)))
    return doc_score


def msa_topk_workspace(B, n_docs, k):
    return lib.msa_topk_workspace(B, n_docs, k)


def msa_topk(doc_score, k, ids=None, vals=None, ws=None, stream=None):
    B, n_docs = doc_score.shape
    if ids is None:
        ids = torch.empty((B, k), dtype=torch.int32, device=doc_score.device)
    if vals is None:
        vals = torch.empty((B, k), dtype=torch.float32, device=doc_score.device)
    ws, wsb = _ws(msa_topk_workspace(B, n_docs, k), doc_score.device, ws)
    _check("msa_topk", lib.msa_topk(_ptr(doc_score), B, n_docs, k, _ptr(ids), _ptr(vals), _ptr(ws), wsb,
                                    _stream(stream)))
    return ids, vals


def msa_gather_kv(ids, chunk_off, k_bar, v_bar, max_doc_chunks, max_ctx, src_mode=MSA_SRC_DEVICE,
                  chunk_off_h=None, k_ctx=None, v_ctx=None, ctx_pos=None, ctx_len=None, ids_h=None,
                  stream=None, copy_stream=None, device=None):
    B, k = ids.shape
    n_chunks, Hkv, d = k_bar.shape
    dev = device if device is not None else ids.device
    if k_ctx is None:
        k_ctx = torch.empty((B, max_ctx, Hkv, d), dtype=k_bar.dtype, device=dev)
    if v_ctx is None:
        v_ctx = torch.empty((B, max_ctx, Hkv, d), dtype=v_bar.dtype, device=dev)
    if ctx_pos is None:
        ctx_pos = torch.empty((B, max_ctx), dtype=torch.int32, device=dev)
    if ctx_len is None:
        ctx_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if src_mode == MSA_SRC_HOST_MEMCPY and ids_h is None:
        ids_h = torch.empty((B, k), dtype=torch.int32, pin_memory=True)
    _check("msa_gather_kv", lib.msa_gather_kv(
        _dtype(k_bar), _ptr(ids), B, k, _ptr(chunk_off), _ptr(chunk_off_h), chunk_off.numel() - 1,
        max_doc_chunks, _ptr(k_bar), _ptr(v_bar), n_chunks, Hkv, d, src_mode, max_ctx, _ptr(k_ctx),
        _ptr(v_ctx), _ptr(ctx_pos), _ptr(ctx_len), _ptr(ids_h), _stream(stream),
        None if copy_stream is None else _stream(copy_stream)))
    return k_ctx, v_ctx, ctx_pos, ctx_len


def msa_context_index(ids, chunk_off, n_chunks, max_doc_chunks, max_ctx, ctx_row=None, ctx_pos=None, ctx_len=None,
                      stream=None):
    B, k = ids.shape
    dev = ids.device
    if ctx_row is None:
        ctx_row = torch.empty((B, max_ctx), dtype=torch.int32, device=dev)
    if ctx_pos is None:
        ctx_pos = torch.empty((B, max_ctx), dtype=torch.int32, device=dev)
    if ctx_len is None:
        ctx_len = torch.empty((B,), dtype=torch.int32, device=dev)
    _check("msa_context_index", lib.msa_context_index(
        _ptr(ids), B, k, _ptr(chunk_off), chunk_off.numel() - 1, max_doc_chunks, n_chunks, max_ctx, _ptr(ctx_row),
        _ptr(ctx_pos), _ptr(ctx_len), _stream(stream)))
    return ctx_row, ctx_pos, ctx_len


def msa_topk_context_index(doc_score, k, chunk_off, n_chunks, max_doc_chunks, max_ctx, ids=None, vals=None,
                           ctx_row=None, ctx_pos=None, ctx_len=None, ws=None, stream=None):
    """msa_topk then msa_context_index on its ids, in one pass for k <= 64."""
    B, n_docs = doc_score.shape
    dev = doc_score.device
    if ids is None:
        ids = torch.empty((B, k), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((B, k), dtype=torch.float32, device=dev)
    if ctx_row is None:
        ctx_row = torch.empty((B, max_ctx), dtype=torch.int32, device=dev)
    if ctx_pos is None:
        ctx_pos = torch.empty((B, max_ctx), dtype=torch.int32, device=dev)
    if ctx_len is None:
        ctx_len = torch.empty((B,), dtype=torch.int32, device=dev)
    ws, wsb = _ws(msa_topk_workspace(B, n_docs, k), dev, ws)
    _check("msa_topk_context_index", lib.msa_topk_context_index(
        _ptr(doc_score), B, n_docs, k, _ptr(ids), _ptr(vals), _ptr(chunk_off), max_doc_chunks, n_chunks, max_ctx,
        _ptr(ctx_row), _ptr(ctx_pos), _ptr(ctx_len), _ptr(ws), wsb, _stream(stream)))
    return ids, vals, ctx_row, ctx_pos, ctx_len


def msa_exclude_docs(doc_score, ids_sets, stream=None):
    """ids_sets: [n_sets, B, k] int32 (earlier rounds' selections)."""
    B, n_docs = doc_score.shape
    n_sets, _, k = ids_sets.shape
    _check("msa_exclude_docs", lib.msa_exclude_docs(_ptr(doc_score), B, n_docs, _ptr(ids_sets) if n_sets else None,
                                                    n_sets, k, _stream(stream)))
    return doc_score


def msa_context_append(ids, chunk_off, n_chunks, max_doc_chunks, ctx_row, ctx_pos, ctx_len_in, ctx_len_out,
                       stream=None):
    B, k = ids.shape
    _check("msa_context_append", lib.msa_context_append(
        _ptr(ids), B, k, _ptr(chunk_off), chunk_off.numel() - 1, max_doc_chunks, n_chunks, ctx_row.shape[1],
        _ptr(ctx_row), _ptr(ctx_pos), _ptr(ctx_len_in), _ptr(ctx_len_out), _stream(stream)))
    return ctx_row, ctx_pos, ctx_len_out


def msa_sparse_attn_workspace(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset):
    return lib.msa_sparse_attn_workspace(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset)


def msa_rope_table_rows(max_ctx, L_loc, q_pos_offset):
    return lib.msa_rope_table_rows(max_ctx, L_loc, q_pos_offset)


def msa_rope_table(rows, d, rope_base=1e6, table=None, device=None, stream=None):
    if table is None:
        table = torch.empty((rows, d // 2, 2), dtype=torch.float32, device=device)
    _check("msa_rope_table", lib.msa_rope_table(rows, d, float(rope_base), _ptr(table), _stream(stream)))
    return table


def msa_sparse_attn(q, k_ctx, v_ctx, ctx_pos, ctx_len, k_loc, v_loc, q_pos_offset, rope_base=1e6,
                    sm_scale=None, out=None, ws=None, rope_table=None, stream=None):
    B, T, Hq, d = q.shape
    max_ctx, Hkv = k_ctx.shape[1], k_ctx.shape[2]
    L_loc = k_loc.shape[1]
    dt = _dtype(q)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, T, Hq, d), dtype=torch.float32, device=q.device)
    ws, wsb = _ws(msa_sparse_attn_workspace(dt, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset), q.device, ws)
    _check("msa_sparse_attn", lib.msa_sparse_attn(
        dt, _ptr(q), B, T, Hq, Hkv, d, _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_pos), _ptr(ctx_len), max_ctx,
        _ptr(k_loc), _ptr(v_loc), L_loc, q_pos_offset, float(rope_base), _ptr(rope_table),
        0 if rope_table is None else rope_table.shape[0], float(sm_scale), _ptr(out), _ptr(ws), wsb,
        _stream(stream)))
    return out


def msa_sparse_attn_indexed(q, k_bar, v_bar, ctx_row, ctx_pos, ctx_len, k_loc, v_loc, q_pos_offset, rope_base=1e6,
                            sm_scale=None, out=None, ws=None, rope_table=None, stream=None):
    B, T, Hq, d = q.shape
    n_chunks, Hkv = k_bar.shape[0], k_bar.shape[1]
    max_ctx = ctx_row.shape[1]
    L_loc = k_loc.shape[1]
    dt = _dtype(q)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, T, Hq, d), dtype=torch.float32, device=q.device)
    ws, wsb = _ws(msa_sparse_attn_workspace(dt, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset), q.device, ws)
    _check("msa_sparse_attn_indexed", lib.msa_sparse_attn_indexed(
        dt, _ptr(q), B, T, Hq, Hkv, d, _ptr(k_bar), _ptr(v_bar), n_chunks, _ptr(ctx_row), _ptr(ctx_pos),
        _ptr(ctx_len), max_ctx, _ptr(k_loc), _ptr(v_loc), L_loc, q_pos_offset, float(rope_base), _ptr(rope_table),
        0 if rope_table is None else rope_table.shape[0], float(sm_scale), _ptr(out), _ptr(ws), wsb,
        _stream(stream)))
    return out


# ---------------------------------------------------------------- training-time path

def msa_route_argmax_workspace(dtype, B, T, H, d, n_docs, n_chunks):
    return lib.msa_route_argmax_workspace(dtype, B, T, H, d, n_docs, n_chunks)


def msa_route_argmax(q_r, kr_hat, chunk_doc, n_docs, doc_score=None, arg_chunk=None, arg_tok=None, ws=None,
                     stream=None):
    B, T, H, d = q_r.shape
    n_chunks = chunk_doc.numel()
    if kr_hat.shape[0] < n_chunks:
        raise ValueError("kr_hat holds fewer chunks than chunk_doc names")
    dev = q_r.device
    dt = _dtype(q_r)
    if doc_score is None:
        doc_score = torch.empty((B, n_docs), dtype=torch.float32, device=dev)
    if arg_chunk is None:
        arg_chunk = torch.empty((B, n_docs), dtype=torch.int32, device=dev)
    if arg_tok is None:
        arg_tok = torch.empty((B, n_docs), dtype=torch.int32, device=dev)
    ws, wsb = _ws(msa_route_argmax_workspace(dt, B, T, H, d, n_docs, n_chunks), dev, ws)
    _check("msa_route_argmax", lib.msa_route_argmax(
        dt, _ptr(q_r), B, T, H, d, _ptr(kr_hat), _ptr(chunk_doc), n_docs, n_chunks, _ptr(doc_score),
        _ptr(arg_chunk), _ptr(arg_tok), _ptr(ws), wsb, _stream(stream)))
    return doc_score, arg_chunk, arg_tok


def msa_route_loss(doc_score, pos_ids, tau, loss=None, grad=None, stream=None):
    B, n_docs = doc_score.shape
    n_pos = pos_ids.shape[1]
    if loss is None:
        loss = torch.empty((B,), dtype=torch.float32, device=doc_score.device)
    if grad is None:
        grad = torch.empty_like(doc_score)
    _check("msa_route_loss", lib.msa_route_loss(_ptr(doc_score), B, n_docs, _ptr(pos_ids), n_pos, float(tau),
                                                _ptr(loss), _ptr(grad), _stream(stream)))
    return loss, grad


def msa_route_score_backward(q_r, kr_hat, arg_chunk, arg_tok, grad, dkr_hat, dq_r=None, stream=None):
    """dkr_hat [n_chunks, H, d] float32 is accumulated into (zero it first)."""
    B, T, H, d = q_r.shape
    n_chunks = dkr_hat.shape[0]
    n_docs = grad.shape[1]
    if dq_r is None:
        dq_r = torch.empty((B, T, H, d), dtype=torch.float32, device=q_r.device)
    _check("msa_route_score_backward", lib.msa_route_score_backward(
        _dtype(q_r), _ptr(q_r), B, T, H, d, _ptr(kr_hat), n_chunks, _ptr(arg_chunk), _ptr(arg_tok), _ptr(grad),
        n_docs, _ptr(dq_r), _ptr(dkr_hat), _stream(stream)))
    return dq_r, dkr_hat


def msa_pool_backward(dy, tok_off, chunk_off, chunk_doc, n_tok, chunk, x=None, dtype=None, dx=None, stream=None):
    """dx [n_tok, H, d] float32.  x (the token vectors, when the pooled entry
    was L2-normalised) sets the dtype; otherwise ``dtype`` (default bf16)."""
    n_chunks, H, d = dy.shape
    if dx is None:
        dx = torch.empty((n_tok, H, d), dtype=torch.float32, device=dy.device)
    dt = _dtype(x) if x is not None else (MSA_BF16 if dtype is None else dtype)
    _check("msa_pool_backward", lib.msa_pool_backward(
        dt, _ptr(dy), _ptr(tok_off), _ptr(chunk_off), _ptr(chunk_doc), tok_off.numel() - 1, n_tok, n_chunks, H, d,
        chunk, _ptr(x), _ptr(dx), _stream(stream)))
    return dx


def msa_sparse_attn_backward_workspace(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset):
    return lib.msa_sparse_attn_backward_workspace(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset)


def msa_sparse_attn_backward(q, k_bar, v_bar, ctx_row, ctx_pos, ctx_len, k_loc, v_loc, q_pos_offset, dout,
                             dk_bar, dv_bar, rope_base=1e6, sm_scale=None, rope_table=None, dq=None, dk_loc=None,
                             dv_loc=None, ws=None, stream=None):
    """Gradients of msa_sparse_attn_indexed.  dk_bar / dv_bar [n_chunks, Hkv, d]
    float32 are accumulated into (zero them first); dq, dk_loc, dv_loc are
    written.  Returns (dq, dk_loc, dv_loc, dk_bar, dv_bar)."""
    B, T, Hq, d = q.shape
    n_chunks, Hkv = k_bar.shape[0], k_bar.shape[1]
    max_ctx = ctx_row.shape[1]
    L_loc = k_loc.shape[1]
    dt = _dtype(q)
    dev_ = q.device
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if dq is None:
        dq = torch.empty((B, T, Hq, d), dtype=torch.float32, device=dev_)
    if dk_loc is None:
        dk_loc = torch.empty((B, L_loc, Hkv, d), dtype=torch.float32, device=dev_)
    if dv_loc is None:
        dv_loc = torch.empty((B, L_loc, Hkv, d), dtype=torch.float32, device=dev_)
    ws, wsb = _ws(msa_sparse_attn_backward_workspace(dt, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset), dev_, ws)
    _check("msa_sparse_attn_backward", lib.msa_sparse_attn_backward(
        dt, _ptr(q), B, T, Hq, Hkv, d, _ptr(k_bar), _ptr(v_bar), n_chunks, _ptr(ctx_row), _ptr(ctx_pos),
        _ptr(ctx_len), max_ctx, _ptr(k_loc), _ptr(v_loc), L_loc, q_pos_offset, float(rope_base), _ptr(rope_table),
        0 if rope_table is None else rope_table.shape[0], float(sm_scale), _ptr(dout), _ptr(dq), _ptr(dk_loc),
        _ptr(dv_loc), _ptr(dk_bar), _ptr(dv_bar), _ptr(ws), wsb, _stream(stream)))
    return dq, dk_loc, dv_loc, dk_bar, dv_bar


def msa_encode(x, w_t, tok_off, chunk_off, chunk_doc, chunk, H, d, kr_layout=MSA_LAYOUT_ROWS, k_bar=None,
               v_bar=None, kr_hat=None, ws=None, stream=None):
    """Stage 1 from hidden states: x [n_tok, hidden], w_t [3*H*d, hidden]
    (rows: K features, then V, then K_r).  Returns (k_bar, v_bar, kr_hat)."""
    n_tok, hidden = x.shape
    n_chunks = chunk_doc.numel()
    dt = _dtype(x)
    dev_ = x.device
    if k_bar is None:
        k_bar = torch.empty((n_chunks, H, d), dtype=x.dtype, device=dev_)
    if v_bar is None:
        v_bar = torch.empty((n_chunks, H, d), dtype=x.dtype, device=dev_)
    if kr_hat is None:
        kr_hat = torch.empty((padded_chunks(n_chunks, kr_layout), H, d), dtype=x.dtype, device=dev_)
    ws, wsb = _ws(lib.msa_encode_workspace(dt, n_chunks, hidden, H, d), dev_, ws)
    _check("msa_encode", lib.msa_encode(
        dt, _ptr(x), _ptr(w_t), hidden, H, d, _ptr(tok_off), _ptr(chunk_off), _ptr(chunk_doc), tok_off.numel() - 1,
        n_tok, n_chunks, chunk, kr_layout, _ptr(k_bar), _ptr(v_bar), _ptr(kr_hat), _ptr(ws), wsb, _stream(stream)))
    return k_bar, v_bar, kr_hat
