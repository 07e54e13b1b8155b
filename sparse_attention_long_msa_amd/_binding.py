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
MSA_ATTN_PART_LOCAL, MSA_ATTN_PART_CONTEXT = 1, 2
MSA_ROUTE_PREFILLED = 1
MSA_TOPK_RESET_SCORES = 1

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
    "msa_route_score": (_I, [_I, _P, _I, _I, _I, _I, _P, _I, _P, _L, _L, _P, _P, _S, _I, _P]),
    "msa_route_score_fetch_workspace": (_S, [_I, _I, _I, _I, _I, _L, _L]),
    "msa_route_score_fetch": (_I, [_I, _P, _I, _I, _I, _I, _P, _I, _P, _L, _L, _P, _P, _S, _I,
                                   _P, _I, _I, _P, _L, _I, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P]),
    "msa_route_balance": (_I, [_I, _P, _I, _I, _I, _I, _P, _I, _P, _L, _L, _P, _P, _S, _I, _P, _P]),
    "msa_chunk_scores": (_I, [_I, _P, _I, _I, _I, _I, _P, _I, _L, _P, _P, _S, _P]),
    "msa_segment_max": (_I, [_P, _I, _L, _P, _L, _P, _P]),
    "msa_topk_workspace": (_S, [_I, _L, _I]),
    "msa_topk": (_I, [_P, _I, _L, _I, _P, _P, _P, _S, _I, _P]),
    "msa_topk_merge": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "msa_gather_kv": (_I, [_I, _P, _I, _I, _P, _P, _L, _I, _P, _P, _L, _I, _I, _I, _I,
                           _P, _P, _P, _P, _P, _P, _P]),
    "msa_context_index": (_I, [_P, _I, _I, _P, _L, _I, _L, _I, _P, _P, _P, _P]),
    "msa_topk_context_index": (_I, [_P, _I, _L, _I, _P, _P, _P, _I, _L, _I, _P, _P, _P, _P, _S, _I, _P]),
    "msa_exclude_docs": (_I, [_P, _I, _L, _P, _I, _I, _P]),
    "msa_context_append": (_I, [_P, _I, _I, _P, _L, _I, _L, _I, _P, _P, _P, _P, _P]),
    "msa_sparse_attn_workspace": (_S, [_I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "msa_sparse_attn": (_I, [_I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _I, _I,
                             _F, _P, _I, _F, _P, _P, _S, _P]),
    "msa_sparse_attn_indexed": (_I, [_I, _P, _I, _I, _I, _I, _I, _P, _P, _L, _P, _P, _P, _I, _P, _P, _I, _I,
                                     _F, _P, _I, _F, _P, _P, _S, _P]),
    "msa_sparse_attn_indexed_noalloc": (_I, [_I, _P, _I, _I, _I, _I, _I, _P, _P, _L, _P, _P, _P, _I, _P, _P, _I,
                                             _I, _F, _P, _I, _F, _P, _P]),
    "msa_sparse_attn_part_workspace": (_S, [_I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "msa_sparse_attn_part": (_I, [_I, _I, _P, _I, _I, _I, _I, _I, _P, _P, _L, _P, _P, _P, _I, _P, _P, _I, _I,
                                  _F, _P, _I, _F, _P, _P, _S, _P]),
    "msa_rope_table_rows": (_I, [_I, _I, _I]),
    "msa_stream_read": (_I, [_P, _L, _P, _P]),
    "msa_rope_table": (_I, [_I, _I, _F, _P, _P]),
    "msa_route_argmax_workspace": (_S, [_I, _I, _I, _I, _I, _L, _L]),
    "msa_route_argmax": (_I, [_I, _P, _I, _I, _I, _I, _P, _P, _L, _L, _P, _P, _P, _P, _S, _P]),
    "msa_route_loss": (_I, [_P, _I, _L, _P, _I, _F, _P, _P, _P]),
    "msa_route_score_backward": (_I, [_I, _P, _I, _I, _I, _I, _P, _L, _P, _P, _P, _L, _P, _P, _P]),
    "msa_pool_backward": (_I, [_I, _P, _P, _P, _P, _L, _L, _L, _I, _I, _I, _P, _P, _P]),
    "msa_encode_workspace": (_S, [_I, _L, _I, _I, _I]),
    "msa_encode": (_I, [_I, _P, _P, _I, _I, _I, _P, _P, _P, _L, _L, _L, _I, _I, _P, _P, _P, _P, _S, _P]),
    "msa_encode_pool": (_I, [_I, _P, _I, _I, _I, _P, _P, _P, _L, _L, _L, _I, _P, _S, _P]),
    "msa_encode_project": (_I, [_I, _P, _I, _I, _I, _L, _I, _P, _P, _P, _P, _S, _P]),
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


def _fail(name, msg):
    raise ValueError(f"{name}: {msg}")


def _shape_ok(t, shape):
    return len(t.shape) == len(shape) and all(w is None or int(g) == int(w) for g, w in zip(t.shape, shape))


def _dev(t, name, dtype=None, shape=None, optional=False):
    """A device operand: a contiguous CUDA tensor (of the given dtype(s) and
    shape, None = any extent).  Checked before the pointer reaches a kernel:
    a host pointer or a strided view read by a kernel would fault the GPU or
    give wrong values without an error."""
    if t is None:
        if optional:
            return
        _fail(name, "required")
    if not isinstance(t, torch.Tensor):
        _fail(name, f"expected a torch tensor in device memory, got {type(t).__name__}")
    if not t.is_cuda:
        _fail(name, f"must be in device memory, got a tensor on {t.device}")
    _layout(t, name, dtype, shape)


def _store(t, name, dtype=None, shape=None):
    """A K/V store that attention reads in place: device memory, or pinned
    host memory, which the kernel then reads over the host link."""
    if isinstance(t, torch.Tensor) and not t.is_cuda:
        _pinned(t, name, dtype, shape)
    else:
        _dev(t, name, dtype, shape)


def _pinned(t, name, dtype=None, shape=None):
    """A host-tier operand that a kernel or an async copy reads: a contiguous
    tensor in pinned (page-locked) host memory."""
    if not isinstance(t, torch.Tensor):
        _fail(name, f"expected a torch tensor in pinned host memory, got {type(t).__name__}")
    if t.is_cuda or not t.is_pinned():
        _fail(name, f"must be in pinned host memory (torch pin_memory), got {'device' if t.is_cuda else 'pageable host'} memory")
    _layout(t, name, dtype, shape)


def _layout(t, name, dtype, shape):
    if not t.is_contiguous():
        _fail(name, "must be contiguous (a strided view would be read with the wrong strides)")
    if dtype is not None:
        ok = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in ok:
            _fail(name, f"dtype {t.dtype}, expected {' or '.join(str(x) for x in ok)}")
    if shape is not None and not _shape_ok(t, shape):
        _fail(name, f"shape {tuple(t.shape)}, expected {tuple('*' if w is None else w for w in shape)}")


def _host_i64(a, name, n=None):
    """Host int64 offsets (numpy)."""
    if not isinstance(a, np.ndarray) or a.dtype != np.int64 or a.ndim != 1 or not a.flags.c_contiguous:
        _fail(name, "expected a contiguous 1-D numpy int64 array")
    if n is not None and len(a) != n:
        _fail(name, f"length {len(a)}, expected {n}")


_FLOAT = (torch.float32, torch.bfloat16)
_I32, _I64, _F32 = torch.int32, torch.int64, torch.float32


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
    _dev(chunk_off, "chunk_off", _I64, (None,))
    if chunk_doc is None:
        chunk_doc = torch.empty(n_chunks, dtype=torch.int32, device=chunk_off.device)
    _dev(chunk_doc, "chunk_doc", _I32, (n_chunks,))
    _check("msa_chunk_doc_map", lib.msa_chunk_doc_map(_ptr(chunk_off), chunk_off.numel() - 1, n_chunks,
                                                      _ptr(chunk_doc), _stream(stream)))
    return chunk_doc


def padded_chunks(n_chunks, layout):
    """Rows a store of n_chunks chunks occupies in the given layout."""
    return (n_chunks + 15) // 16 * 16 if layout == MSA_LAYOUT_TILED else n_chunks


def msa_tile_routing_keys(src, out=None, stream=None):
    _dev(src, "src", _FLOAT, (None, None, None))
    n_chunks, H, d = src.shape
    if out is None:
        out = torch.empty((padded_chunks(n_chunks, MSA_LAYOUT_TILED), H, d), dtype=src.dtype, device=src.device)
    _dev(out, "out", src.dtype, (padded_chunks(n_chunks, MSA_LAYOUT_TILED), H, d))
    _check("msa_tile_routing_keys", lib.msa_tile_routing_keys(_dtype(src), _ptr(src), n_chunks, H, d, _ptr(out),
                                                              _stream(stream)))
    return out


def msa_pool_encode(x, tok_off, chunk_off, chunk_doc, chunk, l2_normalize, out=None, layout=MSA_LAYOUT_ROWS,
                    stream=None):
    _dev(x, "x", _FLOAT, (None, None, None))
    _dev(tok_off, "tok_off", _I64, (None,))
    _dev(chunk_off, "chunk_off", _I64, (tok_off.numel(),))
    _dev(chunk_doc, "chunk_doc", _I32, (None,))
    n_tok, H, d = x.shape
    n_chunks = chunk_doc.numel()
    if out is None:
        out = torch.empty((padded_chunks(n_chunks, layout), H, d), dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype, (padded_chunks(n_chunks, layout), H, d))
    _check("msa_pool_encode", lib.msa_pool_encode(
        _dtype(x), _ptr(x), _ptr(tok_off), _ptr(chunk_off), _ptr(chunk_doc), tok_off.numel() - 1, n_tok,
        n_chunks, H, d, chunk, int(bool(l2_normalize)), layout, _ptr(out), _stream(stream)))
    return out


def msa_route_score_workspace(dtype, B, T, H, d, n_docs, n_chunks):
    return lib.msa_route_score_workspace(dtype, B, T, H, d, n_docs, n_chunks)


def msa_route_score(q_r, kr_hat, chunk_doc, n_docs, doc_score=None, ws=None, layout=MSA_LAYOUT_ROWS, stream=None,
                    prefilled=False):
    """prefilled: doc_score already holds -inf everywhere (msa_topk with
    reset=True left it so); the call then skips its fill."""
    if prefilled and doc_score is None:
        raise ValueError("prefilled needs the doc_score buffer that holds -inf")
    _dev(q_r, "q_r", _FLOAT, (None, None, None, None))
    B, T, H, d = q_r.shape
    _dev(chunk_doc, "chunk_doc", _I32, (None,))
    n_chunks = chunk_doc.numel()
    _dev(kr_hat, "kr_hat", q_r.dtype, (None, H, d))
    if kr_hat.shape[0] < padded_chunks(n_chunks, layout):
        raise ValueError("kr_hat holds fewer chunks than chunk_doc names")
    dt = _dtype(q_r)
    if doc_score is None:
        doc_score = torch.empty((B, n_docs), dtype=torch.float32, device=q_r.device)
    _dev(doc_score, "doc_score", _F32, (B, n_docs))
    _dev(ws, "ws", optional=True)
    ws, wsb = _ws(msa_route_score_workspace(dt, B, T, H, d, n_docs, n_chunks), q_r.device, ws)
    _check("msa_route_score", lib.msa_route_score(
        dt, _ptr(q_r), B, T, H, d, _ptr(kr_hat), layout, _ptr(chunk_doc), n_docs, n_chunks, _ptr(doc_score),
        _ptr(ws), wsb, MSA_ROUTE_PREFILLED if prefilled else 0, _stream(stream)))
    return doc_score


def msa_route_score_fetch(q_r, kr_hat, chunk_doc, n_docs, f_ids, f_chunk_off, f_k_bar, f_v_bar, f_max_doc_chunks,
                          k_ctx, v_ctx, ctx_pos, ctx_len, doc_score=None, ws=None, layout=MSA_LAYOUT_ROWS,
                          stream=None, prefilled=False):
    """msa_route_score of this layer, and in the scan's tail the fetch that
    msa_gather_kv makes of another layer's selection f_ids [B', k] from its
    content store f_k_bar / f_v_bar [n, Hkv, d] (device or pinned host memory)
    into k_ctx / v_ctx [B', max_ctx, Hkv, d], ctx_pos, ctx_len."""
    if prefilled and doc_score is None:
        raise ValueError("prefilled needs the doc_score buffer that holds -inf")
    _dev(q_r, "q_r", _FLOAT, (None, None, None, None))
    B, T, H, d = q_r.shape
    _dev(chunk_doc, "chunk_doc", _I32, (None,))
    n_chunks = chunk_doc.numel()
    _dev(kr_hat, "kr_hat", q_r.dtype, (None, H, d))
    if kr_hat.shape[0] < padded_chunks(n_chunks, layout):
        raise ValueError("kr_hat holds fewer chunks than chunk_doc names")
    dt = _dtype(q_r)
    if doc_score is None:
        doc_score = torch.empty((B, n_docs), dtype=torch.float32, device=q_r.device)
    _dev(doc_score, "doc_score", _F32, (B, n_docs))
    _dev(f_ids, "f_ids", _I32, (None, None))
    fB, fk = f_ids.shape
    _dev(f_chunk_off, "f_chunk_off", _I64, (None,))
    if not isinstance(f_k_bar, torch.Tensor) or f_k_bar.dim() != 3:
        _fail("f_k_bar", "expected a [n_chunks, Hkv, d] tensor")
    n_src, Hkv, fd = f_k_bar.shape
    src = _dev if f_k_bar.is_cuda else _pinned
    src(f_k_bar, "f_k_bar", q_r.dtype, (n_src, Hkv, fd))
    src(f_v_bar, "f_v_bar", q_r.dtype, (n_src, Hkv, fd))
    _dev(k_ctx, "k_ctx", q_r.dtype, (fB, None, Hkv, fd))
    max_ctx = k_ctx.shape[1]
    _dev(v_ctx, "v_ctx", q_r.dtype, (fB, max_ctx, Hkv, fd))
    _dev(ctx_pos, "ctx_pos", _I32, (fB, max_ctx))
    _dev(ctx_len, "ctx_len", _I32, (fB,))
    _dev(ws, "ws", optional=True)
    ws, wsb = _ws(lib.msa_route_score_fetch_workspace(dt, B, T, H, d, n_docs, n_chunks), q_r.device, ws)
    _check("msa_route_score_fetch", lib.msa_route_score_fetch(
        dt, _ptr(q_r), B, T, H, d, _ptr(kr_hat), layout, _ptr(chunk_doc), n_docs, n_chunks, _ptr(doc_score),
        _ptr(ws), wsb, MSA_ROUTE_PREFILLED if prefilled else 0, _ptr(f_ids), fB, fk, _ptr(f_chunk_off),
        f_chunk_off.numel() - 1, f_max_doc_chunks, _ptr(f_k_bar), _ptr(f_v_bar), Hkv, fd, max_ctx, _ptr(k_ctx),
        _ptr(v_ctx), _ptr(ctx_pos), _ptr(ctx_len), _stream(stream)))
    return doc_score


def msa_route_balance(q_r, kr_hat, chunk_doc, n_docs, rounds=3, doc_score=None, ws=None, layout=MSA_LAYOUT_ROWS,
                      stream=None):
    """Sizes msa_route_score's chunk ranges per XCD on the current device from
    `rounds` rounds of timed launches on these arguments (a setup-time call: it
    synchronises and must not be captured); rounds=0 clears them.  Returns the
    8 XCD shares now in use."""
    shares = np.zeros(8, dtype=np.float32)
    if rounds == 0:
        _check("msa_route_balance", lib.msa_route_balance(0, None, 0, 0, 0, 0, None, 0, None, 0, 0, None, None, 0, 0,
                                                          shares.ctypes.data, None))
        return shares
    _dev(q_r, "q_r", _FLOAT, (None, None, None, None))
    B, T, H, d = q_r.shape
    _dev(chunk_doc, "chunk_doc", _I32, (None,))
    n_chunks = chunk_doc.numel()
    _dev(kr_hat, "kr_hat", q_r.dtype, (None, H, d))
    if kr_hat.shape[0] < padded_chunks(n_chunks, layout):
        raise ValueError("kr_hat holds fewer chunks than chunk_doc names")
    dt = _dtype(q_r)
    if doc_score is None:
        doc_score = torch.empty((B, n_docs), dtype=torch.float32, device=q_r.device)
    _dev(doc_score, "doc_score", _F32, (B, n_docs))
    _dev(ws, "ws", optional=True)
    ws, wsb = _ws(msa_route_score_workspace(dt, B, T, H, d, n_docs, n_chunks), q_r.device, ws)
    _check("msa_route_balance", lib.msa_route_balance(
        dt, _ptr(q_r), B, T, H, d, _ptr(kr_hat), layout, _ptr(chunk_doc), n_docs, n_chunks, _ptr(doc_score),
        _ptr(ws), wsb, int(rounds), shares.ctypes.data, _stream(stream)))
    return shares


def msa_chunk_scores(q_r, kr_hat, n_chunks, chunk_score=None, ws=None, layout=MSA_LAYOUT_ROWS, stream=None):
    """Per-chunk routing scores [B, n_chunks]: the max over the query's tokens
    of the head-mean cosine (msa_route_score before its document max)."""
    _dev(q_r, "q_r", _FLOAT, (None, None, None, None))
    B, T, H, d = q_r.shape
    _dev(kr_hat, "kr_hat", q_r.dtype, (None, H, d))
    if kr_hat.shape[0] < padded_chunks(n_chunks, layout):
        raise ValueError("kr_hat holds fewer than n_chunks chunks")
    if chunk_score is None:
        chunk_score = torch.empty((B, n_chunks), dtype=torch.float32, device=q_r.device)
    _dev(chunk_score, "chunk_score", _F32, (B, n_chunks))
    _dev(ws, "ws", optional=True)
    dt = _dtype(q_r)
    ws, wsb = _ws(msa_route_score_workspace(dt, B, T, H, d, n_chunks, n_chunks), q_r.device, ws)
    _check("msa_chunk_scores", lib.msa_chunk_scores(dt, _ptr(q_r), B, T, H, d, _ptr(kr_hat), layout, n_chunks,
                                                    _ptr(chunk_score), _ptr(ws), wsb, _stream(stream)))
    return chunk_score


def msa_segment_max(chunk_score, chunk_off, doc_score=None, stream=None):
    """doc_score[b, i] = max of chunk_score[b, chunk_off[i]:chunk_off[i+1]] (-inf if empty)."""
    _dev(chunk_score, "chunk_score", _F32, (None, None))
    B, n_chunks = chunk_score.shape
    _dev(chunk_off, "chunk_off", _I64, (None,))
    n_docs = chunk_off.numel() - 1
    if doc_score is None:
        doc_score = torch.empty((B, n_docs), dtype=torch.float32, device=chunk_score.device)
    _dev(doc_score, "doc_score", _F32, (B, n_docs))
    _check("msa_segment_max", lib.msa_segment_max(_ptr(chunk_score), B, n_chunks, _ptr(chunk_off), n_docs,
                                                  _ptr(doc_score), _stream(stream)))
    return doc_score


def msa_topk_workspace(B, n_docs, k):
    return lib.msa_topk_workspace(B, n_docs, k)


def msa_topk(doc_score, k, ids=None, vals=None, ws=None, stream=None, reset=False):
    """reset: write -inf over doc_score as it is read (it then no longer
    holds the scores), ready for msa_route_score(prefilled=True)."""
    _dev(doc_score, "doc_score", _F32, (None, None))
    B, n_docs = doc_score.shape
    if ids is None:
        ids = torch.empty((B, k), dtype=torch.int32, device=doc_score.device)
    if vals is None:
        vals = torch.empty((B, k), dtype=torch.float32, device=doc_score.device)
    _dev(ids, "ids", _I32, (B, k))
    _dev(vals, "vals", _F32, (B, k))
    _dev(ws, "ws", optional=True)
    ws, wsb = _ws(msa_topk_workspace(B, n_docs, k), doc_score.device, ws)
    _check("msa_topk", lib.msa_topk(_ptr(doc_score), B, n_docs, k, _ptr(ids), _ptr(vals), _ptr(ws), wsb,
                                    MSA_TOPK_RESET_SCORES if reset else 0, _stream(stream)))
    return ids, vals



def msa_topk_merge(vals, ids, id_offset, k, ids_out=None, vals_out=None, stream=None):
    """Global top-k of G shards' top-k lists.  vals [G, B, k_in] float32 and
    ids [G, B, k_in] int32 (shard-local ids, -1 for an empty slot), id_offset
    [G] int64 (each shard's first global id), all on the device."""
    _dev(vals, "vals", _F32, (None, None, None))
    G, B, k_in = vals.shape
    _dev(ids, "ids", _I32, (G, B, k_in))
    _dev(id_offset, "id_offset", _I64, (G,))
    if ids_out is None:
        ids_out = torch.empty((B, k), dtype=torch.int32, device=vals.device)
    if vals_out is None:
        vals_out = torch.empty((B, k), dtype=torch.float32, device=vals.device)
    _dev(ids_out, "ids_out", _I32, (B, k))
    _dev(vals_out, "vals_out", _F32, (B, k))
    _check("msa_topk_merge", lib.msa_topk_merge(_ptr(vals), _ptr(ids), _ptr(id_offset), G, B, k_in, k, _ptr(ids_out),
                                                _ptr(vals_out), _stream(stream)))
    return ids_out, vals_out

def msa_gather_kv(ids, chunk_off, k_bar, v_bar, max_doc_chunks, max_ctx, src_mode=MSA_SRC_DEVICE,
                  chunk_off_h=None, k_ctx=None, v_ctx=None, ctx_pos=None, ctx_len=None, ids_h=None,
                  stream=None, copy_stream=None, device=None):
    _dev(ids, "ids", _I32, (None, None))
    _dev(chunk_off, "chunk_off", _I64, (None,))
    B, k = ids.shape
    if not isinstance(k_bar, torch.Tensor) or k_bar.dim() != 3:
        _fail("k_bar", "expected a [n_chunks, Hkv, d] tensor")
    n_chunks, Hkv, d = k_bar.shape
    # the source store: device memory, or pinned host memory for the host tier
    src = _dev if src_mode == MSA_SRC_DEVICE else _pinned
    src(k_bar, "k_bar", _FLOAT, (n_chunks, Hkv, d))
    src(v_bar, "v_bar", k_bar.dtype, (n_chunks, Hkv, d))
    if chunk_off_h is not None:
        _host_i64(chunk_off_h, "chunk_off_h", chunk_off.numel())
    dev = device if device is not None else ids.device
    if k_ctx is None:
        k_ctx = torch.empty((B, max_ctx, Hkv, d), dtype=k_bar.dtype, device=dev)
    if v_ctx is None:
        v_ctx = torch.empty((B, max_ctx, Hkv, d), dtype=v_bar.dtype, device=dev)
    if ctx_pos is None:
        ctx_pos = torch.empty((B, max_ctx), dtype=torch.int32, device=dev)
    if ctx_len is None:
        ctx_len = torch.empty((B,), dtype=torch.int32, device=dev)
    _dev(k_ctx, "k_ctx", k_bar.dtype, (B, max_ctx, Hkv, d))
    _dev(v_ctx, "v_ctx", k_bar.dtype, (B, max_ctx, Hkv, d))
    _dev(ctx_pos, "ctx_pos", _I32, (B, max_ctx))
    _dev(ctx_len, "ctx_len", _I32, (B,))
    if src_mode == MSA_SRC_HOST_MEMCPY and ids_h is None:
        ids_h = torch.empty((B, k), dtype=torch.int32, pin_memory=True)
    if ids_h is not None:
        _pinned(ids_h, "ids_h", _I32, (B, k))
    _check("msa_gather_kv", lib.msa_gather_kv(
        _dtype(k_bar), _ptr(ids), B, k, _ptr(chunk_off), _ptr(chunk_off_h), chunk_off.numel() - 1,
        max_doc_chunks, _ptr(k_bar), _ptr(v_bar), n_chunks, Hkv, d, src_mode, max_ctx, _ptr(k_ctx),
        _ptr(v_ctx), _ptr(ctx_pos), _ptr(ctx_len), _ptr(ids_h), _stream(stream),
        None if copy_stream is None else _stream(copy_stream)))
    return k_ctx, v_ctx, ctx_pos, ctx_len


def _index_outputs(B, max_ctx, dev, ctx_row, ctx_pos, ctx_len):
    if ctx_row is None:
        ctx_row = torch.empty((B, max_ctx), dtype=torch.int32, device=dev)
    if ctx_pos is None:
        ctx_pos = torch.empty((B, max_ctx), dtype=torch.int32, device=dev)
    if ctx_len is None:
        ctx_len = torch.empty((B,), dtype=torch.int32, device=dev)
    _dev(ctx_row, "ctx_row", _I32, (B, max_ctx))
    _dev(ctx_pos, "ctx_pos", _I32, (B, max_ctx))
    _dev(ctx_len, "ctx_len", _I32, (B,))
    return ctx_row, ctx_pos, ctx_len


def msa_context_index(ids, chunk_off, n_chunks, max_doc_chunks, max_ctx, ctx_row=None, ctx_pos=None, ctx_len=None,
                      stream=None):
    _dev(ids, "ids", _I32, (None, None))
    _dev(chunk_off, "chunk_off", _I64, (None,))
    B, k = ids.shape
    ctx_row, ctx_pos, ctx_len = _index_outputs(B, max_ctx, ids.device, ctx_row, ctx_pos, ctx_len)
    _check("msa_context_index", lib.msa_context_index(
        _ptr(ids), B, k, _ptr(chunk_off), chunk_off.numel() - 1, max_doc_chunks, n_chunks, max_ctx, _ptr(ctx_row),
        _ptr(ctx_pos), _ptr(ctx_len), _stream(stream)))
    return ctx_row, ctx_pos, ctx_len


def msa_topk_context_index(doc_score, k, chunk_off, n_chunks, max_doc_chunks, max_ctx, ids=None, vals=None,
                           ctx_row=None, ctx_pos=None, ctx_len=None, ws=None, stream=None, reset=False):
    """msa_topk then msa_context_index on its ids, in one pass for k <= 64;
    reset as for msa_topk."""
    _dev(doc_score, "doc_score", _F32, (None, None))
    _dev(chunk_off, "chunk_off", _I64, (doc_score.shape[1] + 1,))
    B, n_docs = doc_score.shape
    dev = doc_score.device
    if ids is None:
        ids = torch.empty((B, k), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((B, k), dtype=torch.float32, device=dev)
    _dev(ids, "ids", _I32, (B, k))
    _dev(vals, "vals", _F32, (B, k))
    ctx_row, ctx_pos, ctx_len = _index_outputs(B, max_ctx, dev, ctx_row, ctx_pos, ctx_len)
    _dev(ws, "ws", optional=True)
    ws, wsb = _ws(msa_topk_workspace(B, n_docs, k), dev, ws)
    _check("msa_topk_context_index", lib.msa_topk_context_index(
        _ptr(doc_score), B, n_docs, k, _ptr(ids), _ptr(vals), _ptr(chunk_off), max_doc_chunks, n_chunks, max_ctx,
        _ptr(ctx_row), _ptr(ctx_pos), _ptr(ctx_len), _ptr(ws), wsb, MSA_TOPK_RESET_SCORES if reset else 0,
        _stream(stream)))
    return ids, vals, ctx_row, ctx_pos, ctx_len


def msa_exclude_docs(doc_score, ids_sets, stream=None):
    """ids_sets: [n_sets, B, k] int32 (earlier rounds' selections)."""
    _dev(doc_score, "doc_score", _F32, (None, None))
    B, n_docs = doc_score.shape
    _dev(ids_sets, "ids_sets", _I32, (None, B, None))
    n_sets, _, k = ids_sets.shape
    _check("msa_exclude_docs", lib.msa_exclude_docs(_ptr(doc_score), B, n_docs, _ptr(ids_sets) if n_sets else None,
                                                    n_sets, k, _stream(stream)))
    return doc_score


def msa_context_append(ids, chunk_off, n_chunks, max_doc_chunks, ctx_row, ctx_pos, ctx_len_in, ctx_len_out,
                       stream=None):
    _dev(ids, "ids", _I32, (None, None))
    _dev(chunk_off, "chunk_off", _I64, (None,))
    B, k = ids.shape
    _dev(ctx_row, "ctx_row", _I32, (B, None))
    max_ctx = ctx_row.shape[1]
    _dev(ctx_pos, "ctx_pos", _I32, (B, max_ctx))
    _dev(ctx_len_in, "ctx_len_in", _I32, (B,))
    _dev(ctx_len_out, "ctx_len_out", _I32, (B,))
    _check("msa_context_append", lib.msa_context_append(
        _ptr(ids), B, k, _ptr(chunk_off), chunk_off.numel() - 1, max_doc_chunks, n_chunks, max_ctx,
        _ptr(ctx_row), _ptr(ctx_pos), _ptr(ctx_len_in), _ptr(ctx_len_out), _stream(stream)))
    return ctx_row, ctx_pos, ctx_len_out


def msa_sparse_attn_workspace(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset):
    return lib.msa_sparse_attn_workspace(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset)


def msa_rope_table_rows(max_ctx, L_loc, q_pos_offset):
    return lib.msa_rope_table_rows(max_ctx, L_loc, q_pos_offset)


def msa_rope_table(rows, d, rope_base=1e6, table=None, device=None, stream=None):
    if table is None:
        table = torch.empty((rows, d // 2, 2), dtype=torch.float32, device=device)
    _dev(table, "table", _F32, (rows, d // 2, 2))
    _check("msa_rope_table", lib.msa_rope_table(rows, d, float(rope_base), _ptr(table), _stream(stream)))
    return table


def _attn_operands(q, k_loc, v_loc, rope_table, out, out_name="out"):
    """Checks shared by the attention entry points; returns (B, T, Hq, d, Hkv, L_loc, out)."""
    _dev(q, "q", _FLOAT, (None, None, None, None))
    B, T, Hq, d = q.shape
    _dev(k_loc, "k_loc", q.dtype, (B, None, None, d))
    L_loc, Hkv = k_loc.shape[1], k_loc.shape[2]
    _dev(v_loc, "v_loc", q.dtype, (B, L_loc, Hkv, d))
    _dev(rope_table, "rope_table", _F32, (None, d // 2, 2), optional=True)
    if out is None:
        out = torch.empty((B, T, Hq, d), dtype=torch.float32, device=q.device)
    _dev(out, out_name, _F32, (B, T, Hq, d))
    return B, T, Hq, d, Hkv, L_loc, out


def msa_sparse_attn(q, k_ctx, v_ctx, ctx_pos, ctx_len, k_loc, v_loc, q_pos_offset, rope_base=1e6,
                    sm_scale=None, out=None, ws=None, rope_table=None, stream=None):
    B, T, Hq, d, Hkv, L_loc, out = _attn_operands(q, k_loc, v_loc, rope_table, out)
    _dev(k_ctx, "k_ctx", q.dtype, (B, None, Hkv, d))
    max_ctx = k_ctx.shape[1]
    _dev(v_ctx, "v_ctx", q.dtype, (B, max_ctx, Hkv, d))
    _dev(ctx_pos, "ctx_pos", _I32, (B, max_ctx))
    _dev(ctx_len, "ctx_len", _I32, (B,))
    _dev(ws, "ws", optional=True)
    dt = _dtype(q)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    ws, wsb = _ws(msa_sparse_attn_workspace(dt, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset), q.device, ws)
    _check("msa_sparse_attn", lib.msa_sparse_attn(
        dt, _ptr(q), B, T, Hq, Hkv, d, _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_pos), _ptr(ctx_len), max_ctx,
        _ptr(k_loc), _ptr(v_loc), L_loc, q_pos_offset, float(rope_base), _ptr(rope_table),
        0 if rope_table is None else rope_table.shape[0], float(sm_scale), _ptr(out), _ptr(ws), wsb,
        _stream(stream)))
    return out


def msa_sparse_attn_indexed(q, k_bar, v_bar, ctx_row, ctx_pos, ctx_len, k_loc, v_loc, q_pos_offset, rope_base=1e6,
                            sm_scale=None, out=None, ws=None, rope_table=None, stream=None):
    B, T, Hq, d, Hkv, L_loc, out = _attn_operands(q, k_loc, v_loc, rope_table, out)
    _store(k_bar, "k_bar", q.dtype, (None, Hkv, d))
    n_chunks = k_bar.shape[0]
    _store(v_bar, "v_bar", q.dtype, (n_chunks, Hkv, d))
    _dev(ctx_row, "ctx_row", _I32, (B, None))
    max_ctx = ctx_row.shape[1]
    _dev(ctx_pos, "ctx_pos", _I32, (B, max_ctx))
    _dev(ctx_len, "ctx_len", _I32, (B,))
    _dev(ws, "ws", optional=True)
    dt = _dtype(q)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    ws, wsb = _ws(msa_sparse_attn_workspace(dt, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset), q.device, ws)
    _check("msa_sparse_attn_indexed", lib.msa_sparse_attn_indexed(
        dt, _ptr(q), B, T, Hq, Hkv, d, _ptr(k_bar), _ptr(v_bar), n_chunks, _ptr(ctx_row), _ptr(ctx_pos),
        _ptr(ctx_len), max_ctx, _ptr(k_loc), _ptr(v_loc), L_loc, q_pos_offset, float(rope_base), _ptr(rope_table),
        0 if rope_table is None else rope_table.shape[0], float(sm_scale), _ptr(out), _ptr(ws), wsb,
        _stream(stream)))
    return out


def msa_sparse_attn_part_workspace(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset):
    return lib.msa_sparse_attn_part_workspace(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset)


def msa_sparse_attn_part(part, q, k_loc, v_loc, q_pos_offset, max_ctx, k_ctx=None, v_ctx=None, ctx_row=None,
                         ctx_pos=None, ctx_len=None, rope_base=1e6, sm_scale=None, out=None, ws=None,
                         rope_table=None, stream=None):
    """One of the two calls of msa_sparse_attn_part: MSA_ATTN_PART_LOCAL (the
    local keys' partials into ws; the context arguments are not needed) or
    MSA_ATTN_PART_CONTEXT (the context keys and the merge into out, with the
    local call's ws).  With ctx_row the context is read in place from the store
    k_ctx/v_ctx [rows, Hkv, d]; without it k_ctx/v_ctx are a gathered context
    [B, max_ctx, Hkv, d].  Both calls take the same max_ctx and ws."""
    B, T, Hq, d, Hkv, L_loc, out = _attn_operands(q, k_loc, v_loc, rope_table, out)
    ctx_rows = 0
    if part == MSA_ATTN_PART_CONTEXT:
        if ctx_row is None:
            _dev(k_ctx, "k_ctx", q.dtype, (B, max_ctx, Hkv, d))
            _dev(v_ctx, "v_ctx", q.dtype, (B, max_ctx, Hkv, d))
        else:
            _store(k_ctx, "k_ctx", q.dtype, (None, Hkv, d))
            ctx_rows = k_ctx.shape[0]
            _store(v_ctx, "v_ctx", q.dtype, (ctx_rows, Hkv, d))
            _dev(ctx_row, "ctx_row", _I32, (B, max_ctx))
        _dev(ctx_pos, "ctx_pos", _I32, (B, max_ctx))
        _dev(ctx_len, "ctx_len", _I32, (B,))
    _dev(ws, "ws", optional=True)
    dt = _dtype(q)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    ws, wsb = _ws(msa_sparse_attn_part_workspace(dt, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset), q.device, ws)
    _check("msa_sparse_attn_part", lib.msa_sparse_attn_part(
        part, dt, _ptr(q), B, T, Hq, Hkv, d, _ptr(k_ctx), _ptr(v_ctx), ctx_rows, _ptr(ctx_row), _ptr(ctx_pos),
        _ptr(ctx_len), max_ctx, _ptr(k_loc), _ptr(v_loc), L_loc, q_pos_offset, float(rope_base), _ptr(rope_table),
        0 if rope_table is None else rope_table.shape[0], float(sm_scale), _ptr(out), _ptr(ws), wsb,
        _stream(stream)))
    return out


MSA_NOALLOC_SCRATCH_BYTES = 32 << 20   # include/msa.h


def msa_sparse_attn_indexed_noalloc(q, k_bar, v_bar, ctx_row, ctx_pos, ctx_len, k_loc, v_loc, q_pos_offset,
                                    rope_base=1e6, sm_scale=None, out=None, rope_table=None, stream=None):
    """msa_sparse_attn_indexed with the library's own device scratch instead
    of a workspace (for callers that cannot allocate; pass ``out`` and
    ``rope_table`` to allocate nothing here either)."""
    B, T, Hq, d, Hkv, L_loc, out = _attn_operands(q, k_loc, v_loc, rope_table, out)
    _store(k_bar, "k_bar", q.dtype, (None, Hkv, d))
    n_chunks = k_bar.shape[0]
    _store(v_bar, "v_bar", q.dtype, (n_chunks, Hkv, d))
    _dev(ctx_row, "ctx_row", _I32, (B, None))
    max_ctx = ctx_row.shape[1]
    _dev(ctx_pos, "ctx_pos", _I32, (B, max_ctx))
    _dev(ctx_len, "ctx_len", _I32, (B,))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    _check("msa_sparse_attn_indexed_noalloc", lib.msa_sparse_attn_indexed_noalloc(
        _dtype(q), _ptr(q), B, T, Hq, Hkv, d, _ptr(k_bar), _ptr(v_bar), n_chunks, _ptr(ctx_row), _ptr(ctx_pos),
        _ptr(ctx_len), max_ctx, _ptr(k_loc), _ptr(v_loc), L_loc, q_pos_offset, float(rope_base), _ptr(rope_table),
        0 if rope_table is None else rope_table.shape[0], float(sm_scale), _ptr(out), _stream(stream)))
    return out


def msa_stream_read(buf, sink, stream=None):
    """Streaming-read reference: reads every byte of ``buf`` once."""
    _dev(buf, "buf")
    _dev(sink, "sink", (torch.int32, torch.uint32) if hasattr(torch, "uint32") else torch.int32, (1,))
    _check("msa_stream_read", lib.msa_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                  _stream(stream)))


# ---------------------------------------------------------------- training-time path

def msa_route_argmax_workspace(dtype, B, T, H, d, n_docs, n_chunks):
    return lib.msa_route_argmax_workspace(dtype, B, T, H, d, n_docs, n_chunks)


def msa_route_argmax(q_r, kr_hat, chunk_doc, n_docs, doc_score=None, arg_chunk=None, arg_tok=None, ws=None,
                     stream=None):
    _dev(q_r, "q_r", _FLOAT, (None, None, None, None))
    B, T, H, d = q_r.shape
    _dev(chunk_doc, "chunk_doc", _I32, (None,))
    n_chunks = chunk_doc.numel()
    _dev(kr_hat, "kr_hat", q_r.dtype, (None, H, d))
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
    _dev(doc_score, "doc_score", _F32, (B, n_docs))
    _dev(arg_chunk, "arg_chunk", _I32, (B, n_docs))
    _dev(arg_tok, "arg_tok", _I32, (B, n_docs))
    _dev(ws, "ws", optional=True)
    ws, wsb = _ws(msa_route_argmax_workspace(dt, B, T, H, d, n_docs, n_chunks), dev, ws)
    _check("msa_route_argmax", lib.msa_route_argmax(
        dt, _ptr(q_r), B, T, H, d, _ptr(kr_hat), _ptr(chunk_doc), n_docs, n_chunks, _ptr(doc_score),
        _ptr(arg_chunk), _ptr(arg_tok), _ptr(ws), wsb, _stream(stream)))
    return doc_score, arg_chunk, arg_tok


def msa_route_loss(doc_score, pos_ids, tau, loss=None, grad=None, stream=None):
    _dev(doc_score, "doc_score", _F32, (None, None))
    B, n_docs = doc_score.shape
    _dev(pos_ids, "pos_ids", _I32, (B, None))
    n_pos = pos_ids.shape[1]
    if loss is None:
        loss = torch.empty((B,), dtype=torch.float32, device=doc_score.device)
    if grad is None:
        grad = torch.empty_like(doc_score)
    _dev(loss, "loss", _F32, (B,))
    _dev(grad, "grad", _F32, (B, n_docs))
    _check("msa_route_loss", lib.msa_route_loss(_ptr(doc_score), B, n_docs, _ptr(pos_ids), n_pos, float(tau),
                                                _ptr(loss), _ptr(grad), _stream(stream)))
    return loss, grad


def msa_route_score_backward(q_r, kr_hat, arg_chunk, arg_tok, grad, dkr_hat, dq_r=None, stream=None):
    """dkr_hat [n_chunks, H, d] float32 is accumulated into (zero it first)."""
    _dev(q_r, "q_r", _FLOAT, (None, None, None, None))
    B, T, H, d = q_r.shape
    _dev(dkr_hat, "dkr_hat", _F32, (None, H, d))
    n_chunks = dkr_hat.shape[0]
    _dev(kr_hat, "kr_hat", q_r.dtype, (None, H, d))
    if kr_hat.shape[0] < n_chunks:
        raise ValueError("kr_hat holds fewer chunks than dkr_hat")
    _dev(grad, "grad", _F32, (B, None))
    n_docs = grad.shape[1]
    _dev(arg_chunk, "arg_chunk", _I32, (B, n_docs))
    _dev(arg_tok, "arg_tok", _I32, (B, n_docs))
    if dq_r is None:
        dq_r = torch.empty((B, T, H, d), dtype=torch.float32, device=q_r.device)
    _dev(dq_r, "dq_r", _F32, (B, T, H, d))
    _check("msa_route_score_backward", lib.msa_route_score_backward(
        _dtype(q_r), _ptr(q_r), B, T, H, d, _ptr(kr_hat), n_chunks, _ptr(arg_chunk), _ptr(arg_tok), _ptr(grad),
        n_docs, _ptr(dq_r), _ptr(dkr_hat), _stream(stream)))
    return dq_r, dkr_hat


def msa_pool_backward(dy, tok_off, chunk_off, chunk_doc, n_tok, chunk, x=None, dtype=None, dx=None, stream=None):
    """dx [n_tok, H, d] float32.  x (the token vectors, when the pooled entry
    was L2-normalised) sets the dtype; otherwise ``dtype`` (default bf16)."""
    _dev(dy, "dy", _F32, (None, None, None))
    n_chunks, H, d = dy.shape
    _dev(tok_off, "tok_off", _I64, (None,))
    _dev(chunk_off, "chunk_off", _I64, (tok_off.numel(),))
    _dev(chunk_doc, "chunk_doc", _I32, (n_chunks,))
    _dev(x, "x", _FLOAT, (n_tok, H, d), optional=True)
    if dx is None:
        dx = torch.empty((n_tok, H, d), dtype=torch.float32, device=dy.device)
    _dev(dx, "dx", _F32, (n_tok, H, d))
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
    if dout is None:
        _fail("dout", "required")
    B, T, Hq, d, Hkv, L_loc, dout = _attn_operands(q, k_loc, v_loc, rope_table, dout, "dout")
    _dev(k_bar, "k_bar", q.dtype, (None, Hkv, d))
    n_chunks = k_bar.shape[0]
    _dev(v_bar, "v_bar", q.dtype, (n_chunks, Hkv, d))
    _dev(ctx_row, "ctx_row", _I32, (B, None))
    max_ctx = ctx_row.shape[1]
    _dev(ctx_pos, "ctx_pos", _I32, (B, max_ctx))
    _dev(ctx_len, "ctx_len", _I32, (B,))
    _dev(dk_bar, "dk_bar", _F32, (n_chunks, Hkv, d))
    _dev(dv_bar, "dv_bar", _F32, (n_chunks, Hkv, d))
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
    _dev(dq, "dq", _F32, (B, T, Hq, d))
    _dev(dk_loc, "dk_loc", _F32, (B, L_loc, Hkv, d))
    _dev(dv_loc, "dv_loc", _F32, (B, L_loc, Hkv, d))
    _dev(ws, "ws", optional=True)
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
    _dev(x, "x", _FLOAT, (None, None))
    n_tok, hidden = x.shape
    _dev(w_t, "w_t", x.dtype, (3 * H * d, hidden))
    _dev(tok_off, "tok_off", _I64, (None,))
    _dev(chunk_off, "chunk_off", _I64, (tok_off.numel(),))
    _dev(chunk_doc, "chunk_doc", _I32, (None,))
    n_chunks = chunk_doc.numel()
    dt = _dtype(x)
    dev_ = x.device
    if k_bar is None:
        k_bar = torch.empty((n_chunks, H, d), dtype=x.dtype, device=dev_)
    if v_bar is None:
        v_bar = torch.empty((n_chunks, H, d), dtype=x.dtype, device=dev_)
    if kr_hat is None:
        kr_hat = torch.empty((padded_chunks(n_chunks, kr_layout), H, d), dtype=x.dtype, device=dev_)
    _dev(k_bar, "k_bar", x.dtype, (n_chunks, H, d))
    _dev(v_bar, "v_bar", x.dtype, (n_chunks, H, d))
    _dev(kr_hat, "kr_hat", x.dtype, (padded_chunks(n_chunks, kr_layout), H, d))
    _dev(ws, "ws", optional=True)
    ws, wsb = _ws(lib.msa_encode_workspace(dt, n_chunks, hidden, H, d), dev_, ws)
    _check("msa_encode", lib.msa_encode(
        dt, _ptr(x), _ptr(w_t), hidden, H, d, _ptr(tok_off), _ptr(chunk_off), _ptr(chunk_doc), tok_off.numel() - 1,
        n_tok, n_chunks, chunk, kr_layout, _ptr(k_bar), _ptr(v_bar), _ptr(kr_hat), _ptr(ws), wsb, _stream(stream)))
    return k_bar, v_bar, kr_hat


def msa_encode_pool(x, tok_off, chunk_off, chunk_doc, chunk, H, d, ws=None, stream=None):
    """The first half of msa_encode: the block's pooled rows into ws (returned)."""
    _dev(x, "x", _FLOAT, (None, None))
    n_tok, hidden = x.shape
    _dev(tok_off, "tok_off", _I64, (None,))
    _dev(chunk_off, "chunk_off", _I64, (tok_off.numel(),))
    _dev(chunk_doc, "chunk_doc", _I32, (None,))
    n_chunks = chunk_doc.numel()
    _dev(ws, "ws", optional=True)
    ws, wsb = _ws(lib.msa_encode_workspace(_dtype(x), n_chunks, hidden, H, d), x.device, ws)
    _check("msa_encode_pool", lib.msa_encode_pool(
        _dtype(x), _ptr(x), hidden, H, d, _ptr(tok_off), _ptr(chunk_off), _ptr(chunk_doc), tok_off.numel() - 1,
        n_tok, n_chunks, chunk, _ptr(ws), wsb, _stream(stream)))
    return ws


def msa_encode_project(w_t, n_chunks, H, d, ws, kr_layout=MSA_LAYOUT_ROWS, k_bar=None, v_bar=None, kr_hat=None,
                       stream=None):
    """The second half of msa_encode: project the pooled rows held in ws
    (from msa_encode_pool) to (k_bar, v_bar, kr_hat)."""
    _dev(w_t, "w_t", _FLOAT, (3 * H * d, None))
    hidden = w_t.shape[1]
    _dev(ws, "ws")
    dev_ = w_t.device
    if k_bar is None:
        k_bar = torch.empty((n_chunks, H, d), dtype=w_t.dtype, device=dev_)
    if v_bar is None:
        v_bar = torch.empty((n_chunks, H, d), dtype=w_t.dtype, device=dev_)
    if kr_hat is None:
        kr_hat = torch.empty((padded_chunks(n_chunks, kr_layout), H, d), dtype=w_t.dtype, device=dev_)
    _dev(k_bar, "k_bar", w_t.dtype, (n_chunks, H, d))
    _dev(v_bar, "v_bar", w_t.dtype, (n_chunks, H, d))
    _dev(kr_hat, "kr_hat", w_t.dtype, (padded_chunks(n_chunks, kr_layout), H, d))
    _check("msa_encode_project", lib.msa_encode_project(
        _dtype(w_t), _ptr(w_t), hidden, H, d, n_chunks, kr_layout, _ptr(k_bar), _ptr(v_bar), _ptr(kr_hat), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return k_bar, v_bar, kr_hat
