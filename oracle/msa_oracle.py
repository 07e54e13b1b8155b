"""Plain, slow, float64 CPU oracle of the MSA online-routing + sparse-attention path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It
shares no code with the HIP path; the only thing both sides share is the
seeded input generator in ``synth``.

Every function follows the plain definition of one step, in float64, with
materialised intermediates (the full token x chunk score tensor, a full sort
for top-k, an explicit concatenation for attention).  Sources, cited by page
and section:

* [P1] "MSA-arXiv26" paper note, section 核心方法 (method): 架构 (architecture),
  Document-wise RoPE, Memory Parallel 推理 (inference).
* [P2] "MSA: Memory Sparse Attention" project README, sections
  Overall Design > Architecture and Overall Design > Inference Pipeline.
* [P3] MSA project note, section 架构设计 > MSA Layer 工作流程 (layer workflow).

Readings where the pages are silent (each also listed in the design notes):

* R1  the token-wise max runs over the query tokens and the document's pooled
      chunks, giving one score per document; the head mean sits inside.
* R2  pool first, then L2-normalise the pooled routing key.
* R3  routing uses as many query heads as key heads (no GQA in routing).
* R4  no RoPE on routing vectors.
* R5  norms are clamped at eps = 1e-8 (a zero vector has cosine 0).
* R6  a partial last chunk is the mean of the tokens it has.
* R9  ranking is by (score descending, document id ascending).
* R10 an empty document scores -inf; k larger than the number of documents
      is an error.
* R11 a pooled chunk sits at its chunk index inside its document (0, 1, ...).
* R12 local token i sits at position q_pos_offset + i, q_pos_offset = k by
      default (the pages offset the query by k).
* R13 the T query tokens are the last T of the L_loc local tokens; causal
      inside the local part; every retrieved entry is visible to every query
      token.
* R14 query head hq reads KV head floor(hq / (Hq / Hkv)).
* R15 softmax scale 1/sqrt(d).
* R16 rotate-half RoPE: pairs (m, m + d/2), angle p * base**(-2m/d).
* R17 context order: retrieved documents in rank order, each in chunk order,
      then the local tokens.
* R18 stores (normalised routing keys, pooled K and V) are rounded once,
      round-to-nearest-even, to the store dtype.
* R23-R26 (Memory Interleave, see ``interleave``): the router stands in for
      the model's document-id generation, fetched documents are appended in
      round order, the query offset is the number of documents fetched, and
      the number of rounds is fixed.
* R32 (``encode``): K, V and K_r are linear projections of the hidden state.
* R27-R31 (training-time path, see ``route_loss`` onwards): the routing loss
      is a supervised contrastive loss over the documents with a temperature,
      the max passes its derivative to one maximiser, the selection is held
      fixed, and the store rounding is the identity in the backward.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-8


# ---------------------------------------------------------------------------
# rounding to the store dtype (R18)
# ---------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significand bits),
    ties to even; returned as float64.  Finite normal inputs only."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                          # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # rint: ties to even


def round_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return round_to_f32(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# document index
# ---------------------------------------------------------------------------

def chunk_offsets(tok_off: np.ndarray, chunk: int) -> np.ndarray:
    """Chunk CSR offsets: document i has ceil(len_i / chunk) pooled chunks."""
    tok_off = np.asarray(tok_off, dtype=np.int64)
    lens = np.diff(tok_off)
    counts = (lens + chunk - 1) // chunk
    out = np.zeros(len(lens) + 1, dtype=np.int64)
    out[1:] = np.cumsum(counts)
    return out


# ---------------------------------------------------------------------------
# Stage 1: chunk-mean pooling and routing-key normalisation
# [P1 架构; P2 Overall Design > Architecture (K, V and K_r are mean-pooled per
#  chunk); P2 Inference Pipeline, stage 1 (global memory encoding); P3 MSA Layer
#  工作流程 step 1]
# ---------------------------------------------------------------------------

def pool(x: np.ndarray, tok_off: np.ndarray, chunk: int) -> np.ndarray:
    """Chunk means of per-token vectors.

    x: [n_tok, H, d]; document i owns tokens tok_off[i] .. tok_off[i+1]-1.
    Chunk j of document i averages tokens tok_off[i] + j*chunk up to (not
    including) min(tok_off[i] + (j+1)*chunk, tok_off[i+1]) (R6).
    Returns [n_chunks, H, d] float64, chunks in document order.
    """
    x = np.asarray(x, dtype=np.float64)
    tok_off = np.asarray(tok_off, dtype=np.int64)
    rows = []
    for i in range(len(tok_off) - 1):
        lo, hi = int(tok_off[i]), int(tok_off[i + 1])
        for s in range(lo, hi, chunk):
            e = min(s + chunk, hi)
            rows.append(x[s:e].sum(axis=0) / (e - s))
    if not rows:
        return np.zeros((0,) + x.shape[1:], dtype=np.float64)
    return np.stack(rows)


def l2_normalize(x: np.ndarray, eps: float = EPS) -> np.ndarray:
    """x / max(||x||_2, eps) over the last axis (R5)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def pool_encode(x: np.ndarray, tok_off: np.ndarray, chunk: int, normalize: bool,
                dtype: str) -> np.ndarray:
    """Pooled store entry: chunk mean, L2-normalised per (chunk, head) for
    the routing keys (R2), rounded once to the store dtype (R18)."""
    p = pool(x, tok_off, chunk)
    if normalize:
        p = l2_normalize(p)
    return round_to_store(p, dtype)


# ---------------------------------------------------------------------------
# Stage 2: routing score, top-k, context assembly
# [P1 架构 (cosine similarity, top-k documents); P2 Overall Design >
#  Architecture (cosine similarity, averaged over heads, then a max over
#  tokens); P2 Inference Pipeline, stage 2 (online routing and context assembly);
#  P3 MSA Layer 工作流程 steps 2-4]
# ---------------------------------------------------------------------------

def chunk_cosines(q_r: np.ndarray, kr_store: np.ndarray, eps: float = EPS) -> np.ndarray:
    """s[b, t, c] = (1/H) sum_h cos(q_r[b, t, h], kr[c, h]).

    q_r: [B, T, H, d] raw routing queries; kr_store: [N, H, d], already
    L2-normalised store entries (their cosine equals their dot product with
    a unit query).  Head mean inside the token/chunk max (R1, R3)."""
    q = l2_normalize(np.asarray(q_r, dtype=np.float64), eps)
    k = np.asarray(kr_store, dtype=np.float64)
    B, T, H, d = q.shape
    N = k.shape[0]
    # per-head dot products, then the mean over heads
    s = np.zeros((B, T, N), dtype=np.float64)
    for h in range(H):
        s += q[:, :, h, :] @ k[:, h, :].T
    return s / H


def route_scores(q_r: np.ndarray, kr_store: np.ndarray, chunk_off: np.ndarray,
                 eps: float = EPS) -> np.ndarray:
    """One score per (query, document): the max over the query's tokens and
    the document's chunks of the head-mean cosine (R1).  Empty documents
    score -inf (R10).  Returns [B, D] float64."""
    s = chunk_cosines(q_r, kr_store, eps)          # [B, T, N]
    per_chunk = s.max(axis=1)                      # token-wise max -> [B, N]
    chunk_off = np.asarray(chunk_off, dtype=np.int64)
    D = len(chunk_off) - 1
    out = np.full((s.shape[0], D), -np.inf, dtype=np.float64)
    for i in range(D):
        lo, hi = int(chunk_off[i]), int(chunk_off[i + 1])
        if hi > lo:
            out[:, i] = per_chunk[:, lo:hi].max(axis=1)
    return out


def topk(doc_score: np.ndarray, k: int):
    """The k best documents per query, ordered by (score desc, id asc) (R9).
    Returns (ids int32 [B, k], vals float64 [B, k])."""
    doc_score = np.asarray(doc_score, dtype=np.float64)
    B, D = doc_score.shape
    if k < 1 or k > D:
        raise ValueError("k must be in [1, n_docs]")
    ids = np.empty((B, k), dtype=np.int32)
    vals = np.empty((B, k), dtype=np.float64)
    doc = np.arange(D)
    for b in range(B):
        order = np.lexsort((doc, -doc_score[b]))   # primary: -score, then id
        ids[b] = order[:k]
        vals[b] = doc_score[b, order[:k]]
    return ids, vals


def topk_merge(vals: np.ndarray, ids: np.ndarray, id_offset: np.ndarray, k: int):
    """Memory Parallel's global reduce of per-shard top-k lists ([P2] Overall
    Design > Inference Pipeline: the routing keys are sharded over GPUs, each
    scores its shard locally and a global reduce follows; [P1] Memory Parallel
    推理).  vals [G, B, k_in] scores and ids [G, B, k_in]
    shard-local document ids (-1 or a NaN score: an empty slot) of G shards
    whose documents start at global id id_offset[g].  The result is the k best
    valid entries per query by (score desc, global id asc) (R9), as
    (ids int32 [B, k], vals float64 [B, k]); when fewer than k are valid the
    trailing ids are -1 and their values NaN."""
    vals = np.asarray(vals, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    G, B, k_in = vals.shape
    out_ids = np.full((B, k), -1, dtype=np.int32)
    out_vals = np.full((B, k), np.nan)
    for b in range(B):
        cand = [(vals[g, b, j], int(ids[g, b, j]) + int(id_offset[g]))
                for g in range(G) for j in range(k_in) if ids[g, b, j] >= 0 and vals[g, b, j] == vals[g, b, j]]
        cand.sort(key=lambda t: (-t[0], t[1]))
        for r, (v, i) in enumerate(cand[:k]):
            out_ids[b, r] = i
            out_vals[b, r] = v
    return out_ids, out_vals


def gather(ids_b: np.ndarray, chunk_off: np.ndarray, k_bar: np.ndarray, v_bar: np.ndarray):
    """Context of one query: the selected documents' pooled K/V in rank order,
    each document's chunks in order (R17), with each entry's position inside
    its document (R11)."""
    ks, vs, pos = [], [], []
    for doc in ids_b:
        lo, hi = int(chunk_off[doc]), int(chunk_off[doc + 1])
        ks.append(np.asarray(k_bar[lo:hi], dtype=np.float64))
        vs.append(np.asarray(v_bar[lo:hi], dtype=np.float64))
        pos.append(np.arange(hi - lo, dtype=np.int64))
    H, d = k_bar.shape[1:]
    if ks:
        return np.concatenate(ks), np.concatenate(vs), np.concatenate(pos)
    return np.zeros((0, H, d)), np.zeros((0, H, d)), np.zeros(0, dtype=np.int64)


# ---------------------------------------------------------------------------
# Stage 3: sparse attention with document-wise and global RoPE
# [P1 Document-wise RoPE; P2 Overall Design > Architecture, "Parallel
#  (document-wise) RoPE and global RoPE items; P2 Inference Pipeline, stage 3
#  (sparse generation); P3 MSA Layer 工作流程 steps 4-5]
# ---------------------------------------------------------------------------

def rope_angles(pos: np.ndarray, d: int, base: float) -> np.ndarray:
    """angle[..., m] = pos * base**(-2m/d), m < d/2, in float64 (R16)."""
    m = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * m / d)
    return np.asarray(pos, dtype=np.float64)[..., None] * theta


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE: the pair (x[m], x[m + d/2]) turns by angle[m].

    x: [..., d]; pos broadcasts against x[..., 0]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a = rope_angles(pos, d, base)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attend_one(q: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray, ctx_pos: np.ndarray,
               k_loc: np.ndarray, v_loc: np.ndarray, q_pos_offset: int, base: float,
               sm_scale: float) -> np.ndarray:
    """Attention of one query (T tokens) over [retrieved context ; local].

    q: [T, Hq, d]; k_ctx/v_ctx: [n_ctx, Hkv, d] pooled, un-rotated;
    ctx_pos: [n_ctx] positions inside their documents (R11);
    k_loc/v_loc: [L_loc, Hkv, d] un-rotated.  Query token t is local token
    L_loc - T + t (R13) at position q_pos_offset + L_loc - T + t (R12); it
    sees every context entry and local tokens 0 .. L_loc - T + t.
    Returns [T, Hq, d] float64."""
    T, Hq, d = q.shape
    L_loc, Hkv = k_loc.shape[:2]
    G = Hq // Hkv
    n_ctx = k_ctx.shape[0]
    # explicit concatenation of the context (R17) and its positions
    k_all = np.concatenate([np.asarray(k_ctx, np.float64), np.asarray(k_loc, np.float64)])
    v_all = np.concatenate([np.asarray(v_ctx, np.float64), np.asarray(v_loc, np.float64)])
    pos_all = np.concatenate([np.asarray(ctx_pos, np.int64),
                              q_pos_offset + np.arange(L_loc, dtype=np.int64)])
    k_rot = rope(k_all, pos_all[:, None], base)                  # [n, Hkv, d]
    q_abs = L_loc - T + np.arange(T)                             # local index of each token
    q_rot = rope(q, (q_pos_offset + q_abs)[:, None], base)       # [T, Hq, d]
    out = np.zeros((T, Hq, d), dtype=np.float64)
    for t in range(T):
        visible = np.ones(n_ctx + L_loc, dtype=bool)
        visible[n_ctx + q_abs[t] + 1:] = False                    # causal on the local part
        for hq in range(Hq):
            g = hq // G                                           # R14
            logits = sm_scale * (k_rot[:, g, :] @ q_rot[t, hq])
            logits = np.where(visible, logits, -np.inf)
            mx = logits.max()
            p = np.exp(logits - mx)
            p /= p.sum()
            out[t, hq] = p @ v_all[:, g, :]
    return out


def sparse_attention(q: np.ndarray, contexts, k_loc: np.ndarray, v_loc: np.ndarray,
                     q_pos_offset: int, base: float, sm_scale: float | None = None) -> np.ndarray:
    """Batched form of ``attend_one``.  contexts[b] = (k_ctx, v_ctx, ctx_pos)."""
    q = np.asarray(q, dtype=np.float64)
    B, T, Hq, d = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)                                # R15
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(B):
        kc, vc, pc = contexts[b]
        out[b] = attend_one(q[b], kc, vc, pc, k_loc[b], v_loc[b], q_pos_offset, base, sm_scale)
    return out


# ---------------------------------------------------------------------------
# one routed layer, end to end (R7, R8: per layer, per query, one top-k)
# ---------------------------------------------------------------------------

def layer(q_r, kr_store, chunk_off, k_bar, v_bar, k, q, k_loc, v_loc,
          q_pos_offset=None, base=1e6, sm_scale=None, ids_override=None):
    """Route -> top-k -> assemble -> attend for one layer.

    ``ids_override`` (B x k) replaces the oracle's own selection for the
    attention step: inside the tie band several selections are correct and
    the attention is then compared on the selection actually made."""
    if q_pos_offset is None:
        q_pos_offset = k
    doc_score = route_scores(q_r, kr_store, chunk_off)
    ids, vals = topk(doc_score, k)
    use = ids if ids_override is None else np.asarray(ids_override)
    ctx = [gather(use[b], chunk_off, k_bar, v_bar) for b in range(q.shape[0])]
    out = sparse_attention(q, ctx, k_loc, v_loc, q_pos_offset, base, sm_scale)
    return dict(doc_score=doc_score, ids=ids, vals=vals, contexts=ctx, out=out)


# ---------------------------------------------------------------------------
# Memory Interleave: rounds of routing with a growing context
# [P1 核心方法 > Memory Interleave (generate doc id -> fetch -> add to the
#  query -> retrieve again); P2 Key Contributions ("generative retrieval ->
#  context expansion -> generation") and Fig. 3 ("optional multi-round
#  interleave"); P3 核心创新 > Memory Interleave]
#
# R23 the model that emits document ids is not part of this path: round r's
#     documents are the top k of round r's routing query among the documents
#     not fetched in earlier rounds.
# R24 fetched documents are appended to the context in round order (rank order
#     inside a round), each restarting its positions at 0; each round's
#     routing query is an input (in a model it follows from the grown context).
# R25 the query's global offset is the number of documents fetched (rounds x k).
# R26 the number of rounds is fixed (the model's stop decision is not modelled).
# ---------------------------------------------------------------------------

def topk_excluding(doc_score: np.ndarray, k: int, excluded) -> tuple:
    """``topk`` over the documents of each query that are not in excluded[b].
    When fewer than k documents remain, the trailing ids are -1 and their
    values NaN."""
    doc_score = np.asarray(doc_score, dtype=np.float64)
    B, D = doc_score.shape
    if k < 1 or k > D:
        raise ValueError("k must be in [1, n_docs]")
    ids = np.full((B, k), -1, dtype=np.int32)
    vals = np.full((B, k), np.nan, dtype=np.float64)
    for b in range(B):
        keep = np.ones(D, dtype=bool)
        ex = np.asarray(list(excluded[b]), dtype=np.int64)
        keep[ex[(ex >= 0) & (ex < D)]] = False
        doc = np.nonzero(keep)[0]
        order = doc[np.lexsort((doc, -doc_score[b, doc]))]
        n = min(k, len(order))
        ids[b, :n] = order[:n]
        vals[b, :n] = doc_score[b, order[:n]]
    return ids, vals


def interleave(q_r_rounds, kr_store, chunk_off, k_bar, v_bar, k, q, k_loc, v_loc, base=1e6, sm_scale=None,
               ids_override=None):
    """Rounds of route -> top-k among documents not yet fetched -> append,
    then attention over every fetched document and the local tokens (R23-R26).

    ``ids_override[r]`` (B x k) replaces round r's own selection for the
    exclusions of later rounds and for the context (inside the tie band
    several selections are correct)."""
    B = q.shape[0]
    fetched = [[] for _ in range(B)]
    rounds = []
    for r, qr in enumerate(q_r_rounds):
        doc_score = route_scores(qr, kr_store, chunk_off)
        ids, vals = topk_excluding(doc_score, k, fetched)
        rounds.append(dict(doc_score=doc_score, ids=ids, vals=vals))
        use = ids if ids_override is None else np.asarray(ids_override[r])
        for b in range(B):
            fetched[b].extend(int(x) for x in use[b] if x >= 0)
    ctx = [gather(np.asarray(fetched[b], dtype=np.int64), chunk_off, k_bar, v_bar) for b in range(B)]
    out = sparse_attention(q, ctx, k_loc, v_loc, len(q_r_rounds) * k, base, sm_scale)
    return dict(rounds=rounds, fetched=fetched, contexts=ctx, out=out)


# ---------------------------------------------------------------------------
# Training-time path: the auxiliary routing loss and the backward of the path
# [P1 训练 (continued pre-training with a generation loss plus an auxiliary
#  supervised contrastive routing loss); P2 Abstract and Key Contributions
#  (the layer is trainable end to end); P2 Implementation Notes (auxiliary
#  routing loss)]
#
# R27 routing-loss form (the pages name it only): per query b and routed
#     layer, the supervised contrastive loss of the query against all
#     documents with the positive set P_b,
#       L_b = -(1/|P_b|) sum_{p in P_b} log( exp(s_bp / tau) / sum_i exp(s_bi / tau) ),
#     s the routing scores of the layer, tau a temperature (an input); empty
#     documents (score -inf) carry no weight.
# R28 the derivative of the token/chunk max goes to one maximiser: the
#     smallest chunk index, then the smallest token, among those attaining it.
# R29 x / max(||x||, eps) has derivative (I - xh xh^T) / ||x|| when
#     ||x|| > eps, else I / eps.
# R30 the selection (ids, context order and positions) is held fixed; the
#     attention's gradients reach the query, the local K/V and the selected
#     pooled rows, summed over every query and context entry that reads a row,
#     and from the pooled rows the tokens of their chunk (the mean's adjoint).
# R31 the store rounding (R18) is taken as the identity in the backward; the
#     routing keys' gradient is taken at the normalised pooled entry and
#     carried through the normalisation (R29) and the pooling to the tokens.
# ---------------------------------------------------------------------------

def route_loss(doc_score: np.ndarray, pos_ids: np.ndarray, tau: float):
    """Routing loss per query (R27) and its gradient with respect to the scores.

    doc_score: [B, D]; pos_ids: [B, P] document ids, -1 = padding (at least one
    valid id per query).  Returns (loss [B], grad [B, D]) with
    grad[b, i] = (softmax(s_b / tau)[i] - [i in P_b] / |P_b|) / tau."""
    s = np.asarray(doc_score, dtype=np.float64)
    B, D = s.shape
    loss = np.zeros(B, dtype=np.float64)
    grad = np.zeros((B, D), dtype=np.float64)
    for b in range(B):
        pos = sorted({int(p) for p in np.asarray(pos_ids[b]).ravel() if 0 <= p < D})
        if not pos:
            raise ValueError("every query needs a positive document")
        z = s[b] / tau
        mx = z[np.isfinite(z)].max()
        lse = mx + np.log(np.exp(z - mx).sum())
        loss[b] = -np.mean([z[p] - lse for p in pos])
        target = np.zeros(D)
        target[pos] = 1.0 / len(pos)
        grad[b] = (np.exp(z - lse) - target) / tau
    return loss, grad


def route_argmax(q_r: np.ndarray, kr_store: np.ndarray, chunk_off: np.ndarray, eps: float = EPS):
    """Routing scores with the maximiser of each (query, document) (R28).

    Returns (doc_score [B, D], arg_chunk [B, D], arg_tok [B, D]); the
    maximiser is the global chunk index and the query token; -1 for an empty
    document."""
    s = chunk_cosines(q_r, kr_store, eps)          # [B, T, N]
    B, T, N = s.shape
    chunk_off = np.asarray(chunk_off, dtype=np.int64)
    D = len(chunk_off) - 1
    score = np.full((B, D), -np.inf)
    ac = np.full((B, D), -1, dtype=np.int64)
    at = np.full((B, D), -1, dtype=np.int64)
    for b in range(B):
        for i in range(D):
            lo, hi = int(chunk_off[i]), int(chunk_off[i + 1])
            if hi == lo:
                continue
            block = s[b, :, lo:hi].T                # [chunks, T], chunk-major
            flat = int(np.argmax(block))            # first maximiser: chunk, then token
            c, t = divmod(flat, T)
            score[b, i], ac[b, i], at[b, i] = block[c, t], lo + c, t
    return score, ac, at


def normalize_backward(x: np.ndarray, dy: np.ndarray, eps: float = EPS) -> np.ndarray:
    """Gradient with respect to x of y = x / max(||x||, eps) over the last axis (R29)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    big = n > eps
    xh = x / np.where(big, n, 1.0)
    proj = dy - xh * (xh * dy).sum(axis=-1, keepdims=True)
    return np.where(big, proj / np.where(big, n, 1.0), dy / eps)


def route_score_backward(q_r: np.ndarray, kr_store: np.ndarray, arg_chunk: np.ndarray, arg_tok: np.ndarray,
                         grad: np.ndarray, eps: float = EPS):
    """Gradients of sum_{b,i} grad[b, i] * s[b, i] with respect to the raw
    routing queries and the (normalised) store entries (R28, R29, R31).

    s[b, i] = (1/H) sum_h qhat[b, t*, h] . kr[c*, h] at the maximiser
    (c*, t*) = (arg_chunk, arg_tok).  Returns (dq_r [B, T, H, d],
    dkr [N, H, d])."""
    q = np.asarray(q_r, dtype=np.float64)
    kr = np.asarray(kr_store, dtype=np.float64)
    B, T, H, d = q.shape
    qh = l2_normalize(q, eps)
    dqh = np.zeros_like(q)
    dkr = np.zeros_like(kr)
    for b in range(B):
        for i in range(arg_chunk.shape[1]):
            c, t = int(arg_chunk[b, i]), int(arg_tok[b, i])
            if c < 0 or grad[b, i] == 0.0:
                continue
            w = grad[b, i] / H
            dqh[b, t] += w * kr[c]
            dkr[c] += w * qh[b, t]
    return normalize_backward(q, dqh, eps), dkr


def pool_backward(dy: np.ndarray, tok_off: np.ndarray, chunk: int, x: np.ndarray | None = None,
                  eps: float = EPS) -> np.ndarray:
    """Adjoint of ``pool``: token tau of chunk c receives dy[c] / n_c.  With x
    (the token vectors) the pooled entry was L2-normalised (R2): dy is then
    the gradient at the normalised entry and is first carried through the
    normalisation of the chunk mean (R29, R31).  Returns [n_tok, H, d]."""
    dy = np.asarray(dy, dtype=np.float64)
    tok_off = np.asarray(tok_off, dtype=np.int64)
    if x is not None:
        dy = normalize_backward(pool(x, tok_off, chunk), dy, eps)
    n_tok = int(tok_off[-1])
    out = np.zeros((n_tok,) + dy.shape[1:], dtype=np.float64)
    c = 0
    for i in range(len(tok_off) - 1):
        lo, hi = int(tok_off[i]), int(tok_off[i + 1])
        for s0 in range(lo, hi, chunk):
            e = min(s0 + chunk, hi)
            out[s0:e] = dy[c] / (e - s0)
            c += 1
    return out


def attend_one_backward(q: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray, ctx_pos: np.ndarray,
                        k_loc: np.ndarray, v_loc: np.ndarray, q_pos_offset: int, base: float,
                        sm_scale: float, dout: np.ndarray):
    """Gradients of sum(attend_one(...) * dout) with respect to q, the context
    entries and the local K/V (R30), each at the un-rotated input.

    Softmax rows p, dp = dout . v, ds = p * (dp - sum(p * dp)); the rotated
    query and keys receive sm_scale * ds times the other operand; a rotation's
    adjoint is the rotation by the opposite angle.  Returns (dq [T, Hq, d],
    dk_ctx, dv_ctx [n_ctx, Hkv, d], dk_loc, dv_loc [L_loc, Hkv, d])."""
    T, Hq, d = q.shape
    L_loc, Hkv = k_loc.shape[:2]
    G = Hq // Hkv
    n_ctx = k_ctx.shape[0]
    k_all = np.concatenate([np.asarray(k_ctx, np.float64), np.asarray(k_loc, np.float64)])
    v_all = np.concatenate([np.asarray(v_ctx, np.float64), np.asarray(v_loc, np.float64)])
    pos_all = np.concatenate([np.asarray(ctx_pos, np.int64),
                              q_pos_offset + np.arange(L_loc, dtype=np.int64)])
    k_rot = rope(k_all, pos_all[:, None], base)
    q_abs = L_loc - T + np.arange(T)
    q_pos = (q_pos_offset + q_abs)[:, None]
    q_rot = rope(q, q_pos, base)
    dout = np.asarray(dout, dtype=np.float64)
    dq_rot = np.zeros_like(q_rot)
    dk_rot = np.zeros_like(k_rot)
    dv_all = np.zeros_like(v_all)
    for t in range(T):
        visible = np.ones(n_ctx + L_loc, dtype=bool)
        visible[n_ctx + q_abs[t] + 1:] = False
        for hq in range(Hq):
            g = hq // G
            logits = sm_scale * (k_rot[:, g, :] @ q_rot[t, hq])
            logits = np.where(visible, logits, -np.inf)
            p = np.exp(logits - logits.max())
            p /= p.sum()
            dp = v_all[:, g, :] @ dout[t, hq]
            ds = p * (dp - (p * dp).sum())
            dq_rot[t, hq] = sm_scale * (ds @ k_rot[:, g, :])
            dk_rot[:, g, :] += sm_scale * np.outer(ds, q_rot[t, hq])
            dv_all[:, g, :] += np.outer(p, dout[t, hq])
    dq = rope(dq_rot, -q_pos, base)
    dk_all = rope(dk_rot, -pos_all[:, None], base)
    return dq, dk_all[:n_ctx], dv_all[:n_ctx], dk_all[n_ctx:], dv_all[n_ctx:]


def sparse_attention_backward(q: np.ndarray, contexts, k_loc: np.ndarray, v_loc: np.ndarray, q_pos_offset: int,
                              base: float, dout: np.ndarray, sm_scale: float | None = None):
    """Batched ``attend_one_backward``.  Returns (dq, ctx_grads, dk_loc, dv_loc)
    with ctx_grads[b] = (dk_ctx, dv_ctx) per context entry of query b."""
    q = np.asarray(q, dtype=np.float64)
    B, T, Hq, d = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    dq = np.zeros(q.shape)
    dk_loc = np.zeros(np.shape(k_loc))
    dv_loc = np.zeros(np.shape(v_loc))
    ctx_grads = []
    for b in range(B):
        kc, vc, pc = contexts[b]
        dq[b], dkc, dvc, dk_loc[b], dv_loc[b] = attend_one_backward(
            q[b], kc, vc, pc, k_loc[b], v_loc[b], q_pos_offset, base, sm_scale, dout[b])
        ctx_grads.append((dkc, dvc))
    return dq, ctx_grads, dk_loc, dv_loc


def gather_backward(ids: np.ndarray, chunk_off: np.ndarray, ctx_grads, n_chunks: int):
    """Adjoint of ``gather`` over all queries: each context entry's gradient is
    added to the pooled row it was read from (R30).  Returns (dk_bar, dv_bar)
    [n_chunks, Hkv, d]."""
    dkb = dvb = None
    for b, (dk, dv) in enumerate(ctx_grads):
        if dkb is None:
            dkb = np.zeros((n_chunks,) + dk.shape[1:])
            dvb = np.zeros((n_chunks,) + dv.shape[1:])
        e = 0
        for doc in ids[b]:
            if doc < 0:
                continue
            lo, hi = int(chunk_off[doc]), int(chunk_off[doc + 1])
            dkb[lo:hi] += dk[e:e + hi - lo]
            dvb[lo:hi] += dv[e:e + hi - lo]
            e += hi - lo
    return dkb, dvb


# ---------------------------------------------------------------------------
# Stage 1 from hidden states: projection, then the chunk-wise pool
# [P2 Inference Pipeline, stage 1, global memory encoding (a forward over the corpus
#  caches the chunk-pooled K, V, K_r); P1 架构 (each document's K/V/K_r, the
#  routing key from an extra projector, chunk-wise mean pooled)]
#
# R32 K, V and K_r are linear projections of the token's hidden state (no
#     per-token normalisation before the pool); K is stored un-rotated (R11).
# ---------------------------------------------------------------------------

def encode(x: np.ndarray, w_t: np.ndarray, tok_off: np.ndarray, chunk: int, H: int, d: int, dtype: str):
    """Pooled stores of a memory from its tokens' hidden states (R32).

    x: [n_tok, hidden]; w_t: [3*H*d, hidden], one row per output feature:
    rows h*d + e of K, then of V, then of K_r.  Every token is projected,
    then ``pool_encode`` pools (and, for K_r, normalises) and rounds.
    Returns (k_bar, v_bar, kr_hat), each [n_chunks, H, d]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_t, dtype=np.float64)
    Hd = H * d
    proj = x @ w.T
    k = proj[:, :Hd].reshape(-1, H, d)
    v = proj[:, Hd:2 * Hd].reshape(-1, H, d)
    r = proj[:, 2 * Hd:].reshape(-1, H, d)
    return (pool_encode(k, tok_off, chunk, False, dtype), pool_encode(v, tok_off, chunk, False, dtype),
            pool_encode(r, tok_off, chunk, True, dtype))
