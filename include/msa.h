/*
 * msa.h - C ABI of the MSA (Memory Sparse Attention) online-routing and
 * sparse-attention hot path for AMD Instinct MI355X (gfx950).
 *
 * The calls follow the three-stage inference pipeline of "MSA: Memory
 * Sparse Attention" (project README, Overall Design > Inference Pipeline):
 *   Stage 1, Global Memory Encoding  -> msa_pool_encode
 *   Stage 2, Online Routing & Context Assembly
 *                                     -> msa_route_score, msa_topk, msa_gather_kv
 *                                        (or msa_context_index for a store in HBM)
 *   Stage 3, Sparse Generation        -> msa_sparse_attn (msa_sparse_attn_indexed)
 * The layer itself is described in the README's Overall Design > Architecture
 * and in the "MSA-arXiv26" paper note, section 核心方法 > 架构 and
 * Document-wise RoPE.
 *
 * Conventions shared by every call
 *  - Return value: an msa_status.  Arguments are validated on the host before
 *    any HIP call; an invalid call enqueues nothing.  msa_last_error() gives a
 *    human-readable detail of the last failure on the calling thread.
 *  - Ownership: the caller owns every buffer.  The library allocates no
 *    device or host memory; scratch space comes from the caller through
 *    `ws` / `ws_bytes`, sized by the matching *_workspace query.  (The one
 *    exception is msa_route_balance, a setup-time calibration that allocates
 *    and frees a 4 KB timing buffer.)
 *  - Pointers are device pointers unless the name ends in `_h` (host).
 *    Device buffers must be 16-byte aligned.
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the
 *    null stream) and the call returns.  The one host synchronisation is
 *    msa_gather_kv in MSA_SRC_HOST_MEMCPY mode (documented there).
 *  - Layouts are row-major with the last index contiguous.  Offsets are
 *    int64; document ids, chunk->document maps, positions and lengths are
 *    int32.
 *  - dtype: MSA_F32 or MSA_BF16 (bfloat16 stored as its 16-bit pattern).
 *  - Device faults of an enqueued kernel surface as MSA_ERR_HIP from the
 *    launch check or at the caller's next synchronisation.
 *  - Calls on distinct streams may run from different threads.  The one
 *    mutable global state is the per-device XCD split of the routing scan set
 *    by msa_route_balance (guarded by a lock); it changes how later routing
 *    launches divide their chunks, never their results.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1, /* a pointer, size or relation between sizes is wrong */
  MSA_ERR_UNSUPPORTED = 2, /* valid, but outside what the kernels implement     */
  MSA_ERR_WORKSPACE = 3,   /* ws_bytes smaller than the *_workspace query       */
  MSA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed        */
} msa_status;

typedef enum { MSA_F32 = 0, MSA_BF16 = 1 } msa_dtype;

typedef enum {
  MSA_LAYOUT_ROWS = 0,  /* [n_chunks, H, d], row-major                                   */
  MSA_LAYOUT_TILED = 1  /* groups of 16 chunks stored as [H][d/32][4][16][8]: chunk c, head h,
                           element e sits at (c/16)*16*H*d + h*16*d + (e/32)*512 + ((e%32)/8)*128
                           + (c%16)*8 + e%8.  Needs d % 32 == 0; the buffer holds
                           ceil(n_chunks/16)*16 chunks and the padding chunks are zero.  It is
                           the MFMA operand order of msa_route_score: every 16-byte-per-lane
                           load of a wave reads 1 KB contiguous.                             */
} msa_layout;

typedef enum {
  MSA_SRC_DEVICE = 0,      /* K/V store in device memory (HBM)                          */
  MSA_SRC_HOST_MAPPED = 1, /* store in pinned host memory, read by the gather kernel     */
  MSA_SRC_HOST_MEMCPY = 2  /* store in pinned host memory, copied with hipMemcpyAsync on
                              a side stream                                             */
} msa_src_mode;

typedef enum {
  MSA_ATTN_PART_LOCAL = 1,   /* msa_sparse_attn_part: the local-window keys only          */
  MSA_ATTN_PART_CONTEXT = 2  /* msa_sparse_attn_part: the context keys, then the merge    */
} msa_attn_part;

typedef enum {
  MSA_ROUTE_PREFILLED = 1    /* msa_route_score: doc_score already holds -inf everywhere (left so
                                by msa_topk with MSA_TOPK_RESET_SCORES); the call skips its fill */
} msa_route_flags;

typedef enum {
  MSA_TOPK_RESET_SCORES = 1  /* msa_topk, msa_topk_context_index: write -inf over doc_score as it
                                is read, ready for the next layer's MSA_ROUTE_PREFILLED call     */
} msa_topk_flags;

/* Version of this ABI (bumped on any signature or workspace-layout change, and on added calls). */
int msa_abi_version(void);

/* Static description of a status code. */
const char* msa_status_string(int status);

/* Detail message of the last failing call on this thread ("" if none). */
const char* msa_last_error(void);

/*
 * msa_chunk_offsets (host only) - the chunk CSR of a tokenised memory.
 * Chunk-wise pooling compresses each document on its own (README, Overall
 * Design > Architecture: document latent states are chunk-mean pooled), so
 * document i of len_i = tok_off_h[i+1] - tok_off_h[i] tokens owns
 * ceil(len_i / chunk) pooled chunks; the last one may be partial.
 *   tok_off_h   [n_docs + 1] non-decreasing, tok_off_h[0] == 0 (host)
 *   chunk_off_h [n_docs + 1] output (host)
 * Errors: INVALID_ARG for NULL pointers, n_docs < 1, chunk < 1, a decreasing
 * or non-zero-based tok_off_h.
 */
int msa_chunk_offsets(const int64_t* tok_off_h, int64_t n_docs, int chunk, int64_t* chunk_off_h);

/*
 * msa_chunk_doc_map - inverse of the chunk CSR: chunk_doc[c] = the document
 * that owns pooled chunk c (README, Inference Pipeline: per-document top-k
 * needs every chunk's document).  Built once per memory, read by
 * msa_pool_encode and msa_route_score.
 *   chunk_off [n_docs + 1] device, non-decreasing, chunk_off[n_docs] == n_chunks
 *   chunk_doc [n_chunks]   device output
 * Errors: INVALID_ARG for NULL pointers or n_docs < 1, n_chunks < 1.
 */
int msa_chunk_doc_map(const int64_t* chunk_off, int64_t n_docs, int64_t n_chunks, int32_t* chunk_doc,
                      void* stream);

/*
 * msa_tile_routing_keys - reorder a row-major pooled routing-key store
 * [n_chunks, H, d] into MSA_LAYOUT_TILED (see msa_layout), zeroing the
 * padding chunks of the last group.  A pure permutation (bit-exact).
 *   src [n_chunks, H, d] dtype; dst ceil(n_chunks/16)*16 chunks, dtype
 * Errors: INVALID_ARG (NULL, sizes, d % 32 != 0, src == dst).
 */
int msa_tile_routing_keys(int dtype, const void* src, int64_t n_chunks, int H, int d, void* dst, void* stream);

/*
 * msa_pool_encode - Stage 1 (global memory encoding, README Inference
 * Pipeline; mean pooling per chunk, paper note 核心方法 > 架构).
 * For pooled chunk c = chunk j of document i and head h:
 *   out[c,h,:] = mean of x[t,h,:] over the tokens t of that chunk
 *                (tokens tok_off[i] + j*chunk ... min(+chunk, tok_off[i+1]) - 1;
 *                a partial last chunk averages the tokens it has),
 *   and if l2_normalize: out[c,h,:] /= max(||out[c,h,:]||_2, 1e-8)
 *   (the routing keys, compared by cosine similarity).
 * Accumulation is float32; each output is rounded once (to nearest even)
 * to dtype.  Keys and values are stored un-rotated: RoPE is applied at
 * attention time.
 *   x         [n_tok, H, d] dtype
 *   tok_off   [n_docs + 1] int64, chunk_off [n_docs + 1] int64 (chunk CSR of
 *             tok_off for this chunk size), chunk_doc [n_chunks] int32
 *   out       [n_chunks, H, d] dtype in out_layout (msa_layout; MSA_LAYOUT_TILED
 *             needs d % 32 == 0 and room for ceil(n_chunks/16)*16 chunks);
 *             must not overlap x (workgroups write their chunks while others
 *             still read tokens)
 * Errors: INVALID_ARG (NULL, non-positive sizes, d odd, bad layout, x not
 * 16-byte aligned, out == x), UNSUPPORTED (H*d > 4096 or H*d not a multiple of 8, or
 * a token row of n = H*d*bytes/16 16-byte vectors where n neither divides
 * 256 nor is a multiple of 256 and is not covered by the wave-per-chunk
 * kernel: n a multiple of 64 with each head d*bytes/16 vectors, a power of
 * two up to 64).
 */
int msa_pool_encode(int dtype, const void* x, const int64_t* tok_off, const int64_t* chunk_off,
                    const int32_t* chunk_doc, int64_t n_docs, int64_t n_tok, int64_t n_chunks, int H,
                    int d, int chunk, int l2_normalize, int out_layout, void* out, void* stream);

/*
 * msa_encode - Stage 1 at corpus scale (global memory encoding, README
 * Inference Pipeline; paper note 核心方法 > 架构: each document's K, V and
 * routing key K_r - the latter from an extra projector - chunk-wise mean
 * pooled).  From the hidden states x of the memory's tokens and the
 * projection weights, for pooled chunk c, head h:
 *   k_bar[c,h,:]  = mean over the chunk's tokens t of (x[t,:] . W_k[h*d + e, :])_e
 *   v_bar[c,h,:]  = the same with W_v
 *   kr_hat[c,h,:] = the same with W_r, then / max(||.||_2, 1e-8)
 * i.e. msa_pool_encode of the projected tokens (reading: the projections are
 * linear, nothing is applied per token before the pool; K is stored
 * un-rotated).  Since the mean commutes with the projection, the library
 * pools the hidden states first (float32) and projects the pooled rows; bf16
 * with d = 128 runs on MFMA with exact products.  Each output is rounded once
 * to dtype.
 *   x     [n_tok, hidden] dtype;  w_t [3*H*d, hidden] dtype: one row per output
 *         feature, rows 0..H*d-1 for K, then V, then K_r (feature h*d + e)
 *   tok_off, chunk_off, chunk_doc as for msa_pool_encode
 *   k_bar, v_bar [n_chunks, H, d] dtype (rows); kr_hat in kr_layout (MSA_LAYOUT_TILED
 *         needs d % 32 == 0 and room for ceil(n_chunks/16)*16 chunks, padding zeroed)
 *   ws    msa_encode_workspace() bytes
 * Errors: INVALID_ARG (NULL, sizes, layout, alignment), UNSUPPORTED (hidden not
 * a whole number of 16-byte vectors), WORKSPACE.
 */
size_t msa_encode_workspace(int dtype, int64_t n_chunks, int hidden, int H, int d);
int msa_encode(int dtype, const void* x, const void* w_t, int hidden, int H, int d, const int64_t* tok_off,
               const int64_t* chunk_off, const int32_t* chunk_doc, int64_t n_docs, int64_t n_tok, int64_t n_chunks,
               int chunk, int kr_layout, void* k_bar, void* v_bar, void* kr_hat, void* ws, size_t ws_bytes,
               void* stream);

/*
 * msa_encode_pool, msa_encode_project - the two halves of msa_encode, for a
 * caller that overlaps one block's pooling with the previous block's
 * projection on two streams (the pool reads the hidden states at HBM rate,
 * the projection runs on MFMA).  msa_encode_pool writes the block's pooled
 * rows into ws; msa_encode_project reads them from ws (same sizes: the
 * workspace is the hand-off) and writes k_bar, v_bar and kr_hat.  Their
 * composition on one stream is msa_encode, bit for bit.  Arguments, errors
 * and the workspace size are those of msa_encode; ws must hold the pool's
 * result when the projection starts (the caller orders the two streams), and
 * a double-buffered caller uses one workspace per block in flight.
 */
int msa_encode_pool(int dtype, const void* x, int hidden, int H, int d, const int64_t* tok_off,
                    const int64_t* chunk_off, const int32_t* chunk_doc, int64_t n_docs, int64_t n_tok,
                    int64_t n_chunks, int chunk, void* ws, size_t ws_bytes, void* stream);
int msa_encode_project(int dtype, const void* w_t, int hidden, int H, int d, int64_t n_chunks, int kr_layout,
                       void* k_bar, void* v_bar, void* kr_hat, const void* ws, size_t ws_bytes, void* stream);

/*
 * msa_route_score - Stage 2 routing score (README, Overall Design >
 * Architecture: each chunk's cosine with the routing query is averaged across
 * heads, and the largest value over the query's tokens is kept; paper note
 * 核心方法 > 架构: every document's compressed routing key is compared by
 * cosine).  For query b and document i:
 *   doc_score[b,i] = max over tokens t < T and chunks c of document i of
 *                    (1/H) * sum_h < q_r[b,t,h,:] / max(||q_r[b,t,h,:]||, 1e-8), kr_hat[c,h,:] >
 * kr_hat must already be L2-normalised (msa_pool_encode with l2_normalize),
 * so the dot product is the cosine.  A document with no chunk scores -inf.
 * Products are exact (bf16 x bf16 or f32 x f32) with float32 accumulation;
 * the query norm is applied per (token, head) in float32.  The score matrix
 * is never materialised; the store is streamed once.
 *   q_r        [B, T, H, d] dtype (raw routing queries)
 *   kr_hat     [n_chunks, H, d] dtype in kr_layout (msa_layout).  The MFMA
 *              path (bf16, H = 8, d = 128) streams MSA_LAYOUT_TILED at full
 *              HBM rate; MSA_LAYOUT_ROWS is accepted by every path.
 *   chunk_doc  [n_chunks] int32 (msa_chunk_doc_map); entries outside
 *              [0, n_docs) are ignored; the valid entries must be
 *              non-decreasing (each document's chunks contiguous, as the
 *              chunk CSR lays them out)
 *   doc_score  [B, n_docs] float32 output
 *   ws         msa_route_score_workspace() bytes (may be 0 -> ws may be NULL)
 * Errors: INVALID_ARG (NULL, non-positive sizes, bad layout), WORKSPACE,
 * UNSUPPORTED (d > 256 or d % 8 != 0; MSA_LAYOUT_TILED outside the MFMA path).
 *   flags      0, or MSA_ROUTE_PREFILLED: the call does not fill doc_score
 *              with -inf first (a separate launch); the caller guarantees
 *              that every entry already holds -inf, as a previous msa_topk
 *              with MSA_TOPK_RESET_SCORES on the same buffer leaves it.  Any
 *              other content is max-combined into the result (wrong scores,
 *              no error).
 */
size_t msa_route_score_workspace(int dtype, int B, int T, int H, int d, int64_t n_docs, int64_t n_chunks);
int msa_route_score(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat, int kr_layout,
                    const int32_t* chunk_doc, int64_t n_docs, int64_t n_chunks, float* doc_score,
                    void* ws, size_t ws_bytes, int flags, void* stream);

/*
 * msa_route_score_fetch - msa_route_score of one routing call, with the
 * context assembly of a selection it does not depend on done inside the same
 * launch (README, Overall Design > Inference Pipeline: the content K/V stays
 * in host memory and the selected documents are fetched asynchronously).
 * The scan's workgroups that finish their chunk ranges first copy the
 * selected documents, one (query, rank) at a time, while the others still
 * stream: the host link and the HBM scan overlap.  The order suits
 * independent queries served together (one query's fetch inside another's
 * routing); one query's next-layer routing needs this layer's attention
 * output, so its own layers cannot use it.  Results are exactly those of
 * msa_route_score followed by msa_gather_kv in MSA_SRC_DEVICE /
 * MSA_SRC_HOST_MAPPED mode.
 *   routing arguments and flags as msa_route_score
 *   f_ids       [f_B, f_k] int32: the selection to fetch (msa_topk)
 *   f_chunk_off [f_n_docs + 1] int64 (device) of its documents
 *   f_k_bar, f_v_bar [n, f_Hkv, f_d] dtype: its content store, in device
 *               memory or in pinned host memory the GPU can map
 *   f_max_ctx, f_k_ctx, f_v_ctx [f_B, f_max_ctx, f_Hkv, f_d], f_ctx_pos
 *               [f_B, f_max_ctx], f_ctx_len [f_B]: as msa_gather_kv's outputs
 *   ws          msa_route_score_fetch_workspace() bytes: the routing
 *               workspace, then 256 bytes for the fetch's counter (no
 *               initial contents needed; the launch clears it)
 * The fetch's outputs must not be read by anything running beside the call.
 * Off the MFMA path the two calls run one after the other.
 * Errors: those of msa_route_score and msa_gather_kv; WORKSPACE.
 */
size_t msa_route_score_fetch_workspace(int dtype, int B, int T, int H, int d, int64_t n_docs, int64_t n_chunks);
int msa_route_score_fetch(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat, int kr_layout,
                          const int32_t* chunk_doc, int64_t n_docs, int64_t n_chunks, float* doc_score, void* ws,
                          size_t ws_bytes, int flags, const int32_t* f_ids, int f_B, int f_k,
                          const int64_t* f_chunk_off, int64_t f_n_docs, int f_max_doc_chunks, const void* f_k_bar,
                          const void* f_v_bar, int f_Hkv, int f_d, int f_max_ctx, void* f_k_ctx, void* f_v_ctx,
                          int32_t* f_ctx_pos, int32_t* f_ctx_len, void* stream);

/*
 * msa_route_balance - sizes msa_route_score's chunk ranges per XCD on the
 * current device (not a step of the method: a calibration of how the scan is
 * spread over MI355X's eight XCDs).  Workgroup b of the scan runs on XCD
 * b % 8; when the XCDs stream at different rates, equal ranges leave the
 * launch waiting for the slowest.  The call runs four untimed routing
 * launches, then `rounds` rounds of three timed ones, on the caller's
 * arguments (those of msa_route_score;
 * doc_score receives the scores), and after each round moves every XCD's
 * share by the ratio of the XCDs' mean workgroup end time to its own (each
 * share kept within 0.75x..1.25x of 1/8).  Later msa_route_score and
 * msa_chunk_scores calls on this device use the shares wherever the scan runs
 * one workgroup per CU (a chunk range, or a range and its column groups of 64
 * query columns) and every range holds at least 128 tiles of 16 chunks
 * (shorter scans measured no faster); the calibration needs such a scan too.
 * Elsewhere ranges stay equal.  Scores
 * do not depend on the split (maxima are exact): only the launch time does.
 *   rounds      0 clears the device's shares (equal ranges again); at most 64
 *   shares_out  8 floats (host), may be NULL: the shares in use after the call
 *               (unchanged when the shape cannot be calibrated: then nothing is stored)
 * Setup-time call: it allocates a small device buffer, synchronises the stream
 * and must not be captured into a graph.  Errors: those of msa_route_score;
 * INVALID_ARG also for rounds outside [0, 64].
 */
int msa_route_balance(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat, int kr_layout,
                      const int32_t* chunk_doc, int64_t n_docs, int64_t n_chunks, float* doc_score, void* ws,
                      size_t ws_bytes, int rounds, float* shares_out, void* stream);

/*
 * msa_chunk_scores, msa_segment_max - msa_route_score in two launches (the
 * same definition, README Overall Design > Architecture): the per-chunk
 * scores, then a standalone segmented max by document.  For every chunk c
 *   chunk_score[b,c] = max over tokens t < T of
 *                      (1/H) * sum_h < q_r[b,t,h,:] / max(||q_r[b,t,h,:]||, 1e-8), kr_hat[c,h,:] >
 * and then
 *   doc_score[b,i] = max over c in [chunk_off[i], chunk_off[i+1]) of chunk_score[b,c]
 * (-inf for an empty document).  Max is exact, so the composition equals
 * msa_route_score bit for bit; msa_route_score fuses the second step into the
 * scan and never writes the [B, n_chunks] scores.
 *   msa_chunk_scores: arguments as msa_route_score without the document map;
 *     chunk_score [B, n_chunks] float32 output; the workspace is
 *     msa_route_score_workspace(dtype, B, T, H, d, n_chunks, n_chunks) bytes.
 *     UNSUPPORTED also for n_chunks >= 2^31.
 *   msa_segment_max: chunk_score [B, n_chunks] float32, chunk_off [n_docs+1]
 *     int64 (device), doc_score [B, n_docs] float32 output.  Offsets outside
 *     [0, n_chunks] are clamped.  INVALID_ARG for NULL or non-positive sizes.
 */
int msa_chunk_scores(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat, int kr_layout,
                     int64_t n_chunks, float* chunk_score, void* ws, size_t ws_bytes, void* stream);
int msa_segment_max(const float* chunk_score, int B, int64_t n_chunks, const int64_t* chunk_off, int64_t n_docs,
                    float* doc_score, void* stream);

/*
 * msa_topk - Stage 2 selection (README, Overall Design > Architecture:
 * the router keeps the k best documents; paper note 核心方法 > 架构: top-k documents by
 * cosine similarity).  For each query b the k documents with the largest
 * doc_score, ordered by (score descending, document id ascending); ties are
 * broken by the lower id, so the result is unique.
 *   doc_score [B, n_docs] float32; a NaN score marks an excluded document
 *              (msa_exclude_docs), which is never selected
 *   ids       [B, k] int32 output, vals [B, k] float32 output (rank order);
 *              when fewer than k documents are left, the trailing ids are -1
 *              (their vals NaN)
 *   ws        msa_topk_workspace() bytes
 *   flags     0, or MSA_TOPK_RESET_SCORES: the first selection pass writes
 *              -inf over each score once it has read it, so doc_score leaves
 *              the call ready for msa_route_score with MSA_ROUTE_PREFILLED
 *              (the fill moves into a pass that reads the buffer anyway);
 *              doc_score then no longer holds the scores
 * Errors: INVALID_ARG (NULL, B < 1, k < 1, k > n_docs, unknown flags),
 * UNSUPPORTED (k > 256), WORKSPACE.
 */
size_t msa_topk_workspace(int B, int64_t n_docs, int k);
int msa_topk(float* doc_score, int B, int64_t n_docs, int k, int32_t* ids, float* vals, void* ws,
             size_t ws_bytes, int flags, void* stream);

/*
 * msa_topk_merge - Memory Parallel's global reduce (README, Overall Design >
 * Inference Pipeline: the routing keys are sharded over GPUs, each scores its
 * shard and a global reduce follows; paper note 核心方法 > Memory Parallel 推理).
 * G shards each ran msa_route_score + msa_topk over a contiguous range of the
 * documents with shard-local ids; for each query b the result is the k best of
 * their entries by (score descending, global id ascending), which equals
 * msa_topk over the whole memory when every shard kept at least min(k, its
 * documents) entries.
 *   vals      [G, B, k_in] float32 device, ids [G, B, k_in] int32 device:
 *              shard g's lists; a slot with id < 0 or a NaN score is empty
 *   id_offset [G] int64 device: the global id of shard g's first document
 *              (global ids must stay below 2^31)
 *   ids_out   [B, k] int32 output (global ids), vals_out [B, k] float32 output;
 *              when fewer than k entries are valid the trailing ids are -1
 *              (their vals NaN)
 * Errors: INVALID_ARG (NULL, non-positive sizes, k > G * k_in),
 * UNSUPPORTED (k > 64, G * k_in > 2^24).
 */
int msa_topk_merge(const float* vals, const int32_t* ids, const int64_t* id_offset, int G, int B, int k_in, int k,
                   int32_t* ids_out, float* vals_out, void* stream);

/*
 * msa_exclude_docs - Memory Interleave (paper note 核心方法 > Memory
 * Interleave; README, Key Contributions and Fig. 3: rounds of retrieval, each
 * adding documents to the context).  Marks the documents fetched in earlier
 * rounds so that the next msa_topk skips them:
 *   doc_score[b, ids[s, b, j]] = NaN   for s < n_sets, j < k
 *   doc_score [B, n_docs] float32, updated in place (after msa_route_score)
 *   ids       [n_sets, B, k] int32 device (earlier rounds' msa_topk ids);
 *             ids outside [0, n_docs) (-1 included) are ignored
 * Errors: INVALID_ARG (NULL, sizes).  n_sets = 0 does nothing.
 */
int msa_exclude_docs(float* doc_score, int B, int64_t n_docs, const int32_t* ids, int n_sets, int k, void* stream);

/*
 * msa_gather_kv - Stage 2 context assembly (README, Inference Pipeline:
 * only the selected documents' K/V are loaded; tiered storage with the content K/V in host
 * DRAM fetched when selected: README Inference Pipeline and paper note
 * Memory Parallel 推理).  For query b:
 *   the context is the chunks of documents ids[b,0], ids[b,1], ... (rank
 *   order), each document's chunks in order:
 *     k_ctx[b,e,:,:] = k_bar[c,:,:], v_ctx[b,e,:,:] = v_bar[c,:,:],
 *     ctx_pos[b,e]   = c - chunk_off[doc]   (position inside the document,
 *                                            document-wise RoPE)
 *   ctx_len[b] = sum of the selected documents' chunk counts.
 * Entries e >= ctx_len[b] are left untouched.
 *   ids        [B, k] int32 (device); ids outside [0, n_docs) are an error
 *              only in the sense that they contribute no entries
 *   chunk_off  [n_docs + 1] int64 device; chunk_off_h the same on the host
 *              (required for MSA_SRC_HOST_MEMCPY, else may be NULL)
 *   k_bar/v_bar [n_chunks, Hkv, d] dtype: device memory (MSA_SRC_DEVICE) or
 *              pinned host memory from hipHostMalloc (the two host modes)
 *   max_doc_chunks  an upper bound of any document's chunk count
 *   k_ctx/v_ctx [B, max_ctx, Hkv, d] dtype, ctx_pos [B, max_ctx] int32,
 *   ctx_len [B] int32 outputs
 *   ids_h      pinned host staging of B*k int32 (MSA_SRC_HOST_MEMCPY only)
 *   copy_stream  side stream of the host copies (MSA_SRC_HOST_MEMCPY only);
 *              `stream` waits for it before returning work on `stream`.
 * MSA_SRC_HOST_MEMCPY copies the ids to ids_h and synchronises `stream`
 * once (the host must know the selection to issue the copies).
 * Errors: INVALID_ARG (NULL, sizes, max_ctx < k * max_doc_chunks),
 * UNSUPPORTED (src_mode), HIP.
 */
int msa_gather_kv(int dtype, const int32_t* ids, int B, int k, const int64_t* chunk_off,
                  const int64_t* chunk_off_h, int64_t n_docs, int max_doc_chunks, const void* k_bar,
                  const void* v_bar, int64_t n_chunks, int Hkv, int d, int src_mode, int max_ctx,
                  void* k_ctx, void* v_ctx, int32_t* ctx_pos, int32_t* ctx_len, int32_t* ids_h,
                  void* stream, void* copy_stream);

/*
 * msa_context_index - Stage 2 context assembly for a store that stays in
 * device memory (README, Inference Pipeline: only the selected documents'
 * K/V take part; the concatenation with the local context is then an index,
 * not a copy).  Same context definition as msa_gather_kv, but instead of the
 * rows themselves it writes where they live:
 *   ctx_row[b,e] = c (row of the pooled K/V store), ctx_pos[b,e] = c - chunk_off[doc]
 *   ctx_len[b]   = sum of the selected documents' chunk counts
 * Entries e >= ctx_len[b] are left untouched.
 *   ids        [B, k] int32 device; ids outside [0, n_docs) contribute nothing
 *   chunk_off  [n_docs + 1] int64 device
 *   n_chunks   rows of the store (< 2^31, rows are int32)
 *   ctx_row, ctx_pos [B, max_ctx] int32, ctx_len [B] int32 device outputs
 * Errors: INVALID_ARG (NULL, sizes, max_ctx < k * max_doc_chunks),
 * UNSUPPORTED (n_chunks >= 2^31, B or k > 65535), HIP.
 */
int msa_context_index(const int32_t* ids, int B, int k, const int64_t* chunk_off, int64_t n_docs,
                      int max_doc_chunks, int64_t n_chunks, int max_ctx, int32_t* ctx_row, int32_t* ctx_pos,
                      int32_t* ctx_len, void* stream);

/*
 * msa_topk_context_index - msa_topk followed by msa_context_index on its ids
 * (Stage 2 selection and context assembly for a store in HBM), in one pass
 * for k <= 64: the final selection pass, which holds each query's k
 * documents, also writes their context entries.  Outputs are exactly those
 * of the two calls (ids, vals, ctx_row, ctx_pos, ctx_len).  For k > 64 the
 * two calls run one after the other.
 *   arguments as for msa_topk and msa_context_index; ws: msa_topk_workspace();
 *   flags as for msa_topk
 * Errors: those of msa_topk and of msa_context_index.
 */
int msa_topk_context_index(float* doc_score, int B, int64_t n_docs, int k, int32_t* ids, float* vals,
                           const int64_t* chunk_off, int max_doc_chunks, int64_t n_chunks, int max_ctx,
                           int32_t* ctx_row, int32_t* ctx_pos, int32_t* ctx_len, void* ws, size_t ws_bytes,
                           int flags, void* stream);

/*
 * msa_context_append - msa_context_index for one more round of Memory
 * Interleave: the documents ids[b, :] (rank order) are appended after the
 * ctx_len_in[b] entries already in the context, which are kept.
 *   ctx_row, ctx_pos [B, max_ctx] int32 device, updated from entry
 *             ctx_len_in[b] on (same definitions as msa_context_index)
 *   ctx_len_in [B] int32 device input; ctx_len_out [B] int32 device output
 *             (a different array) = ctx_len_in + the appended chunk counts,
 *             never beyond max_ctx (entries that do not fit are dropped)
 *   ids       [B, k] int32; -1 (an exhausted msa_topk) contributes nothing
 * Errors: INVALID_ARG (NULL, aliased lengths, sizes, max_ctx < k *
 * max_doc_chunks), UNSUPPORTED (n_chunks >= 2^31, B or k > 65535), HIP.
 */
int msa_context_append(const int32_t* ids, int B, int k, const int64_t* chunk_off, int64_t n_docs,
                       int max_doc_chunks, int64_t n_chunks, int max_ctx, int32_t* ctx_row, int32_t* ctx_pos,
                       const int32_t* ctx_len_in, int32_t* ctx_len_out, void* stream);

/*
 * msa_sparse_attn - Stage 3 sparse attention (README, Overall Design >
 * Architecture: the chosen documents' pooled K/V placed ahead of the query's
 * own recent K/V, attended over at each decoding step; its parallel
 * (document-wise) RoPE and global RoPE items; paper note, Document-wise RoPE).
 * For query b, token t < T and query head hq (KV head g = hq / (Hq/Hkv)):
 *   keys: context entries e < ctx_len[b] at position ctx_pos[b,e] (each
 *         document restarts at 0), all visible; local tokens i < L_loc at
 *         position q_pos_offset + i, visible iff i <= L_loc - T + t (the T
 *         query tokens are the last T local tokens; causal).
 *   query position: q_pos_offset + L_loc - T + t (the pages offset the query by k: pass k).
 *   RoPE: rotate-half, the pair (m, m + d/2) turns by pos * rope_base^(-2m/d)
 *         (angles reduced in float64), applied to q and every key on the fly.
 *         The (cos, sin) rows come from rope_table (msa_rope_table with the same
 *         rope_base and d, at least msa_rope_table_rows() rows) or, when
 *         rope_table is NULL, are computed into the workspace on every call.
 *   out[b,t,hq,:] = softmax_j(sm_scale * <R q, R k_j>) . v_j   (float32)
 *   q     [B, T, Hq, d] dtype; k_ctx/v_ctx/ctx_pos/ctx_len from msa_gather_kv
 *   k_loc/v_loc [B, L_loc, Hkv, d] dtype, un-rotated
 *   ctx_pos values must lie in [0, max_ctx)
 *   out   [B, T, Hq, d] float32
 *   ws    msa_sparse_attn_workspace() bytes
 * Errors: INVALID_ARG (NULL, sizes, Hq % Hkv != 0, L_loc < T, d odd,
 * q_pos_offset < 0), UNSUPPORTED (d > 256), WORKSPACE.
 */
size_t msa_sparse_attn_workspace(int dtype, int B, int T, int Hq, int Hkv, int d, int max_ctx, int L_loc,
                                 int q_pos_offset);
int msa_sparse_attn(int dtype, const void* q, int B, int T, int Hq, int Hkv, int d, const void* k_ctx,
                    const void* v_ctx, const int32_t* ctx_pos, const int32_t* ctx_len, int max_ctx,
                    const void* k_loc, const void* v_loc, int L_loc, int q_pos_offset, float rope_base,
                    const float* rope_table, int rope_table_rows, float sm_scale, float* out, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * msa_sparse_attn_indexed - msa_sparse_attn over a context given by
 * msa_context_index: context entry e of query b is row ctx_row[b,e] of the
 * pooled store k_bar/v_bar [n_chunks, Hkv, d] dtype, read in place.  The
 * store may be in device memory or in pinned host memory mapped for the
 * device (README, Overall Design > Inference Pipeline: the content K/V stays
 * in host memory and only the selected documents are loaded): the kernel
 * then reads the selected rows over the host link, and those reads overlap
 * the local-window keys' work of the same launch, so no copy of the context
 * is made.  Every other argument, the result and the workspace
 * (msa_sparse_attn_workspace) are those of msa_sparse_attn; the two give
 * bit-identical outputs for the same context.  Rows outside [0, n_chunks) are
 * clamped into the store (they are a caller error, never an out-of-bounds read).
 * Errors: those of msa_sparse_attn; INVALID_ARG also for ctx_row NULL or
 * n_chunks outside [1, 2^31).
 */
int msa_sparse_attn_indexed(int dtype, const void* q, int B, int T, int Hq, int Hkv, int d, const void* k_bar,
                            const void* v_bar, int64_t n_chunks, const int32_t* ctx_row, const int32_t* ctx_pos,
                            const int32_t* ctx_len, int max_ctx, const void* k_loc, const void* v_loc, int L_loc,
                            int q_pos_offset, float rope_base, const float* rope_table, int rope_table_rows,
                            float sm_scale, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * msa_sparse_attn_part - msa_sparse_attn (or, with ctx_row, _indexed) in two
 * calls, so that the local-window half of the attention can run while the
 * selected documents' K/V are still being fetched (README, Overall Design >
 * Inference Pipeline: the pooled content K/V live in host memory and are brought
 * over in the background once the top-k is known; the local tokens need no
 * fetch).
 *   part = MSA_ATTN_PART_LOCAL: the local keys only, as partial softmax sums
 *     into ws.  Reads q, k_loc, v_loc and the RoPE rows; the context arguments
 *     (k_ctx, v_ctx, ctx_row, ctx_pos, ctx_len) and out are not read and may be
 *     NULL, so the call may run before or while the context is assembled.
 *   part = MSA_ATTN_PART_CONTEXT: the context keys, then the merge of both
 *     parts' partials into out.  ws must hold the local call's partials: the
 *     same arguments, the same ws, and the local call complete (the caller
 *     orders the two, e.g. with an event between two streams).
 * The result is msa_sparse_attn's definition; the keys are split between
 * partials differently, so it agrees with msa_sparse_attn to float rounding
 * (the partials are float16), not bit for bit.
 *   ctx_row NULL: k_ctx/v_ctx are a gathered context [B, max_ctx, Hkv, d]
 *   (msa_gather_kv) and ctx_rows is ignored; otherwise they are the pooled
 *   store [ctx_rows, Hkv, d] read in place (msa_context_index).
 *   ws    msa_sparse_attn_part_workspace() bytes (not msa_sparse_attn_workspace)
 * Errors: those of msa_sparse_attn; INVALID_ARG also for a bad part or, with
 * ctx_row, ctx_rows outside [1, 2^31); UNSUPPORTED off the MFMA path (bf16,
 * d = 128, Hq/Hkv in {1, 2, 4, 8, 16}).
 */
size_t msa_sparse_attn_part_workspace(int dtype, int B, int T, int Hq, int Hkv, int d, int max_ctx, int L_loc,
                                      int q_pos_offset);
int msa_sparse_attn_part(int part, int dtype, const void* q, int B, int T, int Hq, int Hkv, int d, const void* k_ctx,
                         const void* v_ctx, int64_t ctx_rows, const int32_t* ctx_row, const int32_t* ctx_pos,
                         const int32_t* ctx_len, int max_ctx, const void* k_loc, const void* v_loc, int L_loc,
                         int q_pos_offset, float rope_base, const float* rope_table, int rope_table_rows,
                         float sm_scale, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * msa_sparse_attn_indexed_noalloc - msa_sparse_attn_indexed for callers that
 * cannot allocate memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, same kernels and the
 * same result, bit for bit, as msa_sparse_attn_indexed, without ws/ws_bytes:
 * the workspace is a device array inside the library, MSA_NOALLOC_SCRATCH_BYTES
 * long, that each GPU the library runs on holds until the process ends.  The
 * call allocates nothing.  The caller still owns the inputs and `out`.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or host threads) race and must be serialised by
 * the caller.
 * Errors: those of msa_sparse_attn_indexed; UNSUPPORTED when the shape's
 * workspace (msa_sparse_attn_workspace) exceeds MSA_NOALLOC_SCRATCH_BYTES;
 * HIP when the array's device address cannot be taken.
 */
#define MSA_NOALLOC_SCRATCH_BYTES (32u << 20)
int msa_sparse_attn_indexed_noalloc(int dtype, const void* q, int B, int T, int Hq, int Hkv, int d,
                                    const void* k_bar, const void* v_bar, int64_t n_chunks, const int32_t* ctx_row,
                                    const int32_t* ctx_pos, const int32_t* ctx_len, int max_ctx, const void* k_loc,
                                    const void* v_loc, int L_loc, int q_pos_offset, float rope_base,
                                    const float* rope_table, int rope_table_rows, float sm_scale, float* out,
                                    void* stream);

/*
 * msa_rope_table - the (cos, sin) rows msa_sparse_attn rotates with, built
 * once and reused by every layer and call with the same base and d.  Row p,
 * pair m holds (cos, sin)(p * rope_base^(-2m/d)) with the angle formed and
 * reduced in float64 and rounded to float32 (document-wise RoPE: positions
 * are document-local chunk indices and the query's offset positions).
 *   table [rows, d/2, 2] float32 device output
 * msa_rope_table_rows gives the rows msa_sparse_attn needs:
 * max(q_pos_offset + L_loc, max_ctx, 32).
 * Errors: INVALID_ARG (NULL, rows < 1, d odd, rope_base <= 1).
 */
int msa_rope_table_rows(int max_ctx, int L_loc, int q_pos_offset);
int msa_rope_table(int rows, int d, float rope_base, float* table, void* stream);

/*
 * msa_stream_read - measurement reference, not a step of the path: reads
 * `bytes` of device memory at `buf` once, with the access pattern of the
 * routing-key scan (each wave load instruction 1 KB contiguous, 16-byte
 * non-temporal loads), computing nothing but an XOR of the data.  Its rate
 * is the achievable streaming-read ceiling that the HBM-bound kernels are
 * compared with next to the nominal 8 TB/s.  `sink` (one uint32, device) is
 * written only if the XOR equals 0x9E3779B9.  bytes: a positive multiple of
 * 16; buf 16-byte aligned.
 */
int msa_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------
 * Training-time path (paper note 核心方法 > 训练: continued pre-training with
 * a generation loss and an auxiliary supervised contrastive routing loss;
 * README Abstract and Key Contributions: the layer is trained end to end;
 * README Implementation Notes: auxiliary routing loss).  The selection
 * (top-k ids, context order and positions) is held fixed; gradients are
 * float32; a store's bf16 rounding is taken as the identity.
 * ------------------------------------------------------------------------ */

/*
 * msa_route_argmax - msa_route_score together with the maximiser of each
 * score, for the routing backward.  doc_score[b,i] as in msa_route_score;
 * (arg_chunk[b,i], arg_tok[b,i]) = the global chunk index and query token
 * attaining it, the smallest chunk and then the smallest token among equal
 * values; -1 for a document with no chunk.
 *   q_r [B, T, H, d] dtype, kr_hat [n_chunks, H, d] dtype (MSA_LAYOUT_ROWS),
 *   chunk_doc [n_chunks] int32, doc_score [B, n_docs] float32,
 *   arg_chunk / arg_tok [B, n_docs] int32 outputs,
 *   ws msa_route_argmax_workspace() bytes.
 * bf16 with d % 32 == 0 runs on MFMA (exact products, float32 sums).
 * Errors: INVALID_ARG (NULL, sizes), WORKSPACE, UNSUPPORTED (d > 256,
 * B*T >= 2^24, n_chunks * T >= 2^32 - 1).
 */
size_t msa_route_argmax_workspace(int dtype, int B, int T, int H, int d, int64_t n_docs, int64_t n_chunks);
int msa_route_argmax(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat,
                     const int32_t* chunk_doc, int64_t n_docs, int64_t n_chunks, float* doc_score,
                     int32_t* arg_chunk, int32_t* arg_tok, void* ws, size_t ws_bytes, void* stream);

/*
 * msa_route_loss - the auxiliary routing loss (reading: the supervised
 * contrastive form over all documents).  For query b with positive set P_b
 * (the distinct ids of pos_ids[b,:] inside [0, n_docs); -1 pads):
 *   loss[b]    = -(1/|P_b|) sum_{p in P_b} log( exp(s_bp/tau) / sum_i exp(s_bi/tau) )
 *   grad[b,i]  = d loss[b] / d s_bi = (softmax_i(s_b/tau) - [i in P_b]/|P_b|) / tau
 * Documents scoring -inf (no chunk) or NaN carry no weight (grad 0).  A query
 * without a valid positive gets loss NaN.
 *   doc_score [B, n_docs] float32, pos_ids [B, n_pos] int32,
 *   loss [B] float32, grad [B, n_docs] float32 outputs
 * Errors: INVALID_ARG (NULL, sizes, tau <= 0), UNSUPPORTED (B > 65535,
 * n_pos > 256).
 */
int msa_route_loss(const float* doc_score, int B, int64_t n_docs, const int32_t* pos_ids, int n_pos, float tau,
                   float* loss, float* grad, void* stream);

/*
 * msa_route_score_backward - gradients of sum_{b,i} grad[b,i] * doc_score[b,i]:
 * the score's derivative reaches its maximiser (c*, t*) = (arg_chunk, arg_tok)
 * only, through s = (1/H) sum_h <q_r[b,t*,h]/||q_r[b,t*,h]||, kr_hat[c*,h]>.
 *   dq_r    [B, T, H, d] float32, overwritten: w.r.t. the raw routing query
 *           (through its normalisation; below norm 1e-8 the map is q / 1e-8)
 *   dkr_hat [n_chunks, H, d] float32, ACCUMULATED (+=): w.r.t. the normalised
 *           store entries (msa_pool_backward with x carries it to the tokens)
 *   arg_chunk / arg_tok from msa_route_argmax; entries out of range or with
 *   grad 0 contribute nothing.  Float atomics: the summation order varies.
 * Errors: INVALID_ARG (NULL, sizes), UNSUPPORTED (n_chunks >= 2^31,
 * B * n_docs * H > 2^32).
 */
int msa_route_score_backward(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat,
                             int64_t n_chunks, const int32_t* arg_chunk, const int32_t* arg_tok,
                             const float* grad, int64_t n_docs, float* dq_r, float* dkr_hat, void* stream);

/*
 * msa_pool_backward - adjoint of msa_pool_encode's chunk mean: token t of
 * pooled chunk c receives dy[c] / n_c (n_c the chunk's token count).  With x
 * (the token vectors given to msa_pool_encode with l2_normalize) dy is the
 * gradient at the normalised entry and is first carried back through the
 * normalisation of the chunk mean (recomputed in float32).
 *   dy [n_chunks, H, d] float32; x [n_tok, H, d] dtype or NULL;
 *   dx [n_tok, H, d] float32 output (every token of a chunk is written)
 *   tok_off, chunk_off, chunk_doc as for msa_pool_encode
 * Errors: INVALID_ARG (NULL, sizes), UNSUPPORTED (d > 256).
 */
int msa_pool_backward(int dtype, const float* dy, const int64_t* tok_off, const int64_t* chunk_off,
                      const int32_t* chunk_doc, int64_t n_docs, int64_t n_tok, int64_t n_chunks, int H, int d,
                      int chunk, const void* x, float* dx, void* stream);

/*
 * msa_sparse_attn_backward - gradients of msa_sparse_attn_indexed (same
 * arguments, same definition of the keys, positions and mask) given dout, the
 * gradient of its output:
 *   dq     [B, T, Hq, d] float32, overwritten
 *   dk_loc, dv_loc [B, L_loc, Hkv, d] float32, overwritten
 *   dk_bar, dv_bar [n_chunks, Hkv, d] float32, ACCUMULATED (+=): each context
 *          entry adds its gradient to the store row it reads (ctx_row), so a
 *          row read by several queries receives their sum (float atomics).
 * The forward is recomputed inside (its log-sum-exp per query row kept);
 * then with P the softmax, D = <dout, out>, dP = dout . v and
 * dS = P * (dP - D): dv = sum P dout, dk = R(-pos) sm_scale sum dS R q,
 * dq = R(-pos_q) sm_scale sum dS R k (R the RoPE rotation; its adjoint turns
 * by the opposite angle).  The bf16 d = 128 path runs on MFMA with bf16
 * operands (dout rounded to bf16) and float32 accumulation; other shapes use
 * a float32 vector path (at most 16384 - d - 256 keys and 8192 query rows
 * per KV head).
 *   ws  msa_sparse_attn_backward_workspace() bytes
 * Errors: those of msa_sparse_attn_indexed; INVALID_ARG for NULL gradients;
 * WORKSPACE; UNSUPPORTED beyond the vector path's sizes.
 */
size_t msa_sparse_attn_backward_workspace(int dtype, int B, int T, int Hq, int Hkv, int d, int max_ctx, int L_loc,
                                          int q_pos_offset);
int msa_sparse_attn_backward(int dtype, const void* q, int B, int T, int Hq, int Hkv, int d, const void* k_bar,
                             const void* v_bar, int64_t n_chunks, const int32_t* ctx_row, const int32_t* ctx_pos,
                             const int32_t* ctx_len, int max_ctx, const void* k_loc, const void* v_loc, int L_loc,
                             int q_pos_offset, float rope_base, const float* rope_table, int rope_table_rows,
                             float sm_scale, const float* dout, float* dq, float* dk_loc, float* dv_loc,
                             float* dk_bar, float* dv_bar, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
