// Stage 2 selection: the k best documents per query by (score desc, id asc).
// (MSA README, Overall Design > Architecture: the router keeps the k best documents;
//  paper note 核心方法 > 架构: top-k documents by cosine similarity.)
//
// A NaN score marks a document excluded from the selection (msa_exclude_docs):
// it gets the absent key, and when fewer than k documents remain the trailing
// ids are -1.  Every (score, id) pair becomes one 64-bit key whose ascending
// order is the ranking: the high word is the bit-complement of the order-preserving image
// of the float score, the low word the document id.  Keys are unique, so
// the selection is exact and deterministic.  Each pass sorts slices of 4096
// keys in LDS with a bitonic network and keeps the k smallest of each slice;
// passes repeat until one slice is left.
#include <algorithm>
#include <vector>

#include "common.h"
#include "wave_select.h"

namespace msa {

constexpr int TK_THREADS = 256;
constexpr int TK_SLICE = 4096;
constexpr int TK_MAXK = 256;


// in:  scores [B][n] (FROM_SCORES) or keys [B][n]
// out: keys [B][n_slices][k] (sorted ascending inside a slice), or, when
//      FINAL, ids/vals [B][k]
//
// reset (FROM_SCORES passes only): once its scores are read, each workgroup
// writes -inf over them, leaving the buffer ready for a routing call that
// max-accumulates (msa_route_score with MSA_ROUTE_PREFILLED).
template <bool FROM_SCORES, bool FINAL>
__global__ __launch_bounds__(TK_THREADS) void topk_pass_kernel(float* __restrict__ scores,
                                                               const uint64_t* __restrict__ keys_in, int64_t n,
                                                               int k, uint64_t* __restrict__ keys_out,
                                                               int32_t* __restrict__ ids, float* __restrict__ vals,
                                                               int reset) {
  __shared__ uint64_t sk[TK_SLICE];
  const int b = blockIdx.y;
  const int64_t slice = blockIdx.x;
  const int64_t base = slice * TK_SLICE;
  for (int i = threadIdx.x; i < TK_SLICE; i += TK_THREADS) {
    const int64_t g = base + i;
    uint64_t key = ~uint64_t(0);
    if (g < n) {
      if constexpr (FROM_SCORES) {
        const float sc = scores[int64_t(b) * n + g];
        if (sc == sc) key = score_key(sc, uint32_t(g));   // NaN: an excluded document
      } else {
        key = keys_in[int64_t(b) * n + g];
      }
    }
    sk[i] = key;
  }
  __syncthreads();
  if (FROM_SCORES && reset) {   // the slice is read (its keys are in LDS)
    for (int i = threadIdx.x; i < TK_SLICE; i += TK_THREADS)
      if (base + i < n) scores[int64_t(b) * n + base + i] = -INFINITY;
  }
  for (int size = 2; size <= TK_SLICE; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < TK_SLICE / 2; i += TK_THREADS) {
        // i-th compare-exchange of this stage: pair (lo, lo + stride)
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = sk[lo], c = sk[hi];
        if ((a > c) == up) {
          sk[lo] = c;
          sk[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < k; i += TK_THREADS) {
    const uint64_t key = sk[i];
    if constexpr (FINAL) {
      ids[int64_t(b) * k + i] = int32_t(uint32_t(key));
      vals[int64_t(b) * k + i] = order_key_float(~uint32_t(key >> 32));
    } else {
      keys_out[(int64_t(b) * gridDim.x + slice) * k + i] = key;
    }
  }
}

// Reducing passes: 4 waves of 8 keys per lane (many workgroups in flight).
// Final pass (one workgroup per query): the same shape when the candidates
// fit it, else 16 waves of 16 keys per lane (up to 16,384 candidates).
constexpr int TW_WAVES = 4;
constexpr int TW_PL_FIRST = 8;
constexpr int TW_WAVES_WIDE = 16;
constexpr int TW_PL_WIDE = 16;
constexpr int tw_per_wg(int waves, int pl) { return waves * 64 * pl; }
// survivor slots per wave: at most k lanes hold keys <= the bound, and the
// merge stage needs 64
constexpr int tw_slots(int k, int pl) { return k * pl > 64 ? k * pl : 64; }

// Optional context index of the final pass (msa_topk_context_index): the
// selected documents' chunks, in rank order, as (store row, position in the
// document) entries, as msa_context_index writes them.
struct CtxOut {
  const int64_t* chunk_off;   // NULL: no context index
  int64_t n_docs;
  int max_ctx;
  int32_t* row;
  int32_t* pos;
  int32_t* len;
};

__device__ __forceinline__ int64_t shfl_up_i64(int64_t v, int s) {
  const int lo = __shfl_up(int(uint32_t(uint64_t(v))), s), hi = __shfl_up(int(uint32_t(uint64_t(v) >> 32)), s);
  return int64_t((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo));
}

// One wave, lane r < k holding the rank-r key: rank r's chunks start at the
// exclusive prefix of the chunk counts; the entries are then written lane-
// parallel, each finding its rank by a binary search over the starts.
__device__ void context_index_wave(uint64_t key, int lane, int k, int b, const CtxOut& cx, int64_t* sdest,
                                   int64_t* slo) {
  const int32_t id = lane < k ? int32_t(uint32_t(key)) : -1;
  int64_t lo = 0, n = 0;
  if (id >= 0 && id < cx.n_docs) {
    lo = cx.chunk_off[id];
    n = cx.chunk_off[id + 1] - lo;
  }
  int64_t incl = n;
#pragma unroll
  for (int sft = 1; sft < 64; sft <<= 1) {
    const int64_t o = shfl_up_i64(incl, sft);
    if (lane >= sft) incl += o;
  }
  const int64_t dest = incl - n;
  int64_t nc = n;
  if (dest + nc > cx.max_ctx) nc = dest < cx.max_ctx ? cx.max_ctx - dest : 0;   // never past the context
  if (lane == k - 1) cx.len[b] = int32_t(dest + nc);
  sdest[lane] = dest;
  slo[lane] = lo;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int64_t end = __shfl(int(dest + nc), k - 1);
  const int64_t total = end < cx.max_ctx ? end : cx.max_ctx;
  for (int64_t e = lane; e < total; e += 64) {
    int r0 = 0, r1 = k - 1;   // the last rank whose start is <= e (empty ranks share the next start)
    while (r0 < r1) {
      const int mid = (r0 + r1 + 1) / 2;
      if (sdest[mid] <= e) r0 = mid; else r1 = mid - 1;
    }
    const int64_t i = e - sdest[r0];
    cx.pos[int64_t(b) * cx.max_ctx + e] = int32_t(i);
    cx.row[int64_t(b) * cx.max_ctx + e] = int32_t(slo[r0] + i);
  }
}

// Each wave selects the k best of up to 64 * TW_PER_LANE inputs.
// Filter first: the k-th smallest of the 64 lane minima bounds the k-th
// smallest key from above (those k lane minima are k distinct keys), so
// only keys <= that bound can be selected.  The survivors (at most
// k * TW_PER_LANE, usually about k) are compacted into LDS and sorted /
// merged 64 at a time.
// The waves' sorted lists are then merged through LDS into the workgroup's k best:
// not FINAL, they go to keys_out[b][workgroup][k]; FINAL (one workgroup per
// query), they are written as ids/vals.
template <bool FROM_SCORES, bool FINAL, int TW_PER_LANE, int W>
__global__ __launch_bounds__(64 * W) void topk_wave_kernel(float* __restrict__ scores,
                                                           const uint64_t* __restrict__ keys_in, int64_t n, int k,
                                                           uint64_t* __restrict__ keys_out, int32_t* __restrict__ ids,
                                                           float* __restrict__ vals, CtxOut cx, int reset) {
  constexpr int TW_PER_WAVE = 64 * TW_PER_LANE;
  extern __shared__ uint64_t surv_lds[];   // [W][tw_slots(k, TW_PER_LANE)]
  const int slots = tw_slots(k, TW_PER_LANE);
  const int b = blockIdx.y;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t wave_id = int64_t(blockIdx.x) * W + wave;
  const int64_t base = wave_id * TW_PER_WAVE;
  constexpr uint64_t SENT = ~uint64_t(0);
  uint64_t v[TW_PER_LANE];
  uint64_t lmin = SENT;
#pragma unroll
  for (int i = 0; i < TW_PER_LANE; ++i) {
    const int64_t g = base + int64_t(i) * 64 + lane;
    uint64_t key = SENT;
    if (g < n) {
      if constexpr (FROM_SCORES) {
        const float sc = scores[int64_t(b) * n + g];
        if (sc == sc) key = score_key(sc, uint32_t(g));   // NaN: an excluded document
      } else {
        key = keys_in[int64_t(b) * n + g];
      }
    }
    v[i] = key;
    lmin = key < lmin ? key : lmin;
  }
  const uint64_t bound = readlane64(wave_sort64(lmin, lane), k - 1);
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < TW_PER_LANE; ++i) cnt += (v[i] <= bound && v[i] != SENT) ? 1 : 0;
  // exclusive prefix of the survivor counts across the wave
  int incl = cnt;
#pragma unroll
  for (int sft = 1; sft < 64; sft <<= 1) {
    const int o = __shfl_up(incl, sft);
    if (lane >= sft) incl += o;
  }
  const int total = __builtin_amdgcn_readlane(incl, 63);
  int pos = incl - cnt;
  uint64_t* sw = surv_lds + wave * slots;
#pragma unroll
  for (int i = 0; i < TW_PER_LANE; ++i)
    if (v[i] <= bound && v[i] != SENT) sw[pos++] = v[i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  uint64_t best = wave_sort64(lane < total ? sw[lane] : SENT, lane);
  for (int s0 = 64; s0 < total; s0 += 64) best = wave_insert(best, s0 + lane < total ? sw[s0 + lane] : SENT, lane, k);
  // pairwise tree merge of the waves' sorted lists: wave w < half takes in
  // the list of wave w + half, log2(W) rounds
  static_assert((W & (W - 1)) == 0, "a power-of-two number of waves");
  __syncthreads();
  if (FROM_SCORES && reset) {   // every score of this wave is read (its keys are sorted)
#pragma unroll
    for (int i = 0; i < TW_PER_LANE; ++i) {
      const int64_t g = base + int64_t(i) * 64 + lane;
      if (g < n) scores[int64_t(b) * n + g] = -INFINITY;
    }
  }
  sw[lane] = best;
  __syncthreads();
#pragma unroll
  for (int half = W / 2; half >= 1; half /= 2) {
    if (wave < half) {
      best = wave_merge_sorted(best, surv_lds[(wave + half) * slots + lane], lane, k);
      sw[lane] = best;
    }
    __syncthreads();
  }
  if (wave == 0) {
    const uint64_t acc = best;
    if (lane < k) {
      if constexpr (FINAL) {
        ids[int64_t(b) * k + lane] = int32_t(uint32_t(acc));
        vals[int64_t(b) * k + lane] = order_key_float(~uint32_t(acc >> 32));
      } else {
        keys_out[(int64_t(b) * gridDim.x + blockIdx.x) * k + lane] = acc;
      }
    }
    if constexpr (FINAL) {
      __shared__ int64_t sdest[64], slo[64];
      if (cx.chunk_off) context_index_wave(acc, lane, k, b, cx, sdest, slo);
    }
  }
}

// Memory Parallel's global reduce (README, Overall Design > Inference
// Pipeline: sharded routing keys, local scoring, then a global reduce): the
// per-shard top-k lists of G shards merged into the k best by (score desc,
// global id asc).  One wave per query walks the G * k_in candidates 64 at a
// time, keeping its 64 smallest keys sorted across the lanes (the first batch
// is sorted, later batches are merged in when one of them beats the k-th key).
// A slot with id < 0 or a NaN score is empty.
__global__ __launch_bounds__(64) void topk_merge_kernel(const float* __restrict__ vals,
                                                        const int32_t* __restrict__ ids,
                                                        const int64_t* __restrict__ id_offset, int G, int B,
                                                        int k_in, int k, int32_t* __restrict__ ids_out,
                                                        float* __restrict__ vals_out) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int64_t n = int64_t(G) * k_in;
  constexpr uint64_t SENT = ~uint64_t(0);
  uint64_t best = SENT;
  for (int64_t i0 = 0; i0 < n; i0 += 64) {   // uniform in the wave
    const int64_t i = i0 + lane;
    uint64_t key = SENT;
    if (i < n) {
      const int g = int(i / k_in), j = int(i % k_in);
      const int64_t e = (int64_t(g) * B + b) * k_in + j;
      const int32_t id = ids[e];
      const float v = vals[e];
      if (id >= 0 && v == v) key = score_key(v, uint32_t(int64_t(id) + id_offset[g]));
    }
    best = i0 == 0 ? wave_sort64(key, lane) : wave_insert(best, key, lane, k);
  }
  if (lane < k) {
    ids_out[int64_t(b) * k + lane] = int32_t(uint32_t(best));
    vals_out[int64_t(b) * k + lane] = order_key_float(~uint32_t(best >> 32));
  }
}

// Candidate counts of the wave passes: inputs > one workgroup's capacity are
// reduced by non-final passes (every workgroup keeps k of its 2048 inputs;
// idle waves of the last workgroup contribute sentinel keys).
static std::vector<int64_t> topk_wave_plan(int64_t n_docs, int k) {
  constexpr int64_t first = tw_per_wg(TW_WAVES, TW_PL_FIRST), wide = tw_per_wg(TW_WAVES_WIDE, TW_PL_WIDE);
  std::vector<int64_t> ns{n_docs};
  while (ns.back() > wide) ns.push_back((ns.back() + first - 1) / first * k);
  return ns;
}

// Candidate counts of successive passes: n0 = n_docs, n_{i+1} = slices(n_i) * k.
static std::vector<int64_t> topk_plan(int64_t n_docs, int k) {
  std::vector<int64_t> ns{n_docs};
  while ((ns.back() + TK_SLICE - 1) / TK_SLICE > 1) ns.push_back((ns.back() + TK_SLICE - 1) / TK_SLICE * k);
  return ns;
}

}  // namespace msa

extern "C" size_t msa_topk_workspace(int B, int64_t n_docs, int k) {
  if (B < 1 || n_docs < 1 || k < 1 || k > msa::TK_MAXK) return 0;
  const auto ns = k <= 64 ? msa::topk_wave_plan(n_docs, k) : msa::topk_plan(n_docs, k);
  int64_t mx = 0;
  for (size_t i = 1; i < ns.size(); ++i) mx = std::max(mx, ns[i]);
  return 2 * msa::align_up(size_t(B) * size_t(mx) * sizeof(uint64_t), 256);
}

namespace msa {
static int topk_run(float* doc_score, int B, int64_t n_docs, int k, int32_t* ids, float* vals, void* ws,
                    size_t ws_bytes, void* stream, const CtxOut& cx, int flags);
}

extern "C" int msa_topk(float* doc_score, int B, int64_t n_docs, int k, int32_t* ids, float* vals, void* ws,
                        size_t ws_bytes, int flags, void* stream) {
  return msa::topk_run(doc_score, B, n_docs, k, ids, vals, ws, ws_bytes, stream,
                       msa::CtxOut{nullptr, 0, 0, nullptr, nullptr, nullptr}, flags);
}

extern "C" int msa_topk_context_index(float* doc_score, int B, int64_t n_docs, int k, int32_t* ids,
                                      float* vals, const int64_t* chunk_off, int max_doc_chunks, int64_t n_chunks,
                                      int max_ctx, int32_t* ctx_row, int32_t* ctx_pos, int32_t* ctx_len, void* ws,
                                      size_t ws_bytes, int flags, void* stream) {
  using namespace msa;
  MSA_REQUIRE(chunk_off && ctx_row && ctx_pos && ctx_len, MSA_ERR_INVALID_ARG,
              "msa_topk_context_index: NULL pointer");
  MSA_REQUIRE(n_chunks >= 1 && max_doc_chunks >= 1, MSA_ERR_INVALID_ARG, "msa_topk_context_index: non-positive size");
  MSA_REQUIRE(n_chunks <= INT32_MAX, MSA_ERR_UNSUPPORTED, "msa_topk_context_index: n_chunks must be below 2^31");
  MSA_REQUIRE(int64_t(max_ctx) >= int64_t(k) * max_doc_chunks, MSA_ERR_INVALID_ARG,
              "msa_topk_context_index: max_ctx < k * max_doc_chunks");
  if (k > 64) {   // the slice passes: the selection, then the index on its own
    const int rc = topk_run(doc_score, B, n_docs, k, ids, vals, ws, ws_bytes, stream,
                            CtxOut{nullptr, 0, 0, nullptr, nullptr, nullptr}, flags);
    if (rc != MSA_OK) return rc;
    return msa_context_index(ids, B, k, chunk_off, n_docs, max_doc_chunks, n_chunks, max_ctx, ctx_row, ctx_pos,
                             ctx_len, stream);
  }
  return topk_run(doc_score, B, n_docs, k, ids, vals, ws, ws_bytes, stream,
                  CtxOut{chunk_off, n_docs, max_ctx, ctx_row, ctx_pos, ctx_len}, flags);
}

namespace msa {
static int topk_run(float* doc_score, int B, int64_t n_docs, int k, int32_t* ids, float* vals, void* ws,
                    size_t ws_bytes, void* stream, const CtxOut& cx, int flags) {
  MSA_REQUIRE(doc_score && ids && vals, MSA_ERR_INVALID_ARG, "msa_topk: NULL pointer");
  MSA_REQUIRE((flags & ~MSA_TOPK_RESET_SCORES) == 0, MSA_ERR_INVALID_ARG, "msa_topk: unknown flags");
  const int reset = (flags & MSA_TOPK_RESET_SCORES) ? 1 : 0;
  MSA_REQUIRE(B >= 1 && n_docs >= 1, MSA_ERR_INVALID_ARG, "msa_topk: non-positive size");
  MSA_REQUIRE(k >= 1 && k <= n_docs, MSA_ERR_INVALID_ARG, "msa_topk: k must be in [1, n_docs]");
  MSA_REQUIRE(k <= TK_MAXK, MSA_ERR_UNSUPPORTED, "msa_topk: k > 256");
  MSA_REQUIRE(n_docs < (int64_t(1) << 31) && B <= 65535, MSA_ERR_UNSUPPORTED, "msa_topk: too many documents or queries");
  const size_t need = msa_topk_workspace(B, n_docs, k);
  MSA_REQUIRE(ws_bytes >= need, MSA_ERR_WORKSPACE, "msa_topk: workspace too small");
  MSA_REQUIRE(need == 0 || ws, MSA_ERR_INVALID_ARG, "msa_topk: NULL workspace");
  hipStream_t s = as_stream(stream);
  uint64_t* buf[2] = {static_cast<uint64_t*>(ws),
                      reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + need / 2)};
  if (k <= 64) {
    const auto ns = topk_wave_plan(n_docs, k);
    for (size_t p = 0; p < ns.size(); ++p) {
      const int64_t n = ns[p];
      const bool first = p == 0, last = p + 1 == ns.size();
      const bool wide = last && n > tw_per_wg(TW_WAVES, TW_PL_FIRST);
      const int waves = wide ? TW_WAVES_WIDE : TW_WAVES;
      const size_t lds = size_t(waves) * tw_slots(k, wide ? TW_PL_WIDE : TW_PL_FIRST) * sizeof(uint64_t);
      const dim3 block(64 * waves);
      const dim3 grid{unsigned(last ? 1 : (n + tw_per_wg(TW_WAVES, TW_PL_FIRST) - 1) / tw_per_wg(TW_WAVES, TW_PL_FIRST)),
                      unsigned(B)};
      const uint64_t* kin = first ? nullptr : buf[(p - 1) % 2];
      uint64_t* kout = last ? nullptr : buf[p % 2];
#define TW_LAUNCH(FS, FIN, PL, W)                                                                                   \
  MSA_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_wave_kernel<FS, FIN, PL, W>),               \
                                    hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)));                         \
  hipLaunchKernelGGL((topk_wave_kernel<FS, FIN, PL, W>), grid, block, lds, s, doc_score, kin, n, k, kout, ids, vals, \
                     last ? cx : CtxOut{nullptr, 0, 0, nullptr, nullptr, nullptr}, first ? reset : 0)
      if (first && last && wide) {
        TW_LAUNCH(true, true, TW_PL_WIDE, TW_WAVES_WIDE);
      } else if (first && last) {
        TW_LAUNCH(true, true, TW_PL_FIRST, TW_WAVES);
      } else if (first) {
        TW_LAUNCH(true, false, TW_PL_FIRST, TW_WAVES);
      } else if (last && wide) {
        TW_LAUNCH(false, true, TW_PL_WIDE, TW_WAVES_WIDE);
      } else if (last) {
        TW_LAUNCH(false, true, TW_PL_FIRST, TW_WAVES);
      } else {
        TW_LAUNCH(false, false, TW_PL_FIRST, TW_WAVES);
      }
#undef TW_LAUNCH
      MSA_LAUNCH_CHECK();
    }
    return MSA_OK;
  }
  const auto ns = topk_plan(n_docs, k);
  const dim3 block(TK_THREADS);
  for (size_t p = 0; p < ns.size(); ++p) {
    const int64_t n = ns[p];
    const int64_t slices = (n + TK_SLICE - 1) / TK_SLICE;
    const dim3 grid{unsigned(slices), unsigned(B)};
    const bool first = p == 0, last = p + 1 == ns.size();
    const uint64_t* kin = first ? nullptr : buf[(p - 1) % 2];
    uint64_t* kout = last ? nullptr : buf[p % 2];
    if (first && last)
      hipLaunchKernelGGL((topk_pass_kernel<true, true>), grid, block, 0, s, doc_score, kin, n, k, kout, ids, vals,
                         first ? reset : 0);
    else if (first)
      hipLaunchKernelGGL((topk_pass_kernel<true, false>), grid, block, 0, s, doc_score, kin, n, k, kout, ids, vals,
                         first ? reset : 0);
    else if (last)
      hipLaunchKernelGGL((topk_pass_kernel<false, true>), grid, block, 0, s, doc_score, kin, n, k, kout, ids, vals,
                         first ? reset : 0);
    else
      hipLaunchKernelGGL((topk_pass_kernel<false, false>), grid, block, 0, s, doc_score, kin, n, k, kout, ids, vals,
                         first ? reset : 0);
    MSA_LAUNCH_CHECK();
  }
  return MSA_OK;
}

}  // namespace msa

namespace msa {

// doc_score[b, ids[s][b][j]] = NaN for every set s and j < k (ids [n_sets][B][k])
__global__ void exclude_kernel(float* __restrict__ doc_score, int B, int64_t n_docs, const int32_t* __restrict__ ids,
                               int k, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t doc = ids[i];
  const int64_t b = (i / k) % B;
  if (doc >= 0 && doc < n_docs) doc_score[b * n_docs + doc] = __uint_as_float(0x7FC00000u);
}

}  // namespace msa

extern "C" int msa_exclude_docs(float* doc_score, int B, int64_t n_docs, const int32_t* ids, int n_sets, int k,
                                void* stream) {
  using namespace msa;
  MSA_REQUIRE(doc_score && (ids || n_sets == 0), MSA_ERR_INVALID_ARG, "msa_exclude_docs: NULL pointer");
  MSA_REQUIRE(B >= 1 && n_docs >= 1 && n_sets >= 0 && k >= 1, MSA_ERR_INVALID_ARG, "msa_exclude_docs: bad size");
  const int64_t n = int64_t(n_sets) * B * k;
  if (n == 0) return MSA_OK;
  hipLaunchKernelGGL(exclude_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, as_stream(stream), doc_score, B,
                     n_docs, ids, k, n);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

extern "C" int msa_topk_merge(const float* vals, const int32_t* ids, const int64_t* id_offset, int G, int B, int k_in,
                              int k, int32_t* ids_out, float* vals_out, void* stream) {
  using namespace msa;
  MSA_REQUIRE(vals && ids && id_offset && ids_out && vals_out, MSA_ERR_INVALID_ARG, "msa_topk_merge: NULL pointer");
  MSA_REQUIRE(G >= 1 && B >= 1 && k_in >= 1 && k >= 1, MSA_ERR_INVALID_ARG, "msa_topk_merge: non-positive size");
  MSA_REQUIRE(int64_t(G) * k_in >= k, MSA_ERR_INVALID_ARG, "msa_topk_merge: k > G * k_in");
  MSA_REQUIRE(k <= 64, MSA_ERR_UNSUPPORTED, "msa_topk_merge: k > 64");
  MSA_REQUIRE(int64_t(G) * k_in <= (int64_t(1) << 24), MSA_ERR_UNSUPPORTED, "msa_topk_merge: G * k_in > 2^24");
  hipLaunchKernelGGL(topk_merge_kernel, dim3(unsigned(B)), dim3(64), 0, as_stream(stream), vals, ids, id_offset, G, B,
                     k_in, k, ids_out, vals_out);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}
