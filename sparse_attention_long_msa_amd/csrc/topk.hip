// Stage 2 selection: the k best documents per query by (score desc, id asc).
// (MSA README, Overall Design > Architecture: "selects Top-k documents";
//  paper note 核心方法 > 架构: top-k documents by cosine similarity.)
//
// Every (score, id) pair becomes one 64-bit key whose ascending order is the
// ranking: the high word is the bit-complement of the order-preserving image
// of the float score, the low word the document id.  Keys are unique, so
// the selection is exact and deterministic.  Each pass sorts slices of 4096
// keys in LDS with a bitonic network and keeps the k smallest of each slice;
// passes repeat until one slice is left.
#include <algorithm>
#include <vector>

#include "common.h"

namespace msa {

constexpr int TK_THREADS = 256;
constexpr int TK_SLICE = 4096;
constexpr int TK_MAXK = 256;

__device__ __forceinline__ uint64_t score_key(float s, uint32_t id) {
  return (uint64_t(~float_order_key(s)) << 32) | uint64_t(id);
}

// in:  scores [B][n] (FROM_SCORES) or keys [B][n]
// out: keys [B][n_slices][k] (sorted ascending inside a slice), or, when
//      FINAL, ids/vals [B][k]
template <bool FROM_SCORES, bool FINAL>
__global__ __launch_bounds__(TK_THREADS) void topk_pass_kernel(const float* __restrict__ scores,
                                                               const uint64_t* __restrict__ keys_in, int64_t n,
                                                               int k, uint64_t* __restrict__ keys_out,
                                                               int32_t* __restrict__ ids, float* __restrict__ vals) {
  __shared__ uint64_t sk[TK_SLICE];
  const int b = blockIdx.y;
  const int64_t slice = blockIdx.x;
  const int64_t base = slice * TK_SLICE;
  for (int i = threadIdx.x; i < TK_SLICE; i += TK_THREADS) {
    const int64_t g = base + i;
    uint64_t key = ~uint64_t(0);
    if (g < n) {
      if constexpr (FROM_SCORES)
        key = score_key(scores[int64_t(b) * n + g], uint32_t(g));
      else
        key = keys_in[int64_t(b) * n + g];
    }
    sk[i] = key;
  }
  __syncthreads();
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

// Candidate counts of successive passes: n0 = n_docs, n_{i+1} = slices(n_i) * k.
static std::vector<int64_t> topk_plan(int64_t n_docs, int k) {
  std::vector<int64_t> ns{n_docs};
  while ((ns.back() + TK_SLICE - 1) / TK_SLICE > 1) ns.push_back((ns.back() + TK_SLICE - 1) / TK_SLICE * k);
  return ns;
}

}  // namespace msa

extern "C" size_t msa_topk_workspace(int B, int64_t n_docs, int k) {
  if (B < 1 || n_docs < 1 || k < 1 || k > msa::TK_MAXK) return 0;
  const auto ns = msa::topk_plan(n_docs, k);
  int64_t mx = 0;
  for (size_t i = 1; i < ns.size(); ++i) mx = std::max(mx, ns[i]);
  return 2 * msa::align_up(size_t(B) * size_t(mx) * sizeof(uint64_t), 256);
}

extern "C" int msa_topk(const float* doc_score, int B, int64_t n_docs, int k, int32_t* ids, float* vals, void* ws,
                        size_t ws_bytes, void* stream) {
  using namespace msa;
  MSA_REQUIRE(doc_score && ids && vals, MSA_ERR_INVALID_ARG, "msa_topk: NULL pointer");
  MSA_REQUIRE(B >= 1 && n_docs >= 1, MSA_ERR_INVALID_ARG, "msa_topk: non-positive size");
  MSA_REQUIRE(k >= 1 && k <= n_docs, MSA_ERR_INVALID_ARG, "msa_topk: k must be in [1, n_docs]");
  MSA_REQUIRE(k <= TK_MAXK, MSA_ERR_UNSUPPORTED, "msa_topk: k > 256");
  MSA_REQUIRE(n_docs < (int64_t(1) << 31) && B <= 65535, MSA_ERR_UNSUPPORTED, "msa_topk: too many documents or queries");
  const size_t need = msa_topk_workspace(B, n_docs, k);
  MSA_REQUIRE(ws_bytes >= need, MSA_ERR_WORKSPACE, "msa_topk: workspace too small");
  MSA_REQUIRE(need == 0 || ws, MSA_ERR_INVALID_ARG, "msa_topk: NULL workspace");
  hipStream_t s = as_stream(stream);
  const auto ns = topk_plan(n_docs, k);
  uint64_t* buf[2] = {static_cast<uint64_t*>(ws),
                      reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + need / 2)};
  const dim3 block(TK_THREADS);
  for (size_t p = 0; p < ns.size(); ++p) {
    const int64_t n = ns[p];
    const int64_t slices = (n + TK_SLICE - 1) / TK_SLICE;
    const dim3 grid{unsigned(slices), unsigned(B)};
    const bool first = p == 0, last = p + 1 == ns.size();
    const uint64_t* kin = first ? nullptr : buf[(p - 1) % 2];
    uint64_t* kout = last ? nullptr : buf[p % 2];
    if (first && last)
      hipLaunchKernelGGL((topk_pass_kernel<true, true>), grid, block, 0, s, doc_score, kin, n, k, kout, ids, vals);
    else if (first)
      hipLaunchKernelGGL((topk_pass_kernel<true, false>), grid, block, 0, s, doc_score, kin, n, k, kout, ids, vals);
    else if (last)
      hipLaunchKernelGGL((topk_pass_kernel<false, true>), grid, block, 0, s, doc_score, kin, n, k, kout, ids, vals);
    else
      hipLaunchKernelGGL((topk_pass_kernel<false, false>), grid, block, 0, s, doc_score, kin, n, k, kout, ids, vals);
    MSA_LAUNCH_CHECK();
  }
  return MSA_OK;
}
