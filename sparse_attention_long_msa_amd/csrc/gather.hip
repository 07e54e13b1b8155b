// Stage 2 context assembly: copy the selected documents' pooled K / V into a
// contiguous per-query context, in rank order, with each entry's position
// inside its document (document-wise RoPE restarts at 0 per document).
// (MSA README, Inference Pipeline: only the selected documents' K/V are
//  loaded and joined to the local context; content K/V may live in host DRAM and be
//  fetched when selected: README Inference Pipeline, paper note Memory
//  Parallel 推理.)
//
// One workgroup per (query, rank).  The source may be device memory or
// mapped pinned host memory (the kernel then reads over the host link);
// MSA_SRC_HOST_MEMCPY instead issues hipMemcpyAsync per document on a side
// stream after one host synchronisation on the ids.  msa_context_index writes
// only each entry's store row, for attention that reads a device-resident
// store in place.
#include <vector>

#include "common.h"

namespace msa {

constexpr int GK_THREADS = 256;

// dest offset of rank r = sum of the chunk counts of ranks < r
__device__ int64_t rank_offset(const int32_t* __restrict__ ids_b, int r, const int64_t* __restrict__ chunk_off,
                               int64_t n_docs, int64_t* red) {
  int64_t mine = 0;
  for (int q = threadIdx.x; q < r; q += GK_THREADS) {
    const int32_t doc = ids_b[q];
    if (doc >= 0 && doc < n_docs) mine += chunk_off[doc + 1] - chunk_off[doc];
  }
  red[threadIdx.x] = mine;
  __syncthreads();
  for (int st = GK_THREADS / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  const int64_t v = red[0];
  __syncthreads();
  return v;
}

// MODE: GK_POS writes positions and lengths only, GK_COPY also copies the
// rows, GK_ROWS writes each entry's store row instead of copying it.
enum { GK_POS = 0, GK_COPY = 1, GK_ROWS = 2 };

template <int MODE>
__global__ __launch_bounds__(GK_THREADS) void gather_kernel(const int32_t* __restrict__ ids, int k,
                                                            const int64_t* __restrict__ chunk_off, int64_t n_docs,
                                                            const uint4* __restrict__ k_bar,
                                                            const uint4* __restrict__ v_bar, int64_t row_vec,
                                                            int max_ctx, uint4* __restrict__ k_ctx,
                                                            uint4* __restrict__ v_ctx, int32_t* __restrict__ ctx_pos,
                                                            int32_t* __restrict__ ctx_len,
                                                            int32_t* __restrict__ ctx_row,
                                                            const int32_t* __restrict__ ctx_len_in) {
  __shared__ int64_t red[GK_THREADS];
  const int r = blockIdx.x, b = blockIdx.y;
  const int32_t* ids_b = ids + int64_t(b) * k;
  // entries already in the context (appending): they are kept
  int64_t base = ctx_len_in ? int64_t(ctx_len_in[b]) : 0;
  base = base < 0 ? 0 : (base > max_ctx ? max_ctx : base);
  const int64_t dest = base + rank_offset(ids_b, r, chunk_off, n_docs, red);
  const int32_t doc = ids_b[r];
  int64_t lo = 0, n = 0;
  if (doc >= 0 && doc < n_docs) {
    lo = chunk_off[doc];
    n = chunk_off[doc + 1] - lo;
  }
  if (dest + n > max_ctx) n = dest < max_ctx ? max_ctx - dest : 0;  // never write past the context
  if (r == k - 1 && threadIdx.x == 0) ctx_len[b] = int32_t(dest + n);
  for (int64_t i = threadIdx.x; i < n; i += GK_THREADS) {
    ctx_pos[int64_t(b) * max_ctx + dest + i] = int32_t(i);
    if constexpr (MODE == GK_ROWS) ctx_row[int64_t(b) * max_ctx + dest + i] = int32_t(lo + i);
  }
  if constexpr (MODE == GK_COPY) {
    const int64_t total = n * row_vec;
    const uint4* ks = k_bar + lo * row_vec;
    const uint4* vs = v_bar + lo * row_vec;
    uint4* kd = k_ctx + (int64_t(b) * max_ctx + dest) * row_vec;
    uint4* vd = v_ctx + (int64_t(b) * max_ctx + dest) * row_vec;
    // four independent 16-byte loads of K and of V in flight per thread
    constexpr int U = 4;
    int64_t i = threadIdx.x;
    for (; i + (U - 1) * GK_THREADS < total; i += U * GK_THREADS) {
      uint4 a[U], c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a[u] = ks[i + u * GK_THREADS];
        c[u] = vs[i + u * GK_THREADS];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kd[i + u * GK_THREADS] = a[u];
        vd[i + u * GK_THREADS] = c[u];
      }
    }
    for (; i < total; i += GK_THREADS) {
      kd[i] = ks[i];
      vd[i] = vs[i];
    }
  }
}

// the device-side copy (any GPU-readable source): shared with msa_route_score_fetch's fallback
int gather_copy(const int32_t* ids, int B, int k, const int64_t* chunk_off, int64_t n_docs, const void* k_bar,
                const void* v_bar, int64_t row_vec, int max_ctx, void* k_ctx, void* v_ctx, int32_t* ctx_pos,
                int32_t* ctx_len, hipStream_t s) {
  const dim3 grid{unsigned(k), unsigned(B)}, block{GK_THREADS};
  hipLaunchKernelGGL(gather_kernel<GK_COPY>, grid, block, 0, s, ids, k, chunk_off, n_docs,
                     static_cast<const uint4*>(k_bar), static_cast<const uint4*>(v_bar), row_vec, max_ctx,
                     static_cast<uint4*>(k_ctx), static_cast<uint4*>(v_ctx), ctx_pos, ctx_len, nullptr, nullptr);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

struct CopyEvent {
  hipEvent_t ev = nullptr;
  ~CopyEvent() {
    if (ev) (void)hipEventDestroy(ev);
  }
};

}  // namespace msa

extern "C" int msa_gather_kv(int dtype, const int32_t* ids, int B, int k, const int64_t* chunk_off,
                             const int64_t* chunk_off_h, int64_t n_docs, int max_doc_chunks, const void* k_bar,
                             const void* v_bar, int64_t n_chunks, int Hkv, int d, int src_mode, int max_ctx,
                             void* k_ctx, void* v_ctx, int32_t* ctx_pos, int32_t* ctx_len, int32_t* ids_h,
                             void* stream, void* copy_stream) {
  using namespace msa;
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, "msa_gather_kv: bad dtype");
  MSA_REQUIRE(ids && chunk_off && k_bar && v_bar && k_ctx && v_ctx && ctx_pos && ctx_len, MSA_ERR_INVALID_ARG,
              "msa_gather_kv: NULL pointer");
  MSA_REQUIRE(B >= 1 && k >= 1 && n_docs >= 1 && n_chunks >= 1 && Hkv >= 1 && d >= 1 && max_doc_chunks >= 1,
              MSA_ERR_INVALID_ARG, "msa_gather_kv: non-positive size");
  MSA_REQUIRE(k <= n_docs, MSA_ERR_INVALID_ARG, "msa_gather_kv: k > n_docs");
  MSA_REQUIRE(int64_t(max_ctx) >= int64_t(k) * max_doc_chunks, MSA_ERR_INVALID_ARG,
              "msa_gather_kv: max_ctx < k * max_doc_chunks");
  MSA_REQUIRE(src_mode >= MSA_SRC_DEVICE && src_mode <= MSA_SRC_HOST_MEMCPY, MSA_ERR_UNSUPPORTED,
              "msa_gather_kv: unknown src_mode");
  MSA_REQUIRE(B <= 65535 && k <= 65535, MSA_ERR_UNSUPPORTED, "msa_gather_kv: B or k too large");
  const int64_t row_bytes = int64_t(Hkv) * d * dtype_bytes(dtype);
  MSA_REQUIRE(row_bytes % 16 == 0, MSA_ERR_UNSUPPORTED, "msa_gather_kv: Hkv*d*elem_bytes must be a multiple of 16");
  MSA_REQUIRE(uintptr_t(k_bar) % 16 == 0 && uintptr_t(v_bar) % 16 == 0 && uintptr_t(k_ctx) % 16 == 0 &&
                  uintptr_t(v_ctx) % 16 == 0,
              MSA_ERR_INVALID_ARG, "msa_gather_kv: K/V buffers must be 16-byte aligned");
  const int64_t row_vec = row_bytes / 16;
  hipStream_t s = as_stream(stream);
  const dim3 grid{unsigned(k), unsigned(B)}, block{GK_THREADS};
  if (src_mode != MSA_SRC_HOST_MEMCPY)
    return gather_copy(ids, B, k, chunk_off, n_docs, k_bar, v_bar, row_vec, max_ctx, k_ctx, v_ctx, ctx_pos, ctx_len, s);
  // host copies: the selection must be known on the host
  MSA_REQUIRE(chunk_off_h && ids_h, MSA_ERR_INVALID_ARG, "msa_gather_kv: host mode needs chunk_off_h and ids_h");
  hipStream_t cs = copy_stream ? as_stream(copy_stream) : s;
  MSA_HIP_CHECK(hipMemcpyAsync(ids_h, ids, size_t(B) * k * sizeof(int32_t), hipMemcpyDeviceToHost, s));
  MSA_HIP_CHECK(hipStreamSynchronize(s));
  // positions and lengths on the compute stream
  hipLaunchKernelGGL(gather_kernel<GK_POS>, grid, block, 0, s, ids, k, chunk_off, n_docs,
                     static_cast<const uint4*>(k_bar), static_cast<const uint4*>(v_bar), row_vec, max_ctx,
                     static_cast<uint4*>(k_ctx), static_cast<uint4*>(v_ctx), ctx_pos, ctx_len, nullptr, nullptr);
  MSA_LAUNCH_CHECK();
  const char* kb = static_cast<const char*>(k_bar);
  const char* vb = static_cast<const char*>(v_bar);
  char* kc = static_cast<char*>(k_ctx);
  char* vc = static_cast<char*>(v_ctx);
  for (int b = 0; b < B; ++b) {
    int64_t dest = 0;
    for (int r = 0; r < k; ++r) {
      const int32_t doc = ids_h[int64_t(b) * k + r];
      if (doc < 0 || doc >= n_docs) continue;
      const int64_t lo = chunk_off_h[doc];
      int64_t n = chunk_off_h[doc + 1] - lo;
      if (dest + n > max_ctx) n = dest < max_ctx ? max_ctx - dest : 0;
      if (n > 0) {
        const size_t off_d = size_t((int64_t(b) * max_ctx + dest) * row_bytes);
        MSA_HIP_CHECK(hipMemcpyAsync(kc + off_d, kb + lo * row_bytes, size_t(n * row_bytes), hipMemcpyHostToDevice, cs));
        MSA_HIP_CHECK(hipMemcpyAsync(vc + off_d, vb + lo * row_bytes, size_t(n * row_bytes), hipMemcpyHostToDevice, cs));
      }
      dest += n;
    }
  }
  if (cs != s) {
    static thread_local CopyEvent ce;
    if (!ce.ev) MSA_HIP_CHECK(hipEventCreateWithFlags(&ce.ev, hipEventDisableTiming));
    MSA_HIP_CHECK(hipEventRecord(ce.ev, cs));
    MSA_HIP_CHECK(hipStreamWaitEvent(s, ce.ev, 0));
  }
  return MSA_OK;
}

extern "C" int msa_context_index(const int32_t* ids, int B, int k, const int64_t* chunk_off, int64_t n_docs,
                                 int max_doc_chunks, int64_t n_chunks, int max_ctx, int32_t* ctx_row,
                                 int32_t* ctx_pos, int32_t* ctx_len, void* stream) {
  using namespace msa;
  MSA_REQUIRE(ids && chunk_off && ctx_row && ctx_pos && ctx_len, MSA_ERR_INVALID_ARG,
              "msa_context_index: NULL pointer");
  MSA_REQUIRE(B >= 1 && k >= 1 && n_docs >= 1 && n_chunks >= 1 && max_doc_chunks >= 1, MSA_ERR_INVALID_ARG,
              "msa_context_index: non-positive size");
  MSA_REQUIRE(k <= n_docs, MSA_ERR_INVALID_ARG, "msa_context_index: k > n_docs");
  MSA_REQUIRE(n_chunks <= INT32_MAX, MSA_ERR_UNSUPPORTED, "msa_context_index: n_chunks must be below 2^31");
  MSA_REQUIRE(int64_t(max_ctx) >= int64_t(k) * max_doc_chunks, MSA_ERR_INVALID_ARG,
              "msa_context_index: max_ctx < k * max_doc_chunks");
  MSA_REQUIRE(B <= 65535 && k <= 65535, MSA_ERR_UNSUPPORTED, "msa_context_index: B or k too large");
  const dim3 grid{unsigned(k), unsigned(B)}, block{GK_THREADS};
  hipLaunchKernelGGL(gather_kernel<GK_ROWS>, grid, block, 0, as_stream(stream), ids, k, chunk_off, n_docs, nullptr,
                     nullptr, int64_t(0), max_ctx, nullptr, nullptr, ctx_pos, ctx_len, ctx_row, nullptr);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

extern "C" int msa_context_append(const int32_t* ids, int B, int k, const int64_t* chunk_off, int64_t n_docs,
                                  int max_doc_chunks, int64_t n_chunks, int max_ctx, int32_t* ctx_row,
                                  int32_t* ctx_pos, const int32_t* ctx_len_in, int32_t* ctx_len_out, void* stream) {
  using namespace msa;
  MSA_REQUIRE(ids && chunk_off && ctx_row && ctx_pos && ctx_len_in && ctx_len_out, MSA_ERR_INVALID_ARG,
              "msa_context_append: NULL pointer");
  MSA_REQUIRE(ctx_len_in != ctx_len_out, MSA_ERR_INVALID_ARG,
              "msa_context_append: ctx_len_in and ctx_len_out must be different arrays");
  MSA_REQUIRE(B >= 1 && k >= 1 && n_docs >= 1 && n_chunks >= 1 && max_doc_chunks >= 1, MSA_ERR_INVALID_ARG,
              "msa_context_append: non-positive size");
  MSA_REQUIRE(n_chunks <= INT32_MAX, MSA_ERR_UNSUPPORTED, "msa_context_append: n_chunks must be below 2^31");
  MSA_REQUIRE(int64_t(max_ctx) >= int64_t(k) * max_doc_chunks, MSA_ERR_INVALID_ARG,
              "msa_context_append: max_ctx < k * max_doc_chunks");
  MSA_REQUIRE(B <= 65535 && k <= 65535, MSA_ERR_UNSUPPORTED, "msa_context_append: B or k too large");
  const dim3 grid{unsigned(k), unsigned(B)}, block{GK_THREADS};
  hipLaunchKernelGGL(gather_kernel<GK_ROWS>, grid, block, 0, as_stream(stream), ids, k, chunk_off, n_docs, nullptr,
                     nullptr, int64_t(0), max_ctx, nullptr, nullptr, ctx_pos, ctx_len_out, ctx_row, ctx_len_in);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}
