// Stage 1: chunk-mean pooling of per-token K / V / K_r, with the optional
// per-(chunk, head) L2 normalisation of the routing keys.
// (MSA README, Overall Design > Architecture: document latent states are
//  chunk-mean pooled; Inference Pipeline: Global Memory Encoding caches the
//  pooled K, V and K_r.  Paper note 核心方法 > 架构: chunk-wise mean pool.)
//
// One workgroup per pooled chunk.  The chunk's token rows are contiguous
// (H*d elements each), so threads stream them with 16-byte loads; row
// groups of the workgroup take interleaved tokens and are combined in a
// fixed order, so the result is deterministic.
#include <algorithm>

#include "common.h"

namespace msa {

constexpr int kPoolThreads = 256;

// Element offset of (chunk c, head h, element e) in MSA_LAYOUT_TILED.
__device__ __forceinline__ int64_t tiled_offset(int64_t c, int h, int e, int H, int d) {
  return (c / 16) * (16 * int64_t(H) * d) + int64_t(h) * (16 * d) + (e / 32) * 512 + ((e % 32) / 8) * 128 +
         (c % 16) * 8 + (e % 8);
}

template <int DT>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(
    const typename Elem<DT>::T* __restrict__ x, const int64_t* __restrict__ tok_off,
    const int64_t* __restrict__ chunk_off, const int32_t* __restrict__ chunk_doc, int64_t n_chunks,
    int H, int d, int chunk, int normalize, int tiled, typename Elem<DT>::T* __restrict__ out) {
  constexpr int VE = 16 / Elem<DT>::bytes;  // elements per 16-byte vector
  extern __shared__ float smem[];
  const int E = H * d;
  const int V = E / VE;                               // vectors per token row
  const int R = V < kPoolThreads ? kPoolThreads / V : 1;  // row groups
  float* part = smem;                                 // [R][E]
  float* mean = smem + size_t(R) * E;                 // [E]
  float* scale = mean + E;                            // [H]
  const int tid = threadIdx.x;

  for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const int32_t doc = chunk_doc[c];
    const int64_t j = c - chunk_off[doc];
    const int64_t t0 = tok_off[doc] + j * chunk;
    int64_t t1 = t0 + chunk;
    if (t1 > tok_off[doc + 1]) t1 = tok_off[doc + 1];
    const int cnt = int(t1 - t0);

    const int rg = V < kPoolThreads ? tid / V : 0;
    for (int v = (V < kPoolThreads ? tid % V : tid); v < V && rg < R; v += kPoolThreads) {
      float acc[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = 0.f;
      for (int64_t t = t0 + rg; t < t1; t += R) {
        const uint4 w = *reinterpret_cast<const uint4*>(x + t * E + int64_t(v) * VE);
        if constexpr (DT == MSA_BF16) {
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(ww[e] << 16);
            acc[2 * e + 1] += __uint_as_float(ww[e] & 0xFFFF0000u);
          }
        } else {
          acc[0] += __uint_as_float(w.x);
          acc[1] += __uint_as_float(w.y);
          acc[2] += __uint_as_float(w.z);
          acc[3] += __uint_as_float(w.w);
        }
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) part[size_t(rg) * E + v * VE + e] = acc[e];
    }
    __syncthreads();
    for (int e = tid; e < E; e += kPoolThreads) {
      float s = 0.f;
      for (int r = 0; r < R; ++r) s += part[size_t(r) * E + e];
      mean[e] = s / float(cnt);
    }
    __syncthreads();
    if (tid < H) {
      float sc = 1.f;
      if (normalize) {
        float ss = 0.f;
        for (int e = 0; e < d; ++e) {
          const float m = mean[tid * d + e];
          ss += m * m;
        }
        sc = fmaxf(sqrtf(ss), 1e-8f);
      }
      scale[tid] = sc;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kPoolThreads) {
      const float r = normalize ? mean[e] / scale[e / d] : mean[e];
      const int64_t o = tiled ? tiled_offset(c, e / d, e % d, H, d) : c * E + e;
      if constexpr (DT == MSA_BF16)
        out[o] = f32_to_bf16(r);
      else
        out[o] = r;
    }
    __syncthreads();
  }
}

// MSA_LAYOUT_ROWS -> MSA_LAYOUT_TILED; one thread per 8 consecutive elements
// of one (chunk, head); chunks past n_chunks in the last group are zeroed.
template <typename T>
__global__ void tile_kernel(const T* __restrict__ src, int64_t n_chunks, int H, int d, T* __restrict__ dst) {
  const int vpr = d / 8;                                   // 8-element vectors per (chunk, head)
  const int64_t n_pad = (n_chunks + 15) / 16 * 16;
  const int64_t total = n_pad * H * vpr;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
    const int v = int(i % vpr);
    const int h = int((i / vpr) % H);
    const int64_t c = i / (int64_t(vpr) * H);
    T* o = dst + tiled_offset(c, h, 8 * v, H, d);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = c < n_chunks ? src[(c * H + h) * d + 8 * v + e] : T(0);
  }
}

template <typename T>
__global__ void zero_padding_kernel(int64_t n_chunks, int H, int d, T* __restrict__ dst) {
  const int64_t n_pad = (n_chunks + 15) / 16 * 16;
  const int64_t per = int64_t(H) * d;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < (n_pad - n_chunks) * per;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t c = n_chunks + i / per;
    const int h = int((i % per) / d), e = int(i % d);
    dst[tiled_offset(c, h, e, H, d)] = T(0);
  }
}

}  // namespace msa

extern "C" int msa_tile_routing_keys(int dtype, const void* src, int64_t n_chunks, int H, int d, void* dst,
                                     void* stream) {
  using namespace msa;
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, "msa_tile_routing_keys: bad dtype");
  MSA_REQUIRE(src && dst && src != dst, MSA_ERR_INVALID_ARG, "msa_tile_routing_keys: NULL or aliased pointers");
  MSA_REQUIRE(n_chunks >= 1 && H >= 1 && d >= 32 && d % 32 == 0, MSA_ERR_INVALID_ARG,
              "msa_tile_routing_keys: sizes (d must be a multiple of 32)");
  const int64_t total = (n_chunks + 15) / 16 * 16 * H * (d / 8);
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  if (dtype == MSA_BF16)
    hipLaunchKernelGGL(tile_kernel<uint16_t>, dim3(unsigned(blocks)), dim3(256), 0, as_stream(stream),
                       static_cast<const uint16_t*>(src), n_chunks, H, d, static_cast<uint16_t*>(dst));
  else
    hipLaunchKernelGGL(tile_kernel<float>, dim3(unsigned(blocks)), dim3(256), 0, as_stream(stream),
                       static_cast<const float*>(src), n_chunks, H, d, static_cast<float*>(dst));
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

extern "C" int msa_pool_encode(int dtype, const void* x, const int64_t* tok_off, const int64_t* chunk_off,
                               const int32_t* chunk_doc, int64_t n_docs, int64_t n_tok, int64_t n_chunks,
                               int H, int d, int chunk, int l2_normalize, int out_layout, void* out,
                               void* stream) {
  using namespace msa;
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, "msa_pool_encode: bad dtype");
  MSA_REQUIRE(x && tok_off && chunk_off && chunk_doc && out, MSA_ERR_INVALID_ARG,
              "msa_pool_encode: NULL pointer");
  MSA_REQUIRE(n_docs >= 1 && n_tok >= 1 && n_chunks >= 1 && H >= 1 && d >= 2 && chunk >= 1,
              MSA_ERR_INVALID_ARG, "msa_pool_encode: non-positive size");
  MSA_REQUIRE(d % 2 == 0, MSA_ERR_INVALID_ARG, "msa_pool_encode: d must be even");
  MSA_REQUIRE(out_layout == MSA_LAYOUT_ROWS || (out_layout == MSA_LAYOUT_TILED && d % 32 == 0), MSA_ERR_INVALID_ARG,
              "msa_pool_encode: bad out_layout (tiled needs d % 32 == 0)");
  const int E = H * d;
  const int VE = 16 / dtype_bytes(dtype);
  MSA_REQUIRE(E <= 4096 && E % 8 == 0, MSA_ERR_UNSUPPORTED, "msa_pool_encode: H*d must be <= 4096 and a multiple of 8");
  const int V = E / VE;
  MSA_REQUIRE(V >= kPoolThreads || kPoolThreads % V == 0, MSA_ERR_UNSUPPORTED,
              "msa_pool_encode: H*d*elem_bytes/16 must divide 256 or be a multiple of it");
  MSA_REQUIRE(uintptr_t(x) % 16 == 0, MSA_ERR_INVALID_ARG, "msa_pool_encode: x not 16-byte aligned");
  const int R = V < kPoolThreads ? kPoolThreads / V : 1;
  const size_t smem = (size_t(R) * E + E + H) * sizeof(float);
  MSA_REQUIRE(smem <= 160 * 1024, MSA_ERR_UNSUPPORTED, "msa_pool_encode: LDS budget exceeded");
  const int64_t grid = n_chunks < (int64_t(1) << 20) ? n_chunks : (int64_t(1) << 20);
  if (dtype == MSA_BF16)
    hipLaunchKernelGGL(pool_kernel<MSA_BF16>, dim3(unsigned(grid)), dim3(kPoolThreads), smem, as_stream(stream),
                       static_cast<const uint16_t*>(x), tok_off, chunk_off, chunk_doc, n_chunks, H, d, chunk,
                       l2_normalize, out_layout, static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(pool_kernel<MSA_F32>, dim3(unsigned(grid)), dim3(kPoolThreads), smem, as_stream(stream),
                       static_cast<const float*>(x), tok_off, chunk_off, chunk_doc, n_chunks, H, d, chunk,
                       l2_normalize, out_layout, static_cast<float*>(out));
  MSA_LAUNCH_CHECK();
  if (out_layout == MSA_LAYOUT_TILED && n_chunks % 16 != 0) {
    if (dtype == MSA_BF16)
      hipLaunchKernelGGL(zero_padding_kernel<uint16_t>, dim3(64), dim3(256), 0, as_stream(stream), n_chunks, H, d,
                         static_cast<uint16_t*>(out));
    else
      hipLaunchKernelGGL(zero_padding_kernel<float>, dim3(64), dim3(256), 0, as_stream(stream), n_chunks, H, d,
                         static_cast<float*>(out));
    MSA_LAUNCH_CHECK();
  }
  return MSA_OK;
}
