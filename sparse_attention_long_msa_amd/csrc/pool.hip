// Stage 1: chunk-mean pooling of per-token K / V / K_r, with the optional
// per-(chunk, head) L2 normalisation of the routing keys.
// (MSA README, Overall Design > Architecture: document latent states are
//  chunk-mean pooled; Inference Pipeline: Global Memory Encoding caches the
//  pooled K, V and K_r.  Paper note 核心方法 > 架构: chunk-wise mean pool.)
//
// A chunk's token rows are contiguous (H*d elements each) and are streamed
// with 16-byte loads.  The common shapes (a row of whole waves of 16-byte
// vectors, e.g. H = 8, d = 128) take pool_wave_kernel: one wave per chunk,
// 16 chunks per workgroup.  Other shapes take pool_kernel: one workgroup
// per chunk, whose row groups take interleaved tokens and are combined in a
// fixed order.  Both are deterministic.
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

// Wave-per-chunk pooling, for token rows whose 16-byte vectors fill whole
// waves (H*d*bytes/16 a multiple of 64) and heads that span a power-of-two
// number of lanes.  A workgroup of four waves pools 16 consecutive chunks:
// in the tiled layout those form one 16-chunk group, so each output line is
// written by a single workgroup (on a single XCD), and the padding chunks of
// the last group are written as zeros here.  A wave takes CPW chunks at a
// time and streams their token rows together, so the loads of all CPW chunks
// are in flight at once; a chunk's rows are summed in token order.  A head's
// squared norm is reduced over the lanes that hold it.  In the row layout
// every lane writes its 16-byte piece with one store; in the tiled layout the
// 16 results go through LDS first (below).
constexpr int kPoolWaveThreads = 256;

// With chunk == 1 the chunk CSR equals the token CSR, so chunk c is token c
// and the kernel (ONE) reads no index.
template <int DT, int NP, int CPW, bool ONE>
__global__ __launch_bounds__(kPoolWaveThreads) void pool_wave_kernel(
    const typename Elem<DT>::T* __restrict__ x, const int64_t* __restrict__ tok_off,
    const int64_t* __restrict__ chunk_off, const int32_t* __restrict__ chunk_doc, int64_t n_chunks,
    int64_t n_tok, int H, int d, int chunk, int normalize, int tiled, typename Elem<DT>::T* __restrict__ out) {
  using T = typename Elem<DT>::T;
  constexpr int VE = 16 / Elem<DT>::bytes;  // elements per 16-byte vector
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = H * d;
  const int lph = d / VE;                   // lanes per head
  // tiled output: the group's 16 rows are staged in LDS (row stride padded
  // so that the column-wise reads below spread over all banks) and then
  // written out as one contiguous block in the tiled order
  extern __shared__ __align__(16) unsigned char stage[];
  const int row_b = E * Elem<DT>::bytes + 128 / VE;
  const int64_t n_out = tiled ? (n_chunks + 15) / 16 * 16 : n_chunks;
  const int64_t n_groups = (n_out + 15) / 16;
  for (int64_t g = blockIdx.x; g < n_groups; g += gridDim.x) {
    for (int s0 = 0; s0 < 4; s0 += CPW) {
      int64_t c[CPW], t0[CPW];
      int cnt[CPW];
      int max_cnt = 0;
#pragma unroll
      for (int s = 0; s < CPW; ++s) {
        c[s] = g * 16 + wave * 4 + s0 + s;
        t0[s] = 0;
        cnt[s] = 0;
        if (ONE) {
          t0[s] = c[s];
          cnt[s] = c[s] < n_chunks ? 1 : 0;
        } else if (c[s] < n_chunks) {
          const int32_t doc = chunk_doc[c[s]];
          t0[s] = tok_off[doc] + (c[s] - chunk_off[doc]) * chunk;
          const int64_t t1 = min(t0[s] + chunk, tok_off[doc + 1]);
          cnt[s] = int(t1 - t0[s]);
        }
        max_cnt = max(max_cnt, cnt[s]);
      }
      float acc[CPW][NP * VE];
#pragma unroll
      for (int s = 0; s < CPW; ++s)
#pragma unroll
        for (int k = 0; k < NP * VE; ++k) acc[s][k] = 0.f;
      for (int i = 0; i < max_cnt; ++i) {
        uint4 w[CPW][NP];
#pragma unroll
        for (int s = 0; s < CPW; ++s) {
          // a chunk with fewer rows re-reads its last one (added with weight 0)
          int64_t t = t0[s] + min(i, max(cnt[s], 1) - 1);
          t = min(max(t, int64_t(0)), n_tok - 1);
#pragma unroll
          for (int p = 0; p < NP; ++p) w[s][p] = load_global(x + t * E + int64_t(lane + 64 * p) * VE);
        }
#pragma unroll
        for (int s = 0; s < CPW; ++s) {
          if (i >= cnt[s]) continue;
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const uint32_t ww[4] = {w[s][p].x, w[s][p].y, w[s][p].z, w[s][p].w};
            if constexpr (DT == MSA_BF16) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                acc[s][p * VE + 2 * e] += __uint_as_float(ww[e] << 16);
                acc[s][p * VE + 2 * e + 1] += __uint_as_float(ww[e] & 0xFFFF0000u);
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[s][p * VE + e] += __uint_as_float(ww[e]);
            }
          }
        }
      }
#pragma unroll
      for (int s = 0; s < CPW; ++s) {
        if (c[s] >= n_out) continue;
        const float inv_cnt = cnt[s] > 0 ? 1.f / float(cnt[s]) : 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          float r[VE];
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            r[e] = acc[s][p * VE + e] * inv_cnt;
            ss += r[e] * r[e];
          }
          if (normalize) {
            for (int m = 1; m < lph; m <<= 1) ss += __shfl_xor(ss, m);
            const float inv = 1.f / fmaxf(sqrtf(ss), 1e-8f);
#pragma unroll
            for (int e = 0; e < VE; ++e) r[e] *= inv;
          }
          const int e0 = (lane + 64 * p) * VE;
          uint4 v;
          if constexpr (DT == MSA_BF16) {
            v.x = uint32_t(f32_to_bf16(r[0])) | (uint32_t(f32_to_bf16(r[1])) << 16);
            v.y = uint32_t(f32_to_bf16(r[2])) | (uint32_t(f32_to_bf16(r[3])) << 16);
            v.z = uint32_t(f32_to_bf16(r[4])) | (uint32_t(f32_to_bf16(r[5])) << 16);
            v.w = uint32_t(f32_to_bf16(r[6])) | (uint32_t(f32_to_bf16(r[7])) << 16);
          } else {
            v = make_uint4(__float_as_uint(r[0]), __float_as_uint(r[1]), __float_as_uint(r[2]),
                           __float_as_uint(r[3]));
          }
          if (tiled)
            *reinterpret_cast<uint4*>(stage + (wave * 4 + s0 + s) * row_b + e0 * Elem<DT>::bytes) = v;
          else
            *reinterpret_cast<uint4*>(out + c[s] * E + e0) = v;
        }
      }
    }
    if (tiled) {
      __syncthreads();
      T* gout = out + g * 16 * int64_t(E);
      for (int u = threadIdx.x; u < 16 * E / VE; u += kPoolWaveThreads) {
        // 16-byte unit u of the group block: head h, then e/32, (e%32)/8,
        // chunk within the group, e%8
        const int o = u * VE, h = o / (16 * d), rem = o - h * 16 * d;
        const int c16 = (rem & 127) >> 3, e = (rem >> 9) * 32 + ((rem >> 7) & 3) * 8 + (rem & 7);
        *reinterpret_cast<uint4*>(gout + o) =
            *reinterpret_cast<const uint4*>(stage + c16 * row_b + (h * d + e) * Elem<DT>::bytes);
      }
      __syncthreads();
    }
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
  MSA_REQUIRE(out != x, MSA_ERR_INVALID_ARG, "msa_pool_encode: out must not alias x");
  MSA_REQUIRE(n_docs >= 1 && n_tok >= 1 && n_chunks >= 1 && H >= 1 && d >= 2 && chunk >= 1,
              MSA_ERR_INVALID_ARG, "msa_pool_encode: non-positive size");
  MSA_REQUIRE(d % 2 == 0, MSA_ERR_INVALID_ARG, "msa_pool_encode: d must be even");
  MSA_REQUIRE(out_layout == MSA_LAYOUT_ROWS || (out_layout == MSA_LAYOUT_TILED && d % 32 == 0), MSA_ERR_INVALID_ARG,
              "msa_pool_encode: bad out_layout (tiled needs d % 32 == 0)");
  MSA_REQUIRE(chunk != 1 || n_chunks == n_tok, MSA_ERR_INVALID_ARG,
              "msa_pool_encode: with chunk == 1 every token is a chunk (n_chunks must equal n_tok)");
  const int E = H * d;
  const int VE = 16 / dtype_bytes(dtype);
  MSA_REQUIRE(E <= 4096 && E % 8 == 0, MSA_ERR_UNSUPPORTED, "msa_pool_encode: H*d must be <= 4096 and a multiple of 8");
  const int V = E / VE;
  MSA_REQUIRE(uintptr_t(x) % 16 == 0, MSA_ERR_INVALID_ARG, "msa_pool_encode: x not 16-byte aligned");
  const int lph = d / VE;
  if (V % 64 == 0 && V / 64 <= 8 && d % VE == 0 && lph <= 64 && (lph & (lph - 1)) == 0 &&
      uintptr_t(out) % 16 == 0) {
    const int64_t n_groups = (n_chunks + 15) / 16;
    const dim3 grid(unsigned(std::min<int64_t>(n_groups, int64_t(1) << 20)));
    const int tiled = out_layout == MSA_LAYOUT_TILED;
    const size_t lds = tiled ? 16 * size_t(E * dtype_bytes(dtype) + 128 / VE) : 0;
#define MSA_POOL_WAVE_1(NP, CPW, ONE)                                                                         \
  do {                                                                                                        \
    if (lds > 65536) {                                                                                        \
      MSA_HIP_CHECK(hipFuncSetAttribute(                                                                      \
          dtype == MSA_BF16 ? reinterpret_cast<const void*>(&pool_wave_kernel<MSA_BF16, NP, CPW, ONE>)        \
                            : reinterpret_cast<const void*>(&pool_wave_kernel<MSA_F32, NP, CPW, ONE>),        \
          hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)));                                             \
    }                                                                                                         \
    if (dtype == MSA_BF16)                                                                                    \
      hipLaunchKernelGGL((pool_wave_kernel<MSA_BF16, NP, CPW, ONE>), grid, dim3(kPoolWaveThreads), lds,       \
                         as_stream(stream), static_cast<const uint16_t*>(x), tok_off, chunk_off, chunk_doc,   \
                         n_chunks, n_tok, H, d, chunk, l2_normalize, tiled, static_cast<uint16_t*>(out));     \
    else                                                                                                      \
      hipLaunchKernelGGL((pool_wave_kernel<MSA_F32, NP, CPW, ONE>), grid, dim3(kPoolWaveThreads), lds,        \
                         as_stream(stream), static_cast<const float*>(x), tok_off, chunk_off, chunk_doc,      \
                         n_chunks, n_tok, H, d, chunk, l2_normalize, tiled, static_cast<float*>(out));        \
  } while (0)
#define MSA_POOL_WAVE(NP, CPW)              \
  do {                                      \
    if (chunk == 1)                         \
      MSA_POOL_WAVE_1(NP, CPW, true);       \
    else                                    \
      MSA_POOL_WAVE_1(NP, CPW, false);      \
  } while (0)
    switch (V / 64) {
      case 1: MSA_POOL_WAVE(1, 4); break;
      case 2: MSA_POOL_WAVE(2, 4); break;
      case 3: MSA_POOL_WAVE(3, 2); break;
      case 4: MSA_POOL_WAVE(4, 2); break;
      case 5: MSA_POOL_WAVE(5, 1); break;
      case 6: MSA_POOL_WAVE(6, 1); break;
      case 7: MSA_POOL_WAVE(7, 1); break;
      default: MSA_POOL_WAVE(8, 1); break;
    }
#undef MSA_POOL_WAVE
#undef MSA_POOL_WAVE_1
    MSA_LAUNCH_CHECK();
    return MSA_OK;
  }
  MSA_REQUIRE(V >= kPoolThreads || kPoolThreads % V == 0, MSA_ERR_UNSUPPORTED,
              "msa_pool_encode: unsupported H*d (16-byte vectors per token row)");
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
