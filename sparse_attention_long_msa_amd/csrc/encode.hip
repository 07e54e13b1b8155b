// Stage 1 at corpus scale: projection of the document tokens' hidden states
// to K, V and the routing key K_r, then the chunk-wise mean pool (and the
// routing key's L2 normalisation), in one call.
// (README, Overall Design > Inference Pipeline, stage 1, global memory encoding:
//  a forward over the corpus caches the chunk-pooled (K, V, K_r); paper note
//  核心方法 > 架构: each document's K/V/K_r, the routing key from an extra
//  projector, chunk-wise mean pooled.)
//
// The projection is linear and the pool is a mean, so the mean of the
// projected tokens is the projection of the mean token: the hidden states
// are pooled first (float32 sums, the corpus is read once) and the
// projection runs on the 1/chunk as many pooled rows.  Readings: K, V and
// K_r are plain linear projections of the hidden state (no per-token
// normalisation before pooling), stored un-rotated (RoPE is applied at
// attention time with the chunk's index).
//
// bf16 (MFMA): the float32 pooled row is split into two bf16 parts (hi +
// lo, the row to 2^-17 relative); their products with the bf16 weights are
// exact in the float32 accumulator; the result is rounded once to bf16.
#include <algorithm>

#include "common.h"

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int EN_GW = 8;                 // waves per GEMM workgroup
constexpr int EN_THREADS = 64 * EN_GW;
constexpr float EN_EPS = 1e-8f;

// xbar[c, :] = mean of the hidden rows of chunk c (float32).  SPLIT (bf16
// input, MFMA path): the mean is written instead as its two bf16 parts,
// hi = bf16(m) to xbar_hi and lo = bf16(m - hi) to xbar_lo (n_chunks x hidden
// each, the same bytes as the float32 row), once for every projection.
template <int DT, bool SPLIT>
__global__ __launch_bounds__(1024) void pool_hidden_kernel(
    const typename Elem<DT>::T* __restrict__ x, int hidden, const int64_t* __restrict__ tok_off,
    const int64_t* __restrict__ chunk_off, const int32_t* __restrict__ chunk_doc, int64_t n_docs, int64_t n_chunks,
    int chunk, float* __restrict__ xbar) {
  static_assert(!SPLIT || DT == MSA_BF16, "the split rows serve the bf16 MFMA path");
  constexpr int VE = 16 / Elem<DT>::bytes;   // elements per 16-byte vector
  const int nv = hidden / VE;
  for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const int doc = chunk_doc[c];
    if (doc < 0 || doc >= n_docs) continue;
    const int64_t t0 = tok_off[doc] + (c - chunk_off[doc]) * int64_t(chunk);
    const int64_t n = min(int64_t(chunk), tok_off[doc + 1] - t0);
    const float inv = n > 0 ? 1.f / float(n) : 0.f;
    for (int v = threadIdx.x; v < nv; v += blockDim.x) {
      float acc[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = 0.f;
#pragma unroll 8
      for (int64_t t = t0; t < t0 + n; ++t) {
        const uint4 w = load_stream(x + t * hidden + int64_t(v) * VE);   // read once: non-temporal
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
      if constexpr (SPLIT) {
        uint16_t* xh = reinterpret_cast<uint16_t*>(xbar);
        uint16_t* xl = xh + n_chunks * hidden;
        uint32_t hi[VE / 2], lo[VE / 2];
#pragma unroll
        for (int e = 0; e < VE / 2; ++e) {
          const float m0 = acc[2 * e] * inv, m1 = acc[2 * e + 1] * inv;
          const uint16_t h0 = f32_to_bf16(m0), h1 = f32_to_bf16(m1);
          hi[e] = uint32_t(h0) | (uint32_t(h1) << 16);
          lo[e] = uint32_t(f32_to_bf16(m0 - bf16_to_f32(h0))) | (uint32_t(f32_to_bf16(m1 - bf16_to_f32(h1))) << 16);
        }
        const int64_t o = c * hidden + int64_t(v) * VE;
        *reinterpret_cast<uint4*>(xh + o) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4*>(xl + o) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      } else {
        float* o = xbar + c * hidden + int64_t(v) * VE;
#pragma unroll
        for (int e = 0; e < VE; e += 4)
          *reinterpret_cast<float4*>(o + e) =
              make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
      }
    }
  }
}

// This wave's LDS operations are complete, then the workgroup barrier
// (outstanding vector-memory loads stay in flight).
__device__ __forceinline__ void lds_barrier_enc() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// element (c, h, e) of a store in the given layout
__device__ __forceinline__ int64_t store_index(int64_t c, int h, int e, int H, int d, bool tiled) {
  if (!tiled) return (c * H + h) * d + e;
  return (c / 16) * 16 * int64_t(H) * d + int64_t(h) * 16 * d + (e / 32) * 512 + ((e % 32) / 8) * 128 + (c % 16) * 8 +
         e % 8;
}

// Workgroup = 512 pooled rows x one head (128 columns) of one of K, V, K_r,
// in eight waves; wave w computes rows 64w..64w+63 (four 16-row tiles, so
// that each weight fragment read from LDS feeds four products, and each
// staged slice serves 512 rows).  A operand: the pooled rows' two bf16 parts
// (hi + lo, written by the pooling kernel), read by each wave; B operand:
// the 32-wide k-slice of the head's 128 weight rows (w_t [3*H*128, hidden],
// one row per output feature) staged once per workgroup in LDS, the next
// slice loading while the current one is used.
// Workgroups map to (row tile, column block) XCD-aware when the column
// blocks split evenly over the 8 XCDs (workgroup i runs on XCD i % 8): each
// XCD owns a few column blocks, whose weights stay in its L2, and takes the
// row tiles in order, so the workgroups sharing a row tile run together and
// the tile is read once per XCD.
constexpr int EN_D = 128;
constexpr int EN_MW = 4;              // 16-row tiles per wave
constexpr int EN_ROWS = 16 * EN_MW * EN_GW;   // pooled rows per workgroup
constexpr int EN_BS = 5;       // LDS stride of a weight row, in 16-byte pieces (4 + 1 pad)

// Two waves per SIMD: the 128 accumulators fit in 256 VGPRs without AGPRs.
__global__ __launch_bounds__(EN_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void encode_gemm_kernel(
    const uint16_t* __restrict__ xh, const uint16_t* __restrict__ xl, int hidden, const uint16_t* __restrict__ w_t,
    int H, int64_t n_chunks, int kr_tiled, uint16_t* __restrict__ k_bar, uint16_t* __restrict__ v_bar,
    uint16_t* __restrict__ kr_hat) {
  __shared__ uint4 bs[2][EN_D * EN_BS];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, lc = lane % 16, g4 = lane / 16;
  const int64_t n_rt = (n_chunks + EN_ROWS - 1) / EN_ROWS;
  const int n_cb = 3 * H;                          // column blocks: tensor * H + head
  int64_t rt;
  int cb;
  if (n_cb % 8 == 0) {
    const int cpx = n_cb / 8;                      // column blocks per XCD
    const int64_t slot = blockIdx.x / 8;
    cb = int(blockIdx.x % 8) * cpx + int(slot % cpx);
    rt = slot / cpx;
  } else {
    rt = blockIdx.x % n_rt;
    cb = int(blockIdx.x / n_rt);
  }
  const int tensor = cb / H, h = cb % H;
  int64_t arow[EN_MW];
#pragma unroll
  for (int m = 0; m < EN_MW; ++m)   // A-operand row of this lane
    arow[m] = min(rt * EN_ROWS + 16 * EN_MW * wave + 16 * m + lc, n_chunks - 1) * hidden + 8 * g4;
  // staging: thread tid copies pieces (row tid / 2, k-quarters 2 * (tid % 2) + {0, 1}) of the slice
  const int srow = tid / 4, sq = tid % 4;
  const uint16_t* sp = w_t + (int64_t(cb) * EN_D + srow) * hidden + 8 * sq;
  f32x4 acc[EN_MW][8];
#pragma unroll
  for (int m = 0; m < EN_MW; ++m)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int n_k = hidden / 32;
  uint4 w0 = load_global(sp);
  for (int ks = 0; ks < n_k; ++ks) {
    const int buf = ks & 1;
    bs[buf][srow * EN_BS + sq] = w0;
    const int kn = min(ks + 1, n_k - 1) * 32;   // the next slice (the last one again at the end: never used)
    w0 = load_global(sp + kn);
    const int k0 = ks * 32;
    bf16x8 ahi[EN_MW], alo[EN_MW];
#pragma unroll
    for (int m = 0; m < EN_MW; ++m) {
      ahi[m] = __builtin_bit_cast(bf16x8, load_global(xh + arow[m] + k0));
      alo[m] = __builtin_bit_cast(bf16x8, load_global(xl + arow[m] + k0));
    }
    // a buffer is rewritten two slices after it was read; each wave's reads precede its next barrier
    lds_barrier_enc();
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, bs[buf][(16 * t + lc) * EN_BS + g4]);
#pragma unroll
      for (int m = 0; m < EN_MW; ++m) {
        acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[m], b, acc[m][t], 0, 0, 0);
        acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[m], b, acc[m][t], 0, 0, 0);
      }
    }
  }
  // lane (lc, g4) holds out[row 32w + 16m + 4*g4 + i][col 16t + lc]
  uint16_t* out = tensor == 0 ? k_bar : (tensor == 1 ? v_bar : kr_hat);
  const bool tiled = tensor == 2 && kr_tiled;
#pragma unroll
  for (int m = 0; m < EN_MW; ++m) {
    float scale[4] = {1.f, 1.f, 1.f, 1.f};
    if (tensor == 2) {   // routing key: L2-normalise each row of this head
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float ss = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) ss += acc[m][t][i] * acc[m][t][i];
#pragma unroll
        for (int sh = 1; sh < 16; sh <<= 1) ss += __shfl_xor(ss, sh);
        scale[i] = 1.f / fmaxf(sqrtf(ss), EN_EPS);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t c = rt * EN_ROWS + 16 * EN_MW * wave + 16 * m + 4 * g4 + i;
      if (c >= n_chunks) continue;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        out[store_index(c, h, 16 * t + lc, H, EN_D, tiled)] = f32_to_bf16(acc[m][t][i] * scale[i]);
    }
  }
}

// Vector path (float32, or any head size): one thread per (pooled row, output column)
template <int DT>
__global__ void encode_vec_kernel(const float* __restrict__ xbar, int hidden, const typename Elem<DT>::T* __restrict__ w_t,
                                  int H, int d, int64_t n_chunks, int kr_tiled, typename Elem<DT>::T* __restrict__ k_bar,
                                  typename Elem<DT>::T* __restrict__ v_bar, typename Elem<DT>::T* __restrict__ kr_hat,
                                  float* __restrict__ kr_tmp) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int cols = 3 * H * d;
  if (i >= n_chunks * cols) return;
  const int64_t c = i / cols;
  const int col = int(i % cols);
  float acc = 0.f;
  for (int k = 0; k < hidden; ++k) acc += xbar[c * hidden + k] * Elem<DT>::load(w_t, int64_t(col) * hidden + k);
  const int tensor = col / (H * d), h = (col / d) % H, e = col % d;
  if (tensor == 2) {
    kr_tmp[(c * H + h) * d + e] = acc;   // normalised by encode_vec_norm_kernel
    return;
  }
  typename Elem<DT>::T* out = tensor == 0 ? k_bar : v_bar;
  if constexpr (DT == MSA_BF16)
    out[(c * H + h) * d + e] = f32_to_bf16(acc);
  else
    out[(c * H + h) * d + e] = acc;
}

template <int DT>
__global__ void encode_vec_norm_kernel(const float* __restrict__ kr_tmp, int H, int d, int64_t n_chunks, int kr_tiled,
                                       typename Elem<DT>::T* __restrict__ kr_hat) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;   // (chunk, head)
  if (i >= n_chunks * H) return;
  const int64_t c = i / H;
  const int h = int(i % H);
  const float* p = kr_tmp + i * d;
  float ss = 0.f;
  for (int e = 0; e < d; ++e) ss += p[e] * p[e];
  const float s = 1.f / fmaxf(sqrtf(ss), EN_EPS);
  for (int e = 0; e < d; ++e) {
    const int64_t o = store_index(c, h, e, H, d, kr_tiled != 0);
    if constexpr (DT == MSA_BF16)
      kr_hat[o] = f32_to_bf16(p[e] * s);
    else
      kr_hat[o] = p[e] * s;
  }
}

template <typename T>
__global__ void zero_pad_tiled_kernel(int64_t n_chunks, int H, int d, T* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n_pad = (n_chunks + 15) / 16 * 16 - n_chunks;
  if (i >= n_pad * H * d) return;
  const int64_t c = n_chunks + i / (int64_t(H) * d);
  const int h = int((i / d) % H), e = int(i % d);
  out[store_index(c, h, e, H, d, true)] = T(0);
}

static bool encode_mfma(int dtype, int hidden, int d) { return dtype == MSA_BF16 && d == EN_D && hidden % 32 == 0; }

}  // namespace msa

extern "C" size_t msa_encode_workspace(int dtype, int64_t n_chunks, int hidden, int H, int d) {
  if (n_chunks < 1 || hidden < 1 || H < 1 || d < 1) return 0;
  size_t b = msa::align_up(size_t(n_chunks) * hidden * 4, 256);
  if (!msa::encode_mfma(dtype, hidden, d)) b += msa::align_up(size_t(n_chunks) * H * d * 4, 256);
  return b;
}

namespace msa {

// The two halves of msa_encode.  The workspace carries the pooled rows from
// the first to the second: float32 rows, or on the MFMA path their bf16
// hi/lo parts (the same bytes), then on the vector path the routing keys'
// float32 staging after them.
static int encode_pool(const std::string& fn, int dtype, const void* x, int hidden, int H, int d,
                       const int64_t* tok_off, const int64_t* chunk_off, const int32_t* chunk_doc, int64_t n_docs,
                       int64_t n_tok, int64_t n_chunks, int chunk, void* ws, size_t ws_bytes, void* stream) {
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, fn + ": bad dtype");
  MSA_REQUIRE(x && tok_off && chunk_off && chunk_doc && ws, MSA_ERR_INVALID_ARG, fn + ": NULL pointer");
  MSA_REQUIRE(hidden >= 1 && H >= 1 && d >= 1 && n_docs >= 1 && n_tok >= 1 && n_chunks >= 1 && chunk >= 1,
              MSA_ERR_INVALID_ARG, fn + ": non-positive size");
  MSA_REQUIRE(hidden % (16 / dtype_bytes(dtype)) == 0, MSA_ERR_UNSUPPORTED,
              fn + ": hidden must hold whole 16-byte vectors");
  MSA_REQUIRE(uintptr_t(x) % 16 == 0, MSA_ERR_INVALID_ARG, fn + ": x must be 16-byte aligned");
  MSA_REQUIRE(ws_bytes >= msa_encode_workspace(dtype, n_chunks, hidden, H, d), MSA_ERR_WORKSPACE,
              fn + ": workspace too small");
  hipStream_t s = as_stream(stream);
  float* xbar = static_cast<float*>(ws);
  const unsigned pgrid = unsigned(std::min<int64_t>(n_chunks, 1 << 20));
  const int nv = hidden / (16 / dtype_bytes(dtype));
  const unsigned pblock = unsigned(std::min(1024, (nv + 63) / 64 * 64));   // one thread per 16-byte vector of a row
  if (encode_mfma(dtype, hidden, d))
    hipLaunchKernelGGL((pool_hidden_kernel<MSA_BF16, true>), dim3(pgrid), dim3(pblock), 0, s,
                       static_cast<const uint16_t*>(x), hidden, tok_off, chunk_off, chunk_doc, n_docs, n_chunks, chunk,
                       xbar);
  else if (dtype == MSA_BF16)
    hipLaunchKernelGGL((pool_hidden_kernel<MSA_BF16, false>), dim3(pgrid), dim3(pblock), 0, s,
                       static_cast<const uint16_t*>(x), hidden, tok_off, chunk_off, chunk_doc, n_docs, n_chunks, chunk,
                       xbar);
  else
    hipLaunchKernelGGL((pool_hidden_kernel<MSA_F32, false>), dim3(pgrid), dim3(pblock), 0, s,
                       static_cast<const float*>(x), hidden, tok_off, chunk_off, chunk_doc, n_docs, n_chunks, chunk, xbar);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

static int encode_project(const std::string& fn, int dtype, const void* w_t, int hidden, int H, int d,
                          int64_t n_chunks, int kr_layout, void* k_bar, void* v_bar, void* kr_hat, void* ws,
                          size_t ws_bytes, void* stream) {
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, fn + ": bad dtype");
  MSA_REQUIRE(w_t && k_bar && v_bar && kr_hat && ws, MSA_ERR_INVALID_ARG, fn + ": NULL pointer");
  MSA_REQUIRE(hidden >= 1 && H >= 1 && d >= 1 && n_chunks >= 1, MSA_ERR_INVALID_ARG, fn + ": non-positive size");
  MSA_REQUIRE(kr_layout == MSA_LAYOUT_ROWS || (kr_layout == MSA_LAYOUT_TILED && d % 32 == 0), MSA_ERR_INVALID_ARG,
              fn + ": bad kr_layout");
  MSA_REQUIRE(hidden % (16 / dtype_bytes(dtype)) == 0, MSA_ERR_UNSUPPORTED,
              fn + ": hidden must hold whole 16-byte vectors");
  MSA_REQUIRE(uintptr_t(w_t) % 16 == 0, MSA_ERR_INVALID_ARG, fn + ": w_t must be 16-byte aligned");
  MSA_REQUIRE(ws_bytes >= msa_encode_workspace(dtype, n_chunks, hidden, H, d), MSA_ERR_WORKSPACE,
              fn + ": workspace too small");
  hipStream_t s = as_stream(stream);
  float* xbar = static_cast<float*>(ws);
  const int tiled = kr_layout == MSA_LAYOUT_TILED;
  if (encode_mfma(dtype, hidden, d)) {
    const int64_t n_rt = (n_chunks + EN_ROWS - 1) / EN_ROWS;
    const uint16_t* xh = reinterpret_cast<const uint16_t*>(xbar);
    hipLaunchKernelGGL(encode_gemm_kernel, dim3(unsigned(n_rt * 3 * H)), dim3(EN_THREADS), 0, s, xh,
                       xh + n_chunks * hidden, hidden, static_cast<const uint16_t*>(w_t), H, n_chunks, tiled,
                       static_cast<uint16_t*>(k_bar), static_cast<uint16_t*>(v_bar), static_cast<uint16_t*>(kr_hat));
    MSA_LAUNCH_CHECK();
  } else {
    float* kr_tmp = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(size_t(n_chunks) * hidden * 4, 256));
    const int64_t n = n_chunks * 3 * H * d;
    const int64_t nn = n_chunks * H;
    if (dtype == MSA_BF16) {
      hipLaunchKernelGGL(encode_vec_kernel<MSA_BF16>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, xbar, hidden,
                         static_cast<const uint16_t*>(w_t), H, d, n_chunks, tiled, static_cast<uint16_t*>(k_bar),
                         static_cast<uint16_t*>(v_bar), static_cast<uint16_t*>(kr_hat), kr_tmp);
      MSA_LAUNCH_CHECK();
      hipLaunchKernelGGL(encode_vec_norm_kernel<MSA_BF16>, dim3(unsigned((nn + 255) / 256)), dim3(256), 0, s, kr_tmp,
                         H, d, n_chunks, tiled, static_cast<uint16_t*>(kr_hat));
    } else {
      hipLaunchKernelGGL(encode_vec_kernel<MSA_F32>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, xbar, hidden,
                         static_cast<const float*>(w_t), H, d, n_chunks, tiled, static_cast<float*>(k_bar),
                         static_cast<float*>(v_bar), static_cast<float*>(kr_hat), kr_tmp);
      MSA_LAUNCH_CHECK();
      hipLaunchKernelGGL(encode_vec_norm_kernel<MSA_F32>, dim3(unsigned((nn + 255) / 256)), dim3(256), 0, s, kr_tmp,
                         H, d, n_chunks, tiled, static_cast<float*>(kr_hat));
    }
    MSA_LAUNCH_CHECK();
  }
  if (tiled && n_chunks % 16 != 0) {   // the padding chunks of the last tiled group are zero
    const int64_t n = ((n_chunks + 15) / 16 * 16 - n_chunks) * H * d;
    if (dtype == MSA_BF16)
      hipLaunchKernelGGL(zero_pad_tiled_kernel<uint16_t>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, n_chunks, H,
                         d, static_cast<uint16_t*>(kr_hat));
    else
      hipLaunchKernelGGL(zero_pad_tiled_kernel<float>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, n_chunks, H,
                         d, static_cast<float*>(kr_hat));
    MSA_LAUNCH_CHECK();
  }
  return MSA_OK;
}

}  // namespace msa

extern "C" int msa_encode_pool(int dtype, const void* x, int hidden, int H, int d, const int64_t* tok_off,
                               const int64_t* chunk_off, const int32_t* chunk_doc, int64_t n_docs, int64_t n_tok,
                               int64_t n_chunks, int chunk, void* ws, size_t ws_bytes, void* stream) {
  return msa::encode_pool("msa_encode_pool", dtype, x, hidden, H, d, tok_off, chunk_off, chunk_doc, n_docs, n_tok,
                          n_chunks, chunk, ws, ws_bytes, stream);
}

extern "C" int msa_encode_project(int dtype, const void* w_t, int hidden, int H, int d, int64_t n_chunks,
                                  int kr_layout, void* k_bar, void* v_bar, void* kr_hat, const void* ws,
                                  size_t ws_bytes, void* stream) {
  return msa::encode_project("msa_encode_project", dtype, w_t, hidden, H, d, n_chunks, kr_layout, k_bar, v_bar,
                             kr_hat, const_cast<void*>(ws), ws_bytes, stream);
}

extern "C" int msa_encode(int dtype, const void* x, const void* w_t, int hidden, int H, int d, const int64_t* tok_off,
                          const int64_t* chunk_off, const int32_t* chunk_doc, int64_t n_docs, int64_t n_tok,
                          int64_t n_chunks, int chunk, int kr_layout, void* k_bar, void* v_bar, void* kr_hat, void* ws,
                          size_t ws_bytes, void* stream) {
  using namespace msa;
  MSA_REQUIRE(x && w_t && tok_off && chunk_off && chunk_doc && k_bar && v_bar && kr_hat && ws, MSA_ERR_INVALID_ARG,
              "msa_encode: NULL pointer");
  MSA_REQUIRE(kr_layout == MSA_LAYOUT_ROWS || (kr_layout == MSA_LAYOUT_TILED && d % 32 == 0), MSA_ERR_INVALID_ARG,
              "msa_encode: bad kr_layout");
  MSA_REQUIRE(uintptr_t(w_t) % 16 == 0, MSA_ERR_INVALID_ARG, "msa_encode: x and w_t must be 16-byte aligned");
  const int st = encode_pool("msa_encode", dtype, x, hidden, H, d, tok_off, chunk_off, chunk_doc, n_docs, n_tok,
                             n_chunks, chunk, ws, ws_bytes, stream);
  if (st != MSA_OK) return st;
  return encode_project("msa_encode", dtype, w_t, hidden, H, d, n_chunks, kr_layout, k_bar, v_bar, kr_hat, ws,
                        ws_bytes, stream);
}
