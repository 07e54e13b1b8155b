// Training-time path of the routing: the routing scores with their
// maximiser, the auxiliary routing loss, the routing-score backward and the
// pooling backward.
// (Paper note 核心方法 > 训练: continued pre-training with a generation loss
//  plus an auxiliary supervised contrastive routing loss; README Abstract and
//  Key Contributions: the layer is trainable end to end; README
//  Implementation Notes: auxiliary routing loss.)
//
// Readings (the pages name the loss only):
//  - loss of query b: L_b = -(1/|P_b|) sum_{p in P_b} log softmax_i(s_bi / tau)[p]
//    over every document i, P_b the distinct valid positive ids, tau an input;
//  - the max over tokens and chunks passes its derivative to one maximiser,
//    the smallest chunk index and then the smallest token attaining it;
//  - x / max(||x||, 1e-8) has derivative (I - xh xh^T) / ||x|| (else I / 1e-8);
//  - the store rounding is the identity in the backward.
#include <algorithm>

#include "common.h"

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TR_WAVES = 4;
constexpr int TR_THREADS = 64 * TR_WAVES;
constexpr float TR_EPS = 1e-8f;

__device__ __forceinline__ bf16x8 as_bf16x8_tr(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const int lo = __shfl_xor(int(uint32_t(v)), m), hi = __shfl_xor(int(uint32_t(v >> 32)), m);
  return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}

__global__ void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

// winv[j, h] = 1 / (H * max(||q[j, h]||, eps)), one wave per (j, h); the
// same launch clears the n_zero argmax keys (grid-stride)
template <int DT>
__global__ void qscale_kernel(const typename Elem<DT>::T* __restrict__ q, int64_t JH, int H, int d,
                              float* __restrict__ winv, uint64_t* __restrict__ zero, int64_t n_zero) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_zero; i += int64_t(gridDim.x) * blockDim.x)
    zero[i] = 0;
  const int64_t w = int64_t(blockIdx.x) * TR_WAVES + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (w >= JH) return;
  float ss = 0.f;
  for (int e = lane; e < d; e += 64) {
    const float x = Elem<DT>::load(q + w * d, e);
    ss += x * x;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  if (lane == 0) winv[w] = 1.f / (float(H) * fmaxf(sqrtf(ss), TR_EPS));
}

// A (score, chunk, token) candidate as one 64-bit key whose unsigned order is
// (score ascending, then chunk * T + token descending): the atomic maximum
// keeps the largest score and, among equal scores, the smallest index.
__device__ __forceinline__ uint64_t cand_key(float s, uint32_t idx) {
  return (uint64_t(float_order_key(s)) << 32) | uint64_t(~idx);
}

// ---------------------------------------------------------------- scores with maximiser
// bf16 path: one wave per (16-chunk tile, group of 64 query columns), so that
// long queries and small memories still fill the chip.  Per head, the tile's rows are the
// A operand of v_mfma_f32_16x16x32_bf16 (16 bytes per lane, loaded once per
// head) and the raw bf16 queries the B operand; each head's fp32 result is
// scaled by 1 / (H ||q||) and summed, so products are exact.  The token max
// is taken across the 16 lanes of a column tile when its columns belong to
// one query; chunks of one document in a lane's four rows are merged before
// the atomic maximum.
constexpr int AX_NT = 4;   // 16-column tiles per pass

// KKS > 0 (d = 32 KKS, H even): all operands of a head are requested
// together, the next head's while this one is computed; KKS = 0: any d.
template <int KKS>
__global__ __launch_bounds__(TR_THREADS) void route_argmax_mfma_kernel(
    const uint16_t* __restrict__ q, int T, int J, int H, int d, const uint16_t* __restrict__ kr,
    const int32_t* __restrict__ chunk_doc, int64_t n_docs, int64_t n_chunks, const float* __restrict__ winv,
    int n_cg, uint64_t* __restrict__ keys) {
  const int lane = threadIdx.x % 64, lc = lane % 16, g4 = lane / 16;
  const int64_t wid = int64_t(blockIdx.x) * TR_WAVES + threadIdx.x / 64;
  const int64_t tile = wid / n_cg;
  const int cg = int(wid % n_cg);
  const int64_t c0 = tile * 16;
  if (c0 >= n_chunks) return;
  const int64_t crow = c0 + lc;                       // A-operand row of this lane
  const bool crow_ok = crow < n_chunks;
  const int kks = d / 32;
  int rdoc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t c = c0 + 4 * g4 + i;
    rdoc[i] = c < n_chunks ? chunk_doc[c] : -1;
  }
  {
    const int col0 = cg * 16 * AX_NT;
    f32x4 tot[AX_NT];
#pragma unroll
    for (int n = 0; n < AX_NT; ++n) tot[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (KKS > 0) {
      struct HeadOps {
        uint4 a[KKS];
        uint4 b[KKS][AX_NT];
      };
      auto load_ops = [&](int h, HeadOps& o) {
#pragma unroll
        for (int kk = 0; kk < KKS; ++kk) {
          o.a[kk] = crow_ok ? *reinterpret_cast<const uint4*>(kr + (crow * H + h) * d + 32 * kk + 8 * g4)
                            : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int n = 0; n < AX_NT; ++n) {
            const int col = col0 + 16 * n + lc;
            o.b[kk][n] = col < J ? *reinterpret_cast<const uint4*>(q + (int64_t(col) * H + h) * d + 32 * kk + 8 * g4)
                                 : make_uint4(0, 0, 0, 0);
          }
        }
      };
      auto compute = [&](int h, const HeadOps& o) {
        f32x4 acc[AX_NT];
#pragma unroll
        for (int n = 0; n < AX_NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KKS; ++kk)
#pragma unroll
          for (int n = 0; n < AX_NT; ++n)
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_tr(o.a[kk]), as_bf16x8_tr(o.b[kk][n]), acc[n],
                                                              0, 0, 0);
#pragma unroll
        for (int n = 0; n < AX_NT; ++n) {
          const int col = col0 + 16 * n + lc;
          const float wv = col < J ? winv[int64_t(col) * H + h] : 0.f;
          tot[n] += wv * acc[n];
        }
      };
      // heads in pairs; the request after the last pair repeats the last head
      // (in bounds, never used), so no branch sits around the loads
      HeadOps o0, o1;
      load_ops(0, o0);
      for (int h = 0; h < H; h += 2) {
        load_ops(h + 1, o1);
        compute(h, o0);
        load_ops(min(h + 2, H - 1), o0);
        compute(h + 1, o1);
      }
    } else {
      for (int h = 0; h < H; ++h) {
        f32x4 acc[AX_NT];
#pragma unroll
        for (int n = 0; n < AX_NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < kks; ++kk) {
          const uint4 a = crow_ok ? *reinterpret_cast<const uint4*>(kr + (crow * H + h) * d + 32 * kk + 8 * g4)
                                  : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int n = 0; n < AX_NT; ++n) {
            const int col = col0 + 16 * n + lc;
            const uint4 bq = col < J ? *reinterpret_cast<const uint4*>(q + (int64_t(col) * H + h) * d + 32 * kk + 8 * g4)
                                     : make_uint4(0, 0, 0, 0);
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_tr(a), as_bf16x8_tr(bq), acc[n], 0, 0, 0);
          }
        }
#pragma unroll
        for (int n = 0; n < AX_NT; ++n) {
          const int col = col0 + 16 * n + lc;
          const float wv = col < J ? winv[int64_t(col) * H + h] : 0.f;
          tot[n] += wv * acc[n];
        }
      }
    }
    // merge rows of one document in a lane's four rows, then one atomic maximum per run
    auto emit = [&](const uint64_t (&key)[4], int b) {
      uint64_t run = key[0];
      int run_doc = rdoc[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        if (rdoc[i] == run_doc) {
          run = key[i] > run ? key[i] : run;
        } else {
          if (run_doc >= 0 && run_doc < n_docs)
            atomicMax(reinterpret_cast<unsigned long long*>(keys + int64_t(b) * n_docs + run_doc),
                      (unsigned long long)run);
          run = key[i];
          run_doc = rdoc[i];
        }
      }
      if (run_doc >= 0 && run_doc < n_docs)
        atomicMax(reinterpret_cast<unsigned long long*>(keys + int64_t(b) * n_docs + run_doc), (unsigned long long)run);
    };
    // all of the wave's columns are tokens of one query: the token maximum
    // over the whole group in registers, then one set of atomics
    const int col_last = col0 + 16 * AX_NT - 1;
    if (col_last < J && col0 / T == col_last / T) {
      uint64_t key[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t c = c0 + 4 * g4 + i;
        uint64_t kmax = 0;
#pragma unroll
        for (int n = 0; n < AX_NT; ++n) {
          const int t = (col0 + 16 * n + lc) % T;
          const uint64_t kn = rdoc[i] >= 0 ? cand_key(tot[n][i], uint32_t(c * T + t)) : 0;
          kmax = kn > kmax ? kn : kmax;
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
          const uint64_t o = shfl_xor_u64(kmax, m);
          kmax = o > kmax ? o : kmax;
        }
        key[i] = kmax;
      }
      // the workgroup's four waves share the chunk tile (n_cg % TR_WAVES == 0)
      // and their 256 columns one query: merge the waves through LDS first
      const int wcol0 = (cg - cg % TR_WAVES) * 16 * AX_NT, wcol_last = wcol0 + TR_WAVES * 16 * AX_NT - 1;
      if (n_cg % TR_WAVES == 0 && wcol_last < J && wcol0 / T == wcol_last / T) {
        __shared__ uint64_t wk[TR_WAVES][16];
        const int wave = threadIdx.x / 64;
        if (lc == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) wk[wave][4 * g4 + i] = key[i];
        }
        __syncthreads();
        if (wave == 0 && lc == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int w = 1; w < TR_WAVES; ++w) key[i] = wk[w][4 * g4 + i] > key[i] ? wk[w][4 * g4 + i] : key[i];
          }
          emit(key, col0 / T);
        }
        return;
      }
      if (lc == 0) emit(key, col0 / T);
      return;
    }
#pragma unroll
    for (int n = 0; n < AX_NT; ++n) {
      const int cbase = col0 + 16 * n;
      if (cbase >= J) break;
      const int col = cbase + lc;
      const bool col_ok = col < J;
      const int t = col % T, b = col / T;
      uint64_t key[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t c = c0 + 4 * g4 + i;
        key[i] = (col_ok && rdoc[i] >= 0) ? cand_key(tot[n][i], uint32_t(c * T + t)) : 0;
      }
      // the 16 columns of this tile belong to one query: max across them
      const bool one_query = cbase / T == min(cbase + 15, J - 1) / T && cbase + 15 < J;
      if (one_query) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int m = 1; m < 16; m <<= 1) {
            const uint64_t o = shfl_xor_u64(key[i], m);
            key[i] = o > key[i] ? o : key[i];
          }
        }
      }
      if (!col_ok || (one_query && lc != 0)) continue;
      emit(key, b);
    }
  }
}

// bf16, d = 128, the queries staged in LDS: workgroup = (group of 64 query
// columns, four 16-chunk tiles), one tile per wave.  The column group's
// operands of every head (H x 16 KB, in fragment order) and its 1/(H ||q||)
// scales are staged once per workgroup, so each query fragment is read from
// L2 once per four tiles instead of once per tile; the tile's rows stream
// from global memory one head ahead.  Products, the per-head scaling and the
// keys are those of route_argmax_mfma_kernel, so the maxima are identical.
__device__ __forceinline__ void argmax_emit(const f32x4 (&tot)[AX_NT], int64_t c0, int col0, int T, int J,
                                            const int (&rdoc)[4], int64_t n_docs, uint64_t* __restrict__ keys,
                                            int lc, int g4) {
  // merge rows of one document in a lane's four rows, then one atomic maximum per run
  auto emit = [&](const uint64_t (&key)[4], int b) {
    uint64_t run = key[0];
    int run_doc = rdoc[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      if (rdoc[i] == run_doc) {
        run = key[i] > run ? key[i] : run;
      } else {
        if (run_doc >= 0 && run_doc < n_docs)
          atomicMax(reinterpret_cast<unsigned long long*>(keys + int64_t(b) * n_docs + run_doc), (unsigned long long)run);
        run = key[i];
        run_doc = rdoc[i];
      }
    }
    if (run_doc >= 0 && run_doc < n_docs)
      atomicMax(reinterpret_cast<unsigned long long*>(keys + int64_t(b) * n_docs + run_doc), (unsigned long long)run);
  };
  const int col_last = col0 + 16 * AX_NT - 1;
  if (col_last < J && col0 / T == col_last / T) {   // all 64 columns are tokens of one query
    uint64_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t c = c0 + 4 * g4 + i;
      uint64_t kmax = 0;
#pragma unroll
      for (int n = 0; n < AX_NT; ++n) {
        const int t = (col0 + 16 * n + lc) % T;
        const uint64_t kn = rdoc[i] >= 0 ? cand_key(tot[n][i], uint32_t(c * T + t)) : 0;
        kmax = kn > kmax ? kn : kmax;
      }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        const uint64_t o = shfl_xor_u64(kmax, m);
        kmax = o > kmax ? o : kmax;
      }
      key[i] = kmax;
    }
    if (lc == 0) emit(key, col0 / T);
    return;
  }
#pragma unroll
  for (int n = 0; n < AX_NT; ++n) {
    const int cbase = col0 + 16 * n;
    if (cbase >= J) break;
    const int col = cbase + lc;
    const bool col_ok = col < J;
    const int t = col % T, b = col / T;
    uint64_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t c = c0 + 4 * g4 + i;
      key[i] = (col_ok && rdoc[i] >= 0) ? cand_key(tot[n][i], uint32_t(c * T + t)) : 0;
    }
    const bool one_query = cbase / T == min(cbase + 15, J - 1) / T && cbase + 15 < J;
    if (one_query) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
          const uint64_t o = shfl_xor_u64(key[i], m);
          key[i] = o > key[i] ? o : key[i];
        }
      }
    }
    if (!col_ok || (one_query && lc != 0)) continue;
    emit(key, b);
  }
}

constexpr int AX_D = 128;
constexpr int AX_KK = AX_D / 32;

__global__ __launch_bounds__(TR_THREADS) void route_argmax_lds_kernel(
    const uint16_t* __restrict__ q, int T, int J, int H, const uint16_t* __restrict__ kr,
    const int32_t* __restrict__ chunk_doc, int64_t n_docs, int64_t n_chunks, const float* __restrict__ winv,
    int n_cg, uint64_t* __restrict__ keys) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint4* qf = reinterpret_cast<uint4*>(smem);                                     // [H][KK][NT][64 lanes]
  float* wl = reinterpret_cast<float*>(smem + size_t(H) * AX_KK * AX_NT * 1024);  // [H][NT][16]
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, lc = lane % 16, g4 = lane / 16;
  const int cg = int(blockIdx.x % n_cg);
  const int64_t tile = int64_t(blockIdx.x / n_cg) * TR_WAVES + wave;
  const int col0 = cg * 16 * AX_NT;
  // ---- stage the column group's query fragments and scales (every thread takes part)
  const int n_pieces = H * AX_KK * AX_NT * 64;
  for (int p = threadIdx.x; p < n_pieces; p += TR_THREADS) {
    const int l = p % 64, f = p / 64;
    const int n = f % AX_NT, kk = (f / AX_NT) % AX_KK, h = f / (AX_NT * AX_KK);
    const int col = col0 + 16 * n + (l % 16);
    qf[p] = col < J ? *reinterpret_cast<const uint4*>(q + (int64_t(col) * H + h) * AX_D + 32 * kk + 8 * (l / 16))
                    : make_uint4(0, 0, 0, 0);
  }
  for (int p = threadIdx.x; p < H * AX_NT * 16; p += TR_THREADS) {
    const int c16 = p % 16, n = (p / 16) % AX_NT, h = p / (16 * AX_NT);
    const int col = col0 + 16 * n + c16;
    wl[p] = col < J ? winv[int64_t(col) * H + h] : 0.f;
  }
  __syncthreads();
  const int64_t c0 = tile * 16;
  if (c0 >= n_chunks) return;   // after the barrier: this wave has no tile
  const int64_t crow = c0 + lc;
  const bool crow_ok = crow < n_chunks;
  int rdoc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t c = c0 + 4 * g4 + i;
    rdoc[i] = c < n_chunks ? chunk_doc[c] : -1;
  }
  f32x4 tot[AX_NT];
#pragma unroll
  for (int n = 0; n < AX_NT; ++n) tot[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load_a = [&](int h, uint4 (&a)[AX_KK]) {
#pragma unroll
    for (int kk = 0; kk < AX_KK; ++kk)
      a[kk] = crow_ok ? *reinterpret_cast<const uint4*>(kr + (crow * H + h) * AX_D + 32 * kk + 8 * g4)
                      : make_uint4(0, 0, 0, 0);
  };
  auto compute = [&](int h, const uint4 (&a)[AX_KK]) {
    f32x4 acc[AX_NT];
#pragma unroll
    for (int n = 0; n < AX_NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < AX_KK; ++kk)
#pragma unroll
      for (int n = 0; n < AX_NT; ++n)
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_tr(a[kk]),
                                                          as_bf16x8_tr(qf[((h * AX_KK + kk) * AX_NT + n) * 64 + lane]),
                                                          acc[n], 0, 0, 0);
#pragma unroll
    for (int n = 0; n < AX_NT; ++n) tot[n] += wl[(h * AX_NT + n) * 16 + lc] * acc[n];
  };
  // heads in pairs, the next head's rows loading while one is computed; the
  // request after the last head repeats it (in bounds, never used)
  uint4 a0[AX_KK], a1[AX_KK];
  load_a(0, a0);
  for (int h = 0; h < H; h += 2) {
    load_a(h + 1, a1);
    compute(h, a0);
    load_a(min(h + 2, H - 1), a0);
    compute(h + 1, a1);
  }
  argmax_emit(tot, c0, col0, T, J, rdoc, n_docs, keys, lc, g4);
}

// float32 (or any head size) path: one thread per (chunk, column)
template <int DT>
__global__ void route_argmax_vec_kernel(const typename Elem<DT>::T* __restrict__ q, int T, int J, int H, int d,
                                        const typename Elem<DT>::T* __restrict__ kr,
                                        const int32_t* __restrict__ chunk_doc, int64_t n_docs, int64_t n_chunks,
                                        const float* __restrict__ winv, uint64_t* __restrict__ keys) {
  const int64_t p = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p >= n_chunks * J) return;
  const int64_t c = p / J;
  const int j = int(p % J);
  const int doc = chunk_doc[c];
  if (doc < 0 || doc >= n_docs) return;
  float s = 0.f;
  for (int h = 0; h < H; ++h) {
    float dot = 0.f;
    for (int e = 0; e < d; ++e)
      dot += Elem<DT>::load(q + (int64_t(j) * H + h) * d, e) * Elem<DT>::load(kr + (c * H + h) * d, e);
    s += winv[int64_t(j) * H + h] * dot;
  }
  atomicMax(reinterpret_cast<unsigned long long*>(keys + int64_t(j / T) * n_docs + doc),
            (unsigned long long)cand_key(s, uint32_t(c * T + j % T)));
}

__global__ void argmax_unpack_kernel(const uint64_t* __restrict__ keys, int64_t n, int T, float* __restrict__ score,
                                     int32_t* __restrict__ arg_chunk, int32_t* __restrict__ arg_tok) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint64_t k = keys[i];
  if (k == 0) {   // a document with no chunk
    score[i] = -INFINITY;
    arg_chunk[i] = -1;
    arg_tok[i] = -1;
    return;
  }
  const uint32_t idx = ~uint32_t(k);
  score[i] = order_key_float(uint32_t(k >> 32));
  arg_chunk[i] = int32_t(idx / uint32_t(T));
  arg_tok[i] = int32_t(idx % uint32_t(T));
}

// ---------------------------------------------------------------- routing loss
// One workgroup per query: the max and the log-sum-exp of s / tau over the
// documents (an empty document's -inf, or a NaN, carries no weight), the loss
// over the distinct valid positives, and grad = (softmax - [i in P] / |P|) / tau.
__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
  const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float o = __shfl_xor(v, m);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < TR_WAVES; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

__global__ __launch_bounds__(TR_THREADS) void route_loss_kernel(const float* __restrict__ s, int64_t D,
                                                                 const int32_t* __restrict__ pos, int P, float tau,
                                                                 float* __restrict__ loss, float* __restrict__ grad) {
  __shared__ float red[TR_WAVES];
  __shared__ float pz[2];
  const int b = blockIdx.x;
  const float* row = s + int64_t(b) * D;
  float* grow = grad + int64_t(b) * D;
  const float inv_tau = 1.f / tau;
  float m = -INFINITY;
  for (int64_t i = threadIdx.x; i < D; i += TR_THREADS) {
    const float z = row[i] * inv_tau;
    m = z > m ? z : m;   // NaN never wins
  }
  m = block_reduce(m, true, red);
  const float mu = m == -INFINITY ? 0.f : m;
  float acc = 0.f;
  for (int64_t i = threadIdx.x; i < D; i += TR_THREADS) {
    const float z = row[i] * inv_tau;
    acc += (z > -INFINITY) ? __expf(z - mu) : 0.f;
  }
  acc = block_reduce(acc, false, red);
  const float lse = mu + __logf(acc);
  if (threadIdx.x == 0) {
    int np = 0;
    float zs = 0.f;
    for (int k = 0; k < P; ++k) {
      const int p = pos[int64_t(b) * P + k];
      if (p < 0 || p >= D) continue;
      bool dup = false;
      for (int k2 = 0; k2 < k; ++k2) dup |= pos[int64_t(b) * P + k2] == p;
      if (dup) continue;
      ++np;
      zs += row[p] * inv_tau;
    }
    pz[0] = float(np);
    loss[b] = np > 0 ? lse - zs / float(np) : __builtin_nanf("");
  }
  for (int64_t i = threadIdx.x; i < D; i += TR_THREADS) {
    const float z = row[i] * inv_tau;
    grow[i] = (z > -INFINITY) ? __expf(z - lse) * inv_tau : 0.f;
  }
  __syncthreads();
  const float np = pz[0];
  for (int k = threadIdx.x; k < P; k += TR_THREADS) {
    const int p = pos[int64_t(b) * P + k];
    if (p < 0 || p >= D || np == 0.f) continue;
    bool dup = false;
    for (int k2 = 0; k2 < k; ++k2) dup |= pos[int64_t(b) * P + k2] == p;
    if (!dup) grow[p] -= inv_tau / np;
  }
}

// ---------------------------------------------------------------- routing-score backward
// One wave per (query, document, head): the score's derivative reaches the
// maximiser only, dqhat[b, t*] += g/H * kr[c*] and dkr[c*] += g/H * qhat[b, t*]
// (float atomics: several documents share a token, several queries a chunk).
template <int DT>
__global__ __launch_bounds__(TR_THREADS) void route_bwd_scatter_kernel(
    const typename Elem<DT>::T* __restrict__ q, int T, int H, int d, const typename Elem<DT>::T* __restrict__ kr,
    int64_t n_chunks, const int32_t* __restrict__ arg_chunk, const int32_t* __restrict__ arg_tok,
    const float* __restrict__ grad, int64_t n_items, int64_t n_docs, float* __restrict__ dqh,
    float* __restrict__ dkr) {
  const int64_t wv = int64_t(blockIdx.x) * TR_WAVES + threadIdx.x / 64;
  const int64_t it = wv / H;
  const int h = int(wv % H);
  const int lane = threadIdx.x % 64;
  if (it >= n_items) return;
  const int64_t b = it / n_docs;
  const int c = arg_chunk[it], t = arg_tok[it];
  const float g = grad[it];
  if (c < 0 || c >= n_chunks || t < 0 || t >= T || g == 0.f) return;
  const float w = g / float(H);
  {
    const typename Elem<DT>::T* qp = q + ((b * T + t) * H + h) * d;
    const typename Elem<DT>::T* kp = kr + (int64_t(c) * H + h) * d;
    float ss = 0.f;
    for (int e = lane; e < d; e += 64) {
      const float x = Elem<DT>::load(qp, e);
      ss += x * x;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    const float inv = 1.f / fmaxf(sqrtf(ss), TR_EPS);
    float* dq = dqh + ((b * T + t) * H + h) * d;
    float* dk = dkr + (int64_t(c) * H + h) * d;
    for (int e = lane; e < d; e += 64) {
      unsafeAtomicAdd(dq + e, w * Elem<DT>::load(kp, e));
      unsafeAtomicAdd(dk + e, w * Elem<DT>::load(qp, e) * inv);
    }
  }
}

// In place: dq = (dqh - qh (qh . dqh)) / ||q||, or dqh / eps below eps; one
// wave per (query row, head)
template <int DT>
__global__ __launch_bounds__(TR_THREADS) void normalize_bwd_kernel(const typename Elem<DT>::T* __restrict__ q,
                                                                   int64_t rows, int d, float* __restrict__ dq) {
  const int64_t r = int64_t(blockIdx.x) * TR_WAVES + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (r >= rows) return;
  const typename Elem<DT>::T* qp = q + r * d;
  float* dp = dq + r * d;
  float ss = 0.f, dot = 0.f;
  for (int e = lane; e < d; e += 64) {
    const float x = Elem<DT>::load(qp, e);
    ss += x * x;
    dot += x * dp[e];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    ss += __shfl_xor(ss, m);
    dot += __shfl_xor(dot, m);
  }
  const float n = sqrtf(ss);
  if (n > TR_EPS) {
    const float inv = 1.f / n, c = dot * inv * inv;   // qh . dqh = dot / n
    for (int e = lane; e < d; e += 64) dp[e] = (dp[e] - Elem<DT>::load(qp, e) * c) * inv;
  } else {
    for (int e = lane; e < d; e += 64) dp[e] = dp[e] * (1.f / TR_EPS);
  }
}

// ---------------------------------------------------------------- pooling backward
// One wave per (pooled chunk, head): dx[tau] = dm / n for the n tokens of
// the chunk, dm = dy, or, for an L2-normalised entry, dy carried back
// through the normalisation of the chunk mean (recomputed in float32).
constexpr int PB_MAXE = 4;   // d <= 256

template <int DT>
__global__ __launch_bounds__(TR_THREADS) void pool_bwd_kernel(
    const float* __restrict__ dy, int64_t n_chunks, int H, int d, const int64_t* __restrict__ tok_off,
    const int64_t* __restrict__ chunk_off, const int32_t* __restrict__ chunk_doc, int64_t n_docs, int chunk,
    const typename Elem<DT>::T* __restrict__ x, float* __restrict__ dx) {
  const int64_t w = int64_t(blockIdx.x) * TR_WAVES + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (w >= n_chunks * H) return;
  const int64_t c = w / H;
  const int h = int(w % H);
  const int doc = chunk_doc[c];
  if (doc < 0 || doc >= n_docs) return;
  const int64_t t0 = tok_off[doc] + (c - chunk_off[doc]) * int64_t(chunk);
  const int64_t n = min(int64_t(chunk), tok_off[doc + 1] - t0);
  if (n <= 0) return;
  float dm[PB_MAXE];
#pragma unroll
  for (int k = 0; k < PB_MAXE; ++k) {
    const int e = lane + 64 * k;
    dm[k] = e < d ? dy[(c * H + h) * d + e] : 0.f;
  }
  if (x) {
    float mean[PB_MAXE];
#pragma unroll
    for (int k = 0; k < PB_MAXE; ++k) mean[k] = 0.f;
    for (int64_t tau = t0; tau < t0 + n; ++tau) {
#pragma unroll
      for (int k = 0; k < PB_MAXE; ++k) {
        const int e = lane + 64 * k;
        if (e < d) mean[k] += Elem<DT>::load(x + (tau * H + h) * d, e);
      }
    }
    float ss = 0.f, dot = 0.f;
#pragma unroll
    for (int k = 0; k < PB_MAXE; ++k) {
      mean[k] /= float(n);
      ss += mean[k] * mean[k];
      dot += mean[k] * dm[k];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      ss += __shfl_xor(ss, m);
      dot += __shfl_xor(dot, m);
    }
    const float nrm = sqrtf(ss);
    if (nrm > TR_EPS) {
      const float inv = 1.f / nrm, cc = dot * inv * inv;
#pragma unroll
      for (int k = 0; k < PB_MAXE; ++k) dm[k] = (dm[k] - mean[k] * cc) * inv;
    } else {
#pragma unroll
      for (int k = 0; k < PB_MAXE; ++k) dm[k] *= 1.f / TR_EPS;
    }
  }
  const float inv_n = 1.f / float(n);
  for (int64_t tau = t0; tau < t0 + n; ++tau) {
#pragma unroll
    for (int k = 0; k < PB_MAXE; ++k) {
      const int e = lane + 64 * k;
      if (e < d) dx[(tau * H + h) * d + e] = dm[k] * inv_n;
    }
  }
}

// Row path: one workgroup per pooled chunk, H*d/4 threads, thread q owning
// elements 4q..4q+3 of a token row (head q / (d/4)); every token of the
// chunk is written as whole contiguous rows.  Per-head sums reduce across
// the d/4 lanes of the head.
template <int DT>
__global__ void pool_bwd_rows_kernel(const float* __restrict__ dy, int64_t n_chunks, int H, int d,
                                     const int64_t* __restrict__ tok_off, const int64_t* __restrict__ chunk_off,
                                     const int32_t* __restrict__ chunk_doc, int64_t n_docs, int chunk,
                                     const typename Elem<DT>::T* __restrict__ x, float* __restrict__ dx) {
  const int64_t c = blockIdx.x;
  const int qd = threadIdx.x, HD = H * d, lanes = d / 4;
  const int doc = chunk_doc[c];
  if (doc < 0 || doc >= n_docs) return;
  const int64_t t0 = tok_off[doc] + (c - chunk_off[doc]) * int64_t(chunk);
  const int64_t n = min(int64_t(chunk), tok_off[doc + 1] - t0);
  if (n <= 0) return;
  float4 dm = *reinterpret_cast<const float4*>(dy + c * HD + 4 * qd);
  if (x) {
    float4 mean = make_float4(0.f, 0.f, 0.f, 0.f);
    // the token loads are independent: unrolled, eight are in flight
#pragma unroll 8
    for (int64_t tau = t0; tau < t0 + n; ++tau) {
      const typename Elem<DT>::T* xp = x + tau * HD + 4 * qd;
      if constexpr (DT == MSA_BF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(xp);   // four bf16 in one 8-byte load
        mean.x += __uint_as_float(u.x << 16);
        mean.y += __uint_as_float(u.x & 0xFFFF0000u);
        mean.z += __uint_as_float(u.y << 16);
        mean.w += __uint_as_float(u.y & 0xFFFF0000u);
      } else {
        mean.x += Elem<DT>::load(xp, 0);
        mean.y += Elem<DT>::load(xp, 1);
        mean.z += Elem<DT>::load(xp, 2);
        mean.w += Elem<DT>::load(xp, 3);
      }
    }
    const float inv_n = 1.f / float(n);
    mean = mean * inv_n;
    float ss = mean.x * mean.x + mean.y * mean.y + mean.z * mean.z + mean.w * mean.w;
    float dot = mean.x * dm.x + mean.y * dm.y + mean.z * dm.z + mean.w * dm.w;
    for (int m = 1; m < lanes; m <<= 1) {   // the lanes of one head are an aligned power-of-two group
      ss += __shfl_xor(ss, m);
      dot += __shfl_xor(dot, m);
    }
    const float nrm = sqrtf(ss);
    if (nrm > TR_EPS) {
      const float inv = 1.f / nrm, cc = dot * inv * inv;
      dm = (dm - mean * cc) * inv;
    } else {
      dm = dm * (1.f / TR_EPS);
    }
  }
  dm = dm * (1.f / float(n));
  for (int64_t tau = t0; tau < t0 + n; ++tau) *reinterpret_cast<float4*>(dx + tau * HD + 4 * qd) = dm;
}

static bool pool_bwd_rows(int H, int d) {
  const int lanes = d / 4;
  return d % 4 == 0 && lanes >= 1 && lanes <= 64 && (lanes & (lanes - 1)) == 0 && H * d / 4 <= 1024 &&
         (H * d / 4) % 64 == 0;
}

static bool argmax_mfma(int dtype, int d) { return dtype == MSA_BF16 && d % 32 == 0; }

static unsigned grid_for(int64_t n, int64_t per_block) {
  return unsigned(std::min<int64_t>((n + per_block - 1) / per_block, 1 << 30));
}

}  // namespace msa

extern "C" size_t msa_route_argmax_workspace(int dtype, int B, int T, int H, int d, int64_t n_docs,
                                             int64_t n_chunks) {
  (void)dtype;
  (void)d;
  (void)n_chunks;
  if (B < 1 || T < 1 || H < 1 || n_docs < 1) return 0;
  return msa::align_up(size_t(B) * size_t(n_docs) * 8, 256) + msa::align_up(size_t(B) * T * H * 4, 256);
}

extern "C" int msa_route_argmax(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat,
                                const int32_t* chunk_doc, int64_t n_docs, int64_t n_chunks, float* doc_score,
                                int32_t* arg_chunk, int32_t* arg_tok, void* ws, size_t ws_bytes, void* stream) {
  using namespace msa;
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, "msa_route_argmax: bad dtype");
  MSA_REQUIRE(q_r && kr_hat && chunk_doc && doc_score && arg_chunk && arg_tok && ws, MSA_ERR_INVALID_ARG,
              "msa_route_argmax: NULL pointer");
  MSA_REQUIRE(B >= 1 && T >= 1 && H >= 1 && d >= 1 && n_docs >= 1 && n_chunks >= 1, MSA_ERR_INVALID_ARG,
              "msa_route_argmax: non-positive size");
  MSA_REQUIRE(int64_t(B) * T < (int64_t(1) << 24), MSA_ERR_UNSUPPORTED, "msa_route_argmax: B*T too large");
  MSA_REQUIRE(n_chunks * T < (int64_t(1) << 32) - 1, MSA_ERR_UNSUPPORTED,
              "msa_route_argmax: n_chunks * T must be below 2^32");
  MSA_REQUIRE(d <= 256, MSA_ERR_UNSUPPORTED, "msa_route_argmax: d > 256");
  const size_t need = msa_route_argmax_workspace(dtype, B, T, H, d, n_docs, n_chunks);
  MSA_REQUIRE(ws_bytes >= need, MSA_ERR_WORKSPACE, "msa_route_argmax: workspace too small");
  MSA_REQUIRE(uintptr_t(q_r) % 16 == 0 && uintptr_t(kr_hat) % 16 == 0, MSA_ERR_INVALID_ARG,
              "msa_route_argmax: q_r and kr_hat must be 16-byte aligned");
  hipStream_t s = as_stream(stream);
  const int J = B * T;
  const int64_t nkey = int64_t(B) * n_docs;
  uint64_t* keys = static_cast<uint64_t*>(ws);
  float* winv = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(size_t(nkey) * 8, 256));
  const int64_t JH = int64_t(J) * H;
  if (dtype == MSA_BF16)
    hipLaunchKernelGGL(qscale_kernel<MSA_BF16>, dim3(grid_for(JH, TR_WAVES)), dim3(TR_THREADS), 0, s,
                       static_cast<const uint16_t*>(q_r), JH, H, d, winv, keys, nkey);
  else
    hipLaunchKernelGGL(qscale_kernel<MSA_F32>, dim3(grid_for(JH, TR_WAVES)), dim3(TR_THREADS), 0, s,
                       static_cast<const float*>(q_r), JH, H, d, winv, keys, nkey);
  MSA_LAUNCH_CHECK();
  if (argmax_mfma(dtype, d)) {
    const int64_t tiles = (n_chunks + 15) / 16;
    const int n_cg = (J + 16 * AX_NT - 1) / (16 * AX_NT);
    int lds_max = 0, dev = 0;
    MSA_HIP_CHECK(hipGetDevice(&dev));
    MSA_HIP_CHECK(hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
    const size_t lsmem = size_t(H) * AX_KK * AX_NT * 1024 + size_t(H) * AX_NT * 16 * sizeof(float);
    const int64_t groups = (tiles + TR_WAVES - 1) / TR_WAVES;
    if (d == AX_D && H % 2 == 0 && lsmem <= size_t(lds_max) && groups * n_cg < (int64_t(1) << 31)) {
      // the column group's queries staged once per four tiles
      MSA_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&route_argmax_lds_kernel),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, int(lsmem)));
      hipLaunchKernelGGL(route_argmax_lds_kernel, dim3(unsigned(groups * n_cg)), dim3(TR_THREADS), lsmem, s,
                         static_cast<const uint16_t*>(q_r), T, J, H, static_cast<const uint16_t*>(kr_hat), chunk_doc,
                         n_docs, n_chunks, winv, n_cg, keys);
    } else if (d == 128 && H % 2 == 0)
      hipLaunchKernelGGL(route_argmax_mfma_kernel<4>, dim3(grid_for(tiles * n_cg, TR_WAVES)), dim3(TR_THREADS), 0, s,
                         static_cast<const uint16_t*>(q_r), T, J, H, d, static_cast<const uint16_t*>(kr_hat),
                         chunk_doc, n_docs, n_chunks, winv, n_cg, keys);
    else
      hipLaunchKernelGGL(route_argmax_mfma_kernel<0>, dim3(grid_for(tiles * n_cg, TR_WAVES)), dim3(TR_THREADS), 0, s,
                         static_cast<const uint16_t*>(q_r), T, J, H, d, static_cast<const uint16_t*>(kr_hat),
                         chunk_doc, n_docs, n_chunks, winv, n_cg, keys);
  } else if (dtype == MSA_BF16) {
    hipLaunchKernelGGL(route_argmax_vec_kernel<MSA_BF16>, dim3(grid_for(n_chunks * J, 256)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q_r), T, J, H, d, static_cast<const uint16_t*>(kr_hat),
                       chunk_doc, n_docs, n_chunks, winv, keys);
  } else {
    hipLaunchKernelGGL(route_argmax_vec_kernel<MSA_F32>, dim3(grid_for(n_chunks * J, 256)), dim3(256), 0, s,
                       static_cast<const float*>(q_r), T, J, H, d, static_cast<const float*>(kr_hat), chunk_doc,
                       n_docs, n_chunks, winv, keys);
  }
  MSA_LAUNCH_CHECK();
  hipLaunchKernelGGL(argmax_unpack_kernel, dim3(grid_for(nkey, 256)), dim3(256), 0, s, keys, nkey, T, doc_score,
                     arg_chunk, arg_tok);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

extern "C" int msa_route_loss(const float* doc_score, int B, int64_t n_docs, const int32_t* pos_ids, int n_pos,
                              float tau, float* loss, float* grad, void* stream) {
  using namespace msa;
  MSA_REQUIRE(doc_score && pos_ids && loss && grad, MSA_ERR_INVALID_ARG, "msa_route_loss: NULL pointer");
  MSA_REQUIRE(B >= 1 && n_docs >= 1 && n_pos >= 1, MSA_ERR_INVALID_ARG, "msa_route_loss: non-positive size");
  MSA_REQUIRE(tau > 0.f, MSA_ERR_INVALID_ARG, "msa_route_loss: tau must be positive");
  MSA_REQUIRE(B <= 65535 && n_pos <= 256, MSA_ERR_UNSUPPORTED, "msa_route_loss: B > 65535 or n_pos > 256");
  hipLaunchKernelGGL(route_loss_kernel, dim3(unsigned(B)), dim3(TR_THREADS), 0, as_stream(stream), doc_score,
                     n_docs, pos_ids, n_pos, tau, loss, grad);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

extern "C" int msa_route_score_backward(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat,
                                        int64_t n_chunks, const int32_t* arg_chunk, const int32_t* arg_tok,
                                        const float* grad, int64_t n_docs, float* dq_r, float* dkr_hat,
                                        void* stream) {
  using namespace msa;
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, "msa_route_score_backward: bad dtype");
  MSA_REQUIRE(q_r && kr_hat && arg_chunk && arg_tok && grad && dq_r && dkr_hat, MSA_ERR_INVALID_ARG,
              "msa_route_score_backward: NULL pointer");
  MSA_REQUIRE(B >= 1 && T >= 1 && H >= 1 && d >= 1 && n_docs >= 1 && n_chunks >= 1, MSA_ERR_INVALID_ARG,
              "msa_route_score_backward: non-positive size");
  MSA_REQUIRE(n_chunks < (int64_t(1) << 31), MSA_ERR_UNSUPPORTED, "msa_route_score_backward: n_chunks >= 2^31");
  MSA_REQUIRE(int64_t(B) * n_docs * H <= (int64_t(TR_WAVES) << 30), MSA_ERR_UNSUPPORTED,
              "msa_route_score_backward: B * n_docs * H > 2^32");   // one wave per (query, document, head)
  hipStream_t s = as_stream(stream);
  const int64_t nq = int64_t(B) * T * H * d;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_for(nq, 256 * 4)), dim3(256), 0, s, dq_r, nq);
  MSA_LAUNCH_CHECK();
  const int64_t items = int64_t(B) * n_docs;
  const int64_t rows = int64_t(B) * T * H;
  if (dtype == MSA_BF16) {
    hipLaunchKernelGGL(route_bwd_scatter_kernel<MSA_BF16>, dim3(grid_for(items * H, TR_WAVES)), dim3(TR_THREADS), 0, s,
                       static_cast<const uint16_t*>(q_r), T, H, d, static_cast<const uint16_t*>(kr_hat), n_chunks,
                       arg_chunk, arg_tok, grad, items, n_docs, dq_r, dkr_hat);
    MSA_LAUNCH_CHECK();
    hipLaunchKernelGGL(normalize_bwd_kernel<MSA_BF16>, dim3(grid_for(rows, TR_WAVES)), dim3(TR_THREADS), 0, s,
                       static_cast<const uint16_t*>(q_r), rows, d, dq_r);
  } else {
    hipLaunchKernelGGL(route_bwd_scatter_kernel<MSA_F32>, dim3(grid_for(items * H, TR_WAVES)), dim3(TR_THREADS), 0, s,
                       static_cast<const float*>(q_r), T, H, d, static_cast<const float*>(kr_hat), n_chunks,
                       arg_chunk, arg_tok, grad, items, n_docs, dq_r, dkr_hat);
    MSA_LAUNCH_CHECK();
    hipLaunchKernelGGL(normalize_bwd_kernel<MSA_F32>, dim3(grid_for(rows, TR_WAVES)), dim3(TR_THREADS), 0, s,
                       static_cast<const float*>(q_r), rows, d, dq_r);
  }
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

extern "C" int msa_pool_backward(int dtype, const float* dy, const int64_t* tok_off, const int64_t* chunk_off,
                                 const int32_t* chunk_doc, int64_t n_docs, int64_t n_tok, int64_t n_chunks, int H,
                                 int d, int chunk, const void* x, float* dx, void* stream) {
  using namespace msa;
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, "msa_pool_backward: bad dtype");
  MSA_REQUIRE(dy && tok_off && chunk_off && chunk_doc && dx, MSA_ERR_INVALID_ARG, "msa_pool_backward: NULL pointer");
  MSA_REQUIRE(n_docs >= 1 && n_tok >= 1 && n_chunks >= 1 && H >= 1 && d >= 1 && chunk >= 1, MSA_ERR_INVALID_ARG,
              "msa_pool_backward: non-positive size");
  MSA_REQUIRE(d <= 64 * PB_MAXE, MSA_ERR_UNSUPPORTED, "msa_pool_backward: d > 256");
  hipStream_t s = as_stream(stream);
  if (pool_bwd_rows(H, d) && uintptr_t(dy) % 16 == 0 && uintptr_t(dx) % 16 == 0 && uintptr_t(x) % 8 == 0 &&
      n_chunks < (int64_t(1) << 31)) {
    const dim3 grid{unsigned(n_chunks)}, block{unsigned(H * d / 4)};
    if (dtype == MSA_BF16)
      hipLaunchKernelGGL(pool_bwd_rows_kernel<MSA_BF16>, grid, block, 0, s, dy, n_chunks, H, d, tok_off, chunk_off,
                         chunk_doc, n_docs, chunk, static_cast<const uint16_t*>(x), dx);
    else
      hipLaunchKernelGGL(pool_bwd_rows_kernel<MSA_F32>, grid, block, 0, s, dy, n_chunks, H, d, tok_off, chunk_off,
                         chunk_doc, n_docs, chunk, static_cast<const float*>(x), dx);
    MSA_LAUNCH_CHECK();
    return MSA_OK;
  }
  const int64_t waves = n_chunks * H;
  if (dtype == MSA_BF16)
    hipLaunchKernelGGL(pool_bwd_kernel<MSA_BF16>, dim3(grid_for(waves, TR_WAVES)), dim3(TR_THREADS), 0, s, dy,
                       n_chunks, H, d, tok_off, chunk_off, chunk_doc, n_docs, chunk,
                       static_cast<const uint16_t*>(x), dx);
  else
    hipLaunchKernelGGL(pool_bwd_kernel<MSA_F32>, dim3(grid_for(waves, TR_WAVES)), dim3(TR_THREADS), 0, s, dy,
                       n_chunks, H, d, tok_off, chunk_off, chunk_doc, n_docs, chunk, static_cast<const float*>(x),
                       dx);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}
