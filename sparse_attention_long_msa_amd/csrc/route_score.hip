// Stage 2 routing score: cosine of every pooled routing key against the
// routing query, mean over heads, max over query tokens and over the
// document's chunks -> one score per (query, document).
// (MSA README, Overall Design > Architecture: "cosine similarity (mean-pooled
//  over heads, then token-wise max)"; Inference Pipeline, Online Routing;
//  paper note 核心方法 > 架构 and Memory Parallel 推理: the score matrix is tiled
//  rather than materialised.)
//
// MFMA path (bf16, d = 128): the store is streamed exactly once.  Chunks are
// the rows of a v_mfma_f32_16x16x32_bf16 A operand loaded straight from HBM
// (four lanes read 64 contiguous bytes of one chunk per instruction); the
// raw bf16 routing queries are the B operand, staged once per workgroup in
// LDS in fragment order.  Each head is a separate K = 128 contraction whose
// fp32 result is scaled by 1 / (H * ||q[t,h]||) and summed, so the query is
// never rounded after normalisation.  The epilogue takes the token max in
// registers (DPP row reductions) and a segmented max over the tile's chunks
// by document.  Run maxima collect in an LDS table over the documents of the
// workgroup's chunk range; documents inside the range are then stored once,
// and only the range's two boundary documents take an exact ordered global
// atomic max.
#include "common.h"

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int RS_WAVES = 8;
constexpr int RS_THREADS = 64 * RS_WAVES;
constexpr int RS_MT = 1;                 // 16-chunk row tiles per wave tile
constexpr int RS_D = 128;                // head dim of the MFMA path
constexpr int RS_H = 8;                  // heads of the MFMA path
constexpr int RS_KK = RS_D / 32;         // k-steps of 32 per head
constexpr int RS_SCRATCH = 16 * 33 * 4 + 64 * 4;  // per-wave epilogue LDS bytes
static_assert(RS_H % 2 == 0, "heads are processed in pairs");

__global__ void fill_kernel(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

__device__ __forceinline__ float dpp_row_max16(float v) {
  // rotate within each row of 16 lanes by 8, 4, 2, 1: every lane ends with the row max
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xF, 0xF, false)));
  return v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Segmented max over lanes 0..31 (one chunk each) by document id, then one
// emit(doc, max) per run head.  doc < 0 marks a lane with no chunk.
template <class Emit>
__device__ __forceinline__ void seg_max_emit(float v, int doc, int lane, Emit&& emit) {
#pragma unroll
  for (int s = 1; s < 32; s <<= 1) {
    const float w = __shfl_down(v, s, 32);
    const int dd = __shfl_down(doc, s, 32);
    if (lane + s < 32 && dd == doc) v = fmaxf(v, w);
  }
  const int prev = __shfl_up(doc, 1, 32);
  const bool head = (lane < 32) && (lane == 0 || prev != doc);
  if (head && doc >= 0) emit(doc, v);
}

// max of an LDS float through the order-preserving integer image (as atomic_max_float)
__device__ __forceinline__ void lds_max_float(float* addr, float v) {
  if (__float_as_int(v) >= 0)
    atomicMax(reinterpret_cast<int*>(addr), __float_as_int(v));
  else
    atomicMin(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

// NT: 16-column tiles per column group (<= 4); UNIFORM_B: every 16-column
// tile belongs to one query (T % 16 == 0), so the token max is taken in
// registers before the document max.
// D: head loads in flight per wave (the ring)
template <int NT, bool UNIFORM_B, bool TILED, int D>
__global__ __launch_bounds__(RS_THREADS) void route_score_mfma_kernel(
    const uint16_t* __restrict__ q_r, int T, int J, const uint16_t* __restrict__ kr,
    const int32_t* __restrict__ chunk_doc, int64_t n_docs, int64_t n_chunks, float* __restrict__ doc_score,
    int n_groups, int n_ranges, int64_t tiles_per_range, int tab_cap) {
  constexpr int H = RS_H;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint4* qfrag = reinterpret_cast<uint4*>(smem);  // [NT][H][KK][64 lanes] x 16 B
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  float* scratch = reinterpret_cast<float*>(smem + size_t(NT) * H * RS_KK * 1024 + size_t(wave) * RS_SCRATCH);

  // ---- workgroup -> (chunk range, column group); partners of one range sit on one XCD
  int range, group;
  if (n_groups == 1) {
    range = blockIdx.x;
    group = 0;
  } else {
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    group = slot % n_groups;
    range = (slot / n_groups) * 8 + xcd;
  }
  if (range >= n_ranges) return;
  const int col0 = group * 64;

  const int g4 = lane / 16;       // lane group: k-slice of the operands, row block of the result
  const int lc = lane % 16;       // column (query token) of this lane inside a 16-column tile
  constexpr int MT = RS_MT;
  constexpr int TILE = 16 * MT;   // chunks per wave tile
  const int64_t tiles_total = (n_chunks + TILE - 1) / TILE;
  const int64_t t_begin = int64_t(range) * tiles_per_range;
  int64_t t_end = t_begin + tiles_per_range;
  if (t_end > tiles_total) t_end = tiles_total;
  if (t_begin >= t_end) return;             // a range past the last tile (whole workgroup)
  const int64_t rowE = int64_t(H) * RS_D;  // elements per chunk
  int64_t tile = t_begin + wave;

  // Document table: the chunks of the range are contiguous and chunk_doc is
  // non-decreasing, so the range covers documents doc_lo..doc_hi and every
  // document strictly between them lies wholly inside it.  Run maxima go to an
  // LDS table [document][query]; at the end a document wholly inside the range
  // (for a query wholly inside this column group) is stored plainly, only the
  // two boundary documents need global atomics.  Ranges whose table would not
  // fit fall back to one global atomic per run.
  float* tab = reinterpret_cast<float*>(smem + size_t(NT) * H * RS_KK * 1024 + size_t(RS_WAVES) * RS_SCRATCH +
                                        size_t(H) * NT * 16 * 4);
  const int64_t c_last = (t_end * TILE < n_chunks ? t_end * TILE : n_chunks) - 1;
  const int doc_lo = chunk_doc[t_begin * TILE], doc_hi = chunk_doc[c_last];
  const int col_end = col0 + 64 < J ? col0 + 64 : J;
  const int q_lo = col0 / T, q_hi = (col_end - 1) / T;
  const int nq = q_hi - q_lo + 1;
  const bool use_tab = doc_lo >= 0 && doc_hi < n_docs && doc_lo <= doc_hi &&
                       (int64_t(doc_hi) - doc_lo + 1) * nq <= tab_cap;
  const int n_tab = use_tab ? (doc_hi - doc_lo + 1) * nq : 0;
  for (int i = threadIdx.x; i < n_tab; i += RS_THREADS) tab[i] = -INFINITY;
  // query b, document doc (in [0, n_docs)), run maximum v
  auto emit = [&](int b, int doc, float v) {
    if (use_tab && doc >= doc_lo && doc <= doc_hi)
      lds_max_float(tab + (doc - doc_lo) * nq + (b - q_lo), v);
    else
      atomic_max_float(doc_score + int64_t(b) * n_docs + doc, v);
  };

  // A operand of head h for the tile: lane (lc, g4) holds chunk row lc, elements
  // 32*kk + 8*g4 .. +8 of the head.  Row-major stores give four lanes 64
  // contiguous bytes per load; the tiled layout gives the wave 1 KB.
  const int64_t n_cgroups = (n_chunks + 15) / 16;   // 16-chunk groups of the tiled layout
  auto load_head = [&](int64_t tl, int h, uint4 (&dst)[MT][RS_KK]) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if constexpr (TILED) {
        // 16-chunk group: one wave instruction reads 1 KB contiguous (lane-ordered)
        int64_t grp = tl * MT + m;
        if (grp >= n_cgroups) grp = n_cgroups - 1;
        const uint16_t* p = kr + grp * (16 * rowE) + int64_t(h) * (16 * RS_D) + 8 * lane;
#pragma unroll
        for (int kk = 0; kk < RS_KK; ++kk) dst[m][kk] = load_stream(p + kk * 512);   // read once
      } else {
        int64_t c = tl * TILE + 16 * m + lc;
        if (c >= n_chunks) c = n_chunks - 1;
        const uint4* p = reinterpret_cast<const uint4*>(kr + c * rowE + int64_t(h) * RS_D + 8 * g4);
#pragma unroll
        for (int kk = 0; kk < RS_KK; ++kk) dst[m][kk] = p[kk * 4];
      }
    }
  };

  // a ring of D head loads is in flight per wave; the first tile's first D
  // heads load while the queries are staged
  static_assert(H % D == 0, "the head ring divides the heads");
  uint4 buf[D][MT][RS_KK];
  if (tile < t_end) {
#pragma unroll
    for (int d = 0; d < D; ++d) load_head(tile, d, buf[d]);
  }

  // ---- stage the raw routing queries of this column group in fragment order
  const int nfrag_pieces = NT * H * RS_KK * 64;
  for (int p = threadIdx.x; p < nfrag_pieces; p += RS_THREADS) {
    const int l = p % 64, f = p / 64;
    const int kk = f % RS_KK, h = (f / RS_KK) % H, n = f / (RS_KK * H);
    const int col = col0 + 16 * n + (l % 16);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (col < J) v = *reinterpret_cast<const uint4*>(q_r + (int64_t(col) * H + h) * RS_D + 32 * kk + 8 * (l / 16));
    qfrag[p] = v;
  }
  __syncthreads();

  // ---- column scale w[h][n][lc] = 1 / (H * max(||q[col,h]||, eps)), kept in LDS
  float* wl = reinterpret_cast<float*>(smem + size_t(NT) * H * RS_KK * 1024 + size_t(RS_WAVES) * RS_SCRATCH);
  static_assert(RS_WAVES == H, "one wave per head computes the column norms");
  {
    const int h = wave;
    for (int n = 0; n < NT; ++n) {
      float ss = 0.f;
#pragma unroll
      for (int kk = 0; kk < RS_KK; ++kk) {
        const uint4 u = qfrag[((n * H + h) * RS_KK + kk) * 64 + lane];
        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = __uint_as_float(uu[e] << 16), b = __uint_as_float(uu[e] & 0xFFFF0000u);
          ss += a * a + b * b;
        }
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      if (g4 == 0) wl[(h * NT + n) * 16 + lc] = 1.f / (float(H) * fmaxf(sqrtf(ss), 1e-8f));
    }
  }
  __syncthreads();

  // column -> query index
  int colb[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int col = col0 + 16 * n + (UNIFORM_B ? 0 : lc);
    colb[n] = col < J ? col / T : -1;
  }

  f32x4 tot[MT][NT];
  auto head_step = [&](const uint4 (&a)[MT][RS_KK], int h) {
    f32x4 acc[MT][NT];
#pragma unroll
    for (int kk = 0; kk < RS_KK; ++kk) {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const bf16x8 bq = as_bf16x8(qfrag[((n * H + h) * RS_KK + kk) * 64 + lane]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const f32x4 cin = kk == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[m][n];
          acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[m][kk]), bq, cin, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float wv = wl[(h * NT + n) * 16 + lc];
#pragma unroll
      for (int m = 0; m < MT; ++m) tot[m][n] += wv * acc[m][n];
    }
  };

  // waves without a tile skip the loop but still reach the table's barrier
  if (tile < t_end) {
    for (;;) {
      const int mydoc = (lane < TILE && tile * TILE + lane < n_chunks) ? chunk_doc[tile * TILE + lane] : -1;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) tot[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int64_t next_tile = tile + RS_WAVES;
      // past the wave's last tile the ring refills from tile 0 (read by every
      // wave, so cached; never used): the loop stays straight-line code and the
      // compiler's waits on the load counter stay partial
      const int64_t pref_tile = next_tile < t_end ? next_tile : 0;
#pragma unroll 1
      for (int h0 = 0; h0 < H; h0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int h = h0 + d, hn = h + D;
          head_step(buf[d], h);
          load_head(hn < H ? tile : pref_tile, hn < H ? hn : hn - H, buf[d]);
          __builtin_amdgcn_sched_barrier(0);   // refill issued right after its head, not sunk below the ring
        }
      }
      // ---- epilogue: lane (lc, g4) holds score[chunk 16m + 4*g4 + r][column 16n + lc]
      if constexpr (UNIFORM_B) {
        // token max inside each query's columns, then the document max
#pragma unroll
        for (int n0 = 0; n0 < NT; ++n0) {
          const int b = colb[n0];
          if (b < 0) continue;
          bool first = true;
#pragma unroll
          for (int n1 = 0; n1 < n0; ++n1) first = first && (colb[n1] != b);
          if (!first) continue;
          float v[MT][4];
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float x = -INFINITY;
#pragma unroll
              for (int n = 0; n < NT; ++n)
                if (colb[n] == b) x = fmaxf(x, tot[m][n][r]);
              v[m][r] = dpp_row_max16(x);
            }
          if (lc == 0) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int r = 0; r < 4; ++r) scratch[16 * m + 4 * g4 + r] = v[m][r];
          }
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          const float cv = lane < TILE ? scratch[lane] : -INFINITY;
          seg_max_emit(cv, mydoc, lane, [&](int doc, float v) {
            if (doc < n_docs) emit(b, doc, v);
          });
          __builtin_amdgcn_wave_barrier();
        }
      } else {
        // every column is handled on its own: stage [16 columns][32 chunks] in LDS
        int* sdoc = reinterpret_cast<int*>(scratch + 16 * 33);
        if (lane < 32) sdoc[lane] = mydoc;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) scratch[lc * 33 + 16 * m + 4 * g4 + r] = tot[m][n][r];
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          const int b = colb[n];
          if (b >= 0) {
            float run = -INFINITY;
            int run_doc = -1;
            for (int i = 0; i < TILE / 4; ++i) {
              const int rr = (TILE / 4) * g4 + i;
              const int dd = sdoc[rr];
              const float x = scratch[lc * 33 + rr];
              if (dd != run_doc) {
                if (run_doc >= 0 && run_doc < n_docs) emit(b, run_doc, run);
                run_doc = dd;
                run = x;
              } else {
                run = fmaxf(run, x);
              }
            }
            if (run_doc >= 0 && run_doc < n_docs) emit(b, run_doc, run);
          }
          __builtin_amdgcn_wave_barrier();
        }
      }
      tile = next_tile;
      if (tile >= t_end) break;
    }
  }
  if (use_tab) {
    __syncthreads();
    for (int i = threadIdx.x; i < n_tab; i += RS_THREADS) {
      const float v = tab[i];
      if (v == -INFINITY) continue;   // the fill already holds it
      const int doc = doc_lo + i / nq, b = q_lo + i % nq;
      float* dst = doc_score + int64_t(b) * n_docs + doc;
      const bool own_q = b * T >= col0 && (b + 1) * T <= col_end;
      if (doc != doc_lo && doc != doc_hi && own_q)
        *dst = v;
      else
        atomic_max_float(dst, v);
    }
  }
}

// Vector path: float32 (or any head size) - one thread per (chunk, column),
// per-head dot products in float32 scaled by the precomputed column norms.
template <int DT>
__global__ void qnorm_kernel(const typename Elem<DT>::T* __restrict__ q_r, int J, int H, int d,
                             float* __restrict__ winv) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= J * H) return;
  const typename Elem<DT>::T* p = q_r + int64_t(i) * d;
  float ss = 0.f;
  for (int e = 0; e < d; ++e) {
    const float x = Elem<DT>::load(p, e);
    ss += x * x;
  }
  winv[i] = 1.f / (float(H) * fmaxf(sqrtf(ss), 1e-8f));
}

template <int DT>
__global__ void route_score_vec_kernel(const typename Elem<DT>::T* __restrict__ q_r, int T, int J, int H, int d,
                                       const typename Elem<DT>::T* __restrict__ kr,
                                       const int32_t* __restrict__ chunk_doc, int64_t n_docs, int64_t n_chunks,
                                       const float* __restrict__ winv, float* __restrict__ doc_score) {
  const int64_t p = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p >= n_chunks * J) return;
  const int64_t c = p / J;
  const int j = int(p % J);
  const int doc = chunk_doc[c];
  if (doc < 0 || doc >= n_docs) return;
  float s = 0.f;
  for (int h = 0; h < H; ++h) {
    const typename Elem<DT>::T* qp = q_r + (int64_t(j) * H + h) * d;
    const typename Elem<DT>::T* kp = kr + (c * H + h) * d;
    float dot = 0.f;
    for (int e = 0; e < d; ++e) dot += Elem<DT>::load(qp, e) * Elem<DT>::load(kp, e);
    s += winv[j * H + h] * dot;
  }
  atomic_max_float(doc_score + int64_t(j / T) * n_docs + doc, s);
}

static bool use_mfma(int dtype, int H, int d) { return dtype == MSA_BF16 && d == RS_D && H == RS_H; }

}  // namespace msa

extern "C" size_t msa_route_score_workspace(int dtype, int B, int T, int H, int d, int64_t n_docs,
                                            int64_t n_chunks) {
  (void)n_docs;
  (void)n_chunks;
  if (msa::use_mfma(dtype, H, d)) return 0;
  return msa::align_up(size_t(B) * T * H * sizeof(float), 256);
}

extern "C" int msa_route_score(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat,
                               int kr_layout, const int32_t* chunk_doc, int64_t n_docs, int64_t n_chunks,
                               float* doc_score, void* ws, size_t ws_bytes, void* stream) {
  using namespace msa;
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, "msa_route_score: bad dtype");
  MSA_REQUIRE(q_r && kr_hat && chunk_doc && doc_score, MSA_ERR_INVALID_ARG, "msa_route_score: NULL pointer");
  MSA_REQUIRE(B >= 1 && T >= 1 && H >= 1 && d >= 1 && n_docs >= 1 && n_chunks >= 1, MSA_ERR_INVALID_ARG,
              "msa_route_score: non-positive size");
  MSA_REQUIRE(int64_t(B) * T < (int64_t(1) << 24), MSA_ERR_UNSUPPORTED, "msa_route_score: B*T too large");
  MSA_REQUIRE(d <= 256 && d % 8 == 0, MSA_ERR_UNSUPPORTED, "msa_route_score: d must be a multiple of 8, <= 256");
  MSA_REQUIRE(kr_layout == MSA_LAYOUT_ROWS || kr_layout == MSA_LAYOUT_TILED, MSA_ERR_INVALID_ARG,
              "msa_route_score: bad kr_layout");
  MSA_REQUIRE(kr_layout == MSA_LAYOUT_ROWS || use_mfma(dtype, H, d), MSA_ERR_UNSUPPORTED,
              "msa_route_score: the tiled layout needs the MFMA path (bf16, H = 8, d = 128)");
  const size_t need = msa_route_score_workspace(dtype, B, T, H, d, n_docs, n_chunks);
  MSA_REQUIRE(ws_bytes >= need, MSA_ERR_WORKSPACE, "msa_route_score: workspace too small");
  MSA_REQUIRE(need == 0 || ws, MSA_ERR_INVALID_ARG, "msa_route_score: NULL workspace");
  MSA_REQUIRE(uintptr_t(q_r) % 16 == 0 && uintptr_t(kr_hat) % 16 == 0, MSA_ERR_INVALID_ARG,
              "msa_route_score: q_r and kr_hat must be 16-byte aligned");
  hipStream_t s = as_stream(stream);
  const int J = B * T;
  const int64_t nscore = int64_t(B) * n_docs;
  {
    const int64_t blocks = std::min<int64_t>((nscore + 255) / 256, 65536);
    hipLaunchKernelGGL(fill_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, doc_score, nscore, -INFINITY);
    MSA_LAUNCH_CHECK();
  }
  if (use_mfma(dtype, H, d)) {
    const int n_groups = (J + 63) / 64;
    const int NT = std::min(4, (J + 15) / 16);
    const bool uniform = (T % 16) == 0;
    int dev = 0;
    MSA_HIP_CHECK(hipGetDevice(&dev));
    int n_cu = 0;
    MSA_HIP_CHECK(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
    const int64_t tiles_total = (n_chunks + 16 * RS_MT - 1) / (16 * RS_MT);
    int64_t n_ranges = std::min<int64_t>(n_cu, (tiles_total + RS_WAVES - 1) / RS_WAVES);
    if (n_groups > 1) n_ranges = (n_ranges + 7) / 8 * 8;
    const int64_t tiles_per_range = (tiles_total + n_ranges - 1) / n_ranges;
    const size_t smem_base =
        size_t(NT) * RS_H * RS_KK * 1024 + size_t(RS_WAVES) * RS_SCRATCH + size_t(RS_H) * NT * 16 * 4;
    int lds_max = 0;
    MSA_HIP_CHECK(hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
    // the document table takes what LDS is left, up to 32 KB
    const int tab_cap = int(std::min<int64_t>(8192, std::max<int64_t>(0, (int64_t(lds_max) - int64_t(smem_base)) / 4)));
    const size_t smem = smem_base + size_t(tab_cap) * 4;
    const dim3 grid(unsigned(n_ranges * n_groups)), block(RS_THREADS);
#define RS_LAUNCH3(NTV, UNI, TIL, DV)                                                                    \
  MSA_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&route_score_mfma_kernel<NTV, UNI, TIL, DV>), \
                                    hipFuncAttributeMaxDynamicSharedMemorySize, int(smem)));           \
  hipLaunchKernelGGL((route_score_mfma_kernel<NTV, UNI, TIL, DV>), grid, block, smem, s,               \
                     static_cast<const uint16_t*>(q_r), T, J, static_cast<const uint16_t*>(kr_hat),     \
                     chunk_doc, n_docs, n_chunks, doc_score, n_groups, int(n_ranges), tiles_per_range, tab_cap)
// Tiled stores stream one 16-chunk group per wave, a head at a time: one head
// in flight per wave reads each group strictly in order and measured best
// with one column group; column groups sharing a range (their second read
// hits L2) measured best with two.  Row-major stores keep two.
#define RS_LAUNCH(NTV, UNI)                    \
  if (tiled && n_groups == 1) {                \
    RS_LAUNCH3(NTV, UNI, true, 1);             \
  } else if (tiled) {                          \
    RS_LAUNCH3(NTV, UNI, true, 2);             \
  } else {                                     \
    RS_LAUNCH3(NTV, UNI, false, 2);            \
  }
    const bool tiled = kr_layout == MSA_LAYOUT_TILED;
    switch (NT * 2 + (uniform ? 1 : 0)) {
      case 2: RS_LAUNCH(1, false); break;
      case 3: RS_LAUNCH(1, true); break;
      case 4: RS_LAUNCH(2, false); break;
      case 5: RS_LAUNCH(2, true); break;
      case 6: RS_LAUNCH(3, false); break;
      case 7: RS_LAUNCH(3, true); break;
      case 8: RS_LAUNCH(4, false); break;
      default: RS_LAUNCH(4, true); break;
    }
#undef RS_LAUNCH
#undef RS_LAUNCH3
    MSA_LAUNCH_CHECK();
    return MSA_OK;
  }
  float* winv = static_cast<float*>(ws);
  if (dtype == MSA_BF16) {
    hipLaunchKernelGGL(qnorm_kernel<MSA_BF16>, dim3((J * H + 255) / 256), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q_r), J, H, d, winv);
  } else {
    hipLaunchKernelGGL(qnorm_kernel<MSA_F32>, dim3((J * H + 255) / 256), dim3(256), 0, s,
                       static_cast<const float*>(q_r), J, H, d, winv);
  }
  MSA_LAUNCH_CHECK();
  const int64_t work = n_chunks * J;
  const dim3 grid(unsigned((work + 255) / 256)), block(256);
  if (dtype == MSA_BF16)
    hipLaunchKernelGGL(route_score_vec_kernel<MSA_BF16>, grid, block, 0, s, static_cast<const uint16_t*>(q_r), T,
                       J, H, d, static_cast<const uint16_t*>(kr_hat), chunk_doc, n_docs, n_chunks, winv,
                       doc_score);
  else
    hipLaunchKernelGGL(route_score_vec_kernel<MSA_F32>, grid, block, 0, s, static_cast<const float*>(q_r), T, J,
                       H, d, static_cast<const float*>(kr_hat), chunk_doc, n_docs, n_chunks, winv, doc_score);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}
