// Stage 2 routing score: cosine of every pooled routing key against the
// routing query, mean over heads, max over query tokens and over the
// document's chunks -> one score per (query, document).
// (MSA README, Overall Design > Architecture: cosine similarity averaged over
//  heads, then a max over tokens; Inference Pipeline, Online Routing;
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
//
// Workgroup b runs on XCD b % 8.  The XCDs of one device need not stream at
// the same rate (on some MI355X devices the odd ones take 4-5% longer
// for the same bytes), so the chunk ranges may be sized per XCD: shares set
// by msa_route_balance, which times this kernel per workgroup.  Any split of
// the tiles into ranges gives the same scores; only the launch's length
// depends on it.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

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

// The document owning chunk c; without a map every chunk is its own
// "document", which gives the per-chunk scores of msa_chunk_scores.
__device__ __forceinline__ int doc_of(const int32_t* __restrict__ chunk_doc, int64_t c) {
  return chunk_doc ? chunk_doc[c] : int(c);
}

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

// A fetch done in the launch's tail (msa_route_score_fetch): the workgroups
// that finish their chunk ranges first copy the documents another layer
// selected (its pooled K / V rows, in device memory or mapped pinned host
// memory) into that layer's context, one (query, rank) at a time, taken from
// a counter.  The copy is the one msa_gather_kv makes: rank r of query b lands
// at the sum of the chunk counts of ranks < r, never past max_ctx.
struct TailFetch {
  unsigned* counter;          // NULL: no fetch
  const int32_t* ids;         // [B, k]
  int B, k;
  const int64_t* chunk_off;   // [n_docs + 1]
  int64_t n_docs;
  const uint4* k_bar;         // pooled rows of row_vec 16-byte vectors
  const uint4* v_bar;
  int64_t row_vec;
  int max_ctx;
  uint4* k_ctx;               // [B, max_ctx] rows
  uint4* v_ctx;
  int32_t* ctx_pos;           // [B, max_ctx]
  int32_t* ctx_len;           // [B]
};

// The whole workgroup takes (query, rank) items until the counter passes the
// last one.  lds: 16 bytes of LDS no longer in use.  Every item is a plain
// copy of the same bytes to the same place, so an item taken twice (a counter
// that workgroup 0 clears late, at its start) changes nothing.
__device__ void tail_fetch(const TailFetch& tf, unsigned* lds) {
  if (!tf.counter) return;
  const unsigned n_items = unsigned(tf.B) * unsigned(tf.k);
  for (;;) {
    __syncthreads();   // the LDS words are free
    if (threadIdx.x == 0) lds[0] = atomicAdd(tf.counter, 1u);
    __syncthreads();
    const unsigned item = lds[0];
    if (item >= n_items) return;
    const int b = int(item / unsigned(tf.k)), r = int(item % unsigned(tf.k));
    const int32_t* ids_b = tf.ids + int64_t(b) * tf.k;
    if (threadIdx.x < 64) {   // dest: the chunk counts of ranks < r (at most max_ctx in all)
      int mine = 0;
      for (int q = threadIdx.x; q < r; q += 64) {
        const int32_t doc = ids_b[q];
        if (doc >= 0 && doc < tf.n_docs) mine += int(tf.chunk_off[doc + 1] - tf.chunk_off[doc]);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mine += __shfl_xor(mine, o);
      if (threadIdx.x == 0) lds[1] = unsigned(mine);
    }
    __syncthreads();
    const int64_t dest = int64_t(lds[1]);
    const int32_t doc = ids_b[r];
    int64_t lo = 0, n = 0;
    if (doc >= 0 && doc < tf.n_docs) {
      lo = tf.chunk_off[doc];
      n = tf.chunk_off[doc + 1] - lo;
    }
    if (dest + n > tf.max_ctx) n = dest < tf.max_ctx ? tf.max_ctx - dest : 0;   // never past the context
    if (r == tf.k - 1 && threadIdx.x == 0) tf.ctx_len[b] = int32_t(dest + n);
    for (int64_t i = threadIdx.x; i < n; i += RS_THREADS) tf.ctx_pos[int64_t(b) * tf.max_ctx + dest + i] = int32_t(i);
    const int64_t total = n * tf.row_vec;
    const uint4* ks = tf.k_bar + lo * tf.row_vec;
    const uint4* vs = tf.v_bar + lo * tf.row_vec;
    uint4* kd = tf.k_ctx + (int64_t(b) * tf.max_ctx + dest) * tf.row_vec;
    uint4* vd = tf.v_ctx + (int64_t(b) * tf.max_ctx + dest) * tf.row_vec;
    constexpr int U = 4;   // four 16-byte loads of K and of V in flight per thread
    int64_t i = threadIdx.x;
    for (; i + (U - 1) * RS_THREADS < total; i += U * RS_THREADS) {
      uint4 a[U], c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a[u] = ks[i + u * RS_THREADS];
        c[u] = vs[i + u * RS_THREADS];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kd[i + u * RS_THREADS] = a[u];
        vd[i + u * RS_THREADS] = c[u];
      }
    }
    for (; i < total; i += RS_THREADS) {
      kd[i] = ks[i];
      vd[i] = vs[i];
    }
  }
}

// NT: 16-column tiles per column group (<= 4); UNIFORM_B: every 16-column
// tile belongs to one query (T % 16 == 0), so the token max is taken in
// registers before the document max.
// D: head loads in flight per wave (the ring)
// Chunk ranges sized per XCD: range r (on XCD r % 8, with all its column
// groups) takes len[r % 8] tiles, the ranges laid out in order; on = 0: equal
// ranges.
struct XcdSplit {
  int64_t len[8];
  int on;
};

template <int NT, bool UNIFORM_B, bool TILED, int D>
__global__ __launch_bounds__(RS_THREADS) void route_score_mfma_kernel(
    const uint16_t* __restrict__ q_r, int T, int J, const uint16_t* __restrict__ kr,
    const int32_t* __restrict__ chunk_doc, int64_t n_docs, int64_t n_chunks, float* __restrict__ doc_score,
    int n_groups, int n_ranges, int64_t tiles_per_range, int tab_cap, XcdSplit xs, uint64_t* __restrict__ wg_ts,
    TailFetch tf) {
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
  if (tf.counter && blockIdx.x == 0 && threadIdx.x == 0) atomicExch(tf.counter, 0u);   // the tail fetch's counter
  if (range >= n_ranges) {
    tail_fetch(tf, reinterpret_cast<unsigned*>(smem));
    return;
  }
  // per-workgroup start and end stamps (the 100 MHz real-time counter), for msa_route_balance
  if (wg_ts && threadIdx.x == 0) wg_ts[2 * blockIdx.x] = __builtin_amdgcn_s_memrealtime();
  const int col0 = group * 64;

  const int g4 = lane / 16;       // lane group: k-slice of the operands, row block of the result
  const int lc = lane % 16;       // column (query token) of this lane inside a 16-column tile
  constexpr int MT = RS_MT;
  constexpr int TILE = 16 * MT;   // chunks per wave tile
  const int64_t tiles_total = (n_chunks + TILE - 1) / TILE;
  int64_t t_begin = int64_t(range) * tiles_per_range;
  int64_t t_end = t_begin + tiles_per_range;
  if (xs.on) {   // range r and its column groups run on XCD r % 8
    // selects over the unrolled XCDs (no dynamic index into the argument)
    int64_t round = 0, before = 0, mine = 0;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      round += xs.len[x];
      before += x < range % 8 ? xs.len[x] : 0;
      mine = x == range % 8 ? xs.len[x] : mine;
    }
    t_begin = int64_t(range / 8) * round + before;
    t_end = t_begin + mine;
  }
  if (t_end > tiles_total) t_end = tiles_total;
  if (t_begin >= t_end) {                   // a range past the last tile (whole workgroup)
    if (wg_ts && threadIdx.x == 0) wg_ts[2 * blockIdx.x + 1] = wg_ts[2 * blockIdx.x];
    tail_fetch(tf, reinterpret_cast<unsigned*>(smem));
    return;
  }
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
  const int doc_lo = doc_of(chunk_doc, t_begin * TILE), doc_hi = doc_of(chunk_doc, c_last);
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
      const int mydoc = (lane < TILE && tile * TILE + lane < n_chunks) ? doc_of(chunk_doc, tile * TILE + lane) : -1;
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
  if (wg_ts) {
    __syncthreads();
    if (threadIdx.x == 0) wg_ts[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
  }
  tail_fetch(tf, reinterpret_cast<unsigned*>(smem));   // the query fragments are no longer read
}

// Vector path: float32 (or any head size).  The query is first scaled per
// (column, head) by 1 / (H * max(||q||, eps)) into float32 rows q' (one wave
// per (column, head)), so a chunk's score for column j is the flat dot product
// of q'[j] and the chunk's H*d elements.  A workgroup stages a block of CB
// columns of q' in LDS and each wave takes one chunk at a time: lanes stride
// over the chunk's elements (coalesced) with CB accumulators, a wave-wide sum
// per column, then the token max inside each query and one atomic max per
// (query, chunk) into its document.
template <int DT>
__global__ void qscale_vec_kernel(const typename Elem<DT>::T* __restrict__ q_r, int J, int H, int d,
                                  float* __restrict__ qs) {
  // one wave per (column, head): lanes stride over the head's d elements
  const int64_t i = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / 64;
  const int lane = threadIdx.x % 64;
  if (i >= int64_t(J) * H) return;               // uniform in the wave
  const typename Elem<DT>::T* p = q_r + i * d;
  float ss = 0.f;
  for (int e = lane; e < d; e += 64) {
    const float x = Elem<DT>::load(p, e);
    ss += x * x;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float w = 1.f / (float(H) * fmaxf(sqrtf(ss), 1e-8f));
  float* o = qs + i * d;
  for (int e = lane; e < d; e += 64) o[e] = Elem<DT>::load(p, e) * w;
}

constexpr int RV_THREADS = 256;
constexpr int RV_CB = 16;    // largest column block

template <int DT, int CB>
__global__ __launch_bounds__(RV_THREADS) void route_score_vec_kernel(
    const float* __restrict__ qs, int T, int J, int E, const typename Elem<DT>::T* __restrict__ kr,
    const int32_t* __restrict__ chunk_doc, int64_t n_docs, int64_t n_chunks, float* __restrict__ doc_score) {
  extern __shared__ float qcol[];                  // [CB][E]
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int j0 = blockIdx.y * CB;
  const int nc = min(CB, J - j0);
  // the block's columns are consecutive rows of q', so the block is one
  // contiguous span; columns past J are zero.  Eight loads in flight per lane
  // (a serial staging loop is one L2 round trip per element).
  {
    const float* src = qs + int64_t(j0) * E;
    const int n_valid = nc * E, n_all = CB * E;
    if ((E & 3) == 0) {
      float4* dst4 = reinterpret_cast<float4*>(qcol);
      const float4* src4 = reinterpret_cast<const float4*>(src);
      for (int i0 = threadIdx.x; i0 < n_all / 4; i0 += RV_THREADS * 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * RV_THREADS;
          v[u] = i < n_valid / 4 ? src4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + u * RV_THREADS < n_all / 4) dst4[i0 + u * RV_THREADS] = v[u];
      }
    } else {
      for (int i0 = threadIdx.x; i0 < n_all; i0 += RV_THREADS * 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * RV_THREADS;
          v[u] = i < n_valid ? src[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + u * RV_THREADS < n_all) qcol[i0 + u * RV_THREADS] = v[u];
      }
    }
  }
  __syncthreads();
  const int64_t stride = int64_t(gridDim.x) * (RV_THREADS / 64);
  for (int64_t c = int64_t(blockIdx.x) * (RV_THREADS / 64) + wave; c < n_chunks; c += stride) {
    const int doc = doc_of(chunk_doc, c);
    if (doc < 0 || doc >= n_docs) continue;        // uniform in the wave
    const typename Elem<DT>::T* kp = kr + c * E;
    float acc[CB];
#pragma unroll
    for (int jj = 0; jj < CB; ++jj) acc[jj] = 0.f;
    // eight of the chunk's loads in flight per lane
    for (int e0 = lane; e0 < E; e0 += 64 * 8) {
      float kv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) kv[u] = e0 + 64 * u < E ? Elem<DT>::load(kp, e0 + 64 * u) : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (e0 + 64 * u >= E) break;
#pragma unroll
        for (int jj = 0; jj < CB; ++jj) acc[jj] += qcol[jj * E + e0 + 64 * u] * kv[u];
      }
    }
#pragma unroll
    for (int jj = 0; jj < CB; ++jj) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) acc[jj] += __shfl_xor(acc[jj], o);
    }
    // token max inside each query of the block, one atomic per (query, chunk)
    if (lane == 0) {
      int b = -1;
      float v = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < CB; ++jj) {
        if (jj >= nc) break;
        const int bj = (j0 + jj) / T;
        if (bj != b) {
          if (b >= 0) atomic_max_float(doc_score + int64_t(b) * n_docs + doc, v);
          b = bj;
          v = acc[jj];
        } else {
          v = fmaxf(v, acc[jj]);
        }
      }
      if (b >= 0) atomic_max_float(doc_score + int64_t(b) * n_docs + doc, v);
    }
  }
}

static bool use_mfma(int dtype, int H, int d) { return dtype == MSA_BF16 && d == RS_D && H == RS_H; }

// Per-device XCD shares of the chunk ranges (set by msa_route_balance; none: equal ranges),
// used where every range has at least RB_MIN_TILES tiles.
constexpr int RB_MAX_DEVICES = 64;
constexpr int64_t RB_MIN_TILES = 128;
static std::mutex g_balance_mu;
static float g_shares[RB_MAX_DEVICES][8];
static bool g_has_shares[RB_MAX_DEVICES];

// The shares of device dev, if set.
static bool device_shares(int dev, float (&sh)[8]) {
  if (dev < 0 || dev >= RB_MAX_DEVICES) return false;
  std::lock_guard<std::mutex> lock(g_balance_mu);
  if (!g_has_shares[dev]) return false;
  for (int x = 0; x < 8; ++x) sh[x] = g_shares[dev][x];
  return true;
}

// Range lengths per XCD for shares sh (summing to 1): rounds = workgroups per
// XCD; the ranges cover every tile (the last ones may fall short or be empty).
static XcdSplit make_split(const float (&sh)[8], int64_t tiles_total, int64_t rounds) {
  XcdSplit xs{};
  xs.on = 1;
  for (int x = 0; x < 8; ++x)
    xs.len[x] = std::max<int64_t>(1, int64_t(std::ceil(double(tiles_total) * sh[x] / double(rounds))));
  return xs;
}

}  // namespace msa

extern "C" size_t msa_route_score_workspace(int dtype, int B, int T, int H, int d, int64_t n_docs,
                                            int64_t n_chunks) {
  (void)n_docs;
  (void)n_chunks;
  if (msa::use_mfma(dtype, H, d)) return 0;
  return msa::align_up(size_t(B) * T * H * d * sizeof(float), 256);   // the scaled query rows q'

}

namespace msa {

// Shared body of msa_route_score (chunk_doc given) and msa_chunk_scores
// (chunk_doc NULL: every chunk is its own document, n_docs = n_chunks).
// shares (msa_route_balance): the XCD shares to use instead of the device's;
// wg_ts: per-workgroup start and end stamps; *split_used: whether the ranges
// were sized per XCD (one workgroup per CU); prefilled: doc_score already
// holds -inf (MSA_ROUTE_PREFILLED), so the fill is not launched.
static int route_score(const std::string& fn, int dtype, const void* q_r, int B, int T, int H, int d,
                       const void* kr_hat, int kr_layout, const int32_t* chunk_doc, int64_t n_docs,
                       int64_t n_chunks, float* doc_score, void* ws, size_t ws_bytes, void* stream,
                       const float* shares = nullptr, uint64_t* wg_ts = nullptr, bool* split_used = nullptr,
                       int* n_wg = nullptr, bool prefilled = false, const TailFetch* fetch = nullptr) {
  if (split_used) *split_used = false;
  using namespace msa;
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, fn + ": bad dtype");
  MSA_REQUIRE(q_r && kr_hat && doc_score, MSA_ERR_INVALID_ARG, fn + ": NULL pointer");
  MSA_REQUIRE(B >= 1 && T >= 1 && H >= 1 && d >= 1 && n_docs >= 1 && n_chunks >= 1, MSA_ERR_INVALID_ARG,
              fn + ": non-positive size");
  MSA_REQUIRE(int64_t(B) * T < (int64_t(1) << 24), MSA_ERR_UNSUPPORTED, fn + ": B*T too large");
  MSA_REQUIRE(d <= 256 && d % 8 == 0, MSA_ERR_UNSUPPORTED, fn + ": d must be a multiple of 8, <= 256");
  MSA_REQUIRE(kr_layout == MSA_LAYOUT_ROWS || kr_layout == MSA_LAYOUT_TILED, MSA_ERR_INVALID_ARG,
              fn + ": bad kr_layout");
  MSA_REQUIRE(kr_layout == MSA_LAYOUT_ROWS || use_mfma(dtype, H, d), MSA_ERR_UNSUPPORTED,
              fn + ": the tiled layout needs the MFMA path (bf16, H = 8, d = 128)");
  const size_t need = msa_route_score_workspace(dtype, B, T, H, d, n_docs, n_chunks);
  MSA_REQUIRE(ws_bytes >= need, MSA_ERR_WORKSPACE, fn + ": workspace too small");
  MSA_REQUIRE(need == 0 || ws, MSA_ERR_INVALID_ARG, fn + ": NULL workspace");
  MSA_REQUIRE(uintptr_t(q_r) % 16 == 0 && uintptr_t(kr_hat) % 16 == 0, MSA_ERR_INVALID_ARG,
              fn + ": q_r and kr_hat must be 16-byte aligned");
  hipStream_t s = as_stream(stream);
  const int J = B * T;
  const int64_t nscore = int64_t(B) * n_docs;
  if (!prefilled) {
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
    if (n_groups > 1) {
      n_ranges = (n_ranges + 7) / 8 * 8;
      // column groups: one round of workgroups (ranges x groups = CUs) when every range still
      // holds 64+ tiles.  Two rounds measured slower on a 10M-token store (T = 128: 76.8 vs
      // 72.8 us; 200 columns: 170.8 vs 150.9 us) but faster on a 1M-token one (16.7 vs 21.4 us).
      const int64_t one_round = std::max<int64_t>(8, (n_cu / n_groups) / 8 * 8);
      if (one_round < n_ranges && tiles_total >= 64 * one_round) n_ranges = one_round;
    }
    const int64_t tiles_per_range = (tiles_total + n_ranges - 1) / n_ranges;
    XcdSplit xs{};
    // only long ranges: at ~40 tiles per range (a 10M-token store) the split measured no faster
    if (n_ranges * n_groups == n_cu && n_ranges % 8 == 0 && tiles_total >= RB_MIN_TILES * n_ranges) {
      float sh[8];
      bool have = shares != nullptr;
      if (have) {
        for (int x = 0; x < 8; ++x) sh[x] = shares[x];
      } else {
        have = device_shares(dev, sh);
      }
      if (have) xs = make_split(sh, tiles_total, n_ranges / 8);
    }
    if (split_used) *split_used = xs.on != 0;
    if (n_wg) *n_wg = int(n_ranges * n_groups);
    const size_t smem_base =
        size_t(NT) * RS_H * RS_KK * 1024 + size_t(RS_WAVES) * RS_SCRATCH + size_t(RS_H) * NT * 16 * 4;
    int lds_max = 0;
    MSA_HIP_CHECK(hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
    // the document table takes what LDS is left, up to 32 KB
    const int tab_cap = int(std::min<int64_t>(8192, std::max<int64_t>(0, (int64_t(lds_max) - int64_t(smem_base)) / 4)));
    const size_t smem = smem_base + size_t(tab_cap) * 4;
    const dim3 grid(unsigned(n_ranges * n_groups)), block(RS_THREADS);
    const TailFetch tfv = fetch ? *fetch : TailFetch{};
#define RS_LAUNCH3(NTV, UNI, TIL, DV)                                                                    \
  MSA_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&route_score_mfma_kernel<NTV, UNI, TIL, DV>), \
                                    hipFuncAttributeMaxDynamicSharedMemorySize, int(smem)));           \
  hipLaunchKernelGGL((route_score_mfma_kernel<NTV, UNI, TIL, DV>), grid, block, smem, s,               \
                     static_cast<const uint16_t*>(q_r), T, J, static_cast<const uint16_t*>(kr_hat),     \
                     chunk_doc, n_docs, n_chunks, doc_score, n_groups, int(n_ranges), tiles_per_range, tab_cap, \
                     xs, wg_ts, tfv)
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
  float* qs = static_cast<float*>(ws);
  const unsigned qblocks = unsigned((int64_t(J) * H + 3) / 4);   // four waves per block
  if (dtype == MSA_BF16)
    hipLaunchKernelGGL(qscale_vec_kernel<MSA_BF16>, dim3(qblocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q_r), J, H, d, qs);
  else
    hipLaunchKernelGGL(qscale_vec_kernel<MSA_F32>, dim3(qblocks), dim3(256), 0, s,
                       static_cast<const float*>(q_r), J, H, d, qs);
  MSA_LAUNCH_CHECK();
  {
    const int E = H * d;
    int dev = 0, n_cu = 0;
    MSA_HIP_CHECK(hipGetDevice(&dev));
    MSA_HIP_CHECK(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
    // column block: as many columns as fit 64 KB of LDS, at most 16
    const int cb_fit = int(std::max<int64_t>(1, std::min<int64_t>(RV_CB, 65536 / (int64_t(E) * 4))));
    const int CB = cb_fit >= 16 ? 16 : (cb_fit >= 8 ? 8 : (cb_fit >= 4 ? 4 : 1));
    const int n_cb = (J + CB - 1) / CB;
    const int64_t waves_per_wg = RV_THREADS / 64;
    const int64_t gx = std::max<int64_t>(1, std::min<int64_t>((n_chunks + waves_per_wg - 1) / waves_per_wg,
                                                                std::max<int64_t>(1, 4 * int64_t(n_cu) / n_cb)));
    const size_t smem = size_t(CB) * E * sizeof(float);
    MSA_REQUIRE(smem <= 65536 && n_cb <= 65535, MSA_ERR_UNSUPPORTED, fn + ": vector path shape");
    const dim3 grid{unsigned(gx), unsigned(n_cb)}, block{unsigned(RV_THREADS)};
#define RV_LAUNCH(DTV, TV, CBV)                                                                              \
  hipLaunchKernelGGL((route_score_vec_kernel<DTV, CBV>), grid, block, smem, s, qs, T, J, E,                  \
                     static_cast<const TV*>(kr_hat), chunk_doc, n_docs, n_chunks, doc_score)
#define RV_DT(DTV, TV)                                      \
    switch (CB) {                                           \
      case 16: RV_LAUNCH(DTV, TV, 16); break;                \
      case 8: RV_LAUNCH(DTV, TV, 8); break;                  \
      case 4: RV_LAUNCH(DTV, TV, 4); break;                  \
      default: RV_LAUNCH(DTV, TV, 1); break;                 \
    }
    if (dtype == MSA_BF16) {
      RV_DT(MSA_BF16, uint16_t);
    } else {
      RV_DT(MSA_F32, float);
    }
#undef RV_DT
#undef RV_LAUNCH
  }
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

}  // namespace msa

extern "C" int msa_route_score(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat,
                               int kr_layout, const int32_t* chunk_doc, int64_t n_docs, int64_t n_chunks,
                               float* doc_score, void* ws, size_t ws_bytes, int flags, void* stream) {
  MSA_REQUIRE(chunk_doc, MSA_ERR_INVALID_ARG, "msa_route_score: NULL pointer");
  MSA_REQUIRE((flags & ~MSA_ROUTE_PREFILLED) == 0, MSA_ERR_INVALID_ARG, "msa_route_score: unknown flags");
  return msa::route_score("msa_route_score", dtype, q_r, B, T, H, d, kr_hat, kr_layout, chunk_doc, n_docs, n_chunks,
                          doc_score, ws, ws_bytes, stream, nullptr, nullptr, nullptr, nullptr,
                          (flags & MSA_ROUTE_PREFILLED) != 0);
}

extern "C" size_t msa_route_score_fetch_workspace(int dtype, int B, int T, int H, int d, int64_t n_docs,
                                                  int64_t n_chunks) {
  return msa::align_up(msa_route_score_workspace(dtype, B, T, H, d, n_docs, n_chunks), 256) + 256;
}

extern "C" int msa_route_score_fetch(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat,
                                     int kr_layout, const int32_t* chunk_doc, int64_t n_docs, int64_t n_chunks,
                                     float* doc_score, void* ws, size_t ws_bytes, int flags, const int32_t* f_ids,
                                     int f_B, int f_k, const int64_t* f_chunk_off, int64_t f_n_docs,
                                     int f_max_doc_chunks, const void* f_k_bar, const void* f_v_bar, int f_Hkv,
                                     int f_d, int f_max_ctx, void* f_k_ctx, void* f_v_ctx, int32_t* f_ctx_pos,
                                     int32_t* f_ctx_len, void* stream) {
  using namespace msa;
  const std::string fn = "msa_route_score_fetch";
  MSA_REQUIRE(chunk_doc, MSA_ERR_INVALID_ARG, fn + ": NULL pointer");
  MSA_REQUIRE((flags & ~MSA_ROUTE_PREFILLED) == 0, MSA_ERR_INVALID_ARG, fn + ": unknown flags");
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, fn + ": bad dtype");
  MSA_REQUIRE(f_ids && f_chunk_off && f_k_bar && f_v_bar && f_k_ctx && f_v_ctx && f_ctx_pos && f_ctx_len,
              MSA_ERR_INVALID_ARG, fn + ": NULL fetch pointer");
  MSA_REQUIRE(f_B >= 1 && f_k >= 1 && f_n_docs >= 1 && f_max_doc_chunks >= 1 && f_Hkv >= 1 && f_d >= 1,
              MSA_ERR_INVALID_ARG, fn + ": non-positive fetch size");
  MSA_REQUIRE(f_k <= f_n_docs, MSA_ERR_INVALID_ARG, fn + ": f_k > f_n_docs");
  MSA_REQUIRE(int64_t(f_max_ctx) >= int64_t(f_k) * f_max_doc_chunks, MSA_ERR_INVALID_ARG,
              fn + ": f_max_ctx < f_k * f_max_doc_chunks");
  MSA_REQUIRE(f_B <= 65535 && f_k <= 65535, MSA_ERR_UNSUPPORTED, fn + ": f_B or f_k too large");
  const int64_t row_bytes = int64_t(f_Hkv) * f_d * dtype_bytes(dtype);
  MSA_REQUIRE(row_bytes % 16 == 0, MSA_ERR_UNSUPPORTED, fn + ": f_Hkv*f_d*elem_bytes must be a multiple of 16");
  MSA_REQUIRE(uintptr_t(f_k_bar) % 16 == 0 && uintptr_t(f_v_bar) % 16 == 0 && uintptr_t(f_k_ctx) % 16 == 0 &&
                  uintptr_t(f_v_ctx) % 16 == 0,
              MSA_ERR_INVALID_ARG, fn + ": fetch K/V buffers must be 16-byte aligned");
  const size_t rws = msa_route_score_workspace(dtype, B, T, H, d, n_docs, n_chunks);
  MSA_REQUIRE(ws_bytes >= align_up(rws, 256) + 256, MSA_ERR_WORKSPACE, fn + ": workspace too small");
  MSA_REQUIRE(ws, MSA_ERR_INVALID_ARG, fn + ": NULL workspace");
  const bool prefilled = (flags & MSA_ROUTE_PREFILLED) != 0;
  if (!use_mfma(dtype, H, d)) {   // the vector scan has no tail to spare: the two calls in order
    const int rc = route_score(fn, dtype, q_r, B, T, H, d, kr_hat, kr_layout, chunk_doc, n_docs, n_chunks, doc_score,
                               ws, rws, stream, nullptr, nullptr, nullptr, nullptr, prefilled);
    if (rc != MSA_OK) return rc;
    return gather_copy(f_ids, f_B, f_k, f_chunk_off, f_n_docs, f_k_bar, f_v_bar, row_bytes / 16, f_max_ctx, f_k_ctx,
                       f_v_ctx, f_ctx_pos, f_ctx_len, as_stream(stream));
  }
  TailFetch tf{};
  tf.counter = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + align_up(rws, 256));
  tf.ids = f_ids;
  tf.B = f_B;
  tf.k = f_k;
  tf.chunk_off = f_chunk_off;
  tf.n_docs = f_n_docs;
  tf.k_bar = static_cast<const uint4*>(f_k_bar);
  tf.v_bar = static_cast<const uint4*>(f_v_bar);
  tf.row_vec = row_bytes / 16;
  tf.max_ctx = f_max_ctx;
  tf.k_ctx = static_cast<uint4*>(f_k_ctx);
  tf.v_ctx = static_cast<uint4*>(f_v_ctx);
  tf.ctx_pos = f_ctx_pos;
  tf.ctx_len = f_ctx_len;
  return route_score(fn, dtype, q_r, B, T, H, d, kr_hat, kr_layout, chunk_doc, n_docs, n_chunks, doc_score, ws, rws,
                     stream, nullptr, nullptr, nullptr, nullptr, prefilled, &tf);
}

extern "C" int msa_chunk_scores(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat,
                                int kr_layout, int64_t n_chunks, float* chunk_score, void* ws, size_t ws_bytes,
                                void* stream) {
  MSA_REQUIRE(n_chunks < (int64_t(1) << 31), MSA_ERR_UNSUPPORTED, "msa_chunk_scores: n_chunks >= 2^31");
  return msa::route_score("msa_chunk_scores", dtype, q_r, B, T, H, d, kr_hat, kr_layout, nullptr, n_chunks, n_chunks,
                          chunk_score, ws, ws_bytes, stream);
}

namespace msa {

// doc_score[b, i] = max of chunk_score[b, c] over the chunks c of document i
// (chunk_off CSR); -inf for an empty document.  One thread per (query, document).
__global__ void segment_max_kernel(const float* __restrict__ chunk_score, int B, int64_t n_chunks,
                                   const int64_t* __restrict__ chunk_off, int64_t n_docs,
                                   float* __restrict__ doc_score) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(B) * n_docs) return;
  const int64_t b = i / n_docs, doc = i % n_docs;
  int64_t lo = chunk_off[doc], hi = chunk_off[doc + 1];
  lo = lo < 0 ? 0 : (lo > n_chunks ? n_chunks : lo);
  hi = hi < lo ? lo : (hi > n_chunks ? n_chunks : hi);
  const float* row = chunk_score + b * n_chunks;
  float m = -INFINITY;
  for (int64_t c = lo; c < hi; ++c) m = fmaxf(m, row[c]);
  doc_score[i] = m;
}

}  // namespace msa

extern "C" int msa_segment_max(const float* chunk_score, int B, int64_t n_chunks, const int64_t* chunk_off,
                               int64_t n_docs, float* doc_score, void* stream) {
  using namespace msa;
  MSA_REQUIRE(chunk_score && chunk_off && doc_score, MSA_ERR_INVALID_ARG, "msa_segment_max: NULL pointer");
  MSA_REQUIRE(B >= 1 && n_chunks >= 1 && n_docs >= 1, MSA_ERR_INVALID_ARG, "msa_segment_max: non-positive size");
  MSA_REQUIRE(int64_t(B) * n_docs < (int64_t(1) << 40), MSA_ERR_UNSUPPORTED, "msa_segment_max: too many scores");
  const int64_t n = int64_t(B) * n_docs;
  hipLaunchKernelGGL(segment_max_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, as_stream(stream),
                     chunk_score, B, n_chunks, chunk_off, n_docs, doc_score);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

// Calibration of the per-XCD range sizes: rounds of timed launches of the
// routing kernel on the caller's store; after each, every XCD's share moves
// by the ratio of the XCDs' mean workgroup duration to its own.
extern "C" int msa_route_balance(int dtype, const void* q_r, int B, int T, int H, int d, const void* kr_hat,
                                 int kr_layout, const int32_t* chunk_doc, int64_t n_docs, int64_t n_chunks,
                                 float* doc_score, void* ws, size_t ws_bytes, int rounds, float* shares_out,
                                 void* stream) {
  using namespace msa;
  const std::string fn = "msa_route_balance";
  MSA_REQUIRE(rounds >= 0 && rounds <= 64, MSA_ERR_INVALID_ARG, fn + ": rounds must lie in [0, 64]");
  int dev = 0;
  MSA_HIP_CHECK(hipGetDevice(&dev));
  MSA_REQUIRE(dev >= 0 && dev < RB_MAX_DEVICES, MSA_ERR_UNSUPPORTED, fn + ": device ordinal beyond 63");
  float sh[8];
  for (int x = 0; x < 8; ++x) sh[x] = 0.125f;
  if (rounds == 0) {   // back to equal ranges
    std::lock_guard<std::mutex> lock(g_balance_mu);
    g_has_shares[dev] = false;
    if (shares_out)
      for (int x = 0; x < 8; ++x) shares_out[x] = sh[x];
    return MSA_OK;
  }
  MSA_REQUIRE(chunk_doc, MSA_ERR_INVALID_ARG, fn + ": NULL pointer");
  {
    float cur[8];
    if (device_shares(dev, cur))
      for (int x = 0; x < 8; ++x) sh[x] = cur[x];
  }
  int n_cu = 0;
  MSA_HIP_CHECK(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  uint64_t* ts = nullptr;
  MSA_HIP_CHECK(hipMalloc(reinterpret_cast<void**>(&ts), size_t(2) * std::max(n_cu, 1) * sizeof(uint64_t)));
  std::vector<uint64_t> h(size_t(2) * std::max(n_cu, 1));
  hipStream_t s = as_stream(stream);
  int st = MSA_OK;
  bool balanced = false;
  // untimed launches first: the clocks of an idle device take a few launches to settle
  for (int w = 0; w < 4 && st == MSA_OK; ++w)
    st = route_score(fn, dtype, q_r, B, T, H, d, kr_hat, kr_layout, chunk_doc, n_docs, n_chunks, doc_score, ws,
                     ws_bytes, stream, sh);
  for (int r = 0; r < rounds && st == MSA_OK; ++r) {
    double sum[8] = {0}, cnt[8] = {0};
    for (int rep = 0; rep < 3 && st == MSA_OK; ++rep) {
      bool used = false;
      int n_wg = 0;
      st = route_score(fn, dtype, q_r, B, T, H, d, kr_hat, kr_layout, chunk_doc, n_docs, n_chunks, doc_score, ws,
                       ws_bytes, stream, sh, ts, &used, &n_wg);
      if (st != MSA_OK) break;
      if (!used || n_wg != n_cu) {   // this shape does not size ranges per XCD: nothing to balance
        rounds = 0;
        break;
      }
      hipError_t e = hipStreamSynchronize(s);
      if (e == hipSuccess) e = hipMemcpy(h.data(), ts, h.size() * sizeof(uint64_t), hipMemcpyDeviceToHost);
      if (e != hipSuccess) {
        set_error(fn + ": " + hipGetErrorString(e));
        st = MSA_ERR_HIP;
        break;
      }
      uint64_t t0 = UINT64_MAX;
      for (int b = 0; b < n_cu; ++b) t0 = std::min(t0, h[2 * b]);
      for (int b = 0; b < n_cu; ++b) {
        if (h[2 * b + 1] <= h[2 * b]) continue;   // an empty range
        sum[b % 8] += double(h[2 * b + 1] - t0);
        cnt[b % 8] += 1;
      }
    }
    if (st != MSA_OK || rounds == 0) break;
    double mean_end[8], all = 0;
    int n_ok = 0;
    for (int x = 0; x < 8; ++x) {
      mean_end[x] = cnt[x] > 0 ? sum[x] / cnt[x] : 0;
      if (cnt[x] > 0) {
        all += mean_end[x];
        ++n_ok;
      }
    }
    if (n_ok < 8) break;
    all /= 8;
    double tot = 0;
    for (int x = 0; x < 8; ++x) {
      // the share moves by the XCD's rate relative to the others, within 0.75x..1.25x of equal
      const double v = double(sh[x]) * all / mean_end[x];
      sh[x] = float(std::min(1.25 / 8, std::max(0.75 / 8, v)));
      tot += sh[x];
    }
    for (int x = 0; x < 8; ++x) sh[x] = float(sh[x] / tot);
    balanced = true;
  }
  hipFree(ts);
  if (st != MSA_OK) return st;
  {
    std::lock_guard<std::mutex> lock(g_balance_mu);
    if (balanced) {
      for (int x = 0; x < 8; ++x) g_shares[dev][x] = sh[x];
      g_has_shares[dev] = true;
    }
  }
  if (shares_out)   // the shares in use from now on (unchanged when nothing was calibrated)
    for (int x = 0; x < 8; ++x) shares_out[x] = sh[x];
  return MSA_OK;
}
