// Backward of the Stage 3 sparse attention (training-time path).
// (Paper note 核心方法 > 训练 and README Abstract: the MSA layer is trained end
//  to end; the selection is held fixed and the gradients reach the query, the
//  local K/V and the selected pooled rows, summed over every query and
//  context entry that reads a row.)
//
// The forward is recomputed (its kernels, with the per-row base-2
// log-sum-exp), then per query row D = <dO, O>.  With P = softmax of the
// scaled logits, dP = dO V^T and dS = P * (dP - D):
//   dV = P^T dO,  dK_rot = scale dS^T Q_rot,  dQ_rot = scale dS K_rot,
// and a rotation's adjoint is the rotation by the opposite angle.
//
// bf16, d = 128 (MFMA): the rotated query scaled by scale * log2(e) and dO
// are staged once as bf16 rows, and every key once as its rotated K and V
// (so that both kernels address keys affinely).  dK/dV: one wave per 16-key
// tile holds its rotated K and V as MFMA operands and walks a range of the
// head's query row tiles (rows staged in LDS per tile): S and dP come from
// v_mfma_f32_16x16x32_bf16, and P, dS leave the accumulator in exactly the
// B-operand order of v_mfma_f32_16x16x16bf16_1k, whose A operand (dO^T or
// Q^T) is read with LDS transpose loads; a reduce pass adds the ranges.  dQ:
// one wave per 16-row tile over a key split, like the forward prefill;
// partial sums per split are added and turned back by the query's rotation
// in a last pass.
#include "attn_common.h"

namespace msa {

constexpr int BW_WAVES = 4;
constexpr int BW_THREADS = 64 * BW_WAVES;
constexpr float BW_LOG2E = 1.4426950408889634f;
constexpr int BW_DEPTH = 4;   // tiles (dK/dV) or key steps (dQ) whose loads are in flight (even)
static_assert(BW_DEPTH % 2 == 0, "tile i uses LDS buffer i % 2");

// A operand of a 16x16x16 product from a row-major bf16 tile (16 rows, row
// stride AT_VS): lane (lc, g4) receives tile[4*g4 + r][16*dt + lc], r = 0..3
// (the first of pv_operand's two transpose reads).
__device__ __forceinline__ v4s tr_operand4(const unsigned char* tile, int dt, int lane) {
  const int g4 = lane / 16, j = lane % 16;
  const int r = j / 4, q = j % 4;
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(tile + (4 * g4 + r) * AT_VS + (16 * dt + 4 * q) * 2));
}

__device__ __forceinline__ v4s pack4(float a, float b, float c, float d) {
  return __builtin_bit_cast(v4s, make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d)));
}

// Source row and position of key j of query b (context entries first, then
// the local tokens); rows are clamped into their tensor.
struct BwKey {
  int64_t row;
  int pos;
  bool local, valid;
};
__device__ __forceinline__ BwKey bw_key(int j, int b, int ctxl, int n_keys, int max_ctx, int L_loc, int qpo,
                                        const int32_t* __restrict__ ctx_pos, int P, const int32_t* __restrict__ ctx_row,
                                        int64_t ctx_rows) {
  BwKey k;
  k.valid = j >= 0 && j < n_keys;
  k.local = j >= ctxl;
  if (!k.local) {
    const int64_t e = int64_t(b) * max_ctx + j;
    k.row = ctx_src_row(e, ctx_row, ctx_rows);
    const int p = ctx_pos[e];
    k.pos = p < 0 ? 0 : (p >= P ? P - 1 : p);
  } else {
    const int li = min(max(j - ctxl, 0), L_loc - 1);
    k.row = int64_t(b) * L_loc + li;
    k.pos = qpo + li;
  }
  return k;
}

// ---------------------------------------------------------------- key preparation
// Every key of every query once: krot[b, j, g, :] = R(pos_j) k_j (bf16, the
// rounding the forward applies) and vg[b, j, g, :] = v_j, zero past the
// query's keys, so that the backward kernels address keys affinely.  One
// thread per (query, key, KV head, block of 8 rotation pairs).
__global__ void bwd_keys_kernel(int B, int KM, int Hkv, const uint16_t* __restrict__ k_bar,
                                const uint16_t* __restrict__ v_bar, int64_t ctx_rows,
                                const int32_t* __restrict__ ctx_row, const int32_t* __restrict__ ctx_pos,
                                const int32_t* __restrict__ ctx_len, int max_ctx, const uint16_t* __restrict__ k_loc,
                                const uint16_t* __restrict__ v_loc, int L_loc, int qpo, const float2* __restrict__ tab,
                                int P, uint16_t* __restrict__ krot, uint16_t* __restrict__ vg) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(B) * KM * Hkv * 8) return;
  const int blk = int(i % 8);
  const int g = int((i / 8) % Hkv);
  const int j = int((i / (8 * Hkv)) % KM);
  const int b = int(i / (8 * int64_t(Hkv) * KM));
  const int ctxl = min(max(ctx_len[b], 0), max_ctx);
  const BwKey kl = bw_key(j, b, ctxl, ctxl + L_loc, max_ctx, L_loc, qpo, ctx_pos, P, ctx_row, ctx_rows);
  const int64_t o = ((int64_t(b) * KM + j) * Hkv + g) * AT_D + 8 * blk;
  uint4 lo = make_uint4(0, 0, 0, 0), hi = lo, va = lo, vb = lo;
  if (kl.valid) {
    const int64_t src = (kl.row * Hkv + g) * AT_D + 8 * blk;
    const uint16_t* kp = (kl.local ? k_loc : k_bar) + src;
    const uint16_t* vp = (kl.local ? v_loc : v_bar) + src;
    float a[8], bb[8];
    unpack8(load_global(kp), a);
    unpack8(load_global(kp + AT_D / 2), bb);
    const float2* cs = tab + int64_t(kl.pos) * (AT_D / 2) + 8 * blk;
    float ra[8], rb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 c = cs[e];
      ra[e] = a[e] * c.x - bb[e] * c.y;
      rb[e] = bb[e] * c.x + a[e] * c.y;
    }
    lo = pack8(ra);
    hi = pack8(rb);
    va = load_global(vp);
    vb = load_global(vp + AT_D / 2);
  }
  *reinterpret_cast<uint4*>(krot + o) = lo;
  *reinterpret_cast<uint4*>(krot + o + AT_D / 2) = hi;
  *reinterpret_cast<uint4*>(vg + o) = va;
  *reinterpret_cast<uint4*>(vg + o + AT_D / 2) = vb;
}

// ---------------------------------------------------------------- row preparation
// Vector path: one wave per query row (b, t, hq) computes D = <dO, O>.
template <int DT>
__global__ __launch_bounds__(BW_THREADS) void bwd_prep_kernel(const float* __restrict__ out,
                                                              const float* __restrict__ dout, int d, int64_t rows,
                                                              float* __restrict__ Dv) {
  const int64_t r = int64_t(blockIdx.x) * BW_WAVES + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (r >= rows) return;
  float acc = 0.f;
  for (int e = lane; e < d; e += 64) acc += out[r * d + e] * dout[r * d + e];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (lane == 0) Dv[r] = acc;
}

// MFMA path (bf16, d = 128): D = <dO, O>, and the bf16 rows of dO and of the
// rotated query times scale * log2(e) (rotated in float32, rounded once, as
// the forward does).  Sixteen lanes per row; lane i holds dims 4i..4i+3 and
// 64+4i..64+4i+3 (the RoPE pairs).
__global__ __launch_bounds__(BW_THREADS) void bwd_prep128_kernel(
    const uint16_t* __restrict__ q, int T, int Hq, int L_loc, int qpo, const float2* __restrict__ tab, int P,
    float qscale, const float* __restrict__ out, const float* __restrict__ dout, int64_t rows, float* __restrict__ Dv,
    uint16_t* __restrict__ qs16, uint16_t* __restrict__ do16) {
  const int64_t r = (int64_t(blockIdx.x) * BW_THREADS + threadIdx.x) / 16;
  const int i = threadIdx.x % 16;
  if (r >= rows) return;   // the row's sixteen lanes leave together
  const int64_t base = r * AT_D;
  const float4 o0 = *reinterpret_cast<const float4*>(out + base + 4 * i);
  const float4 o1 = *reinterpret_cast<const float4*>(out + base + 64 + 4 * i);
  const float4 g0 = *reinterpret_cast<const float4*>(dout + base + 4 * i);
  const float4 g1 = *reinterpret_cast<const float4*>(dout + base + 64 + 4 * i);
  float acc = o0.x * g0.x + o0.y * g0.y + o0.z * g0.z + o0.w * g0.w + o1.x * g1.x + o1.y * g1.y + o1.z * g1.z +
              o1.w * g1.w;
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (i == 0) Dv[r] = acc;
  const int t = int((r / Hq) % T);
  int pq = qpo + L_loc - T + t;
  pq = pq < 0 ? 0 : (pq >= P ? P - 1 : pq);
  const uint2 qa = *reinterpret_cast<const uint2*>(q + base + 4 * i);
  const uint2 qb = *reinterpret_cast<const uint2*>(q + base + 64 + 4 * i);
  const float4 cs0 = *reinterpret_cast<const float4*>(tab + int64_t(pq) * (AT_D / 2) + 4 * i);
  const float4 cs1 = *reinterpret_cast<const float4*>(tab + int64_t(pq) * (AT_D / 2) + 4 * i + 2);
  const float a[4] = {bf16_to_f32(uint16_t(qa.x)), bf16_to_f32(uint16_t(qa.x >> 16)), bf16_to_f32(uint16_t(qa.y)),
                      bf16_to_f32(uint16_t(qa.y >> 16))};
  const float bb[4] = {bf16_to_f32(uint16_t(qb.x)), bf16_to_f32(uint16_t(qb.x >> 16)), bf16_to_f32(uint16_t(qb.y)),
                       bf16_to_f32(uint16_t(qb.y >> 16))};
  const float c[4] = {cs0.x, cs0.z, cs1.x, cs1.z}, sn[4] = {cs0.y, cs0.w, cs1.y, cs1.w};
  uint16_t ra[4], rb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ra[e] = f32_to_bf16((a[e] * c[e] - bb[e] * sn[e]) * qscale);
    rb[e] = f32_to_bf16((bb[e] * c[e] + a[e] * sn[e]) * qscale);
  }
  auto pack2 = [](uint16_t lo, uint16_t hi) { return uint32_t(lo) | (uint32_t(hi) << 16); };
  *reinterpret_cast<uint2*>(qs16 + base + 4 * i) = make_uint2(pack2(ra[0], ra[1]), pack2(ra[2], ra[3]));
  *reinterpret_cast<uint2*>(qs16 + base + 64 + 4 * i) = make_uint2(pack2(rb[0], rb[1]), pack2(rb[2], rb[3]));
  *reinterpret_cast<uint2*>(do16 + base + 4 * i) =
      make_uint2(pack2(f32_to_bf16(g0.x), f32_to_bf16(g0.y)), pack2(f32_to_bf16(g0.z), f32_to_bf16(g0.w)));
  *reinterpret_cast<uint2*>(do16 + base + 64 + 4 * i) =
      make_uint2(pack2(f32_to_bf16(g1.x), f32_to_bf16(g1.y)), pack2(f32_to_bf16(g1.z), f32_to_bf16(g1.w)));
}

// ---------------------------------------------------------------- dK, dV (MFMA)
// Workgroup = (query b, KV head g, block of 64 keys, range of row tiles); the
// row tiles of the range are staged through two LDS buffers, the next one
// loading while the current one is computed (LDS-only barriers).  Each row
// range writes its partial sums; a reduce pass adds them.
struct BwRows {
  uint4 q, o;      // this thread's 16-byte piece of the tile's q_s and dO rows
  float l, D;      // threads 0..15: the rows' log-sum-exp and D
};

// Row ranges of the dK/dV pass.  Key block kb holds key slots [64 kb, 64 kb + 64);
// slots below max_ctx may be context entries, seen by every row; a block of
// local keys only (local index >= 64 kb - max_ctx) is seen by the rows whose
// causal horizon L_loc - T + t reaches it.  Those rows, from the first row
// tile that can see the block, are cut into ranges of rt_per row tiles.
__host__ __device__ inline int bw_rt_min(int kb, int max_ctx, int L_loc, int T, int G) {
  const int t_min = kb * BW_WAVES * 16 - max_ctx - (L_loc - T);
  return kb * BW_WAVES * 16 < max_ctx || t_min <= 0 ? 0 : (t_min * G) / 16;
}
__host__ __device__ inline int bw_n_ranges(int kb, int max_ctx, int L_loc, int T, int G, int n_rt, int rt_per) {
  const int rt_min = bw_rt_min(kb, max_ctx, L_loc, T, G);
  return rt_min >= n_rt ? 0 : (n_rt - rt_min + rt_per - 1) / rt_per;
}

template <int G>
__global__ __launch_bounds__(BW_THREADS) void attn_bwd_dkdv_kernel(
    int B, int T, int Hq, int Hkv, const uint16_t* __restrict__ krot, const uint16_t* __restrict__ vg, int KM,
    const int32_t* __restrict__ ctx_len, int max_ctx, int L_loc, const uint16_t* __restrict__ qs16,
    const uint16_t* __restrict__ do16, const float* __restrict__ lse, const float* __restrict__ Dv, int n_kb,
    int rt_per, int n_items, float* __restrict__ part_k, float* __restrict__ part_v) {
  __shared__ __attribute__((aligned(16))) unsigned char qt[2][16 * AT_VS];
  __shared__ __attribute__((aligned(16))) unsigned char ot[2][16 * AT_VS];
  __shared__ __attribute__((aligned(16))) float slse[2][16], sD[2][16];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int lc = lane % 16, g4 = lane / 16;
  int64_t wg = blockIdx.x;
  const int item = int(wg % n_items);                // (key block, row range) of this (b, g)
  wg /= n_items;
  const int g = int(wg % Hkv);
  const int b = int(wg / Hkv);
  const int R = T * G;                               // query rows of this KV head
  const int n_rt = (R + 15) / 16;
  int kb = 0, rs = item;
  for (; kb < n_kb; ++kb) {                          // uniform scalar search
    const int nr = bw_n_ranges(kb, max_ctx, L_loc, T, G, n_rt, rt_per);
    if (rs < nr) break;
    rs -= nr;
  }
  if (kb >= n_kb) return;
  const int ctxl = min(max(ctx_len[b], 0), max_ctx);
  const int n_keys = ctxl + L_loc;
  if (kb * BW_WAVES * 16 >= n_keys) return;          // no key of this block exists for query b
  const int j0 = (kb * BW_WAVES + wave) * 16;       // this wave's 16 keys
  const int rt_begin = bw_rt_min(kb, max_ctx, L_loc, T, G) + rs * rt_per, rt_end = min(n_rt, rt_begin + rt_per);
  if (rt_begin >= rt_end) return;

  // the lane's key (column lc of every product) as rotated K and as V
  const bool key_ok = j0 + lc < n_keys;
  uint4 kr[4], vr[4];
  {
    const int64_t o = ((int64_t(b) * KM + min(j0 + lc, KM - 1)) * Hkv + g) * AT_D + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      kr[kk] = load_global(krot + o + 32 * kk);
      vr[kk] = load_global(vg + o + 32 * kk);
    }
  }
  const bool wave_live = j0 < n_keys;
  f32x4 dkT[8], dvT[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    dkT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dvT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int srow = tid / 16, scol = tid % 16;       // staging: one 16-byte piece per thread and tile
  auto grow_of = [&](int r) { return (int64_t(b) * T + r / G) * Hq + g * G + r % G; };
  // loads of row tile rt, always issued (rows past R read row R - 1 and are zeroed)
  auto load_rows = [&](int rt) {
    BwRows x;
    const int r = rt * 16 + srow, rc = min(r, R - 1);
    const int64_t gr = grow_of(rc);
    x.q = load_global(qs16 + gr * AT_D + 8 * scol);
    x.o = load_global(do16 + gr * AT_D + 8 * scol);
    if (r >= R) x.q = x.o = make_uint4(0, 0, 0, 0);
    const int r2 = rt * 16 + (tid % 16), r2c = min(r2, R - 1);
    const float lv = lse[grow_of(r2c)], dv = Dv[grow_of(r2c)];
    x.l = r2 < R ? lv : INFINITY;
    x.D = r2 < R ? dv : 0.f;
    return x;
  };
  auto store_rows = [&](const BwRows& x, int buf) {
    *reinterpret_cast<uint4*>(qt[buf] + srow * AT_VS + 16 * scol) = x.q;
    *reinterpret_cast<uint4*>(ot[buf] + srow * AT_VS + 16 * scol) = x.o;
    if (tid < 16) {
      slse[buf][tid] = x.l;
      sD[buf][tid] = x.D;
    }
  };
  auto compute = [&](int rt, int buf) {
    // rows of this tile see key j iff j < ctxl or j - ctxl <= L_loc - T + t
    const int t_max = min(rt * 16 + 15, R - 1) / G;
    if (!wave_live || (j0 >= ctxl && j0 - ctxl > L_loc - T + t_max)) return;
    const unsigned char* qb = qt[buf];
    const unsigned char* ob = ot[buf];
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint4 qa = *reinterpret_cast<const uint4*>(qb + lc * AT_VS + 64 * kk + 16 * g4);
      const uint4 da = *reinterpret_cast<const uint4*>(ob + lc * AT_VS + 64 * kk + 16 * g4);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa), __builtin_bit_cast(bf16x8, kr[kk]),
                                                   sc, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, da), __builtin_bit_cast(bf16x8, vr[kk]),
                                                   dp, 0, 0, 0);
    }
    // lane (lc, g4) holds S and dP at row 4*g4 + i, key lc.  Rows past R
    // carry lse = +inf (P = 0); keys past n_keys are never written.  Only
    // the causal edge needs a mask (a uniform test finds the tiles without).
    float p[4], ds[4];
    const int j = j0 + lc;
    const float4 l4 = *reinterpret_cast<const float4*>(&slse[buf][4 * g4]);
    const float4 d4 = *reinterpret_cast<const float4*>(&sD[buf][4 * g4]);
    const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
    const bool full = j0 + 15 < ctxl || j0 + 15 - ctxl <= L_loc - T + (rt * 16) / G;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rt * 16 + 4 * g4 + i;
      const bool vis = full || j < ctxl || j - ctxl <= L_loc - T + r / G;
      p[i] = vis ? __builtin_amdgcn_exp2f(sc[i] - lv[i]) : 0.f;
      ds[i] = p[i] * (dp[i] - dv[i]);
    }
    const v4s pb = pack4(p[0], p[1], p[2], p[3]);
    const v4s sb = pack4(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      dvT[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(tr_operand4(ob, dt, lane), pb, dvT[dt], 0, 0, 0);
      dkT[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(tr_operand4(qb, dt, lane), sb, dkT[dt], 0, 0, 0);
    }
  };
  // BW_DEPTH row tiles are in flight in registers.  Buffer i % 2 is
  // rewritten two tiles after it was read and each wave's reads of it
  // precede its next barrier, so one barrier per tile suffices.  Requests
  // past the range repeat its last tile (in bounds, never computed).
  const int n_t = rt_end - rt_begin;
  auto rt_at = [&](int i) { return rt_begin + min(i, n_t - 1); };
  BwRows ring[BW_DEPTH];
#pragma unroll
  for (int u = 0; u < BW_DEPTH; ++u) ring[u] = load_rows(rt_at(u));
  for (int i0 = 0; i0 < n_t; i0 += BW_DEPTH) {
#pragma unroll
    for (int u = 0; u < BW_DEPTH; ++u) {
      store_rows(ring[u], u & 1);
      ring[u] = load_rows(rt_at(i0 + u + BW_DEPTH));
      lds_barrier();
      if (i0 + u < n_t) compute(rt_begin + i0 + u, u & 1);
    }
  }
  if (!key_ok) return;
  // partial sums of this row range: lane holds dK_rot^T, dV^T at dims
  // e = 16*dt + 4*g4 + i of key lc; the query rows carried scale * log2(e),
  // so dK_rot = sum(dS q_s) / log2(e)
  const int64_t slot = ((int64_t(rs) * B + b) * (int64_t(n_kb) * BW_WAVES * 16) + j0 + lc) * Hkv + g;
  float* kd = part_k + slot * AT_D;
  float* vd = part_v + slot * AT_D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    *reinterpret_cast<float4*>(kd + 16 * dt + 4 * g4) =
        make_float4(dkT[dt][0], dkT[dt][1], dkT[dt][2], dkT[dt][3]) * (1.f / BW_LOG2E);
    *reinterpret_cast<float4*>(vd + 16 * dt + 4 * g4) = make_float4(dvT[dt][0], dvT[dt][1], dvT[dt][2], dvT[dt][3]);
  }
}

// Sum of the row ranges' partials per (query, key, KV head, pair block),
// the inverse rotation of dK, then a plain store for a local key and an
// atomic add for a pooled row (several queries may read it).
__global__ void attn_bwd_dkdv_reduce_kernel(const float* __restrict__ part_k, const float* __restrict__ part_v,
                                            int T, int G, int rt_per, int B, int KM, int Hkv, int L_loc, int qpo,
                                            const int32_t* __restrict__ ctx_row, int64_t ctx_rows,
                                            const int32_t* __restrict__ ctx_pos, const int32_t* __restrict__ ctx_len,
                                            int max_ctx, const float2* __restrict__ tab, int P,
                                            float* __restrict__ dk_loc, float* __restrict__ dv_loc,
                                            float* __restrict__ dk_bar, float* __restrict__ dv_bar) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;   // (b, j, g, quad of pairs)
  const int64_t n = int64_t(B) * KM * Hkv * 16;
  if (i >= n) return;
  const int qd = int(i % 16);
  const int g = int((i / 16) % Hkv);
  const int j = int((i / (16 * Hkv)) % KM);
  const int b = int(i / (16 * int64_t(Hkv) * KM));
  const int ctxl = min(max(ctx_len[b], 0), max_ctx);
  const int n_keys = ctxl + L_loc;
  if (j >= n_keys) return;
  const BwKey kl = bw_key(j, b, ctxl, n_keys, max_ctx, L_loc, qpo, ctx_pos, P, ctx_row, ctx_rows);
  float4 ka = make_float4(0.f, 0.f, 0.f, 0.f), kb = ka, va = ka, vb = ka;
  const int n_ranges = bw_n_ranges(j / (BW_WAVES * 16), max_ctx, L_loc, T, G, (T * G + 15) / 16, rt_per);
  for (int r = 0; r < n_ranges; ++r) {
    const int64_t o = (((int64_t(r) * B + b) * KM + j) * Hkv + g) * AT_D + 4 * qd;
    ka += *reinterpret_cast<const float4*>(part_k + o);
    kb += *reinterpret_cast<const float4*>(part_k + o + AT_D / 2);
    va += *reinterpret_cast<const float4*>(part_v + o);
    vb += *reinterpret_cast<const float4*>(part_v + o + AT_D / 2);
  }
  const float4 c0 = reinterpret_cast<const float4*>(tab + int64_t(kl.pos) * (AT_D / 2) + 4 * qd)[0];
  const float4 c1 = reinterpret_cast<const float4*>(tab + int64_t(kl.pos) * (AT_D / 2) + 4 * qd)[1];
  const float c[4] = {c0.x, c0.z, c1.x, c1.z}, sn[4] = {c0.y, c0.w, c1.y, c1.w};
  const float a[4] = {ka.x, ka.y, ka.z, ka.w}, bb[4] = {kb.x, kb.y, kb.z, kb.w};
  float lo[4], hi[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {          // the inverse rotation of the pair (m, m + 64)
    lo[e] = a[e] * c[e] + bb[e] * sn[e];
    hi[e] = bb[e] * c[e] - a[e] * sn[e];
  }
  const int64_t o = (kl.row * Hkv + g) * AT_D + 4 * qd;
  if (kl.local) {
    *reinterpret_cast<float4*>(dk_loc + o) = make_float4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<float4*>(dk_loc + o + AT_D / 2) = make_float4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<float4*>(dv_loc + o) = va;
    *reinterpret_cast<float4*>(dv_loc + o + AT_D / 2) = vb;
  } else {
    const float v4[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      unsafeAtomicAdd(dk_bar + o + e, lo[e]);
      unsafeAtomicAdd(dk_bar + o + AT_D / 2 + e, hi[e]);
      unsafeAtomicAdd(dv_bar + o + e, v4[e]);
      unsafeAtomicAdd(dv_bar + o + AT_D / 2 + e, v4[4 + e]);
    }
  }
}

// ---------------------------------------------------------------- dQ (MFMA)
// One wave per 16-row tile of a KV head, four tiles per workgroup, over one
// key split.  Each 32-key step's rotated K and V rows (prepared once per
// key) go through two LDS buffers; BW_DEPTH steps of loads are in flight.
constexpr int BQ_KV_BYTES = 32 * AT_VS;

struct BqRegs {
  uint4 k[2], v[2];       // dims 8x..8x+7 of keys lk and 16 + lk
};

template <int G>
__global__ __launch_bounds__(BW_THREADS) void attn_bwd_dq_kernel(
    int B, int T, int Hq, int Hkv, const uint16_t* __restrict__ krot, const uint16_t* __restrict__ vg, int KM,
    const int32_t* __restrict__ ctx_len, int max_ctx, int L_loc, const uint16_t* __restrict__ qs16,
    const uint16_t* __restrict__ do16, const float* __restrict__ lse, const float* __restrict__ Dv, int n_rg,
    int n_splits, float* __restrict__ ws_dq, const float2* __restrict__ tab, int P, int qpo, float scale,
    float* __restrict__ dq_out) {
  __shared__ __attribute__((aligned(16))) unsigned char kt[2][BQ_KV_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char vt[2][BQ_KV_BYTES];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int lc = lane % 16, g4 = lane / 16;
  int64_t wg = blockIdx.x;
  const int split = int(wg % n_splits);
  wg /= n_splits;
  const int rg = int(wg % n_rg);
  wg /= n_rg;
  const int g = int(wg % Hkv);
  const int b = int(wg / Hkv);
  const int ctxl = min(max(ctx_len[b], 0), max_ctx);
  const int n_keys = ctxl + L_loc;
  const int R = T * G;
  const int r = (rg * BW_WAVES + wave) * 16 + lc;   // this lane's query row (column lc)
  const bool rok = r < R;
  const int t = rok ? r / G : 0;
  const int64_t grow = (int64_t(b) * T + t) * Hq + g * G + (rok ? r % G : 0);
  const int horizon = L_loc - T + t;
  uint4 qb[4], db[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qb[kk] = rok ? load_global(qs16 + grow * AT_D + 32 * kk + 8 * g4) : make_uint4(0, 0, 0, 0);
    db[kk] = rok ? load_global(do16 + grow * AT_D + 32 * kk + 8 * g4) : make_uint4(0, 0, 0, 0);
  }
  const float l2 = rok ? lse[grow] : INFINITY;
  const float Dr = rok ? Dv[grow] : 0.f;
  f32x4 dqT[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dqT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kps = ((n_keys + n_splits - 1) / n_splits + 31) / 32 * 32;
  const int j_begin = split * kps;
  const int j_end = min(n_keys, j_begin + kps);
  // staging: 16 keys per pass of the workgroup, thread (key lk, 8-dim block lx)
  const int lk = tid / 16, lx = tid % 16;
  const uint16_t* kbase = krot + (int64_t(b) * KM * Hkv + g) * AT_D + 8 * lx;
  const uint16_t* vbase = vg + (int64_t(b) * KM * Hkv + g) * AT_D + 8 * lx;
  auto load_step = [&](int jj) {
    BqRegs x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t o = int64_t(min(jj + 16 * h + lk, KM - 1)) * Hkv * AT_D;
      x.k[h] = load_global(kbase + o);
      x.v[h] = load_global(vbase + o);
    }
    return x;
  };
  auto store_step = [&](const BqRegs& x, int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = 16 * h + lk;
      *reinterpret_cast<uint4*>(kt[buf] + key * AT_VS + 16 * lx) = x.k[h];
      *reinterpret_cast<uint4*>(vt[buf] + key * AT_VS + 16 * lx) = x.v[h];
    }
  };
  auto compute_step = [&](int jj, int buf) {
    float dsv[2][4];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint4 ka = *reinterpret_cast<const uint4*>(kt[buf] + (16 * tau + lc) * AT_VS + 64 * kk + 16 * g4);
        const uint4 va = *reinterpret_cast<const uint4*>(vt[buf] + (16 * tau + lc) * AT_VS + 64 * kk + 16 * g4);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka), __builtin_bit_cast(bf16x8, qb[kk]),
                                                     sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, db[kk]),
                                                     dp, 0, 0, 0);
      }
      // lane (lc, g4): key 16*tau + 4*g4 + i, row lc
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = jj + 16 * tau + 4 * g4 + i;
        const bool vis = rok && j < j_end && (j < ctxl || j - ctxl <= horizon);
        const float p = vis ? __builtin_amdgcn_exp2f(sc[i] - l2) : 0.f;
        dsv[tau][i] = p * (dp[i] - Dr);
      }
    }
    const bf16x8 sb = __builtin_bit_cast(
        bf16x8, make_uint4(pack_bf16x2(dsv[0][0], dsv[0][1]), pack_bf16x2(dsv[0][2], dsv[0][3]),
                           pack_bf16x2(dsv[1][0], dsv[1][1]), pack_bf16x2(dsv[1][2], dsv[1][3])));
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      dqT[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pv_operand(kt[buf], dt, lane), sb, dqT[dt], 0, 0, 0);
  };
  const int n_steps = j_begin < j_end ? (j_end - j_begin + 31) / 32 : 0;
  if (n_steps > 0) {
    // BW_DEPTH steps are in flight; a buffer is rewritten two steps after it
    // was read; requests past the last step repeat its addresses (in bounds,
    // never used)
    auto j_at = [&](int i) { return j_begin + 32 * min(i, n_steps - 1); };
    BqRegs ring[BW_DEPTH];
#pragma unroll
    for (int u = 0; u < BW_DEPTH; ++u) ring[u] = load_step(j_at(u));
    for (int i0 = 0; i0 < n_steps; i0 += BW_DEPTH) {
#pragma unroll
      for (int u = 0; u < BW_DEPTH; ++u) {
        store_step(ring[u], u & 1);
        ring[u] = load_step(j_at(i0 + u + BW_DEPTH));
        lds_barrier();
        if (i0 + u < n_steps) compute_step(j_at(i0 + u), u & 1);
      }
    }
  }
  if (!rok) return;
  if (dq_out) {
    // one split: this is the whole sum, so the scale and the query's inverse
    // rotation are applied here, with attn_bwd_dq_sum_kernel's arithmetic.
    // Lane (lc, g4) holds dims 16*dt + 4*g4 + e: the pair (m, m + 64) of dt < 4
    // sits in dt and dt + 4 of the same lane.
    int pq = qpo + L_loc - T + t;
    pq = pq < 0 ? 0 : (pq >= P ? P - 1 : pq);
    const float2* tr = tab + int64_t(pq) * (AT_D / 2);
    float* dp = dq_out + grow * AT_D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int m0 = 16 * dt + 4 * g4;
      float lo4[4], hi4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 c = tr[m0 + e];
        float a = dqT[dt][e], bb = dqT[dt + 4][e];
        a *= scale;
        bb *= scale;
        lo4[e] = a * c.x + bb * c.y;
        hi4[e] = bb * c.x - a * c.y;
      }
      *reinterpret_cast<float4*>(dp + m0) = make_float4(lo4[0], lo4[1], lo4[2], lo4[3]);
      *reinterpret_cast<float4*>(dp + m0 + AT_D / 2) = make_float4(hi4[0], hi4[1], hi4[2], hi4[3]);
    }
    return;
  }
  float* op = ws_dq + (int64_t(split) * B * T * Hq + grow) * AT_D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<float4*>(op + 16 * dt + 4 * g4) = make_float4(dqT[dt][0], dqT[dt][1], dqT[dt][2], dqT[dt][3]);
}

// dq = R(-pos_q) (scale * sum over splits of the partial dQ_rot), one thread per (row, pair m)
__global__ void attn_bwd_dq_sum_kernel(const float* __restrict__ ws_dq, int n_splits, int64_t rows, int T, int Hq,
                                       int d, int L_loc, int qpo, const float2* __restrict__ tab, int P, float scale,
                                       float* __restrict__ dq) {
  const int half = d / 2;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * half) return;
  const int64_t r = i / half;
  const int m = int(i % half);
  float a = 0.f, bb = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    a += ws_dq[(s * rows + r) * d + m];
    bb += ws_dq[(s * rows + r) * d + m + half];
  }
  a *= scale;
  bb *= scale;
  const int t = int((r / Hq) % T);
  int pq = qpo + L_loc - T + t;
  pq = pq < 0 ? 0 : (pq >= P ? P - 1 : pq);
  const float2 c = tab[int64_t(pq) * half + m];
  dq[r * d + m] = a * c.x + bb * c.y;
  dq[r * d + m + half] = bb * c.x - a * c.y;
}

// ---------------------------------------------------------------- vector path
// float32 or any even d: dQ one workgroup per query row, dK/dV one
// workgroup per (query, KV head, key); float32 arithmetic throughout.
template <int DT>
__device__ __forceinline__ float rot_dot(const typename Elem<DT>::T* kp, const float2* cs, const float* qr, int half,
                                         int lo, int step) {
  float dot = 0.f;
  for (int m = lo; m < half; m += step) {
    const float k1 = Elem<DT>::load(kp, m), k2 = Elem<DT>::load(kp, m + half);
    const float2 c = cs[m];
    dot += qr[m] * (k1 * c.x - k2 * c.y) + qr[m + half] * (k2 * c.x + k1 * c.y);
  }
  return dot;
}

template <int DT>
__global__ __launch_bounds__(AT_VEC_THREADS) void attn_bwd_vec_dq_kernel(
    const typename Elem<DT>::T* __restrict__ q, int B, int T, int Hq, int Hkv, int d,
    const typename Elem<DT>::T* __restrict__ k_bar, const typename Elem<DT>::T* __restrict__ v_bar, int64_t ctx_rows,
    const int32_t* __restrict__ ctx_row, const int32_t* __restrict__ ctx_pos, const int32_t* __restrict__ ctx_len,
    int max_ctx, const typename Elem<DT>::T* __restrict__ k_loc, const typename Elem<DT>::T* __restrict__ v_loc,
    int L_loc, int qpo, const float2* __restrict__ tab, int P, float sm_scale, const float* __restrict__ lse,
    const float* __restrict__ Dv, const float* __restrict__ dout, float* __restrict__ dq) {
  using E = Elem<DT>;
  extern __shared__ float bsm[];
  float* qr = bsm;                  // [d] rotated query
  float* red = bsm + d;             // [AT_VEC_THREADS]
  float* dsv = red + AT_VEC_THREADS;   // [n_keys]
  const int64_t row = blockIdx.x;
  const int hq = int(row % Hq), t = int((row / Hq) % T), b = int(row / (int64_t(Hq) * T));
  const int G = Hq / Hkv, g = hq / G, half = d / 2;
  const int horizon = L_loc - T + t;
  int pq = qpo + L_loc - T + t;
  pq = pq < 0 ? 0 : (pq >= P ? P - 1 : pq);
  for (int m = threadIdx.x; m < half; m += AT_VEC_THREADS) {
    const float a = E::load(q + row * d, m), bb = E::load(q + row * d, m + half);
    const float2 c = tab[int64_t(pq) * half + m];
    qr[m] = a * c.x - bb * c.y;
    qr[m + half] = bb * c.x + a * c.y;
  }
  __syncthreads();
  const int ctxl = min(max(ctx_len[b], 0), max_ctx);
  const int n_keys = ctxl + L_loc;
  const float l_nat = lse[row] * (1.f / BW_LOG2E), D = Dv[row];
  for (int j = threadIdx.x; j < n_keys; j += AT_VEC_THREADS) {
    const BwKey ks = bw_key(j, b, ctxl, n_keys, max_ctx, L_loc, qpo, ctx_pos, P, ctx_row, ctx_rows);
    float ds = 0.f;
    if (!ks.local || int(ks.row - int64_t(b) * L_loc) <= horizon) {
      const typename E::T* kp = (ks.local ? k_loc : k_bar) + (ks.row * Hkv + g) * d;
      const typename E::T* vp = (ks.local ? v_loc : v_bar) + (ks.row * Hkv + g) * d;
      const float p = expf(rot_dot<DT>(kp, tab + int64_t(ks.pos) * half, qr, half, 0, 1) * sm_scale - l_nat);
      float dp = 0.f;
      for (int e = 0; e < d; ++e) dp += dout[row * d + e] * E::load(vp, e);
      ds = p * (dp - D);
    }
    dsv[j] = ds;
  }
  __syncthreads();
  for (int m = threadIdx.x; m < half; m += AT_VEC_THREADS) {
    float a = 0.f, bb = 0.f;
    for (int j = 0; j < n_keys; ++j) {
      const float ds = dsv[j];
      if (ds == 0.f) continue;
      const BwKey ks = bw_key(j, b, ctxl, n_keys, max_ctx, L_loc, qpo, ctx_pos, P, ctx_row, ctx_rows);
      const typename E::T* kp = (ks.local ? k_loc : k_bar) + (ks.row * Hkv + g) * d;
      const float2 c = tab[int64_t(ks.pos) * half + m];
      const float k1 = E::load(kp, m), k2 = E::load(kp, m + half);
      a += ds * (k1 * c.x - k2 * c.y);
      bb += ds * (k2 * c.x + k1 * c.y);
    }
    a *= sm_scale;
    bb *= sm_scale;
    const float2 c = tab[int64_t(pq) * half + m];
    dq[row * d + m] = a * c.x + bb * c.y;
    dq[row * d + m + half] = bb * c.x - a * c.y;
  }
}

template <int DT>
__global__ __launch_bounds__(AT_VEC_THREADS) void attn_bwd_vec_dkdv_kernel(
    const typename Elem<DT>::T* __restrict__ q, int B, int T, int Hq, int Hkv, int d,
    const typename Elem<DT>::T* __restrict__ k_bar, const typename Elem<DT>::T* __restrict__ v_bar, int64_t ctx_rows,
    const int32_t* __restrict__ ctx_row, const int32_t* __restrict__ ctx_pos, const int32_t* __restrict__ ctx_len,
    int max_ctx, const typename Elem<DT>::T* __restrict__ k_loc, const typename Elem<DT>::T* __restrict__ v_loc,
    int L_loc, int qpo, const float2* __restrict__ tab, int P, float sm_scale, const float* __restrict__ lse,
    const float* __restrict__ Dv, const float* __restrict__ dout, int n_keys_max, float* __restrict__ dk_loc,
    float* __restrict__ dv_loc, float* __restrict__ dk_bar, float* __restrict__ dv_bar) {
  using E = Elem<DT>;
  extern __shared__ float bsm[];
  float* kr = bsm;                  // [d] rotated key
  float* pr = bsm + d;              // [T * G] p of each row
  float* dr = pr + T * (Hq / Hkv);  // [T * G] ds of each row
  const int64_t wg = blockIdx.x;
  const int j = int(wg % n_keys_max);
  const int g = int((wg / n_keys_max) % Hkv);
  const int b = int(wg / (int64_t(n_keys_max) * Hkv));
  const int G = Hq / Hkv, half = d / 2, R = T * G;
  const int ctxl = min(max(ctx_len[b], 0), max_ctx);
  const int n_keys = ctxl + L_loc;
  if (j >= n_keys) return;
  const BwKey ks = bw_key(j, b, ctxl, n_keys, max_ctx, L_loc, qpo, ctx_pos, P, ctx_row, ctx_rows);
  const typename E::T* kp = (ks.local ? k_loc : k_bar) + (ks.row * Hkv + g) * d;
  const typename E::T* vp = (ks.local ? v_loc : v_bar) + (ks.row * Hkv + g) * d;
  const float2* kcs = tab + int64_t(ks.pos) * half;
  for (int m = threadIdx.x; m < half; m += AT_VEC_THREADS) {
    const float k1 = E::load(kp, m), k2 = E::load(kp, m + half);
    kr[m] = k1 * kcs[m].x - k2 * kcs[m].y;
    kr[m + half] = k2 * kcs[m].x + k1 * kcs[m].y;
  }
  __syncthreads();
  const int li = j - ctxl;
  for (int r = threadIdx.x; r < R; r += AT_VEC_THREADS) {
    const int t = r / G, hq = g * G + r % G;
    const int64_t row = (int64_t(b) * T + t) * Hq + hq;
    float p = 0.f, ds = 0.f;
    if (j < ctxl || li <= L_loc - T + t) {
      int pq = qpo + L_loc - T + t;
      pq = pq < 0 ? 0 : (pq >= P ? P - 1 : pq);
      const float2* qcs = tab + int64_t(pq) * half;
      float dot = 0.f;
      for (int m = 0; m < half; ++m) {
        const float a = E::load(q + row * d, m), bb = E::load(q + row * d, m + half);
        dot += (a * qcs[m].x - bb * qcs[m].y) * kr[m] + (bb * qcs[m].x + a * qcs[m].y) * kr[m + half];
      }
      p = expf(dot * sm_scale - lse[row] * (1.f / BW_LOG2E));
      float dp = 0.f;
      for (int e = 0; e < d; ++e) dp += dout[row * d + e] * E::load(vp, e);
      ds = p * (dp - Dv[row]);
    }
    pr[r] = p;
    dr[r] = ds;
  }
  __syncthreads();
  for (int m = threadIdx.x; m < half; m += AT_VEC_THREADS) {
    float a = 0.f, bb = 0.f, va = 0.f, vb = 0.f;
    for (int r = 0; r < R; ++r) {
      const int t = r / G, hq = g * G + r % G;
      const int64_t row = (int64_t(b) * T + t) * Hq + hq;
      va += pr[r] * dout[row * d + m];
      vb += pr[r] * dout[row * d + m + half];
      const float ds = dr[r];
      if (ds == 0.f) continue;
      int pq = qpo + L_loc - T + t;
      pq = pq < 0 ? 0 : (pq >= P ? P - 1 : pq);
      const float2 c = tab[int64_t(pq) * half + m];
      const float x = E::load(q + row * d, m), y = E::load(q + row * d, m + half);
      a += ds * (x * c.x - y * c.y);
      bb += ds * (y * c.x + x * c.y);
    }
    a *= sm_scale;
    bb *= sm_scale;
    const float2 c = kcs[m];
    const float ka = a * c.x + bb * c.y, kb = bb * c.x - a * c.y;
    if (ks.local) {
      const int64_t o = (ks.row * Hkv + g) * d;
      dk_loc[o + m] = ka;
      dk_loc[o + m + half] = kb;
      dv_loc[o + m] = va;
      dv_loc[o + m + half] = vb;
    } else {
      const int64_t o = (ks.row * Hkv + g) * d;
      unsafeAtomicAdd(dk_bar + o + m, ka);
      unsafeAtomicAdd(dk_bar + o + m + half, kb);
      unsafeAtomicAdd(dv_bar + o + m, va);
      unsafeAtomicAdd(dv_bar + o + m + half, vb);
    }
  }
}

// ---------------------------------------------------------------- plan
struct BwdPlan {
  bool mfma;
  size_t fwd_bytes, out_bytes, row_bytes, bf_bytes, dq_bytes, part_bytes, key_bytes;
  int n_rg, n_splits, n_kb, rt_per, n_items;
};

static BwdPlan bwd_plan(int dtype, int B, int T, int Hq, int Hkv, int d, int max_ctx, int L_loc, int qpo) {
  BwdPlan p{};
  const int G = Hq / Hkv;
  p.mfma = dtype == MSA_BF16 && d == AT_D && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
  p.fwd_bytes = align_up(msa_sparse_attn_workspace(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, qpo), 256);
  const int64_t rows = int64_t(B) * T * Hq;
  p.out_bytes = align_up(size_t(rows) * d * 4, 256);
  p.row_bytes = align_up(size_t(rows) * 4, 256);                // lse, D
  p.bf_bytes = p.mfma ? align_up(size_t(rows) * d * 2, 256) : 0;  // qs16, do16
  if (p.mfma) {
    const int n_rt = (T * G + 15) / 16;
    p.n_rg = (n_rt + BW_WAVES - 1) / BW_WAVES;
    const int64_t units = int64_t(B) * Hkv * p.n_rg;
    const int64_t n_keys_max = int64_t(max_ctx) + L_loc;
    int64_t s = (256 + units - 1) / units;
    s = std::max<int64_t>(1, std::min<int64_t>(s, (n_keys_max + 127) / 128));
    p.n_splits = int(s);
    p.key_bytes = align_up(size_t(B) * size_t(n_keys_max) * Hkv * d * 2, 256);   // krot, vg
    p.dq_bytes = align_up(size_t(p.n_splits) * rows * d * 4, 256);
    p.n_kb = int((n_keys_max + 16 * BW_WAVES - 1) / (16 * BW_WAVES));
    // dK/dV: the visible row tiles of every key block in ranges of rt_per
    // tiles, sized for about 1,024 workgroups (four per CU), at most 8 ranges
    // per block (the partial sums a key carries)
    int64_t vis = 0;
    for (int kb = 0; kb < p.n_kb; ++kb) vis += n_rt - bw_rt_min(kb, max_ctx, L_loc, T, G);
    vis *= int64_t(B) * Hkv;
    p.rt_per = int(std::max<int64_t>({(vis + 1023) / 1024, (n_rt + 7) / 8, 1}));
    p.n_items = 0;
    for (int kb = 0; kb < p.n_kb; ++kb) p.n_items += bw_n_ranges(kb, max_ctx, L_loc, T, G, n_rt, p.rt_per);
    const int max_nr = (n_rt + p.rt_per - 1) / p.rt_per;
    p.part_bytes = align_up(size_t(max_nr) * B * size_t(p.n_kb) * BW_WAVES * 16 * Hkv * d * 4, 256);
  }
  return p;
}

}  // namespace msa

extern "C" size_t msa_sparse_attn_backward_workspace(int dtype, int B, int T, int Hq, int Hkv, int d, int max_ctx,
                                                     int L_loc, int q_pos_offset) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 2 || max_ctx < 0 || L_loc < 1 || q_pos_offset < 0 || Hq % Hkv)
    return 0;
  const msa::BwdPlan p = msa::bwd_plan(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset);
  return p.fwd_bytes + p.out_bytes + 2 * p.row_bytes + 2 * p.bf_bytes + p.dq_bytes + 2 * p.part_bytes +
         2 * p.key_bytes;
}

extern "C" int msa_sparse_attn_backward(int dtype, const void* q, int B, int T, int Hq, int Hkv, int d,
                                        const void* k_bar, const void* v_bar, int64_t n_chunks, const int32_t* ctx_row,
                                        const int32_t* ctx_pos, const int32_t* ctx_len, int max_ctx,
                                        const void* k_loc, const void* v_loc, int L_loc, int q_pos_offset,
                                        float rope_base, const float* rope_table, int rope_table_rows, float sm_scale,
                                        const float* dout, float* dq, float* dk_loc, float* dv_loc, float* dk_bar,
                                        float* dv_bar, void* ws, size_t ws_bytes, void* stream) {
  using namespace msa;
  const std::string fn = "msa_sparse_attn_backward";
  MSA_REQUIRE(ctx_row && dout && dq && dk_loc && dv_loc && dk_bar && dv_bar, MSA_ERR_INVALID_ARG,
              fn + ": NULL pointer");
  MSA_REQUIRE(n_chunks >= 1 && n_chunks <= INT32_MAX, MSA_ERR_INVALID_ARG, fn + ": n_chunks must lie in [1, 2^31)");
  MSA_REQUIRE(B >= 1 && T >= 1 && Hq >= 1 && Hkv >= 1 && d >= 2 && max_ctx >= 1 && L_loc >= 1 && Hq % Hkv == 0,
              MSA_ERR_INVALID_ARG, fn + ": bad sizes");
  const BwdPlan p = bwd_plan(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset);
  const size_t need =
      p.fwd_bytes + p.out_bytes + 2 * p.row_bytes + 2 * p.bf_bytes + p.dq_bytes + 2 * p.part_bytes + 2 * p.key_bytes;
  MSA_REQUIRE(ws && ws_bytes >= need, MSA_ERR_WORKSPACE, fn + ": workspace too small");
  MSA_REQUIRE(uintptr_t(dout) % 16 == 0, MSA_ERR_INVALID_ARG, fn + ": dout must be 16-byte aligned");
  if (!p.mfma)
    MSA_REQUIRE(size_t(d) + AT_VEC_THREADS + size_t(max_ctx) + L_loc <= 16384, MSA_ERR_UNSUPPORTED,
                fn + ": too many keys for the vector path");
  char* w = static_cast<char*>(ws);
  float* out = reinterpret_cast<float*>(w + p.fwd_bytes);
  float* lse = reinterpret_cast<float*>(w + p.fwd_bytes + p.out_bytes);
  float* Dv = reinterpret_cast<float*>(w + p.fwd_bytes + p.out_bytes + p.row_bytes);
  uint16_t* qs16 = reinterpret_cast<uint16_t*>(w + p.fwd_bytes + p.out_bytes + 2 * p.row_bytes);
  uint16_t* do16 = reinterpret_cast<uint16_t*>(w + p.fwd_bytes + p.out_bytes + 2 * p.row_bytes + p.bf_bytes);
  float* ws_dq = reinterpret_cast<float*>(w + p.fwd_bytes + p.out_bytes + 2 * p.row_bytes + 2 * p.bf_bytes);
  float* part_k = reinterpret_cast<float*>(reinterpret_cast<char*>(ws_dq) + p.dq_bytes);
  float* part_v = reinterpret_cast<float*>(reinterpret_cast<char*>(part_k) + p.part_bytes);
  uint16_t* krot = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(part_v) + p.part_bytes);
  uint16_t* vgat = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(krot) + p.key_bytes);
  // every argument the forward shares is checked before any launch
  {
    const int rc = sparse_attn(fn, dtype, q, B, T, Hq, Hkv, d, k_bar, v_bar, ctx_row, n_chunks, ctx_pos, ctx_len,
                               max_ctx, k_loc, v_loc, L_loc, q_pos_offset, rope_base, rope_table, rope_table_rows,
                               sm_scale, out, lse, ws, p.fwd_bytes, stream, nullptr, nullptr, 0, true);
    if (rc != MSA_OK) return rc;
  }
  hipStream_t s = as_stream(stream);
  const int P = rope_rows(max_ctx, L_loc, q_pos_offset);
  if (!rope_table) {
    // the RoPE rows at the start of the forward's workspace, before the keys are prepared
    const int rc = msa_rope_table(P, d, rope_base, static_cast<float*>(ws), stream);
    if (rc != MSA_OK) return rc;
    rope_table = static_cast<const float*>(ws);
    rope_table_rows = P;
  }
  const float2* tab = reinterpret_cast<const float2*>(rope_table);
  const int KMK = max_ctx + L_loc;   // keys per query in the prepared key buffers
  if (p.mfma) {
    // every key of every query rotated once, in key order: the forward below
    // and both backward kernels read these
    const int64_t n = int64_t(B) * KMK * Hkv * 8;
    hipLaunchKernelGGL(bwd_keys_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, B, KMK, Hkv,
                       static_cast<const uint16_t*>(k_bar), static_cast<const uint16_t*>(v_bar), n_chunks, ctx_row,
                       ctx_pos, ctx_len, max_ctx, static_cast<const uint16_t*>(k_loc),
                       static_cast<const uint16_t*>(v_loc), L_loc, q_pos_offset, tab, P, krot, vgat);
    MSA_LAUNCH_CHECK();
  }
  // the forward with the per-row log-sum-exp; on the MFMA path it may also
  // prepare the rows (D, bf16 dO and rotated query)
  BwdPrep prep;
  prep.dout = dout;
  prep.Dv = Dv;
  prep.qs16 = qs16;
  prep.do16 = do16;
  prep.krot = krot;
  prep.vg = vgat;
  prep.km = KMK;
  bool prep_done = false;
  const int rc = sparse_attn(fn, dtype, q, B, T, Hq, Hkv, d, k_bar, v_bar, ctx_row, n_chunks, ctx_pos, ctx_len,
                             max_ctx, k_loc, v_loc, L_loc, q_pos_offset, rope_base, rope_table, rope_table_rows,
                             sm_scale, out, lse, ws, p.fwd_bytes, stream, p.mfma ? &prep : nullptr, &prep_done);
  if (rc != MSA_OK) return rc;
  const int64_t rows = int64_t(B) * T * Hq;
  const int G = Hq / Hkv;
  const unsigned prep_grid = unsigned((rows + BW_WAVES - 1) / BW_WAVES);
  if (p.mfma) {
    if (!prep_done) {
      hipLaunchKernelGGL(bwd_prep128_kernel, dim3(unsigned((rows * 16 + BW_THREADS - 1) / BW_THREADS)),
                         dim3(BW_THREADS), 0, s, static_cast<const uint16_t*>(q), T, Hq, L_loc, q_pos_offset, tab, P,
                         sm_scale * BW_LOG2E, out, dout, rows, Dv, qs16, do16);
      MSA_LAUNCH_CHECK();
    }
    const dim3 kgrid(unsigned(int64_t(B) * Hkv * p.n_items)),
        qgrid(unsigned(int64_t(B) * Hkv * p.n_rg * p.n_splits));
#define BW_LAUNCH(GV)                                                                                              \
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<GV>), kgrid, dim3(BW_THREADS), 0, s, B, T, Hq, Hkv, krot, vgat, KMK,   \
                     ctx_len, max_ctx, L_loc, qs16, do16, lse, Dv, p.n_kb, p.rt_per, p.n_items, part_k, part_v);    \
  MSA_LAUNCH_CHECK();                                                                                              \
  hipLaunchKernelGGL((attn_bwd_dq_kernel<GV>), qgrid, dim3(BW_THREADS), 0, s, B, T, Hq, Hkv, krot, vgat, KMK,     \
                     ctx_len, max_ctx, L_loc, qs16, do16, lse, Dv, p.n_rg, p.n_splits, ws_dq, tab, P, q_pos_offset, \
                     sm_scale, p.n_splits == 1 ? dq : nullptr)
    switch (G) {
      case 1: BW_LAUNCH(1); break;
      case 2: BW_LAUNCH(2); break;
      case 4: BW_LAUNCH(4); break;
      case 8: BW_LAUNCH(8); break;
      default: BW_LAUNCH(16); break;
    }
#undef BW_LAUNCH
    MSA_LAUNCH_CHECK();
    {
      // every key sums the partials of its block's row ranges
      const int KM = p.n_kb * BW_WAVES * 16;
      const int64_t nr = int64_t(B) * KM * Hkv * 16;
      hipLaunchKernelGGL(attn_bwd_dkdv_reduce_kernel, dim3(unsigned((nr + 255) / 256)), dim3(256), 0, s, part_k,
                         part_v, T, G, p.rt_per, B, KM, Hkv, L_loc, q_pos_offset, ctx_row, n_chunks, ctx_pos, ctx_len,
                         max_ctx, tab, P, dk_loc, dv_loc, dk_bar, dv_bar);
      MSA_LAUNCH_CHECK();
    }
    if (p.n_splits > 1) {   // one split: the dQ kernel wrote dq itself
      const int64_t n = rows * (d / 2);
      hipLaunchKernelGGL(attn_bwd_dq_sum_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, ws_dq, p.n_splits,
                         rows, T, Hq, d, L_loc, q_pos_offset, tab, P, sm_scale, dq);
      MSA_LAUNCH_CHECK();
    }
    return MSA_OK;
  }
  const int n_keys_max = max_ctx + L_loc;
  const size_t qsm = (size_t(d) + AT_VEC_THREADS + size_t(n_keys_max)) * sizeof(float);
  const size_t ksm = (size_t(d) + 2 * size_t(T) * G) * sizeof(float);
  MSA_REQUIRE(ksm <= 65536, MSA_ERR_UNSUPPORTED, fn + ": too many query rows for the vector path");
#define BV_LAUNCH(DTV, TY)                                                                                          \
  hipLaunchKernelGGL((bwd_prep_kernel<DTV>), dim3(prep_grid), dim3(BW_THREADS), 0, s, out, dout, d, rows, Dv);     \
  MSA_LAUNCH_CHECK();                                                                                               \
  hipLaunchKernelGGL((attn_bwd_vec_dq_kernel<DTV>), dim3(unsigned(rows)), dim3(AT_VEC_THREADS), qsm, s,             \
                     static_cast<const TY*>(q), B, T, Hq, Hkv, d, static_cast<const TY*>(k_bar),                    \
                     static_cast<const TY*>(v_bar), n_chunks, ctx_row, ctx_pos, ctx_len, max_ctx,                   \
                     static_cast<const TY*>(k_loc), static_cast<const TY*>(v_loc), L_loc, q_pos_offset, tab, P,     \
                     sm_scale, lse, Dv, dout, dq);                                                                  \
  MSA_LAUNCH_CHECK();                                                                                               \
  hipLaunchKernelGGL((attn_bwd_vec_dkdv_kernel<DTV>), dim3(unsigned(int64_t(B) * Hkv * n_keys_max)),                \
                     dim3(AT_VEC_THREADS), ksm, s, static_cast<const TY*>(q), B, T, Hq, Hkv, d,                     \
                     static_cast<const TY*>(k_bar), static_cast<const TY*>(v_bar), n_chunks, ctx_row, ctx_pos,      \
                     ctx_len, max_ctx, static_cast<const TY*>(k_loc), static_cast<const TY*>(v_loc), L_loc,         \
                     q_pos_offset, tab, P, sm_scale, lse, Dv, dout, n_keys_max, dk_loc, dv_loc, dk_bar, dv_bar)
  if (dtype == MSA_BF16) {
    BV_LAUNCH(MSA_BF16, uint16_t);
  } else {
    BV_LAUNCH(MSA_F32, float);
  }
#undef BV_LAUNCH
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}
