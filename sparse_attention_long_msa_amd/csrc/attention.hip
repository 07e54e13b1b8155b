// Stage 3 sparse attention over [retrieved pooled K/V ; local K/V] with
// document-wise RoPE applied on the fly.
// (MSA README, Overall Design > Architecture: the chosen documents' pooled
//  K/V are placed ahead of the query's own recent K/V, and each generated
//  token attends over both;
//  under the parallel (document-wise) RoPE item every document restarts at
//  position 0; under the global RoPE item the query starts at index k.  Paper note,
//  Document-wise RoPE.)
//
// Keys of query b: context entries e < ctx_len[b] (position ctx_pos[b,e],
// visible to every token) then local tokens i < L_loc (position
// q_pos_offset + i, causal: token t sees i <= L_loc - T + t).
//
// bf16 path (d = 128): flash-decoding.  One wave owns (query b, KV head g,
// 16 query rows = (token, head-in-group) pairs, one key split).  Per step of
// 32 keys: K rows are the A operand of v_mfma_f32_16x16x32_bf16 (loaded
// from HBM, rotated in registers), the rotated query the B operand, giving
// S^T[key][row]; the online softmax runs per column (one lane per row);
// P^T goes straight from the accumulator into the B operand of the PV
// product O^T = V^T P^T, whose A operand is the V tile transposed through
// LDS.  Splits are merged by a combine kernel.  RoPE angles come from a
// cos/sin table computed in float64 per call.
#include <algorithm>
#include <mutex>

#include "attn_common.h"

namespace msa {

// tab[p][m] = (cos, sin)(p * base^(-2m/d)), angle formed and reduced in float64
__global__ void rope_table_kernel(float2* __restrict__ tab, int P, int half, double base, int d) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(P) * half) return;
  const int p = int(i / half), m = int(i % half);
  const double theta = pow(base, -2.0 * double(m) / double(d));
  double sn, cs;
  sincos(double(p) * theta, &sn, &cs);
  tab[i] = make_float2(float(cs), float(sn));
}

// ---------------------------------------------------------------- decode (one row tile)
// One workgroup per (query b, key split, group of up to 4 KV heads); wave w
// owns KV head g = 4 * hg + w and the (at most 16) query rows of that head.
// The RoPE rows of the step's 32 keys are the same for every head, so the
// workgroup stages them once in LDS; each wave streams its own head's K and
// V.  The next step's K, V and RoPE rows are loaded while the current step
// is computed.  Four waves per workgroup (two workgroups per CU) keep the
// per-step barrier that publishes the shared rows to a small group.

constexpr int DC_TAB_STRIDE = 528;                 // bytes per key row of (cos, sin) in LDS (512 + pad)
constexpr int DC_TAB_BYTES = 32 * DC_TAB_STRIDE;

constexpr int DC_WAVES = 4;                        // KV heads (waves) per workgroup; two workgroups per CU
constexpr int DC_THREADS = 64 * DC_WAVES;
constexpr int DC_TAB_PT = 32 * 32 / DC_THREADS;    // RoPE-row pieces staged per thread
static_assert(DC_TAB_PT * DC_THREADS == 32 * 32, "the threads cover the step's RoPE rows");

struct DcRegs {
  uint4 k[2][4];     // K rows (two 16-key tiles) of this wave's head
};
struct VRegs {
  uint4 v[2][4];     // V rows: key 16*rho + 4*g4 + i, dims 8*lc .. +7
};
struct TabRegs {
  uint4 t[DC_TAB_PT];   // this thread's pieces of the step's RoPE rows
};



template <int G, bool IDX>
__global__ __launch_bounds__(DC_THREADS, 2) void attn_decode_kernel(
    const uint16_t* __restrict__ q, int B, int T, int Hq, int Hkv, const uint16_t* __restrict__ k_ctx,
    const uint16_t* __restrict__ v_ctx, const int32_t* __restrict__ ctx_pos, const int32_t* __restrict__ ctx_len,
    int max_ctx, const uint16_t* __restrict__ k_loc, const uint16_t* __restrict__ v_loc, int L_loc, int qpo,
    const int32_t* __restrict__ ctx_row_in, int64_t ctx_rows, const float2* __restrict__ tab, int P, float scale_log2,
    uint16_t* __restrict__ ws_o, float4* __restrict__ ws_ml, int n_splits, int n_hg, int part, int split_base) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int32_t* __restrict__ ctx_row = IDX ? ctx_row_in : nullptr;
  const int nw = blockDim.x / 64;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int lc = lane % 16, g4 = lane / 16;
  unsigned char* tabs = smem;                                     // [2][32 keys][DC_TAB_STRIDE]
  unsigned char* vrm = smem + 2 * DC_TAB_BYTES + size_t(wave) * AT_V_BYTES;   // this wave's V rows

  int64_t wg = blockIdx.x;
  const int split = int(wg % n_splits);
  wg /= n_splits;
  const int hg = int(wg % n_hg);
  const int b = int(wg / n_hg);
  const int g = hg * DC_WAVES + wave;
  const bool head_ok = g < Hkv;
  const int gg = head_ok ? g : 0;
  const int64_t kv_stride = int64_t(Hkv) * AT_D;

  const int r = lc;                       // the only row tile
  const int t = r / G, hh = r % G;
  const bool row_ok = head_ok && t < T;
  const int tt = row_ok ? t : 0;
  const int hq = gg * G + hh;
  const int horizon = L_loc - T + t;

  bf16x8 bq[4];
  {
    uint4 qv[4];
    const uint16_t* qp = q + ((int64_t(b) * T + tt) * Hq + hq) * AT_D + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qv[kk] = *reinterpret_cast<const uint4*>(qp + 32 * kk);
    int pq = qpo + L_loc - T + tt;
    pq = pq < 0 ? 0 : (pq >= P ? P - 1 : pq);
    rope_rotate(qv, tab + int64_t(pq) * (AT_D / 2), g4);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) bq[kk] = __builtin_bit_cast(bf16x8, row_ok ? qv[kk] : make_uint4(0, 0, 0, 0));
  }

  // the keys of this launch: all, the local window only (the context is not
  // read, not even its length) or the context only
  const int ctxl = part == MSA_ATTN_PART_LOCAL ? 0 : min(max(ctx_len[b], 0), max_ctx);
  const int n_keys = part == MSA_ATTN_PART_CONTEXT ? ctxl : ctxl + L_loc;
  // this query's keys split evenly over the n_splits workgroups (32-key steps)
  const int kps = ((n_keys + n_splits - 1) / n_splits + 31) / 32 * 32;
  const int j_begin = split * kps;
  const int j_end = min(n_keys, j_begin + kps);
  const int nthr = nw * 64;
  // a step whose 32 keys are all local tokens addresses them affinely
  auto all_local = [&](int j0) { return j0 >= ctxl && j0 + 32 <= n_keys; };

  const CtxCache cc = stage_ctx(reinterpret_cast<int2*>(smem + 2 * DC_TAB_BYTES + size_t(nw) * AT_V_BYTES), AT_CIDX, b, j_begin,
                                j_end, ctxl, max_ctx, ctx_pos, P, ctx_row, ctx_rows, tid, nthr);
  __syncthreads();
  // Addresses are formed under the (uniform) all-local test, the loads come
  // after it: every path issues the same loads, so the compiler's waits on
  // the load counter stay partial.
  auto load_k = [&](int j0, DcRegs& R) {
    const uint16_t* kp[2];
    if (all_local(j0)) {
      const uint16_t* kb = k_loc + (int64_t(b) * L_loc + (j0 - ctxl)) * kv_stride + int64_t(gg) * AT_D + 8 * g4;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) kp[tau] = kb + int32_t(16 * tau + lc) * int32_t(kv_stride);
    } else {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const KeySrc ks = key_src(j0 + 16 * tau + lc, b, ctxl, n_keys, max_ctx, L_loc, qpo, ctx_pos, P, ctx_row, ctx_rows, cc);
        kp[tau] = (ks.local ? k_loc : k_ctx) + ks.row * kv_stride + int64_t(gg) * AT_D + 8 * g4;
      }
    }
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) R.k[tau][kk] = load_global(kp[tau] + 32 * kk);
  };
  auto load_v = [&](int j0) {
    const uint16_t* vp[2][4];
    if (all_local(j0)) {
      const uint16_t* vb = v_loc + (int64_t(b) * L_loc + (j0 - ctxl)) * kv_stride + int64_t(gg) * AT_D + 8 * lc;
#pragma unroll
      for (int rho = 0; rho < 2; ++rho)
#pragma unroll
        for (int i = 0; i < 4; ++i) vp[rho][i] = vb + int32_t(16 * rho + 4 * g4 + i) * int32_t(kv_stride);
    } else {
#pragma unroll
      for (int rho = 0; rho < 2; ++rho)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const KeySrc ks = key_src(j0 + 16 * rho + 4 * g4 + i, b, ctxl, n_keys, max_ctx, L_loc, qpo, ctx_pos, P,
                                    ctx_row, ctx_rows, cc);
          vp[rho][i] = (ks.local ? v_loc : v_ctx) + ks.row * kv_stride + int64_t(gg) * AT_D + 8 * lc;
        }
    }
    VRegs v;
#pragma unroll
    for (int rho = 0; rho < 2; ++rho)
#pragma unroll
      for (int i = 0; i < 4; ++i) v.v[rho][i] = load_stream(vp[rho][i]);
    return v;
  };
  // The step's 32 RoPE rows (32 x 32 pieces of 16 bytes), DC_TAB_PT pieces per
  // thread, through registers into a padded LDS buffer
  auto load_tab = [&](int j0) {
    TabRegs t;
    const bool loc = all_local(j0);
#pragma unroll
    for (int u = 0; u < DC_TAB_PT; ++u) {
      const int piece = tid + u * DC_THREADS;
      const int key = piece / 32;
      const int pos = loc ? qpo + j0 - ctxl + key
                          : key_src(j0 + key, b, ctxl, n_keys, max_ctx, L_loc, qpo, ctx_pos, P, ctx_row, ctx_rows, cc).pos;
      t.t[u] = reinterpret_cast<const uint4*>(tab + int64_t(pos) * (AT_D / 2))[piece % 32];
    }
    return t;
  };
  auto store_tab = [&](const TabRegs& t, unsigned char* buf) {
#pragma unroll
    for (int u = 0; u < DC_TAB_PT; ++u) {
      const int piece = tid + u * DC_THREADS;
      *reinterpret_cast<uint4*>(buf + (piece / 32) * DC_TAB_STRIDE + (piece % 32) * 16) = t.t[u];
    }
  };
  // V rows stay row-major in LDS; the PV operand is read with transpose loads
  auto store_v = [&](const VRegs& v) {
#pragma unroll
    for (int rho = 0; rho < 2; ++rho)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(vrm + (16 * rho + 4 * g4 + i) * AT_VS + 16 * lc) = v.v[rho][i];
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Pipeline (per wave; the vector-memory counter completes loads in issue
  // order): at the top of step s, K(s) is in flight to registers and V(s),
  // RoPE(s) are in LDS.  Step s first requests RoPE(s+1) and V(s+1) into
  // registers, then computes S^T(s), then requests K(s+1) into the registers
  // K(s) just freed, then finishes step s and writes RoPE(s+1) (other LDS
  // buffer) and V(s+1) to LDS.  The closing barrier waits only for LDS
  // traffic, so K(s+1) stays in flight across it and the memory pipe never
  // drains.
  DcRegs R;
  if (j_begin < j_end) {
    const TabRegs t0 = load_tab(j_begin);
    const VRegs v0 = load_v(j_begin);
    load_k(j_begin, R);
    store_tab(t0, tabs);
    store_v(v0);
  }
  lds_barrier();
  // S^T of the step at j0 from K(s) in registers and RoPE(s) in tbuf
  auto score = [&](const unsigned char* tbuf, f32x4 (&s)[2]) {
    // ---- rotate K with the staged RoPE rows, S^T = K_rot . Q_rot^T
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      uint4 kv[4] = {R.k[tau][0], R.k[tau][1], R.k[tau][2], R.k[tau][3]};
      const unsigned char* row = tbuf + (16 * tau + lc) * DC_TAB_STRIDE;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float lo[8], hi[8];
        unpack8(kv[kk], lo);
        unpack8(kv[kk + 2], hi);
        const float4* c4 = reinterpret_cast<const float4*>(row + (32 * kk + 8 * g4) * 8);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float4 cs = c4[e2];
          const float a0 = lo[2 * e2], b0 = hi[2 * e2], a1 = lo[2 * e2 + 1], b1 = hi[2 * e2 + 1];
          lo[2 * e2] = a0 * cs.x - b0 * cs.y;
          hi[2 * e2] = b0 * cs.x + a0 * cs.y;
          lo[2 * e2 + 1] = a1 * cs.z - b1 * cs.w;
          hi[2 * e2 + 1] = b1 * cs.z + a1 * cs.w;
        }
        kv[kk] = pack8(lo);
        kv[kk + 2] = pack8(hi);
      }
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv[kk]), bq[kk], acc, 0, 0, 0);
      s[tau] = acc;
    }
  };
  // mask, online softmax and O^T += V^T . P^T of the step at j0
  auto finish = [&](int j0, const f32x4 (&s)[2]) {
    // ---- mask and online softmax for column lc (base-2 domain)
    float x[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kj = j0 + 16 * tau + 4 * g4 + i;
        const bool vis = row_ok && kj < j_end && (kj < ctxl || kj - ctxl <= horizon);
        x[tau][i] = vis ? s[tau][i] * scale_log2 : -INFINITY;
        mt = fmaxf(mt, x[tau][i]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
    float p[2][4];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[tau][i] = exp2f(x[tau][i] - m_use);
        psum += p[tau][i];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {   // skip the rescale when no row's running max moved
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }
    const bf16x8 pb = __builtin_bit_cast(
        bf16x8, make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                           pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])));
    // ---- O^T += V^T . P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pv_operand(vrm, dt, lane), pb, o[dt], 0, 0, 0);
  };

  int tb = 0;
  int j0 = j_begin;
  // steps with a successor prefetch it unconditionally (straight-line code
  // keeps the compiler's load-counter waits partial); the last step is peeled
  for (; j0 + 32 < j_end; j0 += 32) {
    const TabRegs tn = load_tab(j0 + 32);
    const VRegs vn = load_v(j0 + 32);
    f32x4 s[2];
    score(tabs + tb * DC_TAB_BYTES, s);
    __builtin_amdgcn_sched_barrier(0);   // K(s) is consumed: its registers take K(s+1)
    load_k(j0 + 32, R);
    finish(j0, s);
    // LDS operations of one wave complete in order, so this step's V reads
    // precede the next step's writes to the same buffer; the other RoPE
    // buffer was last read in step s-1, before its closing barrier
    store_tab(tn, tabs + (tb ^ 1) * DC_TAB_BYTES);
    store_v(vn);
    lds_barrier();
    tb ^= 1;
  }
  if (j0 < j_end) {
    f32x4 s[2];
    score(tabs + tb * DC_TAB_BYTES, s);
    finish(j0, s);
  }

  // ---- partial result of this split: O^T[d = 16dt + 4*g4 + i][row lc]
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const int64_t rowid = ((int64_t(split_base + split) * B + b) * T + t) * Hq + hq;
  store_partial(o, m_run, l_run, row_ok, g4, ws_o + rowid * AT_D, ws_ml + rowid);
}

// ---------------------------------------------------------------- prefill (many query rows)
// One workgroup of 8 waves owns (query b, KV head g, row group, key split);
// its waves hold up to 16 row tiles (RTW per wave).  Each 32-key step is
// loaded once by the whole workgroup, rotated once, and staged in LDS as
// K_rot[key][d] (the A operand of S^T = K Q^T) and V^T[d][slot] (the A
// operand of O^T = V^T P^T); the next step's global loads are in flight
// while the current step is computed (two LDS buffers).

constexpr int PF_WAVES = 8;
constexpr int PF_BOTH = 3;   // part value of a one-launch split of both parts (split_base = context splits)
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_KS = 272;                         // bytes per key row of K_rot in LDS (256 + pad)
constexpr int PF_K_BYTES = 32 * PF_KS;
constexpr int PF_BUF = PF_K_BYTES + AT_V_BYTES;    // one step buffer
constexpr int PF_DEPTH = 2;                        // steps whose loads are in flight (even)
constexpr float PF_LAZY = 8.f;                     // running-max slack (base-2 logits)
static_assert(PF_DEPTH % 2 == 0, "step s uses LDS buffer s % 2");

struct PfRegs {
  uint2 klo, khi;     // dims 4x..4x+3 and 64+4x..64+4x+3 of key t/16
  float4 cs0, cs1;    // (cos, sin) of m = 4x..4x+3 at the key's position
  uint4 v;            // V[t/16][8*(t%16) .. +7]
};

// PRE: the keys come already rotated and in key order, k_ctx/v_ctx being
// [B, km, Hkv, d] with key j of query b at row b * km + j (context entries,
// then the local tokens, zero past the query's keys): the prepared keys of the
// backward, so that its forward recompute neither rotates nor looks keys up.
template <int G, int RTW, bool IDX, bool PRE = false>
__global__ __launch_bounds__(PF_THREADS) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, int B, int T, int Hq, int Hkv, const uint16_t* __restrict__ k_ctx,
    const uint16_t* __restrict__ v_ctx, const int32_t* __restrict__ ctx_pos, const int32_t* __restrict__ ctx_len,
    int max_ctx, const uint16_t* __restrict__ k_loc, const uint16_t* __restrict__ v_loc, int L_loc, int qpo,
    const int32_t* __restrict__ ctx_row_in, int64_t ctx_rows, const float2* __restrict__ tab, int P, float scale_log2,
    uint16_t* __restrict__ ws_o, float4* __restrict__ ws_ml, int n_splits, int n_rt, int n_rg, float* __restrict__ out,
    float* __restrict__ lse, int part, int split_base, int km, BwdPrep prep) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int32_t* __restrict__ ctx_row = IDX && !PRE ? ctx_row_in : nullptr;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int lc = lane % 16, g4 = lane / 16;

  int64_t wg = blockIdx.x;
  const int split = int(wg % n_splits);
  wg /= n_splits;
  const int rg = int(wg % n_rg);
  wg /= n_rg;
  const int g = int(wg % Hkv);
  const int b = int(wg / Hkv);
  if (b >= B) return;
  const int64_t kv_stride = int64_t(Hkv) * AT_D;

  // ---- this wave's row tiles: rotated query fragments and row metadata
  bf16x8 bq[RTW][4];
  int trow[RTW], hqrow[RTW], horizon[RTW];
  bool rok[RTW];
#pragma unroll
  for (int i = 0; i < RTW; ++i) {
    const int rt = rg * (PF_WAVES * RTW) + wave + PF_WAVES * i;
    const int r = rt * 16 + lc;
    const int t = r / G;
    rok[i] = rt < n_rt && t < T;
    trow[i] = rok[i] ? t : 0;
    hqrow[i] = g * G + r % G;
    horizon[i] = L_loc - T + t;
    uint4 qv[4];
    const uint16_t* qp = q + ((int64_t(b) * T + trow[i]) * Hq + hqrow[i]) * AT_D + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qv[kk] = *reinterpret_cast<const uint4*>(qp + 32 * kk);
    int pq = qpo + L_loc - T + trow[i];
    pq = pq < 0 ? 0 : (pq >= P ? P - 1 : pq);
    rope_rotate(qv, tab + int64_t(pq) * (AT_D / 2), g4, scale_log2);   // logits come out in the base-2 domain
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) bq[i][kk] = __builtin_bit_cast(bf16x8, rok[i] ? qv[kk] : make_uint4(0, 0, 0, 0));
  }
  // the smallest causal horizon among this wave's rows: a step whose keys all
  // lie within it (and within the split) needs no mask
  int hmin = INT32_MAX;
#pragma unroll
  for (int i = 0; i < RTW; ++i) {
    const int rt = rg * (PF_WAVES * RTW) + wave + PF_WAVES * i;
    if (rt < n_rt) hmin = min(hmin, L_loc - T + (rt * 16) / G);
  }

  // the keys of this launch: all, the local window only (the context is not
  // read, not even its length) or the context only
  // PF_BOTH (one launch, both parts): the first split_base splits take the
  // context keys and the others the local keys, each set split evenly, so the
  // local splits start loading without waiting for the context's length
  int kpart = part, ksplit = split, kn = n_splits;
  if (part == PF_BOTH) {
    const bool c = split < split_base;
    kpart = c ? MSA_ATTN_PART_CONTEXT : MSA_ATTN_PART_LOCAL;
    ksplit = c ? split : split - split_base;
    kn = c ? split_base : n_splits - split_base;
  }
  const int ctxl = kpart == MSA_ATTN_PART_LOCAL ? 0 : min(max(ctx_len[b], 0), max_ctx);
  const int n_keys = kpart == MSA_ATTN_PART_CONTEXT ? ctxl : ctxl + L_loc;
  // this query's keys split evenly over the kn workgroups (32-key steps)
  const int kps = ((n_keys + kn - 1) / kn + 31) / 32 * 32;
  const int j_begin = ksplit * kps;
  const int j_end = min(n_keys, j_begin + kps);

  // cooperative mapping of one 32-key step
  const int lk = tid / 16, lx = tid % 16;     // K: key, 4-dim block; V: key, 8-dim block
  // prepared keys need no index: the cache stays empty
  const CtxCache cc = stage_ctx(reinterpret_cast<int2*>(smem + 2 * size_t(PF_BUF)), PF_CIDX, b, j_begin,
                                PRE ? j_begin : j_end, ctxl, max_ctx, ctx_pos, P, ctx_row, ctx_rows, tid, PF_THREADS);
  __syncthreads();

  // a step whose 32 keys are all local tokens addresses them affinely
  auto all_local = [&](int j0) { return j0 >= ctxl && j0 + 32 <= n_keys; };
  // Addresses are formed under the (uniform) all-local test and the loads
  // come after it, so every path issues the same five loads and the
  // compiler's waits on the load counter stay partial.
  // element offsets of this thread's K/V row and RoPE row for a local key,
  // less the part that depends on the (uniform) step start j0
  const int64_t loc_kv = (int64_t(b) * L_loc - ctxl + lk) * kv_stride + int64_t(g) * AT_D;
  const int64_t loc_tab = int64_t(qpo - ctxl + lk) * (AT_D / 2) + 4 * lx;
  auto load_step = [&](int j0) {
    PfRegs R;
    if constexpr (PRE) {
      // row b * km + j (clamped into the query's rows; keys past n_keys are masked)
      const int64_t off = (int64_t(b) * km + min(j0 + lk, km - 1)) * kv_stride + int64_t(g) * AT_D;
      R.klo = load_global8(k_ctx + off + 4 * lx);
      R.khi = load_global8(k_ctx + off + 4 * lx + 64);
      R.cs0 = R.cs1 = make_float4(0.f, 0.f, 0.f, 0.f);
      R.v = load_global(v_ctx + off + 8 * lx);
      return R;
    }
    const uint16_t* kp;
    const uint16_t* vp;
    const float2* tp;
    if (all_local(j0)) {
      const int64_t off = loc_kv + int64_t(j0) * kv_stride;
      kp = k_loc + off + 4 * lx;
      vp = v_loc + off + 8 * lx;
      tp = tab + loc_tab + int64_t(j0) * (AT_D / 2);
    } else {
      const KeySrc ks = key_src(j0 + lk, b, ctxl, n_keys, max_ctx, L_loc, qpo, ctx_pos, P, ctx_row, ctx_rows, cc);
      const int64_t off = ks.row * kv_stride + int64_t(g) * AT_D;
      kp = (ks.local ? k_loc : k_ctx) + off + 4 * lx;
      vp = (ks.local ? v_loc : v_ctx) + off + 8 * lx;
      tp = tab + int64_t(ks.pos) * (AT_D / 2) + 4 * lx;
    }
    R.klo = load_global8(kp);
    R.khi = load_global8(kp + 64);
    R.cs0 = __builtin_bit_cast(float4, load_global(tp));
    R.cs1 = __builtin_bit_cast(float4, load_global(tp + 2));
    R.v = load_global(vp);
    return R;
  };
  auto store_step = [&](const PfRegs& R, unsigned char* buf) {
    if constexpr (PRE) {   // already rotated: stored as loaded
      unsigned char* krow = buf + lk * PF_KS;
      *reinterpret_cast<uint2*>(krow + 8 * lx) = R.klo;
      *reinterpret_cast<uint2*>(krow + 128 + 8 * lx) = R.khi;
      *reinterpret_cast<uint4*>(buf + PF_K_BYTES + lk * AT_VS + 16 * lx) = R.v;
      return;
    }
    // rotate the 4 (m, m+64) pairs of this thread and store K_rot[key][d]
    const float c[4] = {R.cs0.x, R.cs0.z, R.cs1.x, R.cs1.z};
    const float sn[4] = {R.cs0.y, R.cs0.w, R.cs1.y, R.cs1.w};
    const uint32_t lo[2] = {R.klo.x, R.klo.y}, hi[2] = {R.khi.x, R.khi.y};
    float a[4], bb[4];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      a[2 * e] = __uint_as_float(lo[e] << 16);
      a[2 * e + 1] = __uint_as_float(lo[e] & 0xFFFF0000u);
      bb[2 * e] = __uint_as_float(hi[e] << 16);
      bb[2 * e + 1] = __uint_as_float(hi[e] & 0xFFFF0000u);
    }
    float ra[4], rb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ra[e] = a[e] * c[e] - bb[e] * sn[e];
      rb[e] = bb[e] * c[e] + a[e] * sn[e];
    }
    unsigned char* krow = buf + lk * PF_KS;
    *reinterpret_cast<uint2*>(krow + 8 * lx) = make_uint2(pack_bf16x2(ra[0], ra[1]), pack_bf16x2(ra[2], ra[3]));
    *reinterpret_cast<uint2*>(krow + 128 + 8 * lx) = make_uint2(pack_bf16x2(rb[0], rb[1]), pack_bf16x2(rb[2], rb[3]));
    // V stays row-major; the PV operand is read with transpose loads
    *reinterpret_cast<uint4*>(buf + PF_K_BYTES + lk * AT_VS + 16 * lx) = R.v;
  };

  float m_run[RTW], l_run[RTW];
  f32x4 o[RTW][8];
#pragma unroll
  for (int i = 0; i < RTW; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Online softmax in the base-2 domain with a lazy running max: a row's
  // reference m moves only when a logit exceeds it by more than PF_LAZY, so
  // the accumulators are rescaled rarely; p = 2^(x - m) then stays below
  // 2^PF_LAZY, and the result, normalised by the same sums, is unchanged.
  auto compute_step = [&](int j0, const unsigned char* kb) {
    const unsigned char* vb = kb + PF_K_BYTES;
    const bool full = j0 + 32 <= j_end && j0 + 31 - ctxl <= hmin;   // uniform
    // S^T for both 16-key tiles, for every row tile of this wave
    bf16x8 ka[2][4];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        ka[tau][kk] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(kb + (16 * tau + lc) * PF_KS + 64 * kk + 16 * g4));
    bf16x8 pb[RTW];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
      float x[2][4];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tau][kk], bq[i][kk], acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[tau][e] = acc[e];
      }
      if (!full) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int kj = j0 + 16 * tau + 4 * g4 + e;
            const bool vis = rok[i] && kj < j_end && (kj < ctxl || kj - ctxl <= horizon[i]);
            x[tau][e] = vis ? x[tau][e] : -INFINITY;
          }
      }
      float mt = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const bool grow = mt > m_run[i] + PF_LAZY;   // false while nothing is visible
      if (__ballot(grow)) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[i] - mt) : 1.f;
        m_run[i] = grow ? mt : m_run[i];
        l_run[i] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[i][dt] *= alpha;
      }
      const float m_use = m_run[i] == -INFINITY ? 0.f : m_run[i];
      float p[2][4], psum = 0.f;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[tau][e] = __builtin_amdgcn_exp2f(x[tau][e] - m_use);
          psum += p[tau][e];
        }
      l_run[i] += psum;
      pb[i] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                                                    pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])));
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x8 a = pv_operand(vb, dt, lane);
#pragma unroll
      for (int i = 0; i < RTW; ++i) o[i][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[i], o[i][dt], 0, 0, 0);
    }
  };

  // Pipeline: the loads of the next PF_DEPTH steps are in flight in
  // registers.  Step s writes its registers (rotating K) to LDS buffer s % 2,
  // requests step s + PF_DEPTH into the registers it just freed, meets the
  // workgroup at an LDS-only barrier (loads stay in flight across it) and
  // computes from the buffer.  A buffer is rewritten two steps after it was
  // read, and each wave's read precedes its next barrier, so one barrier per
  // step suffices.  Requests past the last step repeat the last step's
  // addresses (in bounds, never used), which keeps the loop free of branches
  // around loads; steps of the last group past the end skip the compute.
  const int n_steps = j_begin < j_end ? (j_end - j_begin + 31) / 32 : 0;
  auto step_j = [&](int st) { return j_begin + 32 * min(st, n_steps - 1); };
  PfRegs R[PF_DEPTH];
  if (n_steps > 0) {
#pragma unroll
    for (int u = 0; u < PF_DEPTH; ++u) R[u] = load_step(step_j(u));
  }
  for (int s0 = 0; s0 < n_steps; s0 += PF_DEPTH) {
#pragma unroll
    for (int u = 0; u < PF_DEPTH; ++u) {
      unsigned char* buf = smem + (u % 2) * PF_BUF;
      store_step(R[u], buf);
      R[u] = load_step(step_j(s0 + u + PF_DEPTH));
      lds_barrier();
      if (s0 + u < n_steps) compute_step(j_begin + 32 * (s0 + u), buf);
    }
  }

#pragma unroll
  for (int i = 0; i < RTW; ++i) {
    float l = l_run[i];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (n_splits > 1 || part != 0) {
      const int pidx = part == PF_BOTH ? split : split_base + split;   // this workgroup's partial
      const int64_t rowid = ((int64_t(pidx) * B + b) * T + trow[i]) * Hq + hqrow[i];
      store_partial(o[i], m_run[i], l, rok[i], g4, ws_o + rowid * AT_D, ws_ml + rowid);
      continue;
    }
    if (!rok[i]) continue;   // uniform in each row's four lanes
    {
      // one split: the combine's result directly, with its arithmetic
      // (out = O / l, lse = m + log2 l; a row that saw no visible key gets 0, -inf)
      const int64_t row = (int64_t(b) * T + trow[i]) * Hq + hqrow[i];
      const float r = l > 0.f ? 1.f / l : 0.f;
      if (prep.dout) {
        // the backward's row preparation: lane (lc, g4) holds dims 16*dt + 4*g4 + e of
        // the row, and its rotated query's dims 32*kk + 8*g4 .. + 7
        const float* gp = prep.dout + row * AT_D;
        float dacc = 0.f;
        uint2 dpk[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const float4 g = *reinterpret_cast<const float4*>(gp + 16 * dt + 4 * g4);
          const float o0 = o[i][dt][0] * r, o1 = o[i][dt][1] * r, o2 = o[i][dt][2] * r, o3 = o[i][dt][3] * r;
          dacc += o0 * g.x + o1 * g.y + o2 * g.z + o3 * g.w;
          dpk[dt] = make_uint2(pack_bf16x2(g.x, g.y), pack_bf16x2(g.z, g.w));
        }
        dacc += __shfl_xor(dacc, 16);
        dacc += __shfl_xor(dacc, 32);
        if (g4 == 0) prep.Dv[row] = dacc;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<uint2*>(prep.do16 + row * AT_D + 16 * dt + 4 * g4) = dpk[dt];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          *reinterpret_cast<uint4*>(prep.qs16 + row * AT_D + 32 * kk + 8 * g4) = __builtin_bit_cast(uint4, bq[i][kk]);
      } else {
        float* op = out + row * AT_D;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<float4*>(op + 16 * dt + 4 * g4) =
              make_float4(o[i][dt][0] * r, o[i][dt][1] * r, o[i][dt][2] * r, o[i][dt][3] * r);
      }
      if (lse && g4 == 0) lse[row] = l > 0.f ? m_run[i] + __log2f(l) : -INFINITY;
    }
  }
}

// out[b,t,hq,:] = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s, one pass with
// a running maximum; sixteen splits' loads are issued together.  O_s arrives
// as float16 scaled by 2^-c_s (store_partial), so its weight is 2^(m_s + c_s - m).
__global__ void attn_combine_kernel(const uint16_t* __restrict__ ws_o, const float4* __restrict__ ws_ml, int n_splits,
                                    int64_t rows, int d, float* __restrict__ out, float* __restrict__ lse) {
  // one thread per (row, 4 dims); d is a multiple of 4 on this path
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int dq = d / 4;
  if (i >= rows * dq) return;
  const int64_t row = i / dq;
  const int e = int(i % dq) * 4;
  float m = -INFINITY, den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int U = 16;
  for (int s0 = 0; s0 < n_splits; s0 += U) {
    float4 ml[U];
    uint2 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = min(s0 + u, n_splits - 1);
      ml[u] = ws_ml[sp * rows + row];
      v[u] = *reinterpret_cast<const uint2*>(ws_o + (sp * rows + row) * d + e);
      if (s0 + u >= n_splits) ml[u].x = -INFINITY;   // past the last split: weight 0
    }
    float mg = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mg = fmaxf(mg, ml[u].x);
    if (mg == -INFINITY) continue;   // no split so far saw a visible key
    const float a = __builtin_amdgcn_exp2f(m - mg);   // 0 while m is -inf
    den *= a;
    num.x *= a;
    num.y *= a;
    num.z *= a;
    num.w *= a;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = __builtin_amdgcn_exp2f(ml[u].x - mg);           // 0 for a split that saw no visible key
      const float wo = __builtin_amdgcn_exp2f(ml[u].x + ml[u].z - mg);
      const float2 lo = unpack_f16x2(v[u].x), hi = unpack_f16x2(v[u].y);
      den += w * ml[u].y;
      num.x += wo * lo.x;
      num.y += wo * lo.y;
      num.z += wo * hi.x;
      num.w += wo * hi.y;
    }
    m = mg;
  }
  const float r = den > 0.f ? 1.f / den : 0.f;
  *reinterpret_cast<float4*>(out + row * d + e) = make_float4(num.x * r, num.y * r, num.z * r, num.w * r);
  if (lse && e == 0) lse[row] = den > 0.f ? m + __log2f(den) : -INFINITY;
}

// Vector path (float32 or any even d <= 256): one workgroup per (b, t, hq).
// Logits: one wave per key, the lanes over the rotated pairs (m, m + d/2),
// four keys' loads issued before any is used; a wave-wide sum per key.  The
// softmax is taken over the logits in LDS; the value sum gives each wave a
// quarter of the keys (lanes over d, coalesced) and adds the four partial
// rows at the end.
template <int DT>
__global__ __launch_bounds__(AT_VEC_THREADS) void attn_vec_kernel(
    const typename Elem<DT>::T* __restrict__ q, int B, int T, int Hq, int Hkv, int d,
    const typename Elem<DT>::T* __restrict__ k_ctx, const typename Elem<DT>::T* __restrict__ v_ctx,
    const int32_t* __restrict__ ctx_pos, const int32_t* __restrict__ ctx_len, int max_ctx,
    const typename Elem<DT>::T* __restrict__ k_loc, const typename Elem<DT>::T* __restrict__ v_loc, int L_loc,
    int qpo, const int32_t* __restrict__ ctx_row, int64_t ctx_rows, const float2* __restrict__ tab, int P,
    float sm_scale, float* __restrict__ out, float* __restrict__ lse) {
  using E = Elem<DT>;
  constexpr int NW = AT_VEC_THREADS / 64, KU = 4;
  extern __shared__ float vsm[];
  float* qr = vsm;               // [d]
  float* red = vsm + d;          // [AT_VEC_THREADS]
  float* part = red + AT_VEC_THREADS;   // [NW][d]
  float* logit = part + NW * d;  // [n_keys]
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int hq = blockIdx.x % Hq;
  const int t = (blockIdx.x / Hq) % T;
  const int b = blockIdx.x / (Hq * T);
  const int G = Hq / Hkv, g = hq / G, half = d / 2;
  const int horizon = L_loc - T + t;
  int pq = qpo + L_loc - T + t;
  pq = pq < 0 ? 0 : (pq >= P ? P - 1 : pq);
  const typename E::T* qp = q + ((int64_t(b) * T + t) * Hq + hq) * d;
  for (int m = threadIdx.x; m < half; m += AT_VEC_THREADS) {
    const float2 cs = tab[int64_t(pq) * half + m];
    const float x1 = E::load(qp, m), x2 = E::load(qp, m + half);
    qr[m] = x1 * cs.x - x2 * cs.y;
    qr[m + half] = x2 * cs.x + x1 * cs.y;
  }
  __syncthreads();
  const int ctxl = min(max(ctx_len[b], 0), max_ctx);
  const int n_keys = ctxl + L_loc;
  // the rotated query pairs this lane multiplies (d <= 256: at most two)
  float qa[2], qb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = lane + 64 * i;
    qa[i] = m < half ? qr[m] : 0.f;
    qb[i] = m < half ? qr[m + half] : 0.f;
  }
  float mx = -INFINITY;
  for (int j0 = wave * KU; j0 < n_keys; j0 += NW * KU) {
    float k1[KU][2], k2[KU][2];
    float2 cs[KU][2];
    bool ok[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int j = j0 + u;
      const typename E::T* kp = k_loc;
      int pos = 0;
      ok[u] = false;
      if (j < ctxl) {
        kp = k_ctx + (ctx_src_row(int64_t(b) * max_ctx + j, ctx_row, ctx_rows) * Hkv + g) * d;
        pos = ctx_pos[int64_t(b) * max_ctx + j];
        pos = pos < 0 ? 0 : (pos >= P ? P - 1 : pos);
        ok[u] = true;
      } else if (j < n_keys) {
        const int li = j - ctxl;
        kp = k_loc + ((int64_t(b) * L_loc + li) * Hkv + g) * d;
        pos = qpo + li;
        ok[u] = li <= horizon;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = lane + 64 * i;
        const bool in = ok[u] && m < half;
        k1[u][i] = in ? E::load(kp, m) : 0.f;
        k2[u][i] = in ? E::load(kp, m + half) : 0.f;
        cs[u][i] = in ? tab[int64_t(pos) * half + m] : make_float2(0.f, 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dot += qa[i] * (k1[u][i] * cs[u][i].x - k2[u][i] * cs[u][i].y) +
               qb[i] * (k2[u][i] * cs[u][i].x + k1[u][i] * cs[u][i].y);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
      const int j = j0 + u;
      if (j < n_keys) {
        const float lg = ok[u] ? dot * sm_scale : -INFINITY;
        if (lane == 0) logit[j] = lg;
        mx = fmaxf(mx, lg);
      }
    }
  }
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int st = AT_VEC_THREADS / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + st]);
    __syncthreads();
  }
  const float gmax = red[0];
  __syncthreads();
  float sum = 0.f;
  for (int j = threadIdx.x; j < n_keys; j += AT_VEC_THREADS) {
    const float p = logit[j] == -INFINITY ? 0.f : expf(logit[j] - gmax);
    logit[j] = p;
    sum += p;
  }
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int st = AT_VEC_THREADS / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  const float den = red[0];
  // value sum: wave w takes keys w, w + NW, ...; lanes over d (at most four
  // elements each), four keys' loads in flight
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = wave; j0 < n_keys; j0 += NW * KU) {
    float pv[KU], vv[KU][4];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int j = j0 + NW * u;
      const bool in = j < n_keys;
      pv[u] = in ? logit[j] : 0.f;
      const typename E::T* vp = v_loc;
      if (in)
        vp = j < ctxl ? v_ctx + (ctx_src_row(int64_t(b) * max_ctx + j, ctx_row, ctx_rows) * Hkv + g) * d
                      : v_loc + ((int64_t(b) * L_loc + (j - ctxl)) * Hkv + g) * d;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        vv[u][i] = (pv[u] != 0.f && e < d) ? E::load(vp, e) : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += pv[u] * vv[u][i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    if (e < d) part[wave * d + e] = acc[i];
  }
  __syncthreads();
  float* op = out + ((int64_t(b) * T + t) * Hq + hq) * d;
  if (lse && threadIdx.x == 0)
    lse[(int64_t(b) * T + t) * Hq + hq] = den > 0.f ? (gmax + logf(den)) * 1.4426950408889634f : -INFINITY;
  for (int e = threadIdx.x; e < d; e += AT_VEC_THREADS) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) a += part[w * d + e];
    op[e] = a / den;
  }
}

struct AttnPlan {
  bool mfma;
  bool prefill;     // workgroup-cooperative kernel (2+ row tiles)
  int rtw;          // row tiles per wave (prefill)
  int n_rg;         // row groups (prefill)
  int n_hg;         // KV-head groups of 8 (decode)
  int P;            // rows of the RoPE table
  int n_rt;         // 16-row tiles per (b, g)
  int n_splits;     // partials in the workspace
  int n_sc, n_sl;   // msa_sparse_attn_part: context splits [0, n_sc), local splits [n_sc, n_splits)
  int n_bc;         // one call, prefill: > 0 when the first n_bc of its splits take the context keys
                    // and the others the local keys (PF_BOTH)
  size_t tab_bytes, o_bytes, ml_bytes;
};


static AttnPlan attn_plan_splits(int dtype, int B, int T, int Hq, int Hkv, int d, int max_ctx, int L_loc, int qpo) {
  AttnPlan p{};
  const int G = Hkv > 0 ? Hq / Hkv : 0;
  p.mfma = dtype == MSA_BF16 && d == AT_D && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
  p.P = rope_rows(max_ctx, L_loc, qpo);
  p.tab_bytes = align_up(size_t(p.P) * (d / 2) * sizeof(float2), 256);
  if (!p.mfma) return p;
  p.n_rt = (T * G + 15) / 16;
  const int64_t n_keys_max = int64_t(max_ctx) + L_loc;
  p.prefill = p.n_rt >= 2;
  int64_t units, target;
  if (p.prefill) {
    p.rtw = 1;   // one row tile per wave: more workgroups, fewer key splits
    p.n_rg = (p.n_rt + PF_WAVES * p.rtw - 1) / (PF_WAVES * p.rtw);
    units = int64_t(B) * Hkv * p.n_rg;      // workgroups per split
    target = 256;                            // about one workgroup per CU
  } else {
    p.n_hg = (Hkv + DC_WAVES - 1) / DC_WAVES;
    units = int64_t(B) * p.n_hg;            // workgroups per split
    target = 1024;                           // two rounds of two 4-wave workgroups per CU
  }
  // the kernels split each query's actual keys evenly over n_splits; a split's
  // context entries must fit the workgroup's LDS index cache
  const int64_t want = (target + units - 1) / units;
  const int cap = p.prefill ? PF_CIDX : AT_CIDX;
  int64_t s = std::max<int64_t>(1, std::min<int64_t>(want, (n_keys_max + 63) / 64));
  if (max_ctx > cap) s = std::max<int64_t>(s, (n_keys_max + cap - 33) / (cap - 32));
  p.n_splits = int(s);
  // A context no longer than one split's share of the keys (the 100M and 1M
  // presets: 128 context rows beside 4,096 local tokens) gets a split of its
  // own and the local keys the others, so that the local splits need not wait
  // for the context's length before loading.
  if (p.prefill && s >= 3 && int64_t(max_ctx) <= (n_keys_max + s - 1) / s) p.n_bc = 1;
  // the two-call form: each part fills the chip on its own (the local part
  // runs beside the context's fetch, the context part after it)
  int64_t sc = std::max<int64_t>(1, std::min<int64_t>(want, (int64_t(max_ctx) + 63) / 64));
  if (max_ctx > cap) sc = std::max<int64_t>(sc, (int64_t(max_ctx) + cap - 33) / (cap - 32));
  const int64_t sl = std::max<int64_t>(1, std::min<int64_t>(want, (int64_t(L_loc) + 63) / 64));
  p.n_sc = int(sc);
  p.n_sl = int(sl);
  return p;
}

// workspace byte counts for n partial splits
static void plan_bytes(AttnPlan& p, int B, int T, int Hq, int d, int n) {
  const int64_t rows = int64_t(B) * T * Hq;
  p.o_bytes = p.mfma ? align_up(size_t(n) * rows * d * sizeof(uint16_t), 256) : 0;   // float16 partials
  p.ml_bytes = p.mfma ? align_up(size_t(n) * rows * sizeof(float4), 256) : 0;
}

// part 0: msa_sparse_attn's plan; MSA_ATTN_PART_*: the two-call plan, whose
// n_splits counts both parts' partials
static AttnPlan attn_plan(int dtype, int B, int T, int Hq, int Hkv, int d, int max_ctx, int L_loc, int qpo,
                          int part) {
  AttnPlan p = attn_plan_splits(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, qpo);
  if (part != 0 && p.mfma) p.n_splits = p.n_sc + p.n_sl;
  plan_bytes(p, B, T, Hq, d, p.n_splits);
  return p;
}

}  // namespace msa

extern "C" int msa_rope_table_rows(int max_ctx, int L_loc, int q_pos_offset) {
  if (max_ctx < 0 || L_loc < 1 || q_pos_offset < 0) return 0;
  return msa::rope_rows(max_ctx, L_loc, q_pos_offset);
}

extern "C" int msa_rope_table(int rows, int d, float rope_base, float* table, void* stream) {
  using namespace msa;
  MSA_REQUIRE(table, MSA_ERR_INVALID_ARG, "msa_rope_table: NULL table");
  MSA_REQUIRE(rows >= 1 && d >= 2 && d % 2 == 0, MSA_ERR_INVALID_ARG, "msa_rope_table: bad rows or d");
  MSA_REQUIRE(rope_base > 1.f, MSA_ERR_INVALID_ARG, "msa_rope_table: rope_base must exceed 1");
  const int64_t n = int64_t(rows) * (d / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, as_stream(stream),
                     reinterpret_cast<float2*>(table), rows, d / 2, double(rope_base), d);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

extern "C" size_t msa_sparse_attn_workspace(int dtype, int B, int T, int Hq, int Hkv, int d, int max_ctx, int L_loc,
                                            int q_pos_offset) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 2 || max_ctx < 0 || L_loc < 1 || q_pos_offset < 0) return 0;
  const msa::AttnPlan p = msa::attn_plan(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset, 0);
  return p.tab_bytes + p.o_bytes + p.ml_bytes;
}

extern "C" size_t msa_sparse_attn_part_workspace(int dtype, int B, int T, int Hq, int Hkv, int d, int max_ctx,
                                                 int L_loc, int q_pos_offset) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || d < 2 || max_ctx < 0 || L_loc < 1 || q_pos_offset < 0) return 0;
  const msa::AttnPlan p =
      msa::attn_plan(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset, MSA_ATTN_PART_LOCAL);
  return p.tab_bytes + p.o_bytes + p.ml_bytes;
}

namespace msa {

// Shared body of msa_sparse_attn (gathered context, ctx_row == NULL) and
// msa_sparse_attn_indexed (context rows read in place from the pooled store).
int sparse_attn(const std::string& fn, int dtype, const void* q, int B, int T, int Hq, int Hkv, int d,
                const void* k_ctx, const void* v_ctx, const int32_t* ctx_row, int64_t ctx_rows, const int32_t* ctx_pos,
                const int32_t* ctx_len, int max_ctx, const void* k_loc, const void* v_loc, int L_loc,
                int q_pos_offset, float rope_base, const float* rope_table, int rope_table_rows, float sm_scale,
                float* out, float* lse, void* ws, size_t ws_bytes, void* stream, const BwdPrep* prep,
                bool* prep_done, int part, bool check_only) {
  if (prep_done) *prep_done = false;
  MSA_REQUIRE(dtype_ok(dtype), MSA_ERR_INVALID_ARG, fn + ": bad dtype");
  MSA_REQUIRE(part == 0 || part == MSA_ATTN_PART_LOCAL || part == MSA_ATTN_PART_CONTEXT, MSA_ERR_INVALID_ARG,
              fn + ": bad part");
  const bool local_part = part == MSA_ATTN_PART_LOCAL;   // reads neither the context nor its length
  MSA_REQUIRE(q && k_loc && v_loc && ws && (local_part || (k_ctx && v_ctx && ctx_pos && ctx_len && out)),
              MSA_ERR_INVALID_ARG, fn + ": NULL pointer");
  MSA_REQUIRE(B >= 1 && T >= 1 && Hq >= 1 && Hkv >= 1 && d >= 2 && max_ctx >= 1 && L_loc >= 1, MSA_ERR_INVALID_ARG,
              fn + ": non-positive size");
  MSA_REQUIRE(Hq % Hkv == 0, MSA_ERR_INVALID_ARG, fn + ": Hq % Hkv != 0");
  MSA_REQUIRE(L_loc >= T, MSA_ERR_INVALID_ARG, fn + ": L_loc < T");
  MSA_REQUIRE(d % 2 == 0, MSA_ERR_INVALID_ARG, fn + ": d must be even");
  MSA_REQUIRE(q_pos_offset >= 0, MSA_ERR_INVALID_ARG, fn + ": q_pos_offset < 0");
  MSA_REQUIRE(rope_base > 1.f, MSA_ERR_INVALID_ARG, fn + ": rope_base must exceed 1");
  MSA_REQUIRE(d <= 256, MSA_ERR_UNSUPPORTED, fn + ": d > 256");
  MSA_REQUIRE(int64_t(q_pos_offset) + L_loc < (int64_t(1) << 30), MSA_ERR_UNSUPPORTED, fn + ": positions too large");
  const AttnPlan p = attn_plan(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset, part);
  MSA_REQUIRE(part == 0 || p.mfma, MSA_ERR_UNSUPPORTED,
              fn + ": the two-call form needs the MFMA path (bf16, d = 128, Hq/Hkv in {1, 2, 4, 8, 16})");
  MSA_REQUIRE(ws_bytes >= p.tab_bytes + p.o_bytes + p.ml_bytes, MSA_ERR_WORKSPACE, fn + ": workspace too small");
  if (!p.mfma)
    MSA_REQUIRE(int64_t(max_ctx) + L_loc <= AT_VEC_MAX_KEYS, MSA_ERR_UNSUPPORTED,
                fn + ": more than 32768 keys on the vector path");
  MSA_REQUIRE(!rope_table || rope_table_rows >= p.P, MSA_ERR_INVALID_ARG,
              fn + ": rope_table has fewer rows than msa_rope_table_rows()");
  MSA_REQUIRE(uintptr_t(rope_table) % 16 == 0, MSA_ERR_INVALID_ARG, fn + ": rope_table must be 16-byte aligned");
  if (p.mfma)
    MSA_REQUIRE(uintptr_t(q) % 16 == 0 && uintptr_t(k_ctx) % 16 == 0 && uintptr_t(v_ctx) % 16 == 0 &&
                    uintptr_t(k_loc) % 16 == 0 && uintptr_t(v_loc) % 16 == 0,
                MSA_ERR_INVALID_ARG, fn + ": tensors must be 16-byte aligned");
  if (check_only) return MSA_OK;
  hipStream_t s = as_stream(stream);
  const float2* tab = reinterpret_cast<const float2*>(rope_table);
  if (!tab) {
    float2* wtab = static_cast<float2*>(ws);
    const int64_t n = int64_t(p.P) * (d / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, wtab, p.P, d / 2,
                       double(rope_base), d);
    MSA_LAUNCH_CHECK();
    tab = wtab;
  }
  if (p.mfma) {
    uint16_t* ws_o = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + p.tab_bytes);
    float4* ws_ml = reinterpret_cast<float4*>(static_cast<char*>(ws) + p.tab_bytes + p.o_bytes);
    if (local_part) {
      // stand-ins for the context arguments, which the local part never
      // dereferences: valid device addresses all the same
      k_ctx = k_loc;
      v_ctx = v_loc;
      ctx_pos = ctx_len = reinterpret_cast<const int32_t*>(ws_ml);
      ctx_row = nullptr;
    }
    // this launch's splits and the index of its first partial
    const int n_launch = part == MSA_ATTN_PART_LOCAL ? p.n_sl : (part == MSA_ATTN_PART_CONTEXT ? p.n_sc : p.n_splits);
    int split_base = part == MSA_ATTN_PART_LOCAL ? p.n_sc : 0;
    const int G = Hq / Hkv;
    const float scale_log2_pf = sm_scale * 1.4426950408889634f;
    if (p.prefill) {
      const bool fuse_prep = prep && part == 0 && p.n_splits == 1;
      const BwdPrep pp = fuse_prep ? *prep : BwdPrep{};
      const bool pre = prep && prep->krot && prep->vg && part == 0;   // the backward's prepared keys
      const uint16_t* kk_src = static_cast<const uint16_t*>(pre ? prep->krot : k_ctx);
      const uint16_t* vv_src = static_cast<const uint16_t*>(pre ? prep->vg : v_ctx);
      const int km = pre ? prep->km : 0;
      // one call over both parts in separate splits (the prepared keys keep one order)
      const bool both = part == 0 && p.n_bc > 0 && !pre;
      const int kpart = both ? PF_BOTH : part;
      if (both) split_base = p.n_bc;
      const dim3 pgrid(unsigned(int64_t(B) * Hkv * p.n_rg * n_launch)), pblock(PF_THREADS);
      const size_t psmem = 2 * size_t(PF_BUF) + PF_CIDX_BYTES;
#define PF_LAUNCH3(GV, RV, IV, PV)                                                                                  \
  MSA_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_prefill_kernel<GV, RV, IV, PV>),           \
                                    hipFuncAttributeMaxDynamicSharedMemorySize, int(psmem)));                       \
  hipLaunchKernelGGL((attn_prefill_kernel<GV, RV, IV, PV>), pgrid, pblock, psmem, s, static_cast<const uint16_t*>(q), B, \
                     T, Hq, Hkv, kk_src, vv_src, ctx_pos, ctx_len, max_ctx, static_cast<const uint16_t*>(k_loc),     \
                     static_cast<const uint16_t*>(v_loc), L_loc, q_pos_offset, ctx_row, ctx_rows, tab, p.P,          \
                     scale_log2_pf, ws_o, ws_ml, n_launch, p.n_rt, p.n_rg, out, lse, kpart, split_base, km, pp)
#define PF_LAUNCH(GV, RV)                 \
  if (pre) {                              \
    PF_LAUNCH3(GV, RV, false, true);      \
  } else if (ctx_row) {                   \
    PF_LAUNCH3(GV, RV, true, false);      \
  } else {                                \
    PF_LAUNCH3(GV, RV, false, false);     \
  }
      const int key = G * 4 + p.rtw;
      switch (key) {
        case 1 * 4 + 1: PF_LAUNCH(1, 1); break;
        case 1 * 4 + 2: PF_LAUNCH(1, 2); break;
        case 2 * 4 + 1: PF_LAUNCH(2, 1); break;
        case 2 * 4 + 2: PF_LAUNCH(2, 2); break;
        case 4 * 4 + 1: PF_LAUNCH(4, 1); break;
        case 4 * 4 + 2: PF_LAUNCH(4, 2); break;
        case 8 * 4 + 1: PF_LAUNCH(8, 1); break;
        case 8 * 4 + 2: PF_LAUNCH(8, 2); break;
        case 16 * 4 + 1: PF_LAUNCH(16, 1); break;
        default: PF_LAUNCH(16, 2); break;
      }
#undef PF_LAUNCH
#undef PF_LAUNCH3
      MSA_LAUNCH_CHECK();
      if (local_part) return MSA_OK;   // the context part merges
      if (part == 0 && p.n_splits == 1) {   // the prefill wrote out (or the backward's rows) and lse itself
        if (prep_done) *prep_done = fuse_prep;
        return MSA_OK;
      }
      const int64_t rows = int64_t(B) * T * Hq;
      hipLaunchKernelGGL(attn_combine_kernel, dim3(unsigned((rows * (d / 4) + 255) / 256)), dim3(256), 0, s, ws_o,
                         ws_ml, p.n_splits, rows, d, out, lse);
      MSA_LAUNCH_CHECK();
      return MSA_OK;
    }
    const int nw = DC_WAVES;   // waves beyond Hkv only help stage the RoPE rows
    const dim3 grid{unsigned(int64_t(B) * p.n_hg * n_launch)}, block{unsigned(DC_THREADS)};
    const size_t smem = 2 * size_t(DC_TAB_BYTES) + size_t(nw) * AT_V_BYTES + AT_CIDX_BYTES;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
#define DC_LAUNCH2(GV, IV)                                                                                         \
  MSA_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_decode_kernel<GV, IV>),                    \
                                    hipFuncAttributeMaxDynamicSharedMemorySize, int(smem)));                     \
  hipLaunchKernelGGL((attn_decode_kernel<GV, IV>), grid, block, smem, s, static_cast<const uint16_t*>(q), B, T, Hq, Hkv, \
                     static_cast<const uint16_t*>(k_ctx), static_cast<const uint16_t*>(v_ctx), ctx_pos, ctx_len,     \
                     max_ctx, static_cast<const uint16_t*>(k_loc), static_cast<const uint16_t*>(v_loc), L_loc,       \
                     q_pos_offset, ctx_row, ctx_rows, tab, p.P, scale_log2, ws_o, ws_ml, n_launch, p.n_hg, part,      \
                     split_base)
#define DC_LAUNCH(GV)        \
  if (ctx_row) {             \
    DC_LAUNCH2(GV, true);    \
  } else {                   \
    DC_LAUNCH2(GV, false);   \
  }
    switch (G) {
      case 1: DC_LAUNCH(1); break;
      case 2: DC_LAUNCH(2); break;
      case 4: DC_LAUNCH(4); break;
      case 8: DC_LAUNCH(8); break;
      default: DC_LAUNCH(16); break;
    }
#undef DC_LAUNCH
#undef DC_LAUNCH2
    MSA_LAUNCH_CHECK();
    if (local_part) return MSA_OK;
    const int64_t rows = int64_t(B) * T * Hq;
    hipLaunchKernelGGL(attn_combine_kernel, dim3(unsigned((rows * (d / 4) + 255) / 256)), dim3(256), 0, s, ws_o,
                       ws_ml, p.n_splits, rows, d, out, lse);
    MSA_LAUNCH_CHECK();
    return MSA_OK;
  }
  const size_t smem = (size_t(d) * (1 + AT_VEC_THREADS / 64) + AT_VEC_THREADS + size_t(max_ctx) + L_loc) * sizeof(float);
  const dim3 grid(unsigned(int64_t(B) * T * Hq)), block(AT_VEC_THREADS);
  if (dtype == MSA_BF16)
    hipLaunchKernelGGL(attn_vec_kernel<MSA_BF16>, grid, block, smem, s, static_cast<const uint16_t*>(q), B, T, Hq, Hkv,
                       d, static_cast<const uint16_t*>(k_ctx), static_cast<const uint16_t*>(v_ctx), ctx_pos, ctx_len,
                       max_ctx, static_cast<const uint16_t*>(k_loc), static_cast<const uint16_t*>(v_loc), L_loc,
                       q_pos_offset, ctx_row, ctx_rows, tab, p.P, sm_scale, out, lse);
  else
    hipLaunchKernelGGL(attn_vec_kernel<MSA_F32>, grid, block, smem, s, static_cast<const float*>(q), B, T, Hq, Hkv, d,
                       static_cast<const float*>(k_ctx), static_cast<const float*>(v_ctx), ctx_pos, ctx_len, max_ctx,
                       static_cast<const float*>(k_loc), static_cast<const float*>(v_loc), L_loc, q_pos_offset,
                       ctx_row, ctx_rows, tab, p.P, sm_scale, out, lse);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

}  // namespace msa

extern "C" int msa_sparse_attn(int dtype, const void* q, int B, int T, int Hq, int Hkv, int d, const void* k_ctx,
                               const void* v_ctx, const int32_t* ctx_pos, const int32_t* ctx_len, int max_ctx,
                               const void* k_loc, const void* v_loc, int L_loc, int q_pos_offset, float rope_base,
                               const float* rope_table, int rope_table_rows, float sm_scale, float* out, void* ws,
                               size_t ws_bytes, void* stream) {
  return msa::sparse_attn("msa_sparse_attn", dtype, q, B, T, Hq, Hkv, d, k_ctx, v_ctx, nullptr, 0, ctx_pos, ctx_len,
                          max_ctx, k_loc, v_loc, L_loc, q_pos_offset, rope_base, rope_table, rope_table_rows, sm_scale,
                          out, nullptr, ws, ws_bytes, stream);
}

extern "C" int msa_sparse_attn_indexed(int dtype, const void* q, int B, int T, int Hq, int Hkv, int d,
                                       const void* k_bar, const void* v_bar, int64_t n_chunks, const int32_t* ctx_row,
                                       const int32_t* ctx_pos, const int32_t* ctx_len, int max_ctx, const void* k_loc,
                                       const void* v_loc, int L_loc, int q_pos_offset, float rope_base,
                                       const float* rope_table, int rope_table_rows, float sm_scale, float* out,
                                       void* ws, size_t ws_bytes, void* stream) {
  using namespace msa;
  MSA_REQUIRE(ctx_row, MSA_ERR_INVALID_ARG, "msa_sparse_attn_indexed: NULL pointer");
  MSA_REQUIRE(n_chunks >= 1 && n_chunks <= INT32_MAX, MSA_ERR_INVALID_ARG,
              "msa_sparse_attn_indexed: n_chunks must lie in [1, 2^31)");
  return sparse_attn("msa_sparse_attn_indexed", dtype, q, B, T, Hq, Hkv, d, k_bar, v_bar, ctx_row, n_chunks, ctx_pos,
                     ctx_len, max_ctx, k_loc, v_loc, L_loc, q_pos_offset, rope_base, rope_table, rope_table_rows,
                     sm_scale, out, nullptr, ws, ws_bytes, stream);
}

extern "C" int msa_sparse_attn_part(int part, int dtype, const void* q, int B, int T, int Hq, int Hkv, int d,
                                    const void* k_ctx, const void* v_ctx, int64_t ctx_rows, const int32_t* ctx_row,
                                    const int32_t* ctx_pos, const int32_t* ctx_len, int max_ctx, const void* k_loc,
                                    const void* v_loc, int L_loc, int q_pos_offset, float rope_base,
                                    const float* rope_table, int rope_table_rows, float sm_scale, float* out,
                                    void* ws, size_t ws_bytes, void* stream) {
  using namespace msa;
  const std::string fn = "msa_sparse_attn_part";
  MSA_REQUIRE(part == MSA_ATTN_PART_LOCAL || part == MSA_ATTN_PART_CONTEXT, MSA_ERR_INVALID_ARG, fn + ": bad part");
  MSA_REQUIRE(!ctx_row || (ctx_rows >= 1 && ctx_rows <= INT32_MAX), MSA_ERR_INVALID_ARG,
              fn + ": ctx_rows must lie in [1, 2^31) with ctx_row");
  return sparse_attn(fn, dtype, q, B, T, Hq, Hkv, d, k_ctx, v_ctx, ctx_row, ctx_row ? ctx_rows : 0, ctx_pos, ctx_len,
                     max_ctx, k_loc, v_loc, L_loc, q_pos_offset, rope_base, rope_table, rope_table_rows, sm_scale, out,
                     nullptr, ws, ws_bytes, stream, nullptr, nullptr, part);
}

// ---------------------------------------------------------------- no-alloc variant
// msa_sparse_attn_indexed for callers that cannot allocate: its workspace
// (the RoPE table when the caller passes none, the split partials O, m, l)
// is one file-scope device array that each GPU the library runs on holds
// until the process ends.  In host code the array's name is not a device
// address: its address on each device comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address reaches a
// kernel.  Nothing in the scratch must start at zero: every split writes each
// of its rows' partials before the combine reads them.  Calls that overlap on
// one GPU share the array and race.
namespace msa {

static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[NOALLOC_MAX_DEVICES];

// The device address of `scratch` on the current device.
static int scratch_address(const std::string& fn, void** ptr) {
  int dev = -1;
  MSA_HIP_CHECK(hipGetDevice(&dev));
  MSA_REQUIRE(dev >= 0 && dev < NOALLOC_MAX_DEVICES, MSA_ERR_UNSUPPORTED, fn + ": device ordinal beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    MSA_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    MSA_REQUIRE(p, MSA_ERR_HIP, fn + ": hipGetSymbolAddress gave NULL");
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return MSA_OK;
}

}  // namespace msa

extern "C" int msa_sparse_attn_indexed_noalloc(int dtype, const void* q, int B, int T, int Hq, int Hkv, int d,
                                               const void* k_bar, const void* v_bar, int64_t n_chunks,
                                               const int32_t* ctx_row, const int32_t* ctx_pos, const int32_t* ctx_len,
                                               int max_ctx, const void* k_loc, const void* v_loc, int L_loc,
                                               int q_pos_offset, float rope_base, const float* rope_table,
                                               int rope_table_rows, float sm_scale, float* out, void* stream) {
  using namespace msa;
  const std::string fn = "msa_sparse_attn_indexed_noalloc";
  MSA_REQUIRE(ctx_row, MSA_ERR_INVALID_ARG, fn + ": NULL pointer");
  MSA_REQUIRE(n_chunks >= 1 && n_chunks <= INT32_MAX, MSA_ERR_INVALID_ARG, fn + ": n_chunks must lie in [1, 2^31)");
  MSA_REQUIRE(B >= 1 && T >= 1 && Hq >= 1 && Hkv >= 1 && d >= 2 && max_ctx >= 1 && L_loc >= 1 && q_pos_offset >= 0,
              MSA_ERR_INVALID_ARG, fn + ": non-positive size");
  const size_t need = msa_sparse_attn_workspace(dtype, B, T, Hq, Hkv, d, max_ctx, L_loc, q_pos_offset);
  MSA_REQUIRE(need <= MSA_NOALLOC_SCRATCH_BYTES, MSA_ERR_UNSUPPORTED,
              fn + ": this shape needs " + std::to_string(need) + " bytes of workspace; the no-alloc entry point "
                   "holds " + std::to_string(size_t(MSA_NOALLOC_SCRATCH_BYTES)) +
                   " (use msa_sparse_attn_indexed with a caller workspace)");
  void* ws = nullptr;
  const int st = scratch_address(fn, &ws);
  if (st != MSA_OK) return st;
  return sparse_attn(fn, dtype, q, B, T, Hq, Hkv, d, k_bar, v_bar, ctx_row, n_chunks, ctx_pos, ctx_len, max_ctx,
                     k_loc, v_loc, L_loc, q_pos_offset, rope_base, rope_table, rope_table_rows, sm_scale, out, nullptr,
                     ws, MSA_NOALLOC_SCRATCH_BYTES, stream);
}
