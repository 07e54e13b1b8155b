// Shared pieces of the attention kernels (forward and backward): bf16
// packing, the transpose-read operand of the PV-type products, RoPE rotation
// of a query fragment, the context-key addressing (gathered or indexed
// store), and the LDS-only barrier.
#pragma once

#include <algorithm>
#include <string>

#include "common.h"

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int AT_D = 128;
constexpr int AT_WAVES = 4;
constexpr int AT_THREADS = 64 * AT_WAVES;
constexpr int AT_VEC_THREADS = 256;
constexpr int AT_VEC_MAX_KEYS = 32768;

// two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void unpack8(const uint4& u, float (&x)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(w[e] << 16);
    x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint4 pack8(const float (&x)[8]) {
  return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                    pack_bf16x2(x[6], x[7]));
}

// Row-major V tile in LDS: 32 keys x 128 d (bf16), row stride AT_VS bytes.
constexpr int AT_VS = 288;                   // 256 + 32: the 16 rows of one transpose read hit 8 bank groups
constexpr int AT_V_BYTES = 32 * AT_VS;

typedef short v4s __attribute__((ext_vector_type(4)));

// A operand of O^T = V^T P^T for d-tile dt: lane (lc, g4) receives
// V[16*tau + 4*g4 + r][16*dt + lc] in slot 4*tau + r.  ds_read_b64_tr_b16
// hands lane i of each 16-lane group element i % 4 of the 8-byte chunks
// addressed by lanes 4r + i/4 (r = 0..3); so lane j = 4r + q of group g4
// addresses key 16*tau + 4*g4 + r, dims 16*dt + 4q .. +3.
__device__ __forceinline__ bf16x8 pv_operand(const unsigned char* vlds, int dt, int lane) {
  const int g4 = lane / 16, j = lane % 16;
  const int r = j / 4, q = j % 4;
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  const unsigned char* p0 = vlds + (4 * g4 + r) * AT_VS + (16 * dt + 4 * q) * 2;
  const unsigned char* p1 = p0 + 16 * AT_VS;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p0));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(p1));
  typedef short v8s __attribute__((ext_vector_type(8)));
  const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// Rotate the lane's 16 (m, m + 64) pairs: lo[kk] holds dims 32kk + 8*g4 + e,
// hi[kk] dims 64 + 32kk + 8*g4 + e (kk = 0, 1).  cs points at tab[pos][0].
// The rotated values are multiplied by scale before their one rounding.
__device__ __forceinline__ void rope_rotate(uint4 (&v)[4], const float2* __restrict__ cs, int g4,
                                            float scale = 1.f) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    float lo[8], hi[8];
    unpack8(v[kk], lo);
    unpack8(v[kk + 2], hi);
    const float4* c4 = reinterpret_cast<const float4*>(cs + 32 * kk + 8 * g4);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const float4 t = c4[e2];  // (cos, sin) of two consecutive m
      const float c0 = t.x, s0 = t.y, c1 = t.z, s1 = t.w;
      const float a0 = lo[2 * e2], b0 = hi[2 * e2], a1 = lo[2 * e2 + 1], b1 = hi[2 * e2 + 1];
      lo[2 * e2] = (a0 * c0 - b0 * s0) * scale;
      hi[2 * e2] = (b0 * c0 + a0 * s0) * scale;
      lo[2 * e2 + 1] = (a1 * c1 - b1 * s1) * scale;
      hi[2 * e2 + 1] = (b1 * c1 + a1 * s1) * scale;
    }
    v[kk] = pack8(lo);
    v[kk + 2] = pack8(hi);
  }
}

// A key split's partial result for one query row, as attn_combine_kernel
// reads it: the unnormalised O scaled by 2^-c, with c the exponent of the
// row's largest |O| (frexp), so every element lies in (-1, 1), stored in
// float16; and (m, l, c) in float32.  Half the bytes of a float32 partial;
// the power-of-two scale keeps any O in range, and the float16 rounding stays
// within 2^-12 of the row's largest element.  Lane (lc, g4) holds
// O^T[16*dt + 4*g4 + e][row lc]; the four lanes of a row (g4 = 0..3) must all
// call it (the row maximum crosses them); row_ok selects the lanes that store.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const half2_t v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float2 unpack_f16x2(uint32_t u) {
  const half2_t v = __builtin_bit_cast(half2_t, u);
  return make_float2(static_cast<float>(v.x), static_cast<float>(v.y));
}

__device__ __forceinline__ void store_partial(const f32x4 (&o)[8], float m, float l, bool row_ok, int g4,
                                              uint16_t* __restrict__ ws_oh_row, float4* __restrict__ ws_ml_row) {
  float rmax = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) rmax = fmaxf(rmax, fabsf(o[dt][e]));
  rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
  rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
  int c = 0;
  (void)frexpf(rmax, &c);
  const float sc = ldexpf(1.f, -c);
  if (!row_ok) return;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<uint2*>(ws_oh_row + 16 * dt + 4 * g4) =
        make_uint2(pack_f16x2(o[dt][0] * sc, o[dt][1] * sc), pack_f16x2(o[dt][2] * sc, o[dt][3] * sc));
  if (g4 == 0) *ws_ml_row = make_float4(m, l, float(c), 0.f);
}

struct KeySrc {
  int64_t row;   // row index into the [*, Hkv, d] tensor (already including b)
  int pos;
  bool local;
  bool valid;
};

// Context entry e of query b: row b * max_ctx + e of a gathered context, or,
// when ctx_row is given, row ctx_row[b, e] of the pooled store itself (the
// concatenation is then only an index; rows are clamped into the store).
__device__ __forceinline__ int64_t ctx_src_row(int64_t e, const int32_t* __restrict__ ctx_row, int64_t ctx_rows) {
  if (!ctx_row) return e;
  const int64_t r = ctx_row[e];
  return r < 0 ? 0 : (r >= ctx_rows ? ctx_rows - 1 : r);
}

// A workgroup's context entries [lo, lo + n) as (store row, clamped
// position), staged in LDS once so that no step waits on an index load.  The
// decode kernel (two workgroups per CU) holds 1,024 entries; the prefill
// kernel (one workgroup per CU) 4,096, so that a 4,096-entry context does
// not force extra key splits.
constexpr int AT_CIDX = 1024;
constexpr int AT_CIDX_BYTES = AT_CIDX * 8;
constexpr int PF_CIDX = 4096;
constexpr int PF_CIDX_BYTES = PF_CIDX * 8;
struct CtxCache {
  const int2* e;
  int lo, n, cap;
};

__device__ __forceinline__ CtxCache stage_ctx(int2* lds, int cap, int b, int j_begin, int j_end, int ctxl,
                                              int max_ctx, const int32_t* __restrict__ ctx_pos, int P,
                                              const int32_t* __restrict__ ctx_row, int64_t ctx_rows, int tid,
                                              int nthr) {
  CtxCache c;
  c.e = lds;
  c.lo = j_begin;
  c.cap = cap;
  c.n = max(0, min(min(j_end, ctxl) - j_begin, cap));
  for (int i = tid; i < c.n; i += nthr) {
    const int64_t e = int64_t(b) * max_ctx + j_begin + i;
    int p = ctx_pos[e];
    p = p < 0 ? 0 : (p >= P ? P - 1 : p);
    lds[i] = make_int2(ctx_row ? int(ctx_src_row(e, ctx_row, ctx_rows)) : 0, p);
  }
  return c;
}

__device__ __forceinline__ KeySrc key_src(int j, int b, int ctxl, int n_keys, int max_ctx, int L_loc, int qpo,
                                          const int32_t* __restrict__ ctx_pos, int P,
                                          const int32_t* __restrict__ ctx_row, int64_t ctx_rows,
                                          const CtxCache& cc) {
  // Branch-free (selects only), so the loads that follow stay straight-line
  // code.  Every context key of the workgroup's range is cached (the host
  // sizes the splits for it); the cache read is clamped into the cache and
  // its value is used only for such keys.  Keys past the range end or past
  // n_keys are masked by the caller: any in-bounds row will do.
  (void)ctx_pos;
  (void)P;
  (void)ctx_rows;
  const int i = j - cc.lo;
  const bool in = i >= 0 && i < cc.n;
  const int2 e = cc.e[min(max(i, 0), cc.cap - 1)];
  const bool is_ctx = j < ctxl;
  const int li = min(max(j - ctxl, 0), L_loc - 1);
  const int64_t crow = ctx_row ? int64_t(in ? e.x : 0) : int64_t(b) * max_ctx + (in ? j : 0);
  KeySrc k;
  k.row = is_ctx ? crow : int64_t(b) * L_loc + li;
  k.pos = is_ctx ? (in ? e.y : 0) : qpo + li;
  k.local = !is_ctx;
  k.valid = j < n_keys;
  return k;
}

// This wave's LDS operations are complete, then the workgroup barrier; unlike
// __syncthreads() it does not wait for outstanding vector-memory loads.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// RoPE table rows the attention kernels need: max(qpo + L_loc, max_ctx, 32)
inline int rope_rows(int max_ctx, int L_loc, int qpo) { return std::max(std::max(qpo + L_loc, max_ctx), 32); }

// The backward's row preparation, done by the forward's epilogue when the
// forward runs as one key split of the prefill kernel (the row's O is then in
// registers): D = <dO, O>, dO rounded to bf16, and the rotated query times
// sm_scale * log2(e) as the forward rounded it.  O itself is then not written.
struct BwdPrep {
  const float* dout = nullptr;
  float* Dv = nullptr;
  uint16_t* qs16 = nullptr;
  uint16_t* do16 = nullptr;
  // the backward's prepared keys (rotated K and V in key order, [B, km, Hkv, d]),
  // when already written: the prefill forward then reads them instead of
  // rotating and looking up every key itself
  const uint16_t* krot = nullptr;
  const uint16_t* vg = nullptr;
  int km = 0;
};

// The forward of msa_sparse_attn / msa_sparse_attn_indexed (ctx_row NULL for
// a gathered context); lse, when given, receives per query row the base-2
// log-sum-exp of the logits scaled by sm_scale * log2(e).  With prep, the
// forward also does the backward's row preparation when its plan allows
// (*prep_done tells).  part: 0 for the whole attention, MSA_ATTN_PART_LOCAL /
// MSA_ATTN_PART_CONTEXT for the two calls of msa_sparse_attn_part.  check_only:
// validate the arguments (the status a call would return before launching) and
// launch nothing.
int sparse_attn(const std::string& fn, int dtype, const void* q, int B, int T, int Hq, int Hkv, int d,
                const void* k_ctx, const void* v_ctx, const int32_t* ctx_row, int64_t ctx_rows, const int32_t* ctx_pos,
                const int32_t* ctx_len, int max_ctx, const void* k_loc, const void* v_loc, int L_loc,
                int q_pos_offset, float rope_base, const float* rope_table, int rope_table_rows, float sm_scale,
                float* out, float* lse, void* ws, size_t ws_bytes, void* stream, const BwdPrep* prep = nullptr,
                bool* prep_done = nullptr, int part = 0, bool check_only = false);

}  // namespace msa
