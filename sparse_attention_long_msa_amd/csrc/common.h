// Internal helpers shared by the HIP translation units of libmsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "msa.h"

namespace msa {

// ---------------------------------------------------------------- errors

void set_error(const std::string& msg);
int fail(int status, const std::string& msg);

#define MSA_REQUIRE(cond, status, msg)                   \
  do {                                                   \
    if (!(cond)) return ::msa::fail((status), (msg));    \
  } while (0)

#define MSA_HIP_CHECK(expr)                                                          \
  do {                                                                               \
    hipError_t e_ = (expr);                                                          \
    if (e_ != hipSuccess)                                                            \
      return ::msa::fail(MSA_ERR_HIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

#define MSA_LAUNCH_CHECK() MSA_HIP_CHECK(hipGetLastError())

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- numerics

// bfloat16 is carried as its raw 16-bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float32 -> bfloat16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return uint16_t(b >> 16);
}

// Order-preserving map of a float to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_key_float(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}

// Atomic max of a float in memory that holds a float (no NaN).  Exact and
// order-independent: for non-negative values the IEEE bit patterns order
// like signed integers, for negative values like reversed unsigned ones.
__device__ __forceinline__ void atomic_max_float(float* addr, float v) {
  if (__float_as_int(v) >= 0)
    atomicMax(reinterpret_cast<int*>(addr), __float_as_int(v));
  else
    atomicMin(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

// 16-byte load that bypasses cache allocation (the data is streamed once).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte load from global memory, stated as such: a pointer chosen among
// several at run time would otherwise be read with a flat load, which also
// counts against the LDS counter.
__device__ __forceinline__ uint4 load_global(const void* p) {
  typedef const __attribute__((address_space(1))) u32x4* gptr;
  const u32x4 v = *(gptr)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 8-byte load from global memory (see load_global).
__device__ __forceinline__ uint2 load_global8(const void* p) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  typedef const __attribute__((address_space(1))) u32x2* gptr;
  const u32x2 v = *(gptr)(p);
  return make_uint2(v.x, v.y);
}

template <int DT> struct Elem;
template <> struct Elem<MSA_F32> {
  using T = float;
  static constexpr int bytes = 4;
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
};
template <> struct Elem<MSA_BF16> {
  using T = uint16_t;
  static constexpr int bytes = 2;
  __device__ static float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
};

inline int dtype_bytes(int dt) { return dt == MSA_F32 ? 4 : 2; }

// msa_gather_kv's copy from any GPU-readable source (gather.hip)
int gather_copy(const int32_t* ids, int B, int k, const int64_t* chunk_off, int64_t n_docs, const void* k_bar,
                const void* v_bar, int64_t row_vec, int max_ctx, void* k_ctx, void* v_ctx, int32_t* ctx_pos,
                int32_t* ctx_len, hipStream_t s);
inline bool dtype_ok(int dt) { return dt == MSA_F32 || dt == MSA_BF16; }

}  // namespace msa
