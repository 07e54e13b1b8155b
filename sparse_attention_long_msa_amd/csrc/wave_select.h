// Wave-level ranking primitives of the top-k kernels.  A (score, id) pair is one 64-bit key
// whose ascending order is the ranking (score descending, id ascending): the
// high word is the bit-complement of the order-preserving image of the float
// score, the low word the document id.  Keys are unique, so every selection
// is exact and deterministic.
#pragma once

#include "common.h"

namespace msa {

__device__ __forceinline__ uint64_t score_key(float s, uint32_t id) {
  return (uint64_t(~float_order_key(s)) << 32) | uint64_t(id);
}

// ---------------------------------------------------------------- wave-level selection (k <= 64)
// A wave keeps the 64 smallest keys seen so far, sorted across its lanes.  A
// batch of 64 new keys is skipped when none beats the current k-th key;
// otherwise it is bitonic-sorted across the lanes and merged: the
// elementwise min of the kept list and the reversed batch holds the 64
// smallest of both as a bitonic sequence, which a bitonic merge sorts.

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const int lo = __shfl_xor(int(uint32_t(v)), m), hi = __shfl_xor(int(uint32_t(v >> 32)), m);
  return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}
__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  const int lo = __shfl(int(uint32_t(v)), src), hi = __shfl(int(uint32_t(v >> 32)), src);
  return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(int(uint32_t(v)), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(int(uint32_t(v >> 32)), lane);
  return (uint64_t(hi) << 32) | lo;
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_mov64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp(int(uint32_t(v)), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(int(uint32_t(v >> 32)), CTRL, 0xF, 0xF, false);
  return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}

// value of lane (lane ^ stride): DPP inside a 16-lane row, cross-lane
// permutes for 16 and 32
template <int STRIDE>
__device__ __forceinline__ uint64_t xor_partner64(uint64_t v, int lane) {
  if constexpr (STRIDE == 1) return dpp_mov64<0xB1>(v);          // quad_perm [1,0,3,2]
  else if constexpr (STRIDE == 2) return dpp_mov64<0x4E>(v);     // quad_perm [2,3,0,1]
  else if constexpr (STRIDE == 4) {
    // row_ror:n hands lane i the value of lane (i - n) mod 16 within its row
    const uint64_t a = dpp_mov64<0x124>(v), b = dpp_mov64<0x12C>(v);   // from i - 4 / i + 4
    return (lane & 4) ? a : b;
  } else if constexpr (STRIDE == 8) return dpp_mov64<0x128>(v);  // row_ror 8
  else return shfl_xor64(v, STRIDE);
}

template <int SIZE, int STRIDE>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t key, int lane) {
  const uint64_t other = xor_partner64<STRIDE>(key, lane);
  const bool up = (lane & SIZE) == 0 || SIZE == 64;
  const bool lower = (lane & STRIDE) == 0;
  return (lower == up) ? (key < other ? key : other) : (key < other ? other : key);
}

template <int SIZE, int STRIDE>
__device__ __forceinline__ uint64_t bitonic_stage(uint64_t key, int lane) {
  key = bitonic_step<SIZE, STRIDE>(key, lane);
  if constexpr (STRIDE > 1) key = bitonic_stage<SIZE, STRIDE / 2>(key, lane);
  return key;
}

// ascending bitonic sort of one key per lane over the 64 lanes
__device__ __forceinline__ uint64_t wave_sort64(uint64_t key, int lane) {
  key = bitonic_stage<2, 1>(key, lane);
  key = bitonic_stage<4, 2>(key, lane);
  key = bitonic_stage<8, 4>(key, lane);
  key = bitonic_stage<16, 8>(key, lane);
  key = bitonic_stage<32, 16>(key, lane);
  key = bitonic_stage<64, 32>(key, lane);
  return key;
}

// sorts a bitonic sequence held one key per lane (ascending)
__device__ __forceinline__ uint64_t wave_merge64(uint64_t key, int lane) {
  return bitonic_stage<64, 32>(key, lane);
}

// the 64 smallest of two ascending lists held one key per lane, ascending:
// the elementwise min of one list and the other reversed is bitonic and holds
// them, and a bitonic merge sorts it (skipped when other's head does not beat
// best's k-th key)
__device__ __forceinline__ uint64_t wave_merge_sorted(uint64_t best, uint64_t other, int lane, int k) {
  if (!(readlane64(other, 0) < readlane64(best, k - 1))) return best;
  const uint64_t rev = shfl64(other, 63 - lane);
  return wave_merge64(best < rev ? best : rev, lane);
}

__device__ __forceinline__ uint64_t wave_insert(uint64_t best, uint64_t key, int lane, int k) {
  const uint64_t thr = readlane64(best, k - 1);
  if (__ballot(key < thr) == 0) return best;
  key = wave_sort64(key, lane);
  const uint64_t rev = shfl64(key, 63 - lane);
  return wave_merge64(best < rev ? best : rev, lane);
}

}  // namespace msa
