// Device copy of the seeded input generator of synth/__init__.py (same
// definition, bit-identical output): counter-based SplitMix64 words, the
// four 16-bit lanes summed (Irwin-Hall, n = 4), centred, one float32
// multiply by 1/sqrt((2^32 - 1)/3), an exact power-of-two scale, and
// optional round-to-nearest-even to bfloat16.  It generates inputs only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

__device__ inline float normal_value(uint64_t base, uint64_t i, float mul) {
  const uint64_t w = mix64(base + (i + 1) * kGamma);
  const int64_t tot = int64_t(w & 0xFFFF) + int64_t((w >> 16) & 0xFFFF) + int64_t((w >> 32) & 0xFFFF) +
                      int64_t(w >> 48) - 131070;
  float v = float(int32_t(tot)) * 2.6428997921303014e-05f;
  v = __fmul_rn(v, mul);
  return v;
}

__device__ inline uint16_t to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return uint16_t(b >> 16);
}

__global__ void fill_kernel(int bf16, uint64_t base, int64_t start, int64_t count, float mul, void* out) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += int64_t(gridDim.x) * blockDim.x) {
    const float v = normal_value(base, uint64_t(start + i), mul);
    if (bf16)
      static_cast<uint16_t*>(out)[i] = to_bf16(v);
    else
      static_cast<float*>(out)[i] = v;
  }
}

}  // namespace

extern "C" {

// out[i] = value(seed, stream, start + i) for i < count; returns 0 on success.
int msa_synth_fill(int bf16, uint64_t seed, uint64_t stream_id, int64_t start, int64_t count, int scale_pow2,
                   void* out, void* stream) {
  if (!out || count < 0 || start < 0) return 1;
  if (count == 0) return 0;
  const uint64_t base = mix64(seed * kGamma + stream_id);
  const float mul = ldexpf(1.0f, scale_pow2);
  const int64_t blocks = (count + 255) / 256 < 65536 ? (count + 255) / 256 : 65536;
  hipLaunchKernelGGL(fill_kernel, dim3(unsigned(blocks)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), bf16,
                     base, start, count, mul, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
