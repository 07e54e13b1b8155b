// Streaming-read reference for the roofline of the HBM-bound kernels: the
// rate at which this chip reads a buffer once with the routing-key scan's
// access pattern (each wave load instruction covers 1 KB contiguous, 16-byte
// non-temporal loads), in the configuration that measured fastest among
// 4-32 loads in flight per lane, 256-1024 threads and 1-4 workgroups per CU:
// sixteen loads in flight per lane, one 8-wave workgroup per CU.  Nothing is computed but an XOR of the data, which
// keeps every load alive; nothing is written unless that XOR hits one
// particular value.
#include <algorithm>

#include "common.h"

namespace msa {

constexpr int SR_THREADS = 512;   // 8 waves
constexpr int SR_U = 16;          // 16-byte loads in flight per lane

__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const uint4* __restrict__ p, int64_t n_vec,
                                                                 uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x % 64;
  const int64_t wave = int64_t(blockIdx.x) * (SR_THREADS / 64) + threadIdx.x / 64;
  const int64_t n_waves = int64_t(gridDim.x) * (SR_THREADS / 64);
  constexpr int64_t span = 64 * SR_U;    // vectors per wave per round (16 KB)
  uint32_t acc = 0;
  for (int64_t base = wave * span; base < n_vec; base += n_waves * span) {
    uint4 v[SR_U];
#pragma unroll
    for (int u = 0; u < SR_U; ++u) {
      const int64_t i = base + 64 * u + lane;
      v[u] = i < n_vec ? load_stream(p + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < SR_U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace msa

extern "C" int msa_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  using namespace msa;
  MSA_REQUIRE(buf && sink, MSA_ERR_INVALID_ARG, "msa_stream_read: NULL pointer");
  MSA_REQUIRE(bytes >= 16 && bytes % 16 == 0, MSA_ERR_INVALID_ARG, "msa_stream_read: bytes must be a positive multiple of 16");
  MSA_REQUIRE(uintptr_t(buf) % 16 == 0, MSA_ERR_INVALID_ARG, "msa_stream_read: buffer must be 16-byte aligned");
  int dev = 0, n_cu = 0;
  MSA_HIP_CHECK(hipGetDevice(&dev));
  MSA_HIP_CHECK(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  const int64_t n_vec = bytes / 16;
  const int64_t need = (n_vec + 64 * SR_U * (SR_THREADS / 64) - 1) / (64 * SR_U * (SR_THREADS / 64));
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(int64_t(n_cu), need));
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(grid)), dim3(SR_THREADS), 0, as_stream(stream),
                     static_cast<const uint4*>(buf), n_vec, sink);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}
