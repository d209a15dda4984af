// Seeded synthetic inputs on the GPU: the device twin of synth/generator.py.
// Philox4x32-10 (Salmon et al., SC 2011) + Irwin-Hall sum of eight 16-bit halves; integer
// arithmetic until one fp32 multiply, so host and device agree bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_synth.h"

namespace {

constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
constexpr uint32_t kKey1 = 0x4D6F4531u;

__device__ __forceinline__ void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t p0 = (uint64_t)kM0 * c[0];
    const uint64_t p1 = (uint64_t)kM1 * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[1] = (uint32_t)p1;
    c[3] = (uint32_t)p0;
    c[0] = n0;
    c[2] = n2;
  }
}

__global__ void normal_kernel(float* out, int64_t n, uint64_t start, uint32_t seed, uint32_t c2,
                              uint32_t c3, float scale) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const uint64_t i = start + (uint64_t)j;
  uint32_t c[4] = {(uint32_t)i, (uint32_t)(i >> 32), c2, c3};
  philox10(c, seed, kKey1);
  int32_t s = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) s += (int32_t)(c[w] & 0xFFFFu) + (int32_t)(c[w] >> 16);
  out[j] = (float)(s - 262140) * scale;
}

__global__ void words_kernel(uint32_t* out, int64_t n, uint64_t start, uint32_t seed,
                             uint32_t key1, uint32_t c2, uint32_t c3) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const uint64_t i = start + (uint64_t)j;
  uint32_t c[4] = {(uint32_t)i, (uint32_t)(i >> 32), c2, c3};
  philox10(c, seed, key1);
#pragma unroll
  for (int w = 0; w < 4; ++w) out[4 * j + w] = c[w];
}

}  // namespace

extern "C" int32_t synth_normal_f32(float* out, int64_t n, uint64_t start, uint32_t seed,
                                    uint32_t c2, uint32_t c3, float scale, hipStream_t stream) {
  if (n <= 0) return 0;
  if (!out) return (int32_t)hipErrorInvalidValue;
  const int64_t grid = (n + 255) / 256;
  if (grid > 0x7FFFFFFF) return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(normal_kernel, dim3((unsigned)grid), dim3(256), 0, stream, out, n, start,
                     seed, c2, c3, scale);
  return (int32_t)hipGetLastError();
}

extern "C" int32_t synth_philox_words(uint32_t* out, int64_t n, uint64_t start, uint32_t seed,
                                      uint32_t key1, uint32_t c2, uint32_t c3,
                                      hipStream_t stream) {
  if (n <= 0) return 0;
  if (!out) return (int32_t)hipErrorInvalidValue;
  const int64_t grid = (n + 255) / 256;
  if (grid > 0x7FFFFFFF) return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(words_kernel, dim3((unsigned)grid), dim3(256), 0, stream, out, n, start,
                     seed, key1, c2, c3);
  return (int32_t)hipGetLastError();
}
