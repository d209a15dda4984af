// IQ4_NL encode / decode (format of PocketLLM "Xing4.0-29B-A4B", section "Overview": 32
// weights in 18 bytes, one fp16 scale plus 32 four-bit codebook indices).
//
// Encoder rule: d = fp16_RNE(fp32(max|w|) / 127) (IEEE fp32 division), and each weight
// takes the codebook entry nearest to w / d, measured against the stored d, ties to the
// lower index.  Every midpoint d * (c_j + c_{j+1}) / 2 is exact in fp32, so the index is
// the count of midpoints strictly below w, with no rounding anywhere.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ void __launch_bounds__(256) quantize_kernel(const float* __restrict__ w,
                                                       int64_t n_blocks,
                                                       uint8_t* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_blocks) return;
  const float4* src = reinterpret_cast<const float4*>(w + b * kBlock);
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 f = src[i];
    v[4 * i + 0] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(v[i]));
  const __half dh = __float2half_rn(a / 127.0f);
  const float d = __half2float(dh);
  float mid[15];
#pragma unroll
  for (int j = 0; j < 15; ++j) mid[j] = d * (0.5f * (float)(codebook_at(j) + codebook_at(j + 1)));
  uint32_t q[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 15; ++j) c += (mid[j] < v[i]) ? 1u : 0u;
    q[i] = c;
  }
  // 18 bytes as nine 2-byte stores (block starts are 2-byte aligned)
  uint16_t* dst = reinterpret_cast<uint16_t*>(out + b * kBlockBytes);
  dst[0] = __half_as_ushort(dh);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t lo = q[2 * j] | (q[2 * j + 16] << 4);
    const uint32_t hi = q[2 * j + 1] | (q[2 * j + 17] << 4);
    dst[1 + j] = (uint16_t)(lo | (hi << 8));
  }
}

__global__ void __launch_bounds__(256) dequantize_kernel(const uint8_t* __restrict__ blk,
                                                         int64_t n_blocks,
                                                         float* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_blocks) return;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(blk + b * kBlockBytes);
  const float d = __half2float(__ushort_as_half(src[0]));
  float4* dst = reinterpret_cast<float4*>(out + b * kBlock);
  float v[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t two = src[1 + j];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t byte = (two >> (8 * h)) & 0xFF;
      v[2 * j + h] = d * (float)codebook_at(byte & 15);
      v[2 * j + h + 16] = d * (float)codebook_at(byte >> 4);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

hipError_t launch_quantize(const float* w, int64_t n_blocks, uint8_t* out, hipStream_t s) {
  if (n_blocks == 0) return hipSuccess;
  const int64_t grid = (n_blocks + 255) / 256;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)grid), dim3(256), 0, s, w, n_blocks, out);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* blk, int64_t n_blocks, float* out, hipStream_t s) {
  if (n_blocks == 0) return hipSuccess;
  const int64_t grid = (n_blocks + 255) / 256;
  hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)grid), dim3(256), 0, s, blk, n_blocks,
                     out);
  return hipGetLastError();
}

}  // namespace moe
