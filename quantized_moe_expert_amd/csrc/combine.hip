// Weighted combine and the weight-free RMSNorm glue.
//
// Combine (PocketLLM "Xing4.0-29B-A4B", page section "Where the detail is": deterministic route
// reduction): y_t = sum_{j<k} w_tj * o[slot(t, j)] + o[shared slot of t] (+ residual), summed
// in exactly that order by one thread per output element -- no atomics.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ o,
                                                      const int32_t* __restrict__ pair_slot,
                                                      const float* __restrict__ w, int T,
                                                      int k, int S, int H,
                                                      const float* residual, float* y) {
  const int t = blockIdx.x;
  const int h4 = blockIdx.y * 256 + threadIdx.x;
  if (h4 * 4 >= H) return;
  const size_t H4 = H >> 2;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const int slot = pair_slot[(size_t)t * k + j];
    const float4 v = reinterpret_cast<const float4*>(o)[(size_t)slot * H4 + h4];
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  for (int sidx = 0; sidx < S; ++sidx) {
    const size_t slot = (size_t)T * k + (size_t)sidx * T + t;
    const float4 v = reinterpret_cast<const float4*>(o)[slot * H4 + h4];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (residual) {
    const float4 r = reinterpret_cast<const float4*>(residual)[(size_t)t * H4 + h4];
    acc.x += r.x; acc.y += r.y; acc.z += r.z; acc.w += r.w;
  }
  reinterpret_cast<float4*>(y)[(size_t)t * H4 + h4] = acc;
}

// One workgroup per row: y = x / sqrt(mean(x^2) + eps).  Each thread reads and writes only
// its own elements, so y may alias x.
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* x, int H, float eps,
                                                      float* y) {
  __shared__ float s_part[4];
  const int t = blockIdx.x;
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)t * H);
  float ss = 0.0f;
  for (int h4 = threadIdx.x; h4 < (H >> 2); h4 += 256) {
    const float4 v = xr[h4];
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  ss = group_sum(ss, 64);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  float4* yr = reinterpret_cast<float4*>(y + (size_t)t * H);
  for (int h4 = threadIdx.x; h4 < (H >> 2); h4 += 256) {
    const float4 v = xr[h4];
    yr[h4] = make_float4(v.x * r, v.y * r, v.z * r, v.w * r);
  }
}

hipError_t launch_combine(const Shape& sh, const float* o, const int32_t* pair_slot,
                          const float* w, int T, const float* residual, float* y,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(T, (sh.H / 4 + 255) / 256), dim3(256), 0, s, o,
                     pair_slot, w, T, sh.k, sh.S, sh.H, residual, y);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, int T, int H, float eps, float* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, s, x, H, eps, y);
  return hipGetLastError();
}

}  // namespace moe
