// Router scoring, gating and top-k selection.
//
// PocketLLM "Xing4.0-29B-A4B", section "Overview": a sigmoid-routed MoE, 64 routed experts
// activated top-4 plus one shared; Red Lite "What we learned", section "1. The idea": 512
// experts of which a token uses 10 (softmax gating here); Xolotl, "Why build an engine at
// all": the router picks 6 of 384.  Selection: the k largest logits in descending order,
// ties to the lower expert index, a NaN logit below every number.  Sigmoid and softmax
// are monotone, so selecting on logits equals selecting on scores.
//
// Logits: fp32, fp32 accumulation.  Small batches (decode) use the router-row kernel of the
// fused decode path (a workgroup per expert or few experts, W_r streamed once); larger
// batches use an LDS-tiled fp32 GEMM.
#include "common.h"
#include "kernels.h"
#include "route_core.h"

namespace moe {

constexpr int kSmallT = 16;

// C[T, E] = X[T, H] * W[E, H]^T (+ b): 64x64 tiles, K steps of 16, 4x4 outputs a thread.
__global__ void __launch_bounds__(256) logits_gemm_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          const float* __restrict__ bias,
                                                          int T, int H, int E,
                                                          float* __restrict__ logits) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x;
  const int tm = blockIdx.y * 64, tn = blockIdx.x * 64;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  for (int k0 = 0; k0 < H; k0 += 16) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (tm + lr < T) a = *reinterpret_cast<const float4*>(x + (size_t)(tm + lr) * H + k0 + lk);
    if (tn + lr < E) b = *reinterpret_cast<const float4*>(wr + (size_t)(tn + lr) * H + k0 + lk);
    As[lk + 0][lr] = a.x; As[lk + 1][lr] = a.y; As[lk + 2][lr] = a.z; As[lk + 3][lr] = a.w;
    Bs[lk + 0][lr] = b.x; Bs[lk + 1][lr] = b.y; Bs[lk + 2][lr] = b.z; Bs[lk + 3][lr] = b.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = tm + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tn + tx * 4 + j;
      if (e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.0f);
    }
  }
}

// One wave per token.
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int T,
                                                   int E, int k, int gating, int renorm,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  wave_topk(logits + (size_t)t * E, E, k, gating, renorm, ids + (size_t)t * k, w + (size_t)t * k);
}

hipError_t launch_topk(const Shape& sh, const float* logits, int T, int32_t* ids, float* w,
                       hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, sh.E, sh.k,
                     sh.gating, sh.renorm, ids, w);
  return hipGetLastError();
}

hipError_t launch_route(const Shape& sh, const float* x, const float* wr, const float* bias,
                        int T, int32_t* ids, float* w, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T <= kSmallT) {
    hipError_t e = launch_router_rows(sh, x, wr, bias, T, -1.0f, logits, nullptr, s);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL(logits_gemm_kernel, dim3((sh.E + 63) / 64, (T + 63) / 64), dim3(256), 0,
                       s, x, wr, bias, T, sh.H, sh.E, logits);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_topk(sh, logits, T, ids, w, s);
}

}  // namespace moe
