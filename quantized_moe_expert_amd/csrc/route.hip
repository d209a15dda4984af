// Router scoring, gating and top-k selection.
//
// PocketLLM "Xing4.0-29B-A4B", section "Overview": a sigmoid-routed MoE, 64 routed experts
// activated top-4 plus one shared; Red Lite "What we learned", section "1. The idea": 512
// experts of which a token uses 10 (softmax gating here); Xolotl, "Why build an engine at
// all": the router picks 6 of 384.  Selection: the k largest logits in descending order,
// ties to the lower expert index, a NaN logit below every number.  Sigmoid and softmax
// are monotone, so selecting on logits equals selecting on scores.
//
// Logits: fp32, fp32 accumulation.  Small batches (decode) use one wave per expert row
// (a GEMV that streams W_r once); larger batches use an LDS-tiled fp32 GEMM.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kSmallT = 16;

// One wave per expert; all T (<= 16) tokens at once; W_r read once.
__global__ void __launch_bounds__(256) logits_small_kernel(const float* __restrict__ x,
                                                           const float* __restrict__ wr,
                                                           const float* __restrict__ bias,
                                                           int T, int H, int E,
                                                           float* __restrict__ logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  if (e >= E) return;
  float acc[kSmallT];
#pragma unroll
  for (int t = 0; t < kSmallT; ++t) acc[t] = 0.0f;
  const float4* wrow = reinterpret_cast<const float4*>(wr + (size_t)e * H);
  const int H4 = H >> 2;
  for (int h4 = lane; h4 < H4; h4 += 64) {
    const float4 w = wrow[h4];
#pragma unroll
    for (int t = 0; t < kSmallT; ++t) {
      if (t < T) {
        const float4 v = reinterpret_cast<const float4*>(x + (size_t)t * H)[h4];
        float a = acc[t];
        a = fmaf(w.x, v.x, a);
        a = fmaf(w.y, v.y, a);
        a = fmaf(w.z, v.z, a);
        a = fmaf(w.w, v.w, a);
        acc[t] = a;
      }
    }
  }
  const float b = bias ? bias[e] : 0.0f;
#pragma unroll
  for (int t = 0; t < kSmallT; ++t) {
    if (t < T) {
      const float s = group_sum(acc[t], 64);
      if (lane == 0) logits[(size_t)t * E + e] = s + b;
    }
  }
}

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

// Order-preserving key: larger key = earlier in the selection.  NaN -> 0 (below -inf);
// -0 is treated as +0 (IEEE equality, so the lower index wins the tie).
__device__ __forceinline__ uint32_t order_bits(float v) {
  if (v != v) return 0u;
  if (v == 0.0f) v = 0.0f;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int m = 1; m < 64; m <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

constexpr int kMaxE = 1024;
constexpr int kKeysPerLane = kMaxE / 64;

// One wave per token: k rounds of a wave-wide max over (order_bits(logit), ~index).
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int T,
                                                   int E, int k, int gating, int renorm,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;
  uint64_t key[kKeysPerLane];
#pragma unroll
  for (int i = 0; i < kKeysPerLane; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? (((uint64_t)order_bits(l[e]) << 32) | (uint32_t)(0xFFFFFFFFu - e)) : 0ull;
  }
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    if ((e & 63) == lane) {
#pragma unroll
      for (int i = 0; i < kKeysPerLane; ++i)
        if (i == (e >> 6)) key[i] = 0ull;
    }
    if (lane == j) my_e = e;
  }
  const bool mine = lane < k;
  const float v = mine ? l[my_e] : 0.0f;
  float s;
  if (gating == 0) {
    s = mine ? 1.0f / (1.0f + expf(-v)) : 0.0f;
  } else {
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, l[e]);
    m = wave_max_f(m);
    float z = 0.0f;
    for (int e = lane; e < E; e += 64) z += expf(l[e] - m);
    z = group_sum(z, 64);
    s = mine ? expf(v - m) / z : 0.0f;
  }
  if (renorm) {
    const float tot = group_sum(s, 64);
    s = s / tot;
  }
  if (mine) {
    ids[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = s;
  }
}

hipError_t launch_route(const Shape& sh, const float* x, const float* wr, const float* bias,
                        int T, int32_t* ids, float* w, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T <= kSmallT) {
    hipLaunchKernelGGL(logits_small_kernel, dim3((sh.E + 3) / 4), dim3(256), 0, s, x, wr, bias,
                       T, sh.H, sh.E, logits);
  } else {
    hipLaunchKernelGGL(logits_gemm_kernel, dim3((sh.E + 63) / 64, (T + 63) / 64), dim3(256), 0,
                       s, x, wr, bias, T, sh.H, sh.E, logits);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, sh.E, sh.k,
                     sh.gating, sh.renorm, ids, w);
  return hipGetLastError();
}

}  // namespace moe
