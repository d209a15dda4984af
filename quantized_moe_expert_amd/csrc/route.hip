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

// Partial logits P[z][T, E] = X[T, H] * W[E, H]^T over K range [z*kspan, (z+1)*kspan): 64x64
// tiles, 4x4 outputs a thread, K steps of 16 with double-buffered LDS tiles (the next step's
// global loads are in flight while the current step is multiplied).  Splitting K gives a
// chunk of T = 2048 tokens and 64 experts ~500 workgroups instead of 32.
__global__ void __launch_bounds__(256) logits_gemm_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          int T, int H, int E, int kspan,
                                                          float* __restrict__ part) {
  __shared__ float As[2][16][64 + 4];
  __shared__ float Bs[2][16][64 + 4];
  const int tid = threadIdx.x;
  const int tm = blockIdx.y * 64, tn = blockIdx.x * 64;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const bool aok = tm + lr < T, bok = tn + lr < E;
  const int kz = blockIdx.z * kspan;
  const float* ap = x + (size_t)(aok ? tm + lr : 0) * H + kz + lk;
  const float* bp = wr + (size_t)(bok ? tn + lr : 0) * H + kz + lk;
  float4 a = *reinterpret_cast<const float4*>(ap);
  float4 b = *reinterpret_cast<const float4*>(bp);
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  int buf = 0;
  for (int k0 = 0; k0 < kspan; k0 += 16) {
    const float4 av = aok ? a : z, bv = bok ? b : z;
    As[buf][lk + 0][lr] = av.x; As[buf][lk + 1][lr] = av.y;
    As[buf][lk + 2][lr] = av.z; As[buf][lk + 3][lr] = av.w;
    Bs[buf][lk + 0][lr] = bv.x; Bs[buf][lk + 1][lr] = bv.y;
    Bs[buf][lk + 2][lr] = bv.z; Bs[buf][lk + 3][lr] = bv.w;
    __syncthreads();   // this buffer written; the other one was last read two steps ago
    if (k0 + 16 < kspan) {
      a = *reinterpret_cast<const float4*>(ap + k0 + 16);
      b = *reinterpret_cast<const float4*>(bp + k0 + 16);
    }
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av4[4], bv4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av4[i] = As[buf][kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv4[j] = Bs[buf][kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av4[i], bv4[j], acc[i][j]);
    }
    buf ^= 1;
  }
  float* out = part + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = tm + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tn + tx * 4 + j;
      if (e < E) out[(size_t)t * E + e] = acc[i][j];
    }
  }
}

// One wave per token: logits = sum of the ks partial products in split order (+ bias),
// written out, then the top-k of them (read back from LDS).
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ part, int ks,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ logits, int T, int E,
                                                   int k, int gating, int renorm,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  __shared__ float s_l[4][kMaxE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  for (int e = lane; e < E; e += 64) {
    float v = part[(size_t)t * E + e];
    for (int z = 1; z < ks; ++z) v += part[((size_t)z * T + t) * E + e];
    if (bias) v += bias[e];
    s_l[wave][e] = v;
    logits[(size_t)t * E + e] = v;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
  wave_topk(s_l[wave], E, k, gating, renorm, ids + (size_t)t * k, w + (size_t)t * k);
}

hipError_t launch_topk(const Shape& sh, const float* logits, int T, int32_t* ids, float* w,
                       hipStream_t s) {
  if (T == 0) return hipSuccess;
  // logits are complete: a single "partial", no bias, rewritten in place
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, 1, nullptr,
                     const_cast<float*>(logits), T, sh.E, sh.k, sh.gating, sh.renorm, ids, w);
  return hipGetLastError();
}

// K splits of the logits GEMM: enough workgroups to cover every CU twice, K a multiple of
// 16 per split, the partials fitting `cap_floats`.
int route_splits(const Shape& sh, int T, size_t cap_floats) {
  const int tiles = ((sh.E + 63) / 64) * ((T + 63) / 64);
  int ks = 1;
  while (tiles * ks * 2 <= 2 * device_cu_count() && sh.H % (ks * 2 * 16) == 0 &&
         (size_t)ks * 2 * T * sh.E <= cap_floats)
    ks *= 2;
  return ks;
}

hipError_t launch_route(const Shape& sh, const float* x, const float* wr, const float* bias,
                        int T, int32_t* ids, float* w, float* logits, float* partial,
                        size_t partial_floats, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T <= kSmallT) {
    hipError_t e = launch_router_rows(sh, x, wr, bias, T, -1.0f, logits, nullptr, s);
    if (e != hipSuccess) return e;
    return launch_topk(sh, logits, T, ids, w, s);
  }
  const int ks = partial ? route_splits(sh, T, partial_floats) : 1;
  float* part = ks > 1 ? partial : logits;
  hipLaunchKernelGGL(logits_gemm_kernel, dim3((sh.E + 63) / 64, (T + 63) / 64, ks), dim3(256),
                     0, s, x, wr, T, sh.H, sh.E, sh.H / ks, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, part, ks, bias, logits, T,
                     sh.E, sh.k, sh.gating, sh.renorm, ids, w);
  return hipGetLastError();
}

}  // namespace moe
