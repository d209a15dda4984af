// Top-k selection and gating weights of one token by one wave.
//
// Selection (PocketLLM "Xing4.0-29B-A4B", "Overview": top-4 of 64 sigmoid-routed experts;
// Red Lite "1. The idea": 10 of 512; Xolotl "Why build an engine at all": 6 of 384): the k
// largest logits in descending order, ties to the lower expert index, NaN below every
// number.  k rounds of a wave-wide maximum over the 64-bit key (order_bits(logit), ~index).
#pragma once
#include "common.h"

namespace moe {

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

// ids[0..k-1], w[0..k-1] of one token's logits l[0..E-1] (E <= 1024, k <= 32); all 64
// lanes of the wave take part; lanes j < k write entry j.
__device__ __forceinline__ void wave_topk(const float* __restrict__ l, int E, int k, int gating,
                                          int renorm, int32_t* ids, float* w) {
  const int lane = threadIdx.x & 63;
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
    ids[lane] = my_e;
    w[lane] = s;
  }
}

}  // namespace moe
