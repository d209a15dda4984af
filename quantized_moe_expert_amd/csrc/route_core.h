// Top-k selection and gating weights of one token by one wave.
//
// Selection (PocketLLM "Xing4.0-29B-A4B", "Overview": top-4 of 64 sigmoid-routed experts;
// Red Lite "1. The idea": 10 of 512; Xolotl "Why build an engine at all": 6 of 384): the k
// largest logits in descending order, ties to the lower expert index, NaN below every
// number.  k rounds of a wave-wide maximum of the order-preserving logit bits, then the
// lowest expert index among the lanes holding that maximum (DPP reductions).
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

constexpr int kMaxE = 1024;

// Wave-wide max / min of a 32-bit unsigned value and max of a float: a DPP butterfly inside
// each row of 16 lanes, then the four row results read back with readlane (no LDS round trip).
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppXor1, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppXor2, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppHalfMirror, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kDppMirror, 0xF, 0xF, false));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return op(op(a, b), op(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
}
__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  const int iv = __builtin_bit_cast(int, v);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// KPL logits a lane (experts lane + 64 i).  Each round: the wave-wide largest key (order bits
// + 1, so that a NaN logit, key 1, stays selectable and 0 marks "taken / absent"), then the
// lowest expert index among the lanes holding it.
template <int KPL>
__device__ __forceinline__ int wave_select(const float* __restrict__ l, int E, int k) {
  const int lane = threadIdx.x & 63;
  uint32_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? order_bits(l[e]) + 1u : 0u;
  }
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    uint32_t b = 0;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (key[i] > b) { b = key[i]; bi = i; }             // strict: the lower index wins ties
    const uint32_t m = wave_max_u32(b);
    const uint32_t cand = (b == m && b != 0u) ? (uint32_t)(lane + 64 * bi) : 0xFFFFFFFFu;
    const int e = (int)wave_min_u32(cand);
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (lane + 64 * i == e) key[i] = 0u;
    if (lane == j) my_e = e;
  }
  return my_e;
}

// The target-th member, in expert-index order, of the top-k set of one token's logits (the
// set wave_select picks: the k largest keys, ties to the lower index), or -1 past the set;
// wave-uniform.  No order or weights: the k-th largest key is found bit by bit from the top
// (32 rounds of a compare and a ballot count), which is far shorter than k rounds of
// wave-wide arg-max when only membership is needed.
template <int KPL>
__device__ __forceinline__ int wave_topk_member(const float* __restrict__ l, int E, int k,
                                                int target) {
  const int lane = threadIdx.x & 63;
  uint32_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? order_bits(l[e]) + 1u : 0u;
  }
  // tau = the largest value with at least k keys >= tau: the k-th largest key
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= k) tau = cand;
  }
  int need = k;                                   // members equal to tau, lowest index first
#pragma unroll
  for (int i = 0; i < KPL; ++i) need -= __popcll(__ballot(key[i] > tau));
  int seen = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    uint64_t eq = __ballot(key[i] == tau && tau != 0u);
    uint64_t take = 0;
    while (need > 0 && eq) {
      const uint64_t low = eq & (~eq + 1);
      take |= low;
      eq ^= low;
      --need;
    }
    uint64_t sel = __ballot(key[i] > tau) | take;
    const int c = __popcll(sel);
    if (target < seen + c) {
      for (int j = 0; j < target - seen; ++j) sel &= sel - 1;
      return __ffsll((long long)sel) - 1 + 64 * i;
    }
    seen += c;
  }
  return -1;
}

__device__ __forceinline__ int wave_topk_member_any(const float* __restrict__ l, int E, int k,
                                                    int target) {
  if (E <= 64) return wave_topk_member<1>(l, E, k, target);
  if (E <= 128) return wave_topk_member<2>(l, E, k, target);
  if (E <= 256) return wave_topk_member<4>(l, E, k, target);
  if (E <= 512) return wave_topk_member<8>(l, E, k, target);
  return wave_topk_member<16>(l, E, k, target);
}

// Gating weights of the selection my_e (lane j < k holds the j-th selected expert) and the
// writes of ids[j], w[j].
__device__ __forceinline__ void wave_gate(const float* __restrict__ l, int E, int k, int gating,
                                          int renorm, int my_e, int32_t* ids, float* w) {
  const int lane = threadIdx.x & 63;
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
    z = group_sum_dpp<64>(z);
    s = mine ? expf(v - m) / z : 0.0f;
  }
  if (renorm) {
    const float tot = group_sum_dpp<64>(s);
    s = s / tot;
  }
  if (mine) {
    ids[lane] = my_e;
    w[lane] = s;
  }
}

// ids[0..k-1], w[0..k-1] of one token's logits l[0..E-1] (E <= 1024, k <= 32); all 64
// lanes of the wave take part; lanes j < k write entry j.
__device__ __forceinline__ void wave_topk(const float* __restrict__ l, int E, int k, int gating,
                                          int renorm, int32_t* ids, float* w) {
  int my_e;
  if (E <= 64) my_e = wave_select<1>(l, E, k);
  else if (E <= 128) my_e = wave_select<2>(l, E, k);
  else if (E <= 256) my_e = wave_select<4>(l, E, k);
  else if (E <= 512) my_e = wave_select<8>(l, E, k);
  else my_e = wave_select<16>(l, E, k);
  wave_gate(l, E, k, gating, renorm, my_e, ids, w);
}

// wave_topk with the one lane layout of 16 logits a lane (any E <= 1024): a single code path,
// for kernels where the five layouts' code would raise the register count of the whole kernel.
__device__ __forceinline__ void wave_topk_one_layout(const float* __restrict__ l, int E, int k,
                                                     int gating, int renorm, int32_t* ids,
                                                     float* w) {
  wave_gate(l, E, k, gating, renorm, wave_select<16>(l, E, k), ids, w);
}

}  // namespace moe
