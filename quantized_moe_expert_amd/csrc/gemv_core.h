// Building blocks of the IQ4_NL dequant-GEMV kernels (decode path).
//
// Activations are staged once per workgroup in LDS as bf16 (hi, lo) pairs in the order of
// the code bytes: for block kb of token u, dwords [0,16) are the hi pairs (x_j, x_{j+16}) and
// [16,32) the lo pairs, padded to kXStride dwords so that lanes reading consecutive blocks
// with ds_read_b128 fall into distinct banks.  A lane then holds the pairs of its own blocks
// in registers and reuses them for every weight row it visits.
#pragma once
#include "common.h"

namespace moe {

constexpr int kXStride = 36;        // dwords per (token, block) slot in LDS

// Stage rows of activations into LDS, in two phases so that a wave can issue other loads in
// between: load() issues the global loads into registers, store() converts to bf16 (hi, lo)
// pairs and writes LDS.  Vector-memory loads of a wave complete in issue order, so the
// activation loads (L2 hits) must be issued before the weight stream (HBM) for store() not
// to wait on the weights.  Row u (< n_rows) comes from src_row(u) (K = 32 * NB floats),
// scaled by scale(u); rows n_rows .. n_alloc-1 and blocks NB .. NBP-1 of every row are zero
// (a row occupies NBP block slots).  Work unit = a quarter block (pairs 4q..4q+3 of block
// kb: two float4 loads).  Requires n_alloc * NBP * 4 <= blockDim.x * UPT.
template <int UPT>
struct Stager {
  float4 a[UPT], b[UPT];
  float sc[UPT];
  int units;

  template <class RowFn, class ScaleFn>
  __device__ __forceinline__ void load(int NB, int NBP, int n_rows, int n_alloc, RowFn src_row,
                                       ScaleFn scale) {
    units = n_alloc * NBP * 4;
    // every load is issued (an invalid unit reads row 0 / block 0 and is zeroed by a select):
    // a static load count lets the compiler wait on exactly the loads each use needs
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int unit = threadIdx.x + (int)blockDim.x * i;
      const int ukb = unit >> 2, q = unit & 3;
      const int u = ukb / NBP, kb = ukb - u * NBP;
      const bool ok = unit < units && u < n_rows && kb < NB;
      const float* r = src_row(ok ? u : 0) + (ok ? kb * 32 + 4 * q : 0);
      a[i] = *reinterpret_cast<const float4*>(r);
      b[i] = *reinterpret_cast<const float4*>(r + 16);
      sc[i] = ok ? scale(u) : -0.0f;      // sign bit marks an invalid unit (zeroed in store)
    }
  }

  __device__ __forceinline__ void store(uint32_t* s_x) const {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int unit = threadIdx.x + (int)blockDim.x * i;
      if (unit < units) {
        const int ukb = unit >> 2, q = unit & 3;
        const bool ok = !__builtin_signbit(sc[i]);
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 av = ok ? a[i] : z, bv = ok ? b[i] : z;
        uint4 hi, lo;
        split_pair(av.x * sc[i], bv.x * sc[i], hi.x, lo.x);
        split_pair(av.y * sc[i], bv.y * sc[i], hi.y, lo.y);
        split_pair(av.z * sc[i], bv.z * sc[i], hi.z, lo.z);
        split_pair(av.w * sc[i], bv.w * sc[i], hi.w, lo.w);
        uint4* d = reinterpret_cast<uint4*>(s_x + ukb * kXStride + 4 * q);
        d[0] = hi;
        d[4] = lo;
      }
    }
  }
};

// A lane's activation pairs of ONE of its blocks (kb = lig + LPR * b) for MT tokens, read
// from rows of NBP = LPR * BPL block slots (zero-padded), so every read is unconditional.
// Keeping one block at a time bounds the registers (32 * MT) whatever the row length.
template <int MT>
struct XBlock {
  uint32_t h[MT][16];
  uint32_t l[MT][16];

  __device__ __forceinline__ void load(const uint32_t* s_x, int nbp, int kb) {
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const uint4* p = reinterpret_cast<const uint4*>(s_x + (u * nbp + kb) * kXStride);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 vh = p[q];
        const uint4 vl = p[4 + q];
        h[u][4 * q] = vh.x; h[u][4 * q + 1] = vh.y; h[u][4 * q + 2] = vh.z; h[u][4 * q + 3] = vh.w;
        l[u][4 * q] = vl.x; l[u][4 * q + 1] = vl.y; l[u][4 * q + 2] = vl.z; l[u][4 * q + 3] = vl.w;
      }
    }
  }
};

// A copy of a raw block that the compiler must treat as new on every use: the lookups of a
// block are then formed where it is multiplied instead of being hoisted out of the token
// loops (which keeps 16 table addresses a block live for the whole kernel).
__device__ __forceinline__ RawBlock fresh(const RawBlock& r) {
  RawBlock o = r;
  asm volatile("" : "+v"(o.w[0]), "+v"(o.w[1]), "+v"(o.w[2]), "+v"(o.w[3]), "+v"(o.w[4]));
  return o;
}

// acc[u] += d * sum_j (c[q_j] x_j + c[q_{j+16}] x_{j+16}) over one block, for MT tokens.
template <int MT>
__device__ __forceinline__ void block_dot(const RawBlock& raw, bool odd, const uint32_t* s_tab,
                                          const XBlock<MT>& x, float (&acc)[MT]) {
  const float d = block_scale(raw, odd);
  uint32_t c[4];
  block_codes(raw, odd, c);
  float bs[MT];
#pragma unroll
  for (int u = 0; u < MT; ++u) bs[u] = 0.0f;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const uint32_t ent = s_tab[(c[cc] >> (8 * y)) & 0xFFu];
      const int j = 4 * cc + y;
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        bs[u] = dot2_bf16(ent, x.h[u][j], bs[u]);
        bs[u] = dot2_bf16(ent, x.l[u][j], bs[u]);
      }
    }
#pragma unroll
  for (int u = 0; u < MT; ++u) acc[u] = fmaf(d, bs[u], acc[u]);
}

// acc[p][u] over all PASSES rows and the lane's BPL blocks: block-major, so only one block
// of activations is live at a time; a scheduling barrier between blocks keeps the compiler
// from hoisting every block's LDS reads.
template <int PASSES, int LPR, int BPL, int MT>
__device__ __forceinline__ void rows_dot(const RawBlock (&raw)[PASSES][BPL], bool odd,
                                         const uint32_t* s_tab, const uint32_t* s_x, int lig,
                                         float (&acc)[PASSES][MT]) {
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[p][u] = 0.0f;
#pragma unroll
  for (int b = 0; b < BPL; ++b) {
    XBlock<MT> x;
    x.load(s_x, LPR * BPL, lig + LPR * b);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) block_dot<MT>(fresh(raw[p][b]), odd, s_tab, x, acc[p]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace moe
