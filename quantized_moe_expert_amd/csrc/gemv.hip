// Decode path: grouped dequant-GEMV over the experts a route table uses.
//
// PocketLLM "Xing4.0-29B-A4B", section "Overview": every expert stays resident, read once
// and indexed by expert.  Red Lite "What we learned", section "4. Speculative decoding":
// kernels that decode each weight block once for all token rows that use it (two dot
// products for the price of ~1.06 instead of 1.74).  Here every block is decoded once per
// token tile of up to MT tokens routed to the same expert.
//
// Layout of the work: one workgroup (4 waves) per (active expert, tile of output rows); the
// active expert is found on the device from `offsets`, so the grid is sized from host-known
// bounds only.  Within a wave, groups of LPR lanes share one weight row, each lane owning
// BPL blocks of it (blocks lig, lig + LPR, ...), so one load instruction of the group covers
// LPR consecutive 18-byte blocks of a row: coalesced streaming of the bank.  A lane keeps
// the activations of its blocks in registers as bf16 (hi, lo) pairs and reuses them for all
// PASSES rows it visits; the weights of a row are fetched for all passes before any
// arithmetic, to keep many loads in flight.
//
// Dequantisation in registers: a code byte (indices q_j, q_{j+16}) indexes a 256-entry LDS
// table of bf16 pairs (c[q_j], c[q_{j+16}]) -- exact, |c| <= 127 -- and v_dot2_f32_bf16
// multiplies the pair with the activation pair (x_j, x_{j+16}) twice, once for the hi and once
// for the lo bf16 part of x.  The block sum is scaled by its fp16 d in fp32 and accumulated
// in fp32.  Row sums are reduced across the LPR lanes by a fixed butterfly.
#include <algorithm>

#include "common.h"
#include "gemv_core.h"
#include "kernels.h"

namespace moe {

constexpr int kGemvThreads = 256;
constexpr int kPasses = 8;                 // weight rows a lane group visits (even)
constexpr int kBatchChunk = 4;             // slots a workgroup takes of an expert, 4 < T <= 16
// rows a lane group visits at BPL blocks a lane: half as many for the longest rows, which
// keeps the weight registers of a wave (PASSES x BPL blocks) within two waves a SIMD
constexpr int passes_for(int bpl) { return bpl >= 4 ? kPasses / 2 : kPasses; }

// Work item `item` of the list of (expert, chunk of tch slots) pairs over the experts with
// slots, in index order: e (-1 past the end) and the chunk index.  One wave.  The offsets are
// read 256 bins at a time (four unconditional loads a lane, one memory round trip), not one
// dependent round trip per 64 bins.
__device__ void find_work(const int32_t* __restrict__ offsets, int n_bins, int item, int tch,
                          int& e_out, int& chunk_out) {
  const int lane = threadIdx.x & 63;
  int before = 0;
  for (int base = 0; base < n_bins; base += 256) {
    int cnt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = base + 64 * j + lane;
      const int bb = min(b, n_bins - 1);
      const int m = offsets[bb + 1] - offsets[bb];
      // (masked, not selected: a select makes the compiler branch around the division and
      //  the load, one round trip each)
      cnt[j] = ((m + tch - 1) / tch) & -(int)(b < n_bins);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = cnt[j];
      int incl = c;
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
      }
      const int total = __shfl(incl, 63, 64);
      if (item < before + total) {
        const int lo = before + incl - c;
        const uint64_t mask = __ballot(item >= lo && item < lo + c);
        const int hl = __ffsll((long long)mask) - 1;
        e_out = base + 64 * j + hl;
        chunk_out = item - __shfl(lo, hl, 64);
        return;
      }
      before += total;
    }
  }
  e_out = -1;
  chunk_out = 0;
}

// The work of one (expert, slot chunk) item, MTR tokens a tile.
template <int LPR, int BPL, int MTR, bool GATEUP>
__device__ __forceinline__ void gemv_run(const uint8_t* __restrict__ mat, int64_t row_bytes,
                                         int NB, int NOUT, int K, int F, int H, int T, int k,
                                         int P, int slot0, int m,
                                         const int32_t* __restrict__ sorted_pairs,
                                         const float* __restrict__ in, float* __restrict__ out,
                                         uint32_t* s_x, const uint32_t* s_tab, int* s_row) {
  constexpr int NPASS = passes_for(BPL);
  constexpr int RPP = 64 / LPR;               // rows per pass per wave
  constexpr int WROWS = NPASS * RPP;        // weight rows per wave
  constexpr int OROWS = GATEUP ? WROWS / 2 : WROWS;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane / LPR, lig = lane % LPR;
  const bool odd = (lig & 1) != 0;                   // block parity == lane parity
  const int orow0 = (blockIdx.x * (kGemvThreads / 64) + wave) * OROWS;

  // 1) the token rows of the first tile (a read of sorted_pairs), then every weight load of
  //    this wave, then, once the token rows are known, the activations.  The weight addresses
  //    do not depend on the token rows, so the weights stream during that round trip; loads
  //    complete in issue order, so the activations arrive right behind the weights.  The
  //    weight rows stay in registers for all token tiles
  // the token rows of the first two tiles are read at once (the second tile then needs no
  // read of sorted_pairs of its own)
  constexpr int PRE = 2 * MTR;
  const int sl0 = slot0 + min(tid, PRE - 1);
  // (unconditional, clamped to a routed slot, and a relaxed atomic read so that the compiler
  //  keeps it ahead of the weight loads instead of sinking it to its use)
  const int pair0 =
      GATEUP ? __hip_atomic_load(sorted_pairs + min(sl0, P - 1), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP)
             : 0;
  __builtin_amdgcn_sched_barrier(0);   // ... issued ahead of the weight loads
  RawBlock raw[NPASS][BPL];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int i = p * RPP + g;
    int r, wr;
    if (GATEUP) {
      r = orow0 + (i < OROWS ? i : i - OROWS);
      wr = (i < OROWS ? 0 : F) + r;
    } else {
      r = orow0 + i;
      wr = r;
    }
    const bool ok = r < NOUT;
    const uint8_t* rowp = mat + (int64_t)(ok ? wr : 0) * row_bytes;
    // unconditional loads (a lane past the row end reads a block of the same parity inside
    // it; its activations are zero padding): a static load count, no divergent branches
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
      const int kb = lig + LPR * b;
      raw[p][b] = load_block(rowp, kb < NB ? kb : NB - 2 + (kb & 1));
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // the token rows are used only after every weight load
  if (tid < PRE && tid < m)
    s_row[tid] = GATEUP ? (sl0 < P ? pair0 / k : (sl0 - P) % T) : sl0;
  lds_barrier();
  Stager<4 * MTR> stg;
  // (addresses formed from the kernel argument keep the global address space: global loads,
  //  counted on vmcnt only)
  stg.load(NB, LPR * BPL, min(MTR, m), MTR, [&](int u) { return in + (int64_t)s_row[u] * K; },
           [&](int) { return 1.0f; });

  // 2)-3) per token tile: activations -> LDS (once per workgroup), dequantise and dot.  The
  // first tile is peeled so that its staging waits only on its own (earlier) loads.
  auto tile = [&](int t0, int n_tok) {
    // 3) dequantise and dot
    float acc[NPASS][MTR];
    rows_dot<NPASS, LPR, BPL, MTR>(raw, odd, s_tab, s_x, lig, acc);
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
#pragma unroll
      for (int u = 0; u < MTR; ++u) acc[p][u] = group_sum_dpp<LPR>(acc[p][u]);
    if (lig != 0) return;
#pragma unroll
    for (int u = 0; u < MTR; ++u) {
      if (u >= n_tok) continue;
      const int64_t s = slot0 + t0 + u;
      if (GATEUP) {
#pragma unroll
        for (int p = 0; p < NPASS / 2; ++p) {
          const int r = orow0 + p * RPP + g;
          if (r < F) out[s * F + r] = silu(acc[p][u]) * acc[p + NPASS / 2][u];
        }
      } else {
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
          const int r = orow0 + p * RPP + g;
          if (r < H) out[s * H + r] = acc[p][u];
        }
      }
    }
  };
  stg.store(s_x);
  lds_barrier();
  tile(0, min(MTR, m));
  for (int t0 = MTR; t0 < m; t0 += MTR) {
    const int n_tok = min(MTR, m - t0);
    lds_barrier();
    int rb = t0;                      // the tile's token rows start at s_row[rb]
    if (t0 >= PRE) {
      if (tid < n_tok) {
        const int sl = slot0 + t0 + tid;
        s_row[tid] = GATEUP ? (sl < P ? sorted_pairs[sl] / k : (sl - P) % T) : sl;
      }
      lds_barrier();
      rb = 0;
    }
    stg.load(NB, LPR * BPL, n_tok, MTR, [&](int u) { return in + (int64_t)s_row[rb + u] * K; },
             [&](int) { return 1.0f; });
    stg.store(s_x);
    lds_barrier();
    tile(t0, n_tok);
  }
}

template <int LPR, int BPL, int MT, bool GATEUP>
__global__ void __launch_bounds__(kGemvThreads, 2) gemv_kernel(
    const uint8_t* __restrict__ bank, int64_t stride, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pairs, const float* __restrict__ in,
    float* __restrict__ out, int H, int F, int E, int S, int k, int T, int tch) {
  extern __shared__ __align__(16) uint32_t s_x[];   // MT tokens x LPR*BPL blocks x kXStride dwords
  __shared__ uint32_t s_tab[256];
  __shared__ int s_expert, s_chunk;
  __shared__ int s_row[2 * MT];               // row index of each staged token in `in`

  const int tid = threadIdx.x;
  s_tab[tid] = pair_table_entry(tid);
  if (tid < 64) {
    int e, c;
    find_work(offsets, E + S, blockIdx.y, tch, e, c);
    if (tid == 0) {
      s_expert = e;
      s_chunk = c;
    }
  }
  __syncthreads();
  const int e = s_expert;
  if (e < 0) return;

  const int K = GATEUP ? H : F;
  const int NB = K >> 5;
  const int NOUT = GATEUP ? F : H;
  const int64_t row_bytes = (int64_t)NB * kBlockBytes;
  // expert e: gate [F x H/32 blocks], up [F x H/32], down [H x F/32]
  const uint8_t* wbase = bank + (int64_t)e * stride;
  const uint8_t* mat = GATEUP ? wbase : wbase + 2 * (int64_t)F * ((int64_t)(H >> 5) * kBlockBytes);

  // this workgroup's chunk of the expert's slots (an expert with many tokens is spread over
  // several workgroups, each streaming the weights once for its chunk)
  const int tb = s_chunk * tch;
  const int m_all = offsets[e + 1] - offsets[e];
  if (tb >= m_all) return;
  const int slot0 = offsets[e] + tb;
  const int m = min(tch, m_all - tb);
  const int P = T * k;

  // a chunk holding one token runs the one-token tiles (half the dot products of a tile of 2)
  if (MT > 1 && m == 1)
    gemv_run<LPR, BPL, 1, GATEUP>(mat, row_bytes, NB, NOUT, K, F, H, T, k, P, slot0, m,
                                  sorted_pairs, in, out, s_x, s_tab, s_row);
  else
    gemv_run<LPR, BPL, MT, GATEUP>(mat, row_bytes, NB, NOUT, K, F, H, T, k, P, slot0, m,
                                   sorted_pairs, in, out, s_x, s_tab, s_row);
}

// ---- host-side dispatch ----------------------------------------------------------------

struct GemvGeom {
  int lpr, bpl;
};

// Lanes per row and blocks per lane for NB blocks a row: least idle lanes, BPL <= 4,
// ties to the wider group.
static GemvGeom pick_geom(int NB) {
  GemvGeom best{0, 0};
  int best_waste = 1 << 30;
  const int lprs[5] = {64, 32, 16, 8, 4};
  for (int li = 0; li < 5; ++li) {
    const int lpr = lprs[li];
    const int bpl = (NB + lpr - 1) / lpr;
    if (bpl > 4) continue;
    const int waste = lpr * bpl - NB;
    if (waste < best_waste) {
      best_waste = waste;
      best = GemvGeom{lpr, bpl};
    }
  }
  return best;
}

template <int LPR, int BPL, int MT, bool GU>
static void launch_one(dim3 grid, hipStream_t s, const uint8_t* bank, int64_t stride,
                       const int32_t* offsets, const int32_t* sp, const float* in, float* out,
                       const Shape& sh, int T) {
  const size_t lds = (size_t)MT * LPR * BPL * kXStride * 4;
  // slots a workgroup takes of one expert; work items: (expert, chunk), at most one partial
  // chunk an expert beyond rows / tch
  const int tch = (T > 4 && T <= 16) ? kBatchChunk : T;
  const int rows = T * (sh.k + sh.S);
  // items = sum over the (at most grid.y) bins with slots of ceil(m_e / tch)
  //       <= (rows + bins * (tch - 1)) / tch, and <= rows (an item holds a slot)
  const int64_t bins = grid.y;
  const int64_t bound = std::min<int64_t>(
      {bins + (rows + tch - 1) / tch, (rows + bins * (tch - 1)) / tch, (int64_t)rows});
  grid.y = (unsigned)bound;
  hipLaunchKernelGGL((gemv_kernel<LPR, BPL, MT, GU>), grid, dim3(kGemvThreads), lds, s, bank,
                     stride, offsets, sp, in, out, sh.H, sh.F, sh.E, sh.S, sh.k, T, tch);
}

template <int LPR, int MT, bool GU>
static bool dispatch_bpl(int bpl, dim3 grid, hipStream_t s, const uint8_t* bank, int64_t stride,
                         const int32_t* offsets, const int32_t* sp, const float* in,
                         float* out, const Shape& sh, int T) {
  switch (bpl) {
    case 1: launch_one<LPR, 1, MT, GU>(grid, s, bank, stride, offsets, sp, in, out, sh, T); return true;
    case 2: launch_one<LPR, 2, MT, GU>(grid, s, bank, stride, offsets, sp, in, out, sh, T); return true;
    case 3: launch_one<LPR, 3, MT, GU>(grid, s, bank, stride, offsets, sp, in, out, sh, T); return true;
    case 4: launch_one<LPR, 4, MT, GU>(grid, s, bank, stride, offsets, sp, in, out, sh, T); return true;
  }
  return false;
}

template <int MT, bool GU>
static bool dispatch_lpr(GemvGeom gm, dim3 grid, hipStream_t s, const uint8_t* bank,
                         int64_t stride, const int32_t* offsets, const int32_t* sp,
                         const float* in, float* out, const Shape& sh, int T) {
  switch (gm.lpr) {
    case 64: return dispatch_bpl<64, MT, GU>(gm.bpl, grid, s, bank, stride, offsets, sp, in, out, sh, T);
    case 32: return dispatch_bpl<32, MT, GU>(gm.bpl, grid, s, bank, stride, offsets, sp, in, out, sh, T);
    case 16: return dispatch_bpl<16, MT, GU>(gm.bpl, grid, s, bank, stride, offsets, sp, in, out, sh, T);
    case 8: return dispatch_bpl<8, MT, GU>(gm.bpl, grid, s, bank, stride, offsets, sp, in, out, sh, T);
    case 4: return dispatch_bpl<4, MT, GU>(gm.bpl, grid, s, bank, stride, offsets, sp, in, out, sh, T);
  }
  return false;
}

hipError_t launch_gemv(const Shape& sh, int stage, const uint8_t* bank, int64_t stride,
                       const int32_t* offsets, const int32_t* sorted_pairs, const float* in,
                       float* out, int T, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const bool gu = stage == 0;
  const int K = gu ? sh.H : sh.F;
  const int NOUT = gu ? sh.F : sh.H;
  const GemvGeom gm = pick_geom(K / 32);
  if (gm.lpr == 0) return hipErrorInvalidValue;
  const int rpp = 64 / gm.lpr;
  const int np = passes_for(gm.bpl);
  const int orows_wave = gu ? np * rpp / 2 : np * rpp;
  const int orows_wg = orows_wave * (kGemvThreads / 64);
  const int max_active = (int)std::min<int64_t>((int64_t)sh.E, (int64_t)T * sh.k) + sh.S;
  dim3 grid((NOUT + orows_wg - 1) / orows_wg, max_active);
  const int MT = T > 1 ? 2 : 1;
  bool ok;
  if (MT == 1)
    ok = gu ? dispatch_lpr<1, true>(gm, grid, s, bank, stride, offsets, sorted_pairs, in, out, sh, T)
            : dispatch_lpr<1, false>(gm, grid, s, bank, stride, offsets, sorted_pairs, in, out, sh, T);
  else
    ok = gu ? dispatch_lpr<2, true>(gm, grid, s, bank, stride, offsets, sorted_pairs, in, out, sh, T)
            : dispatch_lpr<2, false>(gm, grid, s, bank, stride, offsets, sorted_pairs, in, out, sh, T);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
