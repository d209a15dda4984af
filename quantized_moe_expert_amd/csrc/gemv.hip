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
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kGemvThreads = 256;
constexpr int kPasses = 8;

// e_slot-th expert (0-based, in index order) whose slot range is non-empty; -1 if none.
__device__ int find_active_expert(const int32_t* __restrict__ offsets, int n_bins, int e_slot) {
  const int lane = threadIdx.x & 63;
  int seen = 0;
  for (int base = 0; base < n_bins; base += 64) {
    const int e = base + lane;
    const bool ne = e < n_bins && offsets[e + 1] > offsets[e];
    const uint64_t mask = __ballot(ne);
    const int cnt = __popcll(mask);
    if (e_slot < seen + cnt) {
      // position of the (e_slot - seen)-th set bit
      int want = e_slot - seen;
      uint64_t m = mask;
      for (int i = 0; i < want; ++i) m &= m - 1;
      return base + __ffsll((long long)m) - 1;
    }
    seen += cnt;
  }
  return -1;
}

template <int LPR, int BPL, int MT, bool GATEUP>
__global__ void __launch_bounds__(kGemvThreads) gemv_kernel(
    const uint8_t* __restrict__ bank, int64_t stride, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pairs, const float* __restrict__ in,
    float* __restrict__ out, int H, int F, int E, int S, int k, int T) {
  constexpr int RPP = 64 / LPR;               // rows per pass per wave
  constexpr int WROWS = kPasses * RPP;        // weight rows per wave
  constexpr int OROWS = GATEUP ? WROWS / 2 : WROWS;
  __shared__ uint32_t s_tab[256];
  __shared__ int s_expert;

  const int tid = threadIdx.x;
  s_tab[tid] = pair_table_entry(tid);
  if (tid < 64) {
    const int e = find_active_expert(offsets, E + S, blockIdx.y);
    if (tid == 0) s_expert = e;
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

  const int slot0 = offsets[e];
  const int m = offsets[e + 1] - slot0;
  const int P = T * k;

  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane / LPR, lig = lane % LPR;
  const bool odd = (lig & 1) != 0;                   // block parity == lane parity
  const int orow0 = (blockIdx.x * (kGemvThreads / 64) + wave) * OROWS;

  // weight rows visited in each pass, and whether they exist
  const uint8_t* rowp[kPasses];
  bool rowok[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int i = p * RPP + g;
    int r, wr;
    if (GATEUP) {
      r = orow0 + (i < OROWS ? i : i - OROWS);
      wr = (i < OROWS ? 0 : F) + r;
    } else {
      r = orow0 + i;
      wr = r;
    }
    rowok[p] = r < NOUT;
    rowp[p] = mat + (int64_t)(rowok[p] ? wr : 0) * row_bytes;
  }

  for (int t0 = 0; t0 < m; t0 += MT) {
    // activations of this lane's blocks, split into bf16 hi/lo pairs (x_j, x_{j+16})
    uint32_t xh[MT][BPL][16], xl[MT][BPL][16];
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const int s = slot0 + t0 + u;
      const bool tok_ok = (t0 + u) < m;
      const float* src;
      if (GATEUP) {
        const int tok = !tok_ok ? 0 : (s < P ? sorted_pairs[s] / k : (s - P) % T);
        src = in + (int64_t)tok * H;
      } else {
        src = in + (int64_t)(tok_ok ? s : slot0) * F;
      }
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const int kb = lig + LPR * b;
        float v[32];
        if (kb < NB) {
          const float4* q = reinterpret_cast<const float4*>(src + kb * 32);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float4 f = q[i];
            v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 32; ++i) v[i] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) split_pair(v[j], v[j + 16], xh[u][b][j], xl[u][b][j]);
      }
    }

    // fetch every block this lane needs for all passes, then compute
    RawBlock raw[kPasses][BPL];
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const int kb = lig + LPR * b;
        if (rowok[p] && kb < NB) raw[p][b] = load_block(rowp[p], kb);
        else raw[p][b] = RawBlock{{0u, 0u, 0u, 0u, 0u}};
      }

    float acc[kPasses][MT];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
#pragma unroll
      for (int u = 0; u < MT; ++u) acc[p][u] = 0.0f;
#pragma unroll
      for (int b = 0; b < BPL; ++b) {
        const float d = block_scale(raw[p][b], odd);       // 0 for absent blocks
        uint32_t c[4];
        block_codes(raw[p][b], odd, c);
        float bs[MT];
#pragma unroll
        for (int u = 0; u < MT; ++u) bs[u] = 0.0f;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            const uint32_t ent = s_tab[(c[cc] >> (8 * y)) & 0xFFu];
            const int j = 4 * cc + y;
#pragma unroll
            for (int u = 0; u < MT; ++u) {
              bs[u] = dot2_bf16(ent, xh[u][b][j], bs[u]);
              bs[u] = dot2_bf16(ent, xl[u][b][j], bs[u]);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[p][u] = fmaf(d, bs[u], acc[p][u]);
      }
    }

#pragma unroll
    for (int p = 0; p < kPasses; ++p)
#pragma unroll
      for (int u = 0; u < MT; ++u) acc[p][u] = group_sum(acc[p][u], LPR);

    if (lig == 0) {
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        if (t0 + u >= m) continue;
        const int64_t s = slot0 + t0 + u;
        if (GATEUP) {
#pragma unroll
          for (int p = 0; p < kPasses / 2; ++p) {
            const int r = orow0 + p * RPP + g;
            if (r < F) out[s * F + r] = silu(acc[p][u]) * acc[p + kPasses / 2][u];
          }
        } else {
#pragma unroll
          for (int p = 0; p < kPasses; ++p) {
            const int r = orow0 + p * RPP + g;
            if (r < H) out[s * H + r] = acc[p][u];
          }
        }
      }
    }
  }
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
  hipLaunchKernelGGL((gemv_kernel<LPR, BPL, MT, GU>), grid, dim3(kGemvThreads), 0, s, bank,
                     stride, offsets, sp, in, out, sh.H, sh.F, sh.E, sh.S, sh.k, T);
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
  const int orows_wave = gu ? kPasses * rpp / 2 : kPasses * rpp;
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
