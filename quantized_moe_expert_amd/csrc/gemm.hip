// Prefill path: grouped GEMM of each expert's slot range against its IQ4_NL weights on bf16
// matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// Xolotl ("DeepSeek-V4.1-Flash at 27 Tokens/s on One RTX 4090"), section "Prompts: fast, and
// exact": a prompt chunk runs each layer's experts as one batched multiply.  Red Lite "What we
// learned", section "3. Speed by release": batched matrix kernels for the experts.
//
// Tiles: 128 slot rows x 128 weight rows per workgroup (4 waves, 2 x 2, 64 x 64 each), K in
// steps of 4 IQ4_NL blocks.  Weight tiles are dequantised once per workgroup into LDS as
// bf16(d * c[q]) (fp32 product, exact; one RNE rounding); activation tiles are copied into
// LDS as they are, in natural K order, with coalesced 16-byte loads.  A code byte holds
// elements j and j+16 of its block, so the dequantisation pairs the lookups of two adjacent
// code bytes: their low nibbles give elements (2m, 2m+1), their high nibbles (16+2m, 17+2m).
// For GATE_UP the workgroup's 128 weight rows are 64 gate rows and the 64 matching up rows,
// arranged so that a lane holds g and u of the same output and applies SwiGLU in registers.
//
// The tile list is built on the device from `offsets` (a prefix of ceil(m_e / 128) over the
// experts); a persistent grid walks it, so nothing depends on host-known expert loads.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kBM = 128;               // slot rows per tile
constexpr int kBN = 128;               // weight rows per tile
constexpr int kKB = 4;                 // IQ4_NL blocks per K step (128 k)
constexpr int kLdsStride = kKB * 16 + 4;   // dwords per LDS row (bf16 pairs + pad)
constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;               // XCDs of an MI355X (each with its own L2)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool GATEUP>
__global__ void __launch_bounds__(kGemmThreads, 2) gemm_kernel(
    const uint8_t* __restrict__ bank, int64_t stride, const int32_t* __restrict__ offsets,
    const uint16_t* __restrict__ in, void* __restrict__ out, int H, int F, int E, int S) {
  __shared__ __attribute__((aligned(16))) uint32_t sA[kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint32_t sB[kBN * kLdsStride];
  __shared__ float2 s_tab[256];
  __shared__ int s_pref[1024];
  __shared__ int s_part[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, c16 = lane & 15;

  s_tab[tid] = make_float2((float)codebook_at(tid & 15), (float)codebook_at(tid >> 4));

  // ---- tile prefix over experts: s_pref[e] = sum_{e' <= e} ceil(m_e' / kBM) ----
  const int nbins = E + S;
  int loc[4];
  int run = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    int t = 0;
    if (e < nbins) t = (offsets[e + 1] - offsets[e] + kBM - 1) / kBM;
    run += t;
    loc[i] = run;
  }
  int incl = run;
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) s_part[wave] = incl;
  __syncthreads();
  int before = incl - run;
  for (int w = 0; w < wave; ++w) before += s_part[w];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if (e < 1024) s_pref[e] = before + loc[i];
  }
  __syncthreads();
  const int total_m = s_pref[nbins - 1];

  const int K = GATEUP ? H : F;
  const int NB = K >> 5;
  const int NKT = NB / kKB;
  const int NT = GATEUP ? F / 64 : H / kBN;
  const int64_t row_bytes = (int64_t)NB * kBlockBytes;
  const int64_t mat_off = GATEUP ? 0 : 2 * (int64_t)F * ((int64_t)(H >> 5) * kBlockBytes);

  // XCD-aware walk: workgroup b runs on XCD b % 8 (dispatch is round-robin over the XCDs);
  // each XCD takes one contiguous range of the tile list, so the workgroups sharing an
  // activation tile (same M tile, consecutive N tiles) and a weight tile (same expert and N
  // tile) meet in the same L2.
  const int n_tiles = total_m * NT;
  const int n_xcd = gridDim.x % kXcds == 0 ? kXcds : 1;
  const int xcd = blockIdx.x % n_xcd, wix = blockIdx.x / n_xcd, nw = gridDim.x / n_xcd;
  const int per_xcd = (n_tiles + n_xcd - 1) / n_xcd;
  const int t_end = min(n_tiles, (xcd + 1) * per_xcd);
  for (int tile = xcd * per_xcd + wix; tile < t_end; tile += nw) {
    const int mt = tile / NT, nt = tile % NT;
    // expert owning M-tile mt: first e with s_pref[e] > mt
    int lo = 0, hi = nbins - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] > mt) hi = mid; else lo = mid + 1;
    }
    const int e = lo;
    const int m0 = (mt - (e ? s_pref[e - 1] : 0)) * kBM;
    const int slot0 = offsets[e];
    const int rows_valid = min(kBM, offsets[e + 1] - slot0 - m0);
    const uint8_t* wmat = bank + (int64_t)e * stride + mat_off;

    // weight rows this thread dequantises (2 units: LDS row n, block kk)
    const uint8_t* brow[2];
    int bn[2], bk[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + kGemmThreads * i;
      const int n = v >> 2;
      bn[i] = n;
      bk[i] = v & 3;
      int wr;
      if (GATEUP) {
        const int half = n >> 6, rr = n & 63;
        wr = (rr < 32) ? (nt * 64 + 32 * half + rr) : (F + nt * 64 + 32 * half + rr - 32);
      } else {
        wr = nt * kBN + n;
      }
      brow[i] = wmat + (int64_t)wr * row_bytes;
    }
    // activation chunks this thread stages (8 units of 16 B: row u >> 4, chunk u & 15).  Rows
    // past the tile's end copy row 0 instead (their output rows are never stored): unconditional
    // loads keep the compiler's load counting exact, so the loads stay in flight
    const uint16_t* arow[8];
    int aoff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = tid + kGemmThreads * i;
      const int r = u >> 4, c = u & 15;
      arow[i] = in + (int64_t)(slot0 + m0 + (r < rows_valid ? r : 0)) * K + 8 * c;
      aoff[i] = r * kLdsStride + 4 * c;
    }

    // 16-row groups of this wave's 64 rows that hold slot rows of the tile
    const int wgroups = min(4, max(0, (rows_valid - wm * 64 + 15) >> 4));
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // K loop, software-pipelined: the global loads of step kt+1 are issued as soon as the
    // registers of step kt are in LDS (activations first, then weights) and stay in flight
    // while the MFMAs of step kt run; barriers order LDS only.
    u32x4_t ga[4][2];   // (a native vector type: whole-struct copies would go through scratch)
    RawBlock gb[2];
    auto gload_a = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        ga[i >> 1][i & 1] = *reinterpret_cast<const u32x4_t*>(arow[i] + kt * kKB * 32);
    };
    auto gload_b = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) gb[i] = load_block(brow[i], kt * kKB + bk[i]);
    };
    gload_a(0);
    gload_b(0);
    for (int kt = 0; kt < NKT; ++kt) {
      lds_barrier();     // every wave is done reading the previous step's tiles
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4_t*>(&sA[aoff[i]]) = ga[i >> 1][i & 1];
      if (kt + 1 < NKT) gload_a(kt + 1);
      // B -> LDS: dequantise to bf16(d * c) in natural K order: dword m < 8 holds elements
      // (2m, 2m+1), the low nibbles of code bytes 2m and 2m+1; dword 8+m their high nibbles
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bool odd = (bk[i] & 1) != 0;
        const float dsc = block_scale(gb[i], odd);
        uint32_t cw[4];
        block_codes(gb[i], odd, cw);
        uint32_t o[16];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float2 ta = s_tab[(cw[m >> 1] >> (16 * (m & 1))) & 0xFFu];
          const float2 tb = s_tab[(cw[m >> 1] >> (16 * (m & 1) + 8)) & 0xFFu];
          o[m] = pack_bf16x2(ta.x * dsc, tb.x * dsc);
          o[8 + m] = pack_bf16x2(ta.y * dsc, tb.y * dsc);
        }
        uint4* dst = reinterpret_cast<uint4*>(&sB[bn[i] * kLdsStride + bk[i] * 16]);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        dst[2] = make_uint4(o[8], o[9], o[10], o[11]);
        dst[3] = make_uint4(o[12], o[13], o[14], o[15]);
      }
      if (kt + 1 < NKT) gload_b(kt + 1);
      lds_barrier();
      // the MFMA phase runs at raised wave priority, so that on a SIMD shared with a wave of
      // the other workgroup the matrix core is fed first and the staging fills the gaps
      __builtin_amdgcn_s_setprio(1);
      // only the 16-row groups of this wave that hold slot rows of the tile are multiplied
      // (a wave whose 64 rows are all past the tile's end has nothing to compute)
      auto mma = [&](auto gc) __attribute__((always_inline)) {
        constexpr int G = decltype(gc)::value;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
          bf16x8_t af[G], bfr[4];
#pragma unroll
          for (int i = 0; i < G; ++i)
            af[i] = *reinterpret_cast<const bf16x8_t*>(
                &sA[(wm * 64 + 16 * i + c16) * kLdsStride + kb * 16 + 4 * q]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            bfr[j] = *reinterpret_cast<const bf16x8_t*>(
                &sB[(wn * 64 + 16 * j + c16) * kLdsStride + kb * 16 + 4 * q]);
#pragma unroll
          for (int i = 0; i < G; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
      };
      switch (wgroups) {
        case 0: break;
        case 1: mma(std::integral_constant<int, 1>{}); break;
        case 2: mma(std::integral_constant<int, 2>{}); break;
        case 3: mma(std::integral_constant<int, 3>{}); break;
        default: mma(std::integral_constant<int, 4>{}); break;
      }
      __builtin_amdgcn_s_setprio(0);
    }

    // epilogue: lane holds column c16 of each 16x16 sub-tile, rows 4q .. 4q+3
    if (GATEUP) {
      uint16_t* hout = static_cast<uint16_t*>(out);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = wm * 64 + 16 * i + 4 * q + r;
          if (m >= rows_valid) continue;
          const int64_t orow = (int64_t)(slot0 + m0 + m) * F;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = nt * 64 + 32 * wn + 16 * j + c16;
            const float h = silu(acc[i][j][r]) * acc[i][j + 2][r];
            hout[orow + col] = (uint16_t)(pack_bf16x2(h, 0.0f) & 0xFFFFu);
          }
        }
    } else {
      float* oout = static_cast<float*>(out);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = wm * 64 + 16 * i + 4 * q + r;
          if (m >= rows_valid) continue;
          const int64_t orow = (int64_t)(slot0 + m0 + m) * H;
#pragma unroll
          for (int j = 0; j < 4; ++j) oout[orow + nt * kBN + wn * 64 + 16 * j + c16] = acc[i][j][r];
        }
    }
  }
}

hipError_t launch_gemm(const Shape& sh, int stage, const uint8_t* bank, int64_t stride,
                       const int32_t* offsets, const void* in, void* out, int T,
                       hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int grid = device_cu_count() * 2;
  if (stage == 0)
    hipLaunchKernelGGL(gemm_kernel<true>, dim3(grid), dim3(kGemmThreads), 0, s, bank, stride,
                       offsets, static_cast<const uint16_t*>(in), out, sh.H, sh.F, sh.E, sh.S);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, dim3(grid), dim3(kGemmThreads), 0, s, bank, stride,
                       offsets, static_cast<const uint16_t*>(in), out, sh.H, sh.F, sh.E, sh.S);
  return hipGetLastError();
}

}  // namespace moe
