// Batched decode layer (5 to 16 tokens) in three launches, the expert products on the bf16
// matrix cores (v_mfma_f32_16x16x32_bf16) with exact codebook values.
//
// PocketLLM "Xing4.0-29B-A4B", section "Known limitations": a decode step is bound by its launch
// count, so a layer should be a few large kernels; Red Lite "What we learned", section "1. The
// idea": the whole token is routed on the GPU, with no host round trip; section "4. Speculative
// decoding": a weight block is decoded once for all the token rows that use it.
//
//   router  (decode_router_kernel, decode.hip): the logits of the T tokens, and each token's row
//           scaled by its RMSNorm factor and split into bf16 (hi, lo) pairs in code-byte order.
//   gate/up (bdec_gateup2_kernel): one workgroup per (expert, 64 FFN rows).  It finds the
//           tokens that picked its expert by counting, for each token, the experts ranked above
//           the expert (fewer than k: picked, and that count is its place j in the token's
//           list), so no workgroup waits for another.  h leaves as bf16 (hi, lo) pairs in pair
//           order (row t * k + j; the shared expert's rows after the P routed ones).  The grid's
//           last row holds one workgroup that runs the full top-k, the gating weights, the
//           route table and the permutation.
//   down    (bdec_down3_kernel): one workgroup per (expert, 128 output rows), the K loop of the
//           gate/up kernel; o of every slot goes to the workspace, and the workgroup that
//           completes a row range (a counter per range) combines it in fixed order (routed
//           j = 0..k-1, the shared expert, the residual) into y.  Shapes whose rows do not fit
//           it take bdec_down2_kernel / bdec_down_kernel: one workgroup per 16 output rows over
//           every active expert, o in LDS.
//
// Matrix products.  An expert's tokens (at most 16: a token picks an expert once) are the 16
// rows of the A operand and 16 weight rows the columns of B.  One instruction covers one IQ4_NL
// block (K = 32) of those rows, so its fp32 result is scaled by the block's d before it is
// added up: the arithmetic of the dequant-GEMV (exact codebook values times the bf16 hi and lo
// parts of the activations, fp32 sums a block, scaled by d in fp32).  Inside a block the K
// order is the code-byte order: lane quarter g holds code bytes 4g..4g+3 of its row's block,
// each byte standing for the pair (element j, element j + 16).  B is then one lookup of a
// 256-entry table of bf16 pairs a byte, and A one 16-byte load of the pre-split pairs.
//
// Weights are read a block pair (36 bytes, dword aligned) at a time: lane quarter g loads dwords
// g, g + 1 (the even block's code bytes 4g..4g+3 straddle them) and 4 + g, 5 + g (the odd
// block's, dword 5 + g); the first quarter also holds both scales (dwords 0 and 4), which one
// lane permute hands to the other three quarters.
#include "common.h"
#include "kernels.h"
#include "route_core.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBdThreads = 256;        // gate/up workgroup
constexpr int kBdDownWaves = 8;        // down workgroup: 8 waves share the experts
constexpr int kBdMaxK = 32;
constexpr uint32_t kOob = 0x80000000u; // buffer offset past every range: the load returns 0
constexpr int kNt = 0;                  // cache policy of the weight loads: default (a 128-byte
                                        // line is read by several instructions: it must stay)
constexpr int kSc1 = 16;                // cache policy bit sc1: device-coherent loads and stores
// Copies of the pair table in the cooperative kernels' LDS: lane l looks up in copy l % kTabRep,
// stored interleaved (entry e of copy g at dword kTabRep e + g), so that the lanes of one copy
// share a few banks that no other copy uses and random code bytes collide in fewer banks.
constexpr int kTabRep = 16;

// Buffer resource over `bytes` bytes from `base`; loads past the end return zeros and touch no
// memory (the rows of A past an expert's tokens).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Four dwords of one weight row's block pair for lane quarter q: dwords q, q + 1, 4 + q, 5 + q
// of the pair; `off` is the byte offset of dword q (buffer loads).
__device__ __forceinline__ void load_bpair(__amdgpu_buffer_rsrc_t rs, uint32_t off,
                                           uint32_t (&w)[4]) {
  const u32x2_t a = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, kNt);
  const u32x2_t b = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(off + 16u), 0, kNt);
  w[0] = a[0];
  w[1] = a[1];
  w[2] = b[0];
  w[3] = b[1];
}

// B operand of four code bytes: the bf16 pairs of their codebook values.
__device__ __forceinline__ bf16x8_t b_pairs(uint32_t cw, const uint32_t* s_tab) {
  u32x4_t v;
  v[0] = s_tab[cw & 0xFFu];
  v[1] = s_tab[(cw >> 8) & 0xFFu];
  v[2] = s_tab[(cw >> 16) & 0xFFu];
  v[3] = s_tab[cw >> 24];
  return __builtin_bit_cast(bf16x8_t, v);
}

// b_pairs in the interleaved copies: tabl = the pair table's copies + this lane's copy.
template <int R>
__device__ __forceinline__ bf16x8_t b_pairs_rep(uint32_t cw, const uint32_t* tabl) {
  u32x4_t v;
  v[0] = tabl[(cw & 0xFFu) * R];
  v[1] = tabl[((cw >> 8) & 0xFFu) * R];
  v[2] = tabl[((cw >> 16) & 0xFFu) * R];
  v[3] = tabl[(cw >> 24) * R];
  return __builtin_bit_cast(bf16x8_t, v);
}

// acc += d_even * (A_even . B_even) + d_odd * (A_odd . B_odd) for one block pair of one tile of
// 16 weight rows; ah / al: the hi and lo activation fragments of the two blocks.  keep = false
// (a block pair past the end, loaded again so that no branch surrounds the loads) zeroes both
// scales: the pair then adds exactly zero.
__device__ __forceinline__ void tile_pair(const uint32_t (&w)[4], const bf16x8_t (&ah)[2],
                                          const bf16x8_t (&al)[2], const uint32_t* s_tab,
                                          int c16, bool keep, f32x4_t& acc) {
  // scales: dword 0 low half (even block) and dword 4 high half (odd block) of quarter 0
  uint32_t dd = __shfl(__builtin_amdgcn_perm(w[2], w[0], 0x07060100u), c16, 64);
  dd = keep ? dd : 0u;
  const float d0 = __half2float(__ushort_as_half((unsigned short)(dd & 0xFFFFu)));
  const float d1 = __half2float(__ushort_as_half((unsigned short)(dd >> 16)));
  const bf16x8_t b0 = b_pairs(__builtin_amdgcn_alignbit(w[1], w[0], 16), s_tab);
  const bf16x8_t b1 = b_pairs(w[3], s_tab);
  const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4_t p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[0], b0, z, 0, 0, 0);
  p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[0], b0, p0, 0, 0, 0);
  f32x4_t p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[1], b1, z, 0, 0, 0);
  p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[1], b1, p1, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = fmaf(d1, p1[r], fmaf(d0, p0[r], acc[r]));
}

// tile_pair with the block pair's 9 dwords in LDS at rw (the weights staged in LDS): dwords
// q, q + 1 (the even block's code bytes 4q..4q+3 straddle them), 5 + q (the odd block's), and
// the scales in dwords 0 (low half) and 4 (high half).  s_tab: the pair table, or with R > 1
// this lane's copy of R interleaved ones (b_pairs_rep).
template <int R = 1>
__device__ __forceinline__ void tile_pair_lds(const uint32_t* rw, int q, const bf16x8_t (&ah)[2],
                                              const bf16x8_t (&al)[2], const uint32_t* s_tab,
                                              f32x4_t& acc, bool keep = true) {
  const uint32_t w0 = rw[q], w1 = rw[q + 1], w3 = rw[5 + q];
  uint32_t dd = __builtin_amdgcn_perm(rw[4], rw[0], 0x07060100u);
  dd = keep ? dd : 0u;
  const float d0 = __half2float(__ushort_as_half((unsigned short)(dd & 0xFFFFu)));
  const float d1 = __half2float(__ushort_as_half((unsigned short)(dd >> 16)));
  const bf16x8_t b0 = b_pairs_rep<R>(__builtin_amdgcn_alignbit(w1, w0, 16), s_tab);
  const bf16x8_t b1 = b_pairs_rep<R>(w3, s_tab);
  const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4_t p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[0], b0, z, 0, 0, 0);
  p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[0], b0, p0, 0, 0, 0);
  f32x4_t p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[1], b1, z, 0, 0, 0);
  p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[1], b1, p1, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = fmaf(d1, p1[r], fmaf(d0, p0[r], acc[r]));
}

// Activation fragments of block pair bp: row offset `aoff` (bytes, or kOob: zeros), 128 bytes a
// block (16 hi pair dwords, then 16 lo).  The loads are buffer loads as well, so that the
// compiler keeps them where they are issued.
__device__ __forceinline__ void load_apair(__amdgpu_buffer_rsrc_t rs, uint32_t aoff, int bp,
                                           u32x4_t (&a)[4]) {
  const uint32_t o = aoff + (uint32_t)bp * 256u;      // kOob + 511 is still past every range
  a[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)o, 0, 0);
  a[1] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(o + 64u), 0, 0);
  a[2] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(o + 128u), 0, 0);
  a[3] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(o + 192u), 0, 0);
}

// kTabRep interleaved copies of the pair table (entry e of copy g at dword kTabRep e + g), by the
// 256 threads of a workgroup.
__device__ __forceinline__ void fill_tab_rep(uint32_t* s_tab) {
  for (int i = threadIdx.x; i < 256 * kTabRep; i += kBdThreads)
    s_tab[i] = pair_table_entry(i / kTabRep);
}

// A cooperative workgroup's stage (one step): the weights of 128 rows x S block pairs (36 S
// bytes a row), then up to 16 activation rows of 2 S blocks (128 bytes a block: 16 hi pair
// dwords, then 16 lo), each row padded by 16 bytes so that the 16 rows of a fragment read hit
// distinct banks.
template <int S>
struct Stage {
  static constexpr int SB = 128 * 36 * S;                  // weight bytes of a stage
  static constexpr int AROW = 256 * S + 16;                // bytes of an activation row
  static constexpr int STG = SB + kDecodeMaxTokens * AROW; // bytes of a stage
};

// The K loop of a cooperative workgroup (4 waves).  Loads go out two steps at a time: each
// stage row's 72 S bytes of two steps as 16-byte pieces of one contiguous run (a row's bytes
// then reach memory in runs twice as long as one step's), the activation rows' 512 S bytes
// likewise; at a double step's start the pieces are written to both LDS stages and the next
// double step's loads are issued into the same registers, so they have two steps of compute
// to arrive.  Wave w multiplies stage rows 32 w + 16 t + (0..15) (tile t = 0, 1) by the m
// activation rows into acc[t] (the matrix instruction's result layout: lane l holds column
// l % 16, rows 4 (l / 16) .. + 3).  wrow(rr): byte offset in wrs of stage row rr's first
// block; route(): the caller's routing, run once the weight pieces are set up, returning m,
// the activation rows (none: the loop returns false at once); arow(i, m): byte offset in xrs
// of activation row i, kOob past the m rows (zeros).  KS: see below.  s_stg: two stages of
// Stage<S>::STG bytes; s_tab: kTabRep interleaved copies of the pair table (fill_tab_rep).
template <int S, bool KS, typename WRow, typename Route, typename ARow>
__device__ __forceinline__ bool staged_kloop(__amdgpu_buffer_rsrc_t wrs,
                                             __amdgpu_buffer_rsrc_t xrs, WRow wrow, Route route,
                                             ARow arow, int nsteps, int wave, int lane,
                                             uint8_t* s_stg, const uint32_t* s_tab,
                                             f32x4_t (&acc)[2]) {
  using G = Stage<S>;
  constexpr int RB = 36 * S;                       // weight bytes of a stage row (a step)
  constexpr int AB = 256 * S;                      // activation bytes of a stage row
  constexpr int PPW = 2 * RB / 16;                 // 16-byte pieces of a row, two steps
  constexpr int NPW = 128 * PPW;
  constexpr int NIW = (NPW + kBdThreads - 1) / kBdThreads;
  constexpr int PPA = 2 * AB / 16;
  constexpr int NIA = kDecodeMaxTokens * PPA / kBdThreads;
  static_assert((2 * RB) % 16 == 0 && NIA * kBdThreads == kDecodeMaxTokens * PPA, "pieces");
  const int tid = threadIdx.x;
  // this thread's pieces: weight piece p = tid + 256 i is bytes 16 j .. 16 j + 15 of stage row
  // rr's two steps (two 8-byte halves, each in the stage of its step); activation piece
  // p = tid + 256 i is bytes 16 j .. of activation row p / PPA's two steps
  uint32_t woff[NIW];
  int wd0[NIW], wd1[NIW];
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int p = tid + kBdThreads * i;
    const int pp = p < NPW ? p : NPW - 1;
    const int rr = pp / PPW, j = pp - rr * PPW;
    woff[i] = wrow(rr) + 16u * j;
    const int x0 = 16 * j, x1 = 16 * j + 8;
    wd0[i] = p < NPW ? (x0 < RB ? 0 : G::STG) + rr * RB + (x0 < RB ? x0 : x0 - RB) : -1;
    wd1[i] = (x1 < RB ? 0 : G::STG) + rr * RB + (x1 < RB ? x1 : x1 - RB);
  }
  const int nds = (nsteps + 1) >> 1;               // double steps
  u32x4_t rw[NIW], ra[NIA];
  auto issue_w = [&](int d) __attribute__((always_inline)) {
    d = d < nds ? d : nds - 1;                     // past the end: the last again, unused
#pragma unroll
    for (int i = 0; i < NIW; ++i)
      rw[i] = __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)woff[i], 2 * RB * d, kNt);
  };
  // (issuing the first weights before the routing, for the experts nobody picked as well,
  // measured slower)
  const int m = route();
  if (m <= 0) return false;
  issue_w(0);
  uint32_t aoff[NIA];
  int ad[NIA];
#pragma unroll
  for (int i = 0; i < NIA; ++i) {
    const int p = tid + kBdThreads * i;
    const int it = p / PPA, j = p - it * PPA;
    aoff[i] = arow(it, m) + 16u * j;
    const int x = 16 * j;
    ad[i] = (x < AB ? 0 : G::STG) + G::SB + it * G::AROW + (x < AB ? x : x - AB);
  }
  auto issue_a = [&](int d) __attribute__((always_inline)) {
    d = d < nds ? d : nds - 1;
#pragma unroll
    for (int i = 0; i < NIA; ++i)
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)(aoff[i] + 2u * AB * d), 0, 0);
  };
  auto stage_write = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NIA; ++i) *reinterpret_cast<u32x4_t*>(s_stg + ad[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < NIW; ++i)
      if (wd0[i] >= 0) {
        *reinterpret_cast<u32x2_t*>(s_stg + wd0[i]) = u32x2_t{rw[i][0], rw[i][1]};
        *reinterpret_cast<u32x2_t*>(s_stg + wd1[i]) = u32x2_t{rw[i][2], rw[i][3]};
      }
  };

  const int c16 = lane & 15, q = lane >> 4;
  // activation fragments of rows past the m rows are never read (their products land in
  // rows of the result that are not stored): zero once, and left alone
  bf16x8_t ah[2], al[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    ah[i] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
    al[i] = ah[i];
  }
  const bool live = c16 < m;       // this lane's activation row is one of the m
  const uint32_t* tabl = s_tab + (lane % kTabRep);
  // KS: the two waves of a pair (2 h, 2 h + 1) split each step's two block pairs (wave parity
  // kh takes block pair kh) over both of their row groups (stage rows 64 h .. 64 h + 63, four
  // tiles), so each activation fragment read serves four tiles, not two; an exchange through
  // LDS after the loop leaves each wave with the sums of its own two tiles.
  static_assert(!KS || S == 2, "the K split takes one block pair a wave");
  const int kh = wave & 1, rh = wave >> 1;
  f32x4_t acc4[4] = {};
  auto compute = [&](int slot) __attribute__((always_inline)) {
    const uint8_t* sb = s_stg + slot * G::STG;
    const uint8_t* sa = sb + G::SB + c16 * G::AROW + 16 * q;
    if constexpr (KS) {
      if (live) {
        ah[0] = *reinterpret_cast<const bf16x8_t*>(sa + 256 * kh);
        ah[1] = *reinterpret_cast<const bf16x8_t*>(sa + 256 * kh + 128);
        al[0] = *reinterpret_cast<const bf16x8_t*>(sa + 256 * kh + 64);
        al[1] = *reinterpret_cast<const bf16x8_t*>(sa + 256 * kh + 192);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t* rw = reinterpret_cast<const uint32_t*>(
            sb + (64 * rh + 16 * t + c16) * 36 * S + 36 * kh);
        tile_pair_lds<kTabRep>(rw, q, ah, al, tabl, acc4[t]);
      }
      return;
    }
#pragma unroll
    for (int b = 0; b < S; ++b) {
      if (live) {
        ah[0] = *reinterpret_cast<const bf16x8_t*>(sa + 256 * b);
        ah[1] = *reinterpret_cast<const bf16x8_t*>(sa + 256 * b + 128);
        al[0] = *reinterpret_cast<const bf16x8_t*>(sa + 256 * b + 64);
        al[1] = *reinterpret_cast<const bf16x8_t*>(sa + 256 * b + 192);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t* rw =
            reinterpret_cast<const uint32_t*>(sb + (32 * wave + 16 * t + c16) * 36 * S + 36 * b);
        tile_pair_lds<kTabRep>(rw, q, ah, al, tabl, acc[t]);
      }
    }
  };

  issue_a(0);
  for (int d = 0; d < nds; ++d) {
    lds_barrier();                                 // every wave is done with both stages
    stage_write();
    __builtin_amdgcn_sched_barrier(0);
    issue_a(d + 1);
    issue_w(d + 1);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    compute(0);
    if (2 * d + 1 < nsteps) compute(1);
  }
  if constexpr (KS) {
    // wave 2 h + kh keeps tiles 2 kh, 2 kh + 1 of its pair's four: it hands the other two
    // partial sums to its partner and adds the partner's partials of its own
    __syncthreads();                               // every wave is done with the stages
    float* s_x = reinterpret_cast<float*>(s_stg);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s_x[((wave * 2 + tt) * 4 + r) * 64 + lane] = kh ? acc4[tt][r] : acc4[2 + tt][r];
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[tt][r] = (kh ? acc4[2 + tt][r] : acc4[tt][r]) +
                     s_x[(((wave ^ 1) * 2 + tt) * 4 + r) * 64 + lane];
  }
  return true;
}

// The route table of T tokens by one workgroup of 256 threads: top-k and gating weights of
// every token (route_core.h), the slot counts, offsets, and the permutation (slots of an expert
// in ascending pair order; the shared expert's slots P + t).
__device__ void publish_routes(const float* __restrict__ logits, int T, int E, int S, int k,
                               int gating, int renorm, int32_t* __restrict__ ids_out,
                               float* __restrict__ w_out, int32_t* __restrict__ offsets_out,
                               int32_t* __restrict__ sp_out, int32_t* __restrict__ ps_out,
                               int* s_ids, float* s_w, int* s_cnt, int* s_off, int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int P = T * k, NBIN = E + S;
  for (int i = tid; i < NBIN; i += kBdThreads) s_cnt[i] = 0;
  for (int t = wave; t < T; t += kBdThreads / 64)
    wave_topk_one_layout(logits + (size_t)t * E, E, k, gating, renorm, s_ids + t * k,
                         s_w + t * k);
  __syncthreads();
  for (int p = tid; p < P; p += kBdThreads) atomicAdd(&s_cnt[s_ids[p]], 1);
  if (tid < S) s_cnt[E + tid] = T;
  __syncthreads();
  // exclusive scan of the NBIN <= 1024 counts, four bins a thread
  int loc[4], run = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = tid * 4 + i;
    run += b < NBIN ? s_cnt[b] : 0;
    loc[i] = run;
  }
  int incl = run;
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int before = incl - run;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = tid * 4 + i;
    const int excl = before + (i ? loc[i - 1] : 0);
    if (b < NBIN) {
      s_off[b] = excl;
      offsets_out[b] = excl;
    }
    if (b == NBIN - 1) offsets_out[NBIN] = before + loc[i];
  }
  __syncthreads();
  for (int p = tid; p < P; p += kBdThreads) {
    const int id = s_ids[p];
    int rank = 0;
    for (int q = 0; q < p; ++q) rank += (s_ids[q] == id) ? 1 : 0;
    const int slot = s_off[id] + rank;
    sp_out[slot] = p;
    ps_out[p] = slot;
    ids_out[p] = id;
    w_out[p] = s_w[p];
  }
}

// ---- gate/up ---------------------------------------------------------------------------

// The tokens of gate/up workgroup row y (expert y < E, or the shared expert for y >= E) into
// s_tok (ascending token order) and their h rows into s_prow (pair t * k + j, or P + t), the
// count into *s_m; 256 threads.  A routed expert's rank in token t's order (the keys of
// route_core.h, ties to the lower index) is counted by 16 threads a token, each over the
// experts e2 = sub, sub + 16, ...: below k it is picked, at place j = rank.
__device__ __forceinline__ void route_expert(const float* __restrict__ logits, int T, int E,
                                             int k, int y, int* s_rank, int* s_tok, int* s_prow,
                                             int* s_m) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = T * k;
  int& s_m_ref = *s_m;
  if (y < E) {
    // rank of expert y in each token's order (keys of route_core.h, ties to the lower index):
    // 16 threads a token, each counting the experts e2 = sub, sub + 16, ... ranked above y
    const int t = tid >> 4, sub = tid & 15;
    int cnt = 0;
    if (t < T) {
      const float* lrow = logits + (size_t)t * E;
      const uint32_t ky = order_bits(lrow[y]);
      for (int e2 = sub; e2 < E; e2 += 16) {
        const uint32_t kk = order_bits(lrow[e2]);
        cnt += (kk > ky || (kk == ky && e2 < y)) ? 1 : 0;
      }
    }
    cnt = (int)group_sum_dpp<16>((float)cnt);     // small integers: exact
    if (sub == 0) s_rank[t] = (t < T && cnt < k) ? cnt : -1;
    __syncthreads();
    if (wave == 0) {
      const int rk = lane < kDecodeMaxTokens ? s_rank[lane] : -1;
      const uint64_t mask = __ballot(rk >= 0);
      if (rk >= 0) {
        const int i = __popcll(mask & ((1ull << lane) - 1));
        s_tok[i] = lane;
        s_prow[i] = lane * k + rk;
      }
      if (lane == 0) s_m_ref = __popcll(mask);
    }
  } else {                                 // the shared expert: every token, rows P + t
    if (tid < T) {
      s_tok[tid] = tid;
      s_prow[tid] = P + tid;
    }
    if (tid == 0) s_m_ref = T;
  }
  __syncthreads();
}


// TP: tiles of 16 FFN rows a wave (each a gate and an up tile); D: block pairs in flight.
template <int TP, int D>
__global__ void __launch_bounds__(kBdThreads) bdec_gateup_kernel(
    const uint8_t* __restrict__ bank, int64_t stride, const uint32_t* __restrict__ xhl,
    const float* __restrict__ logits, int T, int H, int F, int E, int S, int k, int gating,
    int renorm, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ sp_out,
    int32_t* __restrict__ ps_out, uint32_t* __restrict__ hhl, int32_t* __restrict__ done) {
  __shared__ uint32_t s_tab[256];
  __shared__ int s_rank[kDecodeMaxTokens];
  __shared__ int s_tok[kDecodeMaxTokens];
  __shared__ int s_prow[kDecodeMaxTokens];
  __shared__ int s_m;
  __shared__ int s_ids[kDecodeMaxTokens * kBdMaxK];
  __shared__ float s_w[kDecodeMaxTokens * kBdMaxK];
  __shared__ int s_cnt[kMaxE + 1];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_wave[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int y = blockIdx.y;
  if (y == E + S) {                       // the route-table workgroup (grid column 0 only)
    if (blockIdx.x == 0) {
      publish_routes(logits, T, E, S, k, gating, renorm, ids_out, w_out, offsets_out, sp_out,
                     ps_out, s_ids, s_w, s_cnt, s_off, s_wave);
      for (int i = tid; i < (H >> 7); i += kBdThreads) done[i] = 0;   // the down's counters
    }
    return;
  }
  s_tab[tid] = pair_table_entry(tid);
  route_expert(logits, T, E, k, y, s_rank, s_tok, s_prow, &s_m);
  const int m = s_m;
  if (m == 0) return;
  const int ex = y < E ? y : E;

  const int NBH = H >> 5, NBF = F >> 5;
  const int ti0 = ((int)blockIdx.x * (kBdThreads / 64) + wave) * TP;   // first tile of the wave
  if ((ti0 >> 1) >= NBF) return;
  const int c16 = lane & 15, q = lane >> 4;
  const uint32_t rowb = (uint32_t)NBH * kBlockBytes;
  // the expert's gate and up matrices (2 F rows) as one buffer
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(bank + (int64_t)ex * stride, 2u * F * rowb);
  // tile ti: FFN block ti / 2, half ti % 2; column c16 is FFN row 32 (ti / 2) + 8 (ti % 2) +
  // (c16 % 8) + 16 (c16 / 8), so that a row and the row 16 above it (one code-byte pair of h)
  // sit in lanes c16 and c16 + 8
  uint32_t rows[2 * TP];                    // byte offsets of dword q of the rows' first pair
#pragma unroll
  for (int tp = 0; tp < TP; ++tp) {
    const int ti = ti0 + tp;
    const uint32_t f = 32 * (ti >> 1) + 8 * (ti & 1) + (c16 & 7) + 16 * (c16 >> 3);
    rows[tp] = f * rowb + 4u * q;
    rows[TP + tp] = (F + f) * rowb + 4u * q;
  }
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(xhl, (uint32_t)T * (uint32_t)H * 4u);
  const uint32_t aoff = c16 < m ? (uint32_t)s_tok[c16] * (uint32_t)NBH * 128u + 16u * q : kOob;

  const int NP = NBH >> 1;                  // block pairs a row
  f32x4_t acc[2 * TP];
#pragma unroll
  for (int i = 0; i < 2 * TP; ++i) acc[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t wr[D][2 * TP][4];
  u32x4_t ar[D][4];
#pragma unroll
  for (int u = 0; u < D; ++u) {
    const int bp = u < NP ? u : NP - 1;
#pragma unroll
    for (int i = 0; i < 2 * TP; ++i) load_bpair(wrs, rows[i] + 36u * bp, wr[u][i]);
    load_apair(xrs, aoff, bp, ar[u]);
    __builtin_amdgcn_sched_barrier(0);      // the slots are issued in order
  }
  for (int b0 = 0; b0 < NP; b0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int bp = b0 + u;
      {
        const bf16x8_t ah[2] = {__builtin_bit_cast(bf16x8_t, ar[u][0]),
                                __builtin_bit_cast(bf16x8_t, ar[u][2])};
        const bf16x8_t al[2] = {__builtin_bit_cast(bf16x8_t, ar[u][1]),
                                __builtin_bit_cast(bf16x8_t, ar[u][3])};
#pragma unroll
        for (int i = 0; i < 2 * TP; ++i)
          tile_pair(wr[u][i], ah, al, s_tab, c16, bp < NP, acc[i]);
      }
      const int nb = bp + D < NP ? bp + D : NP - 1;
#pragma unroll
      for (int i = 0; i < 2 * TP; ++i) load_bpair(wrs, rows[i] + 36u * nb, wr[u][i]);
      load_apair(xrs, aoff, nb, ar[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // h = silu(g) * u; lane c16 < 8 takes the row 16 above from lane c16 + 8 and writes the
  // (hi, lo) pair dwords of both rows
#pragma unroll
  for (int tp = 0; tp < TP; ++tp) {
    const int ti = ti0 + tp;
    const int j = 8 * (ti & 1) + c16;              // pair index inside the FFN block (c16 < 8)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float hv = silu(acc[tp][r]) * acc[TP + tp][r];
      const float hu = dpp_f<0x128>(hv);           // row_ror:8: the value of lane c16 ^ 8
      const int i = 4 * q + r;
      if (c16 < 8 && i < m) {
        uint32_t hi, lo;
        split_pair(hv, hu, hi, lo);
        uint32_t* dst = hhl + ((size_t)s_prow[i] * NBF + (ti >> 1)) * 32 + j;
        dst[0] = hi;
        dst[16] = lo;
      }
    }
  }
}


// Workgroup-cooperative variant: the 4 waves take 64 FFN rows (a gate and an up tile each) and
// walk K together (staged_kloop): the weights of 128 rows and the activations are fetched as
// whole 16-byte pieces of contiguous memory by all 256 threads, two steps at a time, into LDS;
// the waves read their operands from LDS.  Every cache line of the weights is then read by
// one instruction, where the direct variant above reads 20 bytes of each of 16 rows an
// instruction.  Needs whole steps (H / 64 a multiple of S).  At most three waves a SIMD: the
// schedule the compiler makes in that register budget measured faster than with four (or
// two).
template <int S>
__global__ void __launch_bounds__(kBdThreads) __attribute__((amdgpu_waves_per_eu(1, 3)))
bdec_gateup2_kernel(
    const uint8_t* __restrict__ bank, int64_t stride, const uint32_t* __restrict__ xhl,
    const float* __restrict__ logits, int T, int H, int F, int E, int NS, int k, int gating,
    int renorm, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ sp_out,
    int32_t* __restrict__ ps_out, uint32_t* __restrict__ hhl, int32_t* __restrict__ done) {
  constexpr int STG = Stage<S>::STG;
  static_assert(2 * STG >= (int)(2 * kDecodeMaxTokens * kBdMaxK * 4 + 2 * (kMaxE + 1) * 4 + 16),
                "the route-table workgroup's arrays share the stage memory");
  // the pair table first (LDS address 0: a lookup address is the code byte times 4), then the
  // two stages
  __shared__ __align__(16) uint8_t s_mem[1024 * kTabRep + 2 * STG];
  uint32_t* s_tab = reinterpret_cast<uint32_t*>(s_mem);
  uint8_t* s_stg = s_mem + 1024 * kTabRep;
  __shared__ int s_rank[kDecodeMaxTokens];
  __shared__ int s_tok[kDecodeMaxTokens];
  __shared__ int s_prow[kDecodeMaxTokens];
  __shared__ int s_m;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int y = blockIdx.y;
  if (y == E + NS) {                      // the route-table workgroup (grid column 0 only)
    if (blockIdx.x == 0) {
      int* s_ids = reinterpret_cast<int*>(s_stg);
      float* s_w = reinterpret_cast<float*>(s_ids + kDecodeMaxTokens * kBdMaxK);
      int* s_cnt = reinterpret_cast<int*>(s_w + kDecodeMaxTokens * kBdMaxK);
      int* s_off = s_cnt + kMaxE + 1;
      int* s_wave = s_off + kMaxE + 1;
      publish_routes(logits, T, E, NS, k, gating, renorm, ids_out, w_out, offsets_out, sp_out,
                     ps_out, s_ids, s_w, s_cnt, s_off, s_wave);
      for (int i = tid; i < (H >> 7); i += kBdThreads) done[i] = 0;   // the down's counters
    }
    return;
  }
  fill_tab_rep(s_tab);
  const int ex = y < E ? y : E;
  const int NBH = H >> 5, NBF = F >> 5;
  const int nsteps = (NBH >> 1) / S;
  const uint32_t rowb = (uint32_t)NBH * kBlockBytes;
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(bank + (int64_t)ex * stride, 2u * F * rowb);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(xhl, (uint32_t)T * (uint32_t)H * 4u);

  // stage row rr = 32 w + 16 t + c is column c of wave w's gate (t = 0) or up (t = 1) tile;
  // wave w takes FFN block 2 blockIdx.x + w / 2, half w % 2, and column c is FFN row
  // 32 block + 8 half + (c % 8) + 16 (c / 8) (a row and the row 16 above it, one code-byte
  // pair of h, in lanes c and c + 8)
  auto wrow = [&](int rr) __attribute__((always_inline)) {
    const int w = rr >> 5, t = (rr >> 4) & 1, c = rr & 15;
    const uint32_t f = 32 * (2 * blockIdx.x + (w >> 1)) + 8 * (w & 1) + (c & 7) + 16 * (c >> 3);
    return (t ? F + f : f) * rowb;
  };
  auto route = [&]() __attribute__((always_inline)) {
    route_expert(logits, T, E, k, y, s_rank, s_tok, s_prow, &s_m);
    return s_m;
  };
  auto arow = [&](int it, int m) __attribute__((always_inline)) {
    return it < m ? (uint32_t)s_tok[it] * (uint32_t)NBH * 128u : kOob;
  };
  f32x4_t acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
  if (!staged_kloop<S, true>(wrs, xrs, wrow, route, arow, nsteps, wave, lane, s_stg, s_tab, acc))
    return;                                        // no token picked the expert
  const int m = s_m;
  const int c16 = lane & 15, q = lane >> 4;

  // h = silu(g) * u; lane c16 < 8 takes the row 16 above from lane c16 + 8 and writes the
  // (hi, lo) pair dwords of both rows
  const int kbf = 2 * blockIdx.x + (wave >> 1);
  const int j = 8 * (wave & 1) + c16;              // pair index inside the FFN block (c16 < 8)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float hv = silu(acc[0][r]) * acc[1][r];
    const float hu = dpp_f<0x128>(hv);             // row_ror:8: the value of lane c16 ^ 8
    const int i = 4 * q + r;
    if (c16 < 8 && i < m) {
      uint32_t hi, lo;
      split_pair(hv, hu, hi, lo);
      uint32_t* dst = hhl + ((size_t)s_prow[i] * NBF + kbf) * 32 + j;
      dst[0] = hi;
      dst[16] = lo;
    }
  }
}

// ---- down + combine --------------------------------------------------------------------

template <int D>
__global__ void __launch_bounds__(kBdDownWaves * 64) bdec_down_kernel(
    const uint8_t* __restrict__ bank, int64_t stride, const uint32_t* __restrict__ hhl,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
    const float* __restrict__ w, int T, int H, int F, int E, int S, int k,
    const float* residual, float* y) {
  constexpr int NW = kBdDownWaves;
  __shared__ uint32_t s_tab[256];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_sp[kDecodeMaxTokens * kBdMaxK];
  __shared__ float s_w[kDecodeMaxTokens * kBdMaxK];
  __shared__ int s_act[kMaxE];
  __shared__ int s_nact;
  __shared__ float s_o[kDecodeMaxTokens * (kBdMaxK + 1) * 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int P = T * k, NBIN = E + S;
  const int NBF = F >> 5;
  const int r0 = (int)blockIdx.x * 16;
  if (tid < 256) s_tab[tid] = pair_table_entry(tid);
  for (int i = tid; i <= NBIN; i += NW * 64) s_off[i] = offsets[i];
  for (int i = tid; i < P; i += NW * 64) {
    s_sp[i] = sorted_pairs[i];
    s_w[i] = w[i];
  }
  __syncthreads();
  // experts with slots: the shared expert first, then the routed ones in index order
  if (wave == 0) {
    int seen = 0;
    if (S > 0) {
      if (lane == 0) s_act[0] = E;
      seen = 1;
    }
    for (int base = 0; base < E; base += 64) {
      const int b = base + lane;
      const bool ne = b < E && s_off[b + 1] > s_off[b];
      const uint64_t mask = __ballot(ne);
      if (ne) s_act[seen + __popcll(mask & ((1ull << lane) - 1))] = b;
      seen += __popcll(mask);
    }
    if (lane == 0) s_nact = seen;
  }
  __syncthreads();
  const int nact = s_nact;
  const int n_my = wave < nact ? (nact - wave + NW - 1) / NW : 0;   // experts wave, wave + NW, ..
  const int c16 = lane & 15, q = lane >> 4;
  const int NP = NBF >> 1;
  const int total = n_my * NP;

  if (total > 0) {
    const int64_t rowb = (int64_t)NBF * kBlockBytes;
    const int64_t down_off = 2 * (int64_t)F * ((int64_t)(H >> 5) * kBlockBytes);
    const __amdgpu_buffer_rsrc_t hrs =
        make_rsrc(hhl, (uint32_t)(P + T * S) * (uint32_t)F * 4u);
    // the slot row of lane c16 in expert ex (or none)
    auto prow_of = [&](int ex, int i) __attribute__((always_inline)) {
      const int sa = s_off[ex], m = s_off[ex + 1] - sa;
      return i < m ? (sa + i < P ? s_sp[sa + i] : sa + i) : -1;
    };
    // issue state: the next block pair to load
    int i_ei = 0, i_bp = 0;
    __amdgpu_buffer_rsrc_t i_rs;
    uint32_t i_aoff = kOob;
    const uint32_t i_row = (uint32_t)(r0 + c16) * (uint32_t)rowb + 4u * q;
    auto set_issue = [&](int ei) __attribute__((always_inline)) {
      const int ex = __builtin_amdgcn_readfirstlane(s_act[wave + NW * ei]);
      i_rs = make_rsrc(bank + (int64_t)ex * stride + down_off, (uint32_t)(H * rowb));
      const int pr = prow_of(ex, c16);
      i_aoff = pr >= 0 ? (uint32_t)pr * (uint32_t)NBF * 128u + 16u * q : kOob;
    };
    set_issue(0);
    uint32_t wr[D][4];
    u32x4_t ar[D][4];
    auto issue = [&](int u) __attribute__((always_inline)) {
      load_bpair(i_rs, i_row + 36u * i_bp, wr[u]);
      load_apair(hrs, i_aoff, i_bp, ar[u]);
      if (i_bp + 1 < NP) {
        ++i_bp;
      } else if (i_ei + 1 < n_my) {
        ++i_ei;
        i_bp = 0;
        set_issue(i_ei);
      }                                          // past the last item: it is loaded again
    };
#pragma unroll
    for (int u = 0; u < D; ++u) {
      issue(u);
      __builtin_amdgcn_sched_barrier(0);    // the slots are issued in order
    }
    int c_ei = 0, c_bp = 0;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int i0 = 0; i0 < total; i0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const bool valid = i0 + u < total;
        {
          const bf16x8_t ah[2] = {__builtin_bit_cast(bf16x8_t, ar[u][0]),
                                  __builtin_bit_cast(bf16x8_t, ar[u][2])};
          const bf16x8_t al[2] = {__builtin_bit_cast(bf16x8_t, ar[u][1]),
                                  __builtin_bit_cast(bf16x8_t, ar[u][3])};
          tile_pair(wr[u], ah, al, s_tab, c16, valid, acc);
        }
        if (valid && ++c_bp == NP) {
            const int ex = s_act[wave + NW * c_ei];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int pr = prow_of(ex, 4 * q + r);
              if (pr >= 0) s_o[pr * 16 + c16] = acc[r];
            }
            acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            c_bp = 0;
            ++c_ei;
        }
        issue(u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __syncthreads();

  // combine in fixed order: routed j = 0..k-1, then the shared expert, then the residual
  if (tid < T * 16) {
    const int t = tid >> 4, c = tid & 15;
    float a = 0.0f;
    for (int j = 0; j < k; ++j) a = fmaf(s_w[t * k + j], s_o[(t * k + j) * 16 + c], a);
    for (int sidx = 0; sidx < S; ++sidx) a += s_o[(P + sidx * T + t) * 16 + c];
    const int64_t o = (int64_t)t * H + r0 + c;
    if (residual) a += residual[o];
    y[o] = a;
  }
}

// Staged variant of the down kernel: a wave's 16 rows of its expert are fetched SD block pairs
// at a time as 8-byte pieces of contiguous row segments (36 SD bytes a row; a load instruction
// covers several whole segments instead of 20 bytes of each of 16 rows), two steps ahead into
// registers, and written to the wave's own LDS stage right before its operands are read
// (one wave writes and reads it: its LDS accesses complete in order, no barrier).  The
// activations (h rows) are loaded as in the direct variant.  Rows of an even number of block
// pairs (F a multiple of 128).
template <int SD>
__global__ void __launch_bounds__(kBdDownWaves * 64) bdec_down2_kernel(
    const uint8_t* __restrict__ bank, int64_t stride, const uint32_t* __restrict__ hhl,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
    const float* __restrict__ w, int T, int H, int F, int E, int S, int k,
    const float* residual, float* y) {
  constexpr int NW = kBdDownWaves;
  constexpr int PPR = 36 * SD / 8;                 // 8-byte pieces of a row a step
  constexpr int NPD = 16 * PPR;                    // pieces a step (16 rows)
  constexpr int NID = (NPD + 63) / 64;             // load instructions a step
  __shared__ uint32_t s_tab[256];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_sp[kDecodeMaxTokens * kBdMaxK];
  __shared__ float s_w[kDecodeMaxTokens * kBdMaxK];
  __shared__ int s_act[kMaxE];
  __shared__ int s_nact;
  __shared__ float s_o[kDecodeMaxTokens * (kBdMaxK + 1) * 16];
  __shared__ __align__(16) uint8_t s_wst[NW][NPD * 8];   // each wave's weight stage

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int P = T * k, NBIN = E + S;
  const int NBF = F >> 5;
  const int r0 = (int)blockIdx.x * 16;
  if (tid < 256) s_tab[tid] = pair_table_entry(tid);
  for (int i = tid; i <= NBIN; i += NW * 64) s_off[i] = offsets[i];
  for (int i = tid; i < P; i += NW * 64) {
    s_sp[i] = sorted_pairs[i];
    s_w[i] = w[i];
  }
  __syncthreads();
  // experts with slots: the shared expert first, then the routed ones in index order
  if (wave == 0) {
    int seen = 0;
    if (S > 0) {
      if (lane == 0) s_act[0] = E;
      seen = 1;
    }
    for (int base = 0; base < E; base += 64) {
      const int b = base + lane;
      const bool ne = b < E && s_off[b + 1] > s_off[b];
      const uint64_t mask = __ballot(ne);
      if (ne) s_act[seen + __popcll(mask & ((1ull << lane) - 1))] = b;
      seen += __popcll(mask);
    }
    if (lane == 0) s_nact = seen;
  }
  __syncthreads();
  const int nact = s_nact;
  const int n_my = wave < nact ? (nact - wave + NW - 1) / NW : 0;   // experts wave, wave + NW, ..
  const int c16 = lane & 15, q = lane >> 4;
  const int nst = (NBF >> 1) / SD;                 // steps an expert
  const int total = n_my * nst;

  if (total > 0) {
    const uint32_t rowb = (uint32_t)NBF * kBlockBytes;
    const int64_t down_off = 2 * (int64_t)F * ((int64_t)(H >> 5) * kBlockBytes);
    const __amdgpu_buffer_rsrc_t hrs =
        make_rsrc(hhl, (uint32_t)(P + T * S) * (uint32_t)F * 4u);
    auto prow_of = [&](int ex, int i) __attribute__((always_inline)) {
      const int sa = s_off[ex], m = s_off[ex + 1] - sa;
      return i < m ? (sa + i < P ? s_sp[sa + i] : sa + i) : -1;
    };
    // this lane's pieces: piece p = lane + 64 i is 8-byte piece j of row r = p / PPR
    uint32_t poff[NID];
    int pdst[NID];
#pragma unroll
    for (int i = 0; i < NID; ++i) {
      const int p = lane + 64 * i;
      const int pp = p < NPD ? p : NPD - 1;
      const int r = pp / PPR, j = pp - r * PPR;
      poff[i] = (uint32_t)(r0 + r) * rowb + 8u * j;
      pdst[i] = p < NPD ? 8 * p : -1;
    }
    uint8_t* stg = s_wst[wave];
    // issue state: the next step to load
    int i_ei = 0, i_st = 0;
    __amdgpu_buffer_rsrc_t i_rs;
    uint32_t i_aoff = kOob;
    auto set_issue = [&](int ei) __attribute__((always_inline)) {
      const int ex = __builtin_amdgcn_readfirstlane(s_act[wave + NW * ei]);
      i_rs = make_rsrc(bank + (int64_t)ex * stride + down_off, (uint32_t)H * rowb);
      const int pr = prow_of(ex, c16);
      i_aoff = pr >= 0 ? (uint32_t)pr * (uint32_t)NBF * 128u + 16u * q : kOob;
    };
    set_issue(0);
    u32x2_t wb[2][NID];
    u32x4_t ar[2][SD][4];
    auto issue = [&](int u) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NID; ++i)
        wb[u][i] = __builtin_amdgcn_raw_buffer_load_b64(i_rs, (int)poff[i], 36 * SD * i_st, 0);
#pragma unroll
      for (int b = 0; b < SD; ++b) load_apair(hrs, i_aoff, SD * i_st + b, ar[u][b]);
      if (i_st + 1 < nst) {
        ++i_st;
      } else if (i_ei + 1 < n_my) {
        ++i_ei;
        i_st = 0;
        set_issue(i_ei);
      }                                          // past the last item: it is loaded again
    };
    issue(0);
    __builtin_amdgcn_sched_barrier(0);
    issue(1);
    __builtin_amdgcn_sched_barrier(0);
    int c_ei = 0, c_st = 0;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int i0 = 0; i0 < total; i0 += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bool valid = i0 + u < total;
#pragma unroll
        for (int i = 0; i < NID; ++i)
          if (pdst[i] >= 0) *reinterpret_cast<u32x2_t*>(stg + pdst[i]) = wb[u][i];
#pragma unroll
        for (int b = 0; b < SD; ++b) {
          const bf16x8_t ah[2] = {__builtin_bit_cast(bf16x8_t, ar[u][b][0]),
                                  __builtin_bit_cast(bf16x8_t, ar[u][b][2])};
          const bf16x8_t al[2] = {__builtin_bit_cast(bf16x8_t, ar[u][b][1]),
                                  __builtin_bit_cast(bf16x8_t, ar[u][b][3])};
          const uint32_t* rw = reinterpret_cast<const uint32_t*>(stg + c16 * 36 * SD + 36 * b);
          tile_pair_lds(rw, q, ah, al, s_tab, acc, valid);
        }
        if (valid && ++c_st == nst) {
          const int ex = s_act[wave + NW * c_ei];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int pr = prow_of(ex, 4 * q + r);
            if (pr >= 0) s_o[pr * 16 + c16] = acc[r];
          }
          acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          c_st = 0;
          ++c_ei;
        }
        issue(u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __syncthreads();

  // combine in fixed order: routed j = 0..k-1, then the shared expert, then the residual
  if (tid < T * 16) {
    const int t = tid >> 4, c = tid & 15;
    float a = 0.0f;
    for (int j = 0; j < k; ++j) a = fmaf(s_w[t * k + j], s_o[(t * k + j) * 16 + c], a);
    for (int sidx = 0; sidx < S; ++sidx) a += s_o[(P + sidx * T + t) * 16 + c];
    const int64_t o = (int64_t)t * H + r0 + c;
    if (residual) a += residual[o];
    y[o] = a;
  }
}

// Down by cooperative tiles: one workgroup per (expert, 128 output rows), the K loop of the
// gate/up kernel over the expert's h rows (A) and its down rows (B).  Each slot's 128 outputs
// go to o; then the workgroup adds its slot count to the row range's counter in `done`, and
// the one that brings it to P + T S (every slot of every expert done) combines the range in
// fixed order (routed j = 0..k-1, the shared expert, the residual) and clears the counter.
// Every expert's h is then read once a row range, where the per-16-row kernel above reads it
// once every 16 rows.  Needs H a multiple of 128 and whole steps (F / 64 a multiple of S).
template <int S>
__global__ void __launch_bounds__(kBdThreads) bdec_down3_kernel(
    const uint8_t* __restrict__ bank, int64_t stride, const uint32_t* __restrict__ hhl,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
    const float* __restrict__ w, int T, int H, int F, int E, int NS, int k, float* o,
    int32_t* __restrict__ done, const float* residual, float* y) {
  using G = Stage<S>;
  __shared__ __align__(16) uint8_t s_mem[1024 * kTabRep + 2 * G::STG];
  uint32_t* s_tab = reinterpret_cast<uint32_t*>(s_mem);
  uint8_t* s_stg = s_mem + 1024 * kTabRep;
  __shared__ int s_prow[kDecodeMaxTokens];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ex = blockIdx.y;                       // E: the shared expert
  const int sa = offsets[ex], m = offsets[ex + 1] - sa;
  if (m <= 0) return;
  const int P = T * k, nslots = P + T * NS;
  fill_tab_rep(s_tab);
  if (tid < m) s_prow[tid] = sa + tid < P ? sorted_pairs[sa + tid] : sa + tid;
  __syncthreads();
  const int NBF = F >> 5;
  const int nsteps = (NBF >> 1) / S;
  const uint32_t rowb = (uint32_t)NBF * kBlockBytes;
  const int r0 = (int)blockIdx.x * 128;
  const int64_t down_off = 2 * (int64_t)F * ((int64_t)(H >> 5) * kBlockBytes);
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(bank + (int64_t)ex * stride + down_off + (int64_t)r0 * rowb, 128u * rowb);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(hhl, (uint32_t)nslots * (uint32_t)F * 4u);

  auto wrow = [&](int rr) __attribute__((always_inline)) { return (uint32_t)rr * rowb; };
  auto route = [&]() __attribute__((always_inline)) { return m; };
  auto arow = [&](int it, int mm) __attribute__((always_inline)) {
    return it < mm ? (uint32_t)s_prow[it] * (uint32_t)NBF * 128u : kOob;
  };
  f32x4_t acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
  staged_kloop<S, false>(wrs, xrs, wrow, route, arow, nsteps, wave, lane, s_stg, s_tab, acc);
  // o is stored at the device-coherent level (sc1: as the compiler's device-scope atomic
  // stores), so no workgroup has to write back its L2 (a device-scope release fence writes back
  // the XCD's whole L2: one a workgroup made this kernel four times slower).  Each thread waits
  // until its o stores are complete before the workgroup counts its slots done; the workgroup
  // that finds every slot done invalidates its stale cached lines (an acquire fence) and only
  // then reads o.
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(o, (uint32_t)nslots * (uint32_t)H * 4u);
  const int c16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * q + r;
      if (i < m)
        __builtin_amdgcn_raw_buffer_store_b32(
            __float_as_uint(acc[t][r]), ors,
            (int)(((uint32_t)s_prow[i] * H + r0 + 32 * wave + 16 * t + c16) * 4u), 0, kSc1);
    }
  __builtin_amdgcn_s_waitcnt(0);                   // this thread's o stores are complete
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&done[blockIdx.x], m, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) + m == nslots;
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // drop stale cached lines of o
  // thread (c, u0) = (tid % 128, tid / 128) combines column r0 + c of tokens u0, u0 + 2, ..;
  // the loads of four routed terms of every token go out together (one round trip at k = 4)
  constexpr int NU = kDecodeMaxTokens / 2;
  const int r = r0 + (tid & 127), u0 = tid >> 7;
  const __amdgpu_buffer_rsrc_t wrr = make_rsrc(w, (uint32_t)P * 4u);
  float a[NU], sh[NU], rs[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int t = u0 + 2 * u;
    const bool ok = t < T;
    a[u] = 0.0f;
    sh[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                ors, ok && NS > 0 ? (int)(((uint32_t)(P + t) * H + r) * 4u) : (int)kOob, 0, kSc1));
    rs[u] = ok && residual ? residual[(int64_t)t * H + r] : 0.0f;
  }
  for (int j0 = 0; j0 < k; j0 += 4) {
    float v[4][NU], wv[4][NU];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int t = u0 + 2 * u, j = j0 + jj;
        const bool ok = t < T && j < k;          // else an offset past the end: zero
        v[jj][u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                       ors, ok ? (int)(((uint32_t)(t * k + j) * H + r) * 4u) : (int)kOob, 0,
                       kSc1));
        wv[jj][u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                        wrr, ok ? (t * k + j) * 4 : (int)kOob, 0, 0));
      }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int u = 0; u < NU; ++u)
        if (j0 + jj < k) a[u] = fmaf(wv[jj][u], v[jj][u], a[u]);
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int t = u0 + 2 * u;
    if (t < T) {
      float b = a[u];
      if (NS > 0) b += sh[u];
      if (residual) b += rs[u];
      y[(int64_t)t * H + r] = b;
    }
  }
  if (tid == 0) __hip_atomic_store(&done[blockIdx.x], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- host side -------------------------------------------------------------------------

bool bdecode_supported(const Shape& sh, int T) {
  return T >= 1 && T <= kDecodeMaxTokens && sh.k <= kBdMaxK && sh.E + sh.S <= kMaxE &&
         sh.S <= 1 && sh.H % 64 == 0 && sh.F % 64 == 0;
}

hipError_t launch_bdecode_layer(const Shape& sh, const uint8_t* bank, int64_t stride,
                                const float* wr, const float* bias, const float* x, int T,
                                float eps, const float* residual, float* y, DecodeScratch sc,
                                int stages, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!bdecode_supported(sh, T)) return hipErrorInvalidValue;
  uint32_t* xhl = reinterpret_cast<uint32_t*>(sc.xn);
  uint32_t* hhl = reinterpret_cast<uint32_t*>(sc.h);
  hipError_t err;
  if (stages & 1) {
    err = launch_router_rows(sh, x, wr, bias, T, eps, sc.logits, nullptr, s, nullptr, xhl);
    if (err != hipSuccess) return err;
  }
  if (stages & 2) {
    // two tiles a wave (128 FFN rows a workgroup) when that still gives every CU a few
    // workgroups a routed expert's worth of rows
    if ((sh.H / 64) % 2 == 0) {
      const dim3 grid(sh.F / 64, sh.E + sh.S + 1);
      hipLaunchKernelGGL((bdec_gateup2_kernel<2>), grid, dim3(kBdThreads), 0, s, bank, stride,
                         xhl, sc.logits, T, sh.H, sh.F, sh.E, sh.S, sh.k, sh.gating, sh.renorm,
                         sc.ids, sc.w, sc.offsets, sc.sorted_pairs, sc.pair_slot, hhl,
                         sc.done);
    } else {
      const int wg_rows = 64 * 1;
      const dim3 grid((sh.F + wg_rows - 1) / wg_rows, sh.E + sh.S + 1);
      hipLaunchKernelGGL((bdec_gateup_kernel<1, 4>), grid, dim3(kBdThreads), 0, s, bank, stride,
                         xhl, sc.logits, T, sh.H, sh.F, sh.E, sh.S, sh.k, sh.gating, sh.renorm,
                         sc.ids, sc.w, sc.offsets, sc.sorted_pairs, sc.pair_slot, hhl,
                         sc.done);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (stages & 4) {
    if (sh.H % 128 == 0 && (sh.F / 64) % 2 == 0)
      hipLaunchKernelGGL((bdec_down3_kernel<2>), dim3(sh.H / 128, sh.E + sh.S),
                         dim3(kBdThreads), 0, s, bank, stride, hhl, sc.offsets, sc.sorted_pairs,
                         sc.w, T, sh.H, sh.F, sh.E, sh.S, sh.k, sc.o, sc.done, residual, y);
    else if ((sh.F / 64) % 2 == 0)
      hipLaunchKernelGGL((bdec_down2_kernel<2>), dim3(sh.H / 16), dim3(kBdDownWaves * 64), 0, s,
                         bank, stride, hhl, sc.offsets, sc.sorted_pairs, sc.w, T, sh.H, sh.F,
                         sh.E, sh.S, sh.k, residual, y);
    else
      hipLaunchKernelGGL((bdec_down_kernel<4>), dim3(sh.H / 16), dim3(kBdDownWaves * 64), 0, s,
                         bank, stride, hhl, sc.offsets, sc.sorted_pairs, sc.w, T, sh.H, sh.F,
                         sh.E, sh.S, sh.k, residual, y);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
