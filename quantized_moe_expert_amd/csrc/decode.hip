// Fused decode layer: y = MoE(xn) + residual with xn = x / rms(x) (or xn = x), for small
// batches (T <= 16), in three kernels a layer.
//
// PocketLLM "Xing4.0-29B-A4B", section "Known limitations": a decode step made of thousands of
// small launches is bound by host submission, and fewer, larger kernels plus graphs are the
// lever; Red Lite "What we learned", section "1. The idea": a whole token routed on the GPU,
// with no CPU round trip between layers.  Here every step of the layer stays on the device:
//
//   router  : one workgroup per EPW experts; logits of all T tokens from one pass over W_r,
//             together with sum(x^2) per token (the RMSNorm scale is applied to the dot
//             product: (W_r x) / rms(x) = W_r (x / rms(x))).
//   gate/up : every workgroup redoes the routing of the T tokens it needs (no
//             cross-workgroup state), picks its expert (the blockIdx.y-th active one),
//             streams its rows and writes h in slot order; one extra workgroup, the last row
//             of the grid, only routes and writes the route table and the permutation, so
//             that this work is not added to any workgroup's weight stream.
//   down    : one workgroup per tile of output rows loops over every active expert, keeps
//             o for its rows in LDS and applies the combine (fixed order: routed j = 0..k-1,
//             then shared, then residual) before writing y -- no o buffer, no combine launch.
#include "common.h"
#include "gemv_core.h"
#include "kernels.h"
#include "route_core.h"

namespace moe {

constexpr int kDecThreads = 256;
constexpr int kDecMaxT = 16;
constexpr int kDecMaxK = 32;
constexpr int kDownRing = 16;       // passes in flight in the down kernel
constexpr int kDownStageUnits = 12; // staging units a thread: rows * F/32 * 4 <= 3072

// ---- router --------------------------------------------------------------------------

// KM: float4 a thread of one W_r row (ceil(H / 1024)).  Tokens are processed in groups of TG
// whose activation loads are issued together.
template <int EPW, int KM, int TG>
__global__ void __launch_bounds__(kDecThreads) decode_router_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    int T, int H, int E, float eps, int use_norm, float* __restrict__ logits,
    float* __restrict__ rscale, float* __restrict__ xn, uint32_t* __restrict__ xhl) {
  __shared__ float s_red[4][(EPW + 1) * kDecMaxT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e0 = blockIdx.x * EPW;
  // grid row y takes tokens [y * tpg, y * tpg + tpg): fewer activation rows a workgroup reads
  {
    const int tpg = (T + (int)gridDim.y - 1) / (int)gridDim.y;
    const int t0 = (int)blockIdx.y * tpg;
    T = min(tpg, T - t0);
    x += (size_t)t0 * H;
    logits += (size_t)t0 * E;
    if (rscale) rscale += t0;
    if (xn) xn += (size_t)t0 * H;
    if (xhl) xhl += (size_t)t0 * H;
  }
  float acc[EPW][kDecMaxT], ss[kDecMaxT];
#pragma unroll
  for (int t = 0; t < kDecMaxT; ++t) {
    ss[t] = 0.0f;
#pragma unroll
    for (int q = 0; q < EPW; ++q) acc[q][t] = 0.0f;
  }
  // every W_r load of this thread first, then the activations TG tokens at a time
  const int H4 = H >> 2;
  float4 w[EPW][KM];
#pragma unroll
  for (int i = 0; i < KM; ++i) {
    const int h4 = tid + kDecThreads * i;
#pragma unroll
    for (int q = 0; q < EPW; ++q)
      w[q][i] = (h4 < H4 && e0 + q < E)
                    ? reinterpret_cast<const float4*>(wr + (size_t)(e0 + q) * H)[h4]
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int t0 = 0; t0 < kDecMaxT; t0 += TG) {
    if (t0 < T) {
      float4 v[TG][KM];
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        const int t = min(t0 + g, T - 1);          // past T: a valid row, zeroed below
#pragma unroll
        for (int i = 0; i < KM; ++i) {
          const int h4 = tid + kDecThreads * i;
          v[g][i] = reinterpret_cast<const float4*>(x + (size_t)t * H)[h4 < H4 ? h4 : 0];
          if (h4 >= H4 || t0 + g >= T) v[g][i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        const int t = t0 + g;
#pragma unroll
        for (int i = 0; i < KM; ++i) {
          float a = ss[t];
          a = fmaf(v[g][i].x, v[g][i].x, a); a = fmaf(v[g][i].y, v[g][i].y, a);
          a = fmaf(v[g][i].z, v[g][i].z, a); a = fmaf(v[g][i].w, v[g][i].w, a);
          ss[t] = a;
#pragma unroll
          for (int q = 0; q < EPW; ++q) {
            float c = acc[q][t];
            c = fmaf(w[q][i].x, v[g][i].x, c); c = fmaf(w[q][i].y, v[g][i].y, c);
            c = fmaf(w[q][i].z, v[g][i].z, c); c = fmaf(w[q][i].w, v[g][i].w, c);
            acc[q][t] = c;
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kDecMaxT; ++t) {
    if (t < T) {
      const float s0 = group_sum_dpp<64>(ss[t]);
      if (lane == 0) s_red[wave][EPW * kDecMaxT + t] = s0;
#pragma unroll
      for (int q = 0; q < EPW; ++q) {
        const float s1 = group_sum_dpp<64>(acc[q][t]);
        if (lane == 0) s_red[wave][q * kDecMaxT + t] = s1;
      }
    }
  }
  __syncthreads();
  if (tid < EPW * kDecMaxT) {
    const int q = tid / kDecMaxT, t = tid % kDecMaxT;
    const int e = e0 + q;
    if (t < T && e < E) {
      const float dot = (s_red[0][tid] + s_red[1][tid]) + (s_red[2][tid] + s_red[3][tid]);
      float r = 1.0f;
      if (use_norm) {
        const int i = EPW * kDecMaxT + t;
        const float sq = (s_red[0][i] + s_red[1][i]) + (s_red[2][i] + s_red[3][i]);
        r = 1.0f / sqrtf(sq / (float)H + eps);
      }
      logits[(size_t)t * E + e] = r * dot + (bias ? bias[e] : 0.0f);
      if (use_norm && rscale && blockIdx.x == 0 && q == 0) rscale[t] = r;
    }
  }
  // optional rows of x * r split into bf16 (hi, lo) pairs in code-byte order: per block of 32,
  // dword j < 16 = (hi(x_j), hi(x_{j+16})), dword 16 + j the lo parts; workgroup b writes
  // token rows b, b + grid, ...
  if (xhl) {
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
      float r = 1.0f;
      if (use_norm) {
        const int i = EPW * kDecMaxT + t;
        const float sq = (s_red[0][i] + s_red[1][i]) + (s_red[2][i] + s_red[3][i]);
        r = 1.0f / sqrtf(sq / (float)H + eps);
      }
      const float* src = x + (size_t)t * H;
      uint32_t* dst = xhl + (size_t)t * H;
      for (int pi = tid; pi < (H >> 1); pi += kDecThreads) {
        const int kb = pi >> 4, j = pi & 15;
        uint32_t hi, lo;
        split_pair(src[kb * 32 + j] * r, src[kb * 32 + 16 + j] * r, hi, lo);
        dst[kb * 32 + j] = hi;
        dst[kb * 32 + 16 + j] = lo;
      }
    }
  }
  // optional normalised rows: workgroup b writes token rows b, b + grid, ... (same r)
  if (xn && use_norm) {
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
      const int i = EPW * kDecMaxT + t;
      const float sq = (s_red[0][i] + s_red[1][i]) + (s_red[2][i] + s_red[3][i]);
      const float r = 1.0f / sqrtf(sq / (float)H + eps);
      const float4* src = reinterpret_cast<const float4*>(x + (size_t)t * H);
      float4* dst = reinterpret_cast<float4*>(xn + (size_t)t * H);
      for (int h4 = tid; h4 < H4; h4 += kDecThreads) {
        const float4 v = src[h4];
        dst[h4] = make_float4(v.x * r, v.y * r, v.z * r, v.w * r);
      }
    }
  }
}

// ---- gate/up with in-workgroup routing -------------------------------------------------

// PASSES: weight rows a lane group visits (even: gate rows, then the matching up rows).
template <int LPR, int BPL, int MT, int kUpPasses>
__global__ void __launch_bounds__(kDecThreads) decode_gateup_kernel(
    const uint8_t* __restrict__ bank, int64_t stride, const float* __restrict__ x,
    const float* __restrict__ rscale, const float* __restrict__ logits, int T, int H, int F,
    int E, int S, int k, int gating, int renorm, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out, int32_t* __restrict__ offsets_out,
    int32_t* __restrict__ sp_out, int32_t* __restrict__ ps_out, float* __restrict__ h_out,
    int tch) {
  constexpr int RPP = 64 / LPR;
  constexpr int WROWS = kUpPasses * RPP;
  constexpr int OROWS = WROWS / 2;
  extern __shared__ __align__(16) uint32_t s_x[];
  __shared__ uint32_t s_tab[256];
  __shared__ int s_ids[kDecMaxT * kDecMaxK];
  __shared__ float s_w[kDecMaxT * kDecMaxK];
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1025];
  __shared__ int s_tok[kDecMaxT];
  __shared__ int s_e, s_slot0, s_m;
  __shared__ int s_wave[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = T * k, NBIN = E + S;
  const int nch = (T + tch - 1) / tch;             // token chunks an expert is split into
  s_tab[tid] = pair_table_entry(tid);
  // the first nch rows of the grid take the shared expert: slots P.., tokens 0..T-1 in
  // order, known without the routing, so their weight stream starts at once (and they are
  // dispatched first); the routed experts take the rows from y0 on
  const int y0 = S > 0 ? nch : 0;
  const bool shared_wg = (int)blockIdx.y < y0;
  const bool publisher = (int)blockIdx.y == (int)gridDim.y - 1;
  if (publisher && blockIdx.x != 0) return;
  const bool fast1 = T == 1 && !publisher;
  if (shared_wg) {
    if (tid == 0) {
      s_e = E;
      s_slot0 = P;
      s_m = T;
    }
    __syncthreads();
  } else if (fast1) {
    // one token: a routed workgroup needs only which expert is the target-th member of the
    // top-k set in index order (its slot is that rank); order and weights are the route-table
    // workgroup's business (it runs the full top-k)
    if (wave == 0) {
      const int target = (int)blockIdx.y - y0;
      const int e1 = wave_topk_member_any(logits, E, k, target);
      if (lane == 0) {
        s_e = e1;
        s_slot0 = target;
        s_m = e1 >= 0 ? 1 : 0;
      }
    }
    __syncthreads();
  } else {
    for (int i = tid; i < NBIN; i += kDecThreads) s_cnt[i] = 0;
    for (int t = wave; t < T; t += 4)
      wave_topk(logits + (size_t)t * E, E, k, gating, renorm, s_ids + t * k, s_w + t * k);
    __syncthreads();
    for (int p = tid; p < P; p += kDecThreads) atomicAdd(&s_cnt[s_ids[p]], 1);   // counts only
    if (tid < S) s_cnt[E + tid] = T;
    __syncthreads();

    // the blockIdx.y-th routed expert with routes, and the number of slots before it
    if (wave == 0) {
      const int target = ((int)blockIdx.y - y0) / nch;
      int seen = 0, run = 0, found = -1, slot0 = 0;
      for (int base = 0; base < E && found < 0; base += 64) {
        const int b = base + lane;
        const int c = b < E ? s_cnt[b] : 0;
        const uint64_t mask = __ballot(c > 0);
        const int cnt = __popcll(mask);
        if (target < seen + cnt) {
          uint64_t mm = mask;
          for (int i = 0; i < target - seen; ++i) mm &= mm - 1;
          const int pos = __ffsll((long long)mm) - 1;
          // slot counts are small integers: exact as float sums
          slot0 = run + (int)group_sum_dpp<64>((float)(lane < pos ? c : 0));
          found = base + pos;
        } else {
          seen += cnt;
          run += (int)group_sum_dpp<64>((float)c);
        }
      }
      if (lane == 0) {
        s_e = found;
        s_slot0 = slot0;
        s_m = found >= 0 ? s_cnt[found] : 0;
      }
    }
    __syncthreads();
  }
  if (publisher) {
    // the route table and the permutation of the T tokens
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
    lds_barrier();
    int before = incl - run;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = tid * 4 + i;
      const int excl = before + (i ? loc[i - 1] : 0);
      if (b < NBIN) { s_off[b] = excl; offsets_out[b] = excl; }
      if (b == NBIN - 1) offsets_out[NBIN] = before + loc[i];
    }
    lds_barrier();
    for (int p = tid; p < P; p += kDecThreads) {
      const int id = s_ids[p];
      int rank = 0;
      for (int q = 0; q < p; ++q) rank += (s_ids[q] == id) ? 1 : 0;
      const int slot = s_off[id] + rank;
      sp_out[slot] = p;
      ps_out[p] = slot;
      ids_out[p] = id;
      w_out[p] = s_w[p];
    }
    return;
  }
  const int e = s_e;
  if (e < 0) return;
  const int slot0 = s_slot0;
  // this workgroup's share of the expert's tokens: [tb, tb + m)
  const int tb = (blockIdx.y % nch) * tch;
  if (tb >= s_m) return;
  const int m = min(tch, s_m - tb);

  // tokens of expert e, in pair order
  if (wave == 0) {
    if (fast1) {
      if (lane == 0) s_tok[0] = 0;
    } else if (e < E) {
      int seen = 0;
      for (int base = 0; base < P; base += 64) {
        const int p = base + lane;
        const bool hit = p < P && s_ids[p] == e;
        const uint64_t mask = __ballot(hit);
        if (hit) s_tok[seen + __popcll(mask & ((1ull << lane) - 1))] = p / k;
        seen += __popcll(mask);
      }
    } else if (lane < T) {
      s_tok[lane] = lane;
    }
  }

  lds_barrier();                                     // s_tok ready

  // activation loads of the first token tile, then the weight stream (loads complete in
  // issue order, so the activations arrive first)
  const int NB = H >> 5;
  Stager<4 * MT> stg;
  stg.load(NB, LPR * BPL, min(MT, m), MT,
           [&](int u) -> const float* { return x + (int64_t)s_tok[tb + u] * H; },
           [&](int u) { return rscale ? rscale[s_tok[tb + u]] : 1.0f; });
  // weight loads of this wave (rows stay in registers for every token tile)
  const int64_t row_bytes = (int64_t)NB * kBlockBytes;
  const uint8_t* mat = bank + (int64_t)e * stride;
  const int g = lane / LPR, lig = lane % LPR;
  const bool odd = (lig & 1) != 0;
  const int orow0 = (blockIdx.x * (kDecThreads / 64) + wave) * OROWS;
  RawBlock raw[kUpPasses][BPL];
#pragma unroll
  for (int p = 0; p < kUpPasses; ++p) {
    const int i = p * RPP + g;
    const int r = orow0 + (i < OROWS ? i : i - OROWS);
    const bool ok = r < F;
    const uint8_t* rowp = mat + (int64_t)(ok ? (i < OROWS ? 0 : F) + r : 0) * row_bytes;
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
      const int kb = lig + LPR * b;
      raw[p][b] = load_block(rowp, kb < NB ? kb : NB - 2 + (kb & 1));
    }
  }

  for (int t0 = 0; t0 < m; t0 += MT) {
    const int n_tok = min(MT, m - t0);
    if (t0) {
      lds_barrier();
      stg.load(NB, LPR * BPL, n_tok, MT,
               [&](int u) -> const float* { return x + (int64_t)s_tok[tb + t0 + u] * H; },
               [&](int u) { return rscale ? rscale[s_tok[tb + t0 + u]] : 1.0f; });
    }
    stg.store(s_x);
    lds_barrier();
    float acc[kUpPasses][MT];
    rows_dot<kUpPasses, LPR, BPL, MT>(raw, odd, s_tab, s_x, lig, acc);
#pragma unroll
    for (int p = 0; p < kUpPasses; ++p)
#pragma unroll
      for (int u = 0; u < MT; ++u) acc[p][u] = group_sum_dpp<LPR>(acc[p][u]);
    if (lig == 0) {
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        if (u >= n_tok) continue;
        const int64_t s = slot0 + tb + t0 + u;
#pragma unroll
        for (int p = 0; p < kUpPasses / 2; ++p) {
          const int r = orow0 + p * RPP + g;
          if (r < F) h_out[s * F + r] = silu(acc[p][u]) * acc[p + kUpPasses / 2][u];
        }
      }
    }
  }
}

// ---- down + combine ------------------------------------------------------------------

// NRP row passes of RPP rows per wave and expert; the workgroup owns 4 * NRP * RPP rows.
template <int LPR, int BPL, int NRP, int UPT>
__global__ void __launch_bounds__(kDecThreads) decode_down_combine_kernel(
    const uint8_t* __restrict__ bank, int64_t stride, const float* __restrict__ h,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ pair_slot,
    const float* __restrict__ w, int T, int H, int F, int E, int S, int k,
    const float* residual, float* y) {
  constexpr int RPP = 64 / LPR;
  constexpr int RW = NRP * RPP;                  // rows per wave
  constexpr int R = 4 * RW;                      // rows per workgroup
  extern __shared__ __align__(16) uint32_t s_dyn[];
  __shared__ uint32_t s_tab[256];
  __shared__ int s_off[1025];
  __shared__ int s_act[1024];
  __shared__ int s_nact;
  __shared__ float s_cw[2 * kDecThreads];        // gating weights w[0 .. P)
  __shared__ int s_cps[2 * kDecThreads];         // pair_slot[0 .. P)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = T * k, NBIN = E + S;
  const int rows_total = P + T * S;
  const int NB = F >> 5;
  constexpr int NBP = LPR * BPL;                           // block slots a staged row holds
  uint32_t* s_x = s_dyn;                                   // rows_total x NBP x kXStride
  float* s_o = reinterpret_cast<float*>(s_dyn + rows_total * NBP * kXStride);  // R x rows

  // the codebook pair table first: its two reads of the codebook are waited on at once, and
  // loads complete in issue order, so any load issued before them would be waited on too
  s_tab[tid] = pair_table_entry(tid);
  // load order: the route table (the routed weight addresses wait on it), every slot's h,
  // then the shared expert's weights, which need no route table (loads complete in order)
  int ov[(1025 + kDecThreads - 1) / kDecThreads];
#pragma unroll
  for (int j = 0; j < (1025 + kDecThreads - 1) / kDecThreads; ++j)
    ov[j] = offsets[min(tid + kDecThreads * j, NBIN)];
  // the combine's inputs, read now rather than after the dot products (they were written by
  // earlier launches); relaxed atomic reads, so that the compiler keeps them here instead of
  // sinking them to their use.  P <= 2 * kDecThreads and T * R <= kDecThreads are checked on
  // the host; the reads are clamped and unconditional
  float cwv[2];
  int cpsv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = min(tid + kDecThreads * j, P - 1);
    cwv[j] = __hip_atomic_load(w + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    cpsv[j] = __hip_atomic_load(pair_slot + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  const int rl_c = tid % R, t_c = min(tid / R, T - 1);
  // (read through a pointer that is always valid, then selected: no branch around the load)
  const float* res_p =
      residual ? residual + (int64_t)t_c * H + min((int)blockIdx.x * R + rl_c, H - 1) : w;
  const float res_v = __hip_atomic_load(res_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  Stager<UPT> stg;
  stg.load(NB, NBP, rows_total, rows_total,
           [&](int u) -> const float* { return h + (int64_t)u * F; }, [&](int) { return 1.0f; });

  const int g = lane / LPR, lig = lane % LPR;
  const bool odd = (lig & 1) != 0;
  const int r0 = blockIdx.x * R;
  const int64_t row_bytes = (int64_t)NB * kBlockBytes;
  const int64_t down_off = 2 * (int64_t)F * ((int64_t)(H >> 5) * kBlockBytes);

  auto load_rows = [&](int e, int p, RawBlock (&dst)[BPL]) {
    const int r = r0 + wave * RW + (p % NRP) * RPP + g;
    const bool ok = r < H;
    const uint8_t* rowp = bank + (int64_t)e * stride + down_off + (int64_t)(ok ? r : 0) * row_bytes;
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
      const int kb = lig + LPR * b;
      dst[b] = load_block(rowp, kb < NB ? kb : NB - 2 + (kb & 1));
    }
  };
  // pass p: expert s_act[p / NRP], row pass p % NRP; the shared expert's passes come first
  auto load_pass = [&](int p, RawBlock (&dst)[BPL]) { load_rows(s_act[p / NRP], p, dst); };
  const int pre = S > 0 ? NRP : 0;
  RawBlock ring[kDownRing][BPL];
#pragma unroll
  for (int d = 0; d < kDownRing; ++d)
    if (d < pre) load_rows(E, d, ring[d]);

#pragma unroll
  for (int j = 0; j < (1025 + kDecThreads - 1) / kDecThreads; ++j)
    if (tid + kDecThreads * j <= NBIN) s_off[tid + kDecThreads * j] = ov[j];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    s_cw[tid + kDecThreads * j] = cwv[j];
    s_cps[tid + kDecThreads * j] = cpsv[j];
  }
  lds_barrier();
  // compact list of experts with slots: the shared expert, then the routed ones in index order
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
  lds_barrier();
  const int nact = s_nact;
  const int npass = nact * NRP;
#pragma unroll
  for (int d = 0; d < kDownRing; ++d)
    if (d >= pre && d < npass) load_pass(d, ring[d]);

  // every slot's h -> LDS as bf16 (hi, lo) pairs
  stg.store(s_x);
  lds_barrier();

  for (int p0 = 0; p0 < npass; p0 += kDownRing) {
#pragma unroll
    for (int d = 0; d < kDownRing; ++d) {
      const int p = p0 + d;
      if (p < npass) {
        const int e = s_act[p / NRP];
        const int rl = wave * RW + (p % NRP) * RPP + g;          // row within the tile
        const int sa = s_off[e], sb = s_off[e + 1];
        for (int u = sa; u < sb; ++u) {
          float acc[1] = {0.0f};
#pragma unroll
          for (int b = 0; b < BPL; ++b) {
            XBlock<1> xb;
            xb.load(s_x + u * NBP * kXStride, NBP, lig + LPR * b);
            block_dot<1>(ring[d][b], odd, s_tab, xb, acc);
          }
          const float v = group_sum_dpp<LPR>(acc[0]);
          if (lig == 0) s_o[rl * rows_total + u] = v;
        }
        if (p + kDownRing < npass) load_pass(p + kDownRing, ring[d]);
      }
    }
  }
  __syncthreads();

  // combine in fixed order: routed j = 0..k-1, then shared experts, then the residual
  if (tid < T * R) {
    const int t = tid / R, rl = tid % R;
    const int r = r0 + rl;
    if (r < H) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j)
        acc = fmaf(s_cw[t * k + j], s_o[rl * rows_total + s_cps[t * k + j]], acc);
      for (int sidx = 0; sidx < S; ++sidx) acc += s_o[rl * rows_total + P + sidx * T + t];
      if (residual) acc += res_v;
      y[(int64_t)t * H + r] = acc;
    }
  }
}

// ---- host side -------------------------------------------------------------------------

struct DecGeom {
  int lpr, bpl;
};

static DecGeom dec_geom(int NB) {
  DecGeom best{0, 0};
  int best_waste = 1 << 30;
  const int lprs[5] = {64, 32, 16, 8, 4};
  for (int li = 0; li < 5; ++li) {
    const int bpl = (NB + lprs[li] - 1) / lprs[li];
    if (bpl > 4) continue;
    const int waste = lprs[li] * bpl - NB;
    if (waste < best_waste) {
      best_waste = waste;
      best = DecGeom{lprs[li], bpl};
    }
  }
  return best;
}

static size_t down_lds_bytes(const Shape& sh, int T, int R, int nbp) {
  const int rows_total = T * (sh.k + sh.S);
  return (size_t)rows_total * nbp * kXStride * 4 + (size_t)R * rows_total * 4;
}

constexpr size_t kDownLdsBudget = 96 * 1024;

bool decode_down_fused_fits(const Shape& sh, int T) {
  const int rows_total = T * (sh.k + sh.S);
  const DecGeom g = dec_geom(sh.F / 32);
  const int nbp = g.lpr * g.bpl;
  return g.lpr > 0 && down_lds_bytes(sh, T, 64, nbp) <= kDownLdsBudget &&
         rows_total * nbp * 4 <= kDecThreads * kDownStageUnits;
}

template <int LPR, int BPL, int MT, int P>
static void launch_up(dim3 grid, hipStream_t s, const uint8_t* bank, int64_t stride,
                      const float* x, const float* rs, const float* logits, int T,
                      const Shape& sh, int32_t* ids, float* w, int32_t* off, int32_t* sp,
                      int32_t* ps, float* h, int tch) {
  const size_t lds = (size_t)MT * LPR * BPL * kXStride * 4;
  hipLaunchKernelGGL((decode_gateup_kernel<LPR, BPL, MT, P>), grid, dim3(kDecThreads), lds, s,
                     bank, stride, x, rs, logits, T, sh.H, sh.F, sh.E, sh.S, sh.k, sh.gating,
                     sh.renorm, ids, w, off, sp, ps, h, tch);
}

template <int MT, int P>
static bool dispatch_up(DecGeom gm, dim3 grid, hipStream_t s, const uint8_t* bank,
                        int64_t stride, const float* x, const float* rs, const float* logits,
                        int T, const Shape& sh, int32_t* ids, float* w, int32_t* off,
                        int32_t* sp, int32_t* ps, float* h) {
#define UP(L, B) \
  if (gm.lpr == L && gm.bpl == B) { launch_up<L, B, MT, P>(grid, s, bank, stride, x, rs, logits, T, sh, ids, w, off, sp, ps, h, T); return true; }
  UP(64, 1) UP(64, 2) UP(64, 3) UP(64, 4) UP(32, 1) UP(32, 2) UP(32, 3) UP(32, 4)
  UP(16, 1) UP(16, 2) UP(16, 3) UP(16, 4) UP(8, 1) UP(8, 2) UP(8, 3) UP(8, 4) UP(4, 1)
  UP(4, 2) UP(4, 3) UP(4, 4)
#undef UP
  return false;
}

template <int LPR, int BPL, int NRP>
static void launch_down(hipStream_t s, const uint8_t* bank, int64_t stride, const float* h,
                        const int32_t* off, const int32_t* ps, const float* w, int T,
                        const Shape& sh, const float* residual, float* y) {
  constexpr int R = 4 * NRP * (64 / LPR);
  const size_t lds = down_lds_bytes(sh, T, R, LPR * BPL);
  const dim3 grid((sh.H + R - 1) / R);
  const int units = T * (sh.k + sh.S) * LPR * BPL * 4;
  if (units <= kDecThreads * 4)
    hipLaunchKernelGGL((decode_down_combine_kernel<LPR, BPL, NRP, 4>), grid, dim3(kDecThreads),
                       lds, s, bank, stride, h, off, ps, w, T, sh.H, sh.F, sh.E, sh.S, sh.k,
                       residual, y);
  else
    hipLaunchKernelGGL((decode_down_combine_kernel<LPR, BPL, NRP, kDownStageUnits>), grid,
                       dim3(kDecThreads), lds, s, bank, stride, h, off, ps, w, T, sh.H, sh.F,
                       sh.E, sh.S, sh.k, residual, y);
}

static bool dispatch_down(DecGeom gm, hipStream_t s, const uint8_t* bank, int64_t stride,
                          const float* h, const int32_t* off, const int32_t* ps, const float* w,
                          int T, const Shape& sh, const float* residual, float* y) {
  // rows per workgroup 4 * NRP * RPP: about 16 for every group width, 8 for one-block rows of
  // 32 lanes (FFN 1024: twice the workgroups, 448 over 256 CUs, measured faster).  The
  // combine's inputs are read by one thread each: T * k <= 2 * kDecThreads and T * R <=
  // kDecThreads (R <= 64)
  if ((int64_t)T * sh.k > 2 * kDecThreads || T * 64 > kDecThreads) return false;
#define DN(L, B, N) \
  if (gm.lpr == L && gm.bpl == B) { launch_down<L, B, N>(s, bank, stride, h, off, ps, w, T, sh, residual, y); return true; }
  DN(64, 1, 4) DN(64, 2, 4) DN(64, 3, 4) DN(64, 4, 4) DN(32, 1, 1) DN(32, 2, 2) DN(32, 3, 2)
  DN(32, 4, 2) DN(16, 1, 1) DN(16, 2, 1) DN(16, 3, 1) DN(16, 4, 1) DN(8, 1, 1) DN(8, 2, 1)
  DN(8, 3, 1) DN(8, 4, 1) DN(4, 1, 1) DN(4, 2, 1) DN(4, 3, 1) DN(4, 4, 1)
#undef DN
  return false;
}

// token group: one token at a time when there are few tokens or many W_r registers
template <int EPW, int KM>
static void launch_router(dim3 grid, hipStream_t s, const float* x, const float* wr,
                          const float* bias, int T, const Shape& sh, float e_arg, int use_norm,
                          float* logits, float* rscale, float* xn, uint32_t* xhl) {
  constexpr int kTg = EPW * KM >= 16 ? 1 : (EPW * KM >= 8 ? 2 : 4);
  const int tpg = (T + (int)grid.y - 1) / (int)grid.y;
  if (tpg <= 2 || kTg == 1)
    hipLaunchKernelGGL((decode_router_kernel<EPW, KM, 1>), dim3(grid), dim3(kDecThreads), 0, s,
                       x, wr, bias, T, sh.H, sh.E, e_arg, use_norm, logits, rscale, xn, xhl);
  else
    hipLaunchKernelGGL((decode_router_kernel<EPW, KM, kTg>), dim3(grid), dim3(kDecThreads), 0, s,
                       x, wr, bias, T, sh.H, sh.E, e_arg, use_norm, logits, rscale, xn, xhl);
}

template <int EPW>
static bool dispatch_router(int km, dim3 grid, hipStream_t s, const float* x, const float* wr,
                            const float* bias, int T, const Shape& sh, float e_arg, int use_norm,
                            float* logits, float* rscale, float* xn, uint32_t* xhl) {
  switch (km) {
    case 1: launch_router<EPW, 1>(grid, s, x, wr, bias, T, sh, e_arg, use_norm, logits, rscale, xn, xhl); return true;
    case 2: launch_router<EPW, 2>(grid, s, x, wr, bias, T, sh, e_arg, use_norm, logits, rscale, xn, xhl); return true;
    case 3: case 4: launch_router<EPW, 4>(grid, s, x, wr, bias, T, sh, e_arg, use_norm, logits, rscale, xn, xhl); return true;
    case 5: case 6: case 7: launch_router<EPW, 7>(grid, s, x, wr, bias, T, sh, e_arg, use_norm, logits, rscale, xn, xhl); return true;
    case 8: launch_router<EPW, 8>(grid, s, x, wr, bias, T, sh, e_arg, use_norm, logits, rscale, xn, xhl); return true;
  }
  return false;
}

hipError_t launch_router_rows(const Shape& sh, const float* x, const float* wr,
                              const float* bias, int T, float eps, float* logits,
                              float* rscale, hipStream_t s, float* xn, uint32_t* xhl) {
  // experts a workgroup: at least 256 workgroups where the expert count allows
  const int epw = sh.E >= 256 ? 1 : (sh.E >= 128 ? 2 : 1);
  const int use_norm = eps >= 0.0f ? 1 : 0;
  const float e_arg = use_norm ? eps : 0.0f;
  const int km = (sh.H + 1023) / 1024;
  // more than 4 tokens: groups of at most 4 tokens along the grid's y
  const dim3 grid((sh.E + epw - 1) / epw, T > 4 ? (T + 3) / 4 : 1);
  bool ok;
  if (epw == 2)
    ok = dispatch_router<2>(km, grid, s, x, wr, bias, T, sh, e_arg, use_norm, logits, rscale, xn, xhl);
  else
    ok = dispatch_router<1>(km, grid, s, x, wr, bias, T, sh, e_arg, use_norm, logits, rscale, xn, xhl);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_layer(const Shape& sh, const uint8_t* bank, int64_t stride,
                               const float* wr, const float* bias, const float* x, int T,
                               float eps, const float* residual, float* y, DecodeScratch sc,
                               int stages, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int use_norm = eps >= 0.0f ? 1 : 0;
  hipError_t err = hipSuccess;
  // more tokens, or every slot's h too large for the down workgroup's LDS: the batched
  // kernels (bdecode.hip), also three launches
  if (T > kDecodeFusedMaxT || !decode_down_fused_fits(sh, T))
    return launch_bdecode_layer(sh, bank, stride, wr, bias, x, T, eps, residual, y, sc, stages, s);
  if (stages & 1) {
    err = launch_router_rows(sh, x, wr, bias, T, eps, sc.logits, sc.rscale, s);
    if (err != hipSuccess) return err;
  }
  if (stages & 2) {

  // gate/up with routing: 4 passes of the least-waste geometry (a 16-lane x 7-block geometry
  // with 2 passes for hidden 3584 at 2-4 tokens measured 1.65x slower)
  const int nb = sh.H / 32;
  const DecGeom gu = dec_geom(nb);
  if (gu.lpr == 0) return hipErrorInvalidValue;
  // several tokens over many experts make the in-workgroup routing costly: fewer, larger
  // workgroups (8 passes)
  const bool heavy = T > 1 && sh.E >= 256;
  const int passes = heavy ? 8 : 4;
  const int orows_wg = (kDecThreads / 64) * passes * (64 / gu.lpr) / 2;
  const int max_active = (int)std::min<int64_t>(sh.E, (int64_t)T * sh.k) + sh.S;
  const int tch = T;                               // every token of an expert in one workgroup
  // the last row of the grid is the route-table workgroup (only its column 0 stays)
  dim3 grid((sh.F + orows_wg - 1) / orows_wg, max_active * ((T + tch - 1) / tch) + 1);
  const float* rs = use_norm ? sc.rscale : nullptr;
  bool ok;
  if (heavy && gu.bpl <= 2)
    ok = dispatch_up<2, 8>(gu, grid, s, bank, stride, x, rs, sc.logits, T, sh, sc.ids, sc.w,
                           sc.offsets, sc.sorted_pairs, sc.pair_slot, sc.h);
  else if (heavy)
    ok = dispatch_up<1, 8>(gu, grid, s, bank, stride, x, rs, sc.logits, T, sh, sc.ids, sc.w,
                           sc.offsets, sc.sorted_pairs, sc.pair_slot, sc.h);
  else if (T > 1 && gu.bpl <= 2)
    ok = dispatch_up<2, 4>(gu, grid, s, bank, stride, x, rs, sc.logits, T, sh, sc.ids, sc.w,
                           sc.offsets, sc.sorted_pairs, sc.pair_slot, sc.h);
  else
    ok = dispatch_up<1, 4>(gu, grid, s, bank, stride, x, rs, sc.logits, T, sh, sc.ids, sc.w,
                           sc.offsets, sc.sorted_pairs, sc.pair_slot, sc.h);
  if (!ok) return hipErrorInvalidValue;
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  }
  if (!(stages & 4)) return hipSuccess;

  // down + combine
  const DecGeom dn = dec_geom(sh.F / 32);
  if (!dispatch_down(dn, s, bank, stride, sc.h, sc.offsets, sc.pair_slot, sc.w, T, sh, residual,
                     y))
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
