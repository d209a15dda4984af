// Persistent decode of a stack of MoE layers: ONE launch runs, for l = 0 .. L-1,
//   x <- x + MoE_l(xn),   xn = x / sqrt(mean(x^2) + eps)   (or xn = x)
// for a batch of T <= 16 tokens, with every step of every layer on the device.
//
// PocketLLM "Xing4.0-29B-A4B", section "Known limitations": a decode step made of thousands
// of small launches is bound by submission, and fewer, larger kernels are the lever.  Red
// Lite "What we learned", section "1. The idea": the whole token routed on the GPU, no host
// round trip between layers.  Section "Overview" of the PocketLLM page: every expert stays
// resident and is read in place, indexed by expert.
//
// Work items.  Layer l is a run of tickets: nR router items (logits of RE experts each), nG
// gate/up items (OI output rows of one active expert: gate and up rows, SwiGLU, h in slot
// order), nD down items (R output rows over every active expert, plus the fixed-order
// weighted combine and the residual, written back into x).  The last router item to finish
// selects the top-k of every token and publishes the route table (slots grouped by expert,
// the list of active experts, slot -> token).  Workgroups take tickets from one counter and
// run them in ticket order.  An item waits only for items with SMALLER tickets:
//   router l   waits for every down item of l-1   (x of layer l is final)
//   gate/up l  waits for the route of l            (its expert and tokens)
//   down l     waits for the route of l, then for every gate/up item of l (h is complete)
// so the smallest unfinished ticket is always held by a running workgroup whose waits are
// already met: the queue drains whatever number of workgroups is resident.  Every wait is
// also bounded in time; on expiry the kernel records it in a status word and goes on, so the
// grid always exits.
//
// Before waiting, an item issues the loads that do not depend on what it waits for: router
// items their W_r rows, shared-expert gate/up items their weights, down items their weights
// (they need only the route).  The weights of the next phase are thus streaming while the
// previous phase finishes.
//
// Cross-workgroup data (logits, route table, h, x) never needs cache maintenance: every layer
// has its own buffers, so no L2 of any XCD can hold a line of them from before they were
// written, and producers write them through with device-scope stores.  A producer waits for
// its stores to complete before it counts itself done; a consumer reads them with ordinary
// (cached) loads after it has seen the count, so an XCD fetches shared data such as x once
// into its L2 and its CUs share it.  The last workgroup to exit sets every counter back to
// zero for the next launch.
#include "common.h"
#include "gemv_core.h"
#include "kernels.h"
#include "route_core.h"

namespace moe {

namespace {

constexpr int kChThreads = 256;
constexpr int kChMaxT = 16;
constexpr int kChRing = 16;              // down passes in flight (kChRing / BPL ring slots)
constexpr uint64_t kWaitTicks = 100000000ull;   // bound of one wait, in wall-clock ticks

struct ChainCounter {
  uint32_t v;
  uint32_t pad[31];                      // one counter per 128-byte line
};

struct ChainCtl {
  ChainCounter ticket, exited;
  ChainCounter layer[kChainMaxLayers][4];   // router done, route published, gate/up done, down done
};

enum { kDoneR = 0, kRoute = 1, kDoneG = 2, kDoneD = 3 };

struct ChainParams {
  ChainLayer layer[kChainMaxLayers];
  ChainCtl* ctl;
  uint32_t* status;          // bit 0: a bounded wait expired
  float* x;                  // [T, H]: input of layer 0, output of the last layer
  uint8_t* lay;              // per-layer buffers, lay_stride bytes a layer
  int64_t lay_stride;
  int32_t off_x, off_logits, off_rscale, off_w, off_ps, off_slot_tok, off_act, off_h;
  int32_t* ids_out;          // optional [L, T, k]
  float* w_out;              // optional [L, T, k]
  int T, H, F, E, S, k, gating, renorm, use_norm;
  float eps;
  int n_layers, nR, nG, nD, g_chunks;
};

// Buffers of layer l (fresh addresses for every layer):
//   x      [T, H]   input of layer l (layer 0 reads the caller's x)
//   logits [T, E]; rscale [T]; w, pair_slot [T*k]; slot_tok [rows];
//   act    [1 + 3E] number of active routed experts, then (expert, first slot, slots)
//   h      [rows, F]
template <class V>
__device__ __forceinline__ V* lay_ptr(const ChainParams& p, int l, int32_t off) {
  return reinterpret_cast<V*>(p.lay + (int64_t)l * p.lay_stride + off);
}
__device__ __forceinline__ float* x_in(const ChainParams& p, int l) {
  return l == 0 ? p.x : lay_ptr<float>(p, l, p.off_x);
}
__device__ __forceinline__ float* x_out(const ChainParams& p, int l) {
  return l == p.n_layers - 1 ? p.x : lay_ptr<float>(p, l + 1, p.off_x);
}

// Device-scope (write-through) stores of cross-workgroup data.
__device__ __forceinline__ void st_dev(float* a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t* a, int32_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- cross-workgroup synchronisation ---------------------------------------------------

__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whole workgroup: wait until *ctr >= target (thread 0 polls the device-scope value).
__device__ __forceinline__ void wg_wait(const ChainParams& p, const uint32_t* ctr,
                                        uint32_t target) {
  if (threadIdx.x == 0 && load_agent(ctr) < target) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (true) {
      __builtin_amdgcn_s_sleep(1);
      if (load_agent(ctr) >= target) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
        atomicOr(p.status, 1u);
        break;
      }
    }
  }
  lds_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");   // later loads stay after the wait
}

// Whole workgroup: once every store of the workgroup has completed, count it in *ctr.
// Returns the counter's value before the increment (the same in every thread).
__device__ __forceinline__ uint32_t wg_signal(uint32_t* ctr, int* s_i) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);                            // this wave's stores are done
  lds_barrier();
  if (threadIdx.x == 0) s_i[1] = (int)atomicAdd(ctr, 1u);
  lds_barrier();
  return (uint32_t)s_i[1];
}

__device__ __forceinline__ uint32_t* counter(const ChainParams& p, int l, int which) {
  return &p.ctl->layer[l][which].v;
}

// ---- route table (by the last router item of a layer) ---------------------------------

__device__ __forceinline__ void publish_route(const ChainParams& p, int l, uint32_t* s_dyn, int* s_i) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = p.T, E = p.E, k = p.k, S = p.S, P = T * k, NBIN = E + S;
  int* s_ids = reinterpret_cast<int*>(s_dyn);            // [P]
  float* s_w = reinterpret_cast<float*>(s_ids + P);      // [P]
  int* s_cnt = reinterpret_cast<int*>(s_w + P);          // [NBIN]
  int* s_off = s_cnt + NBIN;                             // [NBIN + 1]
  int* s_wave = s_off + NBIN + 1;                        // [4]

  for (int t = wave; t < T; t += 4)
    wave_topk(lay_ptr<float>(p, l, p.off_logits) + (size_t)t * E, E, k, p.gating, p.renorm,
              s_ids + t * k, s_w + t * k);
  for (int i = tid; i < NBIN; i += kChThreads) s_cnt[i] = 0;
  lds_barrier();
  for (int i = tid; i < P; i += kChThreads) atomicAdd(&s_cnt[s_ids[i]], 1);   // counts only
  lds_barrier();
  if (tid < S) s_cnt[E + tid] = T;
  lds_barrier();

  // exclusive scan of the bins (<= 1024: four a thread)
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
  for (int wv = 0; wv < wave; ++wv) before += s_wave[wv];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = tid * 4 + i;
    if (b < NBIN) s_off[b] = before + (i ? loc[i - 1] : 0);
    if (b == NBIN - 1) s_off[NBIN] = before + loc[i];
  }
  lds_barrier();

  // routed slots: pairs of an expert in ascending pair id
  int32_t* pair_slot = lay_ptr<int32_t>(p, l, p.off_ps);
  int32_t* slot_tok = lay_ptr<int32_t>(p, l, p.off_slot_tok);
  int32_t* act = lay_ptr<int32_t>(p, l, p.off_act);
  float* wl = lay_ptr<float>(p, l, p.off_w);
  for (int q = tid; q < P; q += kChThreads) {
    const int id = s_ids[q];
    int rank = 0;
    for (int o = 0; o < q; ++o) rank += (s_ids[o] == id) ? 1 : 0;
    const int slot = s_off[id] + rank;
    st_dev(pair_slot + q, slot);
    st_dev(slot_tok + slot, q / k);
    st_dev(wl + q, s_w[q]);
    if (p.ids_out) p.ids_out[(size_t)l * P + q] = id;
    if (p.w_out) p.w_out[(size_t)l * P + q] = s_w[q];
  }
  for (int i = tid; i < T * S; i += kChThreads) st_dev(slot_tok + P + i, i % T);   // slot P + s*T + t
  // active routed experts in index order
  if (wave == 0) {
    int seen = 0;
    for (int base = 0; base < E; base += 64) {
      const int b = base + lane;
      const int c = b < E ? s_cnt[b] : 0;
      const uint64_t mask = __ballot(c > 0);
      if (c > 0) {
        const int j = seen + __popcll(mask & ((1ull << lane) - 1));
        st_dev(act + 1 + 3 * j, b);
        st_dev(act + 2 + 3 * j, s_off[b]);
        st_dev(act + 3 + 3 * j, c);
      }
      seen += __popcll(mask);
    }
    if (lane == 0) st_dev(act, seen);
  }
  wg_signal(counter(p, l, kRoute), s_i);
}

// ---- router item: logits of experts [ri*RE, ri*RE + RE) for every token ----------------

template <int RE, int RK>
__device__ __forceinline__ void router_item(const ChainParams& p, int l, int ri, uint32_t* s_dyn,
                                            int* s_i) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = p.T, H = p.H, E = p.E;
  const int H4 = H >> 2;
  const ChainLayer& L = p.layer[l];
  const int e0 = ri * RE;
  // W_r rows first: they do not depend on the previous layer
  float4 w[RE][RK];
#pragma unroll
  for (int i = 0; i < RK; ++i) {
    const int h4 = tid + kChThreads * i;
#pragma unroll
    for (int q = 0; q < RE; ++q)
      w[q][i] = (h4 < H4 && e0 + q < E)
                    ? reinterpret_cast<const float4*>(L.wr + (size_t)(e0 + q) * H)[h4]
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (l > 0) wg_wait(p, counter(p, l - 1, kDoneD), (uint32_t)p.nD);

  float* s_red = reinterpret_cast<float*>(s_dyn);        // [4][kChMaxT][RE + 1]
  const float* xl = x_in(p, l);
  for (int t = 0; t < T; ++t) {
    float4 v[RK];
#pragma unroll
    for (int i = 0; i < RK; ++i) {
      const int h4 = tid + kChThreads * i;
      v[i] = h4 < H4 ? reinterpret_cast<const float4*>(xl + (size_t)t * H)[h4]
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float ss = 0.0f, acc[RE];
#pragma unroll
    for (int q = 0; q < RE; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int i = 0; i < RK; ++i) {
      ss = fmaf(v[i].x, v[i].x, ss); ss = fmaf(v[i].y, v[i].y, ss);
      ss = fmaf(v[i].z, v[i].z, ss); ss = fmaf(v[i].w, v[i].w, ss);
#pragma unroll
      for (int q = 0; q < RE; ++q) {
        float c = acc[q];
        c = fmaf(w[q][i].x, v[i].x, c); c = fmaf(w[q][i].y, v[i].y, c);
        c = fmaf(w[q][i].z, v[i].z, c); c = fmaf(w[q][i].w, v[i].w, c);
        acc[q] = c;
      }
    }
    float* red = s_red + (wave * kChMaxT + t) * (RE + 1);
    const float s0 = group_sum_dpp<64>(ss);
    if (lane == 0) red[RE] = s0;
#pragma unroll
    for (int q = 0; q < RE; ++q) {
      const float s1 = group_sum_dpp<64>(acc[q]);
      if (lane == 0) red[q] = s1;
    }
  }
  lds_barrier();
  if (tid < RE * T) {
    const int q = tid / T, t = tid - q * T;
    const int e = e0 + q;
    if (e < E) {
      auto at = [&](int wv, int c) { return s_red[(wv * kChMaxT + t) * (RE + 1) + c]; };
      const float dot = (at(0, q) + at(1, q)) + (at(2, q) + at(3, q));
      float r = 1.0f;
      if (p.use_norm) {
        const float sq = (at(0, RE) + at(1, RE)) + (at(2, RE) + at(3, RE));
        r = 1.0f / sqrtf(sq / (float)H + p.eps);
      }
      st_dev(lay_ptr<float>(p, l, p.off_logits) + (size_t)t * E + e,
             r * dot + (L.bias ? L.bias[e] : 0.0f));
      if (ri == 0 && q == 0) st_dev(lay_ptr<float>(p, l, p.off_rscale) + t, r);
    }
  }
  if (wg_signal(counter(p, l, kDoneR), s_i) == (uint32_t)(p.nR - 1)) publish_route(p, l, s_dyn, s_i);
}

// ---- gate/up item: output rows [c*OI, c*OI + OI) of the j-th active expert -------------
// j < S: shared expert j (known without the route); j >= S: routed active expert j - S.

template <int LPR, int BPL, int NP>
__device__ __forceinline__ void gu_weights(const uint8_t* mat, int NB, int F, int orow0,
                                           RawBlock (&raw)[NP][BPL]) {
  constexpr int RPP = 64 / LPR;
  constexpr int OW = NP * RPP / 2;
  const int lane = threadIdx.x & 63;
  const int g = lane / LPR, lig = lane % LPR;
  const int64_t row_bytes = (int64_t)NB * kBlockBytes;
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int i = q * RPP + g;
    const int r = orow0 + (i < OW ? i : i - OW);
    const bool ok = r < F;
    const uint8_t* rowp = mat + (int64_t)(ok ? (i < OW ? 0 : F) + r : 0) * row_bytes;
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
      const int kb = lig + LPR * b;
      raw[q][b] = load_block(rowp, kb < NB ? kb : NB - 2 + (kb & 1));
    }
  }
}

template <int LPR, int BPL, int NP, int MT, bool SHARED>
__device__ __forceinline__ void gateup_body(const ChainParams& p, int l, int j, int c,
                                            uint32_t* s_x, const uint32_t* s_tab, int* s_i,
                                            int* s_tok) {
  constexpr int RPP = 64 / LPR;
  constexpr int OW = NP * RPP / 2;                 // output rows per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = p.T, H = p.H, F = p.F, E = p.E, P = T * p.k;
  const int NB = H >> 5;
  const int g = lane / LPR, lig = lane % LPR;
  const bool odd = (lig & 1) != 0;
  const int orow0 = c * 4 * OW + wave * OW;
  const ChainLayer& L = p.layer[l];

  RawBlock raw[NP][BPL];
  int slot0, m;
  if constexpr (SHARED) {
    gu_weights<LPR, BPL, NP>(L.bank + (int64_t)(E + j) * L.stride, NB, F, orow0, raw);
    wg_wait(p, counter(p, l, kRoute), 1u);
    slot0 = P + j * T;
    m = T;
    if (tid < T) s_tok[tid] = tid;
  } else {
    wg_wait(p, counter(p, l, kRoute), 1u);
    const int jr = j - p.S;
    const uint32_t* act = lay_ptr<const uint32_t>(p, l, p.off_act);
    if (tid == 0) {
      const int n = (int)load_agent(act);
      s_i[2] = n;
      if (jr < n) {
        s_i[3] = (int)load_agent(act + 1 + 3 * jr);
        s_i[4] = (int)load_agent(act + 2 + 3 * jr);
        s_i[5] = (int)load_agent(act + 3 + 3 * jr);
      }
    }
    lds_barrier();
    if (jr >= s_i[2]) return;                      // fewer active experts than the bound
    slot0 = s_i[4];
    m = s_i[5];
    if (tid < m) s_tok[tid] = lay_ptr<const int32_t>(p, l, p.off_slot_tok)[slot0 + tid];
  }
  lds_barrier();                                   // s_tok

  // activations of the first token tile, then (routed) the weight stream
  const float* rs = p.use_norm ? lay_ptr<const float>(p, l, p.off_rscale) : nullptr;
  const float* xl = x_in(p, l);
  float* hl = lay_ptr<float>(p, l, p.off_h);
  constexpr int UPT = (MT * LPR * BPL * 4 + kChThreads - 1) / kChThreads;
  Stager<UPT> stg;
  stg.load(NB, LPR * BPL, min(MT, m), MT,
           [&](int u) -> const float* { return xl + (int64_t)s_tok[u] * H; },
           [&](int u) { return rs ? rs[s_tok[u]] : 1.0f; });
  if constexpr (!SHARED)
    gu_weights<LPR, BPL, NP>(L.bank + (int64_t)s_i[3] * L.stride, NB, F, orow0, raw);

  for (int t0 = 0; t0 < m; t0 += MT) {
    const int n_tok = min(MT, m - t0);
    if (t0) {
      lds_barrier();
      stg.load(NB, LPR * BPL, n_tok, MT,
               [&](int u) -> const float* { return xl + (int64_t)s_tok[t0 + u] * H; },
               [&](int u) { return rs ? rs[s_tok[t0 + u]] : 1.0f; });
    }
    stg.store(s_x);
    lds_barrier();
    float acc[NP][MT];
    rows_dot<NP, LPR, BPL, MT>(raw, odd, s_tab, s_x, lig, acc);
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int u = 0; u < MT; ++u) acc[q][u] = group_sum_dpp<LPR>(acc[q][u]);
    if (lig == 0) {
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        if (u >= n_tok) continue;
        const int64_t s = slot0 + t0 + u;
#pragma unroll
        for (int q = 0; q < NP / 2; ++q) {
          const int r = orow0 + q * RPP + g;
          if (r < F) st_dev(hl + s * F + r, silu(acc[q][u]) * acc[q + NP / 2][u]);
        }
      }
    }
  }
}

// ---- down item: rows [di*R, di*R + R) of y over every active expert, then the combine ---

template <int LPR, int BPL, int NRP, int UPT>
__device__ __forceinline__ void down_item(const ChainParams& p, int l, int di, uint32_t* s_dyn,
                                          const uint32_t* s_tab, int* s_i) {
  constexpr int RPP = 64 / LPR;
  constexpr int RW = NRP * RPP;                    // rows per wave
  constexpr int R = 4 * RW;                        // rows per item
  constexpr int NBP = LPR * BPL;                   // block slots of a staged row
  constexpr int RING = kChRing / BPL;              // passes in flight
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = p.T, H = p.H, F = p.F, E = p.E, S = p.S, k = p.k, P = T * k;
  const int rows_total = P + T * S;
  const int NB = F >> 5;
  const ChainLayer& L = p.layer[l];
  uint32_t* s_x = s_dyn;                                               // rows_total x NBP slots
  float* s_o = reinterpret_cast<float*>(s_dyn + rows_total * NBP * kXStride);  // R x rows_total
  int* s_ae = reinterpret_cast<int*>(s_o + R * rows_total);            // active: expert
  int* s_as = s_ae + (E + S);                                          //         first slot
  int* s_am = s_as + (E + S);                                          //         slot count

  wg_wait(p, counter(p, l, kRoute), 1u);
  const int32_t* act = lay_ptr<const int32_t>(p, l, p.off_act);
  if (tid == 0) s_i[2] = (int)load_agent(reinterpret_cast<const uint32_t*>(act));
  lds_barrier();
  const int nr = s_i[2];
  const int nact = nr + S;
  for (int j = tid; j < nact; j += kChThreads) {
    if (j < nr) {
      s_ae[j] = act[1 + 3 * j];
      s_as[j] = act[2 + 3 * j];
      s_am[j] = act[3 + 3 * j];
    } else {
      s_ae[j] = E + (j - nr);
      s_as[j] = P + (j - nr) * T;
      s_am[j] = T;
    }
  }
  lds_barrier();
  const int npass = nact * NRP;

  const int g = lane / LPR, lig = lane % LPR;
  const bool odd = (lig & 1) != 0;
  const int r0 = di * R;
  const int64_t row_bytes = (int64_t)NB * kBlockBytes;
  const int64_t down_off = 2 * (int64_t)F * ((int64_t)(H >> 5) * kBlockBytes);

  auto load_pass = [&](int q, RawBlock (&dst)[BPL]) {
    const int e = s_ae[q / NRP];
    const int r = r0 + wave * RW + (q % NRP) * RPP + g;
    const bool ok = r < H;
    const uint8_t* rowp = L.bank + (int64_t)e * L.stride + down_off + (int64_t)(ok ? r : 0) * row_bytes;
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
      const int kb = lig + LPR * b;
      dst[b] = load_block(rowp, kb < NB ? kb : NB - 2 + (kb & 1));
    }
  };

  RawBlock ring[RING][BPL];
#pragma unroll
  for (int d = 0; d < RING; ++d)
    if (d < npass) load_pass(d, ring[d]);

  // h of every slot, once all gate/up items of the layer are done
  wg_wait(p, counter(p, l, kDoneG), (uint32_t)p.nG);
  Stager<UPT> stg;
  const float* hl = lay_ptr<const float>(p, l, p.off_h);
  stg.load(NB, NBP, rows_total, rows_total,
           [&](int u) -> const float* { return hl + (int64_t)u * F; }, [&](int) { return 1.0f; });
  stg.store(s_x);
  lds_barrier();

  for (int q0 = 0; q0 < npass; q0 += RING) {
#pragma unroll
    for (int d = 0; d < RING; ++d) {
      const int q = q0 + d;
      if (q < npass) {
        const int ja = q / NRP;
        const int rl = wave * RW + (q % NRP) * RPP + g;          // row within the item
        const int sa = s_as[ja], sb = sa + s_am[ja];
        for (int u = sa; u < sb; ++u) {
          float acc[1] = {0.0f};
#pragma unroll
          for (int b = 0; b < BPL; ++b) {
            XBlock<1> xb;
            xb.load(s_x + u * NBP * kXStride, NBP, lig + LPR * b);
            block_dot<1>(fresh(ring[d][b]), odd, s_tab, xb, acc);
          }
          const float v = group_sum_dpp<LPR>(acc[0]);
          if (lig == 0) s_o[rl * rows_total + u] = v;
        }
        if (q + RING < npass) load_pass(q + RING, ring[d]);
      }
    }
  }
  lds_barrier();

  // combine in fixed order: routed j = 0..k-1, then the shared expert, then the residual x
  const float* wl = lay_ptr<const float>(p, l, p.off_w);
  const int32_t* psl = lay_ptr<const int32_t>(p, l, p.off_ps);
  const float* xi = x_in(p, l);
  float* xo = x_out(p, l);
  for (int i = tid; i < T * R; i += kChThreads) {
    const int t = i / R, rl = i % R;
    const int r = r0 + rl;
    if (r >= H) continue;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j)
      acc = fmaf(wl[t * k + j], s_o[rl * rows_total + psl[t * k + j]], acc);
    for (int sidx = 0; sidx < S; ++sidx) acc += s_o[rl * rows_total + P + sidx * T + t];
    acc += xi[(int64_t)t * H + r];
    st_dev(xo + (int64_t)t * H + r, acc);
  }
}

// ---- the kernel --------------------------------------------------------------------------

template <int RE, int RK, int GL, int GB, int GN, int GMT, int DL, int DB, int DN, int DU>
__global__ void __launch_bounds__(kChThreads, 2) chain_kernel(const ChainParams p) {
  extern __shared__ __align__(16) uint32_t s_dyn[];
  __shared__ uint32_t s_tab[256];
  __shared__ int s_i[8];
  __shared__ int s_tok[kChMaxT];
  const int tid = threadIdx.x;
  s_tab[tid] = pair_table_entry(tid);
  if (tid == 0) s_i[0] = (int)atomicAdd(&p.ctl->ticket.v, 1u);
  lds_barrier();
  const int per_layer = p.nR + p.nG + p.nD;
  const int total = per_layer * p.n_layers;
  int cur = s_i[0];
  while (cur < total) {
    int next = 0;
    if (tid == 0) next = (int)atomicAdd(&p.ctl->ticket.v, 1u);   // the next ticket, early
    const int l = cur / per_layer, r = cur - l * per_layer;
    if (r < p.nR) {
      router_item<RE, RK>(p, l, r, s_dyn, s_i);
    } else if (r < p.nR + p.nG) {
      const int gi = r - p.nR;
      const int j = gi / p.g_chunks, c = gi - j * p.g_chunks;
      if (j < p.S)
        gateup_body<GL, GB, GN, GMT, true>(p, l, j, c, s_dyn, s_tab, s_i, s_tok);
      else
        gateup_body<GL, GB, GN, GMT, false>(p, l, j, c, s_dyn, s_tab, s_i, s_tok);
      wg_signal(counter(p, l, kDoneG), s_i);
    } else {
      down_item<DL, DB, DN, DU>(p, l, r - p.nR - p.nG, s_dyn, s_tab, s_i);
      wg_signal(counter(p, l, kDoneD), s_i);
    }
    lds_barrier();
    if (tid == 0) s_i[0] = next;
    lds_barrier();
    cur = s_i[0];
  }
  // the last workgroup out resets the counters for the next launch
  if (tid == 0) {
    const uint32_t old = atomicAdd(&p.ctl->exited.v, 1u);
    if (old == gridDim.x - 1) {
      p.ctl->ticket.v = 0;
      p.ctl->exited.v = 0;
      for (int l = 0; l < p.n_layers; ++l)
        for (int q = 0; q < 4; ++q) p.ctl->layer[l][q].v = 0;
    }
  }
}

// ---- host side ---------------------------------------------------------------------------

struct ChainGeom {
  int re, rk;               // router: experts an item, float4 a thread and expert row
  int gl, gb, gn, gmt;      // gate/up: lanes a row, blocks a lane, passes, token tile
  int dl, db, dn, du;       // down: lanes a row, blocks a lane, passes an expert, staging units
};

template <int RE, int RK, int GL, int GB, int GN, int GMT, int DL, int DB, int DN, int DU>
static void* kernel_of() {
  return reinterpret_cast<void*>(&chain_kernel<RE, RK, GL, GB, GN, GMT, DL, DB, DN, DU>);
}

// The instantiated configurations: (H, F) shapes of the decode workloads, T = 1 and T > 1.
struct ChainInst {
  int H, F, gmt, du;
  ChainGeom g;
  void* (*fn)();
};

#define CH_INST(H_, F_, RE, RK, GL, GB, GN, GMT, DL, DB, DN, DU)                          \
  ChainInst{H_, F_, GMT, DU, ChainGeom{RE, RK, GL, GB, GN, GMT, DL, DB, DN, DU},           \
            &kernel_of<RE, RK, GL, GB, GN, GMT, DL, DB, DN, DU>}

static const ChainInst kInst[] = {
    // hidden 3584, ffn 1024 (64 experts)
    CH_INST(3584, 1024, 4, 4, 16, 7, 2, 1, 32, 1, 2, 4),
    CH_INST(3584, 1024, 4, 4, 16, 7, 2, 2, 32, 1, 2, 8),
    // hidden 2048, ffn 512 (512 experts)
    CH_INST(2048, 512, 8, 2, 16, 4, 4, 1, 16, 1, 2, 4),
    CH_INST(2048, 512, 8, 2, 16, 4, 4, 2, 16, 1, 2, 8),
    // hidden 7168, ffn 1536 (384 experts)
    CH_INST(7168, 1536, 2, 7, 32, 7, 2, 1, 16, 3, 1, 8),
    // hidden 256, ffn 128 (small layers)
    CH_INST(256, 128, 2, 1, 8, 1, 2, 1, 4, 1, 1, 4),
    CH_INST(256, 128, 2, 1, 8, 1, 2, 2, 4, 1, 1, 4),
};

struct ChainPlan {
  const ChainInst* inst;
  int nR, nG, nD, g_chunks;
  size_t lds;
};

constexpr size_t kChainLdsLimit = 64 * 1024;

static bool plan_chain(const Shape& sh, int T, ChainPlan& pl) {
  const int gmt = T > 1 ? 2 : 1;
  const int rows_total = T * (sh.k + sh.S);
  for (const ChainInst& in : kInst) {
    if (in.H != sh.H || in.F != sh.F || in.gmt != gmt) continue;
    const ChainGeom& g = in.g;
    const int dnbp = g.dl * g.db;
    if (rows_total * dnbp * 4 > kChThreads * g.du) continue;       // staging units
    const int oi = 4 * g.gn * (64 / g.gl) / 2;                   // gate/up output rows an item
    const int rd = 4 * g.dn * (64 / g.dl);                       // down rows an item
    const int na_max = std::min(sh.E, T * sh.k) + sh.S;
    pl.inst = &in;
    pl.g_chunks = (sh.F + oi - 1) / oi;
    pl.nR = (sh.E + g.re - 1) / g.re;
    pl.nG = na_max * pl.g_chunks;
    pl.nD = (sh.H + rd - 1) / rd;
    const int P = T * sh.k, NBIN = sh.E + sh.S;
    const size_t lds_r = (size_t)4 * kChMaxT * (g.re + 1) * 4;
    const size_t lds_pub = (size_t)(2 * P + 2 * NBIN + 1 + 4) * 4;
    const size_t lds_g = (size_t)gmt * g.gl * g.gb * kXStride * 4;
    const size_t lds_d = (size_t)rows_total * dnbp * kXStride * 4 + (size_t)rd * rows_total * 4 +
                         (size_t)3 * NBIN * 4;
    pl.lds = std::max(std::max(lds_r, lds_pub), std::max(lds_g, lds_d));
    if (pl.lds > kChainLdsLimit) return false;
    return true;
  }
  return false;
}

}  // namespace

static_assert(sizeof(ChainCtl) == kChainControlBytes, "control block layout");

bool chain_supported(const Shape& sh, int T) {
  ChainPlan pl;
  return T >= 1 && T <= kChMaxT && plan_chain(sh, T, pl);
}

hipError_t launch_decode_chain(const Shape& sh, const ChainLayer* layers, int n_layers,
                               float* x, int T, float eps, int32_t* ids_out, float* w_out,
                               const ChainScratch& sc, hipStream_t s) {
  ChainPlan pl;
  if (T < 1 || T > kChMaxT || n_layers < 1 || n_layers > kChainMaxLayers || !plan_chain(sh, T, pl))
    return hipErrorInvalidValue;
  ChainParams p;
  for (int l = 0; l < n_layers; ++l) p.layer[l] = layers[l];
  for (int l = n_layers; l < kChainMaxLayers; ++l) p.layer[l] = ChainLayer{nullptr, 0, nullptr, nullptr};
  p.ctl = reinterpret_cast<ChainCtl*>(sc.control);
  p.status = sc.status;
  p.x = x;
  p.lay = static_cast<uint8_t*>(sc.layers);
  p.lay_stride = sc.layer_stride;
  p.off_x = sc.off_x; p.off_logits = sc.off_logits; p.off_rscale = sc.off_rscale;
  p.off_w = sc.off_w; p.off_ps = sc.off_ps; p.off_slot_tok = sc.off_slot_tok;
  p.off_act = sc.off_act; p.off_h = sc.off_h;
  p.ids_out = ids_out;
  p.w_out = w_out;
  p.T = T; p.H = sh.H; p.F = sh.F; p.E = sh.E; p.S = sh.S; p.k = sh.k;
  p.gating = sh.gating; p.renorm = sh.renorm;
  p.use_norm = eps >= 0.0f ? 1 : 0;
  p.eps = p.use_norm ? eps : 0.0f;
  p.n_layers = n_layers;
  p.nR = pl.nR; p.nG = pl.nG; p.nD = pl.nD; p.g_chunks = pl.g_chunks;
  const int total = (pl.nR + pl.nG + pl.nD) * n_layers;
  const int grid = std::min(total, 2 * device_cu_count());
  void* args[] = {&p};
  return hipLaunchKernel(pl.inst->fn(), dim3(grid), dim3(kChThreads), args, pl.lds, s);
}

}  // namespace moe
