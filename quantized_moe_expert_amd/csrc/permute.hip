// Route sanitisation and the token-to-expert permutation.
//
// "Running Qwen Flash-Next NVFP4 in vLLM", B12x integration: a route is valid only when its
// expert id is non-negative and below the expert count; an invalid route is redirected to
// expert zero AND its routing weight is set to zero, so padding contributes nothing.
// PocketLLM "Xing4.0-29B-A4B", section "Without a server": the grouped MoE kernel works on a
// route table.  The pairs (t, j) (pair id p = t*k + j) are grouped by expert: a histogram over
// the experts, an exclusive scan, and a stable scatter (rank = number of earlier pairs with
// the same expert), then the inverse map.  Ranks are counted, never decided by atomics, so
// the result is exact and identical on every run.
//
// Small route tables (decode) run in one workgroup; larger ones in three kernels
// (per-block histograms -> one scan workgroup -> scatter), plus an optional row gather.
#include "common.h"
#include "kernels.h"
#include "route_core.h"

namespace moe {

constexpr int kSmallThreads = 1024;
constexpr int kPairsPerBlock = 256;

// Inclusive prefix sum over a workgroup of 1024 threads (fixed order).
__device__ int block_scan_1024(int v, int* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int t = lane < 16 ? s_wave[lane] : 0;
    for (int d = 1; d < 16; d <<= 1) {
      const int o = __shfl_up(t, d, 64);
      if (lane >= d) t += o;
    }
    if (lane < 16) s_wave[lane] = t;
  }
  __syncthreads();
  const int r = v + (wave ? s_wave[wave - 1] : 0);
  __syncthreads();
  return r;
}

__device__ __forceinline__ int sanitize_one(int32_t* ids, float* w, int p, int E, int& bad) {
  int id = ids[p];
  if (id < 0 || id >= E) {
    id = 0;
    ids[p] = 0;
    w[p] = 0.0f;
    bad = 1;
  }
  return id;
}

// Offsets, sorted pairs and the inverse map of P <= 1024 sanitised pair ids in s_id (LDS),
// by one workgroup of 1024 threads: histogram, scan, stable rank.
__device__ void permute_small_core(const int* s_id, int P, int T, int E, int S, int* s_cnt,
                                   int* s_off, int* s_wave, int32_t* __restrict__ offsets,
                                   int32_t* __restrict__ sorted_pairs,
                                   int32_t* __restrict__ pair_slot) {
  const int tid = threadIdx.x;
  const int NB = E + S;
  s_cnt[tid] = 0;
  __syncthreads();
  const int id = tid < P ? s_id[tid] : 0;
  if (tid < P) atomicAdd(&s_cnt[id], 1);
  __syncthreads();
  const int c = tid < E ? s_cnt[tid] : (tid < NB ? T : 0);
  const int incl = block_scan_1024(c, s_wave);
  if (tid < NB) {
    s_off[tid] = incl - c;
    offsets[tid] = incl - c;
  }
  if (tid == NB - 1) offsets[NB] = incl;
  __syncthreads();
  if (tid < P) {
    int rank = 0;
    for (int q = 0; q < tid; ++q) rank += (s_id[q] == id) ? 1 : 0;
    const int slot = s_off[id] + rank;
    sorted_pairs[slot] = tid;
    pair_slot[tid] = slot;
  }
}

// Whole permutation in one workgroup: P = T*k <= 1024 pairs and E + S <= 1024 bins.
__global__ void __launch_bounds__(1024) permute_small_kernel(
    int32_t* __restrict__ ids, float* __restrict__ w, int T, int k, int E, int S,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_slot, int32_t* __restrict__ invalid_count) {
  __shared__ int s_id[kSmallThreads];
  __shared__ int s_cnt[kSmallThreads];
  __shared__ int s_off[kSmallThreads + 1];
  __shared__ int s_wave[16];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int P = T * k;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (tid < P) {
    int bad = 0;
    s_id[tid] = sanitize_one(ids, w, tid, E, bad);
    if (bad) atomicAdd(&s_bad, 1);          // a count: the order of adds does not matter
  }
  __syncthreads();
  permute_small_core(s_id, P, T, E, S, s_cnt, s_off, s_wave, offsets, sorted_pairs, pair_slot);
  if (tid == 0) *invalid_count = s_bad;
}

// Pass 1: sanitise, per-block histogram -> counts[blk * E + e]; invalid count per block.
__global__ void __launch_bounds__(kPairsPerBlock) permute_count_kernel(
    int32_t* __restrict__ ids, float* __restrict__ w, int P, int E,
    int32_t* __restrict__ counts, int32_t* __restrict__ bad_counts) {
  extern __shared__ int s_hist[];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPairsPerBlock) s_hist[e] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  const int p = blockIdx.x * kPairsPerBlock + tid;
  if (p < P) {
    int bad = 0;
    const int id = sanitize_one(ids, w, p, E, bad);
    if (bad) atomicAdd(&s_bad, 1);
    atomicAdd(&s_hist[id], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPairsPerBlock) counts[(size_t)blockIdx.x * E + e] = s_hist[e];
  if (tid == 0) bad_counts[blockIdx.x] = s_bad;
}

// Pass 2 (one workgroup): per expert, exclusive prefix over blocks (in place) and the
// expert total; exclusive scan of the totals -> offsets; sum of invalid counts.
__global__ void __launch_bounds__(1024) permute_scan_kernel(
    int32_t* __restrict__ counts, const int32_t* __restrict__ bad_counts, int nblk, int T,
    int k, int E, int S, int32_t* __restrict__ offsets, int32_t* __restrict__ invalid_count) {
  __shared__ int s_wave[16];
  __shared__ int s_tot[1024];
  const int tid = threadIdx.x;
  const int NB = E + S;
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      const int c = counts[(size_t)b * E + e];
      counts[(size_t)b * E + e] = run;
      run += c;
    }
    s_tot[e] = run;
  }
  __syncthreads();
  const int c = tid < E ? s_tot[tid] : (tid < NB ? T : 0);
  const int incl = block_scan_1024(c, s_wave);
  if (tid < NB) offsets[tid] = incl - c;
  if (tid == NB - 1) offsets[NB] = incl;
  if (tid == 0) {
    int bad = 0;
    for (int b = 0; b < nblk; ++b) bad += bad_counts[b];
    *invalid_count = bad;
  }
}

// Pass 3: stable scatter.  slot = offsets[e] + (pairs of e in earlier blocks) + rank in block.
__global__ void __launch_bounds__(kPairsPerBlock) permute_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_slot) {
  __shared__ int s_id[kPairsPerBlock];
  const int tid = threadIdx.x;
  const int p = blockIdx.x * kPairsPerBlock + tid;
  const int id = p < P ? ids[p] : -1;
  s_id[tid] = id;
  __syncthreads();
  if (p < P) {
    int rank = 0;
    for (int q = 0; q < tid; ++q) rank += (s_id[q] == id) ? 1 : 0;
    const int slot = offsets[id] + counts[(size_t)blockIdx.x * E + id] + rank;
    sorted_pairs[slot] = p;
    pair_slot[p] = slot;
  }
}

// x_perm[slot] = x[token(slot)]: routed slots from sorted_pairs, then T rows per shared expert.
__global__ void __launch_bounds__(256) gather_kernel(const float* __restrict__ x,
                                                     const int32_t* __restrict__ sorted_pairs,
                                                     int T, int k, int H, int bf16,
                                                     void* __restrict__ x_perm) {
  const int s = blockIdx.x;
  const int P = T * k;
  const int tok = s < P ? sorted_pairs[s] / k : (s - P) % T;
  const int h4 = blockIdx.y * 256 + threadIdx.x;
  if (h4 * 4 >= H) return;
  const float4 v = reinterpret_cast<const float4*>(x + (size_t)tok * H)[h4];
  if (bf16) {
    uint2 o;
    o.x = pack_bf16x2(v.x, v.y);
    o.y = pack_bf16x2(v.z, v.w);
    reinterpret_cast<uint2*>(static_cast<uint16_t*>(x_perm) + (size_t)s * H)[h4] = o;
  } else {
    reinterpret_cast<float4*>(static_cast<float*>(x_perm) + (size_t)s * H)[h4] = v;
  }
}

static int num_blocks(int P) { return (P + kPairsPerBlock - 1) / kPairsPerBlock; }

static bool use_small(const Shape& sh, int T) {
  return (int64_t)T * sh.k <= kSmallThreads && sh.E + sh.S <= kSmallThreads;
}

size_t permute_scratch_bytes(const Shape& sh, int T) {
  if (use_small(sh, T)) return 0;
  const size_t nblk = num_blocks(T * sh.k);
  return nblk * (size_t)sh.E * 4 + nblk * 4;
}

hipError_t launch_permute(const Shape& sh, int32_t* ids, float* w, int T, const float* x,
                          void* x_perm, int x_perm_bf16, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_slot, int32_t* invalid_count,
                          void* scratch, hipStream_t s) {
  const int P = T * sh.k;
  if (use_small(sh, T)) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kSmallThreads), 0, s, ids, w, T, sh.k,
                       sh.E, sh.S, offsets, sorted_pairs, pair_slot, invalid_count);
  } else {
    const int nblk = num_blocks(P);
    int32_t* counts = static_cast<int32_t*>(scratch);
    int32_t* bad = counts + (size_t)nblk * sh.E;
    hipLaunchKernelGGL(permute_count_kernel, dim3(nblk), dim3(kPairsPerBlock), sh.E * 4, s, ids,
                       w, P, sh.E, counts, bad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, counts, bad, nblk, T,
                       sh.k, sh.E, sh.S, offsets, invalid_count);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(kPairsPerBlock), 0, s, ids, P,
                       sh.E, counts, offsets, sorted_pairs, pair_slot);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || x_perm == nullptr) return e;
  const int rows = P + T * sh.S;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3(rows, (sh.H / 4 + 255) / 256), dim3(256), 0, s, x,
                     sorted_pairs, T, sh.k, sh.H, x_perm_bf16, x_perm);
  return hipGetLastError();
}

}  // namespace moe
