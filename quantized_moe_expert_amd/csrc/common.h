// Device-side building blocks shared by the kernels of libmoe_iq4nl.so (gfx950).
//
// IQ4_NL block (PocketLLM "Xing4.0-29B-A4B", section "Overview": 4.5 bits a weight, 32
// weights in 18 bytes): fp16 scale d in bytes 0-1, then 16 bytes whose low nibbles are
// indices q_0..q_15 and high nibbles q_16..q_31; weight i = d * c[q_i].
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace moe {

constexpr int kBlock = 32;        // weights per block
constexpr int kBlockBytes = 18;   // bytes per block

// The 16-entry signed int8 non-linear codebook (16-level Lloyd-Max levels of a unit normal,
// scaled to a largest magnitude of 127).
constexpr int8_t kCodebookValues[16] = {
    -127, -96, -75, -58, -44, -31, -18, -6, 6, 18, 31, 44, 58, 75, 96, 127};

constexpr uint64_t codebook_bytes(int first) {
  uint64_t r = 0;
  for (int i = 0; i < 8; ++i) r |= (uint64_t)(uint8_t)kCodebookValues[first + i] << (8 * i);
  return r;
}

// Codebook value q (0..15) without a memory read: the 16 bytes live in two 64-bit literals.
// (A table in memory would be a load, and a wave's loads complete in issue order: waiting
// for it would also wait for every load issued before it.)
__device__ __forceinline__ int codebook_at(int q) {
  constexpr uint64_t lo = codebook_bytes(0), hi = codebook_bytes(8);
  const uint64_t v = (q & 8) ? hi : lo;
  return (int)(int8_t)(uint8_t)(v >> (8 * (q & 7)));
}

// bf16 bit pattern of a small integer (exact: |v| <= 127 needs 7 significant bits).
__device__ __forceinline__ uint32_t bf16_bits_of_int(int v) {
  return __float_as_uint((float)v) >> 16;
}

// Byte table: entry b = (bf16(c[b & 15]) | bf16(c[b >> 4]) << 16), i.e. one code byte of a
// block (indices q_j low, q_{j+16} high) to the bf16 pair of its two codebook values.
__device__ __forceinline__ uint32_t pair_table_entry(int b) {
  return bf16_bits_of_int(codebook_at(b & 15)) | (bf16_bits_of_int(codebook_at(b >> 4)) << 16);
}

// The 18 bytes of block number `blk` of a row that starts 4-byte aligned, read as five
// aligned dwords starting at the block's start rounded down to 4 bytes.  Blocks with an even
// index start aligned; odd ones start 2 bytes past a dword boundary.  All five dwords stay
// inside the row when the row holds an even number of blocks.
struct RawBlock {
  uint32_t w[5];
};

__device__ __forceinline__ RawBlock load_block(const uint8_t* row, int blk) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row + blk * kBlockBytes - (blk & 1) * 2);
  RawBlock r;
  // dwords 0-3 and 4 (the compiler forms wide loads; dword alignment suffices on gfx950)
  r.w[0] = __builtin_nontemporal_load(p + 0);
  r.w[1] = __builtin_nontemporal_load(p + 1);
  r.w[2] = __builtin_nontemporal_load(p + 2);
  r.w[3] = __builtin_nontemporal_load(p + 3);
  r.w[4] = __builtin_nontemporal_load(p + 4);
  return r;
}

// Scale d (fp16 -> fp32) and the 16 code bytes realigned into 4 dwords.
// odd: the block index parity (odd blocks sit 2 bytes into dword 0).
__device__ __forceinline__ float block_scale(const RawBlock& r, bool odd) {
  uint32_t bits = odd ? (r.w[0] >> 16) : (r.w[0] & 0xFFFFu);
  return __half2float(__ushort_as_half((unsigned short)bits));
}

__device__ __forceinline__ void block_codes(const RawBlock& r, bool odd, uint32_t c[4]) {
  // v_perm_b32(hi, lo, sel): byte k of the result = byte sel_k of {hi:lo}.
  const uint32_t sel = odd ? 0x07060504u : 0x05040302u;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_perm(r.w[i + 1], r.w[i], sel);
}

// fp32 -> (bf16 hi, bf16 lo) split of a pair: hi = RNE(x), lo = RNE(x - hi).
// hi + lo carries 16 significant bits of x (relative error <= 2^-17).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  const float ah = __uint_as_float(hi << 16);
  const float bh = __uint_as_float(hi & 0xFFFF0000u);
  lo = pack_bf16x2(a - ah, b - bh);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// silu from the hardware base-2 exponential and reciprocal (a few ulp of fp32): for results
// rounded to bf16 right after, where the library exp and the IEEE division cost five times
// the instructions.  e^-g = 2^(-g log2 e); overflow gives 1/inf = 0, so g -> -inf gives -0.
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64); every lane of
// the group ends with the group sum.  Fixed butterfly order: deterministic.
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// DPP lane moves (data-parallel primitives: no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                            0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // row_mirror: lane i <-> 15 - i within 16

// Sum over groups of W consecutive lanes (W a power of two, 2..64), fixed order.  Within a
// row of 16 lanes a DPP butterfly; across rows, s_readlane of the row sums.  The result is
// valid in every lane of the group.
template <int W>
__device__ __forceinline__ float group_sum_dpp(float v) {
  static_assert(W >= 2 && W <= 64 && (W & (W - 1)) == 0, "group width");
  v += dpp_f<kDppXor1>(v);
  if constexpr (W >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (W >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (W >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (W == 32) {
    const int lane = threadIdx.x & 63;
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    v = lane < 32 ? a + b : c + d;
  } else if constexpr (W == 64) {
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    v = (a + b) + (c + d);
  }
  return v;
}

// Workgroup barrier that orders LDS accesses only: global loads stay in flight across it
// (__syncthreads() also waits for every outstanding global access of the wave).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int group_sum_int(int v, int width) {
  for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace moe
