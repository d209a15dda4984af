// Prefill path: grouped GEMM of each expert's slot range against its IQ4_NL weights on bf16
// matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Xolotl ("DeepSeek-V4.1-Flash at 27 Tokens/s on One RTX 4090"), section "Prompts: fast, and
// exact": a prompt chunk runs each layer's experts as one batched multiply.  Red Lite "What we
// learned", section "3. Speed by release": batched matrix kernels for the experts.
//
// Tile: 256 slot rows x 256 weight rows a workgroup, eight waves side by side along the weight
// rows (each wave all 256 slot rows x 32 weight rows: 8 accumulator tiles of 32 x 32, 128
// accumulator registers a lane), two waves a SIMD so that one wave's waits for LDS, memory and
// the barrier are covered by the other's matrix instructions; K in steps of 64 (two IQ4_NL
// blocks).
//
//   activations  copied from HBM straight into LDS by the LDS-direct loads of gfx950
//                (global_load_lds_dwordx4: no registers, no LDS write instructions), one
//                instruction per 8 whole rows (coalesced), into a ring of 2 G stages (K
//                steps go in groups of G, one wait and one barrier a group; G = 2, or 4 for
//                tiles of at most 64 rows), the copies of a step spread evenly over the eight
//                waves; the 16-byte
//                chunks of a row are XOR-swizzled so that every fragment read is a
//                conflict-free ds_read_b128, and the reads run five matrix instructions
//                ahead of their use;
//   weights      never touch LDS: each lane loads whole 18-byte blocks into registers, a
//                group ahead (a ring of 2 G register slots, through a buffer resource with
//                the step's offset in a scalar register), and dequantises them there; each weight
//                row belongs to one wave, so every weight is dequantised once a workgroup and
//                is shared by its 256 slot rows.
//
// K order inside a step: the 32 x 32 x 16 instruction takes 8 consecutive k of one operand
// row per lane, from lane half h = lane / 32.  Instruction i = 0..3 of a step gives lane half
// h elements 8i .. 8i+7 of block h of the step, for A and B alike (a sum over k may take its
// terms in any order, so A and B only have to agree), so a lane dequantises one whole block of
// its weight row a step.
//
// Dequantisation, bf16(d * c[q]) with one RNE rounding of the exact fp32 product: the
// codebook is symmetric (c[q] = -c[15 - q]), so a block needs the 8 products d * c[q] for
// q = 0..7 only.  Their bf16 high and low bytes form two 8-byte tables, and one v_perm_b32
// looks up four elements at a time: magnitude index m = q ^ (q >= 8 ? 8 : 7), then the sign
// bit flipped for q >= 8.  That is 11 VALU operations per four weights plus 18 per block,
// no memory access, where a table in LDS costs bank conflicts and LDS bandwidth that the
// fragment reads need.
//
// For GATE_UP a wave's 32 weight rows are 16 gate rows (lanes c < 16 of a half) and the 16
// matching up rows (lanes c + 16), so u reaches the lane holding g by one lane swap and SwiGLU
// is applied in registers.
//
// The tile list is built on the device from `offsets` (whole tiles first, then the experts'
// last partial tiles by falling height); the grid is an upper bound on the tile count and a
// workgroup without a tile exits, so nothing depends on host-known expert loads.
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kBM = 256;                 // slot rows per tile
constexpr int kBN = 256;                 // weight rows per tile
constexpr int kKS = 64;                  // k per step (2 IQ4_NL blocks)
constexpr int kGemmThreads = 512;
constexpr int kStageBytes = kBM * kKS * 2;     // bf16 activations of one step: 32 KB
constexpr int kXcds = 8;                  // XCDs of an MI355X (each with its own L2)
constexpr int kWin = 6;                   // A-fragment reads in flight, plus one

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

static_assert(kCodebookValues[0] == -kCodebookValues[15] && kCodebookValues[1] == -kCodebookValues[14] &&
                  kCodebookValues[2] == -kCodebookValues[13] && kCodebookValues[3] == -kCodebookValues[12] &&
                  kCodebookValues[4] == -kCodebookValues[11] && kCodebookValues[5] == -kCodebookValues[10] &&
                  kCodebookValues[6] == -kCodebookValues[9] && kCodebookValues[7] == -kCodebookValues[8],
              "the byte-table dequantisation needs a symmetric codebook");

// Byte tables of one block: entry m (0..7) = bf16(d * c[7 - m]), high bytes in h, low in l.
struct BlockTab {
  uint32_t h0, h1, l0, l1;
};

__device__ __forceinline__ BlockTab block_tab(const RawBlock& r, bool odd) {
  const float d = block_scale(r, odd);
  uint32_t p[4];
#pragma unroll
  for (int m = 0; m < 8; m += 2)
    p[m >> 1] = pack_bf16x2(d * (float)kCodebookValues[7 - m], d * (float)kCodebookValues[6 - m]);
  BlockTab t;
  t.h0 = __builtin_amdgcn_perm(p[1], p[0], 0x07050301u);
  t.h1 = __builtin_amdgcn_perm(p[3], p[2], 0x07050301u);
  t.l0 = __builtin_amdgcn_perm(p[1], p[0], 0x06040200u);
  t.l1 = __builtin_amdgcn_perm(p[3], p[2], 0x06040200u);
  return t;
}

// Four weights from the low (HI = 0) or high (HI = 1) nibbles of one code dword, as two bf16
// pairs (elements 0,1 and 2,3 of the four).
template <int HI>
__device__ __forceinline__ void dequant4(uint32_t cw, const BlockTab& t, uint32_t& o0,
                                         uint32_t& o1) {
  uint32_t q, s;                               // q: four 4-bit indices as bytes
  if (HI) {                                    // s: 0x80 in the bytes whose index is >= 8
    q = (cw >> 4) & 0x0F0F0F0Fu;
    s = cw & 0x80808080u;
  } else {
    q = cw & 0x0F0F0F0Fu;
    s = (cw << 4) & 0x80808080u;
  }
  const uint32_t m = q ^ (0x07070707u + (s >> 7));           // magnitude index 0..7
  const uint32_t hb = __builtin_amdgcn_perm(t.h1, t.h0, m) ^ s;
  const uint32_t lb = __builtin_amdgcn_perm(t.l1, t.l0, m);
  o0 = __builtin_amdgcn_perm(hb, lb, 0x05010400u);
  o1 = __builtin_amdgcn_perm(hb, lb, 0x07030602u);
}

// B operand of elements 8C .. 8C+7 of a block, from the block's four code dwords.
template <int C>
__device__ __forceinline__ bf16x8_t b_frag(const uint32_t (&c)[4], const BlockTab& t) {
  u32x4_t v;
  uint32_t a0, a1, a2, a3;
  dequant4<C / 2>(c[2 * (C & 1)], t, a0, a1);
  dequant4<C / 2>(c[2 * (C & 1) + 1], t, a2, a3);
  v[0] = a0; v[1] = a1; v[2] = a2; v[3] = a3;
  return __builtin_bit_cast(bf16x8_t, v);
}

// s_waitcnt vmcnt(N): at most N vector-memory instructions of this wave are outstanding.
// Loads into registers complete in issue order; LDS-direct copies are waited for with N = 0.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}

// f(std::integral_constant<int, 0>{}) .. f(std::integral_constant<int, N - 1>{}), in order
template <int N, typename F, int... J>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// s_waitcnt lgkmcnt(N): every LDS instruction of this wave but the last N issued has completed.
// The compiler counts the activation copies into LDS as outstanding on both counters and, while
// one is in flight, turns every wait it adds itself into a full drain; a wait written here that
// already covers the dependency leaves it nothing to add.
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (N << 8));
}

// One workgroup tile: RG 32-row groups of slot rows hold rows of the tile (the rest of the
// 256 are past the expert's last slot and are neither multiplied nor stored).
template <bool GATEUP, int RG>
__device__ __forceinline__ void gemm_tile(uint8_t* lds0, uint8_t* lds1, uint8_t* lds2,
                                          uint8_t* lds3, const uint8_t* __restrict__ wmat,
                                          int64_t row_bytes, const uint16_t* __restrict__ in,
                                          int64_t row0, int rows_valid, int K, int nt,
                                          void* __restrict__ out, int H, int F) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // uniform: scalar branches
  const int c32 = lane & 31, h = lane >> 5;
  const int NKT = K / kKS;

  // the weight row of this lane: column c32 of the wave's 32 (the columns of a last, partial
  // DOWN tile past H repeat row H - 1 and are not stored)
  int wr;
  if (GATEUP) {                     // c32 < 16: gate rows; c32 >= 16: the matching up rows
    wr = nt * 128 + 16 * wave + (c32 & 15) + (c32 >= 16 ? F : 0);
  } else {
    wr = nt * kBN + 32 * wave + c32;
    if (wr >= H) wr = H - 1;
  }
  // this lane's blocks 2 kd + h through a buffer resource over the expert's matrix: block
  // 2 kd + h starts at byte 36 kd + 18 h of the row, read from the dword at 36 kd + 16 h (an
  // odd block starts 2 bytes past a dword boundary), so a step's offset is the uniform 36 kd
  // on a per-lane base (no per-step address multiply)
  const int wrows = GATEUP ? 2 * F : H;
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wmat), 0, (int)(wrows * row_bytes), 0x00020000);
  const uint32_t bvoff = (uint32_t)(wr * row_bytes) + 16u * h;

  // Activations of a step in LDS: row-major, 256 rows x 8 chunks of 16 bytes (8 k each);
  // chunk c of row r sits at position c ^ ((r >> 1) & 7): the 16 lanes that read rows
  // r0 .. r0 + 15 at one chunk cover all 64 banks once.  One copy instruction moves 8 whole
  // rows (each 128 contiguous bytes of global memory, one cache line): lane l copies chunk
  // (l & 7) ^ ((row >> 1) & 7) of row 8 n + l / 8 into position l & 7.  The tile's rows
  // holding slot rows are 4 RG groups of 8; wave w copies groups n = w + 8 s, s < RG / 2, and
  // when RG is odd one more, n = (w & 3) + 8 (RG / 2) -- waves w and w + 4 then copy the same
  // group, the same bytes to the same place.  Every wave issues the same number of copies
  // (NA), so the vector-memory counts of all waves agree and no branch surrounds a load (a
  // branch around loads makes the compiler drain every outstanding load where the paths
  // meet).  n < 4 RG: inside the stage (RG x 4 KB).  Rows past rows_valid repeat row 0.
  constexpr int NA = (RG + 1) / 2;
  const uint16_t* tile_in = in + row0 * (int64_t)K;              // uniform
  uint32_t arow[NA];                        // element offsets from tile_in (< 256 K)
  int an[NA];
#pragma unroll
  for (int s = 0; s < NA; ++s) {
    an[s] = s < RG / 2 ? wave + 8 * s : (wave & 3) + 8 * s;
    const int row = 8 * an[s] + (lane >> 3);
    arow[s] = (uint32_t)((row < rows_valid ? row : 0) * K + 8 * ((lane & 7) ^ ((row >> 1) & 7)));
  }
  // instruction i of a step: lane (c32, h) reads row 32 rg + c32, chunk 4 h + i
  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = c32 * 128 + (((4 * h + i) ^ ((c32 >> 1) & 7)) << 4);

  // K runs in groups of G steps with one wait and one barrier a group.  A tile of RG row
  // groups fills RG x 4 KB of a step's stage, so shorter tiles afford deeper rings in the same
  // 128 KB of LDS: G = 4 for one or two row groups, 2 otherwise (8-step groups for one or two
  // row groups, and 4-step groups for three or four, measured slower on the skewed loads: a
  // longer first fill and more clamped loads past the end of a short K).  The stages of a group
  // come from one half of the LDS (arrays 0 and 1 for even groups, 2 and 3 for odd ones), G
  // stages of 64 KB / G each; the four arrays are separate, so the compiler knows that the
  // fragment reads of one group do not alias the copies into the next and adds no wait of
  // its own between them.
  constexpr int G = RG > 2 ? 2 : 4;
  constexpr int SB = 2 * kStageBytes / G;            // bytes of a stage
  static_assert(RG * 4096 <= SB, "a stage holds the tile's rows of one step");
  auto stage_of = [&](auto pc, auto jc) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value, OFF = decltype(jc)::value * SB;
    if constexpr (OFF < kStageBytes) return (P ? lds2 : lds0) + OFF;
    else return (P ? lds3 : lds1) + (OFF - kStageBytes);
  };
  // copies of step kd into a stage (kd clamped to the last step: the same instructions
  // every group)
  auto dma_a = [&](int kd, uint8_t* stage) __attribute__((always_inline)) {
    kd = kd < NKT ? kd : NKT - 1;
#pragma unroll
    for (int s = 0; s < NA; ++s)          // rows 8 n .. 8 n + 7
      __builtin_amdgcn_global_load_lds(tile_in + arow[s] + kd * kKS, stage + an[s] * 1024, 16,
                                       0, 0);
  };
  // weight blocks: 2 G register slots, step kt + j of a group of parity P in slot P G + j
  RawBlock bq[2 * G];
  auto load_b = [&](int kd, RawBlock& dst) __attribute__((always_inline)) {
    kd = kd < NKT ? kd : NKT - 1;
    const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(brs, (int)bvoff, 36 * kd, 0);
    dst.w[0] = a[0]; dst.w[1] = a[1]; dst.w[2] = a[2]; dst.w[3] = a[3];
    dst.w[4] = __builtin_amdgcn_raw_buffer_load_b32(brs, (int)(bvoff + 16u), 36 * kd, 0);
  };

  f32x16_t acc[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) acc[r] = f32x16_t{};

  // A group starts with a wait until every load of this wave has completed, then a barrier:
  // every wave's copies of the group's stages are in, and every wave is done reading the
  // previous group's stages, which the copies of the next group then overwrite.  The wait is
  // a full one (vmcnt(0)): the LDS-direct copies need not complete in issue order, and a wait
  // for all but the last N loads did not order them -- a producer/consumer version whose
  // waits let later copies stay in flight read stale activations.  So a load has from its
  // issue to the start of the next group to arrive.  For G = 2 each step refills its weight
  // slot with the block 4 steps ahead as it takes it (the loads in flight at a wait were
  // issued during the group, the last one step before it); for G = 4 the whole next group's
  // weight blocks go out right after the barrier with its copies, so every load has a full
  // group of steps to arrive: a tile of one or two row groups runs ~850 cycles of
  // dequantisation a step on each SIMD and a quarter or half of that on the matrix cores,
  // which a wait one step after the last load left exposed to memory latency (3584/1024 gate/
  // up over 65 bins of 32 rows: 168 -> 132 us; 7168/384 at 8,192 tokens: gate/up 3,760 ->
  // 3,543 us, down 2,130 -> 2,014 us).  The
  // barrier carries no memory fence: a workgroup release fence makes the compiler wait for
  // every copy still in flight (vmcnt(0)), which would undo the prefetch; the explicit waits
  // order the copies, the lgkmcnt(0) this wave's LDS reads, and the memory clobber keeps the
  // compiler from moving LDS accesses across.
  constexpr bool kEarly = G > 2;
  auto step = [&](int kt, const uint8_t* stage, RawBlock& blk) __attribute__((always_inline)) {
    const BlockTab tab = block_tab(blk, h != 0);
    uint32_t code[4];
    block_codes(blk, h != 0, code);
    if constexpr (!kEarly) load_b(kt + 2 * G, blk);
    __builtin_amdgcn_sched_barrier(0);
    // Matrix instruction j of the step (j < 4 RG): group I = j / RG (k 16 I .. 16 I + 15),
    // row group r = j % RG.  Its A fragment is read kWin - 1 instructions ahead, so that
    // kWin - 1 LDS reads are in flight behind every matrix instruction instead of one read
    // waited for before each; the B fragment of group I + 1 is dequantised, one half at a
    // time, beside the first two instructions of group I.  A scheduling barrier after each
    // instruction keeps this order (left alone, the compiler issues a read and waits for it
    // before each one).
    constexpr int NJ = 4 * RG;
    bf16x8_t af[kWin];
    bf16x8_t bf[2];
    uint32_t bn[4];
    auto read_a = [&](auto jc) __attribute__((always_inline)) {
      constexpr int J = decltype(jc)::value;
      af[J % kWin] = *reinterpret_cast<const bf16x8_t*>(stage + (J % RG) * 4096 + aoff[J / RG]);
    };
    static_for<(kWin - 1 < NJ ? kWin - 1 : NJ)>([&](auto jc) { read_a(jc); });
    bf[0] = b_frag<0>(code, tab);
    __builtin_amdgcn_sched_barrier(0);
    static_for<NJ>([&](auto jc) __attribute__((always_inline)) {
      constexpr int J = decltype(jc)::value, I = J / RG, R = J % RG;
      // fragment J's read is done once at most the reads issued after it (kWin - 2 of them, or
      // to the step's end) are in flight; the read of fragment J + kWin - 1 goes out after
      wait_lgkm<(kWin - 2 < NJ - 1 - J ? kWin - 2 : NJ - 1 - J)>();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (J + kWin - 1 < NJ) read_a(std::integral_constant<int, J + kWin - 1>{});
      __builtin_amdgcn_sched_barrier(0);
      acc[R] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[J % kWin], bf[I & 1], acc[R], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (I < 3) {
        constexpr int C = I + 1;                // the next group's fragment, in two halves
        if constexpr (R == 0)
          dequant4<C / 2>(code[2 * (C & 1)], tab, bn[0], bn[1]);
        if constexpr (R == (RG > 1 ? 1 : 0)) {
          dequant4<C / 2>(code[2 * (C & 1) + 1], tab, bn[2], bn[3]);
          u32x4_t v;
          v[0] = bn[0]; v[1] = bn[1]; v[2] = bn[2]; v[3] = bn[3];
          bf[C & 1] = __builtin_bit_cast(bf16x8_t, v);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // group of steps kt .. kt + G - 1 (kt a multiple of G, parity P = (kt / G) % 2); a tail
  // group (TAIL) computes only its first nv steps -- its loads and copies still go out, clamped
  auto group = [&](int kt, auto pc, auto tc, int nv) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    constexpr bool TAIL = decltype(tc)::value;
    wait_vm<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    static_for<G>([&](auto jc) __attribute__((always_inline)) {
      dma_a(kt + G + decltype(jc)::value, stage_of(std::integral_constant<int, 1 - P>{}, jc));
    });
    if constexpr (kEarly)
      static_for<G>([&](auto jc) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        load_b(kt + G + J, bq[(1 - P) * G + J]);
      });
    __builtin_amdgcn_sched_barrier(0);
    static_for<G>([&](auto jc) __attribute__((always_inline)) {
      constexpr int J = decltype(jc)::value;
      if (!TAIL || J < nv) step(kt + J, stage_of(pc, jc), bq[P * G + J]);
    });
  };
  // prologue: the first group's weight blocks and copies (and for G = 2 the second group's
  // weight blocks)
  static_for<G>([&](auto jc) __attribute__((always_inline)) {
    load_b(decltype(jc)::value, bq[decltype(jc)::value]);
  });
  __builtin_amdgcn_sched_barrier(0);
  static_for<G>([&](auto jc) __attribute__((always_inline)) {
    dma_a(decltype(jc)::value, stage_of(std::integral_constant<int, 0>{}, jc));
  });
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!kEarly)
    static_for<G>([&](auto jc) __attribute__((always_inline)) {
      load_b(G + decltype(jc)::value, bq[G + decltype(jc)::value]);
    });
  __builtin_amdgcn_sched_barrier(0);

  // whole groups in pairs in the loop (no conditional step inside, whose paths would meet
  // with different loads outstanding), then the rest: for G = 2 one whole group (K is a
  // multiple of 128, so the step count is even), for G = 4 up to two tail groups
  constexpr std::integral_constant<int, 0> kP0{};
  constexpr std::integral_constant<int, 1> kP1{};
  constexpr std::false_type kWhole{};
  int kt = 0;
  for (; kt + 2 * G <= NKT; kt += 2 * G) {
    group(kt, kP0, kWhole, G);
    group(kt + G, kP1, kWhole, G);
  }
  const int rest = NKT - kt;
  if constexpr (kEarly) {
    if (rest > 0) group(kt, kP0, std::true_type{}, rest);
    if (rest > G) group(kt + G, kP1, std::true_type{}, rest - G);
  } else {
    if (rest > 0) group(kt, kP0, kWhole, G);
  }
  wait_vm<0>();                           // no copy may land in LDS after the tile is done

  // epilogue: lane (c32, h) holds column c32 of each 32 x 32 tile; register e is row
  // 8 (e / 4) + 4 h + e % 4.  Stores go through a buffer resource over the tile's valid rows
  // (rows past rows_valid fall past its end and are dropped, as are stores at offset kOff):
  // one 32-bit offset a store, no 64-bit address arithmetic
  constexpr uint32_t kOff = 0x80000000u;
  if (GATEUP) {
    const int col = nt * 128 + 16 * wave + (c32 & 15);
    const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint16_t*>(out) + row0 * (int64_t)F, 0, rows_valid * F * 2, 0x00020000);
    // lanes c32 >= 16 hold the up values: they store nothing
    const uint32_t vbase = c32 < 16 ? (uint32_t)(4 * h * F + col) * 2u : kOff;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float g = acc[r][e];
        const float u = __shfl_xor(g, 16, 64);         // the up value of the same output
        const float hv = silu_fast(g) * u;             // h is rounded to bf16 at once
        const uint32_t mo = (uint32_t)(32 * r + 8 * (e >> 2) + (e & 3)) * (uint32_t)F * 2u;
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pack_bf16x2(hv, 0.0f) & 0xFFFFu), hrs,
                                              (int)(vbase + mo), 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);          // one row group's values live at a time
    }
  } else {
    const int col = nt * kBN + 32 * wave + c32;
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<float*>(out) + row0 * (int64_t)H, 0, rows_valid * H * 4, 0x00020000);
    const uint32_t vbase = col < H ? (uint32_t)(4 * h * H + col) * 4u : kOff;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t mo = (uint32_t)(32 * r + 8 * (e >> 2) + (e & 3)) * (uint32_t)H * 4u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[r][e]), ors, (int)(vbase + mo),
                                              0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <bool GATEUP>
__global__ void __launch_bounds__(kGemmThreads, 1) gemm_kernel(
    const uint8_t* __restrict__ bank, int64_t stride, const int32_t* __restrict__ offsets,
    const uint16_t* __restrict__ in, void* __restrict__ out, int H, int F, int E, int S) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_a0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_a1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_a2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_a3[kStageBytes];
  __shared__ int s_pref[1024];
  __shared__ int s_bin[1024];
  __shared__ uint64_t s_part[2][kGemmThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // ---- the tile list, longest first ----
  // An expert with m slots has m / 256 whole tiles and, if m % 256 > 0, a last tile of
  // c = ceil((m % 256) / 32) row groups.  The list holds every whole tile (and every last
  // tile of 8 groups) in expert order, then the last tiles of 7 groups, of 6, .. of 1, each
  // in expert order: the workgroups are dispatched in list order, so the tiles that take
  // longest start first and the short ones fill in behind them, instead of a heavy tile
  // (the shared expert's, the last bin) starting in the last round of workgroups.  Per bin
  // two packed counters are summed over the bins in one scan: A holds the last tiles of
  // 1..5 groups (11 bits each), B the whole-tile count (bits 0..20) and the last tiles of 6
  // and 7 groups (bits 21 and 32).  s_pref[e] = whole tiles of bins 0..e; s_bin[j] = the bin
  // of the j-th last tile after the whole ones.  Against expert order: 3584/64 gate/up at
  // 2,048 tokens 285-291 -> 243-247 us, 2048/512 at 2,048 tokens 329-365 -> 310-320 us.  The
  // down GEMM keeps expert order.
  const int nbins = E + S;
  int n_whole, total_m;
  if constexpr (GATEUP) {
    uint64_t locA[4], locB[4], ownA[4], ownB[4];
    uint64_t runA = 0, runB = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      uint64_t a = 0, b = 0;
      if (e < nbins) {
        const int m = offsets[e + 1] - offsets[e];
        const int c = ((m % kBM) + 31) >> 5;                  // groups of the last tile, 0..8
        b = (uint64_t)(m / kBM + (c == 8 ? 1 : 0));
        if (c >= 1 && c <= 5) a = 1ull << (11 * (c - 1));
        else if (c == 6 || c == 7) b |= 1ull << (21 + 11 * (c - 6));
      }
      ownA[i] = a; ownB[i] = b;
      runA += a; runB += b;
      locA[i] = runA; locB[i] = runB;
    }
    uint64_t inclA = runA, inclB = runB;
    for (int d = 1; d < 64; d <<= 1) {
      const uint64_t oa = __shfl_up(inclA, d, 64), ob = __shfl_up(inclB, d, 64);
      if (lane >= d) { inclA += oa; inclB += ob; }
    }
    if (lane == 63) { s_part[0][wave] = inclA; s_part[1][wave] = inclB; }
    __syncthreads();
    uint64_t beforeA = inclA - runA, beforeB = inclB - runB, totA = 0, totB = 0;
#pragma unroll
    for (int w = 0; w < kGemmThreads / 64; ++w) {
      if (w < wave) { beforeA += s_part[0][w]; beforeB += s_part[1][w]; }
      totA += s_part[0][w]; totB += s_part[1][w];
    }
    auto count_of = [](uint64_t A, uint64_t B, int c) __attribute__((always_inline)) {
      return (int)(c <= 5 ? (A >> (11 * (c - 1))) & 0x7FF : (B >> (21 + 11 * (c - 6))) & 0x7FF);
    };
    const int n_whole_ = (int)(totB & 0x1FFFFF);
    int start[8];                          // list position of the first last tile of c groups
    start[7] = n_whole_;
#pragma unroll
    for (int c = 6; c >= 1; --c) start[c] = start[c + 1] + count_of(totA, totB, c + 1);
    const int total_m_ = start[1] + count_of(totA, totB, 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e >= nbins) continue;
      s_pref[e] = (int)((beforeB + locB[i]) & 0x1FFFFF);
      const uint64_t xa = beforeA + locA[i] - ownA[i], xb = beforeB + locB[i] - ownB[i];
#pragma unroll
      for (int c = 1; c <= 7; ++c)
        if (count_of(ownA[i], ownB[i], c))
          s_bin[start[c] - n_whole_ + count_of(xa, xb, c)] = e;
    }
    __syncthreads();

    n_whole = n_whole_;
    total_m = total_m_;
  } else {
    // expert order, every tile counted as whole: s_pref[e] = sum over e' <= e of
    // ceil(m_e' / 256) (longest first cost the down GEMM ~3% in this prologue and gained
    // nothing: its K is short and its output fp32)
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
    if (lane == 63) s_part[0][wave] = (uint64_t)incl;
    __syncthreads();
    int before = incl - run;
    for (int w = 0; w < wave; ++w) before += (int)s_part[0][w];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid * 4 + i;
      if (e < nbins) s_pref[e] = before + loc[i];
    }
    __syncthreads();
    total_m = n_whole = s_pref[nbins - 1];
  }

  const int K = GATEUP ? H : F;
  const int NT = GATEUP ? F / 128 : (H + kBN - 1) / kBN;
  // XCD-aware order: workgroup b runs on XCD b % 8 (dispatch is round-robin over the XCDs).
  // XCD x takes M tiles x, x + 8, x + 16, .. of the list and each of them with all its N
  // tiles in a row, so the workgroups that share an activation panel meet in the same L2,
  // and the heavy M tiles are spread over the XCDs instead of filling one: against
  // contiguous ranges of the tile list (in expert order), 3584/64 at 2,048 tokens gate/up
  // 308 -> 293 us and down 173 -> 161 us, 7168/384 at 8,192 tokens 569 -> 628 TFLOP/s.
  const int xcd = blockIdx.x % kXcds, idx = blockIdx.x / kXcds;
  const int mt = xcd + kXcds * (idx / NT), nt = idx % NT;
  if (mt >= total_m) return;
  int e, m0;
  if (mt < n_whole) {
    // expert owning whole tile mt: first e with s_pref[e] > mt
    int lo = 0, hi = nbins - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] > mt) hi = mid; else lo = mid + 1;
    }
    e = lo;
    m0 = (mt - (e ? s_pref[e - 1] : 0)) * kBM;
  } else {
    e = s_bin[mt - n_whole];
    m0 = ((offsets[e + 1] - offsets[e]) / kBM) * kBM;
  }
  const int64_t row0 = (int64_t)offsets[e] + m0;
  const int rows_valid = min(kBM, offsets[e + 1] - offsets[e] - m0);
  const int64_t row_bytes = (int64_t)(K >> 5) * kBlockBytes;
  const int64_t mat_off = GATEUP ? 0 : 2 * (int64_t)F * ((int64_t)(H >> 5) * kBlockBytes);
  const uint8_t* wmat = bank + (int64_t)e * stride + mat_off;
  const int rg = (rows_valid + 31) >> 5;

#define TILE(N) \
  case N: gemm_tile<GATEUP, N>(s_a0, s_a1, s_a2, s_a3, wmat, row_bytes, in, row0, rows_valid, K, nt, out, H, F); break;
  switch (rg) {
    TILE(1) TILE(2) TILE(3) TILE(4) TILE(5) TILE(6) TILE(7) TILE(8)
    default: break;
  }
#undef TILE
}

hipError_t launch_gemm(const Shape& sh, int stage, const uint8_t* bank, int64_t stride,
                       const int32_t* offsets, const void* in, void* out, int T,
                       hipStream_t s) {
  if (T == 0) return hipSuccess;
  // upper bound on the tiles: every expert with slots adds at most one partial M tile
  const int64_t rows = (int64_t)T * (sh.k + sh.S);
  const int64_t bins = std::min<int64_t>(sh.E + sh.S, rows);
  const int64_t mtiles = (rows + kBM - 1) / kBM + bins;
  const int NT = stage == 0 ? sh.F / 128 : (sh.H + kBN - 1) / kBN;
  // every XCD gets M tiles x, x + 8, .. (each with its NT N tiles)
  const int64_t grid = ((mtiles + kXcds - 1) / kXcds) * kXcds * NT;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (stage == 0)
    hipLaunchKernelGGL(gemm_kernel<true>, dim3((unsigned)grid), dim3(kGemmThreads), 0, s, bank,
                       stride, offsets, static_cast<const uint16_t*>(in), out, sh.H, sh.F, sh.E,
                       sh.S);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, dim3((unsigned)grid), dim3(kGemmThreads), 0, s,
                       bank, stride, offsets, static_cast<const uint16_t*>(in), out, sh.H, sh.F,
                       sh.E, sh.S);
  return hipGetLastError();
}

}  // namespace moe
