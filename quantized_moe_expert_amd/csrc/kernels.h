// Internal launchers of libmoe_iq4nl.so (C++ linkage, not exported).  Each enqueues its
// kernels on `stream` and returns the hipError_t of the last launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace moe {

struct Shape {
  int H, F, E, k, S, gating, renorm;
};

hipError_t launch_quantize(const float* w, int64_t n_blocks, uint8_t* out, hipStream_t s);
hipError_t launch_dequantize(const uint8_t* blk, int64_t n_blocks, float* out, hipStream_t s);

// partial: scratch for the split-K partial logits (partial_floats floats; NULL: no split)
hipError_t launch_route(const Shape& sh, const float* x, const float* wr, const float* bias,
                        int T, int32_t* ids, float* w, float* logits, float* partial,
                        size_t partial_floats, hipStream_t s);
int route_splits(const Shape& sh, int T, size_t cap_floats);
hipError_t launch_topk(const Shape& sh, const float* logits, int T, int32_t* ids, float* w,
                       hipStream_t s);

// scratch: workspace region for the permutation (size from permute_scratch_bytes)
size_t permute_scratch_bytes(const Shape& sh, int T);
hipError_t launch_permute(const Shape& sh, int32_t* ids, float* w, int T, const float* x,
                          void* x_perm, int x_perm_bf16, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_slot, int32_t* invalid_count,
                          void* scratch, hipStream_t s);

hipError_t launch_gemv(const Shape& sh, int stage, const uint8_t* bank, int64_t stride,
                       const int32_t* offsets, const int32_t* sorted_pairs, const float* in,
                       float* out, int T, hipStream_t s);

hipError_t launch_gemm(const Shape& sh, int stage, const uint8_t* bank, int64_t stride,
                       const int32_t* offsets, const void* in, void* out, int T,
                       hipStream_t s);

hipError_t launch_combine(const Shape& sh, const float* o, const int32_t* pair_slot,
                          const float* w, int T, const float* residual, float* y,
                          hipStream_t s);

hipError_t launch_rmsnorm(const float* x, int T, int H, float eps, float* y, hipStream_t s);

// Intermediates of the fused decode layer (device pointers inside the caller's workspace).
struct DecodeScratch {
  float* logits;          // [T, E]
  float* rscale;          // [T]
  int32_t* ids;           // [T, k]
  float* w;               // [T, k]
  int32_t* offsets;       // [E + S + 1]
  int32_t* sorted_pairs;  // [T * k]
  int32_t* pair_slot;     // [T * k]
  float* h;               // [rows, F]
  float* xn;              // [T, H]: the batched kernels' pre-split input rows
  float* o;               // [rows, H]: the batched down's slot outputs
  int32_t* done;          // [H / 128]: the batched down's counters (zero between launches)
  int32_t* count;         // sanitised-pair count of the permutation
};

constexpr int kDecodeMaxTokens = 16;
// Up to this many tokens a decode layer runs the dequant-GEMV kernels of decode.hip; above it
// the batched kernels of bdecode.hip (matrix cores).  Both take three launches a layer.
constexpr int kDecodeFusedMaxT = 4;
// logits (and, with eps >= 0, the RMSNorm scale of each row into rscale and the normalised
// rows into xn, where those are non-null; with xhl non-null, the rows times their scale as
// bf16 (hi, lo) pairs in code-byte order) for T <= 16 rows
hipError_t launch_router_rows(const Shape& sh, const float* x, const float* wr,
                              const float* bias, int T, float eps, float* logits,
                              float* rscale, hipStream_t s, float* xn = nullptr,
                              uint32_t* xhl = nullptr);
// The batched decode layer (bdecode.hip): sc.xn holds the pre-split input rows and sc.h the
// pre-split h rows in pair order; no o buffer.
bool bdecode_supported(const Shape& sh, int T);
hipError_t launch_bdecode_layer(const Shape& sh, const uint8_t* bank, int64_t stride,
                                const float* wr, const float* bias, const float* x, int T,
                                float eps, const float* residual, float* y, DecodeScratch sc,
                                int stages, hipStream_t s);
bool decode_down_fused_fits(const Shape& sh, int T);
hipError_t launch_decode_layer(const Shape& sh, const uint8_t* bank, int64_t stride,
                               const float* wr, const float* bias, const float* x, int T,
                               float eps, const float* residual, float* y, DecodeScratch sc,
                               int stages, hipStream_t s);

int device_cu_count();

}  // namespace moe
