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

hipError_t launch_route(const Shape& sh, const float* x, const float* wr, const float* bias,
                        int T, int32_t* ids, float* w, float* logits, hipStream_t s);

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

int device_cu_count();

}  // namespace moe
