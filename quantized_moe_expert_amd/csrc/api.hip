// C-ABI entry points of libmoe_iq4nl.so: host-side checks, workspace layout, launches on the
// caller's stream.  Declarations and contracts: include/moe_iq4nl.h.
#include <algorithm>
#include <mutex>

#include "../../include/moe_iq4nl.h"
#include "kernels.h"

namespace moe {

static thread_local int32_t g_last_hip_error = 0;

// Device scratch of moe_decode_layer_noalloc: one array per GPU, resident until the process
// ends.  Host code never passes the array's name to a kernel (on the host it is a stand-in,
// not a device address); it uses the address hipGetSymbolAddress returns for each device.
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// Address of this device's scratch array (looked up once per device, with it current).
static hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

int device_cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace moe

using moe::Shape;

namespace {

// Workspace: bytes 0..3 the sanitised-pair count of moe_permute, then (from byte 256)
// scratch.
constexpr size_t kHeaderBytes = 256;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  moe::g_last_hip_error = (int32_t)e;
  return MOE_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

moe_status check_desc(const moe_desc* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->hidden < 64 || d->hidden > 8192 || d->hidden % 64) return MOE_ERR_SHAPE;
  if (d->ffn < 64 || d->ffn > 8192 || d->ffn % 64) return MOE_ERR_SHAPE;
  if (d->n_shared < 0 || d->n_shared > 1) return MOE_ERR_SHAPE;
  if (d->n_experts < 1 || d->n_experts + d->n_shared > 1024) return MOE_ERR_SHAPE;
  if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > 32) return MOE_ERR_SHAPE;
  if (d->gating != MOE_GATING_SIGMOID && d->gating != MOE_GATING_SOFTMAX)
    return MOE_ERR_UNSUPPORTED;
  if (d->renormalize != 0 && d->renormalize != 1) return MOE_ERR_UNSUPPORTED;
  if (d->max_tokens < 1) return MOE_ERR_SHAPE;
  return MOE_OK;
}

moe_status check_tokens(const moe_desc* d, int32_t T) {
  if (T < 0 || T > d->max_tokens) return MOE_ERR_SHAPE;
  // every slot index and row offset must fit int32 arithmetic on the device
  if ((int64_t)T * (d->top_k + d->n_shared) > (int64_t)1 << 30) return MOE_ERR_SHAPE;
  return MOE_OK;
}

Shape shape_of(const moe_desc* d) {
  return Shape{d->hidden, d->ffn, d->n_experts, d->top_k, d->n_shared, d->gating,
               d->renormalize};
}

size_t logits_bytes(const moe_desc* d, int32_t T) { return align256((size_t)T * d->n_experts * 4); }

// Fused decode layer: header | logits | rscale | ids | w | offsets | sorted_pairs | pair_slot |
// h | xn | o | done.  For the batched kernels (above kDecodeFusedMaxT tokens, or when the down stage's
// LDS cannot hold every slot's h) xn and h hold bf16 (hi, lo) pair rows: the same bytes as
// fp32 rows.
struct DecodeLayout {
  size_t logits, rscale, ids, w, offsets, sp, ps, h, xn, o, done, total;
};

DecodeLayout decode_layout(const moe_desc* d, int32_t T) {
  const size_t P = (size_t)T * d->top_k;
  const size_t rows = P + (size_t)T * d->n_shared;
  DecodeLayout L;
  size_t off = kHeaderBytes;
  L.logits = off; off += align256((size_t)T * d->n_experts * 4);
  L.rscale = off; off += align256((size_t)T * 4);
  L.ids = off; off += align256(P * 4);
  L.w = off; off += align256(P * 4);
  L.offsets = off; off += align256((size_t)(d->n_experts + d->n_shared + 1) * 4);
  L.sp = off; off += align256(P * 4);
  L.ps = off; off += align256(P * 4);
  L.h = off; off += align256(rows * d->ffn * 4);
  L.xn = off; off += align256((size_t)T * d->hidden * 4);
  L.o = off; off += align256(rows * d->hidden * 4);
  L.done = off; off += align256((size_t)(d->hidden / 128 + 1) * 4);
  L.total = off;
  return L;
}

size_t ws_bytes_for(const moe_desc* d, int32_t T) {
  const size_t route_part = (size_t)moe::route_splits(shape_of(d), T, ~size_t(0)) * T *
                           d->n_experts * 4;
  size_t b = kHeaderBytes + logits_bytes(d, T) +
             align256(std::max(moe::permute_scratch_bytes(shape_of(d), T), route_part));
  if (T <= moe::kDecodeMaxTokens) b = std::max(b, decode_layout(d, T).total);
  return b;
}

moe_status check_bank(const moe_desc* d, const moe_bank* bank) {
  if (!bank || !bank->base) return MOE_ERR_NULL;
  const int64_t esz = 2 * (int64_t)d->ffn * (d->hidden / 32) * 18 +
                      (int64_t)d->hidden * (d->ffn / 32) * 18;
  if (bank->expert_stride < esz) return MOE_ERR_SHAPE;
  if (!aligned(bank->base, 16) || bank->expert_stride % 16) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int32_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or not a supported multiple";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_size() reported";
    case MOE_ERR_UNSUPPORTED: return "unsupported enum value or feature";
    case MOE_ERR_HIP: return "a HIP launch failed (see moe_last_hip_error)";
    case MOE_ERR_ALIGNMENT: return "a pointer or stride violates the alignment contract";
    case MOE_ERR_SCRATCH_LIMIT:
      return "the call needs more scratch than the fixed device array of the allocation-free "
             "entry point holds (MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int32_t moe_last_hip_error(void) { return moe::g_last_hip_error; }

moe_status moe_workspace_size(const moe_desc* desc, int32_t n_tokens, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (n_tokens < 0) return MOE_ERR_SHAPE;
  *bytes = ws_bytes_for(desc, n_tokens);
  return MOE_OK;
}

moe_status moe_quantize_iq4nl(const float* w, int64_t n_blocks, uint8_t* out,
                              hipStream_t stream) {
  if (n_blocks < 0) return MOE_ERR_SHAPE;
  if (n_blocks == 0) return MOE_OK;
  if (!w || !out) return MOE_ERR_NULL;
  if (!aligned(w, 16) || !aligned(out, 2)) return MOE_ERR_ALIGNMENT;
  if (n_blocks > ((int64_t)1 << 40)) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_quantize(w, n_blocks, out, stream));
}

moe_status moe_dequantize_iq4nl(const uint8_t* blocks, int64_t n_blocks, float* out,
                                hipStream_t stream) {
  if (n_blocks < 0) return MOE_ERR_SHAPE;
  if (n_blocks == 0) return MOE_OK;
  if (!blocks || !out) return MOE_ERR_NULL;
  if (!aligned(blocks, 2) || !aligned(out, 16)) return MOE_ERR_ALIGNMENT;
  if (n_blocks > ((int64_t)1 << 40)) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_dequantize(blocks, n_blocks, out, stream));
}

moe_status moe_route(const moe_desc* desc, const float* x, const float* w_router,
                     const float* bias, int32_t n_tokens, int32_t* topk_ids, float* topk_w,
                     float* logits, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(desc, n_tokens)) != MOE_OK) return st;
  if (n_tokens == 0) return MOE_OK;
  if (!x || !w_router || !topk_ids || !topk_w) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_router, 16)) return MOE_ERR_ALIGNMENT;
  if (!logits) {
    if (!ws) return MOE_ERR_NULL;
    if (ws_bytes < kHeaderBytes + logits_bytes(desc, n_tokens)) return MOE_ERR_WORKSPACE;
    logits = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kHeaderBytes);
  }
  // split-K partial logits in the workspace after the logits, when it has room (else no split)
  float* partial = nullptr;
  size_t partial_floats = 0;
  const size_t base = kHeaderBytes + logits_bytes(desc, n_tokens);
  if (ws && aligned(ws, 256) && ws_bytes > base) {
    partial = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + base);
    partial_floats = (ws_bytes - base) / 4;
  }
  return hip_status(moe::launch_route(shape_of(desc), x, w_router, bias, n_tokens, topk_ids,
                                      topk_w, logits, partial, partial_floats, stream));
}

moe_status moe_permute(const moe_desc* desc, int32_t* topk_ids, float* topk_w,
                       int32_t n_tokens, const float* x, void* x_perm, int32_t x_perm_dtype,
                       int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_slot, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(desc, n_tokens)) != MOE_OK) return st;
  if (!offsets || !ws) return MOE_ERR_NULL;
  if (n_tokens > 0 && (!topk_ids || !topk_w || !sorted_pairs || !pair_slot)) return MOE_ERR_NULL;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_NULL;
  if (x_perm && x_perm_dtype != MOE_DTYPE_F32 && x_perm_dtype != MOE_DTYPE_BF16)
    return MOE_ERR_UNSUPPORTED;
  if (x && (!aligned(x, 16) || !aligned(x_perm, 16))) return MOE_ERR_ALIGNMENT;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  if (ws_bytes < ws_bytes_for(desc, n_tokens)) return MOE_ERR_WORKSPACE;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  int32_t* invalid = reinterpret_cast<int32_t*>(w8);
  void* scratch = w8 + kHeaderBytes + logits_bytes(desc, n_tokens);
  return hip_status(moe::launch_permute(shape_of(desc), topk_ids, topk_w, n_tokens, x, x_perm,
                                        x_perm_dtype == MOE_DTYPE_BF16, offsets, sorted_pairs,
                                        pair_slot, invalid, scratch, stream));
}

moe_status moe_expert_gemv_iq4nl(const moe_desc* desc, int32_t stage, const moe_bank* bank,
                                 const int32_t* offsets, const int32_t* sorted_pairs,
                                 const float* in, float* out, int32_t n_tokens, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(desc, n_tokens)) != MOE_OK) return st;
  if (stage != MOE_STAGE_GATE_UP && stage != MOE_STAGE_DOWN) return MOE_ERR_UNSUPPORTED;
  if ((st = check_bank(desc, bank)) != MOE_OK) return st;
  if (n_tokens == 0) return MOE_OK;
  if (!offsets || !in || !out) return MOE_ERR_NULL;
  if (stage == MOE_STAGE_GATE_UP && !sorted_pairs) return MOE_ERR_NULL;
  if (!aligned(in, 16) || !aligned(out, 4)) return MOE_ERR_ALIGNMENT;
  return hip_status(moe::launch_gemv(shape_of(desc), stage, bank->base, bank->expert_stride,
                                     offsets, sorted_pairs, in, out, n_tokens, stream));
}

moe_status moe_grouped_gemm_iq4nl(const moe_desc* desc, int32_t stage, const moe_bank* bank,
                                  const int32_t* offsets, const void* in_bf16, void* out,
                                  int32_t n_tokens, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(desc, n_tokens)) != MOE_OK) return st;
  if (stage != MOE_STAGE_GATE_UP && stage != MOE_STAGE_DOWN) return MOE_ERR_UNSUPPORTED;
  if ((st = check_bank(desc, bank)) != MOE_OK) return st;
  // tiles: K in steps of 128, DOWN output columns in tiles of 128
  if (desc->hidden % 128 || desc->ffn % 128) return MOE_ERR_SHAPE;
  if (n_tokens == 0) return MOE_OK;
  if (!offsets || !in_bf16 || !out) return MOE_ERR_NULL;
  if (!aligned(in_bf16, 16) || !aligned(out, 4)) return MOE_ERR_ALIGNMENT;
  return hip_status(moe::launch_gemm(shape_of(desc), stage, bank->base, bank->expert_stride,
                                     offsets, in_bf16, out, n_tokens, stream));
}

moe_status moe_combine(const moe_desc* desc, const float* o, const int32_t* pair_slot,
                       const float* topk_w, int32_t n_tokens, const float* residual, float* y,
                       hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(desc, n_tokens)) != MOE_OK) return st;
  if (n_tokens == 0) return MOE_OK;
  if (!o || !pair_slot || !topk_w || !y) return MOE_ERR_NULL;
  if (!aligned(o, 16) || !aligned(y, 16) || (residual && !aligned(residual, 16)))
    return MOE_ERR_ALIGNMENT;
  return hip_status(moe::launch_combine(shape_of(desc), o, pair_slot, topk_w, n_tokens,
                                        residual, y, stream));
}

}  // extern "C"

namespace {

// Checks shared by the two fused decode-layer entry points (everything but the workspace).
moe_status check_decode_layer(const moe_desc* desc, const moe_bank* bank, const float* w_router,
                              const float* x, int32_t n_tokens, float norm_eps,
                              const float* residual, float* y, int32_t stages) {
  moe_status st = check_desc(desc);
  if (stages < 1 || stages > MOE_DECODE_ALL) return MOE_ERR_UNSUPPORTED;
  if (st != MOE_OK) return st;
  if ((st = check_tokens(desc, n_tokens)) != MOE_OK) return st;
  if (n_tokens > moe::kDecodeMaxTokens) return MOE_ERR_SHAPE;
  if ((st = check_bank(desc, bank)) != MOE_OK) return st;
  if (n_tokens == 0) return MOE_OK;
  if (!w_router || !x || !y) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(y, 16) ||
      (residual && !aligned(residual, 16)))
    return MOE_ERR_ALIGNMENT;
  if (norm_eps != norm_eps) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// The fused decode layer's launches with the workspace at ws (layout decode_layout).
moe_status run_decode_layer(const moe_desc* desc, const moe_bank* bank, const float* w_router,
                            const float* bias, const float* x, int32_t n_tokens, float norm_eps,
                            const float* residual, float* y, int32_t* topk_ids, float* topk_w,
                            int32_t stages, void* ws, hipStream_t stream) {
  const DecodeLayout L = decode_layout(desc, n_tokens);
  uint8_t* b = static_cast<uint8_t*>(ws);
  moe::DecodeScratch sc;
  sc.logits = reinterpret_cast<float*>(b + L.logits);
  sc.rscale = reinterpret_cast<float*>(b + L.rscale);
  sc.ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(b + L.ids);
  sc.w = topk_w ? topk_w : reinterpret_cast<float*>(b + L.w);
  sc.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  sc.sorted_pairs = reinterpret_cast<int32_t*>(b + L.sp);
  sc.pair_slot = reinterpret_cast<int32_t*>(b + L.ps);
  sc.h = reinterpret_cast<float*>(b + L.h);
  sc.xn = reinterpret_cast<float*>(b + L.xn);
  sc.o = reinterpret_cast<float*>(b + L.o);
  sc.done = reinterpret_cast<int32_t*>(b + L.done);
  sc.count = reinterpret_cast<int32_t*>(b);
  return hip_status(moe::launch_decode_layer(shape_of(desc), bank->base, bank->expert_stride,
                                             w_router, bias, x, n_tokens, norm_eps, residual, y,
                                             sc, stages, stream));
}

}  // namespace

extern "C" {

moe_status moe_decode_layer(const moe_desc* desc, const moe_bank* bank, const float* w_router,
                            const float* bias, const float* x, int32_t n_tokens, float norm_eps,
                            const float* residual, float* y, int32_t* topk_ids, float* topk_w,
                            int32_t stages, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_decode_layer(desc, bank, w_router, x, n_tokens, norm_eps, residual, y,
                                     stages);
  if (st != MOE_OK || n_tokens == 0) return st;
  if (!ws) return MOE_ERR_NULL;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  if (ws_bytes < decode_layout(desc, n_tokens).total) return MOE_ERR_WORKSPACE;
  return run_decode_layer(desc, bank, w_router, bias, x, n_tokens, norm_eps, residual, y,
                          topk_ids, topk_w, stages, ws, stream);
}

moe_status moe_decode_layer_noalloc(const moe_desc* desc, const moe_bank* bank,
                                    const float* w_router, const float* bias, const float* x,
                                    int32_t n_tokens, float norm_eps, const float* residual,
                                    float* y, int32_t* topk_ids, float* topk_w, int32_t stages,
                                    hipStream_t stream) {
  moe_status st = check_decode_layer(desc, bank, w_router, x, n_tokens, norm_eps, residual, y,
                                     stages);
  if (st != MOE_OK || n_tokens == 0) return st;
  if (decode_layout(desc, n_tokens).total > moe::kNoAllocScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const hipError_t e = moe::scratch_address(&ws);
  if (e != hipSuccess) return hip_status(e);
  return run_decode_layer(desc, bank, w_router, bias, x, n_tokens, norm_eps, residual, y,
                          topk_ids, topk_w, stages, ws, stream);
}

moe_status moe_decode_chain(const moe_desc* desc, const moe_layer* layers, int32_t n_layers,
                            float* x, int32_t n_tokens, float norm_eps, int32_t* topk_ids,
                            float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(desc, n_tokens)) != MOE_OK) return st;
  if (n_tokens > moe::kDecodeMaxTokens) return MOE_ERR_SHAPE;
  if (n_layers < 0 || n_layers > MOE_CHAIN_MAX_LAYERS) return MOE_ERR_SHAPE;
  if (n_layers > 0 && !layers) return MOE_ERR_NULL;
  for (int32_t l = 0; l < n_layers; ++l) {
    if ((st = check_bank(desc, &layers[l].bank)) != MOE_OK) return st;
    if (!layers[l].w_router) return MOE_ERR_NULL;
    if (!aligned(layers[l].w_router, 16)) return MOE_ERR_ALIGNMENT;
  }
  if (n_tokens == 0 || n_layers == 0) return MOE_OK;
  if (!x || !ws) return MOE_ERR_NULL;
  if ((topk_ids == nullptr) != (topk_w == nullptr)) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  if (norm_eps != norm_eps) return MOE_ERR_SHAPE;
  if (ws_bytes < ws_bytes_for(desc, n_tokens)) return MOE_ERR_WORKSPACE;
  const Shape sh = shape_of(desc);
  uint8_t* b = static_cast<uint8_t*>(ws);
  const size_t P = (size_t)n_tokens * desc->top_k;
  // every layer through the fused decode layer, the route table kept on the device
  const DecodeLayout L = decode_layout(desc, n_tokens);
  moe::DecodeScratch sc;
  sc.logits = reinterpret_cast<float*>(b + L.logits);
  sc.rscale = reinterpret_cast<float*>(b + L.rscale);
  sc.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  sc.sorted_pairs = reinterpret_cast<int32_t*>(b + L.sp);
  sc.pair_slot = reinterpret_cast<int32_t*>(b + L.ps);
  sc.h = reinterpret_cast<float*>(b + L.h);
  sc.xn = reinterpret_cast<float*>(b + L.xn);
  sc.o = reinterpret_cast<float*>(b + L.o);
  sc.done = reinterpret_cast<int32_t*>(b + L.done);
  sc.count = reinterpret_cast<int32_t*>(b);
  for (int32_t l = 0; l < n_layers; ++l) {
    sc.ids = topk_ids ? topk_ids + l * P : reinterpret_cast<int32_t*>(b + L.ids);
    sc.w = topk_w ? topk_w + l * P : reinterpret_cast<float*>(b + L.w);
    const moe_status s2 = hip_status(moe::launch_decode_layer(
        sh, layers[l].bank.base, layers[l].bank.expert_stride, layers[l].w_router,
        layers[l].bias, x, n_tokens, norm_eps, x, x, sc, MOE_DECODE_ALL, stream));
    if (s2 != MOE_OK) return s2;
  }
  return MOE_OK;
}

moe_status moe_rmsnorm(const float* x, int32_t n_tokens, int32_t hidden, float eps, float* y,
                       hipStream_t stream) {
  if (n_tokens < 0 || hidden <= 0 || hidden % 4) return MOE_ERR_SHAPE;
  if (!(eps >= 0.0f)) return MOE_ERR_SHAPE;
  if (n_tokens == 0) return MOE_OK;
  if (!x || !y) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16)) return MOE_ERR_ALIGNMENT;
  return hip_status(moe::launch_rmsnorm(x, n_tokens, hidden, eps, y, stream));
}

}  // extern "C"
