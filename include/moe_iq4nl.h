/*
 * moe_iq4nl.h -- C-ABI of libmoe_iq4nl.so: the routed mixture-of-experts FFN layer with
 * IQ4_NL-quantised SwiGLU experts on AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages describe it:
 *   - PocketLLM "Xing4.0-29B-A4B", section "Overview": a sigmoid-routed MoE with a shared
 *     expert (64 routed experts activated top-4 plus 1 shared, expert_ffn 1,024, hidden
 *     3,584); every expert resident on the card, indexed by expert; IQ4_NL experts, 4.5 bits
 *     a weight, 32 weights in 18 bytes.  Section "Without a server": a grouped MoE kernel
 *     over a route table.  Section "Where the detail is": deterministic route reduction.
 *   - Red Lite "What we learned", section "1. The idea": 512 experts, a token uses 10.
 *   - "DeepSeek-V4.1-Flash at 27 Tokens/s on One RTX 4090", section "Why build an engine at
 *     all": the router picks 6 of 384 experts; section "Prompts: fast, and exact": prompt
 *     chunks run each layer's experts as one batched multiply.
 *   - "Running Qwen Flash-Next NVFP4 in vLLM": route validation (an invalid expert id is
 *     redirected to expert 0 with routing weight 0) and caller-owned workspaces reused by
 *     layers that run one after another in stream order.
 *
 * Conventions for every entry point
 *   - Every pointer argument is DEVICE memory owned by the caller, except the descriptor
 *     and bank structs and `bytes` out-parameters, which are host memory read or written
 *     during the call only.
 *   - The library never allocates, frees, synchronises or copies device to host.  All work
 *     is enqueued on the given HIP stream (NULL = the default stream) and completes in
 *     stream order; inputs must stay valid until it does.
 *   - Return MOE_OK after enqueuing.  Any other status is returned from host-side checks
 *     BEFORE anything is enqueued, except MOE_ERR_HIP (a launch failed; nothing after the
 *     failing launch was enqueued; moe_last_hip_error() gives the HIP code).
 *   - Calls are reentrant and stateless; two calls may share a workspace only if they are
 *     ordered on one stream.
 *
 * IQ4_NL block (18 bytes, 32 weights): bytes 0-1 the fp16 scale d (little-endian); byte
 * 2+j (j < 16) holds index q_j in its low nibble and q_{j+16} in its high nibble; weight
 * i = d * c[q_i] with c the fixed 16-entry signed int8 codebook
 * {-127,-96,-75,-58,-44,-31,-18,-6,6,18,31,44,58,75,96,127} (16-level Lloyd-Max levels of a
 * unit normal, scaled to 127).  A weight matrix W [N rows, K cols] is stored row-major as
 * N * K/32 consecutive blocks, blocks along K.
 *
 * Expert bank (one buffer per layer): expert e (0 <= e < E routed; e == E the shared
 * expert) starts at base + e * expert_stride and holds W_gate [F, H], then W_up [F, H],
 * then W_down [H, F], each as above.  base must be 16-byte aligned, expert_stride a
 * multiple of 16 and >= the expert's size; H and F multiples of 64.
 *
 * Slots: the route pairs (t, j), pair id p = t*k + j, are grouped by expert.  offsets[e] ..
 * offsets[e+1]-1 are the slots of routed expert e (pairs in ascending p), and the shared
 * expert's slots follow: slot T*k + t is token t's shared row.  rows = T*k + T*S.
 */
#ifndef MOE_IQ4NL_H
#define MOE_IQ4NL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,          /* a required pointer is NULL                              */
    MOE_ERR_SHAPE = 2,         /* a size is out of range or not a supported multiple      */
    MOE_ERR_WORKSPACE = 3,     /* workspace smaller than moe_workspace_size() reported    */
    MOE_ERR_UNSUPPORTED = 4,   /* an enum value or feature the library does not support   */
    MOE_ERR_HIP = 5,           /* a HIP launch failed                                     */
    MOE_ERR_ALIGNMENT = 6,     /* a pointer or stride violates the alignment contract     */
    MOE_ERR_SCRATCH_LIMIT = 7  /* more scratch than moe_decode_layer_noalloc's array holds */
} moe_status;

typedef enum { MOE_GATING_SIGMOID = 0, MOE_GATING_SOFTMAX = 1 } moe_gating;
typedef enum { MOE_STAGE_GATE_UP = 0, MOE_STAGE_DOWN = 1 } moe_stage;
typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;

/* Layer descriptor (host memory). */
typedef struct moe_desc {
    int32_t hidden;        /* H, multiple of 64 (of 128 for the grouped GEMM), <= 8192  */
    int32_t ffn;           /* F, expert FFN width, same rules as hidden                 */
    int32_t n_experts;     /* E routed experts, E + n_shared <= 1024                    */
    int32_t top_k;         /* k, 1 .. min(E, 32)                                        */
    int32_t n_shared;      /* S, 0 or 1 shared expert (weight 1, not routed)            */
    int32_t gating;        /* moe_gating                                                */
    int32_t renormalize;   /* 1: selected weights are divided by their sum              */
    int32_t max_tokens;    /* T upper bound for workspace sizing and checks, >= 1       */
} moe_desc;

/* Expert bank of one layer (host struct; base is device memory). */
typedef struct moe_bank {
    const uint8_t *base;
    int64_t expert_stride;  /* bytes between consecutive experts                         */
} moe_bank;

/* ABI version of the loaded library (MOE_ABI_VERSION). */
int32_t moe_abi_version(void);

/* Static text for a status code; never NULL. */
const char *moe_status_string(int32_t status);

/* HIP error code of the most recent MOE_ERR_HIP on the calling thread (0 if none). */
int32_t moe_last_hip_error(void);

/* Bytes of the workspace that moe_route, moe_permute, moe_expert_gemv_iq4nl,
 * moe_grouped_gemm_iq4nl, moe_decode_layer and moe_decode_chain need for n_tokens tokens of
 * this layer shape (one size covers all calls).  Workspace layout:
 *   bytes 0..3   after moe_permute, the number of route pairs it sanitised (int32)
 *   bytes 256..  scratch (contents are not preserved between calls) */
moe_status moe_workspace_size(const moe_desc *desc, int32_t n_tokens, size_t *bytes);

/* Encode fp32 weights as IQ4_NL: w holds n_blocks groups of 32 consecutive weights; out
 * receives n_blocks * 18 bytes.  Per block: d = fp16_RNE(fp32(max|w|) / 127), each weight
 * the nearest codebook entry scaled by the stored d, ties to the lower index.  (Format of
 * PocketLLM "Xing4.0-29B-A4B", section "Overview".)  Weights must be finite. */
moe_status moe_quantize_iq4nl(const float *w, int64_t n_blocks, uint8_t *out,
                              hipStream_t stream);

/* Decode IQ4_NL to fp32: out[32*b + i] = d_b * c[q_{b,i}] (exact in fp32). */
moe_status moe_dequantize_iq4nl(const uint8_t *blocks, int64_t n_blocks, float *out,
                                hipStream_t stream);

/* Router scoring, gating and top-k (PocketLLM page "Overview": sigmoid routing with a shared
 * expert; Red Lite "1. The idea"; Xolotl "Why build an engine at all").
 *   x        [T, H] fp32 activations
 *   w_router [E, H] fp32, row e scores expert e
 *   bias     [E] fp32 or NULL; added to the logits (affects selection and weights)
 *   topk_ids [T, k] int32 out: experts by (logit descending, index ascending); a NaN logit
 *            orders below every number
 *   topk_w   [T, k] fp32 out: SIGMOID: s = 1/(1+exp(-l)); SOFTMAX: softmax over all E;
 *            divided by their sum when desc->renormalize
 *   logits   [T, E] fp32 out, or NULL (then kept in the workspace)
 * Logits are fp32 with fp32 accumulation. */
moe_status moe_route(const moe_desc *desc, const float *x, const float *w_router,
                     const float *bias, int32_t n_tokens, int32_t *topk_ids, float *topk_w,
                     float *logits, void *ws, size_t ws_bytes, hipStream_t stream);

/* Route sanitisation and token-to-expert permutation ("Running Qwen Flash-Next NVFP4 in
 * vLLM", B12x route validation; PocketLLM page, "Without a server": the route table).
 *   topk_ids, topk_w [T, k] in/out: an id < 0 or >= E becomes 0 and its weight 0 (in place);
 *            the count is written to workspace bytes 0..3
 *   offsets      [E+S+1] int32 out (see "Slots" above)
 *   sorted_pairs [T*k] int32 out: pair id at each routed slot, stable in p
 *   pair_slot    [T*k] int32 out: inverse of sorted_pairs
 *   x, x_perm    optional (both NULL or both set): x_perm[slot] = x[token(slot)] for all
 *                rows = T*k + T*S slots, as fp32 or bf16 (RNE), per x_perm_dtype
 * Integer results are exact and deterministic (no atomics decide any order). */
moe_status moe_permute(const moe_desc *desc, int32_t *topk_ids, float *topk_w,
                       int32_t n_tokens, const float *x, void *x_perm, int32_t x_perm_dtype,
                       int32_t *offsets, int32_t *sorted_pairs, int32_t *pair_slot,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/* Decode path: grouped dequant-GEMV over the experts that the route table uses, fp32
 * activations, fp32 accumulation (PocketLLM page "Overview": resident experts indexed by
 * expert; Red Lite "4. Speculative decoding": decode each weight block once for all rows
 * that share it).
 *   GATE_UP: in = x [T, H] fp32 in TOKEN order (row of slot s: x[token(s)], via
 *            sorted_pairs); out = h [rows, F] fp32, h = silu(W_g x) * (W_u x)
 *   DOWN:    in = h [rows, F] fp32 in slot order (sorted_pairs may be NULL);
 *            out = o [rows, H] fp32, o = W_d h
 * Activations are split into two bf16 terms (hi + lo, 16 significant bits) inside the
 * kernel; products with the exact bf16 codebook entries are summed in fp32. */
/* (ws / ws_bytes: reserved; may be NULL / 0.) */
moe_status moe_expert_gemv_iq4nl(const moe_desc *desc, int32_t stage, const moe_bank *bank,
                                 const int32_t *offsets, const int32_t *sorted_pairs,
                                 const float *in, float *out, int32_t n_tokens,
                                 void *ws, size_t ws_bytes, hipStream_t stream);

/* Prefill path: grouped GEMM over the experts' slot ranges on bf16 matrix cores
 * (v_mfma_f32_16x16x32_bf16), weights dequantised tile by tile into LDS as bf16(d * c),
 * fp32 accumulation (Xolotl "Prompts: fast, and exact": each layer's experts run once per
 * chunk as one batched multiply).
 *   GATE_UP: in = x_perm [rows, H] bf16 in slot order; out = h [rows, F] bf16,
 *            h = bf16_RNE(silu(g) * u) from fp32 g, u
 *   DOWN:    in = h [rows, F] bf16 in slot order; out = o [rows, H] fp32
 * The tile schedule is built on the device from offsets; no host round trip. */
/* (ws / ws_bytes: reserved; may be NULL / 0.) */
moe_status moe_grouped_gemm_iq4nl(const moe_desc *desc, int32_t stage, const moe_bank *bank,
                                  const int32_t *offsets, const void *in_bf16, void *out,
                                  int32_t n_tokens, void *ws, size_t ws_bytes,
                                  hipStream_t stream);

/* Weighted combine in fixed order (PocketLLM page, "Where the detail is": deterministic
 * route reduction):
 *   y[t] = sum_{j<k} topk_w[t,j] * o[pair_slot[t*k+j]] + sum_s o[T*k + s*T + t]
 *          (+ residual[t] if residual != NULL)
 * o [rows, H] fp32; y [T, H] fp32 (y may alias residual). */
moe_status moe_combine(const moe_desc *desc, const float *o, const int32_t *pair_slot,
                       const float *topk_w, int32_t n_tokens, const float *residual,
                       float *y, hipStream_t stream);

/* Fused decode layer for small batches (1 <= T <= 16): three launches (router, gate/up, down
 * with the combine) at every T, no host round trip
 * (PocketLLM page, "Known limitations": decode bound by launch count; Red Lite "1. The idea":
 * a whole token routed on the GPU).  Computes
 *   xn = norm_eps >= 0 ? x / sqrt(mean(x^2) + norm_eps) : x        (per row)
 *   y  = MoE(xn) (+ residual if residual != NULL)
 * with the routing of moe_route (bias nullable), the permutation of moe_permute, the expert
 * GEMV arithmetic of moe_expert_gemv_iq4nl and the fixed-order combine of moe_combine.
 *   x [T, H], residual [T, H], y [T, H] fp32; y may alias x and residual.
 *   topk_ids [T, k], topk_w [T, k]: optional outputs of the route table (NULL: kept in ws).
 * stages: bitmask of the parts to enqueue -- MOE_DECODE_ROUTER (RMSNorm and logits),
 * MOE_DECODE_GATE_UP (gate/up, the routing redone in every workgroup, and the route table
 * and permutation), MOE_DECODE_DOWN (down + combine); MOE_DECODE_ALL for the layer.
 * Split calls must be enqueued in that order on one stream with the same arguments and
 * workspace.
 * ws: at least moe_workspace_size(desc, T) bytes, 256-byte aligned; holds the logits, the
 * permutation, h, the per-slot down outputs and the down's row-range counters (set by the
 * gate/up launch).  The route table never leaves the device between the launches. */
#define MOE_DECODE_ROUTER 1
#define MOE_DECODE_GATE_UP 2
#define MOE_DECODE_DOWN 4
#define MOE_DECODE_ALL 7
moe_status moe_decode_layer(const moe_desc *desc, const moe_bank *bank, const float *w_router,
                            const float *bias, const float *x, int32_t n_tokens, float norm_eps,
                            const float *residual, float *y, int32_t *topk_ids, float *topk_w,
                            int32_t stages, void *ws, size_t ws_bytes, hipStream_t stream);

/* Allocation-free variant of moe_decode_layer, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same checks, launches and results as moe_decode_layer, with the workspace replaced by a
 * fixed scratch array of MOE_NOALLOC_SCRATCH_BYTES that the library holds in device memory on
 * each GPU it runs on, from that GPU's first call until the process ends.  Nothing is
 * allocated or freed by the call.  Inputs and outputs are the caller's, as in
 * moe_decode_layer.
 *   - Returns MOE_ERR_SCRATCH_LIMIT (nothing enqueued) when the layer shape and n_tokens need
 *     more workspace than the array holds (moe_workspace_size() reports what is needed; the
 *     shapes of the 3584/64, 2048/512 and 7168/384 layers need at most 4.4 MB at 16 tokens).
 *   - Every call on one GPU uses that GPU's single array and leaves its contents behind; no
 *     part of it needs to start at zero (every launch writes what a later one reads).  Calls
 *     that overlap in time on one GPU (two streams, two threads) race on it: order them on one
 *     stream.
 *   - The first call on a device looks up the array's device address (hipGetSymbolAddress)
 *     and may return MOE_ERR_HIP if that fails. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
moe_status moe_decode_layer_noalloc(const moe_desc *desc, const moe_bank *bank,
                                    const float *w_router, const float *bias, const float *x,
                                    int32_t n_tokens, float norm_eps, const float *residual,
                                    float *y, int32_t *topk_ids, float *topk_w, int32_t stages,
                                    hipStream_t stream);

/* One layer of a decode stack: its expert bank, router [E, H] fp32 and bias [E] (or NULL). */
typedef struct moe_layer {
    moe_bank bank;
    const float *w_router;
    const float *bias;
} moe_layer;

#define MOE_CHAIN_MAX_LAYERS 64

/* Decode step of a stack of layers, 1 <= T <= 16 tokens, with no host round trip between
 * layers (PocketLLM page, "Known limitations": a decode step bound by its launch count; Red
 * Lite "1. The idea": the whole token routed on the GPU).  For l = 0 .. n_layers-1, in place:
 *   x <- x + MoE_l(xn),  xn = norm_eps >= 0 ? x / sqrt(mean(x^2) + norm_eps) : x  (per row)
 * with MoE_l as in moe_decode_layer on layers[l], enqueued as that entry point's launches,
 * layer after layer, on one stream (capture the call in a HIP graph to replay a whole step).
 *   layers    host array of n_layers (<= MOE_CHAIN_MAX_LAYERS) entries, read during the call
 *   x         [T, H] fp32, in/out
 *   topk_ids, topk_w: both NULL, or [n_layers, T, k] outputs of every layer's route
 *   ws        >= moe_workspace_size(desc, T) bytes, 256-byte aligned
 * Every layer's bank and router are checked before anything is enqueued. */
moe_status moe_decode_chain(const moe_desc *desc, const moe_layer *layers, int32_t n_layers,
                            float *x, int32_t n_tokens, float norm_eps, int32_t *topk_ids,
                            float *topk_w, void *ws, size_t ws_bytes, hipStream_t stream);

/* Weight-free RMSNorm y = x / sqrt(mean(x^2) + eps) over rows of [T, H] fp32: the glue a
 * chain of layers puts between x and each layer's input (y may alias x). */
moe_status moe_rmsnorm(const float *x, int32_t n_tokens, int32_t hidden, float eps, float *y,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_IQ4NL_H */
