"""Orchestration of the C-ABI calls for whole layers and chains (no arithmetic here).

``LayerBuffers`` owns the per-call device tensors of one layer shape and token count;
``decode_layer`` / ``prefill_layer`` enqueue route -> permute -> experts -> combine on the
current stream; ``make_bank`` builds a layer's IQ4_NL expert bank on the GPU from the seeded
generator (``synth.device``) and the library's own encoder.
"""
import torch

from . import (MOE_DTYPE_BF16, MOE_STAGE_DOWN, MOE_STAGE_GATE_UP, make_bank as _make_bank,
               make_desc, make_layers, moe_combine, moe_decode_chain, moe_decode_layer,
               moe_expert_gemv_iq4nl,
               moe_grouped_gemm_iq4nl, moe_permute, moe_quantize_iq4nl, moe_rmsnorm, moe_route,
               moe_workspace_size)


def desc_of(shape, max_tokens):
    return make_desc(shape.hidden, shape.ffn, shape.n_experts, shape.top_k, shape.n_shared,
                     shape.gating, shape.renormalize, max_tokens)


class LayerBuffers:
    """Device buffers for one layer call with T tokens (reusable across layers in stream order)."""

    def __init__(self, shape, T, prefill=False, device="cuda"):
        self.shape, self.T, self.prefill = shape, T, prefill
        s = shape
        self.desc = desc_of(shape, max(T, 1))
        rows = T * s.top_k + T * s.n_shared
        self.rows = rows
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.ids = torch.empty((T, s.top_k), **i32)
        self.w = torch.empty((T, s.top_k), **f32)
        self.logits = torch.empty((T, s.n_experts), **f32)
        self.offsets = torch.empty(s.n_experts + s.n_shared + 1, **i32)
        self.sorted_pairs = torch.empty(max(T * s.top_k, 1), **i32)
        self.pair_slot = torch.empty(max(T * s.top_k, 1), **i32)
        self.ws_bytes = moe_workspace_size(self.desc, T)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=device)
        if prefill:
            self.x_perm = torch.empty((rows, s.hidden), dtype=torch.bfloat16, device=device)
            self.h = torch.empty((rows, s.ffn), dtype=torch.bfloat16, device=device)
        else:
            self.x_perm = None
            self.h = torch.empty((rows, s.ffn), **f32)
        self.o = torch.empty((rows, s.hidden), **f32)
        self.y = torch.empty((T, s.hidden), **f32)
        self.xn = torch.empty((T, s.hidden), **f32)


def route_and_permute(buf, x, w_router, bias, gather_bf16=False):
    T = buf.T
    moe_route(buf.desc, x, w_router, bias, T, buf.ids, buf.w, buf.logits, buf.ws, buf.ws_bytes)
    moe_permute(buf.desc, buf.ids, buf.w, T, x if gather_bf16 else None,
                buf.x_perm if gather_bf16 else None, MOE_DTYPE_BF16, buf.offsets,
                buf.sorted_pairs, buf.pair_slot, buf.ws, buf.ws_bytes)


def decode_layer(buf, x, w_router, bias, bank, residual=None, out=None):
    """y = MoE(x) (+ residual) through the GEMV path; returns the output tensor."""
    route_and_permute(buf, x, w_router, bias)
    moe_expert_gemv_iq4nl(buf.desc, MOE_STAGE_GATE_UP, bank, buf.offsets, buf.sorted_pairs, x,
                          buf.h, buf.T)
    moe_expert_gemv_iq4nl(buf.desc, MOE_STAGE_DOWN, bank, buf.offsets, None, buf.h, buf.o, buf.T)
    y = buf.y if out is None else out
    moe_combine(buf.desc, buf.o, buf.pair_slot, buf.w, buf.T, residual, y)
    return y


def prefill_layer(buf, x, w_router, bias, bank, residual=None, out=None):
    """y = MoE(x) (+ residual) through the grouped-GEMM (bf16 MFMA) path."""
    route_and_permute(buf, x, w_router, bias, gather_bf16=True)
    moe_grouped_gemm_iq4nl(buf.desc, MOE_STAGE_GATE_UP, bank, buf.offsets, buf.x_perm, buf.h,
                           buf.T)
    moe_grouped_gemm_iq4nl(buf.desc, MOE_STAGE_DOWN, bank, buf.offsets, buf.h, buf.o, buf.T)
    y = buf.y if out is None else out
    moe_combine(buf.desc, buf.o, buf.pair_slot, buf.w, buf.T, residual, y)
    return y


def decode_layer_fused(buf, x, w_router, bias, bank, norm_eps=-1.0, residual=None, out=None,
                       stages=None):
    """y = MoE(xn) (+ residual) through moe_decode_layer (three launches, T <= 16)."""
    y = buf.y if out is None else out
    moe_decode_layer(buf.desc, bank, w_router, bias, x, buf.T, norm_eps, residual, y, buf.ids,
                     buf.w, buf.ws, buf.ws_bytes, stages=stages)
    return y


def decode_chain_step(buf, x, layers, eps=1e-6, fused=True):
    """x <- x + MoE_l(rmsnorm(x)) for every (w_router, bias, bank) in layers, in place.

    fused: one moe_decode_layer call a layer (the RMSNorm folded into it); otherwise the
    separate entry points (rmsnorm, route, permute, two GEMVs, combine)."""
    for (w_router, bias, bank) in layers:
        if fused:
            decode_layer_fused(buf, x, w_router, bias, bank, norm_eps=eps, residual=x, out=x)
        else:
            moe_rmsnorm(x, buf.T, buf.shape.hidden, eps, buf.xn)
            decode_layer(buf, buf.xn, w_router, bias, bank, residual=x, out=x)
    return x


def decode_chain(buf, x, layers, eps=1e-6, ids=None, w=None):
    """x <- x + MoE_l(rmsnorm(x)) for every layer, in place, in ONE moe_decode_chain call.

    layers: list of (w_router, bias, bank) or the ctypes array of ``make_layers``;
    ids / w: optional [L, T, k] outputs of every layer's route."""
    if not hasattr(layers, "_type_"):
        layers = make_layers([(bank, wr, bias) for (wr, bias, bank) in layers])
    moe_decode_chain(buf.desc, layers, len(layers), x, buf.T, eps, ids, w, buf.ws, buf.ws_bytes)
    return x


# ---- expert banks from the seeded generator ----------------------------------------------

def make_bank(workload, layer, device="cuda", scratch=None, experts=None):
    """IQ4_NL bank [E+S experts] of one layer, generated and encoded on the GPU.

    Returns (bank_tensor uint8, moe_bank struct).  ``experts``: optional subset of expert
    indices to fill (others left zero) -- for tests that need only a few.
    """
    from synth import device as SD, generator as G
    s = workload.shape
    stride = s.expert_bytes
    n_exp = s.n_experts + s.n_shared
    bank = torch.zeros(stride * n_exp, dtype=torch.uint8, device=device)
    big = max(s.ffn * s.hidden, s.hidden * s.ffn)
    if scratch is None or scratch.numel() < big:
        scratch = torch.empty(big, dtype=torch.float32, device=device)
    for e in (range(n_exp) if experts is None else experts):
        off = e * stride
        for tensor, rows, cols in ((G.T_GATE, s.ffn, s.hidden), (G.T_UP, s.ffn, s.hidden),
                                   (G.T_DOWN, s.hidden, s.ffn)):
            n = rows * cols
            w = scratch[:n]
            SD.fill_normal(w, workload.seed, workload.cfg_id, layer, e, tensor, 0,
                           workload.weight_sigma)
            nbytes = n // 32 * 18
            moe_quantize_iq4nl(w, n // 32, bank[off:off + nbytes])
            off += nbytes
    return bank, _make_bank(bank, stride)


def make_router(workload, layer, device="cuda"):
    from synth import device as SD, generator as G
    s = workload.shape
    wr = torch.empty((s.n_experts, s.hidden), dtype=torch.float32, device=device)
    SD.fill_normal(wr, workload.seed, workload.cfg_id, layer, 0, G.T_ROUTER, 0,
                   workload.router_sigma)
    bias = None
    if workload.zipf_s is not None:
        bias = torch.from_numpy(G.zipf_bias(workload, layer)).to(device)
    return wr, bias


def make_activations(workload, T, device="cuda"):
    from synth import device as SD, generator as G
    x = torch.empty((T, workload.shape.hidden), dtype=torch.float32, device=device)
    SD.fill_normal(x, workload.seed, workload.cfg_id, 0, 0, G.T_X, 0, workload.x_sigma)
    return x
