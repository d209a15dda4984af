"""GPU parity of whole layers at the workloads' full sizes, through the same C-ABI calls and
launch configuration that bench.py times.

The oracle is too slow for every token of a 2,048- or 8,192-token chunk, so those tests check
sampled tokens (a token's output depends only on that token); small batches are checked in
full.  The 38-layer decode chain is checked against the oracle on its first two layers and by
properties (finite, bounded RMS, bit-identical reruns, identical HIP-graph replays) on all.
"""
import numpy as np
import pytest
import torch

import quantized_moe_expert_amd as M
from quantized_moe_expert_amd import layer as L
from oracle import moe as omoe
from synth import generator as G
from synth.configs import (WORKLOADS, TINY, XING4_DECODE, LayerShape, SIGMOID, SOFTMAX,
                           Workload)

from .helpers import (REL_L2_GEMV, REL_L2_MFMA, assert_close, desc_of, oracle_bank,
                      oracle_layer, topk_gap)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu_layer(wl, T, prefill, layer=0):
    bank_t, bank = L.make_bank(wl, layer)
    wr, bias = L.make_router(wl, layer)
    x = L.make_activations(wl, T)
    buf = L.LayerBuffers(wl.shape, T, prefill=prefill)
    run = L.prefill_layer if prefill else L.decode_layer
    y = run(buf, x, wr, bias, bank).clone()
    torch.cuda.synchronize()
    return y.cpu().numpy(), buf, (bank_t, bank, wr, bias, x)


def _pick_tokens(wl, x, count, seed):
    """Tokens away from routing near-ties (gap between k-th and (k+1)-th logit)."""
    s = wl.shape
    b = G.zipf_bias(wl, 0) if wl.zipf_s is not None else None
    l = omoe.router_logits(x, G.router_weight(wl, 0), b)
    ok = np.where(topk_gap(l, s.top_k) > 1e-3)[0]
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(ok, size=min(count, len(ok)), replace=False))


@pytest.mark.parametrize("prefill", [False, True])
def test_tiny_layer_full(prefill):
    wl = TINY
    T = wl.decode_tokens[0]
    y, buf, _ = _gpu_layer(wl, T, prefill)
    x = G.activations(wl, T)
    ref, parts = oracle_layer(wl, 0, x, return_parts=True)
    assert np.array_equal(buf.ids.cpu().numpy(), parts["ids"])
    assert_close(y, ref, REL_L2_MFMA if prefill else REL_L2_GEMV, f"tiny prefill={prefill}")


@pytest.mark.parametrize("name,T,n_check", [("xing4_decode", 1, 1), ("xing4_decode", 16, 16),
                                            ("qwen3next_like", 1, 1), ("qwen3next_like", 2, 2),
                                            ("dsv41_like", 16, 4)])
def test_decode_layer_full_size(name, T, n_check):
    wl = WORKLOADS[name]
    y, buf, _ = _gpu_layer(wl, T, prefill=False)
    x = G.activations(wl, T)
    toks = np.arange(T) if n_check >= T else _pick_tokens(wl, x, n_check, T)
    ref, parts = oracle_layer(wl, 0, x[toks], return_parts=True)
    assert np.array_equal(buf.ids.cpu().numpy()[toks], parts["ids"])
    assert_close(y[toks], ref, REL_L2_GEMV, f"{name} T={T}")


@pytest.mark.parametrize("name,T,n_check", [("xing4_prefill", 2048, 2), ("qwen3next_like", 2048, 2),
                                            ("dsv41_like", 8192, 1), ("xing4_prefill", 1, 1)])
def test_prefill_layer_full_size(name, T, n_check):
    wl = WORKLOADS[name]
    y, buf, keep = _gpu_layer(wl, T, prefill=True)
    assert np.all(np.isfinite(y))
    x = G.activations(wl, T)
    toks = _pick_tokens(wl, x, n_check, T)
    ref, parts = oracle_layer(wl, 0, x[toks], return_parts=True)
    assert np.array_equal(buf.ids.cpu().numpy()[toks], parts["ids"])
    assert_close(y[toks], ref, REL_L2_MFMA, f"{name} T={T}")
    # every token's route is the selection on the GPU's own logits
    lg = buf.logits.cpu().numpy().astype(np.float64)
    assert np.array_equal(buf.ids.cpu().numpy(), omoe.select_topk(lg, wl.shape.top_k))
    # rerun: bit-identical
    bank_t, bank, wr, bias, xd = keep
    y2 = L.prefill_layer(buf, xd, wr, bias, bank).clone()
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy(), y)


@pytest.mark.parametrize("name,T,n_check", [("tiny", 4, 4), ("xing4_decode", 1, 1),
                                            ("xing4_decode", 16, 16), ("qwen3next_like", 1, 1),
                                            ("qwen3next_like", 2, 2), ("dsv41_like", 16, 1),
                                            # ragged batches: partial token tiles and chunks
                                            ("xing4_decode", 3, 3), ("xing4_decode", 7, 2),
                                            ("qwen3next_like", 5, 2), ("dsv41_like", 9, 1)])
def test_fused_decode_layer_full_size(name, T, n_check):
    wl = WORKLOADS[name]
    s = wl.shape
    bank_t, bank = L.make_bank(wl, 0)
    wr, bias = L.make_router(wl, 0)
    x = L.make_activations(wl, T)
    buf = L.LayerBuffers(s, T)
    y = L.decode_layer_fused(buf, x, wr, bias, bank).clone()
    ids = buf.ids.clone()
    # the unfused entry points on the same inputs: same routes, same outputs within tolerance
    buf2 = L.LayerBuffers(s, T)
    y2 = L.decode_layer(buf2, x, wr, bias, bank).clone()
    # split stages: bit-identical to one call
    y3 = torch.empty_like(y)
    for st in (M.MOE_DECODE_ROUTER, M.MOE_DECODE_GATE_UP, M.MOE_DECODE_DOWN):
        L.decode_layer_fused(buf, x, wr, bias, bank, out=y3, stages=st)
    torch.cuda.synchronize()
    assert torch.equal(ids, buf2.ids)
    assert torch.equal(y3, y)
    assert_close(y.cpu().numpy(), y2.cpu().numpy().astype(np.float64), REL_L2_GEMV, "fused vs unfused")
    xh = G.activations(wl, T)
    toks = np.arange(T) if n_check >= T else _pick_tokens(wl, xh, n_check, T)
    ref, parts = oracle_layer(wl, 0, xh[toks], return_parts=True)
    assert np.array_equal(ids.cpu().numpy()[toks], parts["ids"])
    assert_close(y.cpu().numpy()[toks], ref, REL_L2_GEMV, f"fused {name} T={T}")


# row lengths whose lane geometry is 4 or 8 lanes of 3 blocks (hidden 384 and 768, FFN 384);
# hidden 320 (5 blocks of 64 and an odd half of 128) takes the matrix-core path's fallback
# kernels (a gate/up workgroup of 64 FFN rows, a down workgroup of 16 output rows)
ODD_SHAPES = {
    "h384_f384": Workload(name="h384_f384", cfg_id=7,
                          shape=LayerShape(hidden=384, ffn=384, n_experts=16, top_k=3, n_shared=1,
                                           gating=SIGMOID, renormalize=1), layers=1),
    "h768_f384": Workload(name="h768_f384", cfg_id=8,
                          shape=LayerShape(hidden=768, ffn=384, n_experts=16, top_k=2, n_shared=1,
                                           gating=SIGMOID, renormalize=1), layers=1),
    "h320_f256": Workload(name="h320_f256", cfg_id=12,
                          shape=LayerShape(hidden=320, ffn=256, n_experts=16, top_k=3, n_shared=1,
                                           gating=SIGMOID, renormalize=1), layers=1),
}


@pytest.mark.parametrize("name", sorted(ODD_SHAPES))
@pytest.mark.parametrize("T", [1, 3, 9])
def test_fused_decode_layer_odd_row_lengths(name, T):
    wl = ODD_SHAPES[name]
    bank_t, bank = L.make_bank(wl, 0)
    wr, bias = L.make_router(wl, 0)
    x = L.make_activations(wl, T)
    buf = L.LayerBuffers(wl.shape, T)
    y = L.decode_layer_fused(buf, x, wr, bias, bank, norm_eps=1e-6).clone()
    torch.cuda.synchronize()
    xh = omoe.rmsnorm(G.activations(wl, T), 1e-6)
    ref, parts = oracle_layer(wl, 0, xh, return_parts=True)
    assert np.array_equal(buf.ids.cpu().numpy(), parts["ids"])
    assert_close(y.cpu().numpy(), ref, REL_L2_GEMV, f"{name} T={T}")


# degenerate routes: no shared expert; one expert that every token picks; k = E (every
# expert picked by every token); softmax gating without renormalisation
EDGE_SHAPES = {
    "no_shared": Workload(name="no_shared", cfg_id=9,
                          shape=LayerShape(hidden=512, ffn=256, n_experts=16, top_k=4, n_shared=0,
                                           gating=SIGMOID, renormalize=1), layers=1),
    "one_expert": Workload(name="one_expert", cfg_id=10,
                           shape=LayerShape(hidden=256, ffn=128, n_experts=1, top_k=1,
                                            n_shared=0, gating=SIGMOID, renormalize=1), layers=1),
    "k_equals_e": Workload(name="k_equals_e", cfg_id=11,
                           shape=LayerShape(hidden=256, ffn=192, n_experts=4, top_k=4, n_shared=1,
                                            gating=SOFTMAX, renormalize=0), layers=1),
}


@pytest.mark.parametrize("name", sorted(EDGE_SHAPES))
@pytest.mark.parametrize("T", [1, 5, 16])
def test_fused_decode_degenerate_routes(name, T):
    """Both decode paths (T = 1: dequant-GEMV; T = 5, 16: matrix cores) on routes with no
    shared expert, a single expert, or k = E; ids bit-exact, y against the oracle, and the
    split stages bit-identical to one call."""
    wl = EDGE_SHAPES[name]
    bank_t, bank = L.make_bank(wl, 0)
    wr, bias = L.make_router(wl, 0)
    x = L.make_activations(wl, T)
    buf = L.LayerBuffers(wl.shape, T)
    y = L.decode_layer_fused(buf, x, wr, bias, bank).clone()
    y3 = torch.empty_like(y)
    for st in (M.MOE_DECODE_ROUTER, M.MOE_DECODE_GATE_UP, M.MOE_DECODE_DOWN):
        L.decode_layer_fused(buf, x, wr, bias, bank, out=y3, stages=st)
    torch.cuda.synchronize()
    assert torch.equal(y3, y)
    ref, parts = oracle_layer(wl, 0, G.activations(wl, T), return_parts=True)
    assert np.array_equal(buf.ids.cpu().numpy(), parts["ids"])
    assert_close(buf.w.cpu().numpy(), parts["weights"], 1e-5, f"weights {name} T={T}")
    assert_close(y.cpu().numpy(), ref, REL_L2_GEMV, f"{name} T={T}")


def test_fused_decode_rejects_large_batches():
    wl = XING4_DECODE
    s = wl.shape
    desc = L.desc_of(s, 17)
    bank_t, bank = L.make_bank(wl, 0, experts=[0])
    x = torch.zeros((17, s.hidden), device=DEV)
    with pytest.raises(M.MoeError) as ei:
        M.moe_decode_layer(desc, bank, x, None, x, 17, -1.0, None, x, None, None, x, 1 << 20)
    assert ei.value.status == M.MOE_ERR_SHAPE


@pytest.mark.parametrize("fused", [True, False])
def test_decode_chain_two_layers_vs_oracle(fused):
    wl = XING4_DECODE
    s = wl.shape
    T = 1
    layers = []
    for l in range(2):
        bank_t, bank = L.make_bank(wl, l)
        wr, bias = L.make_router(wl, l)
        layers.append((wr, bias, bank, bank_t))
    x = L.make_activations(wl, T)
    buf = L.LayerBuffers(s, T)
    L.decode_chain_step(buf, x, [(a, b, c) for (a, b, c, _) in layers], fused=fused)
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    # oracle chain: x <- x + MoE_l(rmsnorm(x))
    xr = G.activations(wl, T).astype(np.float64)
    desc = desc_of(s)
    for l in range(2):
        xn = omoe.rmsnorm(xr)
        wr = G.router_weight(wl, l)
        _, ids, _ = omoe.route(xn, wr, None, desc)
        bank, stride = oracle_bank(wl, l, set(ids.reshape(-1).tolist()) | {s.n_experts})
        xr = xr + omoe.moe_layer(xn, wr, None, bank, stride, desc)
    assert_close(got, xr, REL_L2_GEMV, "2-layer chain")


def test_decode_chain_38_layers_properties_and_graph_replay():
    wl = XING4_DECODE
    s = wl.shape
    T = 1
    layers, keep = [], []
    for l in range(wl.layers):
        bank_t, bank = L.make_bank(wl, l)
        wr, bias = L.make_router(wl, l)
        layers.append((wr, bias, bank))
        keep.append(bank_t)
    x0 = L.make_activations(wl, T)
    buf = L.LayerBuffers(s, T)
    x = x0.clone()
    rms = []
    for lay in layers:
        L.decode_chain_step(buf, x, [lay])
        rms.append(float(torch.sqrt(torch.mean(x * x)).item()))
    assert all(np.isfinite(rms)) and max(rms) < 10.0 and min(rms) > 0.5, rms
    eager = x.clone()
    # rerun: bit-identical
    x.copy_(x0)
    L.decode_chain_step(buf, x, layers)
    torch.cuda.synchronize()
    assert torch.equal(x, eager)
    # HIP graph of the whole 38-layer step; several replays with eager work in between
    xg = x0.clone()
    g = torch.cuda.CUDAGraph()
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        L.decode_chain_step(buf, xg, layers)          # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s_)
    xg.copy_(x0)
    with torch.cuda.graph(g):
        L.decode_chain_step(buf, xg, layers)
    for _ in range(3):
        xg.copy_(x0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xg, eager)
        junk = torch.randn(1000, device=DEV).sum()    # unrelated eager work between replays
        torch.cuda.synchronize()
        del junk


def test_invalid_routes_contribute_nothing():
    wl = TINY
    s = wl.shape
    T = 4
    bank_t, bank = L.make_bank(wl, 0)
    x = L.make_activations(wl, T)
    buf = L.LayerBuffers(s, T)
    ids = np.array([[1, -1], [9, 2], [3, 3], [2 ** 31 - 1, 0]], np.int32)
    w = np.array([[0.6, 0.4], [0.5, 0.5], [0.2, 0.8], [0.3, 0.7]], np.float32)
    buf.ids.copy_(torch.from_numpy(ids))
    buf.w.copy_(torch.from_numpy(w))
    M.moe_permute(buf.desc, buf.ids, buf.w, T, None, None, 0, buf.offsets, buf.sorted_pairs,
                  buf.pair_slot, buf.ws, buf.ws_bytes)
    M.moe_expert_gemv_iq4nl(buf.desc, M.MOE_STAGE_GATE_UP, bank, buf.offsets, buf.sorted_pairs,
                            x, buf.h, T)
    M.moe_expert_gemv_iq4nl(buf.desc, M.MOE_STAGE_DOWN, bank, buf.offsets, None, buf.h, buf.o, T)
    M.moe_combine(buf.desc, buf.o, buf.pair_slot, buf.w, T, None, buf.y)
    torch.cuda.synchronize()
    assert int(buf.ws[:4].view(torch.int32).item()) == 3
    xh = G.activations(wl, T)
    bank_np, stride = oracle_bank(wl, 0, range(s.n_experts + 1))
    ref = omoe.moe_layer(xh, None, None, bank_np, stride, desc_of(s), ids=ids, weights=w)
    assert_close(buf.y.cpu().numpy(), ref, REL_L2_GEMV, "invalid routes")


@pytest.mark.parametrize("name,lift,T", [("xing4_decode", (20, 40), 1),
                                         ("qwen3next_like", (3, 500, 77), 1), ("tiny", (5,), 1),
                                         ("xing4_decode", (20, 40), 16),
                                         ("qwen3next_like", (3, 500, 77), 9),
                                         ("dsv41_like", (383, 0), 16)])
def test_decode_with_exact_logit_ties(name, lift, T):
    """Every expert gets the same router row, so all logits tie except the lifted experts'
    (bias +1): the top-k set is the lifted experts plus the lowest-index tied ones.  The
    routed workgroups of the one-token path pick their experts by set membership, those of
    the batched path by counting the experts ranked above theirs, the publishing one by the
    full top-k; all must agree with the oracle's tie rule."""
    wl = WORKLOADS[name]
    s = wl.shape
    wr_h = np.repeat(G.router_weight(wl, 0)[:1], s.n_experts, axis=0)
    bias_h = np.zeros(s.n_experts, np.float32)
    for e in lift:
        bias_h[e] = 1.0
    wr = torch.from_numpy(wr_h).to(DEV)
    bias = torch.from_numpy(bias_h).to(DEV)
    bank_t, bank = L.make_bank(wl, 0)
    x = L.make_activations(wl, T)
    buf = L.LayerBuffers(s, T)
    y = L.decode_layer_fused(buf, x, wr, bias, bank).clone()
    torch.cuda.synchronize()
    xh = G.activations(wl, T)
    ref, parts = oracle_layer(wl, 0, xh, return_parts=True, bias=bias_h, w_router=wr_h)
    want = sorted(lift) + [e for e in range(s.n_experts) if e not in lift][:s.top_k - len(lift)]
    for t in range(T):
        assert sorted(parts["ids"][t].tolist()) == sorted(want)
    assert np.array_equal(buf.ids.cpu().numpy(), parts["ids"])
    assert_close(y.cpu().numpy(), ref, REL_L2_GEMV, f"ties {name} T={T}")
