"""GPU parity of moe_decode_chain: a stack of decode layers in one call.

Each layer is x <- x + MoE_l(rmsnorm(x)).  Checked against the oracle's chain (fp64) on short
stacks, against the per-layer entry point on the full 38-layer stack, for bit-identical
reruns and HIP-graph replays, and for the host-side argument checks.
"""
import numpy as np
import pytest
import torch

import quantized_moe_expert_amd as M
from quantized_moe_expert_amd import layer as L
from oracle import moe as omoe
from synth import generator as G
from synth.configs import WORKLOADS, XING4_DECODE

from .helpers import REL_L2_GEMV, assert_close, desc_of, oracle_bank, topk_gap

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _layers(wl, n):
    out, keep = [], []
    for l in range(n):
        bt, bank = L.make_bank(wl, l)
        wr, bias = L.make_router(wl, l)
        out.append((wr, bias, bank))
        keep.append(bt)
    return out, keep


def _oracle_chain(wl, T, n):
    s = wl.shape
    desc = desc_of(s)
    x = G.activations(wl, T).astype(np.float64)
    ids_all, gaps = [], []
    for l in range(n):
        xn = omoe.rmsnorm(x, EPS)
        wr = G.router_weight(wl, l)
        b = G.zipf_bias(wl, l) if wl.zipf_s is not None else None
        logits, ids, _ = omoe.route(xn, wr, b, desc)
        bank, stride = oracle_bank(wl, l, set(ids.reshape(-1).tolist()) | {s.n_experts})
        x = x + omoe.moe_layer(xn, wr, b, bank, stride, desc)
        ids_all.append(ids)
        gaps.append(topk_gap(logits, s.top_k))
    return x, np.stack(ids_all), np.stack(gaps)


@pytest.mark.parametrize("name,T,n", [("tiny", 4, 3), ("xing4_decode", 1, 2),
                                      ("xing4_decode", 2, 2), ("qwen3next_like", 1, 2),
                                      ("qwen3next_like", 2, 2)])
def test_chain_vs_oracle(name, T, n):
    wl = WORKLOADS[name]
    s = wl.shape
    layers, keep = _layers(wl, n)
    buf = L.LayerBuffers(s, T)
    x = L.make_activations(wl, T)
    ids = torch.empty((n, T, s.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((n, T, s.top_k), dtype=torch.float32, device="cuda")
    L.decode_chain(buf, x, layers, EPS, ids, w)
    torch.cuda.synchronize()
    ref, ref_ids, gaps = _oracle_chain(wl, T, n)
    assert gaps.min() > 1e-4, "fixture has a routing near-tie"
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.all(np.isfinite(w.cpu().numpy()))
    assert_close(x.cpu().numpy(), ref, REL_L2_GEMV, f"chain {name} T={T} layers={n}")


def test_chain_38_layers_vs_per_layer_path():
    wl = XING4_DECODE
    s = wl.shape
    T = 1
    layers, keep = _layers(wl, wl.layers)
    x0 = L.make_activations(wl, T)
    # per-layer entry point (three launches a layer), route of every layer kept
    buf1 = L.LayerBuffers(s, T)
    xr = x0.clone()
    ref_ids = []
    for lay in layers:
        L.decode_chain_step(buf1, xr, [lay], EPS)
        ref_ids.append(buf1.ids.clone())
    ref_ids = torch.stack(ref_ids)
    # one call for the whole stack
    buf = L.LayerBuffers(s, T)
    x = x0.clone()
    ids = torch.empty((wl.layers, T, s.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((wl.layers, T, s.top_k), dtype=torch.float32, device="cuda")
    L.decode_chain(buf, x, layers, EPS, ids, w)
    torch.cuda.synchronize()
    assert torch.equal(ids, ref_ids)
    assert_close(x.cpu().numpy(), xr.cpu().numpy().astype(np.float64), REL_L2_GEMV,
                 "chain vs per-layer, 38 layers")
    # rerun: bit-identical
    x2 = x0.clone()
    L.decode_chain(buf, x2, layers, EPS)
    torch.cuda.synchronize()
    assert torch.equal(x2, x)


@pytest.mark.parametrize("T", [1, 16])
def test_chain_graph_replay(T):
    # T = 16: the batched kernels, whose down stage counts finished workgroups in the
    # workspace (cleared by the gate/up launch and by the workgroup that combines)
    wl = XING4_DECODE
    s = wl.shape
    layers, keep = _layers(wl, 6)
    arr = M.make_layers([(bank, wr, bias) for (wr, bias, bank) in layers])
    x0 = L.make_activations(wl, T)
    buf = L.LayerBuffers(s, T)
    eager = x0.clone()
    L.decode_chain(buf, eager, arr, EPS)
    torch.cuda.synchronize()
    xg = x0.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.decode_chain(buf, xg, arr, EPS)             # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        L.decode_chain(buf, xg, arr, EPS)
    for _ in range(3):
        xg.copy_(x0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xg, eager)
        torch.cuda.synchronize()
        junk = torch.randn(1000, device="cuda").sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        del junk


def test_chain_sixteen_tokens_equals_per_layer_path():
    # 16 tokens of the 3584/1024 shape: the stack call equals the per-layer calls bit for bit
    wl = XING4_DECODE
    s = wl.shape
    T = 16
    layers, keep = _layers(wl, 2)
    x0 = L.make_activations(wl, T)
    buf = L.LayerBuffers(s, T)
    x = x0.clone()
    L.decode_chain(buf, x, layers, EPS)
    buf2 = L.LayerBuffers(s, T)
    xr = x0.clone()
    L.decode_chain_step(buf2, xr, layers, EPS)
    torch.cuda.synchronize()
    assert torch.equal(x, xr)


def test_chain_argument_checks():
    wl = XING4_DECODE
    s = wl.shape
    layers, keep = _layers(wl, 1)
    buf = L.LayerBuffers(s, 16)
    x = L.make_activations(wl, 16)
    arr = M.make_layers([(bank, wr, bias) for (wr, bias, bank) in layers])
    desc17 = L.desc_of(s, 17)
    with pytest.raises(M.MoeError) as ei:
        M.moe_decode_chain(desc17, arr, 1, x, 17, EPS, None, None, buf.ws, buf.ws_bytes)
    assert ei.value.status == M.MOE_ERR_SHAPE
    with pytest.raises(M.MoeError) as ei:
        M.moe_decode_chain(buf.desc, arr, 65, x, 1, EPS, None, None, buf.ws, buf.ws_bytes)
    assert ei.value.status == M.MOE_ERR_SHAPE
    ids = torch.empty((1, 1, s.top_k), dtype=torch.int32, device="cuda")
    with pytest.raises(M.MoeError) as ei:
        M.moe_decode_chain(buf.desc, arr, 1, x, 1, EPS, ids, None, buf.ws, buf.ws_bytes)
    assert ei.value.status == M.MOE_ERR_NULL
    with pytest.raises(M.MoeError) as ei:
        M.moe_decode_chain(buf.desc, arr, 1, x, 1, EPS, None, None, buf.ws, 1024)
    assert ei.value.status == M.MOE_ERR_WORKSPACE
