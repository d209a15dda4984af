"""Pins of the oracle's MoE layer against invariants, closed forms, printed values and a
scalar brute force.  Pages: PocketLLM "Xing4.0-29B-A4B" (sections "Overview", "Without a
server", "Where the detail is"); "Running Qwen Flash-Next NVFP4 in vLLM" (route validation).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import iq4nl, moe, bruteforce


def _rand_layer(rng, H, F, E, k, gating=moe.SIGMOID, renorm=1, same_experts=False, T=5,
                bias=False):
    desc = moe.Desc(H, F, E, k, 1, gating, renorm)
    mats = []
    for e in range(E + 1):
        if same_experts and 0 < e < E:
            mats.append(mats[0])
            continue
        mats.append(tuple((rng.standard_normal(s) * 0.05).astype(np.float32)
                          for s in [(F, H), (F, H), (H, F)]))
    bank = moe.build_bank(mats, desc)
    stride = bank.size // (E + 1)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(E) * 0.5).astype(np.float32) if bias else None
    return desc, bank, stride, x, wr, b


# ---- selection -------------------------------------------------------------------------

def _full_sort(row, k):
    key = []
    for e, v in enumerate(row):
        if np.isnan(v):
            key.append((1, 0.0, e))
        else:
            key.append((0, -(v + 0.0), e))
    return [kk[2] for kk in sorted(key)][:k]


@pytest.mark.parametrize("E,k", [(8, 2), (64, 4), (384, 6), (512, 10), (7, 7)])
def test_topk_equals_full_sort(E, k):
    rng = np.random.default_rng(E * 31 + k)
    l = rng.standard_normal((40, E))
    l[::3] = np.round(l[::3] * 2) / 2                      # many exact ties
    l[1, :5] = np.inf
    l[2, -4:] = -np.inf
    l[4, ::2] = np.nan
    l[5, :] = 0.0
    l[5, 1::2] = -0.0                                      # +0/-0 tie: lower index wins
    ids = moe.select_topk(l, k)
    for t in range(40):
        assert list(ids[t]) == _full_sort(l[t], k), t


def test_topk_nan_lowest_and_permutation_when_k_equals_E():
    l = np.array([[np.nan, 1.0, np.nan, -np.inf, 0.5]])
    assert list(moe.select_topk(l, 5)[0]) == [1, 4, 3, 0, 2]


def test_sigmoid_weights_positive_sum_one():
    rng = np.random.default_rng(7)
    l = rng.standard_normal((100, 64)) * 3
    ids = moe.select_topk(l, 4)
    w = moe.gating_weights(l, ids, moe.SIGMOID, 1)
    assert np.all(w > 0) and np.allclose(w.sum(1), 1.0, atol=1e-15)
    s = 1 / (1 + np.exp(-np.take_along_axis(l, ids.astype(int), 1)))
    assert np.allclose(w, s / s.sum(1, keepdims=True))
    # selection on the logits equals selection on the (monotone) scores
    assert np.array_equal(ids, moe.select_topk(1 / (1 + np.exp(-l)), 4))


def test_softmax_weights_closed_form():
    l = np.array([[0.0, np.log(2.0), np.log(3.0), np.log(4.0)]])
    ids = moe.select_topk(l, 2)
    assert list(ids[0]) == [3, 2]
    w = moe.gating_weights(l, ids, moe.SOFTMAX, 0)
    assert np.allclose(w, [[0.4, 0.3]], atol=1e-15)
    w = moe.gating_weights(l, ids, moe.SOFTMAX, 1)
    assert np.allclose(w, [[4 / 7, 3 / 7]], atol=1e-15)


# ---- sanitisation ----------------------------------------------------------------------

def test_sanitize_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "p4_route_sanitize.json")))
    ids, w, n = moe.sanitize(np.array(g["ids_in"]), np.array(g["weights_in"]), g["n_experts"])
    assert list(ids) == g["ids_out"] and list(w) == g["weights_out"] and n == 2


# ---- permutation -----------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E", [(1, 4, 64), (16, 4, 64), (300, 6, 16), (37, 10, 512),
                                   (4, 2, 8), (0, 3, 5)])
def test_permutation_properties(T, k, E):
    rng = np.random.default_rng(T + k + E)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T:
        ids[0, :] = 0                           # duplicates inside one token (sanitised pads)
    off, sp, slot = moe.permute(ids, E, 1)
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and off[E] == T * k
    assert off[E + 1] == T * k + T
    assert sorted(sp.tolist()) == list(range(T * k))
    assert np.array_equal(slot[sp], np.arange(T * k))
    # brute force: pairs ordered by (expert, pair id)
    bf = sorted(range(T * k), key=lambda p: (int(ids.reshape(-1)[p]), p))
    assert sp.tolist() == bf
    for e in range(E):
        seg = sp[off[e]:off[e + 1]]
        assert np.all(ids.reshape(-1)[seg] == e)


# ---- combine, norm, bytes --------------------------------------------------------------

def test_combine_fixed_order_and_residual():
    T, k, H = 3, 2, 4
    ids = np.array([[1, 0], [0, 1], [1, 1]])
    off, sp, slot = moe.permute(ids, 2, 1)
    o = np.arange((T * k + T) * H, dtype=np.float64).reshape(-1, H)
    w = np.array([[0.25, 0.75], [1.0, 0.0], [0.5, 0.5]])
    res = np.ones((T, H))
    y = moe.combine(o, slot, w, T, k, 1, residual=res)
    for t in range(T):
        exp = res[t] + o[T * k + t]
        for j in range(k):
            exp = exp + w[t, j] * o[slot[t * k + j]]
        assert np.allclose(y[t], exp)


def test_rmsnorm_closed_form():
    x = np.array([[3.0, 4.0], [0.0, 0.0], [1e3, -1e3]])
    y = moe.rmsnorm(x, 1e-6)
    assert np.allclose(y[0], np.array([3.0, 4.0]) / np.sqrt(12.5 + 1e-6))
    assert np.all(y[1] == 0.0)
    assert np.allclose(np.mean(y[2] ** 2), 1e6 / (1e6 + 1e-6))


def test_decode_bytes_match_page(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "p1_decode_bytes.json")))
    desc = moe.Desc(g["hidden"], g["ffn"], g["n_experts"], g["top_k"], g["n_shared"])
    routed, shared = moe.decode_bytes_per_token(desc, g["moe_layers"])
    assert routed == 4 * 6_193_152 * 38 and shared == 6_193_152 * 38
    nd = g["printed_decimals"]
    assert round(routed / 2 ** 30, nd) == g["routed_gib"]
    assert round(shared / 2 ** 30, nd) == g["shared_gib"]


# ---- the layer -------------------------------------------------------------------------

@pytest.mark.parametrize("H,F,E,k,gating,renorm,bias", [
    (32, 32, 4, 2, moe.SIGMOID, 1, False),
    (64, 32, 8, 3, moe.SOFTMAX, 0, True),
    (32, 64, 6, 1, moe.SOFTMAX, 1, False),
    (64, 64, 8, 8, moe.SIGMOID, 0, True),
])
def test_layer_equals_scalar_bruteforce(H, F, E, k, gating, renorm, bias):
    rng = np.random.default_rng(H + F + E + k)
    desc, bank, stride, x, wr, b = _rand_layer(rng, H, F, E, k, gating, renorm, T=3, bias=bias)
    y = moe.moe_layer(x, wr, b, bank, stride, desc)
    ref = np.asarray(bruteforce.layer(x.tolist(), wr.tolist(), None if b is None else b.tolist(),
                                      bank.tolist(), stride, H, F, E, k, gating, renorm))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_tiny_config_layer_equals_bruteforce():
    # the 4-token, hidden 256, 8-expert top-2 sigmoid shape
    import synth.generator as G
    from synth.configs import TINY
    s = TINY.shape
    desc = moe.Desc(s.hidden, s.ffn, s.n_experts, s.top_k, s.n_shared, s.gating, s.renormalize)
    mats = [tuple(G.expert_matrix(TINY, 0, e, w) for w in ("gate", "up", "down"))
            for e in range(s.n_experts + 1)]
    bank = moe.build_bank(mats, desc)
    x = G.activations(TINY, 2)
    wr = G.router_weight(TINY, 0)
    y = moe.moe_layer(x, wr, None, bank, s.expert_bytes, desc)
    ref = np.asarray(bruteforce.layer(x.tolist(), wr.tolist(), None, bank.tolist(),
                                      s.expert_bytes, s.hidden, s.ffn, s.n_experts, s.top_k,
                                      s.gating, s.renormalize))
    assert np.allclose(y, ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("gating,renorm", [(moe.SIGMOID, 1), (moe.SOFTMAX, 0), (moe.SOFTMAX, 1)])
def test_grouped_equals_dense_masked(gating, renorm):
    rng = np.random.default_rng(11 + gating + renorm)
    desc, bank, stride, x, wr, b = _rand_layer(rng, 64, 64, 8, 3, gating, renorm, T=20, bias=True)
    assert np.allclose(moe.moe_layer(x, wr, b, bank, stride, desc),
                       moe.moe_layer_dense(x, wr, b, bank, stride, desc), rtol=1e-12, atol=1e-12)


def test_softmax_k_equals_E_is_dense_mixture():
    rng = np.random.default_rng(12)
    E = 6
    desc, bank, stride, x, wr, b = _rand_layer(rng, 64, 32, E, E, moe.SOFTMAX, 0, T=7)
    y = moe.moe_layer(x, wr, b, bank, stride, desc)
    l = x.astype(np.float64) @ wr.astype(np.float64).T
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = np.zeros_like(y)
    raw = bank.tolist()
    for e in range(E + 1):
        # each expert's FFN from the scalar-loop twin, weighted by its softmax probability
        out = np.asarray([bruteforce._ffn(raw, e * stride, 64, 32, [float(v) for v in xt])
                          for xt in x])
        ref += (p[:, e:e + 1] if e < E else 1.0) * out
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_identical_experts_collapse():
    rng = np.random.default_rng(13)
    E = 8
    desc, bank, stride, x, wr, b = _rand_layer(rng, 64, 64, E, 3, moe.SIGMOID, 1,
                                               same_experts=True, T=9, bias=True)
    y = moe.moe_layer(x, wr, b, bank, stride, desc)
    xd = x.astype(np.float64)
    wg, wu, wd = moe.expert_weights(bank, stride, 0, desc)
    f = moe.expert_down(wd, moe.expert_gate_up(wg, wu, xd))
    wg, wu, wd = moe.expert_weights(bank, stride, E, desc)
    sh = moe.expert_down(wd, moe.expert_gate_up(wg, wu, xd))
    assert np.allclose(y, f + sh, rtol=1e-12, atol=1e-12)


def test_invalid_routes_contribute_nothing():
    rng = np.random.default_rng(14)
    desc, bank, stride, x, wr, b = _rand_layer(rng, 32, 32, 4, 2, T=3)
    ids = np.array([[1, -1], [7, 2], [3, 3]])
    w = np.array([[0.6, 0.4], [0.5, 0.5], [0.2, 0.8]])
    y, parts = moe.moe_layer(x, wr, b, bank, stride, desc, ids=ids, weights=w,
                             return_parts=True)
    assert parts["n_invalid"] == 2
    y2 = moe.moe_layer(x, wr, b, bank, stride, desc, ids=np.array([[1, 0], [0, 2], [3, 3]]),
                       weights=np.array([[0.6, 0.0], [0.0, 0.5], [0.2, 0.8]]))
    assert np.allclose(y, y2)


def test_chain_one_layer_and_two_layers():
    rng = np.random.default_rng(15)
    desc, bank, stride, x, wr, b = _rand_layer(rng, 32, 32, 4, 2, T=2)
    y1 = moe.chain(x, [(wr, b, bank, stride)], desc)
    assert np.allclose(y1, x + moe.moe_layer(moe.rmsnorm(x), wr, b, bank, stride, desc))
    y2 = moe.chain(x, [(wr, b, bank, stride)] * 2, desc)
    assert np.allclose(y2, y1 + moe.moe_layer(moe.rmsnorm(y1), wr, b, bank, stride, desc))


def _scalar_rmsnorm(row, eps):
    """x / sqrt(mean(x^2) + eps) of one row, written as loops."""
    ss = 0.0
    for v in row:
        ss += v * v
    r = 1.0 / math.sqrt(ss / len(row) + eps)
    return [v * r for v in row]


@pytest.mark.parametrize("eps", [1e-6, 0.25])
def test_chain_against_scalar_twin_three_distinct_layers(eps):
    """The chain glue (weight-free RMSNorm on each layer's input, residual of the un-normalised
    x, layers in order) against the scalar-loop twin of the layer, chained by hand over three
    layers with different weights, routers and biases.  eps = 0.25 on small activations makes
    the norm's epsilon visible; a wrong eps, norm placement, residual or layer order fails."""
    rng = np.random.default_rng(16)
    H, F, E, k, T = 64, 32, 4, 2, 3
    layers = []
    for l in range(3):
        desc, bank, stride, _, wr, b = _rand_layer(rng, H, F, E, k, T=T, bias=(l != 1))
        layers.append((wr, b, bank, stride))
    x = (rng.standard_normal((T, H)) * 0.3).astype(np.float32)
    got = moe.chain(x, layers, desc, eps)
    ref = []
    for t in range(T):
        xt = [float(v) for v in x[t]]
        for (wr, b, bank, stride) in layers:
            xn = _scalar_rmsnorm(xt, eps)
            y = bruteforce.layer([xn], wr.tolist(), None if b is None else b.tolist(),
                                 bank.tolist(), stride, H, F, E, k, desc.gating,
                                 desc.renormalize)[0]
            xt = [xt[i] + y[i] for i in range(H)]
        ref.append(xt)
    assert np.allclose(got, np.asarray(ref), rtol=1e-12, atol=1e-12)
    # the layers do not commute: the reversed stack gives a different result
    rev = moe.chain(x, layers[::-1], desc, eps)
    assert not np.allclose(rev, got, rtol=1e-6, atol=1e-6)
