"""Pins of the elementwise error bounds that judge the grouped GEMM's per-stage outputs
(``tests/helpers.py``: ``gate_up_bf16_bound``, ``down_bf16_bound``).

A bound that the GPU result must meet is only worth something if (1) it holds for the
arithmetic the kernel performs and (2) it is not so loose that any result passes.  Both are
checked here, on the CPU, against a numpy emulation of that arithmetic (the bf16 roundings
read from "bf16 MFMA compute" for the prefill chunk: x -> bf16 RNE, each weight d * c -> bf16
RNE, products exact in fp32, fp32 accumulation, SwiGLU in fp32, h -> bf16 RNE), with the
accumulation done in three different orders (sequential, pairwise, and partial sums of 32
products added in turn, as a 16x16x32 matrix instruction does).  The expected values are the
oracle's fp64 products of the dequantised IQ4_NL weights.
"""
import numpy as np
import pytest

from oracle import iq4nl, moe as omoe

from .helpers import down_bf16_bound, gate_up_bf16_bound


def _bf16(a):
    """fp32 -> bf16 (round to nearest even), returned as fp32 values."""
    b = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = ((b >> 16) & 1) + 0x7FFF
    return (((b + r) >> 16) << 16).astype(np.uint32).view(np.float32)


def _acc(a, w, order):
    """fp32 sum over k of a[m, k] * w[n, k] (operands already bf16 values in fp32, so every
    product is exact in fp32), additions rounded to fp32 in the given order."""
    p = (a[:, None, :].astype(np.float32) * w[None, :, :].astype(np.float32))   # exact
    K = p.shape[-1]
    if order == "sequential":
        s = np.zeros(p.shape[:2], np.float32)
        for k in range(K):
            s = (s + p[:, :, k]).astype(np.float32)
        return s
    if order == "pairwise":
        q = p
        while q.shape[-1] > 1:
            if q.shape[-1] % 2:
                q = np.concatenate([q, np.zeros(q.shape[:2] + (1,), np.float32)], axis=-1)
            q = (q[:, :, 0::2] + q[:, :, 1::2]).astype(np.float32)
        return q[:, :, 0]
    # blocks of 32 products summed sequentially, the partials added in turn
    s = np.zeros(p.shape[:2], np.float32)
    for k0 in range(0, K, 32):
        part = np.zeros(p.shape[:2], np.float32)
        for k in range(k0, min(K, k0 + 32)):
            part = (part + p[:, :, k]).astype(np.float32)
        s = (s + part).astype(np.float32)
    return s


def _weights(rng, rows, cols):
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    return iq4nl.dequantize_matrix(iq4nl.quantize_matrix(w), rows, cols)   # fp64, exact d*c


ORDERS = ("sequential", "pairwise", "blocks32")


@pytest.mark.parametrize("K", [256, 1024])
def test_gate_up_bound_holds(K):
    rng = np.random.default_rng(K)
    m, n = 24, 40
    x = rng.standard_normal((m, K)).astype(np.float32)
    wg, wu = _weights(rng, n, K), _weights(rng, n, K)
    ref = omoe.expert_gate_up(wg, wu, x.astype(np.float64))
    bound = gate_up_bf16_bound(wg, wu, x)
    xb = _bf16(x)
    wgb, wub = _bf16(wg.astype(np.float32)), _bf16(wu.astype(np.float32))
    for order in ORDERS:
        g = _acc(xb, wgb, order)
        u = _acc(xb, wub, order)
        sg = (g / (np.float32(1) + np.exp(-g, dtype=np.float32))).astype(np.float32)
        h = _bf16((sg * u).astype(np.float32)).astype(np.float64)
        err = np.abs(h - ref)
        assert np.all(err <= bound), (order, float(np.max(err / bound)))


@pytest.mark.parametrize("K", [128, 1024])
def test_down_bound_holds(K):
    rng = np.random.default_rng(K + 1)
    m, n = 24, 40
    h = (rng.standard_normal((m, K)) * 0.7).astype(np.float32)
    wd = _weights(rng, n, K)
    ref = omoe.expert_down(wd, h.astype(np.float64))
    bound = down_bf16_bound(wd, h)
    for order in ORDERS:
        o = _acc(_bf16(h), _bf16(wd.astype(np.float32)), order).astype(np.float64)
        err = np.abs(o - ref)
        assert np.all(err <= bound), (order, float(np.max(err / bound)))


def _aligned_operands(K):
    """Operands whose bf16 roundings all err the same way, by almost a unit roundoff: every
    activation just below the midpoint between bf16 1 and its successor (rounds down), and
    every weight 127 d with the fp16 scale d whose product 127 d loses the most to RNE."""
    best, best_d = 0.0, None
    for bits in range(0x1C00, 0x2400):                       # d around 2^-8 .. 2^-7
        d = float(np.array([bits], np.uint16).view(np.float16)[0])
        w = 127.0 * d                                         # exact
        r = float(_bf16(np.float32(w))[()])
        rel = (w - r) / w
        if rel > best:
            best, best_d = rel, d
    h = np.full((1, K), 1.0 + 2.0 ** -8 - 2.0 ** -20, np.float32)
    wd = np.full((2, K), 127.0 * best_d)
    return h, wd, best


@pytest.mark.parametrize("K", [128, 1024])
def test_dot_bound_is_attained_by_aligned_roundings(K):
    """The bound is tight: with every rounding of both operands pushing the same way (by
    almost 2^-8 each) the emulated error reaches at least 90% of it, in every order.  A bound
    built on a smaller unit roundoff (2^-9) or on one rounded operand fails this input."""
    h, wd, rel_w = _aligned_operands(K)
    assert rel_w > 0.9 * 2.0 ** -8
    ref = omoe.expert_down(wd, h.astype(np.float64))
    bound = down_bf16_bound(wd, h)
    for order in ORDERS:
        o = _acc(_bf16(h), _bf16(wd.astype(np.float32)), order).astype(np.float64)
        err = np.abs(o - ref)
        assert np.all(err <= bound), order
        assert np.all(err >= 0.9 * bound), (order, float(np.min(err / bound)))
