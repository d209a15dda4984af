"""Shared helpers of the parity tests: oracle-side inputs from the seeded generator, and the
comparison metrics with the tolerances of the two GPU paths.

Tolerances (written here, used by every parity test):
  * integer results (ids, permutation, invalid count, IQ4_NL bytes, dequantised weights):
    bit-exact;
  * fp32 GEMV path (decode): relative L2 error <= 1e-4 and max-abs <= 2e-2 x output RMS;
  * bf16 MFMA path (prefill): relative L2 error <= 5e-3 and max-abs <= 2e-2 x output RMS.
"""
import numpy as np

from oracle import iq4nl, moe as omoe
from synth import generator as G

REL_L2_GEMV = 1e-4
REL_L2_MFMA = 5e-3
MAXABS_FRAC = 2e-2


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, rel, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    mx = float(np.max(np.abs(got - ref))) if got.size else 0.0
    assert r <= rel, f"{what}: rel-L2 {r:.3e} > {rel:.1e}"
    assert mx <= MAXABS_FRAC * rms, f"{what}: max-abs {mx:.3e} > {MAXABS_FRAC} x rms {rms:.3e}"
    return r, mx / max(rms, 1e-300)


def desc_of(shape):
    return omoe.Desc(shape.hidden, shape.ffn, shape.n_experts, shape.top_k, shape.n_shared,
                     shape.gating, shape.renormalize)


_EXPERT_CACHE = {}


def oracle_expert_bytes(wl, layer, e):
    """One expert's IQ4_NL bytes, generated on the host and quantised by the oracle (cached)."""
    key = (wl.name, wl.cfg_id, layer, e)
    if key not in _EXPERT_CACHE:
        if len(_EXPERT_CACHE) > 64:
            _EXPERT_CACHE.clear()
        _EXPERT_CACHE[key] = np.concatenate(
            [iq4nl.quantize_matrix(G.expert_matrix(wl, layer, e, w)) for w in ("gate", "up", "down")])
    return _EXPERT_CACHE[key]


def oracle_bank(wl, layer, experts):
    """Bank bytes (numpy) with the listed experts quantised by the oracle; others zero."""
    s = wl.shape
    stride = s.expert_bytes
    bank = np.zeros(stride * (s.n_experts + s.n_shared), np.uint8)
    for e in sorted(set(int(v) for v in experts)):
        bank[e * stride:(e + 1) * stride] = oracle_expert_bytes(wl, layer, e)
    return bank, stride


def oracle_layer(wl, layer, x, return_parts=False, bias=None, w_router=None):
    """The oracle's layer on host inputs x [T, H] (fp32) with the workload's weights."""
    s = wl.shape
    desc = desc_of(s)
    wr = G.router_weight(wl, layer) if w_router is None else w_router
    b = G.zipf_bias(wl, layer) if (bias is None and wl.zipf_s is not None) else bias
    _, ids, _ = omoe.route(x, wr, b, desc)
    experts = set(ids.reshape(-1).tolist()) | {s.n_experts}
    bank, stride = oracle_bank(wl, layer, experts)
    return omoe.moe_layer(x, wr, b, bank, stride, desc, return_parts=return_parts)


U_BF16 = 2.0 ** -9        # unit roundoff of round-to-nearest-even bf16
SILU_LIPSCHITZ = 1.0999   # max |d silu / dg| (attained near g = 2.4)


def _gamma(K):
    u = 2.0 ** -24
    return K * u / (1 - K * u)


def bf16_dot_bound(a_abs, K):
    """Bound on |fp32-accumulated sum of bf16(a_i) * bf16(b_i) - sum a_i b_i| given
    a_abs = sum |a_i b_i|: each operand rounded once (RNE), products exact in fp32."""
    e = 2 * U_BF16 + U_BF16 ** 2
    return (e + _gamma(K) * (1 + U_BF16) ** 2) * a_abs


def gate_up_bf16_bound(wg, wu, x):
    """Elementwise bound on |h_gpu - h| for h = silu(W_g x) * (W_u x) computed from bf16 x and
    bf16 weights with fp32 accumulation, SwiGLU in fp32 and h rounded to bf16 at the end."""
    x = np.asarray(x, np.float64)
    K = x.shape[1]
    g = x @ wg.T
    u = x @ wu.T
    dg = bf16_dot_bound(np.abs(x) @ np.abs(wg).T, K)
    du = bf16_dot_bound(np.abs(x) @ np.abs(wu).T, K)
    sg = g / (1 + np.exp(-g))
    pre = SILU_LIPSCHITZ * dg * (np.abs(u) + du) + np.abs(sg) * du
    h = np.abs(sg * u)
    return pre + U_BF16 * (h + pre) + 1e-6 * h


def down_bf16_bound(wd, h):
    h = np.asarray(h, np.float64)
    return bf16_dot_bound(np.abs(h) @ np.abs(wd).T, h.shape[1])


def assert_within_bound(got, ref, bound, rel, what=""):
    """rel-L2 <= rel and |got - ref| <= bound elementwise."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    assert r <= rel, f"{what}: rel-L2 {r:.3e} > {rel:.1e}"
    excess = np.abs(got - ref) - bound
    assert np.all(excess <= 0), f"{what}: {int(np.sum(excess > 0))} elements beyond the bound"
    return r


def topk_gap(logits, k):
    """Per token: gap between the k-th and (k+1)-th largest logit (inf when k == E)."""
    l = np.sort(np.asarray(logits, np.float64), axis=1)[:, ::-1]
    if l.shape[1] <= k:
        return np.full(l.shape[0], np.inf)
    return l[:, k - 1] - l[:, k]


def logit_error_bound(x, wr, bias=None):
    """Forward error bound of an fp32 dot product with fp32 accumulation, per logit:
    gamma_K * sum |x_i w_i| (+ rounding of the bias add), gamma_K = K u / (1 - K u)."""
    x = np.abs(np.asarray(x, np.float64))
    w = np.abs(np.asarray(wr, np.float64))
    K = x.shape[1] + 1
    u = 2.0 ** -24
    g = K * u / (1 - K * u)
    mag = x @ w.T
    if bias is not None:
        mag = mag + np.abs(np.asarray(bias, np.float64))[None, :]
    return g * mag
