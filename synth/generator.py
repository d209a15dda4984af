"""Seeded, addressable synthetic inputs (host side, numpy).

This module draws the random inputs of the workloads: activations, router weights, router
bias and the fp32 expert weights that are later quantised.  It holds none of the method's
arithmetic.  The same definition is implemented for the GPU in ``synth/csrc/synth.hip``;
both produce bit-identical fp32 values, because every step is integer arithmetic followed
by one IEEE fp32 multiply.

Counter-based generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011): a 10-round SP network on a 128-bit counter under a
64-bit key, each round two 32x32->64 multiplies (constants 0xD2511F53, 0xCD9E8D57) and a
Weyl key schedule (0x9E3779B9, 0xBB67AE85).

Counter layout for element ``i`` of a tensor::

    counter = (i mod 2^32, i div 2^32, (layer << 16) | expert, (cfg_id << 8) | tensor)
    key     = (seed, 0x4D6F4531)

Normal deviates: an Irwin-Hall sum of the eight 16-bit halves of one Philox output,
centred and scaled, ``z = (sum16 - 262140) * (sigma / sd)`` with
``sd = sqrt(8 * (65536^2 - 1) / 12)``.  Its variance is sigma^2, its range is
+-4.90 sigma and its excess kurtosis -0.15: a close stand-in for N(0, sigma) that needs
no transcendental function, so host and device agree to the bit.
"""
import math
import numpy as np

from .configs import Workload

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
KEY1 = 0x4D6F4531
_MASK = np.uint64(0xFFFFFFFF)

# tensor tags (low byte of counter word 3)
T_X = 0
T_ROUTER = 1
T_GATE = 2
T_UP = 3
T_DOWN = 4
T_ZIPF = 5

IH_CENTRE = 262140                      # 8 * 32767.5
IH_SD = math.sqrt(8.0 * (65536.0 ** 2 - 1.0) / 12.0)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on arrays of 32-bit counters; returns 4 uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    s32 = np.uint64(32)
    for r in range(10):
        if r:
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
        p0 = c0 * m0
        p1 = c2 * m1
        n0 = (p1 >> s32) ^ c1 ^ np.uint64(k0)
        n2 = (p0 >> s32) ^ c3 ^ np.uint64(k1)
        c1 = p1 & _MASK
        c3 = p0 & _MASK
        c0 = n0
        c2 = n2
    return (c0.astype(np.uint32), c1.astype(np.uint32),
            c2.astype(np.uint32), c3.astype(np.uint32))


def stream_words(cfg_id: int, layer: int, expert: int, tensor: int):
    assert 0 <= layer < 65536 and 0 <= expert < 65536
    assert 0 <= cfg_id < (1 << 24) and 0 <= tensor < 256
    return (layer << 16) | expert, (cfg_id << 8) | tensor


def ih_scale(sigma: float) -> np.float32:
    """fp32 factor that maps the centred Irwin-Hall integer to a deviate of std sigma."""
    return np.float32(sigma / IH_SD)


def normal_f32(seed: int, cfg_id: int, layer: int, expert: int, tensor: int,
               start: int, count: int, sigma: float, chunk: int = 1 << 18) -> np.ndarray:
    """Elements ``start .. start+count-1`` of one tensor stream, as fp32."""
    c2, c3 = stream_words(cfg_id, layer, expert, tensor)
    scale = ih_scale(sigma)
    out = np.empty(count, dtype=np.float32)
    for off in range(0, count, chunk):
        n = min(chunk, count - off)
        idx = np.arange(start + off, start + off + n, dtype=np.uint64)
        w = philox4x32_10(idx & _MASK, idx >> np.uint64(32), np.full(n, c2, np.uint64),
                          np.full(n, c3, np.uint64), seed, KEY1)
        s = np.zeros(n, dtype=np.int64)
        for word in w:
            word = word.astype(np.int64)
            s += (word & 0xFFFF) + (word >> 16)
        z = (s - IH_CENTRE).astype(np.float32)        # exact: |z| < 2^24
        out[off:off + n] = z * scale                   # one IEEE fp32 rounding
    return out


# ---- tensors of a workload -------------------------------------------------------------

def activations(wl: Workload, n_tokens: int, token0: int = 0) -> np.ndarray:
    """x [n_tokens, H] fp32, rows token0 .. token0+n_tokens-1 of the activation stream."""
    H = wl.shape.hidden
    v = normal_f32(wl.seed, wl.cfg_id, 0, 0, T_X, token0 * H, n_tokens * H, wl.x_sigma)
    return v.reshape(n_tokens, H)


def router_weight(wl: Workload, layer: int) -> np.ndarray:
    """W_r [E, H] fp32 of one layer."""
    E, H = wl.shape.n_experts, wl.shape.hidden
    v = normal_f32(wl.seed, wl.cfg_id, layer, 0, T_ROUTER, 0, E * H, wl.router_sigma)
    return v.reshape(E, H)


def expert_matrix(wl: Workload, layer: int, expert: int, which: str,
                  row0: int = 0, n_rows: int = None) -> np.ndarray:
    """fp32 weights of one expert matrix, stored [out, in]; rows row0 .. row0+n_rows-1.

    which: 'gate' [F, H], 'up' [F, H], 'down' [H, F].  Expert index E is the shared expert.
    """
    s = wl.shape
    tensor = {"gate": T_GATE, "up": T_UP, "down": T_DOWN}[which]
    rows, cols = (s.ffn, s.hidden) if which != "down" else (s.hidden, s.ffn)
    if n_rows is None:
        n_rows = rows - row0
    v = normal_f32(wl.seed, wl.cfg_id, layer, expert, tensor, row0 * cols, n_rows * cols,
                   wl.weight_sigma)
    return v.reshape(n_rows, cols)


def zipf_bias(wl: Workload, layer: int) -> np.ndarray:
    """Per-expert router bias that skews expert loads: b_e = ln(E * p_{r(e)}), fp32.

    p_r = r^-s / sum_{r'=1..E} r'^-s (Zipf law with exponent s); the rank r(e) of expert e
    comes from a Fisher-Yates shuffle of 1..E driven by the Philox stream (layer, 0xFFFF,
    T_ZIPF).  A uniform load gives b = 0.  Returns zeros when the workload has no skew.
    """
    E = wl.shape.n_experts
    if wl.zipf_s is None:
        return np.zeros(E, dtype=np.float32)
    c2, c3 = stream_words(wl.cfg_id, layer, 0xFFFF, T_ZIPF)
    ranks = list(range(1, E + 1))
    idx = np.arange(E, dtype=np.uint64)
    r0, _, _, _ = philox4x32_10(idx, np.zeros(E, np.uint64), np.full(E, c2, np.uint64),
                                np.full(E, c3, np.uint64), wl.seed, KEY1)
    for i in range(E - 1, 0, -1):
        j = (int(r0[i]) * (i + 1)) >> 32
        ranks[i], ranks[j] = ranks[j], ranks[i]
    harm = sum(r ** -wl.zipf_s for r in range(1, E + 1))
    b = [math.log(E * (r ** -wl.zipf_s) / harm) for r in ranks]
    return np.asarray(b, dtype=np.float32)
