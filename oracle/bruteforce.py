"""Scalar-loop twin of the MoE layer for tiny shapes (pure Python, no numpy arithmetic).

Used only as a pin of ``oracle.moe``: every sum is an explicit loop, every block is
unpacked byte by byte, selection is a full sort, and no permutation is built -- each
token walks its own k experts and the shared expert.  It follows the same pages as
``oracle.moe`` (see that module's header).
"""
import math
import struct

from .iq4nl import CODEBOOK


def _fp16(lo: int, hi: int) -> float:
    return struct.unpack("<e", bytes([lo, hi]))[0]


def _row(bank, off: int, cols: int):
    """Dequantise one stored row of ``cols`` weights starting at byte ``off``."""
    out = []
    for b in range(cols // 32):
        blk = bank[off + 18 * b: off + 18 * b + 18]
        d = _fp16(int(blk[0]), int(blk[1]))
        w = [0.0] * 32
        for j in range(16):
            byte = int(blk[2 + j])
            w[j] = d * CODEBOOK[byte & 15]
            w[j + 16] = d * CODEBOOK[byte >> 4]
        out.extend(w)
    return out


def _ffn(bank, base: int, H: int, F: int, x):
    nbh, nbf = H // 32, F // 32
    up0 = base + F * nbh * 18
    dn0 = up0 + F * nbh * 18
    h = []
    for f in range(F):
        wg = _row(bank, base + f * nbh * 18, H)
        wu = _row(bank, up0 + f * nbh * 18, H)
        g = sum(wg[i] * x[i] for i in range(H))
        u = sum(wu[i] * x[i] for i in range(H))
        h.append(g / (1.0 + math.exp(-g)) * u)
    o = []
    for r in range(H):
        wd = _row(bank, dn0 + r * nbf * 18, F)
        o.append(sum(wd[i] * h[i] for i in range(F)))
    return o


def layer(x, w_router, bias, bank, stride, H, F, E, k, gating, renormalize):
    """y for each token of x (lists of floats)."""
    ys = []
    for t in range(len(x)):
        xt = [float(v) for v in x[t]]
        logits = []
        for e in range(E):
            s = sum(float(w_router[e][i]) * xt[i] for i in range(H))
            logits.append(s + (float(bias[e]) if bias is not None else 0.0))
        order = sorted(range(E), key=lambda e: (-logits[e], e))
        ids = order[:k]
        if gating == 0:
            w = [1.0 / (1.0 + math.exp(-logits[e])) for e in ids]
        else:
            m = max(logits)
            ex = [math.exp(v - m) for v in logits]
            z = sum(ex)
            w = [ex[e] / z for e in ids]
        if renormalize:
            tot = sum(w)
            w = [v / tot for v in w]
        y = [0.0] * H
        for j, e in enumerate(ids):
            o = _ffn(bank, e * stride, H, F, xt)
            for i in range(H):
                y[i] += w[j] * o[i]
        o = _ffn(bank, E * stride, H, F, xt)
        for i in range(H):
            y[i] += o[i]
        ys.append(y)
    return ys
