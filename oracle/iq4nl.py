"""IQ4_NL block format, oracle side.

Format (PocketLLM "Xing4.0-29B-A4B", section "Overview", model table row "Quantization"):
IQ4_NL is 4.5 bits a weight, GGML type 20, 32 weights in 18 bytes.  A block is one fp16
scale ``d`` plus 32 four-bit indices into a fixed 16-entry signed int8 non-linear codebook;
a weight is ``d * c[q]``.

Readings where the page is silent:

* Byte layout: ``d`` little-endian in bytes 0-1; byte ``2+j`` (j < 16) holds index ``q_j``
  in its low nibble and ``q_{j+16}`` in its high nibble.
* Codebook values: the pages never print them.  The table here is the 16-level
  Lloyd-Max quantiser of the standard normal (S. P. Lloyd, "Least squares quantization
  in PCM", 1957/1982; J. Max, "Quantizing for minimum distortion", 1960) scaled so that its
  largest magnitude is 127 and rounded to integers; ``derive_codebook`` re-derives it.
* Quantiser (used to make inputs, never by the GPU hot path): per block
  ``a = max |w|`` in fp32, ``d = fp16_RNE(fp32(a) / 127.0f)``, and each weight takes the
  nearest codebook entry scaled by the stored ``d``, ties to the lower index.  All
  ``d * (c_j + c_{j+1}) / 2`` midpoints are exact in fp32, so the choice is exact.
  A zero block gives ``d = 0`` and all-zero weights.
"""
import math
import numpy as np

BLOCK = 32
BLOCK_BYTES = 18

# 16-level Lloyd-Max levels of N(0,1), scaled to max |level| = 127, rounded.
CODEBOOK = (-127, -96, -75, -58, -44, -31, -18, -6, 6, 18, 31, 44, 58, 75, 96, 127)


def derive_codebook(levels: int = 16, iterations: int = 2000, peak: int = 127):
    """Lloyd's algorithm for the MSE-optimal scalar quantiser of the standard normal.

    Alternates the two optimality conditions: each threshold is the midpoint of adjacent
    levels; each level is the conditional mean of N(0,1) on its cell,
    E[X | a < X < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  Fixed iteration count from
    evenly spaced levels on [-3, 3]; the result is scaled so its largest magnitude is
    ``peak`` and rounded to the nearest integer.
    """
    def phi(t):
        return 0.0 if math.isinf(t) else math.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)

    def cdf(t):
        if math.isinf(t):
            return 0.0 if t < 0 else 1.0
        return 0.5 * (1.0 + math.erf(t / math.sqrt(2.0)))

    lv = [-3.0 + 6.0 * (i + 0.5) / levels for i in range(levels)]
    for _ in range(iterations):
        th = [-math.inf] + [(lv[i] + lv[i + 1]) / 2 for i in range(levels - 1)] + [math.inf]
        lv = [(phi(th[i]) - phi(th[i + 1])) / (cdf(th[i + 1]) - cdf(th[i]))
              for i in range(levels)]
    s = peak / max(abs(v) for v in lv)
    return tuple(int(round(v * s)) for v in lv)


def fp16_bits_to_float(bits) -> np.ndarray:
    """IEEE 754 binary16 bit patterns -> float64, decoded field by field."""
    bits = np.asarray(bits, dtype=np.int64)
    sign = np.where(bits & 0x8000, -1.0, 1.0)
    exp = (bits >> 10) & 0x1F
    man = (bits & 0x3FF).astype(np.float64)
    normal = sign * np.ldexp(1.0 + man / 1024.0, (exp - 15).astype(np.int64))
    sub = sign * np.ldexp(man / 1024.0, -14)
    special = np.where(man == 0, sign * np.inf, np.nan)
    return np.where(exp == 0, sub, np.where(exp == 31, special, normal))


def unpack_blocks(raw: np.ndarray):
    """raw uint8 [..., 18] -> (d_bits uint16 [...], q uint8 [..., 32])."""
    raw = np.asarray(raw, dtype=np.uint8)
    d_bits = raw[..., 0].astype(np.uint16) | (raw[..., 1].astype(np.uint16) << 8)
    codes = raw[..., 2:18]
    q = np.concatenate([codes & 0x0F, codes >> 4], axis=-1)
    return d_bits, q


def pack_blocks(d_bits, q) -> np.ndarray:
    """Inverse of ``unpack_blocks``."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    q = np.asarray(q, dtype=np.uint8)
    assert q.shape[-1] == BLOCK and np.all(q < 16)
    out = np.empty(q.shape[:-1] + (BLOCK_BYTES,), dtype=np.uint8)
    out[..., 0] = d_bits & 0xFF
    out[..., 1] = d_bits >> 8
    out[..., 2:18] = q[..., :16] | (q[..., 16:] << 4)
    return out


def dequantize_blocks(raw: np.ndarray) -> np.ndarray:
    """raw uint8 [..., 18] -> float64 weights [..., 32]: w_i = d * c[q_i]."""
    d_bits, q = unpack_blocks(raw)
    d = fp16_bits_to_float(d_bits)
    c = np.asarray(CODEBOOK, dtype=np.float64)
    return d[..., None] * c[q]


def dequantize_matrix(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """A row-major [rows, cols] matrix stored as rows * (cols/32) consecutive blocks."""
    assert cols % BLOCK == 0
    nb = cols // BLOCK
    blk = np.asarray(raw, dtype=np.uint8).reshape(rows, nb, BLOCK_BYTES)
    return dequantize_blocks(blk).reshape(rows, cols)


def quantize_blocks(w: np.ndarray) -> np.ndarray:
    """fp32 weights [..., 32] -> raw IQ4_NL blocks [..., 18] (the quantiser reading above)."""
    w = np.asarray(w, dtype=np.float32)
    assert w.shape[-1] == BLOCK
    a = np.max(np.abs(w), axis=-1)                                   # fp32
    d16 = (a / np.float32(127.0)).astype(np.float32).astype(np.float16)   # IEEE div, RNE
    d_bits = d16.view(np.uint16)
    d = d16.astype(np.float64)
    c = np.asarray(CODEBOOK, dtype=np.float64)
    mids = (c[:-1] + c[1:]) / 2.0                                     # 15 half-integers
    wd = w.astype(np.float64)
    q = np.zeros(w.shape, dtype=np.uint8)
    for m in mids:                                  # q = number of midpoints below w
        q += (d[..., None] * m < wd)                # d * m exact in fp64
    return pack_blocks(d_bits, q)


def quantize_matrix(w: np.ndarray) -> np.ndarray:
    """fp32 [rows, cols] -> uint8 [rows * cols/32 * 18], blocks along each row."""
    rows, cols = w.shape
    return quantize_blocks(np.asarray(w, np.float32).reshape(rows, cols // BLOCK, BLOCK)).reshape(-1)


def matrix_bytes(rows: int, cols: int) -> int:
    return rows * (cols // BLOCK) * BLOCK_BYTES
