"""Pins of the oracle's IQ4_NL codec against what the format and mathematics fix.

Format: PocketLLM "Xing4.0-29B-A4B", section "Overview" (IQ4_NL, 4.5 bits a weight, 32
weights in 18 bytes).  Codebook: 16-level Lloyd-Max quantiser of N(0,1) scaled to 127.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import iq4nl

CB = np.asarray(iq4nl.CODEBOOK, np.float64)


def test_block_size_matches_page(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "p1_decode_bytes.json")))
    assert iq4nl.BLOCK == g["block_weights"] and iq4nl.BLOCK_BYTES == g["block_bytes"]
    assert iq4nl.BLOCK_BYTES * 8 / iq4nl.BLOCK == g["bits_per_weight"]
    assert iq4nl.matrix_bytes(1024, 3584) == 1024 * 112 * 18


def test_codebook_rederived_by_lloyd_max():
    assert iq4nl.derive_codebook() == iq4nl.CODEBOOK


def test_codebook_shape():
    c = iq4nl.CODEBOOK
    assert len(c) == 16 and len(set(c)) == 16
    assert list(c) == sorted(c)
    assert all(-128 <= v <= 127 for v in c) and max(abs(v) for v in c) == 127
    gaps = np.diff(c)
    assert len(set(gaps.tolist())) > 1           # non-uniform


def test_lloyd_max_levels_are_centroids():
    # independent check of the optimality condition with a numeric integral (scipy-free):
    # each unscaled level equals the mean of N(0,1) over its Voronoi cell.
    import math
    lv = np.asarray(iq4nl.CODEBOOK, np.float64)
    s = 2.7325895709951546 / 127.0        # published 16-level Lloyd-Max extreme level
    t = np.linspace(-12, 12, 2_400_001)
    dens = np.exp(-0.5 * t * t) / math.sqrt(2 * math.pi)
    levels = lv * s
    mids = (levels[:-1] + levels[1:]) / 2
    cell = np.searchsorted(mids, t)
    for i in range(16):
        m = cell == i
        mean = np.sum(t[m] * dens[m]) / np.sum(dens[m])
        assert abs(mean - levels[i]) < 0.5 * s      # agrees within the int8 rounding


def test_fp16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = iq4nl.fp16_bits_to_float(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_pack_unpack_exhaustive_nibbles():
    # every index value in every position, with several scales
    q = (np.arange(32)[None, :] + np.arange(16)[:, None]) % 16
    d = np.array([0x0000, 0x3C00, 0x1234, 0x7BFF, 0x0001, 0x8000, 0xABCD, 0x3555,
                  0x0400, 0x03FF, 0x2000, 0x5555, 0x6666, 0x7777, 0x1111, 0x2222], np.uint16)
    raw = iq4nl.pack_blocks(d, q.astype(np.uint8))
    d2, q2 = iq4nl.unpack_blocks(raw)
    assert np.array_equal(d2, d) and np.array_equal(q2, q)


def test_pack_unpack_random_roundtrip_and_layout():
    rng = np.random.default_rng(1)
    raw = rng.integers(0, 256, size=(500, 18), dtype=np.uint8)
    d, q = iq4nl.unpack_blocks(raw)
    assert np.array_equal(iq4nl.pack_blocks(d, q), raw)
    # layout: element j < 16 is the low nibble of byte 2+j, element j+16 its high nibble
    b = raw[7]
    assert d[7] == int(b[0]) + 256 * int(b[1])
    for j in range(16):
        assert q[7, j] == b[2 + j] & 15 and q[7, j + 16] == b[2 + j] >> 4


def test_dequant_values():
    # worked example: d = 1.0 (0x3C00), indices 0..15,15..0
    q = np.array(list(range(16)) + list(range(15, -1, -1)), np.uint8)
    raw = iq4nl.pack_blocks(np.uint16(0x3C00), q)
    w = iq4nl.dequantize_blocks(raw)
    assert np.array_equal(w, CB[q])
    # d = 2^-10 (0x1400)
    raw = iq4nl.pack_blocks(np.uint16(0x1400), q)
    assert np.array_equal(iq4nl.dequantize_blocks(raw), CB[q] * 2.0 ** -10)


def _round_binary(x: Fraction, man_bits: int, emin: int) -> Fraction:
    """Exact round-to-nearest-even of a positive rational to a binary format with
    ``man_bits`` significand bits and minimum normal exponent ``emin`` (no overflow)."""
    if x == 0:
        return Fraction(0)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - man_bits + 1)
    n = x / ulp
    f = n.numerator // n.denominator
    r = n - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f * ulp


def test_scale_rule_matches_exact_double_rounding():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((2000, 32)) * 0.02).astype(np.float32)
    w[::97] *= np.float32(1e-4)           # some tiny blocks (fp16 subnormal scales)
    raw = iq4nl.quantize_blocks(w)
    d_bits, _ = iq4nl.unpack_blocks(raw)
    for i in range(0, 2000, 7):
        a = Fraction(float(np.max(np.abs(w[i]))))
        d32 = _round_binary(a / 127, 24, -126)            # fp32 division
        d16 = _round_binary(d32, 11, -14)                  # then fp16 RNE
        assert Fraction(float(iq4nl.fp16_bits_to_float(d_bits[i]))) == d16


def test_quantize_is_nearest_codeword_ties_low():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((400, 32)) * 0.02).astype(np.float32)
    # plant exact ties: put weights on midpoints of the stored scale
    raw0 = iq4nl.quantize_blocks(w)
    d = iq4nl.fp16_bits_to_float(iq4nl.unpack_blocks(raw0)[0])
    mids = (CB[:-1] + CB[1:]) / 2
    for i in range(0, 400, 5):
        for j in range(1, 31, 3):
            cand = np.float32(d[i] * mids[(i + j) % 15])
            if abs(cand) < np.max(np.abs(w[i])) and float(cand) == d[i] * mids[(i + j) % 15]:
                w[i, j] = cand
    raw = iq4nl.quantize_blocks(w)
    dd, q = iq4nl.unpack_blocks(raw)
    d = iq4nl.fp16_bits_to_float(dd)
    for i in range(400):
        for j in range(32):
            dist = [abs(float(w[i, j]) - d[i] * c) for c in iq4nl.CODEBOOK]
            best = min(range(16), key=lambda m: (dist[m], m))
            assert q[i, j] == best


def test_quantize_error_bound_and_zero_block():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((3000, 32)) * 0.02).astype(np.float32)
    w[5] = 0.0
    raw = iq4nl.quantize_blocks(w)
    wh = iq4nl.dequantize_blocks(raw)
    assert np.all(wh[5] == 0.0) and iq4nl.unpack_blocks(raw)[0][5] == 0
    d = iq4nl.fp16_bits_to_float(iq4nl.unpack_blocks(raw)[0])
    half_gap = np.max(np.diff(CB)) / 2
    inside = np.abs(w) <= 127 * d[:, None]
    err = np.abs(w.astype(np.float64) - wh)
    assert np.all(err[inside] <= (d[:, None] * half_gap + 0 * err)[inside] + 1e-12)
    # relative reconstruction error of a Gaussian block stays modest
    assert np.linalg.norm(err) / np.linalg.norm(w) < 0.12


def test_quantize_idempotent_on_grid_blocks():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(300, 32)).astype(np.uint8)
    q[:, 0] = 15                        # absmax hits +127 * d
    q[::2, 1] = 0                       # and -127 * d
    d_bits = rng.integers(0x1000, 0x2C00, size=300).astype(np.uint16)
    raw = iq4nl.pack_blocks(d_bits, q)
    w = iq4nl.dequantize_blocks(raw).astype(np.float32)
    raw2 = iq4nl.quantize_blocks(w)
    assert np.array_equal(raw2, raw)


def test_matrix_layout_rows_of_blocks():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((5, 96)) * 0.02).astype(np.float32)
    raw = iq4nl.quantize_matrix(w)
    assert raw.size == 5 * 3 * 18
    full = iq4nl.dequantize_matrix(raw, 5, 96)
    for r in range(5):
        for b in range(3):
            blk = raw[(r * 3 + b) * 18:(r * 3 + b + 1) * 18]
            assert np.array_equal(full[r, 32 * b:32 * b + 32], iq4nl.dequantize_blocks(blk))
