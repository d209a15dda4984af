"""Pins of the seeded input generator (host side)."""
import numpy as np

from synth import generator as G
from synth.configs import WORKLOADS, XING4_PREFILL, DSV41_LIKE


def test_philox_known_answers():
    # Known-answer vectors of Philox4x32-10 (Random123 distribution, kat_vectors)
    cases = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, want in cases:
        got = G.philox4x32_10(*[np.array([c], np.uint64) for c in ctr], *key)
        assert tuple(int(w[0]) for w in got) == want


def test_normal_moments_range_and_addressing():
    v = G.normal_f32(0, 2, 3, 5, G.T_GATE, 0, 2_000_000, 0.02)
    assert abs(v.mean()) < 1e-4 and abs(v.std() - 0.02) < 1e-4
    assert np.max(np.abs(v)) <= 0.02 * 4.9
    # addressable: any window equals the same slice of a longer draw
    w = G.normal_f32(0, 2, 3, 5, G.T_GATE, 123_457, 1000, 0.02)
    assert np.array_equal(w, v[123_457:124_457])
    # distinct streams differ
    u = G.normal_f32(0, 2, 3, 6, G.T_GATE, 0, 1000, 0.02)
    assert not np.array_equal(u, v[:1000])


def test_expert_matrix_rows_window():
    wl = WORKLOADS["tiny"]
    full = G.expert_matrix(wl, 0, 3, "down")
    assert full.shape == (256, 128)
    assert np.array_equal(G.expert_matrix(wl, 0, 3, "down", 17, 5), full[17:22])


def test_zipf_bias_ranges():
    b = G.zipf_bias(XING4_PREFILL, 0)
    assert abs(b.min() - (-1.80)) < 0.01 and abs(b.max() - 2.77) < 0.01
    b = G.zipf_bias(DSV41_LIKE, 0)
    assert abs(b.min() - (-2.22)) < 0.01 and abs(b.max() - 4.33) < 0.01
    # a permutation of one fixed profile
    b2 = G.zipf_bias(DSV41_LIKE, 1)
    assert np.array_equal(np.sort(b), np.sort(b2)) and not np.array_equal(b, b2)
    assert not np.any(G.zipf_bias(WORKLOADS["xing4_decode"], 0))
