"""GPU parity of each entry point against the oracle (through the C-ABI binding).

Integer results are compared bit for bit; floating results with the tolerances in
``tests/helpers.py``.  Inputs come from the seeded generator; expected values from ``oracle``.
"""
import zlib

import numpy as np
import pytest
import torch

import quantized_moe_expert_amd as M
from quantized_moe_expert_amd import layer as L
from oracle import iq4nl, moe as omoe
from synth import device as SD, generator as G
from synth.configs import (WORKLOADS, TINY, XING4_DECODE, XING4_PREFILL, QWEN3NEXT_LIKE, DSV41_LIKE,
                           LayerShape, SOFTMAX, Workload)

from .helpers import (REL_L2_GEMV, REL_L2_MFMA, assert_close, assert_within_bound, desc_of,
                      down_bf16_bound, gate_up_bf16_bound, logit_error_bound, oracle_bank,
                      topk_gap)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(DEV) if dtype is None else t.to(DEV, dtype)


def _bf16_rne(a):
    """fp32 -> bf16 round-to-nearest-even on finite values, as uint16 bit patterns."""
    b = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = ((b >> 16) & 1) + 0x7FFF
    return ((b + r) >> 16).astype(np.uint16)


def _bf16_tensor(a):
    return _to_dev(_bf16_rne(a).view(np.int16)).view(torch.bfloat16)


# ---- synthetic inputs: device twin == host generator ---------------------------------

def test_philox_known_answers_on_device():
    out = torch.zeros(4, dtype=torch.int32, device=DEV)
    SD.philox_words(out, 0, 0, 0, 0, 0)
    assert [v & 0xFFFFFFFF for v in out.cpu().tolist()] == \
        [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    SD.philox_words(out, 0xA4093822, 0x299F31D0, 0x13198A2E, 0x03707344,
                    start=(0x85A308D3 << 32) | 0x243F6A88)
    assert [v & 0xFFFFFFFF for v in out.cpu().tolist()] == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


@pytest.mark.parametrize("cfg,layer,expert,tensor,start,n,sigma", [
    (1, 0, 0, G.T_X, 0, 5000, 1.0),
    (2, 37, 64, G.T_DOWN, 1_234_567, 70_000, 0.02),
    (5, 0, 383, G.T_GATE, (1 << 32) - 100, 300, 0.02),
])
def test_device_generator_bitexact(cfg, layer, expert, tensor, start, n, sigma):
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    SD.fill_normal(out, 0, cfg, layer, expert, tensor, start, sigma)
    ref = G.normal_f32(0, cfg, layer, expert, tensor, start, n, sigma)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ---- IQ4_NL encode / decode ----------------------------------------------------------

def test_quantize_bitexact_with_ties_and_edge_blocks():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((6001, 32)) * 0.02).astype(np.float32)
    w[3] = 0.0                                   # zero block
    w[7] *= np.float32(1e-5)                     # fp16-subnormal scales
    w[11] *= np.float32(3e3)                     # large scales
    w[13, :] = np.float32(0.5)                   # constant block
    d = iq4nl.fp16_bits_to_float(iq4nl.unpack_blocks(iq4nl.quantize_blocks(w))[0])
    mids = (np.asarray(iq4nl.CODEBOOK[:-1], float) + np.asarray(iq4nl.CODEBOOK[1:], float)) / 2
    for i in range(20, 6000, 9):                 # exact midpoint ties
        v = np.float32(d[i] * mids[i % 15])
        if float(v) == d[i] * mids[i % 15] and abs(v) < np.max(np.abs(w[i])):
            w[i, (i // 9) % 31 + 1] = v
    ref = iq4nl.quantize_blocks(w)
    out = torch.empty(w.shape[0] * 18, dtype=torch.uint8, device=DEV)
    M.moe_quantize_iq4nl(_to_dev(w), w.shape[0], out)
    assert np.array_equal(out.cpu().numpy(), ref.reshape(-1))


def test_dequantize_bitexact_all_codes():
    rng = np.random.default_rng(1)
    n = 4099                                     # odd count: last block is even-indexed
    raw = rng.integers(0, 256, size=(n, 18), dtype=np.uint8)
    d_bits = rng.integers(0, 0x7C00, size=n).astype(np.uint16)      # finite, non-negative
    d_bits[::5] |= 0x8000                                            # some negative scales
    raw[:, 0] = d_bits & 0xFF
    raw[:, 1] = d_bits >> 8
    out = torch.empty(n * 32, dtype=torch.float32, device=DEV)
    M.moe_dequantize_iq4nl(_to_dev(raw.reshape(-1)), n, out)
    ref = iq4nl.dequantize_blocks(raw).astype(np.float32).reshape(-1)
    assert np.array_equal(out.cpu().numpy(), ref)


# ---- routing -------------------------------------------------------------------------

def _route_gpu(desc, x, wr, b, T, k, E):
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    wsb = M.moe_workspace_size(desc, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    M.moe_route(desc, _to_dev(x), _to_dev(wr), None if b is None else _to_dev(b), T, ids, w,
                logits, ws, wsb)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy()


@pytest.mark.parametrize("name,T", [("tiny", 4), ("xing4_decode", 1), ("xing4_decode", 16),
                                    ("qwen3next_like", 2), ("xing4_prefill", 300),
                                    ("dsv41_like", 40), ("qwen3next_like", 129)])
def test_route_against_oracle(name, T):
    wl = WORKLOADS[name]
    s = wl.shape
    x = G.activations(wl, T)
    wr = G.router_weight(wl, 0)
    b = G.zipf_bias(wl, 0) if wl.zipf_s is not None else None
    desc = L.desc_of(s, T)
    ids, w, lg = _route_gpu(desc, x, wr, b, T, s.top_k, s.n_experts)
    od = desc_of(s)
    # (i) selection applied to the GPU's own logits reproduces the GPU ids exactly
    assert np.array_equal(ids, omoe.select_topk(lg.astype(np.float64), s.top_k))
    # (ii) fp32 logits within the fp32 dot-product error bound of the fp64 logits
    l64 = omoe.router_logits(x, wr, b)
    bound = logit_error_bound(x, wr, b)
    assert np.all(np.abs(lg - l64) <= bound)
    # (iii) ids equal the fp64 selection except at near-ties (listed, expected none here)
    ref_ids = omoe.select_topk(l64, s.top_k)
    gap = topk_gap(l64, s.top_k)
    near = gap < 2 * bound.max(axis=1)
    mism = np.where(np.any(ids != ref_ids, axis=1))[0]
    assert set(mism.tolist()) <= set(np.where(near)[0].tolist()), mism
    # weights from the fp64 logits
    ref_w = omoe.gating_weights(l64, ids, s.gating, s.renormalize)
    assert np.allclose(w, ref_w, rtol=2e-5, atol=1e-6)


def test_route_exact_ties_and_nan():
    s = TINY.shape
    T, E, k, H = 3, s.n_experts, s.top_k, s.hidden
    rng = np.random.default_rng(5)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    wr[5] = wr[2]                  # experts 2 and 5 always tie
    wr[6] = wr[1]
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[2] = np.nan                  # every logit NaN: the k lowest indices, in order
    desc = L.desc_of(s, T)
    ids, w, lg = _route_gpu(desc, x, wr, None, T, k, E)
    assert np.array_equal(ids, omoe.select_topk(lg.astype(np.float64), k))
    assert list(ids[2]) == list(range(k))
    for t in range(2):
        for a, bb in ((2, 5), (1, 6)):
            if a in ids[t] and bb in ids[t]:
                assert list(ids[t]).index(a) < list(ids[t]).index(bb)


@pytest.mark.parametrize("E,k,gating,renorm,T", [(1023, 32, 0, 1, 5), (1023, 32, 1, 0, 3),
                                                 (1000, 17, 1, 1, 20), (33, 32, 0, 1, 2)])
def test_route_largest_expert_counts_and_k(E, k, gating, renorm, T):
    """Top-k at the descriptor's limits (E + S = 1024 bins, k = 32; k = E - 1) on synthetic
    logits: the selection equals a full stable sort of the GPU's own logits, the weights the
    closed forms of the oracle."""
    H = 256
    rng = np.random.default_rng(E + k + T)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    wr[7] = wr[3]                                  # an exact tie
    desc = M.make_desc(H, 128, E, k, 1, gating, renorm, T)
    ids, w, lg = _route_gpu(desc, x, wr, None, T, k, E)
    assert np.array_equal(ids, omoe.select_topk(lg.astype(np.float64), k))
    ref_w = omoe.gating_weights(lg.astype(np.float64), ids, gating, renorm)
    assert np.allclose(w, ref_w, rtol=2e-5, atol=1e-6)


# ---- permutation ---------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E", [(0, 4, 64), (1, 4, 64), (16, 4, 64), (4, 2, 8), (37, 10, 512),
                                   (2048, 4, 64), (8192, 6, 384), (1000, 3, 1023), (300, 1, 5),
                                   # the one-workgroup path's limit (T k = 1024) and one past it
                                   (256, 4, 64), (257, 4, 64), (32, 32, 1023)])
def test_permute_bitexact(T, k, E):
    rng = np.random.default_rng(T * 7 + k + E)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T:
        ids.reshape(-1)[::97] = -1
        ids.reshape(-1)[5::131] = E
        ids.reshape(-1)[7::173] = 2 ** 31 - 1
        ids.reshape(-1)[11::199] = -2 ** 31
    w = rng.random((T, k)).astype(np.float32)
    desc = M.make_desc(256, 128, E, k, 1, 0, 1, max(T, 1))
    gid, gw = _to_dev(ids), _to_dev(w)
    off = torch.full((E + 2,), -7, dtype=torch.int32, device=DEV)
    sp = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device=DEV)
    ps = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device=DEV)
    wsb = M.moe_workspace_size(desc, T)
    ws = torch.full((wsb,), 0x55, dtype=torch.uint8, device=DEV)
    H = 256
    x = rng.standard_normal((T, H)).astype(np.float32)
    xp32 = torch.empty((T * (k + 1), H), dtype=torch.float32, device=DEV)
    M.moe_permute(desc, gid, gw, T, _to_dev(x) if T else None, xp32 if T else None,
                  M.MOE_DTYPE_F32, off, sp, ps, ws, wsb)
    torch.cuda.synchronize()
    sid, sw, n_bad = omoe.sanitize(ids, w, E)
    o_off, o_sp, o_ps = omoe.permute(sid, E, 1)
    assert np.array_equal(gid.cpu().numpy(), sid)
    assert np.array_equal(gw.cpu().numpy(), sw.astype(np.float32))
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert int(ws[:4].view(torch.int32).item()) == n_bad
    if T:
        assert np.array_equal(sp.cpu().numpy(), o_sp)
        assert np.array_equal(ps.cpu().numpy(), o_ps)
        tok = omoe.slot_tokens(o_sp, T, k, 1)
        assert np.array_equal(xp32.cpu().numpy(), x[tok])
        # bf16 gather (RNE)
        xpb = torch.empty((T * (k + 1), H), dtype=torch.bfloat16, device=DEV)
        M.moe_permute(desc, gid, gw, T, _to_dev(x), xpb, M.MOE_DTYPE_BF16, off, sp, ps, ws, wsb)
        torch.cuda.synchronize()
        assert np.array_equal(xpb.cpu().view(torch.int16).numpy().view(np.uint16),
                              _bf16_rne(x[tok]))


@pytest.mark.parametrize("H", [64, 1088, 3584, 8192])
def test_gather_row_lengths(H):
    """The slot-row gather at row lengths from a partial workgroup (64) to the 8,192 maximum
    (eight workgroups a row), fp32 and bf16, bit-exact."""
    T, k, E = 37, 3, 16
    rng = np.random.default_rng(H)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    desc = M.make_desc(H, 128, E, k, 1, 0, 1, T)
    off = torch.empty((E + 2,), dtype=torch.int32, device=DEV)
    sp = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    ps = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    wsb = M.moe_workspace_size(desc, T)
    ws = torch.zeros((wsb,), dtype=torch.uint8, device=DEV)
    x = rng.standard_normal((T, H)).astype(np.float32)
    o_off, o_sp, o_ps = omoe.permute(ids, E, 1)
    tok = omoe.slot_tokens(o_sp, T, k, 1)
    xp32 = torch.full((T * (k + 1), H), np.nan, dtype=torch.float32, device=DEV)
    M.moe_permute(desc, _to_dev(ids), _to_dev(w), T, _to_dev(x), xp32, M.MOE_DTYPE_F32, off, sp, ps,
                  ws, wsb)
    xpb = torch.zeros((T * (k + 1), H), dtype=torch.bfloat16, device=DEV)
    M.moe_permute(desc, _to_dev(ids), _to_dev(w), T, _to_dev(x), xpb, M.MOE_DTYPE_BF16, off, sp, ps,
                  ws, wsb)
    torch.cuda.synchronize()
    assert np.array_equal(xp32.cpu().numpy(), x[tok])
    assert np.array_equal(xpb.cpu().view(torch.int16).numpy().view(np.uint16), _bf16_rne(x[tok]))


# ---- expert GEMV (decode) and grouped GEMM (prefill) ---------------------------------

def _route_table(wl, T, rng, force_invalid=False):
    """A route table (oracle-made) and its permutation, as numpy arrays."""
    s = wl.shape
    x = G.activations(wl, T)
    l, ids, w = omoe.route(x, G.router_weight(wl, 0), None, desc_of(s))
    ids = ids.astype(np.int32)
    off, sp, ps = omoe.permute(ids, s.n_experts, s.n_shared)
    return x, ids, w, off, sp, ps


def _sample_rows(n, count, rng):
    if n <= count:
        return np.arange(n)
    return np.sort(rng.choice(n, size=count, replace=False))


def _oracle_rows(wl, e, which, rows):
    w = np.stack([G.expert_matrix(wl, 0, e, which, int(r), 1)[0] for r in rows])
    return iq4nl.dequantize_matrix(iq4nl.quantize_matrix(w), len(rows), w.shape[1])


# T = 40: one chunk of all 40 slots an expert, so the shared expert runs 20 two-token tiles
# (the tiles past the first two read their token rows on their own)
@pytest.mark.parametrize("name,T", [("tiny", 4), ("xing4_decode", 1), ("xing4_decode", 16),
                                    ("xing4_decode", 40), ("qwen3next_like", 2),
                                    ("dsv41_like", 3)])
@pytest.mark.parametrize("stage", ["gate_up", "down"])
def test_gemv_against_oracle(name, T, stage):
    wl = WORKLOADS[name]
    s = wl.shape
    rng = np.random.default_rng(zlib.crc32(f"{name}/{T}/{stage}".encode()))
    x, ids, w, off, sp, ps = _route_table(wl, T, rng)
    rows = T * s.top_k + T
    used = sorted(set(ids.reshape(-1).tolist()) | {s.n_experts})
    bank_t, bank = L.make_bank(wl, 0, experts=used)
    desc = L.desc_of(s, T)
    if stage == "gate_up":
        out = torch.full((rows, s.ffn), np.nan, dtype=torch.float32, device=DEV)
        M.moe_expert_gemv_iq4nl(desc, M.MOE_STAGE_GATE_UP, bank, _to_dev(off), _to_dev(sp),
                                _to_dev(x), out, T)
        nout = s.ffn
    else:
        hin = (rng.standard_normal((rows, s.ffn)) * 0.7).astype(np.float32)
        out = torch.full((rows, s.hidden), np.nan, dtype=torch.float32, device=DEV)
        M.moe_expert_gemv_iq4nl(desc, M.MOE_STAGE_DOWN, bank, _to_dev(off), None, _to_dev(hin),
                                out, T)
        nout = s.hidden
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    tok = omoe.slot_tokens(sp, T, s.top_k, 1)
    sample = _sample_rows(nout, 96, rng)
    for e in used:
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        if stage == "gate_up":
            wg = _oracle_rows(wl, e, "gate", sample)
            wu = _oracle_rows(wl, e, "up", sample)
            ref = omoe.expert_gate_up(wg, wu, x[tok[a:b]].astype(np.float64))
        else:
            wd = _oracle_rows(wl, e, "down", sample)
            ref = omoe.expert_down(wd, hin[a:b].astype(np.float64))
        assert_close(got[a:b][:, sample], ref, REL_L2_GEMV, f"{name} e={e} {stage}")


# expert row counts on every edge of the GEMM's 128-row tiles and 16-row MFMA groups
_EDGE_COUNTS = {3: 1, 10: 15, 17: 16, 22: 17, 29: 63, 33: 64, 40: 65, 45: 127, 51: 128,
                58: 129, 61: 256, 63: 300}


@pytest.mark.parametrize("stage", ["gate_up", "down"])
def test_grouped_gemm_tile_edges(stage):
    """Slot ranges of 0, 1, 15, 16, 17, 63 .. 65, 127 .. 129, 256 and 300 rows (empty first
    and last bins, a shared bin of 47): every row of every non-empty expert against the oracle
    on sampled columns, and nothing written past the last slot."""
    wl = WORKLOADS["xing4_prefill"]
    s = wl.shape
    rng = np.random.default_rng(zlib.crc32(f"gemm-edges/{stage}".encode()))
    counts = np.zeros(s.n_experts + 1, np.int64)
    for e, c in _EDGE_COUNTS.items():
        counts[e] = c
    counts[s.n_experts] = 47
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n_rows = int(off[-1])
    T = -(-n_rows // (s.top_k + 1))
    rows = T * (s.top_k + 1)
    used = [e for e in range(s.n_experts + 1) if counts[e] > 0]
    bank_t, bank = L.make_bank(wl, 0, experts=used)
    desc = L.desc_of(s, T)
    K, nout = (s.hidden, s.ffn) if stage == "gate_up" else (s.ffn, s.hidden)
    xin = (rng.standard_normal((rows, K)) * (1.0 if stage == "gate_up" else 0.7)).astype(np.float32)
    dt = torch.bfloat16 if stage == "gate_up" else torch.float32
    out = torch.full((rows, nout), np.nan, dtype=dt, device=DEV)
    M.moe_grouped_gemm_iq4nl(desc, M.MOE_STAGE_GATE_UP if stage == "gate_up" else M.MOE_STAGE_DOWN,
                             bank, _to_dev(off), _bf16_tensor(xin), out, T)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isnan(got[n_rows:]).all(), "rows past the last slot were written"
    sample = _sample_rows(nout, 48, rng)
    for e in used:
        a, b = int(off[e]), int(off[e + 1])
        xs = xin[a:b].astype(np.float64)
        if stage == "gate_up":
            wg = _oracle_rows(wl, e, "gate", sample)
            wu = _oracle_rows(wl, e, "up", sample)
            ref = omoe.expert_gate_up(wg, wu, xs)
            bound = gate_up_bf16_bound(wg, wu, xs)
        else:
            wd = _oracle_rows(wl, e, "down", sample)
            ref = omoe.expert_down(wd, xs)
            bound = down_bf16_bound(wd, xin[a:b])
        assert_within_bound(got[a:b][:, sample], ref, bound, REL_L2_MFMA,
                            f"edges e={e} rows={b - a} {stage}")
        if stage == "down":                     # the fp32 output: the layer tolerance as well
            assert_close(got[a:b][:, sample], ref, REL_L2_MFMA, f"edges e={e} {stage}")


# K lengths that leave the GEMM's step groups ragged: hidden 384 is 6 steps of 64 (one group of
# 4 and a tail of 2 for the short tiles' four-step groups), ffn 640 is 10 (a whole pair of
# groups and a tail of 2)
_ODD_K = {"h384_f640": Workload(name="h384_f640", cfg_id=13,
                                shape=LayerShape(hidden=384, ffn=640, n_experts=16, top_k=3,
                                                 n_shared=1, gating=SOFTMAX, renormalize=1),
                                layers=1, prefill_tokens=(40,)),
          # the most bins a layer may have (1,023 experts + the shared one): the tile list's
          # per-bin scan and last-tile placement at their limit
          "e1023": Workload(name="e1023", cfg_id=14,
                            shape=LayerShape(hidden=256, ffn=128, n_experts=1023, top_k=4,
                                             n_shared=1, gating=SOFTMAX, renormalize=1),
                            layers=1, prefill_tokens=(600,))}


@pytest.mark.parametrize("name,T", [("tiny", 4), ("xing4_prefill", 300), ("qwen3next_like", 200),
                                    ("dsv41_like", 260), ("h384_f640", 40), ("h384_f640", 150),
                                    ("e1023", 600)])
@pytest.mark.parametrize("stage", ["gate_up", "down"])
def test_grouped_gemm_against_oracle(name, T, stage):
    wl = _ODD_K.get(name) or WORKLOADS[name]
    s = wl.shape
    rng = np.random.default_rng(zlib.crc32(f"{name}/{T}/{stage}/gemm".encode()))
    x, ids, w, off, sp, ps = _route_table(wl, T, rng)
    rows = T * s.top_k + T
    used = sorted(set(ids.reshape(-1).tolist()) | {s.n_experts})
    bank_t, bank = L.make_bank(wl, 0, experts=used)
    desc = L.desc_of(s, T)
    tok = omoe.slot_tokens(sp, T, s.top_k, 1)
    if stage == "gate_up":
        xin = x[tok]
        out = torch.full((rows, s.ffn), np.nan, dtype=torch.bfloat16, device=DEV)
        M.moe_grouped_gemm_iq4nl(desc, M.MOE_STAGE_GATE_UP, bank, _to_dev(off),
                                 _bf16_tensor(xin), out, T)
        nout = s.ffn
    else:
        hin = (rng.standard_normal((rows, s.ffn)) * 0.7).astype(np.float32)
        out = torch.full((rows, s.hidden), np.nan, dtype=torch.float32, device=DEV)
        M.moe_grouped_gemm_iq4nl(desc, M.MOE_STAGE_DOWN, bank, _to_dev(off), _bf16_tensor(hin),
                                 out, T)
        nout = s.hidden
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    sample = _sample_rows(nout, 64, rng)
    # experts with the most rows (tile edges, several tiles) and a few small ones
    counts = np.diff(off)
    order = [int(e) for e in np.argsort(-counts[:s.n_experts + 1], kind="stable")]
    check = [e for e in order[:3] + order[-6:] if counts[e] > 0] + [s.n_experts]
    for e in sorted(set(check)):
        a, b = int(off[e]), int(off[e + 1])
        # every output against the error bound of the bf16 arithmetic elementwise, plus the
        # rel-L2 bar; the fp32 down output also against the max-abs bar.  (h is bf16: its own
        # rounding is 2^-8 of |h|, above 2e-2 x RMS(h) wherever |h| > 5 RMS(h).)
        if stage == "gate_up":
            wg = _oracle_rows(wl, e, "gate", sample)
            wu = _oracle_rows(wl, e, "up", sample)
            xs = x[tok[a:b]].astype(np.float64)
            ref = omoe.expert_gate_up(wg, wu, xs)
            bound = gate_up_bf16_bound(wg, wu, xs)
        else:
            wd = _oracle_rows(wl, e, "down", sample)
            ref = omoe.expert_down(wd, hin[a:b].astype(np.float64))
            bound = down_bf16_bound(wd, hin[a:b])
        assert_within_bound(got[a:b][:, sample], ref, bound, REL_L2_MFMA, f"{name} e={e} {stage}")
        if stage == "down":                     # the fp32 output: the layer tolerance as well
            assert_close(got[a:b][:, sample], ref, REL_L2_MFMA, f"{name} e={e} {stage}")


@pytest.mark.parametrize("stage", ["gate_up", "down"])
def test_grouped_gemm_reruns_bit_identical(stage):
    """The grouped GEMM is deterministic: eight launches on the same 2,048-token chunk of the
    3584/64 shape (every expert routed; partial and full tiles) give the same bits.  A copy into LDS read before it has landed, or a stage overwritten while still
    read, shows up here as a run that differs."""
    wl = WORKLOADS["xing4_prefill"]
    s = wl.shape
    T = 2048
    rng = np.random.default_rng(zlib.crc32(f"gemm-reruns/{stage}".encode()))
    x, ids, w, off, sp, ps = _route_table(wl, T, rng)
    rows = T * s.top_k + T
    used = sorted(set(ids.reshape(-1).tolist()) | {s.n_experts})
    bank_t, bank = L.make_bank(wl, 0, experts=used)
    desc = L.desc_of(s, T)
    K, nout = (s.hidden, s.ffn) if stage == "gate_up" else (s.ffn, s.hidden)
    xin = _bf16_tensor((rng.standard_normal((rows, K)) * 0.7).astype(np.float32))
    dt = torch.bfloat16 if stage == "gate_up" else torch.float32
    st = M.MOE_STAGE_GATE_UP if stage == "gate_up" else M.MOE_STAGE_DOWN
    offd = _to_dev(off)
    outs = []
    for _ in range(8):
        out = torch.full((rows, nout), np.nan, dtype=dt, device=DEV)
        M.moe_grouped_gemm_iq4nl(desc, st, bank, offd, xin, out, T)
        outs.append(out)
    torch.cuda.synchronize()
    ref = outs[0].view(torch.int16 if stage == "gate_up" else torch.int32)
    assert torch.isfinite(outs[0].float()).all()
    for i, o in enumerate(outs[1:], 1):
        same = torch.equal(o.view(ref.dtype), ref)
        assert same, f"run {i} differs from run 0 ({stage})"


def _bf16_cpu(a):
    """fp32 [rows, K] -> bf16 tensor on the device, rounded on the host by torch (RNE)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("name,T", [("xing4_prefill", 2048), ("dsv41_like", 8192)])
@pytest.mark.parametrize("stage", ["gate_up", "down"])
def test_grouped_gemm_full_size(name, T, stage):
    """The grouped GEMM at the prefill chunk's full size, in the launch configuration the
    benchmark times: EVERY row of the hottest routed expert (1,642 of 8,192 routes on the
    3584/64 shape, 5,616 of 49,152 on the 7168/384 one: every M tile of it) and of the shared
    expert (all T tokens), on 64 sampled output columns, against the oracle."""
    wl = WORKLOADS[name]
    s = wl.shape
    rng = np.random.default_rng(zlib.crc32(f"{name}/{T}/{stage}/full".encode()))
    x = G.activations(wl, T)
    _, ids, _ = omoe.route(x, G.router_weight(wl, 0), G.zipf_bias(wl, 0), desc_of(s))
    off, sp, ps = omoe.permute(ids.astype(np.int32), s.n_experts, s.n_shared)
    counts = np.diff(off)
    hot = int(np.argmax(counts[:s.n_experts]))
    check = [hot, s.n_experts]
    rows = T * (s.top_k + 1)
    bank_t, bank = L.make_bank(wl, 0, experts=check)
    desc = L.desc_of(s, T)
    tok = omoe.slot_tokens(sp, T, s.top_k, 1)
    sample = _sample_rows(s.ffn if stage == "gate_up" else s.hidden, 64, rng)
    if stage == "gate_up":
        xin = x[tok]
        out = torch.full((rows, s.ffn), np.nan, dtype=torch.bfloat16, device=DEV)
        M.moe_grouped_gemm_iq4nl(desc, M.MOE_STAGE_GATE_UP, bank, _to_dev(off), _bf16_cpu(xin),
                                 out, T)
    else:
        xin = (rng.standard_normal((rows, s.ffn)) * 0.7).astype(np.float32)
        out = torch.full((rows, s.hidden), np.nan, dtype=torch.float32, device=DEV)
        M.moe_grouped_gemm_iq4nl(desc, M.MOE_STAGE_DOWN, bank, _to_dev(off), _bf16_cpu(xin), out, T)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all(), "a slot row was not written"
    for e in check:
        a, b = int(off[e]), int(off[e + 1])
        xs = xin[a:b].astype(np.float64)
        if stage == "gate_up":
            wg = _oracle_rows(wl, e, "gate", sample)
            wu = _oracle_rows(wl, e, "up", sample)
            ref = omoe.expert_gate_up(wg, wu, xs)
            bound = gate_up_bf16_bound(wg, wu, xs)
        else:
            wd = _oracle_rows(wl, e, "down", sample)
            ref = omoe.expert_down(wd, xs)
            bound = down_bf16_bound(wd, xin[a:b])
            assert_close(got[a:b][:, sample], ref, REL_L2_MFMA, f"{name} full e={e} {stage}")
        assert_within_bound(got[a:b][:, sample], ref, bound, REL_L2_MFMA,
                            f"{name} full e={e} rows={b - a} {stage}")


# ---- combine and glue ----------------------------------------------------------------

@pytest.mark.parametrize("T,k,H", [(1, 4, 3584), (16, 10, 2048), (33, 6, 256)])
def test_combine_against_oracle(T, k, H):
    rng = np.random.default_rng(T + k)
    E = 64
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, sp, ps = omoe.permute(ids, E, 1)
    o = rng.standard_normal((T * (k + 1), H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    res = rng.standard_normal((T, H)).astype(np.float32)
    desc = M.make_desc(H, 128, E, k, 1, 0, 1, T)
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    M.moe_combine(desc, _to_dev(o), _to_dev(ps), _to_dev(w), T, _to_dev(res), y)
    torch.cuda.synchronize()
    ref = omoe.combine(o, ps, w, T, k, 1, residual=res)
    assert_close(y.cpu().numpy(), ref, 1e-6, "combine")


def test_rmsnorm_against_oracle():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((5, 3584)) * 3).astype(np.float32)
    y = torch.empty_like(_to_dev(x))
    M.moe_rmsnorm(_to_dev(x), 5, 3584, 1e-6, y)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), omoe.rmsnorm(x, 1e-6), 1e-6, "rmsnorm")


def test_host_checks_enqueue_nothing():
    s = TINY.shape
    desc = L.desc_of(s, 4)
    with pytest.raises(M.MoeError) as ei:
        M.moe_route(desc, None, None, None, 4, None, None, None, None, 0)
    assert ei.value.status == M.MOE_ERR_NULL
    with pytest.raises(M.MoeError) as ei:
        M.moe_route(desc, _to_dev(np.zeros((5, 256), np.float32)), None, None, 5, None, None,
                    None, None, 0)
    assert ei.value.status == M.MOE_ERR_SHAPE        # T > max_tokens
