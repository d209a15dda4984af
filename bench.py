#!/usr/bin/env python3
"""Benchmark of the routed IQ4_NL MoE layer on one MI355X.

Headline (the default line's `value`): decode of the Xing4.0-29B-A4B-shaped stack -- T tokens
(default 1) through 38 chained MoE layers, x <- x + MoE_l(rmsnorm(x)), hidden 3,584, 64 routed
experts top-4 (sigmoid, renormalised) + 1 shared, expert FFN 1,024, all experts IQ4_NL and
resident.  A step is one pass of the whole hot path (per layer: router with the RMSNorm glue,
top-k, permutation, gate/up GEMV with SwiGLU, down GEMV, combine) over one batch, captured
once in a HIP graph and replayed.  Inputs and weights are synthetic (seeded generator) and
resident in HBM before the timed region.

Measured in the same run and reported in the same JSON line:
  * roofline of the dominant kernel (the headline's gate/up GEMV): per-launch duration from HIP
    events around replays of a HIP graph holding that stage's launches for all 38 distinct
    layers (each layer's weights are cold: the 38 layers' 0.8 GB exceed the 256 MB Infinity
    Cache), its algorithmic bytes a launch, and the HBM traffic its counters recorded;
  * the other workloads of the configuration table, each with its dominant kernel's fraction
    of its roofline: 16-token decode of the same stack; 512-expert softmax-routed decode at 1
    and 2 tokens through 48 layers; one 7168/384 layer decoding 16 tokens; the 2,048-token
    prefill chunks of the 3584/64 and 2048/512 shapes and the 8,192-token chunk of the
    7168/384 shape through the grouped bf16-MFMA GEMM;
  * the oracle (fp64 numpy) on the host cores on bounded samples of the headline decode and
    of the 2,048-token prefill, with BLAS on all the process's cores;
  * GPU clocks before and after.

Prints ONE JSON line.  --gpus N with N > 1 exits: the benchmark runs on one GPU.
"""
import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, published
COPY_BYTES = 256 << 20         # calibration copy: reads and writes this many bytes
METRIC = "MoE-layer decode tok/s + expert GB/s (% of 8 TB/s); prefill TFLOP/s (% MFMA)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic(kernel, grid=None):
    from quantized_moe_expert_amd import profiling
    return profiling.traffic(kernel, ROOT, grid)


def _lanes_blocks(nb):
    """Lanes a weight row and blocks a lane the decode kernels pick for rows of nb blocks
    (least idle lanes, at most 4 blocks a lane): the template arguments of the kernel."""
    best, waste = None, 1 << 30
    for lpr in (64, 32, 16, 8, 4):
        bpl = -(-nb // lpr)
        if bpl <= 4 and lpr * bpl - nb < waste:
            best, waste = (lpr, bpl), lpr * bpl - nb
    return best


def add_gemm_traffic(record, wl):
    """The grouped GEMMs' HBM bytes a launch (copy-calibrated counters of the profiles/
    summary, for this workload's grid) next to their algorithmic bytes."""
    T = wl.prefill_tokens[0]
    s = wl.shape
    rows = T * (s.top_k + s.n_shared)
    experts = min(s.n_experts, T * s.top_k) + s.n_shared          # upper bound on active
    for stage, key, w_bytes, io in ((0, "gate_up", 2 * s.gate_bytes,
                                     rows * s.hidden * 2 + rows * s.ffn * 2),
                                    (1, "down", s.down_bytes,
                                     rows * s.ffn * 2 + rows * s.hidden * 4)):
        t = traffic("gemm_kernel<%s>" % ("true" if stage == 0 else "false"),
                    gemm_grid(s, T, stage))
        record[f"{key}_traffic_bytes"] = t
        record[f"{key}_algorithmic_bytes_max"] = experts * w_bytes + io


def gemm_grid(shape, tokens, stage):
    """Threads of a grouped-GEMM launch (the tile bound the library launches)."""
    rows = tokens * (shape.top_k + shape.n_shared)
    mtiles = -(-rows // 256) + min(shape.n_experts + shape.n_shared, rows)
    nt = shape.ffn // 128 if stage == 0 else -(-shape.hidden // 256)
    return -(-mtiles // 8) * 8 * nt * 512


# ---- CPU baseline (the oracle), run before the GPU is touched ----------------------------

def _oracle_expert(args):
    name, layer, e = args
    import numpy as np
    from oracle import iq4nl
    from synth import generator as G
    from synth.configs import WORKLOADS
    wl = WORKLOADS[name]
    return e, np.concatenate([iq4nl.quantize_matrix(G.expert_matrix(wl, layer, e, w))
                              for w in ("gate", "up", "down")])


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(n_layers, T, prefill_tokens, min_seconds):
    """The oracle as it stands (plain fp64 numpy), BLAS on all of this process's cores:
    decode of T tokens through the first n_layers layers of the 38-layer stack (rate scaled to
    38 layers), and a sample of prefill_tokens tokens of the 2,048-token 3584/64 chunk.  Input
    preparation (host generator and oracle quantiser, in worker processes) is untimed."""
    import concurrent.futures as cf
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import moe as omoe
    from synth import generator as G
    from synth.configs import XING4_DECODE, XING4_PREFILL

    cores = len(os.sched_getaffinity(0))
    out = dict(cores=cores, cpu_model=_cpu_model())
    t_prep = time.time()
    with cf.ProcessPoolExecutor(max(1, min(16, cores))) as ex:
        # decode: the experts each of the first n_layers layers routes to
        wl = XING4_DECODE
        s = wl.shape
        desc = omoe.Desc(s.hidden, s.ffn, s.n_experts, s.top_k, s.n_shared, s.gating, s.renormalize)
        stride = s.expert_bytes
        x = G.activations(wl, T).astype(np.float64)
        banks, routers = [], []
        for l in range(n_layers):
            wr = G.router_weight(wl, l)
            xn = omoe.rmsnorm(x)
            _, ids, _ = omoe.route(xn, wr, None, desc)
            need = sorted(set(ids.reshape(-1).tolist()) | {s.n_experts})
            bank = np.zeros(stride * (s.n_experts + 1), np.uint8)
            for e, b in ex.map(_oracle_expert, [(wl.name, l, e) for e in need]):
                bank[e * stride:(e + 1) * stride] = b
            x = x + omoe.moe_layer(xn, wr, None, bank, stride, desc)
            banks.append(bank)
            routers.append(wr)
        # prefill: every expert of layer 0 of the prefill chunk's shape
        wp = XING4_PREFILL
        sp = wp.shape
        dp = omoe.Desc(sp.hidden, sp.ffn, sp.n_experts, sp.top_k, sp.n_shared, sp.gating,
                       sp.renormalize)
        pbank = np.zeros(sp.expert_bytes * (sp.n_experts + 1), np.uint8)
        for e, b in ex.map(_oracle_expert, [(wp.name, 0, e) for e in range(sp.n_experts + 1)]):
            pbank[e * sp.expert_bytes:(e + 1) * sp.expert_bytes] = b
    t_prep = time.time() - t_prep
    xp = G.activations(wp, prefill_tokens).astype(np.float64)
    wrp, bp = G.router_weight(wp, 0), G.zipf_bias(wp, 0)

    with threadpool_limits(limits=cores):
        passes = 0
        t0 = time.perf_counter()
        while True:
            x = G.activations(wl, T).astype(np.float64)
            for l in range(n_layers):
                xn = omoe.rmsnorm(x)
                x = x + omoe.moe_layer(xn, routers[l], None, banks[l], stride, desc)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds or passes >= 50:
                break
        per_layer = dt / (n_layers * passes)
        reps = 0
        t1 = time.perf_counter()
        while True:
            omoe.moe_layer(xp, wrp, bp, pbank, sp.expert_bytes, dp)
            reps += 1
            dtp = time.perf_counter() - t1
            if dtp >= min_seconds or reps >= 20:
                break
    prefill_s = dtp / reps
    flop = 2.0 * prefill_tokens * (sp.top_k + sp.n_shared) * 3 * sp.hidden * sp.ffn
    out.update(
        value=T / (per_layer * wl.layers), unit="tok/s", kind="oracle",
        sample=(f"decode: {T} token(s) through layers 0..{n_layers - 1} of the {wl.layers}-layer "
                f"3584/64 stack, {passes} passes, {dt:.2f} s timed, rate scaled to {wl.layers} "
                f"layers; prefill: {prefill_tokens} of the 2,048 tokens of the 3584/64 chunk, "
                f"{reps} passes, {dtp:.2f} s timed; fp64 numpy oracle including dequantisation "
                f"of the experts, BLAS on {cores} threads; input preparation {t_prep:.0f} s "
                f"untimed"),
        prefill={"tok_s": round(prefill_tokens / prefill_s, 2),
                 "GFLOPs": round(flop / prefill_s / 1e9, 2),
                 "tokens": prefill_tokens},
        seconds=dt + dtp)
    return out


# ---- GPU helpers ---------------------------------------------------------------------------

def gpu_clocks():
    """Current and maximum shader / memory clocks as rocm-smi reports them (or None)."""
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=30)
        d = json.loads(r.stdout)
        card = d[sorted(d)[0]]
        return {k: v for k, v in card.items() if "clk" in k.lower()}
    except Exception:
        return None


def build_stack(wl, n_layers):
    from quantized_moe_expert_amd import layer as L
    layers, keep = [], []
    for l in range(n_layers):
        bank_t, bank = L.make_bank(wl, l)
        wr, bias = L.make_router(wl, l)
        layers.append((wr, bias, bank))
        keep.append(bank_t)
    return layers, keep


class Timer:
    """HIP events on torch's current stream, the stream every launch here goes to."""

    def __init__(self):
        import torch
        self.torch = torch
        self.marks = []

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.marks.append(e)

    def spans_ms(self):
        self.torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in zip(self.marks, self.marks[1:])]


def decode_bench(wl, T, layers, steps, warmup, rounds):
    """Decode of T tokens through the stack: graph-replayed steps, and each stage's launches
    timed back to back over all distinct layers (cold weights)."""
    import torch
    import quantized_moe_expert_amd as M
    from quantized_moe_expert_amd import layer as L

    s = wl.shape
    eps = 1e-6
    n = len(layers)
    x0 = L.make_activations(wl, T)
    buf = L.LayerBuffers(s, T)

    # inputs of every layer and the experts each one routes to, from one eager step
    bufs = [L.LayerBuffers(s, T) for _ in range(n)]
    xs, U = [], []
    x = x0.clone()
    for l, (wr, bias, bank) in enumerate(layers):
        xs.append(x.clone())
        L.decode_layer_fused(bufs[l], xs[l], wr, bias, bank, norm_eps=eps, residual=xs[l], out=x)
    torch.cuda.synchronize()
    for l in range(n):
        U.append(len(set(bufs[l].ids.cpu().reshape(-1).tolist())) + s.n_shared)
    xg = x0.clone()

    def step():
        xg.copy_(x0)
        L.decode_chain_step(buf, xg, layers, eps)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    t = Timer()
    t.mark()
    g.replay()
    t.mark()
    cold_ms = t.spans_ms()[0]
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t = Timer()
    t.mark()
    for _ in range(steps):
        g.replay()
    t.mark()
    ms_step = t.spans_ms()[0] / steps

    # each stage's launches back to back over the n distinct layers, captured in one HIP graph
    # a stage (no host launch cost between them) and replayed `rounds` times
    ys = [torch.empty_like(x0) for _ in range(n)]
    stage_ms = {}
    for st, key in ((M.MOE_DECODE_ROUTER, "router"), (M.MOE_DECODE_GATE_UP, "gate_up"),
                    (M.MOE_DECODE_DOWN, "down")):
        def launches():
            for l, (wr, bias, bank) in enumerate(layers):
                L.decode_layer_fused(bufs[l], xs[l], wr, bias, bank, norm_eps=eps,
                                     residual=xs[l], out=ys[l], stages=st)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            launches()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs):
            launches()
        gs.replay()
        t = Timer()
        t.mark()
        for _ in range(rounds):
            gs.replay()
        t.mark()
        stage_ms[key] = t.spans_ms()[0] / (rounds * n)
        del gs
    avg = stage_ms

    rows = T * s.top_k + T * s.n_shared
    gu_w, dn_w = 2 * s.gate_bytes, s.down_bytes
    # algorithmic bytes a launch: the active experts' weights + activations in + out
    gu_bytes = sum(u * gu_w + T * s.hidden * 4 + rows * s.ffn * 4 for u in U) / n
    dn_bytes = sum(u * dn_w + rows * s.ffn * 4 + 2 * T * s.hidden * 4 for u in U) / n
    rt_bytes = s.n_experts * s.hidden * 4 + T * s.hidden * 4
    expert_bytes_step = sum(u * s.expert_bytes for u in U)
    router_bytes_step = n * s.n_experts * s.hidden * 4
    floor_us = (expert_bytes_step + router_bytes_step) / (HBM_PEAK_GBS * 1e9) * 1e6
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    return dict(
        T=T, layers=n, U=U, ms_step=ms_step, cold_ms=cold_ms, tok_s=T / (ms_step * 1e-3),
        floor_us=floor_us, expert_bytes_step=expert_bytes_step,
        router_bytes_step=router_bytes_step,
        stage_us={k: v * 1e3 for k, v in avg.items()},
        gate_up_bytes=gu_bytes, down_bytes=dn_bytes, router_bytes=rt_bytes,
        gate_up_gbs=gbs(gu_bytes, avg["gate_up"]), down_gbs=gbs(dn_bytes, avg["down"]),
        router_gbs=gbs(rt_bytes, avg["router"]),
        expert_gbs=expert_bytes_step / ((avg["gate_up"] + avg["down"]) * n * 1e-3) / 1e9)


def prefill_bench(wl, layer_data, reps):
    import torch
    import quantized_moe_expert_amd as M
    from quantized_moe_expert_amd import layer as L

    s = wl.shape
    T = wl.prefill_tokens[0]
    wr, bias, bank = layer_data
    x = L.make_activations(wl, T)
    buf = L.LayerBuffers(s, T, prefill=True)
    for _ in range(2):
        L.prefill_layer(buf, x, wr, bias, bank)
    torch.cuda.synchronize()
    lay, gu, dn = [], [], []
    for _ in range(reps):
        t = Timer()
        t.mark()
        L.route_and_permute(buf, x, wr, bias, gather_bf16=True)
        t.mark()
        M.moe_grouped_gemm_iq4nl(buf.desc, M.MOE_STAGE_GATE_UP, bank, buf.offsets, buf.x_perm,
                                 buf.h, T)
        t.mark()
        M.moe_grouped_gemm_iq4nl(buf.desc, M.MOE_STAGE_DOWN, bank, buf.offsets, buf.h, buf.o, T)
        t.mark()
        M.moe_combine(buf.desc, buf.o, buf.pair_slot, buf.w, T, None, buf.y)
        t.mark()
        sp = t.spans_ms()
        lay.append(sum(sp))
        gu.append(sp[1])
        dn.append(sp[2])
    layer_ms, gu_ms, dn_ms = (sum(v) / len(v) for v in (lay, gu, dn))
    rows = T * (s.top_k + s.n_shared)
    flop_gu = 2.0 * rows * s.hidden * 2 * s.ffn
    flop_dn = 2.0 * rows * s.ffn * s.hidden
    off = buf.offsets.cpu()
    counts = (off[1:] - off[:-1])
    used = int((counts > 0).sum().item())
    # algorithmic bytes of the two GEMMs: weights of the experts with rows (once each),
    # x_perm (bf16) in, h (bf16) out and in, o (fp32) out
    gemm_bytes = (used * s.expert_bytes + rows * s.hidden * 2 + 2 * rows * s.ffn * 2
                  + rows * s.hidden * 4)
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12
    return dict(
        T=T, layer_ms=layer_ms, gate_up_ms=gu_ms, down_ms=dn_ms,
        gemm_tflops=tf(flop_gu + flop_dn, gu_ms + dn_ms), gate_up_tflops=tf(flop_gu, gu_ms),
        down_tflops=tf(flop_dn, dn_ms), flop=flop_gu + flop_dn,
        gemm_gbs=gemm_bytes / ((gu_ms + dn_ms) * 1e-3) / 1e9, gemm_bytes=gemm_bytes,
        load_max_over_mean=float(counts[:s.n_experts].max()) / float(
            counts[:s.n_experts].float().mean()))


def shape_text(wl):
    s = wl.shape
    gate = "sigmoid" if s.gating == 0 else "softmax"
    return (f"H {s.hidden}, {s.n_experts} experts top-{s.top_k} {gate}"
            f"{' renormalised' if s.renormalize else ''} + {s.n_shared} shared, F {s.ffn}, IQ4_NL")


def decode_record(name, wl, d):
    dom = max(("gate_up", "down"), key=lambda k: d["stage_us"][k])
    return {
        "workload": f"{name}: decode, {d['T']} token(s) x {d['layers']} chained layer(s), "
                    f"{shape_text(wl)}",
        "tok_s": round(d["tok_s"], 2), "us_per_step": round(d["ms_step"] * 1e3, 2),
        "cold_first_step_us": round(d["cold_ms"] * 1e3, 2),
        "byte_floor_us": round(d["floor_us"], 2),
        "frac_of_byte_floor": round(d["floor_us"] / (d["ms_step"] * 1e3), 4),
        "launch_us": {k: round(v, 3) for k, v in d["stage_us"].items()},
        "GBps": {"gate_up": round(d["gate_up_gbs"], 1), "down": round(d["down_gbs"], 1),
                 "router": round(d["router_gbs"], 1), "experts": round(d["expert_gbs"], 1)},
        "dominant": {"stage": dom, "bound": "hbm",
                     "frac": round(d[f"{dom}_gbs"] / HBM_PEAK_GBS, 4)},
        "active_experts_per_layer_mean": round(sum(d["U"]) / len(d["U"]), 2),
        **batched_traffic(wl, d),
    }


def batched_traffic(wl, d):
    """For the batched decode kernels (5 to 16 tokens): their HBM bytes a launch from the
    profiles/ summary (looked up by grid) next to the algorithmic bytes a launch."""
    s = wl.shape
    if d["T"] <= 4:
        return {}
    gu_grid = (s.ffn // 64) * (s.n_experts + s.n_shared + 1) * 256
    dn_grid = (s.hidden // 128) * (s.n_experts + s.n_shared) * 256
    return {"gate_up_traffic_bytes": traffic("bdec_gateup2_kernel<2>", gu_grid),
            "gate_up_algorithmic_bytes": round(d["gate_up_bytes"]),
            "down_traffic_bytes": traffic("bdec_down3_kernel<2>", dn_grid),
            "down_algorithmic_bytes": round(d["down_bytes"])}


def prefill_record(name, wl, p):
    # the 2048/512 chunk's intensity (about 115 flop/B) is below the MFMA ridge: HBM-bound
    hbm = wl.shape.n_experts >= 512
    frac = (p["gemm_gbs"] / HBM_PEAK_GBS) if hbm else (p["gemm_tflops"] / BF16_PEAK_TFLOPS)
    return {
        "workload": f"{name}: prefill, {p['T']}-token chunk, one layer, {shape_text(wl)}",
        "grouped_gemm_TFLOPs": round(p["gemm_tflops"], 2),
        "frac_of_bf16_peak": round(p["gemm_tflops"] / BF16_PEAK_TFLOPS, 4),
        "gate_up_ms": round(p["gate_up_ms"], 4), "down_ms": round(p["down_ms"], 4),
        "gate_up_TFLOPs": round(p["gate_up_tflops"], 2), "down_TFLOPs": round(p["down_tflops"], 2),
        "layer_ms": round(p["layer_ms"], 4),
        "layer_tok_s": round(p["T"] / (p["layer_ms"] * 1e-3), 1),
        "gemm_GBps": round(p["gemm_gbs"], 1),
        "gemm_frac_of_hbm": round(p["gemm_gbs"] / HBM_PEAK_GBS, 4),
        "expert_load_max_over_mean": round(p["load_max_over_mean"], 2),
        "dominant": {"stage": "gate_up", "bound": "hbm" if hbm else "mfma",
                     "frac": round(frac, 4)},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--tokens", type=int, default=1, help="headline decode batch (1 to 16)")
    ap.add_argument("--rounds", type=int, default=10,
                    help="replays of each stage's graph (all layers' launches of that stage)")
    ap.add_argument("--prefill-reps", type=int, default=5)
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline decode (and its roofline), no other workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=8)
    ap.add_argument("--cpu-prefill-tokens", type=int, default=128)
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the rocm-smi clock readings (for runs under a profiler)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy 3 times (the reference kernel "
                         "of known traffic for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: bench.py measures one GPU "
              f"(the layer would shard by replicas or by experts across GPUs)", file=sys.stderr)
        sys.exit(2)

    # the oracle first, before anything touches the GPU (its input preparation forks workers)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        cpu = cpu_baseline(args.cpu_layers, args.tokens, args.cpu_prefill_tokens,
                           args.cpu_seconds)
        log(f"[bench] cpu baseline: decode {cpu['value']:.3f} tok/s, prefill "
            f"{cpu['prefill']['tok_s']} tok/s on {cpu['cores']} cores")

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import quantized_moe_expert_amd as M
    M.lib()
    from synth.configs import XING4_DECODE, XING4_PREFILL, QWEN3NEXT_LIKE, DSV41_LIKE

    clocks_before = None if args.no_clocks else gpu_clocks()
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    t_start = time.time()
    log("[bench] building the 38-layer 3584/64 stack ...")
    stack, keep = build_stack(XING4_DECODE, XING4_DECODE.layers)
    torch.cuda.synchronize()
    d = decode_bench(XING4_DECODE, args.tokens, stack, args.steps, args.warmup, args.rounds)
    log(f"[bench] headline decode T={d['T']}: {d['ms_step'] * 1e3:.1f} us/step "
        f"({d['tok_s']:.1f} tok/s); launches {d['stage_us']}")
    configs = []
    prefill_main = None
    if not args.headline_only:
        if args.tokens != 16:
            d16 = decode_bench(XING4_DECODE, 16, stack, max(20, args.steps // 4), 5, args.rounds)
            configs.append(decode_record("xing4_decode", XING4_DECODE, d16))
            log(f"[bench] xing4 decode T=16: {d16['tok_s']:.1f} tok/s")
        del stack, keep
        torch.cuda.empty_cache()

        from quantized_moe_expert_amd import layer as L
        wr, bias = L.make_router(XING4_PREFILL, 0)
        bank_t, bank = L.make_bank(XING4_PREFILL, 0)
        prefill_main = prefill_bench(XING4_PREFILL, (wr, bias, bank), args.prefill_reps)
        log(f"[bench] xing4 prefill: GEMM {prefill_main['gemm_tflops']:.1f} TFLOP/s")
        del bank_t, bank
        torch.cuda.empty_cache()

        log("[bench] building the 48-layer 2048/512 stack ...")
        stack, keep = build_stack(QWEN3NEXT_LIKE, QWEN3NEXT_LIKE.layers)
        for T in QWEN3NEXT_LIKE.decode_tokens:
            dq = decode_bench(QWEN3NEXT_LIKE, T, stack, max(20, args.steps // 4), 5, args.rounds)
            configs.append(decode_record("qwen3next_like", QWEN3NEXT_LIKE, dq))
            log(f"[bench] qwen3next decode T={T}: {dq['tok_s']:.1f} tok/s")
        pq = prefill_bench(QWEN3NEXT_LIKE, stack[0], args.prefill_reps)
        configs.append(prefill_record("qwen3next_like", QWEN3NEXT_LIKE, pq))
        add_gemm_traffic(configs[-1], QWEN3NEXT_LIKE)
        log(f"[bench] qwen3next prefill: GEMM {pq['gemm_tflops']:.1f} TFLOP/s, "
            f"{pq['gemm_gbs']:.0f} GB/s")
        del stack, keep
        torch.cuda.empty_cache()

        log("[bench] building one 7168/384 layer ...")
        stack, keep = build_stack(DSV41_LIKE, 1)
        dd = decode_bench(DSV41_LIKE, DSV41_LIKE.decode_tokens[0], stack,
                          max(20, args.steps // 4), 5, args.rounds)
        configs.append(decode_record("dsv41_like", DSV41_LIKE, dd))
        log(f"[bench] dsv41 decode T=16: {dd['tok_s']:.1f} tok/s")
        pd = prefill_bench(DSV41_LIKE, stack[0], max(2, args.prefill_reps // 2))
        configs.append(prefill_record("dsv41_like", DSV41_LIKE, pd))
        add_gemm_traffic(configs[-1], DSV41_LIKE)
        log(f"[bench] dsv41 prefill: GEMM {pd['gemm_tflops']:.1f} TFLOP/s")
        del stack, keep
        torch.cuda.empty_cache()
    clocks_after = None if args.no_clocks else gpu_clocks()

    gu_gbs = d["gate_up_gbs"]
    rec = {
        "metric": METRIC,
        "value": round(d["tok_s"], 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"xing4_decode: {d['T']} token(s) x {d['layers']} chained MoE layers, "
                        f"{shape_text(XING4_DECODE)}",
            "global_batch": d["T"], "layers": d["layers"], "parallelism": "none (1 GPU)"},
        "roofline": {
            "kernel": ("decode_gateup_kernel (routing + IQ4_NL dequant-GEMV gate/up + SwiGLU)"
                       if d["T"] <= 4 else
                       "bdec_gateup2_kernel (routing + IQ4_NL gate/up on bf16 matrix cores + "
                       "SwiGLU)"),
            "bound": "hbm",
            "achieved": round(gu_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
            "traffic": (traffic("decode_gateup_kernel<%d, %d, 1, 4>"
                                % _lanes_blocks(XING4_DECODE.shape.hidden // 32))
                        if d["T"] == 1 else None),
            "bytes_per_launch": round(d["gate_up_bytes"]),
            "avg_launch_us": round(d["stage_us"]["gate_up"], 3),
            "timing": f"HIP events around {args.rounds} replays of a HIP graph of the stage's "
                      f"{d['layers']} launches, one per distinct layer (weights cold)",
        },
        "decode": decode_record("xing4_decode", XING4_DECODE, d),
    }
    if prefill_main:
        rec["prefill"] = prefill_record("xing4_prefill", XING4_PREFILL, prefill_main)
        add_gemm_traffic(rec["prefill"], XING4_PREFILL)
    if configs:
        rec["configs"] = configs
    if cpu:
        rec["cpu_baseline"] = {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample",
                                                  "cpu_model", "prefill")}
        rec["cpu_baseline"]["value"] = round(cpu["value"], 4)
    dig = M.LIB_PATH + ".digest"
    rec["build"] = {"lib": os.path.basename(M.LIB_PATH),
                    "sources_sha256": open(dig).read().strip()[:16] if os.path.exists(dig) else None,
                    "device": torch.cuda.get_device_name(0)}
    rec["gpu_clocks"] = {"before": clocks_before, "after": clocks_after}
    rec["gpu_seconds"] = round(time.time() - t_start, 1)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
