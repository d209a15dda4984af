#!/usr/bin/env python3
"""Benchmark of the routed IQ4_NL MoE layer on one MI355X.

Headline (the default): decode of the Xing4.0-29B-A4B-shaped stack -- T tokens (default 1)
through 38 chained MoE layers, x <- x + MoE_l(rmsnorm(x)), hidden 3,584, 64 routed experts
top-4 (sigmoid, renormalised) + 1 shared, expert FFN 1,024, all experts IQ4_NL and resident.
A step is one pass of the whole hot path (per layer: rmsnorm glue, router + top-k,
permutation, gate/up GEMV with SwiGLU, down GEMV, combine) over one batch, captured once in a
HIP graph and replayed.  Inputs and weights are synthetic (seeded generator), resident in HBM
before the timed region.

Also measured in the same run: the dominant kernel (gate/up GEMV), launched back to back per
layer between HIP events (-> achieved GB/s against 8 TB/s); the same stack through the
single-launch persistent entry point (moe_decode_chain); the
2,048-token prefill chunk of the same shape through the grouped bf16-MFMA GEMM (-> TFLOP/s
against the bf16 dense peak); the oracle on the host cores on a bounded sample.

Prints ONE JSON line.  --gpus N with N > 1 exits: this build runs on one GPU.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, published
COPY_BYTES = 256 << 20         # calibration copy: reads and writes this many bytes


def traffic(kernel):
    from quantized_moe_expert_amd import profiling
    return profiling.traffic(kernel, ROOT)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_stack(wl, n_layers):
    from quantized_moe_expert_amd import layer as L
    layers, keep = [], []
    for l in range(n_layers):
        bank_t, bank = L.make_bank(wl, l)
        wr, bias = L.make_router(wl, l)
        layers.append((wr, bias, bank))
        keep.append(bank_t)
    return layers, keep


def active_experts_per_layer(buf, x0, layers, eps):
    """Unique experts (routed + shared) each layer's launches touch, from one eager step."""
    import torch
    import quantized_moe_expert_amd as M
    from quantized_moe_expert_amd import layer as L
    x = x0.clone()
    U = []
    for lay in layers:
        M.moe_rmsnorm(x, buf.T, buf.shape.hidden, eps, buf.xn)
        L.decode_layer(buf, buf.xn, lay[0], lay[1], lay[2], residual=x, out=x)
        off = buf.offsets.cpu()
        U.append(int(((off[1:] - off[:-1]) > 0).sum().item()))
    torch.cuda.synchronize()
    return U


def decode_bench(args):
    import torch
    import quantized_moe_expert_amd as M
    from quantized_moe_expert_amd import layer as L
    from synth.configs import WORKLOADS

    wl = WORKLOADS[args.decode_workload]
    s = wl.shape
    T = args.tokens
    eps = 1e-6
    log(f"[bench] building {wl.layers} layers of IQ4_NL experts on the GPU ...")
    t0 = time.time()
    layers, keep = build_stack(wl, wl.layers)
    x0 = L.make_activations(wl, T)
    buf = L.LayerBuffers(s, T)
    torch.cuda.synchronize()
    log(f"[bench] built in {time.time() - t0:.1f}s; bank {s.bank_bytes / 2**20:.1f} MiB/layer")

    U = active_experts_per_layer(buf, x0, layers, eps)
    rows = T * s.top_k + T * s.n_shared
    gu_w = 2 * s.gate_bytes
    dn_w = s.down_bytes
    # algorithmic bytes per launch: weights of the active experts + activations in + out
    gu_bytes = [u * gu_w + rows * s.hidden * 4 + rows * s.ffn * 4 for u in U]
    dn_bytes = [u * dn_w + rows * s.ffn * 4 + rows * s.hidden * 4 for u in U]
    expert_bytes_step = sum(u * s.expert_bytes for u in U)
    router_bytes_step = wl.layers * s.n_experts * s.hidden * 4

    x = x0.clone()

    def step():
        x.copy_(x0)
        L.decode_chain_step(buf, x, layers, eps)

    # capture one step in a HIP graph
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

    # cold first replay reported separately
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    g.replay()
    c1.record()
    torch.cuda.synchronize()
    cold_ms = c0.elapsed_time(c1)

    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # dominant kernel (gate/up GEMV): per layer, its router stage once, then `reps` launches of
    # the gate/up stage back to back between two HIP events on torch's current stream (the
    # stream the kernels run on); the same for the down stage.  The per-launch average is the
    # kernel's steady-state duration plus the launch-to-launch gap.
    reps = args.event_reps
    gu_ms, dn_ms = [], []
    x.copy_(x0)
    for li, (wr, bias, bank) in enumerate(layers):
        L.decode_layer_fused(buf, x, wr, bias, bank, norm_eps=eps, residual=x, out=buf.y,
                             stages=M.MOE_DECODE_ROUTER)
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record()
        for _ in range(reps):
            L.decode_layer_fused(buf, x, wr, bias, bank, norm_eps=eps, residual=x, out=buf.y,
                                 stages=M.MOE_DECODE_GATE_UP)
        b.record()
        for _ in range(reps):
            L.decode_layer_fused(buf, x, wr, bias, bank, norm_eps=eps, residual=x, out=buf.y,
                                 stages=M.MOE_DECODE_DOWN)
        c.record()
        gu_ms.append((a, b))
        dn_ms.append((b, c))
        x.copy_(buf.y)
    torch.cuda.synchronize()
    gu_ms = [a.elapsed_time(b) / reps for (a, b) in gu_ms]
    dn_ms = [b.elapsed_time(c) / reps for (b, c) in dn_ms]
    gu_avg_ms = sum(gu_ms) / len(gu_ms)
    dn_avg_ms = sum(dn_ms) / len(dn_ms)
    gu_avg_bytes = sum(gu_bytes) / len(gu_bytes)
    gu_gbs = gu_avg_bytes / (gu_avg_ms * 1e-3) / 1e9
    gemv_total_ms = sum(gu_ms) + sum(dn_ms)
    gemv_gbs = expert_bytes_step / (gemv_total_ms * 1e-3) / 1e9

    # the same stack in one persistent launch (moe_decode_chain)
    chain_us = None
    if T <= 16:
        arr = M.make_layers([(bank, wr, bias) for (wr, bias, bank) in layers])
        bufc = L.LayerBuffers(s, T)
        xc = x0.clone()
        for _ in range(3):
            xc.copy_(x0)
            L.decode_chain(bufc, xc, arr, eps)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_chain = max(1, args.steps // 4)
        a.record()
        for _ in range(n_chain):
            xc.copy_(x0)
            L.decode_chain(bufc, xc, arr, eps)
        b.record()
        torch.cuda.synchronize()
        chain_us = a.elapsed_time(b) / n_chain * 1e3
        assert L.chain_status(bufc) == 0, "a bounded wait of the persistent decode expired"

    return dict(
        T=T, U=U, ms_step=ms_step, cold_ms=cold_ms,
        tok_s=T / (ms_step * 1e-3),
        gu_avg_us=gu_avg_ms * 1e3, dn_avg_us=dn_avg_ms * 1e3,
        gu_avg_bytes=gu_avg_bytes, gu_gbs=gu_gbs,
        gemv_gbs=gemv_gbs, expert_bytes_step=expert_bytes_step, chain_us=chain_us,
        router_bytes_step=router_bytes_step,
        floor_us=(expert_bytes_step + router_bytes_step) / (HBM_PEAK_GBS * 1e9) * 1e6,
        layers=wl.layers, keep=keep, name=wl.name, H=s.hidden, F=s.ffn, E=s.n_experts,
        k=s.top_k, gating="sigmoid" if s.gating == M.MOE_GATING_SIGMOID else "softmax")


def prefill_bench(args):
    import torch
    import quantized_moe_expert_amd as M
    from quantized_moe_expert_amd import layer as L
    from synth.configs import WORKLOADS

    wl = WORKLOADS[args.prefill_workload]
    s = wl.shape
    T = wl.prefill_tokens[0]
    bank_t, bank = L.make_bank(wl, 0)
    wr, bias = L.make_router(wl, 0)
    x = L.make_activations(wl, T)
    buf = L.LayerBuffers(s, T, prefill=True)
    for _ in range(2):
        L.prefill_layer(buf, x, wr, bias, bank)
    torch.cuda.synchronize()
    n = args.prefill_steps
    ev = []
    l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    l0.record()
    for _ in range(n):
        L.route_and_permute(buf, x, wr, bias, gather_bf16=True)
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record()
        M.moe_grouped_gemm_iq4nl(buf.desc, M.MOE_STAGE_GATE_UP, bank, buf.offsets, buf.x_perm,
                                 buf.h, T)
        b.record()
        M.moe_grouped_gemm_iq4nl(buf.desc, M.MOE_STAGE_DOWN, bank, buf.offsets, buf.h, buf.o, T)
        c.record()
        M.moe_combine(buf.desc, buf.o, buf.pair_slot, buf.w, T, None, buf.y)
        ev.append((a, b, c))
    l1.record()
    torch.cuda.synchronize()
    layer_ms = l0.elapsed_time(l1) / n
    gu_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / n
    dn_ms = sum(b.elapsed_time(c) for _, b, c in ev) / n
    rows = T * (s.top_k + s.n_shared)
    flop_gu = 2.0 * rows * s.hidden * 2 * s.ffn
    flop_dn = 2.0 * rows * s.ffn * s.hidden
    off = buf.offsets.cpu()
    counts = (off[1:] - off[:-1])[:s.n_experts]
    # algorithmic bytes of the two GEMMs: weights of the experts with rows (once each),
    # x_perm (bf16) in, h (bf16) out and in, o (fp32) out
    used = int(((off[1:] - off[:-1]) > 0).sum().item())
    gemm_bytes = (used * s.expert_bytes + rows * s.hidden * 2 + 2 * rows * s.ffn * 2
                  + rows * s.hidden * 4)
    return dict(workload=wl.name, T=T, layer_ms=layer_ms, gu_ms=gu_ms, dn_ms=dn_ms,
                gemm_gbs=gemm_bytes / ((gu_ms + dn_ms) * 1e-3) / 1e9, gemm_bytes=gemm_bytes,
                gemm_tflops=(flop_gu + flop_dn) / ((gu_ms + dn_ms) * 1e-3) / 1e12,
                gu_tflops=flop_gu / (gu_ms * 1e-3) / 1e12,
                dn_tflops=flop_dn / (dn_ms * 1e-3) / 1e12,
                flop=flop_gu + flop_dn,
                load_max_over_mean=float(counts.max()) / float(counts.float().mean()))


def _oracle_expert(args):
    name, layer, e = args
    import numpy as np
    from oracle import iq4nl
    from synth import generator as G
    from synth.configs import WORKLOADS
    wl = WORKLOADS[name]
    return e, np.concatenate([iq4nl.quantize_matrix(G.expert_matrix(wl, layer, e, w))
                              for w in ("gate", "up", "down")])


def cpu_baseline(n_layers, T, min_seconds=10.0):
    """The oracle (fp64 numpy) decoding T tokens through the first n_layers layers; inputs are
    prepared first (host generator + oracle quantiser, in worker processes), then the oracle's
    chain is timed with its BLAS limited to one thread."""
    import concurrent.futures as cf
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import moe as omoe
    from synth import generator as G
    from synth.configs import XING4_DECODE

    wl = XING4_DECODE
    s = wl.shape
    desc = omoe.Desc(s.hidden, s.ffn, s.n_experts, s.top_k, s.n_shared, s.gating, s.renormalize)
    stride = s.expert_bytes
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    x = G.activations(wl, T).astype(np.float64)
    banks, routers = [], []
    t_prep = time.time()
    with cf.ProcessPoolExecutor(workers) as ex:
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
    t_prep = time.time() - t_prep
    # whole passes over the prepared layers until at least min_seconds of oracle work
    passes = 0
    with threadpool_limits(limits=1):
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
    return dict(value=T / (per_layer * wl.layers), unit="tok/s", cores=1, kind="oracle",
                sample=f"{T} token(s) through layers 0..{n_layers - 1} of the {wl.layers}-layer "
                       f"decode stack, {passes} passes (fp64 numpy oracle incl. dequantisation of "
                       f"the routed experts; BLAS 1 thread), {dt:.2f} s timed, scaled to "
                       f"{wl.layers} layers; input prep {t_prep:.1f} s untimed",
                seconds=dt)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--tokens", type=int, default=1, help="decode batch (1 to 16)")
    ap.add_argument("--decode-workload", default="xing4_decode",
                    help="decode stack: xing4_decode (headline), qwen3next_like, dsv41_like")
    ap.add_argument("--event-reps", type=int, default=20,
                    help="back-to-back launches a layer timed for the dominant kernel")
    ap.add_argument("--prefill-workload", default="xing4_prefill")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=12)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy 3 times (the reference kernel "
                         "of known traffic for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build measures one GPU "
              f"(only one GPU is measured; the layer would shard by experts or by replicas)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import quantized_moe_expert_amd as M
    M.lib()

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    d = decode_bench(args)
    log(f"[bench] decode T={d['T']}: {d['ms_step'] * 1e3:.1f} us/step ({d['tok_s']:.1f} tok/s), "
        f"cold {d['cold_ms'] * 1e3:.1f} us; gate/up GEMV {d['gu_avg_us']:.2f} us "
        f"{d['gu_gbs']:.0f} GB/s; down {d['dn_avg_us']:.2f} us; GEMV expert {d['gemv_gbs']:.0f} GB/s")
    p = None
    if not args.no_prefill:
        p = prefill_bench(args)
        log(f"[bench] prefill {p['workload']} T={p['T']}: layer {p['layer_ms']:.3f} ms; "
            f"grouped GEMM {p['gemm_tflops']:.1f} TFLOP/s (gate/up {p['gu_ms']:.3f} ms, "
            f"down {p['dn_ms']:.3f} ms)")
    cpu = None
    if not args.no_cpu_baseline and args.decode_workload == "xing4_decode":
        cpu = cpu_baseline(args.cpu_layers, d["T"], args.cpu_seconds)
        log(f"[bench] cpu baseline: {cpu['value']:.3f} tok/s ({cpu['sample']})")

    rec = {
        "metric": "MoE-layer decode tok/s + expert GB/s (% of 8 TB/s); prefill TFLOP/s (% MFMA)",
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
            "workload": f"{d['name']}: {d['T']} token(s) x {d['layers']} chained MoE layers, "
                        f"H {d['H']}, {d['E']} experts top-{d['k']} {d['gating']} + 1 shared, "
                        f"F {d['F']}, IQ4_NL",
            "global_batch": d["T"], "layers": d["layers"], "parallelism": "none (1 GPU)"},
        "roofline": {
            "kernel": ("decode_gateup_kernel (routing + IQ4_NL dequant-GEMV gate/up + SwiGLU)"
                       if d["T"] <= 4 else
                       "gemv_kernel<..., true> (IQ4_NL dequant-GEMV gate/up + SwiGLU)"),
            "bytes_note": "active experts' gate+up IQ4_NL bytes + activations in + h out",
            "bound": "hbm",
            "achieved": round(d["gu_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(d["gu_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": (traffic("decode_gateup_kernel")
                        if d["T"] == 1 and d["name"] == "xing4_decode" else None),
            "traffic_note": "HBM bytes a launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from "
                            "profiles/pmc_traffic_xing4.txt (1-token xing4 decode); null if the "
                            "kernel changed since or for another workload",
            "bytes_per_launch": round(d["gu_avg_bytes"]),
            "avg_launch_us": round(d["gu_avg_us"], 3),
        },
        "decode": {
            "us_per_step": round(d["ms_step"] * 1e3, 2),
            "cold_first_step_us": round(d["cold_ms"] * 1e3, 2),
            "byte_floor_us": round(d["floor_us"], 2),
            "expert_bytes_per_step": d["expert_bytes_step"],
            "active_experts_per_layer": d["U"][:4] + (["..."] if len(d["U"]) > 4 else []),
            "gemv_expert_GBps": round(d["gemv_gbs"], 1),
            "gemv_expert_frac_of_hbm": round(d["gemv_gbs"] / HBM_PEAK_GBS, 4),
            "down_avg_launch_us": round(d["dn_avg_us"], 3),
            "persistent_chain_us_per_step": (round(d["chain_us"], 2) if d["chain_us"] else None),
        },
    }
    if p:
        rec["prefill"] = {
            "workload": f"{p['workload']}: {p['T']}-token chunk, one layer",
            "grouped_gemm_TFLOPs": round(p["gemm_tflops"], 2),
            "frac_of_bf16_peak": round(p["gemm_tflops"] / BF16_PEAK_TFLOPS, 4),
            "gate_up_ms": round(p["gu_ms"], 4), "down_ms": round(p["dn_ms"], 4),
            "layer_ms": round(p["layer_ms"], 4),
            "layer_tok_s": round(p["T"] / (p["layer_ms"] * 1e-3), 1),
            "flop_per_layer": p["flop"],
            "expert_load_max_over_mean": round(p["load_max_over_mean"], 2),
            "gemm_GBps": round(p["gemm_gbs"], 1),
            "gemm_frac_of_hbm": round(p["gemm_gbs"] / HBM_PEAK_GBS, 4),
            "gate_up_traffic_bytes": (traffic("gemm_kernel<true>")
                                      if p["workload"] == "xing4_prefill" else None),
            "down_traffic_bytes": (traffic("gemm_kernel<false>")
                                   if p["workload"] == "xing4_prefill" else None),
        }
    dig = M.LIB_PATH + ".digest"
    rec["build"] = {"lib": os.path.basename(M.LIB_PATH),
                    "sources_sha256": open(dig).read().strip()[:16] if os.path.exists(dig) else None,
                    "device": torch.cuda.get_device_name(0)}
    if cpu:
        rec["cpu_baseline"] = {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")}
        rec["cpu_baseline"]["value"] = round(cpu["value"], 4)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
