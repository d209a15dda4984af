"""Summaries of rocprofv3 output for the profiles/ folder, and the HBM traffic they record.

``python -m quantized_moe_expert_amd.profiling stats KERNEL_STATS_CSV "COMMAND" > out.txt``
    a short text table of a ``--kernel-trace --stats`` run (the kernels' average durations).
``python -m quantized_moe_expert_amd.profiling pmc FETCH_CSV WRITE_CSV "COMMANDS" > out.txt``
    per-kernel FETCH_SIZE / WRITE_SIZE (KiB a dispatch) of two ``--pmc`` runs, scaled by what
    the same counters read for the plain 256 MiB device copy that ``bench.py
    --copy-calibration`` runs first (its true traffic is known: 256 MiB read, 256 MiB written),
    with a digest of the kernel sources the numbers belong to.

``traffic(kernel, root)`` reads such a summary back (bench.py's ``roofline.traffic``) and
returns None when the sources have changed since the counters were taken.
"""
import csv
import hashlib
import os
import re
import sys
from collections import defaultdict

COPY_BYTES = 256 << 20
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# sources each profiled kernel is compiled from
KERNEL_SOURCES = {
    "decode_gateup_kernel": ("decode.hip", "gemv_core.h", "common.h", "route_core.h", "kernels.h"),
    "decode_down_combine_kernel": ("decode.hip", "gemv_core.h", "common.h", "kernels.h"),
    "gemm_kernel<true>": ("gemm.hip", "common.h", "kernels.h"),
    "gemm_kernel<false>": ("gemm.hip", "common.h", "kernels.h"),
    "bdec_gateup2_kernel": ("bdecode.hip", "common.h", "route_core.h", "kernels.h"),
    "bdec_down2_kernel": ("bdecode.hip", "common.h", "route_core.h", "kernels.h"),
    "bdec_down3_kernel": ("bdecode.hip", "common.h", "route_core.h", "kernels.h"),
}
PMC_FILE = "pmc_traffic_decode_and_prefill_all_workloads.txt"


def source_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _short(name):
    m = re.search(r"(\w+_kernel(<[^>]*>)?|__amd_rocclr_\w+)", name)
    return m.group(1) if m else name[:60]


def stats_summary(stats_csv, command):
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"command: {command}", "",
           f"{'calls':>7} {'avg us':>10} {'min us':>10} {'max us':>10} {'% time':>7}  kernel"]
    for r in rows[:24]:
        out.append(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                   f"{float(r['Percentage']):7.2f}  {r['Name'][:110]}")
    return "\n".join(out) + "\n"


def _per_kernel(path, counter):
    vals = defaultdict(list)
    by_grid = defaultdict(list)
    calib = None
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        if calib is None and "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= 131072:
            calib = float(r["Counter_Value"])            # first dispatch: the 256 MiB copy
        vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        by_grid[(_short(r["Kernel_Name"]), int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return vals, calib, by_grid


def _source_key(short):
    if short in KERNEL_SOURCES:
        return short
    base = short.split("<")[0]
    return base if base in KERNEL_SOURCES else None


def pmc_summary(fetch_csv, write_csv, commands):
    fetch, cf, fetch_g = _per_kernel(fetch_csv, "FETCH_SIZE")
    write, cw, write_g = _per_kernel(write_csv, "WRITE_SIZE")
    if not cf or not cw:
        raise SystemExit("no calibration copy found (run bench.py with --copy-calibration)")
    sf = COPY_BYTES / (cf * 1024)
    sw = COPY_BYTES / (cw * 1024)
    out = [f"commands: {commands}", "",
           f"calibration: 256 MiB device copy reads FETCH_SIZE {cf:.1f} KiB, WRITE_SIZE {cw:.1f} KiB",
           f"scale: fetch x{sf:.4f}, write x{sw:.4f} (true bytes / counter bytes)", ""]
    for k in sorted(set(fetch) & set(write)):
        f = sum(fetch[k]) / len(fetch[k]) * 1024 * sf
        w = sum(write[k]) / len(write[k]) * 1024 * sw
        line = f"kernel {k}: dispatches {len(fetch[k])}: fetch_bytes {f:.0f} write_bytes {w:.0f}"
        key = _source_key(k)
        if key:
            line += f" source_digest {source_digest(key)}"
        out.append(line)
        grids = sorted(g for (kk, g) in fetch_g if kk == k and (kk, g) in write_g)
        if len(grids) > 1:                 # one line a grid size: the launches of one shape
            for g in grids:
                fg, wg = fetch_g[(k, g)], write_g[(k, g)]
                out.append(f"  grid {g}: dispatches {len(fg)}: fetch_bytes "
                           f"{sum(fg) / len(fg) * 1024 * sf:.0f} write_bytes "
                           f"{sum(wg) / len(wg) * 1024 * sw:.0f}")
    return "\n".join(out) + "\n"


def traffic(kernel, root, grid=None):
    """HBM bytes a dispatch (fetch + write) recorded for `kernel` -- a short kernel name with
    its template arguments as the summary prints it, e.g. ``decode_gateup_kernel<64, 2, 1, 4>``
    -- at grid size `grid` (threads; None: the kernel's mean over all its dispatches), or None
    if missing or recorded from other sources."""
    path = os.path.join(root, "profiles", PMC_FILE)
    if not os.path.exists(path):
        return None
    head = re.compile(r"^kernel (.+): dispatches \d+: fetch_bytes (\d+) write_bytes (\d+)"
                      r" source_digest (\w+)")
    sub = re.compile(r"^\s+grid (\d+): dispatches \d+: fetch_bytes (\d+) write_bytes (\d+)")
    cur = None
    for line in open(path):
        m = head.match(line)
        if m:
            cur = None
            if m.group(1) == kernel:
                key = _source_key(kernel)
                if key is None or m.group(4) != source_digest(key):
                    return None
                cur = int(m.group(2)) + int(m.group(3))
                if grid is None:
                    return cur
            continue
        m = sub.match(line)
        if m and cur is not None and int(m.group(1)) == grid:
            return int(m.group(2)) + int(m.group(3))
    return cur if grid is None else None


def counter_summary(csv_path, command, cu_count=256, xcds=8):
    """Per kernel and grid size: the mean per dispatch of every counter in a rocprofv3 --pmc CSV, and the
    ratios these counters define (LDS bank-conflict share of LDS cycles, MFMA busy share of
    SIMD cycles, LDS active share of CU cycles).  GRBM_GUI_ACTIVE reads as the sum over the
    XCDs (8 x the kernel's cycles), so the elapsed cycles are that value / xcds."""
    per = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
        per[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = [f"command: {command}", "",
           "(one block a kernel and grid size: the launches of one workload shape)", ""]
    for k in sorted(per):
        c = {n: sum(v) / len(v) for n, v in per[k].items()}
        n = max(len(v) for v in per[k].values())
        out.append(f"kernel {k[0]} grid {k[1]}: dispatches {n}")
        for name in sorted(c):
            out.append(f"  {name:28s} {c[name]:.4g}")
        if "SQ_LDS_BANK_CONFLICT" in c and "SQ_LDS_IDX_ACTIVE" in c and c["SQ_LDS_IDX_ACTIVE"]:
            out.append(f"  bank-conflict cycles / LDS active cycles: "
                       f"{c['SQ_LDS_BANK_CONFLICT'] / c['SQ_LDS_IDX_ACTIVE']:.3f}")
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        if cyc:
            out.append(f"  elapsed cycles (GRBM_GUI_ACTIVE / {xcds}): {cyc:.4g}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and cyc:
            out.append(f"  MFMA busy / (elapsed cycles x {4 * cu_count} SIMDs): "
                       f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 4 * cu_count):.3f}")
        if "SQ_LDS_IDX_ACTIVE" in c and cyc:
            out.append(f"  LDS active / (elapsed cycles x {cu_count} CUs): "
                       f"{c['SQ_LDS_IDX_ACTIVE'] / (cyc * cu_count):.3f}")
        out.append("")
    return "\n".join(out)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        sys.stdout.write(stats_summary(sys.argv[2], sys.argv[3]))
    elif sys.argv[1] == "pmc":
        sys.stdout.write(pmc_summary(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif sys.argv[1] == "counters":
        sys.stdout.write(counter_summary(sys.argv[2], sys.argv[3]))
    else:
        raise SystemExit(__doc__)
