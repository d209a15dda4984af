"""Build libmoe_iq4nl.so (and the synthetic-input library) for gfx950 with hipcc, in-tree.

Every source is compiled to an object in parallel, then linked.  All HIP code is compiled
with packed-fp32 instruction selection disabled.
"""
import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]
# per-source additions: the batched decode kernels keep their small matrix results in VGPRs
# (read by VALU right after each instruction) instead of AGPRs that need a copy each
EXTRA_FLAGS = {"bdecode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

LIBS = {
    os.path.join(PKG, "libmoe_iq4nl.so"): [
        os.path.join(PKG, "csrc", f) for f in
        ("api.hip", "quant.hip", "route.hip", "permute.hip", "gemv.hip", "gemm.hip",
         "combine.hip", "decode.hip", "bdecode.hip")],
    os.path.join(ROOT, "synth", "libmoe_synth.so"): [
        os.path.join(ROOT, "synth", "csrc", "synth.hip")],
}


def source_digest(lib):
    """sha256 of the sources a library is built from (its .hip files and every header beside
    them), in a fixed order; written next to the library so a stale build can be refused."""
    srcs = LIBS[lib]
    dirs = sorted({os.path.dirname(s) for s in srcs})
    headers = [os.path.join(d, f) for d in dirs for f in sorted(os.listdir(d)) if f.endswith(".h")]
    h = hashlib.sha256()
    for f in list(srcs) + headers:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _compile(src, obj, verbose):
    cmd = [HIPCC] + FLAGS + EXTRA_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = None) -> list:
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    built = []
    tasks = []
    with cf.ThreadPoolExecutor(jobs) as ex:
        for lib, srcs in LIBS.items():
            for s in srcs:
                obj = os.path.join(out_dir, os.path.basename(s) + ".o")
                tasks.append(ex.submit(_compile, s, obj, verbose))
        for t in tasks:
            t.result()
    for lib, srcs in LIBS.items():
        objs = [os.path.join(out_dir, os.path.basename(s) + ".o") for s in srcs]
        tmp = lib + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed for {lib}:\n{r.stderr}")
        os.replace(tmp, lib)
        with open(lib + ".digest", "w") as fh:
            fh.write(source_digest(lib) + "\n")
        built.append(lib)
        if verbose:
            print("built", lib, flush=True)
    return built


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
