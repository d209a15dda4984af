"""The C-ABI's host-side checks under AddressSanitizer (CPU only, no GPU needed).

api.hip is compiled with AddressSanitizer on its host code only (device code as usual) and
linked with the library's other objects into tests/asan/abi_checks.cpp, which calls every
entry point with arguments that the checks must reject before anything reaches the device
(bad descriptors, sizes, stages, banks, null and misaligned pointers, short workspaces, the
allocation-free entry point's scratch limit, the chain's per-layer checks) plus workspace
sizing over many shapes.  The run fails on a wrong status or on any sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_moe_expert_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "asan")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
def _others():
    """Every source of the library but api.hip, as the build lists them."""
    import sys
    sys.path.insert(0, ROOT)
    from quantized_moe_expert_amd import build
    srcs = build.LIBS[os.path.join(build.PKG, "libmoe_iq4nl.so")]
    return tuple(os.path.basename(f) for f in srcs if os.path.basename(f) != "api.hip")


OTHERS = _others()
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                                        if "packed-fp32-ops" not in l)[-4000:]


@pytest.mark.timeout(600)
def test_host_checks_under_address_sanitizer():
    if not os.path.exists(HIPCC) or not os.path.exists(CLANG):
        pytest.skip("hipcc / clang++ not installed")
    objs = [os.path.join(BUILD, f + ".o") for f in OTHERS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (python -m quantized_moe_expert_amd.build)")
    os.makedirs(OUT, exist_ok=True)
    api_o = os.path.join(OUT, "api.hip.o")
    drv_o = os.path.join(OUT, "abi_checks.o")
    exe = os.path.join(OUT, "abi_checks")
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang",
          "-target-feature", "-Xclang", "-packed-fp32-ops"] + HOST_ASAN +
         ["-c", os.path.join(CSRC, "api.hip"), "-o", api_o])
    _run([CLANG, "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
          "-I/opt/rocm/include", "-fsanitize=address", "-fno-omit-frame-pointer", "-c",
          os.path.join(ROOT, "tests", "asan", "abi_checks.cpp"), "-o", drv_o])
    _run([HIPCC, "--offload-arch=gfx950"] + HOST_ASAN + [drv_o, api_o] + objs + ["-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and "0 failures" in out, out[-4000:]
