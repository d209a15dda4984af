"""The C-ABI libraries load and export every function their headers declare (no GPU needed).

Also the host-side contract that needs no device: version, status strings, workspace sizing,
and argument checks that return before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

import quantized_moe_expert_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = {
    "moe_iq4nl.h": M.LIB_PATH,
    "moe_synth.h": os.path.join(ROOT, "synth", "libmoe_synth.so"),
}


def _declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"if", "sizeof", "defined"} - set(re.findall(r"#define\s+(\w+)\(", text)))


@pytest.mark.parametrize("header", sorted(HEADERS))
def test_library_exports_every_declared_function(header):
    names = _declared(header)
    assert names, header
    lib = ctypes.CDLL(HEADERS[header])
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"{header}: not exported: {missing}"


def test_binding_covers_the_header():
    names = set(_declared("moe_iq4nl.h"))
    assert names <= set(M._SIGNATURES), names - set(M._SIGNATURES)
    for n in names:
        assert callable(getattr(M, n)), n


def test_version_and_status_strings():
    assert M.moe_abi_version() == M.ABI_VERSION
    for s in range(0, 8):
        assert isinstance(M.moe_status_string(s), str) and M.moe_status_string(s)


def test_workspace_size_grows_with_tokens_and_covers_the_header():
    d = M.make_desc(3584, 1024, 64, 4, 1, M.MOE_GATING_SIGMOID, 1, 16)
    sizes = [M.moe_workspace_size(d, T) for T in (1, 2, 16)]
    assert sizes == sorted(sizes)
    assert sizes[0] >= 256                                 # header (sanitised-pair count)


@pytest.mark.parametrize("field,value", [("hidden", 100), ("ffn", 32), ("top_k", 0),
                                         ("top_k", 65), ("n_shared", 2), ("n_experts", 1024)])
def test_bad_descriptors_are_rejected_on_the_host(field, value):
    d = M.make_desc(3584, 1024, 64, 4, 1, M.MOE_GATING_SIGMOID, 1, 16)
    setattr(d, field, value)
    with pytest.raises(M.MoeError) as ei:
        M.moe_workspace_size(d, 1)
    assert ei.value.status == M.MOE_ERR_SHAPE


def test_decode_chain_checks_before_enqueueing():
    d = M.make_desc(3584, 1024, 64, 4, 1, M.MOE_GATING_SIGMOID, 1, 16)
    arr = M.make_layers([(M.make_bank(None, 0), None, None)])
    # more layers than the launch holds
    with pytest.raises(M.MoeError) as ei:
        M.moe_decode_chain(d, arr, M.MOE_CHAIN_MAX_LAYERS + 1, None, 1, 1e-6, None, None, None, 0,
                           stream=0)
    assert ei.value.status == M.MOE_ERR_SHAPE
    # a NULL bank
    with pytest.raises(M.MoeError) as ei:
        M.moe_decode_chain(d, arr, 1, None, 1, 1e-6, None, None, None, 0, stream=0)
    assert ei.value.status == M.MOE_ERR_NULL


def test_stale_library_is_refused(monkeypatch):
    from quantized_moe_expert_amd import build as B
    M._check_fresh(M.LIB_PATH)                    # the tree's build matches its sources
    monkeypatch.setattr(B, "source_digest", lambda lib: "0" * 64)
    with pytest.raises(ImportError, match="stale"):
        M._check_fresh(M.LIB_PATH)
