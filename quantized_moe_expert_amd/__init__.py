"""Python binding of libmoe_iq4nl.so: the routed MoE layer with IQ4_NL experts on MI355X.

Argument marshalling only -- every step runs in the library's HIP kernels.  Functions carry
the names of the C-ABI entry points (include/moe_iq4nl.h) and take torch tensors (their
device pointers are passed), plain integer pointers, or None for NULL.  PyTorch supplies
device memory and the current HIP stream; nothing here computes.

The library must be built (``python -m quantized_moe_expert_amd.build`` or
``__graft_entry__.build()``); importing fails loudly when it is missing.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_iq4nl.so")

MOE_OK = 0
MOE_ERR_NULL = 1
MOE_ERR_SHAPE = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_UNSUPPORTED = 4
MOE_ERR_HIP = 5
MOE_ERR_ALIGNMENT = 6
MOE_ERR_SCRATCH_LIMIT = 7
MOE_NOALLOC_SCRATCH_BYTES = 8 << 20

MOE_GATING_SIGMOID = 0
MOE_GATING_SOFTMAX = 1
MOE_STAGE_GATE_UP = 0
MOE_STAGE_DOWN = 1
MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_DECODE_ROUTER = 1
MOE_DECODE_GATE_UP = 2
MOE_DECODE_DOWN = 4
MOE_DECODE_ALL = 7

ABI_VERSION = 1


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib().moe_status_string(status).decode()
        if status == MOE_ERR_HIP:
            msg += f" (hip error {lib().moe_last_hip_error()})"
        super().__init__(f"{fn}: status {status}: {msg}")


class moe_desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("gating", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("max_tokens", ctypes.c_int32)]


class moe_bank(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("expert_stride", ctypes.c_int64)]


class moe_layer(ctypes.Structure):
    _fields_ = [("bank", moe_bank), ("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


MOE_CHAIN_MAX_LAYERS = 64

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_DESC = ctypes.POINTER(moe_desc)
_BANK = ctypes.POINTER(moe_bank)

_SIGNATURES = {
    "moe_abi_version": (_I32, []),
    "moe_status_string": (ctypes.c_char_p, [_I32]),
    "moe_last_hip_error": (_I32, []),
    "moe_workspace_size": (_I32, [_DESC, _I32, ctypes.POINTER(_SZ)]),
    "moe_quantize_iq4nl": (_I32, [_P, _I64, _P, _P]),
    "moe_dequantize_iq4nl": (_I32, [_P, _I64, _P, _P]),
    "moe_route": (_I32, [_DESC, _P, _P, _P, _I32, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute": (_I32, [_DESC, _P, _P, _I32, _P, _P, _I32, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_gemv_iq4nl": (_I32, [_DESC, _I32, _BANK, _P, _P, _P, _P, _I32, _P, _SZ, _P]),
    "moe_grouped_gemm_iq4nl": (_I32, [_DESC, _I32, _BANK, _P, _P, _P, _I32, _P, _SZ, _P]),
    "moe_combine": (_I32, [_DESC, _P, _P, _P, _I32, _P, _P, _P]),
    "moe_rmsnorm": (_I32, [_P, _I32, _I32, ctypes.c_float, _P, _P]),
    "moe_decode_chain": (_I32, [_DESC, ctypes.POINTER(moe_layer), _I32, _P, _I32, ctypes.c_float,
                                _P, _P, _P, _SZ, _P]),
    "moe_decode_layer": (_I32, [_DESC, _BANK, _P, _P, _P, _I32, ctypes.c_float, _P, _P, _P, _P,
                                _I32, _P, _SZ, _P]),
    "moe_decode_layer_noalloc": (_I32, [_DESC, _BANK, _P, _P, _P, _I32, ctypes.c_float, _P, _P,
                                        _P, _P, _I32, _P]),
}

_lib = None
_DEFAULT_LIB = LIB_PATH


def _check_fresh(path):
    """Refuse a library built from other sources than the ones in the tree (a stale build)."""
    from . import build as _build
    rec = path + ".digest"
    want = _build.source_digest(path)
    have = open(rec).read().strip() if os.path.exists(rec) else None
    if have != want:
        raise ImportError(f"{path} was built from other sources than the tree holds (stale "
                          "build): rebuild it with `python -m quantized_moe_expert_amd.build`")


def lib():
    """The loaded library (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m quantized_moe_expert_amd.build`")
        if LIB_PATH == _DEFAULT_LIB:
            _check_fresh(LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        if l.moe_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH}: ABI {l.moe_abi_version()} != {ABI_VERSION}")
        _lib = l
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status)


def make_desc(hidden, ffn, n_experts, top_k, n_shared=1, gating=MOE_GATING_SIGMOID,
              renormalize=1, max_tokens=1):
    return moe_desc(hidden, ffn, n_experts, top_k, n_shared, gating, renormalize, max_tokens)


def make_bank(base, expert_stride):
    return moe_bank(_ptr(base), int(expert_stride))


def moe_abi_version():
    return lib().moe_abi_version()


def moe_status_string(status):
    return lib().moe_status_string(status).decode()


def moe_last_hip_error():
    return lib().moe_last_hip_error()


def moe_workspace_size(desc, n_tokens):
    n = _SZ(0)
    _check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(desc), n_tokens,
                                                          ctypes.byref(n)))
    return n.value


def moe_quantize_iq4nl(w, n_blocks, out, stream=None):
    _check("moe_quantize_iq4nl",
           lib().moe_quantize_iq4nl(_ptr(w), n_blocks, _ptr(out), _stream(stream)))


def moe_dequantize_iq4nl(blocks, n_blocks, out, stream=None):
    _check("moe_dequantize_iq4nl",
           lib().moe_dequantize_iq4nl(_ptr(blocks), n_blocks, _ptr(out), _stream(stream)))


def moe_route(desc, x, w_router, bias, n_tokens, topk_ids, topk_w, logits, ws, ws_bytes,
              stream=None):
    _check("moe_route", lib().moe_route(ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(bias),
                                        n_tokens, _ptr(topk_ids), _ptr(topk_w), _ptr(logits),
                                        _ptr(ws), ws_bytes, _stream(stream)))


def moe_permute(desc, topk_ids, topk_w, n_tokens, x, x_perm, x_perm_dtype, offsets,
                sorted_pairs, pair_slot, ws, ws_bytes, stream=None):
    _check("moe_permute",
           lib().moe_permute(ctypes.byref(desc), _ptr(topk_ids), _ptr(topk_w), n_tokens, _ptr(x),
                             _ptr(x_perm), x_perm_dtype, _ptr(offsets), _ptr(sorted_pairs),
                             _ptr(pair_slot), _ptr(ws), ws_bytes, _stream(stream)))


def moe_expert_gemv_iq4nl(desc, stage, bank, offsets, sorted_pairs, inp, out, n_tokens,
                          ws=None, ws_bytes=0, stream=None):
    _check("moe_expert_gemv_iq4nl",
           lib().moe_expert_gemv_iq4nl(ctypes.byref(desc), stage, ctypes.byref(bank),
                                       _ptr(offsets), _ptr(sorted_pairs), _ptr(inp), _ptr(out),
                                       n_tokens, _ptr(ws), ws_bytes, _stream(stream)))


def moe_grouped_gemm_iq4nl(desc, stage, bank, offsets, in_bf16, out, n_tokens, ws=None,
                           ws_bytes=0, stream=None):
    _check("moe_grouped_gemm_iq4nl",
           lib().moe_grouped_gemm_iq4nl(ctypes.byref(desc), stage, ctypes.byref(bank),
                                        _ptr(offsets), _ptr(in_bf16), _ptr(out), n_tokens,
                                        _ptr(ws), ws_bytes, _stream(stream)))


def moe_combine(desc, o, pair_slot, topk_w, n_tokens, residual, y, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(desc), _ptr(o), _ptr(pair_slot),
                                            _ptr(topk_w), n_tokens, _ptr(residual), _ptr(y),
                                            _stream(stream)))


def moe_decode_layer(desc, bank, w_router, bias, x, n_tokens, norm_eps, residual, y, topk_ids,
                     topk_w, ws, ws_bytes, stages=None, stream=None):
    _check("moe_decode_layer",
           lib().moe_decode_layer(ctypes.byref(desc), ctypes.byref(bank), _ptr(w_router),
                                  _ptr(bias), _ptr(x), n_tokens, float(norm_eps), _ptr(residual),
                                  _ptr(y), _ptr(topk_ids), _ptr(topk_w),
                                  MOE_DECODE_ALL if stages is None else stages, _ptr(ws),
                                  ws_bytes, _stream(stream)))


def moe_decode_layer_noalloc(desc, bank, w_router, bias, x, n_tokens, norm_eps, residual, y,
                             topk_ids, topk_w, stages=None, stream=None):
    _check("moe_decode_layer_noalloc",
           lib().moe_decode_layer_noalloc(ctypes.byref(desc), ctypes.byref(bank), _ptr(w_router),
                                          _ptr(bias), _ptr(x), n_tokens, float(norm_eps),
                                          _ptr(residual), _ptr(y), _ptr(topk_ids), _ptr(topk_w),
                                          MOE_DECODE_ALL if stages is None else stages,
                                          _stream(stream)))


def make_layers(layers):
    """ctypes array of moe_layer from (bank, w_router, bias) triples (bank: moe_bank)."""
    arr = (moe_layer * max(1, len(layers)))()
    for i, (bank, wr, bias) in enumerate(layers):
        arr[i] = moe_layer(bank, _ptr(wr), _ptr(bias))
    return arr


def moe_decode_chain(desc, layers, n_layers, x, n_tokens, norm_eps, topk_ids, topk_w, ws,
                     ws_bytes, stream=None):
    """layers: the ctypes array of make_layers (or a list of triples)."""
    if not isinstance(layers, ctypes.Array):
        layers = make_layers(layers)
    _check("moe_decode_chain",
           lib().moe_decode_chain(ctypes.byref(desc), layers, n_layers, _ptr(x), n_tokens,
                                  float(norm_eps), _ptr(topk_ids), _ptr(topk_w), _ptr(ws),
                                  ws_bytes, _stream(stream)))


def moe_rmsnorm(x, n_tokens, hidden, eps, y, stream=None):
    _check("moe_rmsnorm", lib().moe_rmsnorm(_ptr(x), n_tokens, hidden, float(eps), _ptr(y),
                                            _stream(stream)))
