"""GPU twin of ``synth.generator``: fills torch CUDA tensors through libmoe_synth.so.

Same counter layout, key and Irwin-Hall transform as the host generator, so every value is
bit-identical to ``generator.normal_f32`` for the same (seed, cfg, layer, expert, tensor,
index).  Used to make multi-GB inputs without host generation or transfer.
"""
import ctypes
import os

from . import generator as G

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_synth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m quantized_moe_expert_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        l.synth_normal_f32.restype = ctypes.c_int32
        l.synth_normal_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                       ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_float, ctypes.c_void_p]
        l.synth_philox_words.restype = ctypes.c_int32
        l.synth_philox_words.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                         ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                         ctypes.c_uint32, ctypes.c_void_p]
        _lib = l
    return _lib


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def fill_normal(out, seed, cfg_id, layer, expert, tensor, start, sigma):
    """out (float32 CUDA tensor, contiguous) <- elements start .. start+numel-1 of a stream."""
    c2, c3 = G.stream_words(cfg_id, layer, expert, tensor)
    err = lib().synth_normal_f32(out.data_ptr(), out.numel(), int(start), seed & 0xFFFFFFFF,
                                 c2, c3, float(G.ih_scale(sigma)), _stream())
    if err:
        raise RuntimeError(f"synth_normal_f32: hip error {err}")


def philox_words(out, seed, key1, c2, c3, start=0):
    """out (int32/uint32 CUDA tensor of 4n words) <- raw Philox4x32-10 outputs."""
    err = lib().synth_philox_words(out.data_ptr(), out.numel() // 4, int(start), seed, key1,
                                   c2, c3, _stream())
    if err:
        raise RuntimeError(f"synth_philox_words: hip error {err}")
