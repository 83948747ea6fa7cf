"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

The streams are defined in ``synth/synth.h`` (SplitMix64 counters, Box-Muller
normals, modular token ids, fp64 uniforms).  This module holds no arithmetic of
the decoding method.  ``libsynth.so`` (host, C + OpenMP) is always used for
CPU-side inputs; ``libsynth_dev.so`` (HIP) fills large device tensors with the
same values.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_host = None
_dev = None

# Seeds of the synthetic workloads: weights, prompts, uniforms.
SEED_WEIGHTS = 0x5EED0001
SEED_PROMPTS = 0x5EED0002
SEED_UNIFORMS = 0x5EED0003
WEIGHT_STD = 0.02

# Tensor ids used in the weight stream ids (same numbering as the C ABI).
T_EMBED, T_ATTN_NORM, T_WQ, T_WK, T_WV, T_WO, T_FFN_NORM, T_W_GATE, T_W_UP, T_W_DOWN, T_FINAL_NORM, T_HEAD = range(12)


def stream_weight(tensor, layer):
    return (tensor + 1) * 0x10000 + layer


def stream_prompt(request):
    return 0x20000000 + request


def stream_uniform(request, rnd):
    return 0x40000000 + request * 0x10000 + rnd


SEED_WORKLOAD = 0x5EED0004  # per-request context lengths and draft lengths of ragged batches
SEED_KV = 0x5EED0005        # committed K/V written straight into the cache by the generator


def stream_workload(what):
    return 0x60000000 + what


def stream_kv(layer, kind):
    """kind 0 = K pool, 1 = V pool of a layer."""
    return 0x70000000 + layer * 2 + kind


def _lib():
    global _host
    if _host is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError("synth/libsynth.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        u64, sz = ctypes.c_uint64, ctypes.c_size_t
        lib.synth_at.restype = u64
        lib.synth_at.argtypes = [u64, u64]
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64]
        for name in ("synth_normal_f32", "synth_normal_bf16"):
            getattr(lib, name).argtypes = [u64, u64, ctypes.c_double, u64, sz, ctypes.c_void_p]
            getattr(lib, name).restype = None
        lib.synth_tokens.argtypes = [u64, u64, ctypes.c_int32, u64, sz, ctypes.c_void_p]
        lib.synth_tokens.restype = None
        lib.synth_uniforms.argtypes = [u64, u64, u64, sz, ctypes.c_void_p]
        lib.synth_uniforms.restype = None
        _host = lib
    return _host


def at(key, i):
    return int(_lib().synth_at(key, i))


def key(seed, stream):
    return int(_lib().synth_key(seed, stream))


def normal_f32(seed, stream, n, std=WEIGHT_STD, first=0):
    out = np.empty(n, dtype=np.float32)
    _lib().synth_normal_f32(seed, stream, std, first, n, out.ctypes.data)
    return out


def normal_bf16_bits(seed, stream, n, std=WEIGHT_STD, first=0):
    """bf16 bit patterns (uint16) of the normal stream."""
    out = np.empty(n, dtype=np.uint16)
    _lib().synth_normal_bf16(seed, stream, std, first, n, out.ctypes.data)
    return out


def tokens(seed, stream, vocab, n, first=0):
    out = np.empty(n, dtype=np.int32)
    _lib().synth_tokens(seed, stream, vocab, first, n, out.ctypes.data)
    return out


def uniforms(seed, stream, n, first=0):
    out = np.empty(n, dtype=np.float64)
    _lib().synth_uniforms(seed, stream, first, n, out.ctypes.data)
    return out


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dev_normal_bf16(seed, stream, n, d_ptr, hip_stream, std=WEIGHT_STD, first=0):
    """Fill n bf16 elements at device address d_ptr on the given HIP stream."""
    global _dev
    if _dev is None:
        path = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError("synth/libsynth_dev.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_dev_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double, ctypes.c_uint64,
                                              ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_dev_normal_bf16.restype = ctypes.c_int
        _dev = lib
    rc = _dev.synth_dev_normal_bf16(seed, stream, std, first, n, d_ptr, hip_stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_normal_bf16 failed ({rc})")
