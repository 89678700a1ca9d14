"""Seeded synthetic inputs shared by the GPU path's tests, the oracle and the benchmark.

Holds no attention arithmetic: only the counter-based normal generator defined in
``synth.c`` (SplitMix64 stream + Box-Muller, rounded to bf16), the workload shapes, and
bf16 bit helpers.  Tensor ids: Q=0, K=1, V=2.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(verbose=False):
    """Compile libsynth.so with gcc (plain C, OpenMP)."""
    import subprocess
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           os.path.join(_HERE, "synth.c"), "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                                          ctypes.c_void_p, ctypes.c_int64]
        lib.synth_normal_bf16.restype = None
        lib.synth_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                       ctypes.c_int64]
        lib.synth_uniforms.restype = None
        lib.synth_bf16_from_double.argtypes = [ctypes.c_double]
        lib.synth_bf16_from_double.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def normal_bf16(seed, tensor_id, shape, mult=1.0):
    """bf16 bit patterns (numpy uint16) of mult * N(0,1), stream (seed, tensor_id)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load().synth_normal_bf16(seed, tensor_id, float(mult), out.ctypes.data, n)
    return out.reshape(shape)


def uniforms(seed, tensor_id, n):
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniforms(seed, tensor_id, out.ctypes.data, n)
    return out


def bf16_from_double(x):
    return int(_load().synth_bf16_from_double(float(x)))


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 bit patterns (nearest, ties to even)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32(x):
    """Round a Python float to the nearest float32 value (returned as a Python float)."""
    return float(np.float32(x))


# Workloads: the shapes of the pages' examples.  `mult` scales N(0,1) before rounding.
WORKLOADS = {
    "tiny_mha": dict(B=1, Sq=256, Sk=256, Hq=2, Hkv=2, d=64, causal=False,
                     scale=f32(1 / 8.0), seed=1, mult=1.0),
    "causal_prefill": dict(B=4, Sq=4096, Sk=4096, Hq=16, Hkv=16, d=128, causal=True,
                           scale=f32(1 / np.sqrt(128.0)), seed=2, mult=1.0),
    "ragged_noncausal": dict(B=2, Sq=5000, Sk=5000, Hq=8, Hkv=8, d=64, causal=False,
                             scale=f32(1 / 8.0), seed=3, mult=1.0),
    "ragged_causal": dict(B=2, Sq=5000, Sk=5000, Hq=8, Hkv=8, d=64, causal=True,
                          scale=f32(1 / 8.0), seed=3, mult=1.0),
    "gqa_decode": dict(B=8, Sq=1, Sk=32768, Hq=32, Hkv=8, d=128, causal=False,
                       scale=f32(1 / np.sqrt(128.0)), seed=4, mult=1.0),
    # gqa_decode's keys and values held in a paged cache of 256-position blocks, dealt to
    # the batches in a seeded random order (block_table)
    "paged_decode": dict(B=8, Sq=1, Sk=32768, Hq=32, Hkv=8, d=128, causal=False,
                         scale=f32(1 / np.sqrt(128.0)), seed=4, mult=1.0, page=256),
    "long_causal_gqa": dict(B=1, Sq=16384, Sk=16384, Hq=32, Hkv=8, d=128, causal=True,
                            scale=f32(1 / np.sqrt(128.0)), seed=5, mult=0.5),
    # long_causal_gqa's tensors with a causal sliding window: each query sees itself and
    # the 4095 keys before it (window_left = 4095, window_right = 0)
    "sliding_window_gqa": dict(B=1, Sq=16384, Sk=16384, Hq=32, Hkv=8, d=128, causal=True,
                               scale=f32(1 / np.sqrt(128.0)), seed=5, mult=0.5,
                               window_left=4095, window_right=0),
    # causal_prefill's tensors, quantized to FP8 E4M3 with 128-row block scales
    "causal_prefill_fp8": dict(B=4, Sq=4096, Sk=4096, Hq=16, Hkv=16, d=128, causal=True,
                               scale=f32(1 / np.sqrt(128.0)), seed=2, mult=1.0, fp8=True),
    # long_causal_gqa's tensors in FP8
    "long_causal_gqa_fp8": dict(B=1, Sq=16384, Sk=16384, Hq=32, Hkv=8, d=128, causal=True,
                                scale=f32(1 / np.sqrt(128.0)), seed=5, mult=0.5, fp8=True),
    # causal_prefill's 16384 tokens as a packed batch of sequences of mixed length
    # (seq_lengths: uniform on [1, 4096]); q/k/v [16384, H, d], cu_seqlens prefix sums
    "varlen_prefill": dict(total=16384, max_len=4096, Hq=16, Hkv=16, d=128, causal=True,
                           scale=f32(1 / np.sqrt(128.0)), seed=6, mult=1.0),
}


def seq_lengths(seed, tensor_id, total, max_len, min_len=1):
    """Sequence lengths, each uniform on [min_len, max_len], drawn until they reach total
    tokens (the last one is cut so that they sum to total exactly)."""
    u = uniforms(seed, tensor_id, total)
    out, acc = [], 0
    for x in u:
        if acc >= total:
            break
        n = min_len + int(x * (max_len - min_len + 1))
        n = min(n, max_len, total - acc)
        out.append(n)
        acc += n
    return out


def prefix_sums(lengths):
    """[0, l0, l0+l1, ...] as int32."""
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def make_qkv(w):
    """(q, k, v) bf16 bit arrays for workload dict w: q [B,Sq,Hq,d], k/v [B,Sk,Hkv,d]."""
    q = normal_bf16(w["seed"], 0, (w["B"], w["Sq"], w["Hq"], w["d"]), w["mult"])
    k = normal_bf16(w["seed"], 1, (w["B"], w["Sk"], w["Hkv"], w["d"]), w["mult"])
    v = normal_bf16(w["seed"], 2, (w["B"], w["Sk"], w["Hkv"], w["d"]), w["mult"])
    return q, k, v


def make_varlen_qkv(w):
    """(q, k, v, lengths) for a packed workload: lengths from seq_lengths (stream 9), q
    [total,Hq,d], k/v [total,Hkv,d] bf16 bits; keys and queries share the lengths."""
    lengths = seq_lengths(w["seed"], 9, w["total"], w["max_len"])
    q = normal_bf16(w["seed"], 0, (w["total"], w["Hq"], w["d"]), w["mult"])
    k = normal_bf16(w["seed"], 1, (w["total"], w["Hkv"], w["d"]), w["mult"])
    v = normal_bf16(w["seed"], 2, (w["total"], w["Hkv"], w["d"]), w["mult"])
    return q, k, v, lengths
