"""CPU oracle for the attention forward and backward passes -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The GPU library never loads it and it never loads the GPU
library.  The arithmetic lives in ``oracle.c`` (plain C, double precision); this module
only marshals numpy arrays into it.

Functions (all return float64 numpy arrays):
  fwd(q, k, v, causal, scale)             -> (o [B,Sq,Hq,d], lse [B,Hq,Sq])   plain definition
  rows(q, k, v, causal, scale, rows)      -> (o [n,d], lse [n])               same, chosen rows
  probs(q, k, v, causal, scale, b, h, i)  -> P [Sk]                           probability row
  online(q, k, v, causal, scale, blk)     -> (o, lse)                         per-row online loop
  split(q, k, v, causal, scale, blk, S)   -> (o_part, lse_part, o, lse)       split + combine
  bwd(q, k, v, dout, causal, scale[, units]) -> (dq, dk, dv, dsum, (dq_abs, dk_abs, dv_abs))
                                             backward; dsum = D per row [B,Hq,Sq]; *_abs =
                                             sums of absolute terms (for error bounds)

Inputs are either float64 arrays or uint16 arrays holding bf16 bit patterns (widened
exactly).  q is [B,Sq,Hq,d]; k and v are [B,Sk,Hkv,d].
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCE = os.path.join(_HERE, "oracle.c")


def build(src=SOURCE, out=LIB_PATH, verbose=False):
    """Compile the oracle with gcc: -O2, OpenMP, no FP contraction, baseline x86-64 ISA."""
    import subprocess
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
           src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


_I = ctypes.c_int
_P = ctypes.c_void_p
_D = ctypes.c_double
_COMMON = [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _D]


class Oracle:
    def __init__(self, lib_path=LIB_PATH):
        if lib_path == LIB_PATH and not os.path.exists(lib_path):
            build()
        lib = ctypes.CDLL(lib_path)
        lib.oracle_attn_fwd.argtypes = _COMMON + [_P, _P]
        lib.oracle_attn_rows.argtypes = _COMMON + [_I, _P, _P, _P]
        lib.oracle_attn_probs.argtypes = _COMMON + [_I, _I, _I, _P]
        lib.oracle_attn_online.argtypes = _COMMON + [_I, _P, _P]
        lib.oracle_attn_split.argtypes = _COMMON + [_I, _I, _P, _P, _P, _P]
        lib.oracle_attn_bwd.argtypes = _COMMON + [_P, _P, _P, _P, _P, _P, _P, _P, _P]
        for f in ("oracle_attn_fwd", "oracle_attn_rows", "oracle_attn_probs",
                  "oracle_attn_online", "oracle_attn_split", "oracle_attn_bwd"):
            getattr(lib, f).restype = ctypes.c_int
        self.lib = lib

    @staticmethod
    def _prep(q, k, v):
        arrs = [np.ascontiguousarray(x) for x in (q, k, v)]
        dt = arrs[0].dtype
        if any(a.dtype != dt for a in arrs):
            raise TypeError("q, k, v must share a dtype")
        if dt == np.uint16:
            in_bf16 = 1
        elif dt == np.float64:
            in_bf16 = 0
        else:
            raise TypeError("oracle inputs are float64 or bf16 bit patterns (uint16)")
        q_, k_, v_ = arrs
        if q_.ndim != 4 or k_.ndim != 4 or v_.ndim != 4 or k_.shape != v_.shape:
            raise ValueError("q [B,Sq,Hq,d], k/v [B,Sk,Hkv,d]")
        B, Sq, Hq, d = q_.shape
        Bk, Sk, Hkv, dk = k_.shape
        if Bk != B or dk != d:
            raise ValueError("batch / head_dim mismatch")
        return arrs, in_bf16, (B, Sq, Sk, Hq, Hkv, d)

    def _args(self, q, k, v, causal, scale):
        arrs, in_bf16, dims = self._prep(q, k, v)
        return arrs, dims, [in_bf16] + [a.ctypes.data for a in arrs] + list(dims) + \
            [int(bool(causal)), float(scale)]

    @staticmethod
    def _ok(rc, name):
        if rc != 0:
            raise ValueError(f"{name} returned {rc}")

    def fwd(self, q, k, v, causal, scale):
        arrs, (B, Sq, Sk, Hq, Hkv, d), a = self._args(q, k, v, causal, scale)
        o = np.zeros((B, Sq, Hq, d))
        lse = np.zeros((B, Hq, Sq))
        self._ok(self.lib.oracle_attn_fwd(*a, o.ctypes.data, lse.ctypes.data), "fwd")
        return o, lse

    def rows(self, q, k, v, causal, scale, rows):
        arrs, (B, Sq, Sk, Hq, Hkv, d), a = self._args(q, k, v, causal, scale)
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
        o = np.zeros((len(r), d))
        lse = np.zeros(len(r))
        self._ok(self.lib.oracle_attn_rows(*a, len(r), r.ctypes.data, o.ctypes.data,
                                           lse.ctypes.data), "rows")
        return o, lse

    def probs(self, q, k, v, causal, scale, b, h, i):
        arrs, (B, Sq, Sk, Hq, Hkv, d), a = self._args(q, k, v, causal, scale)
        p = np.zeros(Sk)
        self._ok(self.lib.oracle_attn_probs(*a, b, h, i, p.ctypes.data), "probs")
        return p

    def online(self, q, k, v, causal, scale, blk):
        arrs, (B, Sq, Sk, Hq, Hkv, d), a = self._args(q, k, v, causal, scale)
        o = np.zeros((B, Sq, Hq, d))
        lse = np.zeros((B, Hq, Sq))
        self._ok(self.lib.oracle_attn_online(*a, int(blk), o.ctypes.data, lse.ctypes.data),
                 "online")
        return o, lse

    def split(self, q, k, v, causal, scale, blk, num_splits):
        arrs, (B, Sq, Sk, Hq, Hkv, d), a = self._args(q, k, v, causal, scale)
        S = int(num_splits)
        op = np.zeros((S, B, Hq, Sq, d))
        lp = np.zeros((S, B, Hq, Sq))
        o = np.zeros((B, Sq, Hq, d))
        lse = np.zeros((B, Hq, Sq))
        self._ok(self.lib.oracle_attn_split(*a, int(blk), S, op.ctypes.data, lp.ctypes.data,
                                            o.ctypes.data, lse.ctypes.data), "split")
        return op, lp, o, lse

    def bwd(self, q, k, v, dout, causal, scale, units=None):
        """units: None (all) or an iterable of (b, hk) key/value units to compute; the
        other units' slices of every output stay zero."""
        arrs, (B, Sq, Sk, Hq, Hkv, d), a = self._args(q, k, v, causal, scale)
        do_ = np.ascontiguousarray(dout)
        if do_.dtype != arrs[0].dtype or do_.shape != arrs[0].shape:
            raise ValueError("dout must match q in dtype and shape")
        umask = None
        if units is not None:
            umask = np.zeros(B * Hkv, dtype=np.int32)
            for b, hk in units:
                umask[b * Hkv + hk] = 1
        dq = np.zeros((B, Sq, Hq, d))
        dk = np.zeros((B, Sk, Hkv, d))
        dv = np.zeros((B, Sk, Hkv, d))
        dsum = np.zeros((B, Hq, Sq))
        dq_a, dk_a, dv_a = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
        self._ok(self.lib.oracle_attn_bwd(*a, do_.ctypes.data,
                                          None if umask is None else umask.ctypes.data,
                                          dq.ctypes.data, dk.ctypes.data,
                                          dv.ctypes.data, dsum.ctypes.data, dq_a.ctypes.data,
                                          dk_a.ctypes.data, dv_a.ctypes.data), "bwd")
        return dq, dk, dv, dsum, (dq_a, dk_a, dv_a)


_default = None


def get():
    """The oracle built from this directory's oracle.c."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
