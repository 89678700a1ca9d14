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
  varlen(q, k, v, cu_q, cu_k, causal, scale) -> (o [total_q,Hq,d], lse [Hq,total_q])
  kv_gather(k_cache, v_cache, block_table, seqlen, leftpad, b) -> (k, v) of batch b
  kvcache(q, k_cache, v_cache, block_table, seqlens, leftpad, causal, scale) -> (o, lse)
  append(k_new, v_new, k_cache, v_cache, block_table, seqlens) -> (k_cache', v_cache')
                                             backward; dsum = D per row [B,Hq,Sq]; *_abs =
                                             sums of absolute terms (for error bounds)

Inputs are either float64 arrays or uint16 arrays holding bf16 bit patterns (widened
exactly).  q is [B,Sq,Hq,d]; k and v are [B,Sk,Hkv,d].

fwd, rows, probs, online, split, varlen and kvcache also take the mask and bias variants
as keywords (the walk-through's Is_local, Has_alibi and Is_softcap):
  window=(left, right)   sliding window around diag = i + Sk - Sq; -1 = no limit
  alibi=slopes           [Hq] or [B, Hq]; -slope * |diag - j| is added to the score
  softcap=c              the scaled score s becomes c * tanh(s / c); 0 = none

FP8 (OCP E4M3; see oracle.c for the format, the block quantizer and the rotation):
  e4m3_decode(codes) -> float64;  e4m3_encode(x float32) -> uint8 codes
  fwht(rows float32 [..., d]) -> the rotated rows (float32)
  quantize_fp8(x, rotate=False) -> (codes uint8 [B,S,H,d], scales float32 [B,H,ceil(S/128)])
  dequantize_fp8(codes, scales) -> float64 [B,S,H,d]
  fwd_fp8(q8, k8, v8, qs, ks, vs, causal, scale) -> (o, lse, o_abs, inv_l)
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
_OPTS = [_I, _I, _P, _D]   # window_left, window_right, alibi [B, Hq], softcap
_FWD_FUNCS = ("oracle_attn_fwd", "oracle_attn_rows", "oracle_attn_probs",
              "oracle_attn_online", "oracle_attn_split")


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
        for f in _FWD_FUNCS + ("oracle_attn_bwd",):
            ext = getattr(lib, f + "_ext")
            ext.argtypes = _COMMON + _OPTS + getattr(lib, f).argtypes[len(_COMMON):]
            ext.restype = ctypes.c_int
        for f in _FWD_FUNCS + ("oracle_attn_bwd",):
            getattr(lib, f).restype = ctypes.c_int
        L = ctypes.c_int64
        lib.oracle_e4m3_decode.argtypes = [_P, L, _P]
        lib.oracle_e4m3_decode.restype = None
        lib.oracle_e4m3_encode.argtypes = [_P, L, _P]
        lib.oracle_e4m3_encode.restype = None
        lib.oracle_fwht_f32.argtypes = [_P, L, _I]
        lib.oracle_fwht_f32.restype = None
        lib.oracle_quantize_fp8.argtypes = [_I, _P, _I, _I, _I, _I, _I, _P, _P]
        lib.oracle_quantize_fp8.restype = ctypes.c_int
        lib.oracle_attn_fwd_fp8.argtypes = [_P] * 6 + [_I] * 7 + [_D, _P, _P, _P, _P]
        lib.oracle_attn_fwd_fp8.restype = ctypes.c_int
        self.lib = lib

    @staticmethod
    def _opts(B, Hq, window, alibi, softcap):
        """None for the plain problem, else (ctypes args, keep-alive array)."""
        wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
        if wl == -1 and wr == -1 and alibi is None and not softcap:
            return None
        slopes = None
        if alibi is not None:
            a = np.asarray(alibi, dtype=np.float64)
            slopes = np.ascontiguousarray(np.broadcast_to(a if a.ndim == 2 else a[None], (B, Hq)))
        return ([wl, wr, None if slopes is None else slopes.ctypes.data, float(softcap)], slopes)

    def _call(self, name, a, dims, opts, rest):
        """Calls name (plain) or name_ext (with the mask/bias options)."""
        B, Hq = dims[0], dims[3]
        o = self._opts(B, Hq, *opts)
        if o is None:
            rc = getattr(self.lib, name)(*a, *rest)
        else:
            rc = getattr(self.lib, name + "_ext")(*a, *o[0], *rest)
        self._ok(rc, name)

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

    def fwd(self, q, k, v, causal, scale, window=None, alibi=None, softcap=0.0):
        arrs, dims, a = self._args(q, k, v, causal, scale)
        B, Sq, Sk, Hq, Hkv, d = dims
        o = np.zeros((B, Sq, Hq, d))
        lse = np.zeros((B, Hq, Sq))
        self._call("oracle_attn_fwd", a, dims, (window, alibi, softcap),
                   [o.ctypes.data, lse.ctypes.data])
        return o, lse

    def rows(self, q, k, v, causal, scale, rows, window=None, alibi=None, softcap=0.0):
        arrs, dims, a = self._args(q, k, v, causal, scale)
        d = dims[5]
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
        o = np.zeros((len(r), d))
        lse = np.zeros(len(r))
        self._call("oracle_attn_rows", a, dims, (window, alibi, softcap),
                   [len(r), r.ctypes.data, o.ctypes.data, lse.ctypes.data])
        return o, lse

    def probs(self, q, k, v, causal, scale, b, h, i, window=None, alibi=None, softcap=0.0):
        arrs, dims, a = self._args(q, k, v, causal, scale)
        p = np.zeros(dims[2])
        self._call("oracle_attn_probs", a, dims, (window, alibi, softcap),
                   [b, h, i, p.ctypes.data])
        return p

    def online(self, q, k, v, causal, scale, blk, window=None, alibi=None, softcap=0.0):
        arrs, dims, a = self._args(q, k, v, causal, scale)
        B, Sq, Sk, Hq, Hkv, d = dims
        o = np.zeros((B, Sq, Hq, d))
        lse = np.zeros((B, Hq, Sq))
        self._call("oracle_attn_online", a, dims, (window, alibi, softcap),
                   [int(blk), o.ctypes.data, lse.ctypes.data])
        return o, lse

    def split(self, q, k, v, causal, scale, blk, num_splits, window=None, alibi=None,
              softcap=0.0):
        arrs, dims, a = self._args(q, k, v, causal, scale)
        B, Sq, Sk, Hq, Hkv, d = dims
        S = int(num_splits)
        op = np.zeros((S, B, Hq, Sq, d))
        lp = np.zeros((S, B, Hq, Sq))
        o = np.zeros((B, Sq, Hq, d))
        lse = np.zeros((B, Hq, Sq))
        self._call("oracle_attn_split", a, dims, (window, alibi, softcap),
                   [int(blk), S, op.ctypes.data, lp.ctypes.data, o.ctypes.data,
                    lse.ctypes.data])
        return op, lp, o, lse

    def bwd(self, q, k, v, dout, causal, scale, units=None, window=None, alibi=None):
        """units: None (all) or an iterable of (b, hk) key/value units to compute; the
        other units' slices of every output stay zero.  window (left, right) and alibi
        slopes as for fwd; the soft cap is not covered by the backward."""
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
        self._call("oracle_attn_bwd", a, (B, Sq, Sk, Hq, Hkv, d), (window, alibi, 0.0),
                   [do_.ctypes.data, None if umask is None else umask.ctypes.data,
                    dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, dsum.ctypes.data,
                    dq_a.ctypes.data, dk_a.ctypes.data, dv_a.ctypes.data])
        return dq, dk, dv, dsum, (dq_a, dk_a, dv_a)

    # -- FP8 (explainer, FlashAttention-3 precision section)

    def e4m3_decode(self, codes):
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(c.shape, dtype=np.float64)
        self.lib.oracle_e4m3_decode(c.ctypes.data, c.size, out.ctypes.data)
        return out

    def e4m3_encode(self, x):
        a = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(a.shape, dtype=np.uint8)
        self.lib.oracle_e4m3_encode(a.ctypes.data, a.size, out.ctypes.data)
        return out

    def fwht(self, rows):
        y = np.array(rows, dtype=np.float32, order="C", copy=True)
        d = y.shape[-1]
        self.lib.oracle_fwht_f32(y.ctypes.data, y.size // d, d)
        return y

    def quantize_fp8(self, x, rotate=False):
        """x: bf16 bits (uint16) or float32 [B,S,H,d]."""
        a = np.ascontiguousarray(x)
        if a.dtype == np.uint16:
            in_bf16 = 1
        elif a.dtype == np.float32:
            in_bf16 = 0
        else:
            raise TypeError("quantize_fp8 takes bf16 bits (uint16) or float32")
        B, S, H, d = a.shape
        codes = np.empty(a.shape, dtype=np.uint8)
        scales = np.empty((B, H, -(-S // 128)), dtype=np.float32)
        self._ok(self.lib.oracle_quantize_fp8(in_bf16, a.ctypes.data, B, S, H, d, int(bool(rotate)),
                                              codes.ctypes.data, scales.ctypes.data),
                 "quantize_fp8")
        return codes, scales

    def dequantize_fp8(self, codes, scales):
        S = codes.shape[1]
        blk = np.arange(S) // 128
        sc = np.asarray(scales, dtype=np.float64)[:, :, blk]       # [B, H, S]
        return self.e4m3_decode(codes) * sc.transpose(0, 2, 1)[..., None]

    def fwd_fp8(self, q8, k8, v8, q_scale, k_scale, v_scale, causal, scale):
        """The plain definition on the dequantized tensors: (o, lse, o_abs, inv_l)."""
        arrs = [np.ascontiguousarray(x, dtype=np.uint8) for x in (q8, k8, v8)]
        scs = [np.ascontiguousarray(x, dtype=np.float32) for x in (q_scale, k_scale, v_scale)]
        B, Sq, Hq, d = arrs[0].shape
        _, Sk, Hkv, _ = arrs[1].shape
        o = np.zeros((B, Sq, Hq, d))
        lse = np.zeros((B, Hq, Sq))
        o_abs = np.zeros((B, Sq, Hq, d))
        inv_l = np.zeros((B, Hq, Sq))
        self._ok(self.lib.oracle_attn_fwd_fp8(*[x.ctypes.data for x in arrs + scs], B, Sq, Sk,
                                              Hq, Hkv, d, int(bool(causal)), float(scale),
                                              o.ctypes.data, lse.ctypes.data, o_abs.ctypes.data,
                                              inv_l.ctypes.data), "fwd_fp8")
        return o, lse, o_abs, inv_l

    # -- variable-length batches and the paged KV cache ("03 forward CUDA kernel" section 8;
    # "flash attention V2 code walk-through": cu_seqlens as prefix sums, block_table, the
    # k_offset with leftpad_k).  Each sequence is an independent problem, so these are the
    # plain definition above applied per sequence to the rows the layout assigns to it.

    def varlen(self, q, k, v, cu_q, cu_k, causal, scale, **opts):
        """q [total_q,Hq,d], k/v [total_k,Hkv,d]; cu_q, cu_k prefix sums [B+1]: sequence b
        owns rows cu[b] .. cu[b+1]-1.  O [total_q,Hq,d] and LSE [Hq,total_q]."""
        total_q, Hq, d = q.shape
        o = np.zeros((total_q, Hq, d))
        lse = np.zeros((Hq, total_q))
        for b in range(len(cu_q) - 1):
            q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
            if q1 == q0:
                continue
            if k1 == k0:   # no key at all: O = 0, LSE = -inf
                lse[:, q0:q1] = -np.inf
                continue
            ob, lb = self.fwd(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], causal, scale,
                              **self._batch_opts(opts, b))
            o[q0:q1] = ob[0]
            lse[:, q0:q1] = lb[0]
        return o, lse

    @staticmethod
    def kv_gather(k_cache, v_cache, block_table, seqlen, leftpad, b):
        """Keys and values of batch b from a paged cache [num_blocks, page, Hkv, d]: logical
        cache position t lives in physical block block_table[b, t // page], row t % page;
        the sequence's keys are positions leftpad .. seqlen-1."""
        page = k_cache.shape[1]
        pos = np.arange(int(leftpad), int(seqlen))
        blk = np.asarray(block_table)[b, pos // page]
        return k_cache[blk, pos % page], v_cache[blk, pos % page]

    @staticmethod
    def _batch_opts(opts, b):
        """The options of batch b alone (ALiBi slopes [B, Hq] -> [Hq])."""
        al = opts.get("alibi")
        if al is not None and np.asarray(al).ndim == 2:
            opts = dict(opts, alibi=np.asarray(al)[b])
        return opts

    def kvcache(self, q, k_cache, v_cache, block_table, seqlens, leftpad, causal, scale,
                **opts):
        """q [B,Sq,Hq,d] against each batch's cached keys (kv_gather).  O [B,Sq,Hq,d], LSE
        [B,Hq,Sq]; a batch without keys gets O = 0, LSE = -inf."""
        B, Sq, Hq, d = q.shape
        o = np.zeros((B, Sq, Hq, d))
        lse = np.full((B, Hq, Sq), -np.inf)
        for b in range(B):
            lp = 0 if leftpad is None else int(leftpad[b])
            kb, vb = self.kv_gather(k_cache, v_cache, block_table, seqlens[b], lp, b)
            if len(kb) == 0:
                continue
            ob, lb = self.fwd(q[b:b + 1], kb[None], vb[None], causal, scale,
                              **self._batch_opts(opts, b))
            o[b], lse[b] = ob[0], lb[0]
        return o, lse

    @staticmethod
    def append(k_new, v_new, k_cache, v_cache, block_table, seqlens):
        """Copies of the caches with k_new[b, t], v_new[b, t] written at logical position
        seqlens[b] + t of batch b (positions past the table's capacity are dropped)."""
        kc, vc = k_cache.copy(), v_cache.copy()
        page = k_cache.shape[1]
        cap = np.asarray(block_table).shape[1] * page
        for b in range(k_new.shape[0]):
            for t in range(k_new.shape[1]):
                p = int(seqlens[b]) + t
                if p >= cap:
                    continue
                blk = block_table[b][p // page]
                kc[blk, p % page] = k_new[b, t]
                vc[blk, p % page] = v_new[b, t]
        return kc, vc


_default = None


def get():
    """The oracle built from this directory's oracle.c."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
