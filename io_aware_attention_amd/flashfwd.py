"""ctypes binding for libflashfwd (include/flashfwd.h): same names, same arguments.

Argument marshalling only -- every step of the attention path runs in the library's
HIP kernels.  Tensor arguments may be torch tensors (their ``data_ptr()`` is passed) or
raw integer device addresses; ``stream`` may be a torch stream, an integer hipStream_t or
None (the null stream).  A non-zero status raises ``FlashFwdError``.  Loading fails loudly
when the library has not been built: there is no other implementation to fall back to.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflashfwd.so")

FF_OK = 0
FF_MAX_SPLITS = 128
FF_SPLIT_BLOCK_N = 128
STATUS_NAMES = {0: "FF_OK", 1: "FF_ERR_NULL", 2: "FF_ERR_SHAPE", 3: "FF_ERR_HEADDIM",
                4: "FF_ERR_GQA", 5: "FF_ERR_ALIGN", 6: "FF_ERR_SPLITS", 7: "FF_ERR_SCALE",
                8: "FF_ERR_HIP", 9: "FF_ERR_ALIAS", 10: "FF_ERR_OPTION", 11: "FF_ERR_SCRATCH"}
FF_NOALLOC_SCRATCH_FLOATS = 4 << 20
EXPORTS = ("attn_fwd", "attn_fwd_ex", "attn_fwd_varlen", "attn_splitkv_num_splits",
           "attn_splits_efficiency_rule", "attn_fwd_splitkv", "attn_splitkv_combine",
           "attn_fwd_kvcache", "attn_fwd_kvcache_ex", "attn_kvcache_append",
           "attn_quantize_fp8", "attn_fwd_fp8", "attn_bwd_workspace_floats", "attn_bwd",
           "attn_bwd_ex", "attn_fwd_splitkv_noalloc", "attn_status_string")


class FlashFwdError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({status_string(status)})")


_lib = None


def _share_hip_runtime():
    """Load torch's HIP runtime first, when torch is installed.

    The library needs libamdhip64.so.7.  PyTorch ships its own copy with the same soname;
    whichever copy is loaded first is the one the process uses.  Loading this library
    before torch would put two HIP runtimes in the process, and device pointers from
    torch would then be invalid in the library's runtime."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def load(path=LIB_PATH):
    """Load libflashfwd.so once; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libflashfwd is not built ({path} missing); run "
                          f"`python __graft_entry__.py build` or io_aware_attention_amd/build.py")
    _share_hip_runtime()
    lib = ctypes.CDLL(os.path.abspath(path))
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, P]
    lib.attn_fwd_ex.argtypes = [P] * 5 + [I] * 9 + [P, I, F, F, P]
    lib.attn_fwd_varlen.argtypes = [P] * 7 + [I] * 8 + [F, P]
    lib.attn_splitkv_num_splits.argtypes = [I, I, I, I, I, I, I]
    lib.attn_splits_efficiency_rule.argtypes = [I, I, I]
    lib.attn_fwd_splitkv.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.attn_splitkv_combine.argtypes = [P, P, P, P, I, I, I, I, I, P]
    lib.attn_fwd_kvcache.argtypes = [P] * 10 + [I] * 10 + [F, I, P]
    lib.attn_fwd_kvcache_ex.argtypes = [P] * 10 + [I] * 12 + [P, I, F, F, I, P]
    lib.attn_kvcache_append.argtypes = [P] * 6 + [I] * 7 + [P]
    lib.attn_quantize_fp8.argtypes = [P, P, P, I, I, I, I, I, P]
    lib.attn_fwd_fp8.argtypes = [P] * 8 + [I] * 7 + [F, P]
    lib.attn_bwd_workspace_floats.argtypes = [I, I, I]
    lib.attn_bwd.argtypes = [P] * 10 + [I, I, I, I, I, I, I, F, P]
    lib.attn_bwd_ex.argtypes = [P] * 10 + [I] * 9 + [P, I, F, F, P]
    lib.attn_fwd_splitkv_noalloc.argtypes = [P] * 5 + [I] * 7 + [F, I, P]
    lib.attn_status_string.argtypes = [I]
    lib.attn_status_string.restype = ctypes.c_char_p
    for name in EXPORTS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    lib.attn_bwd_workspace_floats.restype = ctypes.c_longlong
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc, where):
    if rc != FF_OK:
        raise FlashFwdError(rc, where)


def status_string(status):
    return load().attn_status_string(int(status)).decode()


def attn_status_string(status):
    return status_string(status)


def attn_fwd(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, causal, scale, stream=None):
    _check(load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Sq, Sk, Hq, Hkv,
                           d, int(bool(causal)), float(scale), _stream(stream)), "attn_fwd")


def attn_fwd_ex(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, causal, window_left, window_right,
                alibi_slopes, alibi_batch_stride, softcap, scale, stream=None):
    _check(load().attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Sq, Sk, Hq, Hkv,
                              d, int(bool(causal)), int(window_left), int(window_right),
                              _ptr(alibi_slopes), int(alibi_batch_stride), float(softcap),
                              float(scale), _stream(stream)), "attn_fwd_ex")


def attn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, total_q,
                    total_k, Hq, Hkv, d, causal, scale, stream=None):
    _check(load().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                  _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, max_seqlen_q,
                                  total_q, total_k, Hq, Hkv, d, int(bool(causal)), float(scale),
                                  _stream(stream)), "attn_fwd_varlen")


def attn_splitkv_num_splits(B, Sq, Sk, Hq, Hkv, d, num_cus=0):
    r = load().attn_splitkv_num_splits(B, Sq, Sk, Hq, Hkv, d, num_cus)
    if r < 1:
        raise FlashFwdError(-r, "attn_splitkv_num_splits")
    return r


def attn_splits_efficiency_rule(units, slots, max_splits):
    r = load().attn_splits_efficiency_rule(units, slots, max_splits)
    if r < 1:
        raise FlashFwdError(-r, "attn_splits_efficiency_rule")
    return r


def attn_fwd_splitkv(q, k, v, o_accum, lse_accum, o, lse, B, Sq, Sk, Hq, Hkv, d, causal, scale,
                     num_splits, stream=None):
    _check(load().attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o_accum), _ptr(lse_accum),
                                   _ptr(o), _ptr(lse), B, Sq, Sk, Hq, Hkv, d, int(bool(causal)),
                                   float(scale), int(num_splits), _stream(stream)),
           "attn_fwd_splitkv")


def attn_splitkv_combine(o_accum, lse_accum, o, lse, B, Sq, Hq, d, num_splits, stream=None):
    _check(load().attn_splitkv_combine(_ptr(o_accum), _ptr(lse_accum), _ptr(o), _ptr(lse), B,
                                       Sq, Hq, d, int(num_splits), _stream(stream)),
           "attn_splitkv_combine")


def attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, causal, scale,
                             num_splits, stream=None):
    _check(load().attn_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Sq,
                                           Sk, Hq, Hkv, d, int(bool(causal)), float(scale),
                                           int(num_splits), _stream(stream)),
           "attn_fwd_splitkv_noalloc")


def attn_fwd_kvcache(q, k_cache, v_cache, cache_seqlens, cache_leftpad, block_table, o_accum,
                     lse_accum, o, lse, B, Sq, Hq, Hkv, d, num_blocks, page_size,
                     max_blocks_per_seq, new_keys, causal, scale, num_splits, stream=None):
    _check(load().attn_fwd_kvcache(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens), _ptr(cache_leftpad),
        _ptr(block_table), _ptr(o_accum), _ptr(lse_accum), _ptr(o), _ptr(lse), B, Sq, Hq, Hkv,
        d, num_blocks, page_size, max_blocks_per_seq, new_keys, int(bool(causal)),
        float(scale), int(num_splits), _stream(stream)), "attn_fwd_kvcache")


def attn_fwd_kvcache_ex(q, k_cache, v_cache, cache_seqlens, cache_leftpad, block_table,
                        o_accum, lse_accum, o, lse, B, Sq, Hq, Hkv, d, num_blocks, page_size,
                        max_blocks_per_seq, new_keys, causal, window_left, window_right,
                        alibi_slopes, alibi_batch_stride, softcap, scale, num_splits,
                        stream=None):
    _check(load().attn_fwd_kvcache_ex(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens), _ptr(cache_leftpad),
        _ptr(block_table), _ptr(o_accum), _ptr(lse_accum), _ptr(o), _ptr(lse), B, Sq, Hq, Hkv,
        d, num_blocks, page_size, max_blocks_per_seq, new_keys, int(bool(causal)),
        int(window_left), int(window_right), _ptr(alibi_slopes), int(alibi_batch_stride),
        float(softcap), float(scale), int(num_splits), _stream(stream)), "attn_fwd_kvcache_ex")


def attn_kvcache_append(k_new, v_new, k_cache, v_cache, cache_seqlens, block_table, B, S_new,
                        Hkv, d, num_blocks, page_size, max_blocks_per_seq, stream=None):
    _check(load().attn_kvcache_append(
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens),
        _ptr(block_table), B, S_new, Hkv, d, num_blocks, page_size, max_blocks_per_seq,
        _stream(stream)), "attn_kvcache_append")


def attn_quantize_fp8(x, x_fp8, scales, B, S, H, d, rotate, stream=None):
    _check(load().attn_quantize_fp8(_ptr(x), _ptr(x_fp8), _ptr(scales), B, S, H, d,
                                    int(bool(rotate)), _stream(stream)), "attn_quantize_fp8")


def attn_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, B, Sq, Sk, Hq, Hkv, d, causal,
                 scale, stream=None):
    _check(load().attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale),
                               _ptr(v_scale), _ptr(o), _ptr(lse), B, Sq, Sk, Hq, Hkv, d,
                               int(bool(causal)), float(scale), _stream(stream)), "attn_fwd_fp8")


def attn_bwd_workspace_floats(B, Sq, Hq):
    r = load().attn_bwd_workspace_floats(B, Sq, Hq)
    if r < 0:
        raise FlashFwdError(-r, "attn_bwd_workspace_floats")
    return r


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Sq, Sk, Hq, Hkv, d, causal, scale,
             stream=None):
    _check(load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                           _ptr(dk), _ptr(dv), _ptr(ws), B, Sq, Sk, Hq, Hkv, d, int(bool(causal)),
                           float(scale), _stream(stream)), "attn_bwd")


def attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Sq, Sk, Hq, Hkv, d, causal,
                window_left, window_right, alibi_slopes, alibi_batch_stride, softcap, scale,
                stream=None):
    _check(load().attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), B, Sq, Sk, Hq, Hkv, d,
                              int(bool(causal)), int(window_left), int(window_right),
                              _ptr(alibi_slopes), int(alibi_batch_stride), float(softcap),
                              float(scale), _stream(stream)), "attn_bwd_ex")


# ---------------------------------------------------------------------------
# torch conveniences: allocate outputs with torch, then call the entry points above.

def _alibi_stride(alibi_slopes, Hq):
    """Batch stride of fp32 slopes [Hq] (0) or [B, Hq] (Hq); None for no slopes."""
    if alibi_slopes is None:
        return 0
    return 0 if alibi_slopes.dim() == 1 else Hq


def forward(q, k, v, causal, scale, stream=None, window=(-1, -1), alibi_slopes=None,
            softcap=0.0):
    """O [B,Sq,Hq,d] fp32 and LSE [B,Hq,Sq] fp32 from bf16 q [B,Sq,Hq,d], k/v [B,Sk,Hkv,d].
    window (left, right), fp32 alibi_slopes [Hq] or [B,Hq] and softcap select the mask and
    bias variants (attn_fwd_ex); without them this is attn_fwd."""
    import torch
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    o = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if tuple(window) == (-1, -1) and alibi_slopes is None and not softcap:
        attn_fwd(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, causal, scale, stream)
    else:
        attn_fwd_ex(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, causal, window[0], window[1],
                    alibi_slopes, _alibi_stride(alibi_slopes, Hq), softcap, scale, stream)
    return o, lse


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal, scale,
                   stream=None):
    """O [total_q,Hq,d] fp32 and LSE [Hq,total_q] fp32 from bf16 q [total_q,Hq,d] and k/v
    [total_k,Hkv,d], with int32 device prefix sums cu_seqlens_q/k [B+1]."""
    import torch
    total_q, Hq, d = q.shape
    total_k, Hkv, _ = k.shape
    B = cu_seqlens_q.numel() - 1
    o = torch.empty((total_q, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    attn_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, max_seqlen_q, total_q,
                    total_k, Hq, Hkv, d, causal, scale, stream)
    return o, lse


def forward_splitkv(q, k, v, causal, scale, num_splits=0, stream=None, return_partials=False):
    """Split-KV path: attn_fwd_splitkv then (num_splits > 1) attn_splitkv_combine.
    num_splits = 0 takes attn_splitkv_num_splits' choice."""
    import torch
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    if num_splits == 0:
        num_splits = attn_splitkv_num_splits(B, Sq, Sk, Hq, Hkv, d)
    o = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if num_splits == 1:
        attn_fwd_splitkv(q, k, v, None, None, o, lse, B, Sq, Sk, Hq, Hkv, d, causal, scale, 1,
                         stream)
        return (o, lse, None, None) if return_partials else (o, lse)
    oa = torch.empty((num_splits, B, Hq, Sq, d), dtype=torch.float32, device=q.device)
    la = torch.empty((num_splits, B, Hq, Sq), dtype=torch.float32, device=q.device)
    attn_fwd_splitkv(q, k, v, oa, la, None, None, B, Sq, Sk, Hq, Hkv, d, causal, scale,
                     num_splits, stream)
    attn_splitkv_combine(oa, la, o, lse, B, Sq, Hq, d, num_splits, stream)
    return (o, lse, oa, la) if return_partials else (o, lse)


def _cache_geometry(k_cache, block_table):
    if block_table is None:   # contiguous [B, capacity, Hkv, d]
        B, cap, Hkv, d = k_cache.shape
        return B, cap, 1, cap, Hkv, d
    num_blocks, page, Hkv, d = k_cache.shape
    max_blocks = block_table.shape[1]
    return num_blocks, page, max_blocks, max_blocks * page, Hkv, d


def forward_kvcache(q, k_cache, v_cache, cache_seqlens, causal, scale, block_table=None,
                    cache_leftpad=None, new_keys=0, num_splits=0, stream=None, window=(-1, -1),
                    alibi_slopes=None, softcap=0.0):
    """O [B,Sq,Hq,d] and LSE [B,Hq,Sq] (fp32) of bf16 q [B,Sq,Hq,d] against a key/value
    cache: paged [num_blocks, page, Hkv, d] with int32 block_table [B, max_blocks], or
    contiguous [B, capacity, Hkv, d] without one.  num_splits = 0 takes
    attn_splitkv_num_splits' choice for the capacity; more than one split goes through
    attn_splitkv_combine.  window, alibi_slopes and softcap as for forward (through
    attn_fwd_kvcache_ex)."""
    import torch
    B, Sq, Hq, d = q.shape
    num_blocks, page, max_blocks, cap, Hkv, _ = _cache_geometry(k_cache, block_table)
    if num_splits == 0:
        num_splits = attn_splitkv_num_splits(B, Sq, cap, Hq, Hkv, d)
    o = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    plain = tuple(window) == (-1, -1) and alibi_slopes is None and not softcap
    head = (B, Sq, Hq, Hkv, d, num_blocks, page, max_blocks, new_keys, causal)
    tail = (scale,) if plain else (window[0], window[1], alibi_slopes,
                                   _alibi_stride(alibi_slopes, Hq), softcap, scale)
    call = attn_fwd_kvcache if plain else attn_fwd_kvcache_ex
    if num_splits == 1:
        call(q, k_cache, v_cache, cache_seqlens, cache_leftpad, block_table, None, None, o, lse,
             *head, *tail, 1, stream)
        return o, lse
    oa = torch.empty((num_splits, B, Hq, Sq, d), dtype=torch.float32, device=q.device)
    la = torch.empty((num_splits, B, Hq, Sq), dtype=torch.float32, device=q.device)
    call(q, k_cache, v_cache, cache_seqlens, cache_leftpad, block_table, oa, la, None, None,
         *head, *tail, num_splits, stream)
    attn_splitkv_combine(oa, la, o, lse, B, Sq, Hq, d, num_splits, stream)
    return o, lse


def kvcache_append(k_new, v_new, k_cache, v_cache, cache_seqlens, block_table=None,
                   stream=None):
    """Writes k_new, v_new [B,S_new,Hkv,d] into the caches at cache_seqlens[b] + t."""
    B, S_new, Hkv, d = k_new.shape
    num_blocks, page, max_blocks, _, _, _ = _cache_geometry(k_cache, block_table)
    attn_kvcache_append(k_new, v_new, k_cache, v_cache, cache_seqlens, block_table, B, S_new,
                        Hkv, d, num_blocks, page, max_blocks, stream)


def quantize_fp8(x, rotate=False, stream=None):
    """E4M3 codes (torch.uint8, x's shape) and fp32 block scales [B,H,ceil(S/128)] of a bf16
    tensor x [B,S,H,d]; rotate applies the Walsh-Hadamard transform along d first."""
    import torch
    B, S, H, d = x.shape
    codes = torch.empty((B, S, H, d), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, H, -(-S // 128)), dtype=torch.float32, device=x.device)
    attn_quantize_fp8(x, codes, scales, B, S, H, d, rotate, stream)
    return codes, scales


def forward_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal, scale, stream=None):
    """O [B,Sq,Hq,d] and LSE [B,Hq,Sq] (fp32) from E4M3 q8 [B,Sq,Hq,d], k8/v8 [B,Sk,Hkv,d]
    and their block scales."""
    import torch
    B, Sq, Hq, d = q8.shape
    _, Sk, Hkv, _ = k8.shape
    o = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device=q8.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q8.device)
    attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, Sq, Sk, Hq, Hkv, d, causal,
                 scale, stream)
    return o, lse


def backward(q, k, v, o, lse, dout, causal, scale, stream=None, window=(-1, -1),
             alibi_slopes=None):
    """dq [B,Sq,Hq,d], dk and dv [B,Sk,Hkv,d] fp32 from bf16 q, k, v, dout and the fp32 o, lse
    of the forward (with the same window and ALiBi slopes); the workspace is allocated
    here."""
    import torch
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    dq = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, Sk, Hkv, d), dtype=torch.float32, device=q.device)
    dv = torch.empty((B, Sk, Hkv, d), dtype=torch.float32, device=q.device)
    ws = torch.empty(attn_bwd_workspace_floats(B, Sq, Hq), dtype=torch.float32, device=q.device)
    if tuple(window) == (-1, -1) and alibi_slopes is None:
        attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Sq, Sk, Hq, Hkv, d, causal, scale,
                 stream)
    else:
        attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Sq, Sk, Hq, Hkv, d, causal,
                    window[0], window[1], alibi_slopes, _alibi_stride(alibi_slopes, Hq), 0.0,
                    scale, stream)
    return dq, dk, dv
