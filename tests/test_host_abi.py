"""The C-ABI library on the CPU: it loads, exports every declared symbol, rejects bad
arguments before touching the GPU, and its split-count rule reproduces the forward-kernel
page's worked example.  No compute call is made here."""
import json
import math
import os
import re
import subprocess
import sys

import pytest

from io_aware_attention_amd import flashfwd as ff

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashfwd.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|long long|const char\*)\s+(\w+)\(", text, re.M)))


def test_header_matches_binding():
    assert declared_functions() == sorted(ff.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ff.load()
    out = subprocess.run(["nm", "-D", "--defined-only", ff.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings():
    for code in range(12):
        assert ff.status_string(code)
    assert ff.status_string(0) == "ok"


# Fake but aligned, distinct addresses: every call below must fail validation before any
# HIP call is made, so they are never dereferenced.
Q, K, V, O, L = 1 << 20, 2 << 30, 3 << 30, 4 << 32, 5 << 32
GOOD = dict(B=1, Sq=8, Sk=8, Hq=2, Hkv=1, d=64, causal=0, scale=0.125)


def call_fwd(q=Q, k=K, v=V, o=O, lse=L, **kw):
    a = dict(GOOD, **kw)
    return ff.load().attn_fwd(q, k, v, o, lse, a["B"], a["Sq"], a["Sk"], a["Hq"], a["Hkv"], a["d"],
                              a["causal"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(lse=None), 1),
    (dict(B=0), 2), (dict(Sq=0), 2), (dict(Sk=0), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2),
    (dict(d=96), 3), (dict(d=256), 3), (dict(Hq=3, Hkv=2), 4),
    (dict(q=Q + 8), 5), (dict(o=O + 4), 5),
    (dict(scale=0.0), 7), (dict(scale=-1.0), 7), (dict(scale=float("inf")), 7),
    (dict(scale=float("nan")), 7),
    (dict(o=Q), 9),
    (dict(B=1 << 12, Sq=1 << 12, Hq=1 << 4, d=128), 2),
])
def test_attn_fwd_rejects(kw, code):
    assert call_fwd(**kw) == code


AL = 17 << 32   # fake ALiBi slopes
XGOOD = dict(wl=-1, wr=-1, al=None, ast=0, cap=0.0)


def call_fwd_ex(q=Q, k=K, v=V, o=O, lse=L, **kw):
    a = dict(GOOD, **XGOOD)
    a.update(kw)
    return ff.load().attn_fwd_ex(q, k, v, o, lse, a["B"], a["Sq"], a["Sk"], a["Hq"], a["Hkv"],
                                 a["d"], a["causal"], a["wl"], a["wr"], a["al"], a["ast"],
                                 a["cap"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    # the plain checks still apply with options set
    (dict(q=None, wl=4), 1), (dict(B=0, cap=1.0), 2), (dict(d=96, al=AL), 3),
    (dict(scale=0.0, wr=2), 7), (dict(o=Q, wl=3), 9),
    # the options themselves
    (dict(wl=-2), 10), (dict(wr=-5), 10), (dict(cap=-1.0), 10), (dict(cap=float("inf")), 10),
    (dict(cap=float("nan")), 10), (dict(al=AL, ast=1), 10), (dict(al=AL, ast=3), 10),
    (dict(al=AL + 2), 5),
    (dict(al=O, ast=2), 9), (dict(al=L + 4), 9),
])
def test_attn_fwd_ex_rejects(kw, code):
    assert call_fwd_ex(**kw) == code


def test_attn_fwd_ex_batch_stride_ignored_without_slopes():
    # without slopes the stride is not looked at; the call fails on the scale instead
    assert call_fwd_ex(ast=7, scale=0.0) == 7


CQ, CK = 11 << 32, 12 << 32   # fake prefix-sum arrays
VGOOD = dict(B=2, max_q=8, total_q=12, total_k=12, Hq=2, Hkv=1, d=64, causal=1, scale=0.125)


def call_varlen(q=Q, k=K, v=V, o=O, lse=L, cq=CQ, ck=CK, **kw):
    a = dict(VGOOD, **kw)
    return ff.load().attn_fwd_varlen(q, k, v, o, lse, cq, ck, a["B"], a["max_q"], a["total_q"],
                                     a["total_k"], a["Hq"], a["Hkv"], a["d"], a["causal"],
                                     a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(cq=None), 1), (dict(ck=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(max_q=0), 2), (dict(total_q=0), 2), (dict(total_k=0), 2),
    (dict(max_q=13), 2), (dict(total_q=1 << 24, Hq=1 << 4, d=128), 2),
    (dict(d=80), 3), (dict(Hq=3, Hkv=2), 4),
    (dict(cq=CQ + 2), 5), (dict(k=K + 8), 5),
    (dict(scale=0.0), 7),
    (dict(o=K), 9), (dict(lse=CQ), 9), (dict(cq=O + 64), 9),
])
def test_attn_fwd_varlen_rejects(kw, code):
    assert call_varlen(**kw) == code


SL, LP, BT, VN = 13 << 32, 14 << 32, 15 << 32, 16 << 32   # seqlens, leftpad, table, v_new
KGOOD = dict(B=2, Sq=1, Hq=8, Hkv=2, d=128, nb=16, page=64, mb=8, new=0, causal=0,
             scale=0.1, S=1)


def call_kvcache(q=Q, kc=K, vc=V, sl=SL, lp=LP, bt=BT, oa=None, la=None, o=O, lse=L, **kw):
    a = dict(KGOOD, **kw)
    return ff.load().attn_fwd_kvcache(q, kc, vc, sl, lp, bt, oa, la, o, lse, a["B"], a["Sq"],
                                      a["Hq"], a["Hkv"], a["d"], a["nb"], a["page"], a["mb"],
                                      a["new"], a["causal"], a["scale"], a["S"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(sl=None), 1), (dict(kc=None), 1), (dict(o=None), 1), (dict(S=2), 1),
    (dict(S=0), 6), (dict(S=129), 6),
    (dict(B=0), 2), (dict(Sq=0), 2), (dict(page=0), 2), (dict(page=48), 2), (dict(nb=0), 2),
    (dict(mb=0), 2), (dict(new=-1), 2), (dict(mb=1 << 26), 2),
    (dict(d=96), 3), (dict(Hq=6, Hkv=4), 4),
    (dict(sl=SL + 2), 5), (dict(bt=BT + 1), 5), (dict(kc=K + 8), 5),
    (dict(scale=-1.0), 7),
    (dict(o=K), 9), (dict(lse=SL), 9), (dict(o=BT - 64), 9),
])
def test_attn_fwd_kvcache_rejects(kw, code):
    assert call_kvcache(**kw) == code


def call_kvcache_ex(q=Q, kc=K, vc=V, sl=SL, lp=LP, bt=BT, oa=None, la=None, o=O, lse=L, **kw):
    a = dict(KGOOD, **XGOOD)
    a.update(kw)
    return ff.load().attn_fwd_kvcache_ex(q, kc, vc, sl, lp, bt, oa, la, o, lse, a["B"], a["Sq"],
                                         a["Hq"], a["Hkv"], a["d"], a["nb"], a["page"], a["mb"],
                                         a["new"], a["causal"], a["wl"], a["wr"], a["al"],
                                         a["ast"], a["cap"], a["scale"], a["S"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(sl=None, wl=2), 1), (dict(S=0, cap=2.0), 6), (dict(page=48, al=AL), 2),
    (dict(Hq=6, Hkv=4, wr=0), 4), (dict(scale=-1.0, wl=1), 7), (dict(lse=SL, wl=1), 9),
    (dict(wl=-3), 10), (dict(cap=-0.5), 10), (dict(al=AL, ast=2), 10),
    (dict(al=AL + 1), 5), (dict(al=O + 16, ast=8), 9),
])
def test_attn_fwd_kvcache_ex_rejects(kw, code):
    assert call_kvcache_ex(**kw) == code


QS, KS, VS = 18 << 32, 19 << 32, 20 << 32   # fake scale arrays


def call_fwd_fp8(q=Q, k=K, v=V, qs=QS, ks=KS, vs=VS, o=O, lse=L, **kw):
    a = dict(GOOD, **kw)
    return ff.load().attn_fwd_fp8(q, k, v, qs, ks, vs, o, lse, a["B"], a["Sq"], a["Sk"], a["Hq"],
                                  a["Hkv"], a["d"], a["causal"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(qs=None), 1), (dict(vs=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(Sk=0), 2), (dict(d=96), 3), (dict(Hq=3, Hkv=2), 4),
    (dict(ks=KS + 4), 5), (dict(q=Q + 8), 5),
    (dict(scale=0.0), 7),
    (dict(o=QS - 16), 9), (dict(lse=VS), 9), (dict(o=K), 9),
])
def test_attn_fwd_fp8_rejects(kw, code):
    assert call_fwd_fp8(**kw) == code


def call_quantize(x=Q, x8=K, sc=QS, **kw):
    a = dict(dict(B=2, S=300, H=3, d=128, rotate=0), **kw)
    return ff.load().attn_quantize_fp8(x, x8, sc, a["B"], a["S"], a["H"], a["d"], a["rotate"],
                                       None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(sc=None), 1), (dict(B=0), 2), (dict(S=0), 2),
    (dict(S=1 << 24, H=1 << 4), 2), (dict(d=32), 3), (dict(x8=K + 4), 5),
    (dict(x8=Q + 512), 9), (dict(sc=Q + 64), 9), (dict(sc=K + 64), 9),
])
def test_attn_quantize_fp8_rejects(kw, code):
    assert call_quantize(**kw) == code


def test_kvcache_contiguous_ignores_block_counts():
    # without a block table the caches are [B, page_size, Hkv, d]: page_size need not be a
    # multiple of 32, and num_blocks / max_blocks_per_seq are not looked at (the call
    # still fails, on the scale, before any HIP call)
    assert call_kvcache(bt=None, page=48, nb=0, mb=0, scale=0.0) == 7


def call_append(kn=Q, vn=VN, kc=K, vc=V, sl=SL, bt=BT, **kw):
    a = dict(KGOOD, **kw)
    return ff.load().attn_kvcache_append(kn, vn, kc, vc, sl, bt, a["B"], a.get("S_new", 4),
                                         a["Hkv"], a["d"], a["nb"], a["page"], a["mb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), 1), (dict(vc=None), 1), (dict(sl=None), 1),
    (dict(S_new=0), 2), (dict(page=40), 2), (dict(B=0), 2),
    (dict(d=32), 3), (dict(vn=VN + 4), 5), (dict(sl=SL + 1), 5),
    (dict(vc=K), 9), (dict(kn=K + 64), 9), (dict(bt=V + 128), 9),
])
def test_attn_kvcache_append_rejects(kw, code):
    assert call_append(**kw) == code


def test_splitkv_and_combine_reject():
    lib = ff.load()
    a = (1, 1, 300, 8, 2, 128, 0, 0.1)
    assert lib.attn_fwd_splitkv(Q, K, V, None, None, O, L, *a, 0, None) == 6
    assert lib.attn_fwd_splitkv(Q, K, V, None, None, O, L, *a, 129, None) == 6
    assert lib.attn_fwd_splitkv(Q, K, V, None, None, O, L, *a, 2, None) == 1   # no accum
    assert lib.attn_fwd_splitkv(Q, K, V, O, L, None, None, *a, 1, None) == 1   # no o/lse
    assert lib.attn_fwd_splitkv(Q, K, V, O + 4, L, None, None, *a, 4, None) == 5
    assert lib.attn_splitkv_combine(O, L, None, Q, 1, 1, 8, 128, 4, None) == 1
    assert lib.attn_splitkv_combine(O, L, Q, K, 1, 1, 8, 96, 4, None) == 3
    assert lib.attn_splitkv_combine(O, L, Q, K, 1, 1, 8, 128, 0, None) == 6
    assert lib.attn_splitkv_combine(O, L, O, K, 1, 1, 8, 128, 4, None) == 9


# More fake addresses for the backward's extra buffers (never dereferenced either).
DO, DQ, DK, DV, WS = 6 << 32, 7 << 32, 8 << 32, 9 << 32, 10 << 32


def call_bwd(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, ws=WS, **kw):
    a = dict(GOOD, **kw)
    return ff.load().attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, a["B"], a["Sq"], a["Sk"],
                              a["Hq"], a["Hkv"], a["d"], a["causal"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dout=None), 1), (dict(ws=None), 1), (dict(dk=None), 1),
    (dict(Sk=0), 2), (dict(d=96), 3), (dict(Hq=3, Hkv=2), 4),
    (dict(dout=DO + 8), 5), (dict(ws=WS + 4), 5), (dict(dq=DQ + 2), 5),
    (dict(scale=0.0), 7), (dict(scale=float("nan")), 7),
    (dict(dq=Q), 9), (dict(dk=DV), 9), (dict(ws=O), 9), (dict(dv=DO), 9),
])
def test_attn_bwd_rejects(kw, code):
    assert call_bwd(**kw) == code


def test_bwd_workspace_size():
    # D and the base-2 LSE per row, rows padded to a multiple of 64
    assert ff.attn_bwd_workspace_floats(4, 4096, 16) == 2 * 4 * 16 * 4096
    assert ff.attn_bwd_workspace_floats(2, 333, 4) == 2 * 2 * 4 * 384
    assert ff.attn_bwd_workspace_floats(1, 1, 1) == 128
    with pytest.raises(ff.FlashFwdError):
        ff.attn_bwd_workspace_floats(0, 10, 1)


def test_efficiency_rule_reproduces_printed_example():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "split_heuristic_example.json")))
    blocks, sms = g["blocks"], g["sms"]
    for s, printed in g["printed_efficiency"].items():
        w = blocks * int(s) / sms
        assert round(w / math.ceil(w), 2) == printed
    for max_splits in (3, 8, 64, 128):
        assert ff.attn_splits_efficiency_rule(blocks, sms, max_splits) == g["printed_choice"]
    assert ff.attn_splits_efficiency_rule(108, 108, 16) == 1
    with pytest.raises(ff.FlashFwdError):
        ff.attn_splits_efficiency_rule(0, 108, 4)


def test_num_splits_retuned_for_256_cus():
    # GQA decode, 8 x 8 (batch, kv-head) units of 4 folded rows on 256 CUs, one slot each
    s = ff.attn_splitkv_num_splits(8, 1, 32768, 32, 8, 128, 256)
    assert s == 4
    units, slots = 64, 256
    w = units * s / slots
    assert w / math.ceil(w) >= 0.85 and 1 < s <= 64
    # enough units to fill the GPU: no split
    assert ff.attn_splitkv_num_splits(64, 1, 4096, 64, 8, 128, 256) == 1
    # short key ranges keep at least 4 key blocks per split
    assert ff.attn_splitkv_num_splits(1, 1, 4 * 128, 8, 8, 64, 256) == 1
    assert ff.attn_splitkv_num_splits(1, 1, 8 * 128, 8, 8, 64, 256) <= 2
    with pytest.raises(ff.FlashFwdError):
        ff.attn_splitkv_num_splits(1, 1, 100, 3, 2, 64, 256)


def test_one_hip_runtime_whatever_the_import_order():
    # Loading the library first must not bring a second HIP runtime into the process.
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from io_aware_attention_amd import flashfwd; flashfwd.load()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "libs = {l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}\n"
            "print(len(libs)); assert len(libs) == 1, libs\n") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


NOALLOC = dict(B=1, Sq=1, Sk=64, Hq=8, Hkv=2, d=128, causal=0, scale=0.1, S=4)


def call_noalloc(q=Q, k=K, v=V, o=O, lse=L, **kw):
    a = dict(NOALLOC, **kw)
    return ff.load().attn_fwd_splitkv_noalloc(q, k, v, o, lse, a["B"], a["Sq"], a["Sk"], a["Hq"],
                                              a["Hkv"], a["d"], a["causal"], a["scale"], a["S"],
                                              None)


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), 1), (dict(S=0), 6), (dict(S=129), 6), (dict(d=96), 3), (dict(Hq=6, Hkv=4), 4),
    (dict(lse=L + 4), 5), (dict(scale=0.0), 7), (dict(o=K), 9),
    # partials of 128 splits x 8 x 32 x 16 rows x 129 floats exceed the 4 Mi-float buffer
    (dict(B=8, Hq=32, Hkv=8, Sq=16, S=128), 11),
    (dict(B=1, Hq=8, Hkv=2, Sq=4096, S=2), 11),
])
def test_attn_fwd_splitkv_noalloc_rejects(kw, code):
    assert call_noalloc(**kw) == code


def _run_with_env(code, env):
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       env=dict(os.environ, **env), timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout, r.stderr


def test_plan_log_and_split_override():
    """FLASHFWD_LOG prints the host's plan; FLASHFWD_NUM_SPLITS (benchmark sweeps) replaces
    the split rule's choice when it is an integer in [1, FF_MAX_SPLITS], else is ignored."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from io_aware_attention_amd import flashfwd as f\n"
            "print(f.attn_splitkv_num_splits(8, 1, 32768, 32, 8, 128, 256))\n" % ROOT)
    base, err = _run_with_env(code, {"FLASHFWD_LOG": "0", "FLASHFWD_NUM_SPLITS": ""})
    assert err == ""
    out, err = _run_with_env(code, {"FLASHFWD_LOG": "1", "FLASHFWD_NUM_SPLITS": ""})
    assert out == base and f"attn_splitkv_num_splits: {int(base)}" in err
    out, err = _run_with_env(code, {"FLASHFWD_LOG": "1", "FLASHFWD_NUM_SPLITS": "7"})
    assert int(out) == 7 and "from FLASHFWD_NUM_SPLITS" in err
    for bad in ("0", "-3", "x", "9999", "5x"):
        out, _ = _run_with_env(code, {"FLASHFWD_NUM_SPLITS": bad})
        assert out == base, bad
