"""attn_fwd_splitkv_noalloc (partials in the library's static device buffer) against the
entry points it stands for, attn_fwd_splitkv + attn_splitkv_combine with caller-allocated
partials, through the C ABI: two calls in a row, the second on a smaller problem, so that
what the first left in the buffer cannot leak into the second.  Both also meet the error
bar against the fp64 oracle."""
import math

import numpy as np
import pytest

import synth
from gpu_helpers import check_outputs, host, make_inputs, say, to_dev

pytestmark = pytest.mark.gpu


def reference_and_noalloc(ff, q, k, v, causal, scale, num_splits):
    import torch
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o_ref, lse_ref = ff.forward_splitkv(qd, kd, vd, causal, scale, num_splits=num_splits)
    o = torch.full((B, Sq, Hq, d), float("nan"), dtype=torch.float32, device="cuda:0")
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda:0")
    ff.attn_fwd_splitkv_noalloc(qd, kd, vd, o, lse, B, Sq, Sk, Hq, Hkv, d, causal, scale,
                                num_splits)
    torch.cuda.synchronize()
    return o, lse, o_ref, lse_ref


def test_noalloc_matches_caller_buffers_twice(oracle):
    import torch
    from io_aware_attention_amd import flashfwd as ff
    ff.load()
    # call 1: the decode workload's shape (8 x 32 query heads over 32768 cached keys)
    w = synth.WORKLOADS["gqa_decode"]
    q, k, v = synth.make_qkv(w)
    S = ff.attn_splitkv_num_splits(w["B"], w["Sq"], w["Sk"], w["Hq"], w["Hkv"], w["d"])
    say(f"no-alloc call 1: gqa_decode {w['B']}x{w['Hq']}/{w['Hkv']} Sk={w['Sk']}, {S} splits")
    o, lse, o_ref, lse_ref = reference_and_noalloc(ff, q, k, v, False, w["scale"], S)
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    rows = [(b, h, 0) for b in range(w["B"]) for h in range(w["Hq"])]
    o_or, lse_or = oracle.rows(q, k, v, False, w["scale"], rows)
    check_outputs(host(o).reshape(-1, w["d"]), host(lse).reshape(-1), o_or, lse_or,
                  "no-alloc gqa_decode")
    # call 2: smaller, causal, d = 64, more splits than the first
    q, k, v = make_inputs(2, 3, 1000, 8, 2, 64, seed=71)
    scale = synth.f32(1 / math.sqrt(64))
    say("no-alloc call 2: B=2 Sq=3 Sk=1000 Hq=8 Hkv=2 d=64 causal, 7 splits")
    o, lse, o_ref, lse_ref = reference_and_noalloc(ff, q, k, v, True, scale, 7)
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    o_or, lse_or = oracle.fwd(q, k, v, True, scale)
    check_outputs(host(o), host(lse), o_or, lse_or, "no-alloc small causal")


def test_noalloc_rejects_oversized_partials():
    import torch
    from io_aware_attention_amd import flashfwd as ff
    B, Sq, Sk, Hq, Hkv, d = 1, 4096, 256, 8, 2, 128
    x = torch.zeros((B, Sq, Hq, d), dtype=torch.bfloat16, device="cuda:0")
    kv = torch.zeros((B, Sk, Hkv, d), dtype=torch.bfloat16, device="cuda:0")
    o = torch.zeros((B, Sq, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.zeros((B, Hq, Sq), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ff.FlashFwdError) as e:
        ff.attn_fwd_splitkv_noalloc(x, kv, kv, o, lse, B, Sq, Sk, Hq, Hkv, d, False, 0.1, 2)
    assert e.value.status == 11  # FF_ERR_SCRATCH
    assert not o.any().item()    # nothing was enqueued
