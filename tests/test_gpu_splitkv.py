"""attn_fwd_splitkv + attn_splitkv_combine (the decode path) against the fp64 CPU oracle.

The per-split partials are compared with the oracle's split variant over the same key
blocks (FF_SPLIT_BLOCK_N keys), empty splits included; the combined result with the plain
definition.  The full GQA decode workload is compared on every output row."""
import math

import numpy as np
import pytest

import synth
from gpu_helpers import check_outputs, host, make_inputs, say, to_dev

pytestmark = pytest.mark.gpu
BLOCK_N = 128


@pytest.fixture(scope="module")
def ff():
    import torch
    from io_aware_attention_amd import flashfwd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    flashfwd.load()
    return flashfwd


def run_split(ff, q, k, v, causal, scale, num_splits):
    import torch
    o, lse, oa, la = ff.forward_splitkv(to_dev(q), to_dev(k), to_dev(v), causal, scale,
                                        num_splits=num_splits, return_partials=True)
    torch.cuda.synchronize()
    return host(o), host(lse), (None if oa is None else host(oa)), (None if la is None else host(la))


CASES = [
    # B, Sq, Sk, Hq, Hkv, d, causal
    (2, 1, 3000, 8, 2, 128, False),   # GQA decode, fold of 4
    (2, 1, 3000, 8, 2, 64, False),
    (3, 1, 777, 6, 6, 128, False),    # MHA decode: no fold
    (1, 1, 4100, 16, 1, 128, True),   # MQA, fold of 16; causal is moot at Sq = 1
    (1, 1, 300, 32, 2, 64, False),    # fold of 16 rows
    (1, 37, 300, 4, 2, 128, True),    # several query rows, causal per row
    (2, 20, 515, 6, 2, 64, True),
    (1, 300, 77, 2, 2, 64, True),     # rows that see no key
]


@pytest.mark.parametrize("num_splits", [1, 2, 3, 5, 8, 16, 32])
@pytest.mark.parametrize("shape", CASES, ids=lambda s: "B%d_Sq%d_Sk%d_Hq%d_Hkv%d_d%d_%s" % (
    *s[:6], "causal" if s[6] else "full"))
def test_splitkv_partials_and_combine(ff, oracle, shape, num_splits):
    B, Sq, Sk, Hq, Hkv, d, causal = shape
    say(f"splitkv {shape} S={num_splits}")
    q, k, v = make_inputs(B, Sq, Sk, Hq, Hkv, d, seed=900 + Sk + Sq)
    scale = synth.f32(1 / math.sqrt(d))
    o, lse, oa, la = run_split(ff, q, k, v, causal, scale, num_splits)
    op_ref, lp_ref, o_ref, lse_ref = oracle.split(q, k, v, causal, scale, BLOCK_N, num_splits)
    check_outputs(o, lse, o_ref, lse_ref, f"{shape} S={num_splits} combined")
    if num_splits > 1:
        check_outputs(oa, la, op_ref, lp_ref, f"{shape} S={num_splits} partials")
        nblocks = -(-Sk // BLOCK_N)
        per = -(-nblocks // num_splits)
        for s in range(num_splits):
            if s * per >= nblocks:   # empty split: (0, -inf)
                assert np.all(oa[s] == 0.0) and np.all(np.isneginf(la[s]))


@pytest.mark.parametrize("num_splits", [63, 64, 65, 100, 128])
def test_splitkv_many_splits(ff, oracle, num_splits):
    # The combine loads the LSEs of splits l and l + 64 in lane l: split counts around and
    # past 64, up to the largest allowed.  20000 keys are 157 key blocks, so at these
    # counts a third or more of the splits are empty (0, -inf).
    B, Sq, Sk, Hq, Hkv, d, causal = 2, 1, 20000, 8, 2, 128, False
    say(f"splitkv many splits S={num_splits}")
    q, k, v = make_inputs(B, Sq, Sk, Hq, Hkv, d, seed=1700 + num_splits)
    scale = synth.f32(1 / math.sqrt(d))
    o, lse, oa, la = run_split(ff, q, k, v, causal, scale, num_splits)
    op_ref, lp_ref, o_ref, lse_ref = oracle.split(q, k, v, causal, scale, BLOCK_N, num_splits)
    check_outputs(o, lse, o_ref, lse_ref, f"S={num_splits} combined")
    check_outputs(oa, la, op_ref, lp_ref, f"S={num_splits} partials")
    per = -(-(-(-Sk // BLOCK_N)) // num_splits)
    empty = [s for s in range(num_splits) if s * per >= -(-Sk // BLOCK_N)]
    assert empty, "the case should hold empty splits"
    for s in empty:
        assert np.all(oa[s] == 0.0) and np.all(np.isneginf(la[s]))


def test_gqa_decode_workload_all_rows(ff, oracle):
    import torch
    w = synth.WORKLOADS["gqa_decode"]
    say(f"gqa_decode workload {w}")
    q, k, v = synth.make_qkv(w)
    S = ff.attn_splitkv_num_splits(w["B"], w["Sq"], w["Sk"], w["Hq"], w["Hkv"], w["d"])
    say(f"  heuristic num_splits = {S}")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o, lse = ff.forward_splitkv(qd, kd, vd, False, w["scale"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(q, k, v, False, w["scale"])
    check_outputs(host(o), host(lse), o_ref, lse_ref, "gqa_decode")
    # split count does not change the answer beyond rounding
    o2, lse2 = ff.forward_splitkv(qd, kd, vd, False, w["scale"], num_splits=1)
    torch.cuda.synchronize()
    check_outputs(host(o2), host(lse2), o_ref, lse_ref, "gqa_decode S=1")


def test_splitkv_matches_prefill_kernel(ff):
    import torch
    q, k, v = make_inputs(2, 33, 640, 8, 4, 128, seed=5)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o1, l1 = ff.forward(qd, kd, vd, True, 0.1)
    o2, l2 = ff.forward_splitkv(qd, kd, vd, True, 0.1, num_splits=3)
    torch.cuda.synchronize()
    assert (o1 - o2).abs().max().item() < 2e-2
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(l2))
    assert (l1[fin] - l2[fin]).abs().max().item() < 1e-3


def test_splitkv_is_deterministic(ff):
    import torch
    q, k, v = make_inputs(2, 1, 5000, 16, 4, 128, seed=6)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    a = ff.forward_splitkv(qd, kd, vd, False, 0.08, num_splits=7)
    b = ff.forward_splitkv(qd, kd, vd, False, 0.08, num_splits=7)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
