"""attn_fwd_varlen (packed variable-length batches, prefix-sum boundaries) against the fp64
oracle, element by element; equal-length packing against the dense entry point bit for bit;
the packed 16384-token workload on sampled rows.  Calls go through the C ABI."""
import math

import numpy as np
import pytest

import synth
from gpu_helpers import check_outputs, host, say, tile_edge_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ff():
    import torch
    from io_aware_attention_amd import flashfwd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    flashfwd.load()
    return flashfwd


def packed_inputs(lens_q, lens_k, Hq, Hkv, d, seed):
    q = synth.normal_bf16(seed, 0, (sum(lens_q), Hq, d))
    k = synth.normal_bf16(seed, 1, (sum(lens_k), Hkv, d))
    v = synth.normal_bf16(seed, 2, (sum(lens_k), Hkv, d))
    return q, k, v, synth.prefix_sums(lens_q), synth.prefix_sums(lens_k)


def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


def run_varlen(ff, q, k, v, cu_q, cu_k, max_q, causal, scale):
    import torch
    o, lse = ff.forward_varlen(to_dev(q), to_dev(k), to_dev(v), dev_i32(cu_q), dev_i32(cu_k),
                               max_q, causal, scale)
    torch.cuda.synchronize()
    return host(o), host(lse)


CASES = [
    # query lengths, key lengths, Hq, Hkv, d, causal
    ([5, 0, 130, 1, 257], [5, 0, 130, 1, 257], 4, 2, 128, True),    # an empty sequence
    ([5, 0, 130, 1, 257], [5, 0, 130, 1, 257], 4, 2, 64, False),
    ([100, 300, 64], [300, 100, 0], 2, 1, 128, True),             # Sq != Sk, no keys at all
    ([128, 256, 129], [128, 256, 129], 8, 2, 64, True),           # tile-sized and one over
    ([1, 1, 1, 1, 1, 1, 400], [37, 513, 1, 64, 65, 200, 400], 4, 4, 128, False),
    ([1, 1, 1, 1, 1, 1, 400], [37, 513, 1, 64, 65, 200, 400], 4, 4, 128, True),
    ([333], [333], 2, 2, 64, True),                               # one sequence
]


def ids(c):
    return "q%s_k%s_Hq%d_Hkv%d_d%d_%s" % ("-".join(map(str, c[0])), "-".join(map(str, c[1])),
                                          c[2], c[3], c[4], "causal" if c[5] else "full")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_varlen_matches_oracle(ff, oracle, case):
    lens_q, lens_k, Hq, Hkv, d, causal = case
    say(f"varlen {ids(case)}")
    q, k, v, cu_q, cu_k = packed_inputs(lens_q, lens_k, Hq, Hkv, d, seed=41 + sum(lens_k))
    scale = synth.f32(1 / math.sqrt(d))
    o, lse = run_varlen(ff, q, k, v, cu_q, cu_k, max(lens_q), causal, scale)
    o_ref, lse_ref = oracle.varlen(q, k, v, cu_q, cu_k, causal, scale)
    check_outputs(o, lse, o_ref, lse_ref, ids(case))


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_dense_bitwise(ff, causal):
    # The same sequences packed or batched run the same arithmetic.
    import torch
    B, S, Hq, Hkv, d = 3, 300, 4, 2, 128
    q, k, v, cu_q, cu_k = packed_inputs([S] * B, [S] * B, Hq, Hkv, d, seed=43)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o_p, l_p = ff.forward_varlen(qd, kd, vd, dev_i32(cu_q), dev_i32(cu_k), S, causal, 0.09)
    o_b, l_b = ff.forward(qd.view(B, S, Hq, d), kd.view(B, S, Hkv, d), vd.view(B, S, Hkv, d),
                          causal, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(o_p.view(B, S, Hq, d), o_b)
    assert torch.equal(l_p.view(Hq, B, S).permute(1, 0, 2), l_b)


def test_max_seqlen_bounds_the_grid(ff, oracle):
    # max_seqlen_q above the true maximum only adds idle workgroups
    lens = [70, 190, 5]
    q, k, v, cu_q, cu_k = packed_inputs(lens, lens, 2, 1, 64, seed=44)
    o, lse = run_varlen(ff, q, k, v, cu_q, cu_k, sum(lens), True, 0.125)
    o_ref, lse_ref = oracle.varlen(q, k, v, cu_q, cu_k, True, 0.125)
    check_outputs(o, lse, o_ref, lse_ref, "max_seqlen_q = total_q")


def test_varlen_prefill_workload_every_tile(ff, oracle):
    # the first and last row of every (sequence, head, 128-row query tile): every
    # workgroup of the launch is checked
    import torch
    w = synth.WORKLOADS["varlen_prefill"]
    q, k, v, lens = synth.make_varlen_qkv(w)
    cu = synth.prefix_sums(lens)
    say(f"varlen_prefill: {len(lens)} sequences, lengths {lens}")
    o_d, lse_d = ff.forward_varlen(to_dev(q), to_dev(k), to_dev(v), dev_i32(cu), dev_i32(cu),
                                   max(lens), w["causal"], w["scale"])
    torch.cuda.synchronize()
    assert torch.isfinite(o_d).all().item() and torch.isfinite(lse_d).all().item()
    o_h, lse_h = host(o_d), host(lse_d)
    o_s, l_s, o_r, l_r = [], [], [], []
    for b, n in enumerate(lens):
        s0 = int(cu[b])
        rows = tile_edge_rows(1, n, w["Hq"], seed=b)
        sl = slice(s0, s0 + n)
        o_ref, lse_ref = oracle.rows(q[None, sl], k[None, sl], v[None, sl], w["causal"],
                                     w["scale"], rows)
        for (_, h, i), orow, lrow in zip(rows, o_ref, lse_ref):
            o_s.append(o_h[s0 + i, h])
            l_s.append(lse_h[h, s0 + i])
            o_r.append(orow)
            l_r.append(lrow)
    say(f"  compared {len(o_s)} rows")
    check_outputs(np.array(o_s), np.array(l_s), np.array(o_r), np.array(l_r), "varlen_prefill")
