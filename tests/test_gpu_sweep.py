"""Seeded parity sweeps against the fp64 CPU oracle: prefill, split-KV, backward and
paged key/value-cache decode over random small configurations.

Random small shapes (GQA ratios, ragged lengths, Sq != Sk, both head sizes, causal or
not) with Q and K scaled up to 6x, so that scores span tens of units in base 2 and the
prefill kernel's lazy reference point (raised only when a tile's maximum passes it by
more than 2^8) is raised on later tiles, not only on the first; V stays N(0, 1), so
the absolute error bar on O keeps its meaning.  A constructed case raises it on every
tile: the scores grow by ~46 base-2 units per 64-key tile in the order the kernel
visits the tiles (highest tile first).  The backward and cache sweeps reuse the bounds
and the NaN-poisoned caches of their own test modules.  Calls go through the C ABI."""
import math

import numpy as np
import pytest

import synth
from gpu_helpers import check_outputs, host, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ff():
    import torch
    from io_aware_attention_amd import flashfwd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    flashfwd.load()
    return flashfwd


def sweep_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 3))
        cases.append(dict(B=int(rng.integers(1, 3)), Sq=int(rng.integers(1, 600)),
                          Sk=int(rng.integers(1, 600)), Hq=G * Hkv, Hkv=Hkv,
                          d=int(rng.choice([64, 128])), causal=bool(rng.integers(0, 2)),
                          mult=float(rng.choice([0.5, 1.0, 3.0, 6.0])),
                          seed=int(rng.integers(1, 1 << 30))))
    return cases


CASES = sweep_cases(24, seed=2026)


def case_id(c):
    return "B%(B)d_Sq%(Sq)d_Sk%(Sk)d_Hq%(Hq)d_Hkv%(Hkv)d_d%(d)d_c%(causal)d_x%(mult)g" % c


def qkv(c):
    q = synth.normal_bf16(c["seed"], 0, (c["B"], c["Sq"], c["Hq"], c["d"]), c["mult"])
    k = synth.normal_bf16(c["seed"], 1, (c["B"], c["Sk"], c["Hkv"], c["d"]), c["mult"])
    v = synth.normal_bf16(c["seed"], 2, (c["B"], c["Sk"], c["Hkv"], c["d"]), 1.0)
    return q, k, v


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_prefill_sweep(ff, oracle, c):
    import torch
    say(f"sweep prefill {case_id(c)}")
    q, k, v = qkv(c)
    scale = synth.f32(1 / math.sqrt(c["d"]))
    o, lse = ff.forward(to_dev(q), to_dev(k), to_dev(v), c["causal"], scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(q, k, v, c["causal"], scale)
    check_outputs(host(o), host(lse), o_ref, lse_ref, case_id(c))


@pytest.mark.parametrize("c", CASES[:12], ids=case_id)
def test_splitkv_sweep(ff, oracle, c):
    # the same inputs through the split-KV kernel and the combine, three splits
    import torch
    say(f"sweep split-KV {case_id(c)}")
    q, k, v = qkv(c)
    scale = synth.f32(1 / math.sqrt(c["d"]))
    o, lse = ff.forward_splitkv(to_dev(q), to_dev(k), to_dev(v), c["causal"], scale,
                                num_splits=3)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(q, k, v, c["causal"], scale)
    check_outputs(host(o), host(lse), o_ref, lse_ref, case_id(c))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_reference_point_raised_every_tile(ff, oracle, causal, d):
    # Query i holds (1, ..., 1) in dimension 0 and key j holds -j/8 there (both exact in
    # bf16 up to j = 256; larger keys are rounded, and the oracle sees the same bytes),
    # with scale 4: s_ij = -j/2.  Keys are visited from the highest tile down, so every
    # 64-key tile's maximum lies ~32 units (46 in base 2) above the previous one.
    import torch
    B, S, H = 1, 700, 2
    q = np.zeros((B, S, H, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((B, S, H, d), np.float32)
    k[0, :, :, 0] = -np.arange(S, dtype=np.float32)[:, None] / 8
    v = synth.bf16_bits_to_f32(synth.normal_bf16(77, 2, (B, S, H, d)))
    q, k, v = (synth.f32_to_bf16_bits(x) for x in (q, k, v))
    say(f"reference point raised per tile d={d} causal={causal}")
    o, lse = ff.forward(to_dev(q), to_dev(k), to_dev(v), causal, 4.0)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(q, k, v, causal, 4.0)
    check_outputs(host(o), host(lse), o_ref, lse_ref, f"monotone d={d} causal={causal}")


BWD_CASES = sweep_cases(10, seed=4049)


@pytest.mark.parametrize("c", BWD_CASES, ids=case_id)
def test_backward_sweep(oracle, c):
    # attn_bwd on the sweep's shapes (Q and K scaled by up to 4 here), at the bound the
    # backward tests derive from the bf16 rounding of P and dS
    from test_gpu_backward import check_grad, run_backward
    c = dict(c, mult=min(c["mult"], 4.0))
    say(f"sweep backward {case_id(c)}")
    q, k, v = qkv(c)
    dout = synth.normal_bf16(c["seed"], 3, q.shape)
    scale = synth.f32(1 / math.sqrt(c["d"]))
    o, lse = oracle.fwd(q, k, v, c["causal"], scale)
    dq, dk, dv, _, (bq, bk, bv) = oracle.bwd(q, k, v, dout, c["causal"], scale)
    gq, gk, gv = run_backward(q, k, v, o, lse, dout, c["causal"], scale)
    check_grad(gq, dq, bq, "dQ")
    check_grad(gk, dk, bk, "dK")
    check_grad(gv, dv, bv, "dV")


def cache_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B = int(rng.integers(1, 5))
        page = int(rng.choice([32, 64, 128, 256]))
        mb = int(rng.integers(1, 9))
        lens = rng.integers(0, page * mb + 1, size=B)
        pads = [int(rng.integers(0, n_ + 1)) if rng.integers(0, 2) else 0 for n_ in lens]
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 3))
        cases.append(dict(B=B, Sq=int(rng.integers(1, 5)), Hq=G * Hkv, Hkv=Hkv,
                          d=int(rng.choice([64, 128])), page=page, mb=mb,
                          lens=[int(x) for x in lens], pads=pads,
                          causal=bool(rng.integers(0, 2)), S=int(rng.choice([1, 2, 5])),
                          seed=int(rng.integers(1, 1 << 30))))
    return cases


def cache_id(c):
    return ("B%(B)d_Sq%(Sq)d_Hq%(Hq)d_Hkv%(Hkv)d_d%(d)d_page%(page)d_mb%(mb)d_c%(causal)d_S%(S)d"
            % c + "_len" + "-".join(map(str, c["lens"])))


@pytest.mark.parametrize("c", cache_cases(10, seed=777), ids=cache_id)
def test_kvcache_sweep(ff, oracle, c):
    # paged decode over random lengths, left padding and page sizes; cache rows that no
    # batch owns hold NaN, so a read outside a batch's keys shows up in the output
    from test_gpu_kvcache import paged_cache, poison_unowned, run_kvcache
    say(f"sweep kvcache {cache_id(c)}")
    kc, vc, table = paged_cache(c["B"], c["Hkv"], c["d"], c["page"], c["mb"], 2, c["seed"])
    kc, vc = poison_unowned(kc, vc, table, c["lens"], c["pads"])
    q = synth.normal_bf16(c["seed"], 0, (c["B"], c["Sq"], c["Hq"], c["d"]))
    scale = synth.f32(1 / math.sqrt(c["d"]))
    o, lse = run_kvcache(ff, q, kc, vc, c["lens"], c["causal"], scale, table, c["pads"],
                         num_splits=c["S"])
    o_ref, lse_ref = oracle.kvcache(q, kc, vc, table, c["lens"], c["pads"], c["causal"], scale)
    check_outputs(o, lse, o_ref, lse_ref, cache_id(c))
