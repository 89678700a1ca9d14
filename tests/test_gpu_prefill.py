"""attn_fwd (the fused prefill kernel) against the fp64 CPU oracle, element by element.

Small shapes spanning several query and key tiles with ragged tails are compared in full;
the full-size workloads are compared on the first and last row of every (batch, head,
128-row query tile), so every workgroup of the launch is checked (the oracle computes the
rows one by one), plus properties that hold at any size.  Calls go through the C ABI."""
import math

import numpy as np
import pytest

import synth
from gpu_helpers import check_outputs, host, make_inputs, say, tile_edge_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ff():
    import torch
    from io_aware_attention_amd import flashfwd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    flashfwd.load()
    return flashfwd


def run_fwd(ff, q, k, v, causal, scale):
    import torch
    o, lse = ff.forward(to_dev(q), to_dev(k), to_dev(v), causal, scale)
    torch.cuda.synchronize()
    return host(o), host(lse)


SMALL = [
    # B, Sq, Sk, Hq, Hkv, d, causal
    (2, 333, 333, 4, 2, 64, False),
    (2, 333, 333, 4, 2, 64, True),
    (1, 300, 300, 2, 2, 128, False),
    (1, 300, 300, 2, 2, 128, True),
    (1, 200, 517, 4, 1, 128, True),     # Sq < Sk, bottom-right causal
    (1, 300, 77, 2, 2, 64, True),       # Sq > Sk: the first rows see no key
    (1, 1, 1000, 4, 2, 128, True),      # one query row
    (2, 5, 1, 2, 2, 64, False),         # one key
    (2, 5, 1, 2, 2, 64, True),
    (1, 129, 129, 1, 1, 128, True),
    (1, 64, 64, 1, 1, 64, True),
    (1, 1, 1, 1, 1, 128, False),
    (3, 260, 190, 6, 3, 128, False),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%d_Sq%d_Sk%d_Hq%d_Hkv%d_d%d_%s" % (
    *s[:6], "causal" if s[6] else "full"))
def test_prefill_small_shapes(ff, oracle, shape):
    B, Sq, Sk, Hq, Hkv, d, causal = shape
    say(f"prefill shape {shape}")
    q, k, v = make_inputs(B, Sq, Sk, Hq, Hkv, d, seed=11 + Sq + Sk)
    scale = synth.f32(1 / math.sqrt(d))
    o, lse = run_fwd(ff, q, k, v, causal, scale)
    o_ref, lse_ref = oracle.fwd(q, k, v, causal, scale)
    check_outputs(o, lse, o_ref, lse_ref, str(shape))


@pytest.mark.parametrize("Sk", [63, 64, 65, 127, 129, 150, 191, 193])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_key_tail_residues(ff, oracle, Sk, causal):
    B, Sq, Hq, Hkv, d = 1, 150, 2, 1, 64
    say(f"prefill residues Sk={Sk} causal={causal}")
    q, k, v = make_inputs(B, Sq, Sk, Hq, Hkv, d, seed=500 + Sk)
    o, lse = run_fwd(ff, q, k, v, causal, 0.125)
    o_ref, lse_ref = oracle.fwd(q, k, v, causal, 0.125)
    check_outputs(o, lse, o_ref, lse_ref, f"Sk={Sk}")


@pytest.mark.parametrize("offset", [0, 1, 31, 32, 33, 63, 64, 65, 96, 100])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_causal_diagonal_offsets(ff, oracle, offset, d):
    """Causal with Sk = Sq + offset: the diagonal crosses the 64-key tiles at every
    alignment relative to the 128-row query tiles and their 32-row wavefronts, so the
    first diagonal tile is invisible to one, two or none of a workgroup's wavefronts."""
    B, Sq, Hq, Hkv = 1, 384, 2, 1
    Sk = Sq + offset
    say(f"prefill causal diagonal offset={offset} d={d}")
    q, k, v = make_inputs(B, Sq, Sk, Hq, Hkv, d, seed=900 + offset + d)
    o, lse = run_fwd(ff, q, k, v, True, 0.125)
    o_ref, lse_ref = oracle.fwd(q, k, v, True, 0.125)
    check_outputs(o, lse, o_ref, lse_ref, f"offset={offset} d={d}")


def test_tiny_mha_workload_full(ff, oracle):
    w = synth.WORKLOADS["tiny_mha"]
    q, k, v = synth.make_qkv(w)
    o, lse = run_fwd(ff, q, k, v, w["causal"], w["scale"])
    o_ref, lse_ref = oracle.fwd(q, k, v, w["causal"], w["scale"])
    check_outputs(o, lse, o_ref, lse_ref, "tiny_mha")


@pytest.mark.parametrize("name", ["causal_prefill", "ragged_noncausal", "ragged_causal",
                                  "long_causal_gqa"])
def test_prefill_full_size_every_tile(ff, oracle, name):
    import torch
    w = synth.WORKLOADS[name]
    say(f"full-size workload {name}: {w}")
    q, k, v = synth.make_qkv(w)
    o_d, lse_d = ff.forward(to_dev(q), to_dev(k), to_dev(v), w["causal"], w["scale"])
    torch.cuda.synchronize()
    # properties over every output: finite, every row sees a key (Sq == Sk)
    assert torch.isfinite(o_d).all().item() and torch.isfinite(lse_d).all().item()
    vmax = float(np.abs(synth.bf16_bits_to_f32(v)).max())
    assert o_d.abs().max().item() <= vmax + 2e-2   # O is a convex combination of V rows
    rows = tile_edge_rows(w["B"], w["Sq"], w["Hq"], seed=len(name))
    say(f"  comparing {len(rows)} rows (first and last of every query tile)")
    o_ref, lse_ref = oracle.rows(q, k, v, w["causal"], w["scale"], rows)
    idx = torch.tensor(rows, dtype=torch.long)
    o_s = o_d[idx[:, 0], idx[:, 2], idx[:, 1]]
    lse_s = lse_d[idx[:, 0], idx[:, 1], idx[:, 2]]
    check_outputs(host(o_s), host(lse_s), o_ref, lse_ref, name)


def _one_row_inputs(d, key_col0, val_col0):
    """One query whose scores are key_col0 (q = e0) and whose output dim 0 reads val_col0."""
    n = len(key_col0)
    q = np.zeros((1, 1, 1, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, n, 1, d), np.float32)
    k[0, :, 0, 0] = key_col0
    v = np.zeros((1, n, 1, d), np.float32)
    v[0, :, 0, 0] = val_col0
    return [synth.f32_to_bf16_bits(x) for x in (q, k, v)]


@pytest.mark.parametrize("d", [64, 128])
def test_worked_examples_on_gpu(ff, d):
    # online-softmax worked example: scores [1,2 | 3,0], values [2,8 | 4,10]
    e = math.exp
    q, k, v = _one_row_inputs(d, [1, 2, 3, 0], [2, 8, 4, 10])
    o, lse = run_fwd(ff, q, k, v, False, 1.0)
    exact = (2 * e(1) + 8 * e(2) + 4 * e(3) + 10) / (1 + e(1) + e(2) + e(3))
    assert abs(o[0, 0, 0, 0] - exact) < 2e-2 and abs(o[0, 0, 0, 0] - 4.966) < 2e-2
    assert abs(lse[0, 0, 0] - math.log(1 + e(1) + e(2) + e(3))) < 1e-3
    # one query, two keys: scores [0, ln 3] through the scale argument, values [2, 6]
    q, k, v = _one_row_inputs(d, [0, 1], [2, 6])
    o, lse = run_fwd(ff, q, k, v, False, synth.f32(math.log(3.0)))
    assert abs(o[0, 0, 0, 0] - 5.0) < 2e-2 and abs(lse[0, 0, 0] - math.log(4.0)) < 1e-3
    # the split view of it goes through the decode kernel
    import torch
    o2, l2 = ff.forward_splitkv(to_dev(q), to_dev(k), to_dev(v), False,
                                synth.f32(math.log(3.0)), num_splits=1)
    torch.cuda.synchronize()
    assert abs(host(o2)[0, 0, 0, 0] - 5.0) < 2e-2


def test_prefill_is_deterministic(ff):
    import torch
    q, k, v = make_inputs(2, 700, 700, 4, 2, 128, seed=77)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o1, l1 = ff.forward(qd, kd, vd, True, 0.09)
    o2, l2 = ff.forward(qd, kd, vd, True, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prefill_on_a_side_stream(ff, oracle):
    import torch
    q, k, v = make_inputs(1, 200, 200, 2, 2, 64, seed=3)
    s = torch.cuda.Stream()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = ff.forward(qd, kd, vd, True, 0.125, stream=s)
    s.synchronize()
    o_ref, lse_ref = oracle.fwd(q, k, v, True, 0.125)
    check_outputs(host(o), host(lse), o_ref, lse_ref, "side stream")
