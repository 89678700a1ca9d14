"""GPU parity of attn_bwd against the fp64 oracle's backward.

The GPU backward rounds exactly two kinds of values: P (operand of dV = P^T dO) and dS
(operand of dQ = scale dS K and dK = scale dS^T Q) go to bf16 with round-to-nearest-even,
whose unit roundoff is 2^-8 (8 significant bits); Q, K, V, dO are bf16 already and every
sum is fp32.  So each gradient element differs from the fp64 value by at most 2^-8 times
the sum of the absolute values of its terms (the oracle returns those sums) plus fp32
effects (exp2, the fp32 LSE, fp32 accumulation).  The test allows twice the rounding
bound, 2^-7 * sum|terms|, plus 1e-4 of the tensor's largest magnitude.  O and LSE given
to the GPU come from the oracle's forward (rounded to fp32), so the comparison isolates
the backward.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import host, make_inputs, say, to_dev

pytestmark = pytest.mark.gpu

BOUND_FACTOR = 2.0 ** -7
FLOOR = 1e-4


def check_grad(gpu, ref, abs_terms, what):
    assert gpu.shape == ref.shape, what
    assert not np.isnan(gpu).any(), f"{what}: NaN"
    err = np.abs(gpu - ref)
    tol = BOUND_FACTOR * abs_terms + FLOOR * max(float(np.abs(ref).max()), 1e-30)
    ratio = float((err / tol).max())
    say(f"  {what}: max|err| = {err.max():.3e}  max|ref| = {np.abs(ref).max():.3e}  "
        f"worst err/tol = {ratio:.3f}")
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{what}: {len(bad)} elements out of bound, first {bad[:5].tolist()}"


def run_backward(q, k, v, o, lse, dout, causal, scale):
    import torch
    from io_aware_attention_amd import flashfwd as ff
    o_d = torch.from_numpy(np.ascontiguousarray(o, dtype=np.float32)).to("cuda:0")
    lse_d = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).to("cuda:0")
    dq, dk, dv = ff.backward(to_dev(q), to_dev(k), to_dev(v), o_d, lse_d, to_dev(dout),
                             causal, scale)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


SHAPES = [  # (B, Sq, Sk, Hq, Hkv, d, causal)
    (1, 128, 128, 1, 1, 128, False),
    (1, 128, 128, 1, 1, 128, True),
    (2, 200, 333, 4, 2, 64, False),
    (2, 333, 200, 4, 2, 64, True),     # Sq > Sk: the first rows see no key
    (1, 300, 300, 4, 1, 128, True),    # GQA 4:1, ragged tails in both kernels
    (1, 77, 513, 2, 2, 128, True),     # Sq < Sk
    (2, 129, 129, 2, 2, 64, True),
    (1, 1, 190, 8, 2, 128, False),     # one query row (decode shape)
]


def ids(s):
    B, Sq, Sk, Hq, Hkv, d, causal = s
    return f"B{B}_Sq{Sq}_Sk{Sk}_Hq{Hq}_Hkv{Hkv}_d{d}_{'causal' if causal else 'full'}"


@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_backward_matches_oracle(oracle, shape):
    B, Sq, Sk, Hq, Hkv, d, causal = shape
    say(f"backward parity {ids(shape)}")
    q, k, v = make_inputs(B, Sq, Sk, Hq, Hkv, d, seed=31)
    dout = synth.normal_bf16(31, 3, (B, Sq, Hq, d))
    scale = synth.f32(1.0 / np.sqrt(d))
    o, lse = oracle.fwd(q, k, v, causal, scale)
    dq, dk, dv, _, (bq, bk, bv) = oracle.bwd(q, k, v, dout, causal, scale)
    gq, gk, gv = run_backward(q, k, v, o, lse, dout, causal, scale)
    check_grad(gq, dq, bq, "dQ")
    check_grad(gk, dk, bk, "dK")
    check_grad(gv, dv, bv, "dV")


def test_backward_is_deterministic(oracle):
    B, Sq, Sk, Hq, Hkv, d, causal = 1, 300, 300, 4, 2, 128, True
    q, k, v = make_inputs(B, Sq, Sk, Hq, Hkv, d, seed=32)
    dout = synth.normal_bf16(32, 3, (B, Sq, Hq, d))
    scale = synth.f32(1.0 / np.sqrt(d))
    o, lse = oracle.fwd(q, k, v, causal, scale)
    first = run_backward(q, k, v, o, lse, dout, causal, scale)
    second = run_backward(q, k, v, o, lse, dout, causal, scale)
    for a, b in zip(first, second):
        assert np.array_equal(a, b)


def test_backward_after_gpu_forward(oracle):
    # End to end from the GPU forward's own O and LSE.  Their errors move D and hence dS
    # a little, so this is a sanity check at 1e-2 relative Frobenius error, not the
    # element-wise parity above.
    import torch
    from io_aware_attention_amd import flashfwd as ff
    B, Sq, Sk, Hq, Hkv, d, causal = 2, 257, 257, 4, 2, 128, True
    q, k, v = make_inputs(B, Sq, Sk, Hq, Hkv, d, seed=33)
    dout = synth.normal_bf16(33, 3, (B, Sq, Hq, d))
    scale = synth.f32(1.0 / np.sqrt(d))
    o_d, lse_d = ff.forward(to_dev(q), to_dev(k), to_dev(v), causal, scale)
    dq, dk, dv = ff.backward(to_dev(q), to_dev(k), to_dev(v), o_d, lse_d, to_dev(dout), causal,
                             scale)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.bwd(q, k, v, dout, causal, scale)
    for g, r, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        rel = np.linalg.norm(host(g) - r) / np.linalg.norm(r)
        say(f"  {name}: relative Frobenius error {rel:.2e}")
        assert rel < 1e-2


def test_backward_full_size_causal_prefill(oracle):
    # causal_prefill's shape (B=4, H=16, S=4096, d=128).  One (batch, kv head) unit is
    # checked element by element against the oracle (its O and LSE rows replaced by the
    # oracle's); every unit's dV is checked against a property that holds at any size:
    # the keys' dV sum to the sum of dO over the rows, because each P row sums to one;
    # with P rounded to bf16 the sums move by at most 2^-8 of sum|dO|.
    import torch
    from io_aware_attention_amd import flashfwd as ff
    w = synth.WORKLOADS["causal_prefill"]
    B, Sq, Sk, Hq, Hkv, d = (w[x] for x in ("B", "Sq", "Sk", "Hq", "Hkv", "d"))
    q, k, v = synth.make_qkv(w)
    dout = synth.normal_bf16(w["seed"], 3, q.shape)
    qd, kd, vd, dod = (to_dev(x) for x in (q, k, v, dout))
    o_d, lse_d = ff.forward(qd, kd, vd, True, w["scale"])
    b, hk = 1, 5
    g = Hq // Hkv
    heads = list(range(hk * g, (hk + 1) * g))
    rows = [(b, h, i) for h in heads for i in range(Sq)]
    say("  oracle forward rows of the checked unit ...")
    o_rows, lse_rows = oracle.rows(q, k, v, True, w["scale"], rows)
    for n, h in enumerate(heads):
        o_d[b, :, h, :] = torch.from_numpy(o_rows[n * Sq:(n + 1) * Sq].astype(np.float32)).cuda()
        lse_d[b, h, :] = torch.from_numpy(lse_rows[n * Sq:(n + 1) * Sq].astype(np.float32)).cuda()
    dq, dk, dv = ff.backward(qd, kd, vd, o_d, lse_d, dod, True, w["scale"])
    torch.cuda.synchronize()
    gq, gk, gv = host(dq), host(dk), host(dv)
    say("  oracle backward of the checked unit ...")
    rq, rk, rv, _, (bq, bk, bv) = oracle.bwd(q, k, v, dout, True, w["scale"], units=[(b, hk)])
    check_grad(gq[b][:, heads], rq[b][:, heads], bq[b][:, heads], "dQ (one unit)")
    check_grad(gk[b][:, hk], rk[b][:, hk], bk[b][:, hk], "dK (one unit)")
    check_grad(gv[b][:, hk], rv[b][:, hk], bv[b][:, hk], "dV (one unit)")
    do64 = synth.bf16_bits_to_f32(dout).astype(np.float64)          # [B, Sq, Hq, d]
    want = do64.reshape(B, Sq, Hkv, g, d).sum(axis=(1, 3))          # [B, Hkv, d]
    absum = np.abs(do64).reshape(B, Sq, Hkv, g, d).sum(axis=(1, 3))
    got = gv.sum(axis=1)
    err = np.abs(got - want)
    say(f"  sum_j dV_j vs sum_i dO_i: worst err / (2^-7 sum|dO|) = {(err / (2 ** -7 * absum)).max():.3f}")
    assert (err <= 2.0 ** -7 * absum).all()


VARIANT_CASES = [  # (B, Sq, Sk, Hq, Hkv, d, causal, window, alibi: None | "head" | "batch")
    (1, 300, 300, 4, 2, 128, False, (70, 20), None),     # two-sided window
    (2, 200, 333, 2, 1, 64, True, (100, 0), None),       # causal window, Sq < Sk
    (1, 333, 200, 2, 2, 128, True, (50, -1), None),      # Sq > Sk: rows with no key
    (1, 257, 257, 4, 1, 64, False, (-1, 40), "head"),    # right limit only, ALiBi per head
    (2, 190, 190, 2, 2, 128, True, (130, 0), "batch"),   # ALiBi per (batch, head)
    (1, 400, 400, 2, 1, 128, False, (1, 1), None),       # three keys per query
    (1, 64, 400, 2, 1, 128, False, (10, 0), None),       # keys 0..325 seen by no query
    (1, 400, 64, 2, 1, 64, True, (5, 0), None),          # Sq >> Sk: few query tiles per key block
]


def variant_ids(c):
    B, Sq, Sk, Hq, Hkv, d, causal, win, al = c
    return (f"B{B}_Sq{Sq}_Sk{Sk}_Hq{Hq}_Hkv{Hkv}_d{d}_{'causal' if causal else 'full'}"
            f"_w{win[0]}_{win[1]}_{al}")


@pytest.mark.parametrize("case", VARIANT_CASES, ids=variant_ids)
def test_backward_variants_match_oracle(oracle, case):
    import torch
    from io_aware_attention_amd import flashfwd as ff
    B, Sq, Sk, Hq, Hkv, d, causal, window, al = case
    say(f"backward variants {variant_ids(case)}")
    q, k, v = make_inputs(B, Sq, Sk, Hq, Hkv, d, seed=41)
    dout = synth.normal_bf16(41, 3, (B, Sq, Hq, d))
    scale = synth.f32(1.0 / np.sqrt(d))
    slopes = None
    if al == "head":
        slopes = np.array([2.0 ** -(i + 1) for i in range(Hq)], np.float32)
    elif al == "batch":
        slopes = np.array([[2.0 ** -(i + 1 + b) for i in range(Hq)] for b in range(B)], np.float32)
    o, lse = oracle.fwd(q, k, v, causal, scale, window=window, alibi=slopes)
    dq, dk, dv, _, (bq, bk, bv) = oracle.bwd(q, k, v, dout, causal, scale, window=window,
                                             alibi=slopes)
    o_d = torch.from_numpy(np.ascontiguousarray(o, dtype=np.float32)).to("cuda:0")
    lse_d = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).to("cuda:0")
    sl_d = None if slopes is None else torch.from_numpy(slopes).to("cuda:0")
    gq, gk, gv = ff.backward(to_dev(q), to_dev(k), to_dev(v), o_d, lse_d, to_dev(dout), causal,
                             scale, window=window, alibi_slopes=sl_d)
    torch.cuda.synchronize()
    check_grad(host(gq), dq, bq, "dQ")
    check_grad(host(gk), dk, bk, "dK")
    check_grad(host(gv), dv, bv, "dV")
    # keys that no query sees get exactly zero gradients
    unseen = ~np.any(bk != 0, axis=(0, 2, 3)) if bk.ndim == 4 else None
    if unseen is not None and unseen.any():
        say(f"  {int(unseen.sum())} keys seen by no query: dK, dV must be exact zeros")
        assert not host(gk)[:, unseen].any() and not host(gv)[:, unseen].any()


def test_backward_rejects_softcap():
    import torch
    from io_aware_attention_amd import flashfwd as ff
    B, S, H, d = 1, 64, 1, 64
    x = torch.zeros((B, S, H, d), dtype=torch.bfloat16, device="cuda:0")
    o = torch.zeros((B, S, H, d), dtype=torch.float32, device="cuda:0")
    lse = torch.zeros((B, H, S), dtype=torch.float32, device="cuda:0")
    g = [torch.empty((B, S, H, d), dtype=torch.float32, device="cuda:0") for _ in range(3)]
    ws = torch.empty(ff.attn_bwd_workspace_floats(B, S, H), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ff.FlashFwdError) as e:
        ff.attn_bwd_ex(x, x, x, o, lse, x, *g, ws, B, S, S, H, H, d, False, -1, -1, None, 0,
                       5.0, 0.125)
    assert e.value.status == 10  # FF_ERR_OPTION
