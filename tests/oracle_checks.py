"""Checks that pin the CPU oracle to what the pages and the mathematics fix.

Each check takes an ``oracle.Oracle`` instance and raises AssertionError on failure.
The same battery runs against the real oracle (every check must pass) and against
mutated copies of it (each mutant must fail at least one check).
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
LN3 = math.log(3.0)
TIGHT = 1e-12


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(x):
    return {"0": 0.0, "ln3": LN3}[x] if isinstance(x, str) else float(x)


def one_row(qv, ks, vs):
    """A single query (d=1 per key score) as oracle inputs: q [1,1,1,1], k/v [1,n,1,1]."""
    n = len(ks)
    q = np.array(qv, dtype=np.float64).reshape(1, 1, 1, 1)
    k = np.array(ks, dtype=np.float64).reshape(1, n, 1, 1)
    v = np.array(vs, dtype=np.float64).reshape(1, n, 1, 1)
    return q, k, v


# ---------------------------------------------------------------------------
# Worked examples printed on the pages


def check_online_softmax_example(orc):
    g = golden("online_softmax_worked_example.json")
    scores = sum(g["tile_scores"], [])
    values = sum(g["tile_values"], [])
    q, k, v = one_row([1.0], scores, values)
    e = math.exp
    exact = (2 * e(1) + 8 * e(2) + 4 * e(3) + 10 * e(0)) / (e(1) + e(2) + e(3) + e(0))
    exact_lse = math.log(e(1) + e(2) + e(3) + 1.0)
    tol_printed = 0.5 * 10 ** (-g["printed_digits"])
    o, lse = orc.fwd(q, k, v, False, 1.0)
    assert abs(o[0, 0, 0, 0] - g["printed_O"]) <= tol_printed, o
    assert abs(o[0, 0, 0, 0] - exact) < TIGHT and abs(lse[0, 0, 0] - exact_lse) < TIGHT
    o2, lse2 = orc.online(q, k, v, False, 1.0, 2)
    assert abs(o2[0, 0, 0, 0] - exact) < TIGHT and abs(lse2[0, 0, 0] - exact_lse) < TIGHT
    # Per-tile state: after tile 1, m = 2 with weights exp([-1, 0]).
    op, lp, o3, l3 = orc.split(q, k, v, False, 1.0, 2, 2)
    m1 = g["after_tile_1"]["m"]
    w1 = [math.exp(x) for x in g["after_tile_1"]["weights_exponents"]]
    l1 = sum(w1)
    assert abs(lp[0, 0, 0, 0] - (m1 + math.log(l1))) < TIGHT
    assert abs(op[0, 0, 0, 0, 0] - (w1[0] * 2 + w1[1] * 8) / l1) < TIGHT
    assert abs(o3[0, 0, 0, 0] - exact) < TIGHT and abs(l3[0, 0, 0] - exact_lse) < TIGHT


def check_one_query_two_keys(orc):
    g = golden("one_query_two_keys.json")
    ks = [_num(x) for x in g["k"]]
    q, k, v = one_row(g["q"], ks, g["v"])
    p = orc.probs(q, k, v, False, 1.0, 0, 0, 0)
    assert np.allclose(p, g["printed_P"], rtol=0, atol=TIGHT), p
    o, lse = orc.fwd(q, k, v, False, 1.0)
    assert abs(o[0, 0, 0, 0] - g["printed_O"]) < TIGHT
    assert abs(lse[0, 0, 0] - math.log(4.0)) < TIGHT
    # The same scores through the scale argument: k = [0, 1], scale = ln 3.
    q2, k2, v2 = one_row(g["q"], [0.0, 1.0], g["v"])
    o2, lse2 = orc.fwd(q2, k2, v2, False, LN3)
    assert abs(o2[0, 0, 0, 0] - g["printed_O"]) < TIGHT
    assert abs(lse2[0, 0, 0] - math.log(4.0)) < TIGHT
    o3, _ = orc.online(q2, k2, v2, False, LN3, 1)
    assert abs(o3[0, 0, 0, 0] - g["printed_O"]) < TIGHT


def check_exercise_1(orc):
    g = golden("exercises.json")["exercise_1"]
    s = [_num(g["block_A"]["s"]), _num(g["block_B"]["s"])]
    vv = [g["block_A"]["v"], g["block_B"]["v"]]
    q, k, v = one_row([1.0], s, vv)
    correct = (1.0 * vv[0] + 3.0 * vv[1]) / 4.0          # weights e^0 : e^ln3 = 1 : 3
    wrong = 0.5 * (vv[0] + vv[1])                         # average of the local outputs
    assert correct == 4.0 and wrong == 6.0
    for o, lse in (orc.fwd(q, k, v, False, 1.0), orc.online(q, k, v, False, 1.0, 1)):
        assert abs(o[0, 0, 0, 0] - correct) < TIGHT and abs(lse[0, 0, 0] - math.log(4)) < TIGHT
    op, lp, o, lse = orc.split(q, k, v, False, 1.0, 1, 2)
    assert abs(op[0, 0, 0, 0, 0] - vv[0]) < TIGHT and abs(op[1, 0, 0, 0, 0] - vv[1]) < TIGHT
    assert abs(lp[0, 0, 0, 0]) < TIGHT and abs(lp[1, 0, 0, 0] - LN3) < TIGHT
    assert abs(o[0, 0, 0, 0] - correct) < TIGHT and abs(o[0, 0, 0, 0] - wrong) > 1.0


def check_exercise_2(orc):
    g = golden("exercises.json")["exercise_2"]
    P = g["P"]
    q, k, v = one_row([1.0], [math.log(x) for x in P], g["V"])
    expect = sum(a * b for a, b in zip(P, g["V"]))
    assert abs(expect - 3.6) < 1e-15
    o, lse = orc.fwd(q, k, v, False, 1.0)
    assert abs(o[0, 0, 0, 0] - expect) < TIGHT and abs(lse[0, 0, 0]) < TIGHT
    assert np.allclose(orc.probs(q, k, v, False, 1.0, 0, 0, 0), P, rtol=0, atol=TIGHT)


def check_causal_mask_pictures(orc):
    for case in golden("causal_mask_pictures.json")["cases"]:
        Sq, Sk = case["Sq"], case["Sk"]
        mask = np.array(case["mask"])
        q = np.zeros((1, Sq, 1, 1))
        k = np.zeros((1, Sk, 1, 1))
        v = np.arange(1, Sk + 1, dtype=np.float64).reshape(1, Sk, 1, 1)
        o, lse = orc.fwd(q, k, v, True, 1.0)
        for i in range(Sq):
            p = orc.probs(q, k, v, True, 1.0, 0, 0, i)
            assert np.array_equal(p > 0, mask[i] == 1), (case, i, p)
            nvis = int(mask[i].sum())
            if nvis == 0:
                assert o[0, i, 0, 0] == 0.0 and lse[0, 0, i] == -np.inf
            else:
                assert abs(lse[0, 0, i] - math.log(nvis)) < TIGHT
                assert abs(o[0, i, 0, 0] - np.mean(np.arange(1, nvis + 1))) < TIGHT


def check_tail_tile_case(orc):
    g = golden("tail_tile_case.json")
    N, T, row = g["N"], g["tile"], g["row"]
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, N, 1, 3))
    k = rng.standard_normal((1, N, 1, 3))
    v = rng.standard_normal((1, N, 1, 3))
    p = orc.probs(q, k, v, True, 0.5, 0, 0, row)
    second = [j for j in range(T, min(2 * T, N)) if p[j] > 0]
    assert second == g["valid_keys_in_second_tile"]
    o1, l1 = orc.fwd(q, k, v, True, 0.5)
    o2, l2 = orc.online(q, k, v, True, 0.5, T)
    assert np.allclose(o1, o2, rtol=0, atol=TIGHT) and np.allclose(l1, l2, rtol=0, atol=TIGHT)


# ---------------------------------------------------------------------------
# Closed forms and invariants


def _rand(seed, B, Sq, Sk, Hq, Hkv, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Sq, Hq, d)), rng.standard_normal((B, Sk, Hkv, d)),
            rng.standard_normal((B, Sk, Hkv, d)))


def check_special_cases(orc):
    # Sk = 1: O = v0, LSE = s0.
    q, k, v = _rand(1, 2, 3, 1, 2, 2, 5)
    o, lse = orc.fwd(q, k, v, False, 0.7)
    for b in range(2):
        for h in range(2):
            for i in range(3):
                assert np.allclose(o[b, i, h], v[b, 0, h], rtol=0, atol=TIGHT)
                assert abs(lse[b, h, i] - 0.7 * np.dot(q[b, i, h], k[b, 0, h])) < TIGHT
    # Q = 0: uniform weights over the visible keys (causal, Sq < Sk).
    q, k, v = _rand(2, 1, 4, 7, 1, 1, 3)
    q[:] = 0.0
    o, lse = orc.fwd(q, k, v, True, 1.3)
    for i in range(4):
        nvis = i + 7 - 4 + 1
        assert np.allclose(o[0, i, 0], v[0, :nvis, 0].mean(axis=0), rtol=0, atol=TIGHT)
        assert abs(lse[0, 0, i] - math.log(nvis)) < TIGHT
    # V constant: O = c.
    q, k, v = _rand(3, 1, 5, 6, 2, 1, 4)
    v[:] = -2.5
    o, _ = orc.fwd(q, k, v, True, 0.9)
    assert np.allclose(o, -2.5, rtol=0, atol=TIGHT)
    # Causal row 0 with Sq == Sk: O = v0.
    q, k, v = _rand(4, 1, 6, 6, 1, 1, 4)
    o, lse = orc.fwd(q, k, v, True, 0.5)
    assert np.allclose(o[0, 0, 0], v[0, 0, 0], rtol=0, atol=TIGHT)


def check_probability_rows(orc):
    q, k, v = _rand(5, 1, 6, 9, 2, 2, 4)
    for causal in (False, True):
        o, lse = orc.fwd(q, k, v, causal, 0.6)
        for h in range(2):
            for i in range(6):
                p = orc.probs(q, k, v, causal, 0.6, 0, h, i)
                assert abs(p.sum() - 1.0) < TIGHT
                assert np.allclose(o[0, i, h], p @ v[0, :, h], rtol=0, atol=TIGHT)
                s = 0.6 * (k[0, :, h] @ q[0, i, h])
                vis = np.arange(9) <= (i + 9 - 6) if causal else np.ones(9, bool)
                smax = s[vis].max()
                assert smax - TIGHT <= lse[0, h, i] <= smax + math.log(vis.sum()) + TIGHT
                lo, hi = v[0, vis, h].min(axis=0), v[0, vis, h].max(axis=0)
                assert np.all(o[0, i, h] >= lo - TIGHT) and np.all(o[0, i, h] <= hi + TIGHT)


def check_shift_invariance(orc):
    # Column d-1 of K is 1; adding c/scale to q[i, d-1] adds c to every score of row i.
    q, k, v = _rand(6, 1, 4, 6, 1, 1, 5)
    k[..., -1] = 1.0
    scale, c = 0.8, 1.7
    o1, l1 = orc.fwd(q, k, v, False, scale)
    q2 = q.copy()
    q2[..., -1] += c / scale
    o2, l2 = orc.fwd(q2, k, v, False, scale)
    assert np.allclose(o1, o2, rtol=0, atol=1e-11)
    assert np.allclose(l2 - l1, c, rtol=0, atol=1e-11)


def check_key_permutation(orc):
    q, k, v = _rand(7, 2, 3, 8, 2, 2, 4)
    perm = np.random.default_rng(1).permutation(8)
    o1, l1 = orc.fwd(q, k, v, False, 0.4)
    o2, l2 = orc.fwd(q, k[:, perm], v[:, perm], False, 0.4)
    assert np.allclose(o1, o2, rtol=0, atol=TIGHT) and np.allclose(l1, l2, rtol=0, atol=TIGHT)


def check_gqa_grouping(orc):
    # Query head h reads KV head h // (Hq/Hkv): same as MHA with each KV head repeated g times.
    q, k, v = _rand(8, 2, 5, 6, 6, 2, 3)
    o1, l1 = orc.fwd(q, k, v, True, 0.7)
    o2, l2 = orc.fwd(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), True, 0.7)
    assert np.allclose(o1, o2, rtol=0, atol=TIGHT) and np.allclose(l1, l2, rtol=0, atol=TIGHT)
    # and not the interleaved reading h % Hkv
    o3, _ = orc.fwd(q, np.tile(k, (1, 1, 3, 1)), np.tile(v, (1, 1, 3, 1)), True, 0.7)
    assert not np.allclose(o1, o3, rtol=0, atol=1e-6)


def check_online_and_split_agree(orc):
    for (B, Sq, Sk, Hq, Hkv, d, causal) in ((1, 7, 7, 1, 1, 3, True), (2, 5, 9, 4, 2, 4, True),
                                            (1, 9, 4, 2, 2, 3, True), (2, 6, 11, 2, 1, 5, False)):
        q, k, v = _rand(B * 100 + Sk, B, Sq, Sk, Hq, Hkv, d)
        o, lse = orc.fwd(q, k, v, causal, 0.45)
        for blk in (1, 2, 3, 4, 8, 64):
            o2, l2 = orc.online(q, k, v, causal, 0.45, blk)
            assert np.allclose(o, o2, rtol=0, atol=TIGHT), (blk, np.abs(o - o2).max())
            assert np.array_equal(np.isneginf(lse), np.isneginf(l2))
            fin = np.isfinite(lse)
            assert np.allclose(lse[fin], l2[fin], rtol=0, atol=TIGHT)
        for blk, S in ((1, 1), (2, 3), (3, 2), (1, 7), (4, 5), (2, 7)):
            op, lp, o3, l3 = orc.split(q, k, v, causal, 0.45, blk, S)
            assert np.allclose(o, o3, rtol=0, atol=TIGHT), (blk, S)
            assert np.array_equal(np.isneginf(lse), np.isneginf(l3))
            assert np.allclose(lse[np.isfinite(lse)], l3[np.isfinite(lse)], rtol=0, atol=TIGHT)
            ntiles = -(-Sk // blk)
            per = -(-ntiles // S)
            for s in range(S):
                if s * per >= ntiles:  # empty split -> (0, -inf)
                    assert np.all(op[s] == 0.0) and np.all(np.isneginf(lp[s]))


def check_rows_match_full(orc):
    q, k, v = _rand(9, 2, 6, 7, 4, 2, 3)
    o, lse = orc.fwd(q, k, v, True, 0.3)
    rows = [(1, 3, 5), (0, 0, 0), (1, 1, 2), (0, 2, 4)]
    orow, lrow = orc.rows(q, k, v, True, 0.3, rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.array_equal(orow[n], o[b, i, h]) and lrow[n] == lse[b, h, i]


def check_bf16_widening(orc):
    # bf16 bit patterns are widened exactly: same result as passing the float64 values.
    rng = np.random.default_rng(11)
    shape_q, shape_kv = (1, 3, 2, 4), (1, 5, 1, 4)
    bits = [rng.integers(0, 1 << 16, size=s, dtype=np.uint16) & np.uint16(0xBFFF)
            for s in (shape_q, shape_kv, shape_kv)]
    bits = [np.where((b & 0x7F80) == 0x7F80, b & 0x3FFF, b).astype(np.uint16) for b in bits]
    f64 = [((b.astype(np.uint32) << 16).view(np.float32)).astype(np.float64) for b in bits]
    o1, l1 = orc.fwd(*bits, False, 0.01)
    o2, l2 = orc.fwd(*f64, False, 0.01)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------------------
# Brute force in 50-digit decimal arithmetic


def decimal_attention(q, k, v, causal, scale):
    getcontext().prec = 50
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    g = Hq // Hkv
    o = np.zeros((B, Sq, Hq, d))
    lse = np.zeros((B, Hq, Sq))
    D = Decimal
    sc = D(float(scale))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for i in range(Sq):
                s = []
                for j in range(Sk):
                    if causal and j > i + Sk - Sq:
                        continue
                    acc = sum(D(float(q[b, i, h, c])) * D(float(k[b, j, hk, c])) for c in range(d))
                    s.append((j, sc * acc))
                if not s:
                    lse[b, h, i] = -np.inf
                    continue
                m = max(x for _, x in s)
                w = [(j, (x - m).exp()) for j, x in s]
                l = sum(x for _, x in w)
                for c in range(d):
                    o[b, i, h, c] = float(sum(x * D(float(v[b, j, hk, c])) for j, x in w) / l)
                lse[b, h, i] = float(m + l.ln())
    return o, lse


def check_decimal_brute_force(orc):
    for seed, (B, Sq, Sk, Hq, Hkv, d, causal, scale) in enumerate(
            ((1, 4, 4, 1, 1, 3, False, 0.5), (1, 5, 8, 2, 1, 4, True, 0.35),
             (2, 8, 3, 2, 2, 2, True, 1.1), (1, 6, 7, 4, 2, 3, True, 0.8))):
        q, k, v = _rand(100 + seed, B, Sq, Sk, Hq, Hkv, d)
        od, ld = decimal_attention(q, k, v, causal, scale)
        fin = np.isfinite(ld)
        for o, lse in (orc.fwd(q, k, v, causal, scale), orc.online(q, k, v, causal, scale, 3),
                       orc.split(q, k, v, causal, scale, 2, 3)[2:]):
            assert np.allclose(o, od, rtol=0, atol=TIGHT), np.abs(o - od).max()
            assert np.array_equal(np.isneginf(lse), ~fin)
            assert np.allclose(lse[fin], ld[fin], rtol=0, atol=TIGHT)


# ---------------------------------------------------------------------------
# Backward pass


def check_backward_worked_example(orc):
    g = golden("backward_examples.json")["worked"]
    ks = [_num(x) for x in g["k"]]
    q, k, v = one_row(g["q"], ks, g["v"])
    do_ = np.full((1, 1, 1, 1), g["dO"])
    dq, dk, dv, dsum, _ = orc.bwd(q, k, v, do_, False, g["scale"])
    P = g["printed_P"]
    assert abs(dsum[0, 0, 0] - g["printed_D"]) < TIGHT, dsum
    # q = 1 and scale = 1: dK_j = dS_j exactly.
    assert np.allclose(dk.ravel(), g["printed_dS"], rtol=0, atol=TIGHT), dk.ravel()
    assert abs(sum(g["printed_dS"])) < TIGHT
    assert np.allclose(dv.ravel(), [p * g["dO"] for p in P], rtol=0, atol=TIGHT), dv.ravel()
    assert abs(dq[0, 0, 0, 0] - sum(x * kk for x, kk in zip(g["printed_dS"], ks))) < TIGHT
    assert abs(g["dO"] * g["printed_O"] - g["printed_D"]) < TIGHT
    # The same scores through the scale argument: k = [0, 1], scale = ln 3.  The scale
    # enters both gradients: dQ = ln3 * (dS . k) = 1.5 ln3 again, dK = ln3 * dS * q.
    q2, k2, v2 = one_row(g["q"], [0.0, 1.0], g["v"])
    dq2, dk2, dv2, _, _ = orc.bwd(q2, k2, v2, do_, False, LN3)
    assert abs(dq2[0, 0, 0, 0] - 1.5 * LN3) < TIGHT, dq2
    assert np.allclose(dk2.ravel(), [LN3 * x for x in g["printed_dS"]], rtol=0, atol=TIGHT)
    assert np.allclose(dv2, dv, rtol=0, atol=TIGHT)


def check_backward_exercise_2(orc):
    g = golden("backward_examples.json")["exercise_2"]
    P, V, dO, want = g["P"], g["V"], g["dO"], g["derived"]
    q, k, v = one_row([1.0], [math.log(x) for x in P], V)
    do_ = np.full((1, 1, 1, 1), dO)
    dq, dk, dv, dsum, _ = orc.bwd(q, k, v, do_, False, 1.0)
    assert abs(dsum[0, 0, 0] - want["D"]) < TIGHT and abs(dO * want["O"] - want["D"]) < TIGHT
    assert np.allclose(dk.ravel(), want["dS"], rtol=0, atol=TIGHT), dk.ravel()
    assert np.allclose(dv.ravel(), want["dV"], rtol=0, atol=TIGHT), dv.ravel()
    assert abs(sum(want["dS"])) < TIGHT   # the page's self-check


def check_backward_finite_differences(orc):
    # Independent pin: central differences of the forward oracle's loss <dO, O>
    # (the explainer's CPU lab compares its gradients the same way), also with a sliding
    # window and ALiBi slopes, whose backward is checked against the forward only here.
    h = 1e-5
    for seed, (B, Sq, Sk, Hq, Hkv, d, causal, scale, window, alibi) in enumerate(
            ((1, 3, 4, 2, 1, 3, False, 0.6, None, None),
             (1, 5, 3, 2, 2, 2, True, 0.9, None, None),
             (2, 3, 6, 3, 1, 2, True, 0.45, None, None),
             (1, 4, 4, 1, 1, 4, True, 1.3, None, None),
             (1, 6, 7, 2, 1, 3, False, 0.8, (2, 1), None),
             (1, 5, 6, 2, 2, 2, True, 0.7, (1, 0), [0.5, 0.25]),
             (2, 4, 5, 2, 1, 2, False, 0.9, None, [[0.3, 0.6], [0.1, 0.2]]))):
        q, k, v = _rand(200 + seed, B, Sq, Sk, Hq, Hkv, d)
        do_ = np.random.default_rng(300 + seed).standard_normal(q.shape)
        dq, dk, dv, _, _ = orc.bwd(q, k, v, do_, causal, scale, window=window, alibi=alibi)

        def loss(qq, kk, vv):
            o = orc.fwd(qq, kk, vv, causal, scale, window=window, alibi=alibi)[0]
            return float(np.sum(o * do_))

        for which, grad in ((0, dq), (1, dk), (2, dv)):
            base = [q, k, v]
            for idx in np.ndindex(base[which].shape):
                plus = [x.copy() for x in base]
                minus = [x.copy() for x in base]
                plus[which][idx] += h
                minus[which][idx] -= h
                fd = (loss(*plus) - loss(*minus)) / (2 * h)
                assert abs(fd - grad[idx]) < 2e-8, (seed, which, idx, fd, grad[idx])


def check_backward_invariants(orc):
    for seed, (B, Sq, Sk, Hq, Hkv, d, causal) in enumerate(
            ((2, 6, 9, 4, 2, 3, True), (1, 7, 5, 2, 1, 4, True), (2, 5, 5, 3, 3, 2, False))):
        q, k, v = _rand(400 + seed, B, Sq, Sk, Hq, Hkv, d)
        do_ = np.random.default_rng(500 + seed).standard_normal(q.shape)
        scale = 0.7
        dq, dk, dv, dsum, _ = orc.bwd(q, k, v, do_, causal, scale)
        o, lse = orc.fwd(q, k, v, causal, scale)
        # D is dO . O of the forward output.
        assert np.allclose(dsum, np.einsum("bihc,bihc->bhi", do_, o), rtol=0, atol=TIGHT)
        # Each row's dS sums to zero, so the keys' dK sum to zero per head and column.
        assert np.allclose(dk.sum(axis=1), 0.0, rtol=0, atol=1e-11), dk.sum(axis=1)
        # P rows sum to one (rows with a visible key), so the keys' dV sum to the
        # group's dO over those rows.
        seen = np.isfinite(lse)                                   # [B, Hq, Sq]
        g = Hq // Hkv
        want = np.einsum("bihc,bhi->bhc", do_, seen.astype(float)).reshape(B, Hkv, g, d).sum(2)
        assert np.allclose(dv.sum(axis=1), want, rtol=0, atol=1e-11)
        # A row with no visible key gets dQ = 0.
        for b, h, i in zip(*np.nonzero(~seen)):
            assert np.all(dq[b, i, h] == 0.0)


def check_backward_units(orc):
    # Computing chosen (batch, kv head) units alone gives their slices exactly, zeros elsewhere.
    B, Sq, Sk, Hq, Hkv, d = 2, 5, 6, 4, 2, 3
    q, k, v = _rand(600, B, Sq, Sk, Hq, Hkv, d)
    do_ = np.random.default_rng(601).standard_normal(q.shape)
    full = orc.bwd(q, k, v, do_, True, 0.8)
    part = orc.bwd(q, k, v, do_, True, 0.8, units=[(1, 0)])
    g = Hq // Hkv
    dq_f, dk_f, dv_f, ds_f, _ = full
    dq_p, dk_p, dv_p, ds_p, _ = part
    assert np.array_equal(dk_p[1, :, 0], dk_f[1, :, 0]) and np.array_equal(dv_p[1, :, 0], dv_f[1, :, 0])
    assert np.array_equal(dq_p[1, :, 0:g], dq_f[1, :, 0:g]) and np.array_equal(ds_p[1, 0:g], ds_f[1, 0:g])
    assert not dk_p[0].any() and not dk_p[1, :, 1].any() and not dq_p[0].any()
    assert not dq_p[1, :, g:].any() and not ds_p[0].any()


def check_backward_bf16_widening(orc):
    rng = np.random.default_rng(12)
    shape_q, shape_kv = (1, 5, 2, 4), (1, 7, 1, 4)
    bits = [(rng.integers(0, 2 ** 16, size=s, dtype=np.uint32) & 0x3F7F | 0x3C00).astype(np.uint16)
            for s in (shape_q, shape_kv, shape_kv, shape_q)]
    widened = [(b.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for b in bits]
    r1 = orc.bwd(*bits, True, 0.5)
    r2 = orc.bwd(*widened, True, 0.5)
    for a, b in zip(r1[:4], r2[:4]):
        assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# Variable-length batches and the paged KV cache


def check_varlen_printed_prefix_sums(orc):
    g = golden("varlen_cu_seqlens.json")
    cu = g["cu_seqlens"]
    assert [cu[i + 1] - cu[i] for i in range(len(cu) - 1)] == g["printed_lengths"]
    rng = np.random.default_rng(21)
    total = cu[-1]
    q = rng.standard_normal((total, 2, 3))
    k = rng.standard_normal((total, 1, 3))
    v = rng.standard_normal((total, 1, 3))
    o, lse = orc.varlen(q, k, v, cu, cu, True, 0.6)
    # sequences 2 and 3 hold one query and one key: O = v, LSE = that score
    for r in (248, 249):
        for h in range(2):
            assert np.allclose(o[r, h], v[r, 0], rtol=0, atol=TIGHT)
            assert abs(lse[h, r] - 0.6 * np.dot(q[r, h], k[r, 0])) < TIGHT
    # sequence 1 is the dense problem on rows 0..247
    o1, l1 = orc.fwd(q[None, :248], k[None, :248], v[None, :248], True, 0.6)
    assert np.allclose(o[:248], o1[0], rtol=0, atol=TIGHT)
    assert np.allclose(lse[:, :248], l1[0], rtol=0, atol=TIGHT)


def check_varlen_equal_lengths_and_independence(orc):
    q, k, v = _rand(700, 3, 5, 6, 4, 2, 3)
    o_b, l_b = orc.fwd(q, k, v, True, 0.8)
    cu_q, cu_k = [0, 5, 10, 15], [0, 6, 12, 18]
    o, lse = orc.varlen(q.reshape(15, 4, 3), k.reshape(18, 2, 3), v.reshape(18, 2, 3),
                        cu_q, cu_k, True, 0.8)
    assert np.allclose(o.reshape(3, 5, 4, 3), o_b, rtol=0, atol=TIGHT)
    assert np.allclose(lse.reshape(4, 3, 5).transpose(1, 0, 2), l_b, rtol=0, atol=TIGHT)
    # Changing sequence 1's keys leaves the other sequences' outputs alone.
    k2 = k.reshape(18, 2, 3).copy()
    k2[6:12] += np.random.default_rng(701).standard_normal(k2[6:12].shape)
    o2, l2 = orc.varlen(q.reshape(15, 4, 3), k2, v.reshape(18, 2, 3), cu_q, cu_k, True, 0.8)
    keep = np.r_[0:5, 10:15]
    assert np.array_equal(o2[keep], o[keep]) and np.array_equal(l2[:, keep], lse[:, keep])
    assert not np.allclose(o2[5:10], o[5:10])
    # An empty query sequence and a sequence without keys.
    o3, l3 = orc.varlen(q.reshape(15, 4, 3)[:10], k.reshape(18, 2, 3)[:6], v.reshape(18, 2, 3)[:6],
                        [0, 5, 5, 10], [0, 6, 6, 6], False, 0.8)
    assert np.all(o3[5:10] == 0.0) and np.all(l3[:, 5:10] == -np.inf)


def check_paged_cache_gather(orc):
    rng = np.random.default_rng(22)
    B, Sq, Hq, Hkv, d, page, nblk = 2, 3, 4, 2, 3, 4, 3
    q = rng.standard_normal((B, Sq, Hq, d))
    kc = rng.standard_normal((B * nblk, page, Hkv, d))
    vc = rng.standard_normal((B * nblk, page, Hkv, d))
    ident = np.arange(B * nblk).reshape(B, nblk)
    seqlens, leftpad = [10, 7], [0, 2]
    o, lse = orc.kvcache(q, kc, vc, ident, seqlens, leftpad, True, 0.7)
    for b in range(B):
        kb = kc[ident[b]].reshape(nblk * page, Hkv, d)[leftpad[b]:seqlens[b]]
        vb = vc[ident[b]].reshape(nblk * page, Hkv, d)[leftpad[b]:seqlens[b]]
        ob, lb = orc.fwd(q[b:b + 1], kb[None], vb[None], True, 0.7)
        assert np.allclose(o[b], ob[0], rtol=0, atol=TIGHT) and np.allclose(lse[b], lb[0], rtol=0, atol=TIGHT)
    # Moving the physical blocks (and the table with them) changes nothing.
    perm = rng.permutation(B * nblk)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    o2, l2 = orc.kvcache(q, kc2, vc2, perm[ident], seqlens, leftpad, True, 0.7)
    assert np.array_equal(o2, o) and np.array_equal(l2, lse)
    # A batch whose keys are all padding: O = 0, LSE = -inf.
    o3, l3 = orc.kvcache(q, kc, vc, ident, [10, 5], [0, 5], True, 0.7)
    assert np.all(o3[1] == 0.0) and np.all(l3[1] == -np.inf)


def check_cache_append(orc):
    rng = np.random.default_rng(23)
    B, S_new, Hkv, d, page, nblk = 2, 3, 2, 2, 4, 2
    kc = rng.standard_normal((B * nblk, page, Hkv, d))
    vc = rng.standard_normal((B * nblk, page, Hkv, d))
    table = np.array([[3, 0], [1, 2]])
    kn = rng.standard_normal((B, S_new, Hkv, d))
    vn = rng.standard_normal((B, S_new, Hkv, d))
    seqlens = [2, 6]                       # batch 1 runs past its capacity of 8 after 2 rows
    kc2, vc2 = orc.append(kn, vn, kc, vc, table, seqlens)
    k0, v0 = orc.kv_gather(kc2, vc2, table, 5, 0, 0)
    assert np.array_equal(k0[:2], orc.kv_gather(kc, vc, table, 2, 0, 0)[0]) and np.array_equal(k0[2:], kn[0])
    assert np.array_equal(v0[2:], vn[0])
    k1, _ = orc.kv_gather(kc2, vc2, table, 8, 0, 1)
    assert np.array_equal(k1[6:], kn[1, :2]) and np.array_equal(k1[:6], orc.kv_gather(kc, vc, table, 6, 0, 1)[0])
    changed = np.argwhere(np.any(kc2 != kc, axis=(2, 3)))
    assert len(changed) == 5            # 3 rows for batch 0, 2 for batch 1


# ---------------------------------------------------------------------------
# Mask and bias variants: sliding window, ALiBi, soft cap


def _frac(x):
    a, b = x.split("/")
    return float(a) / float(b)


def _same(r1, r2, tol=TIGHT):
    (o1, l1), (o2, l2) = r1, r2
    assert np.allclose(o1, o2, rtol=0, atol=tol), np.abs(o1 - o2).max()
    assert np.array_equal(np.isneginf(l1), np.isneginf(l2))
    fin = np.isfinite(l1)
    assert np.allclose(l1[fin], l2[fin], rtol=0, atol=tol)


def check_window_reductions(orc):
    # Zero ALiBi slopes take the options path and change nothing; the window (-1, 0) is
    # the causal mask; limits past both ends of the sequence do nothing.
    for seed, (B, Sq, Sk, Hq, Hkv, d) in enumerate(((2, 5, 9, 4, 2, 3), (1, 9, 4, 2, 2, 3))):
        q, k, v = _rand(800 + seed, B, Sq, Sk, Hq, Hkv, d)
        plain = orc.fwd(q, k, v, False, 0.6)
        causal = orc.fwd(q, k, v, True, 0.6)
        zeros = np.zeros(Hq)
        _same(orc.fwd(q, k, v, False, 0.6, alibi=zeros), plain)
        _same(orc.fwd(q, k, v, True, 0.6, alibi=zeros), causal)
        _same(orc.fwd(q, k, v, False, 0.6, window=(-1, 0)), causal)
        _same(orc.fwd(q, k, v, False, 0.6, window=(Sq + Sk, Sq + Sk)), plain)
        _same(orc.fwd(q, k, v, True, 0.6, window=(Sq + Sk, -1)), causal)
        _same(orc.fwd(q, k, v, True, 0.6, window=(-1, 3)), causal)


def check_window_printed_range(orc):
    # q = 0 gives uniform weights over the visible keys, and v_j = j then reads off the
    # visible range: O = (lo + hi) / 2 and LSE = ln(hi - lo + 1) with lo, hi from the
    # printed range (clipped to the sequence; causal also caps hi at diag).
    g = golden("mask_variants.json")["window_range"]
    assert g["no_limit"] == -1
    for Sq, Sk, wl, wr, causal in ((6, 6, 2, 1, False), (4, 9, 0, 0, False), (9, 4, 1, 2, False),
                                   (5, 8, 3, -1, False), (5, 8, -1, 2, False), (7, 7, 2, 3, True),
                                   (3, 10, 4, -1, True), (10, 3, 0, 1, False), (5, 5, 0, 0, True),
                                   (8, 3, 1, 0, False)):
        q = np.zeros((1, Sq, 1, 1))
        k = np.zeros((1, Sk, 1, 1))
        v = np.arange(Sk, dtype=np.float64).reshape(1, Sk, 1, 1)
        o, lse = orc.fwd(q, k, v, causal, 1.0, window=(wl, wr))
        for i in range(Sq):
            diag = i + Sk - Sq
            lo = 0 if wl < 0 else max(0, diag - wl)
            hi = Sk - 1 if wr < 0 else min(Sk - 1, diag + wr)
            if causal:
                hi = min(hi, diag)
            if lo > hi:
                assert o[0, i, 0, 0] == 0.0 and lse[0, 0, i] == -np.inf, (Sq, Sk, wl, wr, i)
            else:
                assert abs(o[0, i, 0, 0] - 0.5 * (lo + hi)) < TIGHT, (Sq, Sk, wl, wr, i)
                assert abs(lse[0, 0, i] - math.log(hi - lo + 1)) < TIGHT


def check_alibi_derived_examples(orc):
    g = golden("mask_variants.json")["derived"]
    ln2 = math.log(2.0)
    e1 = g["alibi_one_sided"]
    q = np.zeros((1, 1, 1, 1))
    k = np.zeros((1, 3, 1, 1))
    v = np.array(e1["v"]).reshape(1, 3, 1, 1)
    p = orc.probs(q, k, v, False, 1.0, 0, 0, 0, alibi=[ln2])
    assert np.allclose(p, [_frac(x) for x in e1["P"]], rtol=0, atol=TIGHT), p
    o, lse = orc.fwd(q, k, v, False, 1.0, alibi=[ln2])
    assert abs(o[0, 0, 0, 0] - e1["O"]) < TIGHT and abs(lse[0, 0, 0] - math.log(7 / 4)) < TIGHT
    e2 = g["alibi_two_sided"]
    q = np.zeros((1, 3, 1, 1))
    for i, want in e2["rows"].items():
        p = orc.probs(q, k, v, False, 1.0, 0, 0, int(i), alibi=[ln2])
        assert np.allclose(p, [_frac(x) for x in want], rtol=0, atol=TIGHT), (i, p)
    # Slopes [B, Hq]: each (batch, head) uses its own slope.
    q, k, v = _rand(810, 2, 4, 6, 4, 2, 3)
    slopes = np.array([[0.1, 0.5, 0.9, 1.3], [0.2, 0.6, 1.0, 1.4]])
    o, lse = orc.fwd(q, k, v, False, 0.5, alibi=slopes)
    for b in range(2):
        for h in range(4):
            ob, lb = orc.fwd(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h // 2:h // 2 + 1],
                             v[b:b + 1, :, h // 2:h // 2 + 1], False, 0.5, alibi=[slopes[b, h]])
            assert np.allclose(o[b, :, h], ob[0, :, 0], rtol=0, atol=TIGHT)
            assert np.allclose(lse[b, h], lb[0, 0], rtol=0, atol=TIGHT)


def check_alibi_as_extra_feature(orc):
    # Where no visible key lies right of the diagonal (causal, or one decode query at the
    # end), -slope |diag - j| = slope j - slope diag.  Appending 1 to q and slope j / scale
    # to k_j makes plain attention add slope j to each score: O is the ALiBi O and the LSE
    # exceeds the ALiBi LSE by slope * diag.  This goes through the pinned plain definition.
    rng = np.random.default_rng(820)
    for seed, (B, Sq, Sk, Hq, Hkv, d, causal) in enumerate(
            ((1, 6, 6, 2, 1, 3, True), (2, 4, 9, 4, 2, 3, True), (2, 1, 12, 4, 2, 3, False),
             (1, 7, 3, 2, 2, 2, True))):
        q, k, v = _rand(830 + seed, B, Sq, Sk, Hq, Hkv, d)
        slopes = rng.uniform(0.05, 1.0, (B, Hq))
        scale = 0.7
        o, lse = orc.fwd(q, k, v, causal, scale, alibi=slopes)
        g = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                hk = h // g
                qa = np.concatenate([q[b:b + 1, :, h:h + 1], np.ones((1, Sq, 1, 1))], axis=3)
                feat = (slopes[b, h] * np.arange(Sk) / scale).reshape(1, Sk, 1, 1)
                ka = np.concatenate([k[b:b + 1, :, hk:hk + 1], feat], axis=3)
                va = np.concatenate([v[b:b + 1, :, hk:hk + 1], np.zeros((1, Sk, 1, 1))], axis=3)
                oa, la = orc.fwd(qa, ka, va, causal, scale)
                assert np.allclose(o[b, :, h], oa[0, :, 0, :d], rtol=0, atol=1e-11), (seed, b, h)
                for i in range(Sq):
                    if np.isneginf(la[0, 0, i]):
                        assert np.isneginf(lse[b, h, i])
                        continue
                    diag = i + Sk - Sq
                    assert abs(lse[b, h, i] - (la[0, 0, i] - slopes[b, h] * diag)) < 1e-11


def check_softcap_closed_forms(orc):
    g = golden("mask_variants.json")["derived"]["softcap"]
    e = math.e
    want_o, want_l = (2 + 6 * e) / (1 + e), math.log(1 + e)
    q, k, v = one_row([g["q"]], [_num(x) for x in g["k"]], g["v"])
    o, lse = orc.fwd(q, k, v, False, g["scale"], softcap=g["softcap"])
    assert abs(o[0, 0, 0, 0] - want_o) < TIGHT and abs(lse[0, 0, 0] - want_l) < TIGHT
    p = orc.probs(q, k, v, False, g["scale"], 0, 0, 0, softcap=g["softcap"])
    assert np.allclose(p, [1 / (1 + e), e / (1 + e)], rtol=0, atol=TIGHT)
    # The cap acts on the scaled score: the same logits through k = [0, 1], scale = ln 3.
    q2, k2, v2 = one_row([1.0], [0.0, 1.0], g["v"])
    o2, l2 = orc.fwd(q2, k2, v2, False, LN3, softcap=2.0)
    assert abs(o2[0, 0, 0, 0] - want_o) < TIGHT and abs(l2[0, 0, 0] - want_l) < TIGHT
    # Saturation: scores far above the cap all become the cap (equal weights) ...
    q3, k3, v3 = one_row([1.0], [100.0, 200.0, 300.0], [1.0, 2.0, 6.0])
    o3, l3 = orc.fwd(q3, k3, v3, False, 1.0, softcap=1.0)
    assert abs(o3[0, 0, 0, 0] - 3.0) < TIGHT and abs(l3[0, 0, 0] - (1 + math.log(3))) < TIGHT
    # ... and a cap far above the scores changes them by about s^3 / (3 c^2).
    q4, k4, v4 = _rand(840, 1, 5, 7, 2, 1, 4)
    _same(orc.fwd(q4, k4, v4, True, 0.5, softcap=1e7), orc.fwd(q4, k4, v4, True, 0.5), 1e-11)


def check_variants_online_split_agree(orc):
    rng = np.random.default_rng(850)
    cases = ((1, 9, 9, 2, 1, 3, False, (2, 1), True, 0.0),
             (2, 5, 11, 4, 2, 3, True, (3, -1), True, 3.0),
             (1, 11, 4, 2, 2, 2, False, (1, 0), False, 1.5),
             (2, 6, 6, 2, 1, 4, False, (-1, -1), True, 0.8),
             (1, 8, 13, 2, 2, 3, False, (0, 2), False, 0.0))
    for seed, (B, Sq, Sk, Hq, Hkv, d, causal, win, use_alibi, cap) in enumerate(cases):
        q, k, v = _rand(860 + seed, B, Sq, Sk, Hq, Hkv, d)
        opts = dict(window=win, alibi=rng.uniform(0.1, 0.9, (B, Hq)) if use_alibi else None,
                    softcap=cap)
        ref = orc.fwd(q, k, v, causal, 0.45, **opts)
        for blk in (1, 2, 3, 5, 64):
            _same(orc.online(q, k, v, causal, 0.45, blk, **opts), ref)
        for blk, S in ((1, 4), (2, 3), (3, 2), (1, 9)):
            _same(orc.split(q, k, v, causal, 0.45, blk, S, **opts)[2:], ref)
        rows = [(B - 1, Hq - 1, Sq - 1), (0, 0, 0), (0, Hq // 2, Sq // 2)]
        orow, lrow = orc.rows(q, k, v, causal, 0.45, rows, **opts)
        for n, (b, h, i) in enumerate(rows):
            assert np.array_equal(orow[n], ref[0][b, i, h]) and lrow[n] == ref[1][b, h, i]


def decimal_attention_variants(q, k, v, causal, scale, window, slopes, cap):
    """The variants in 50-digit decimal: scale, soft cap, ALiBi bias, window/causal mask."""
    getcontext().prec = 50
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    g = Hq // Hkv
    D = Decimal
    o = np.zeros((B, Sq, Hq, d))
    lse = np.zeros((B, Hq, Sq))
    wl, wr = window

    def tanh(x):
        t = (2 * x).exp()
        return (t - 1) / (t + 1)

    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for i in range(Sq):
                diag = i + Sk - Sq
                s = []
                for j in range(Sk):
                    if (causal and j > diag) or (wl >= 0 and j < diag - wl) or \
                            (wr >= 0 and j > diag + wr):
                        continue
                    x = D(float(scale)) * sum(D(float(q[b, i, h, c])) * D(float(k[b, j, hk, c]))
                                              for c in range(d))
                    if cap > 0:
                        x = D(cap) * tanh(x / D(cap))
                    if slopes is not None:
                        x -= D(float(slopes[b, h])) * abs(D(diag - j))
                    s.append((j, x))
                if not s:
                    lse[b, h, i] = -np.inf
                    continue
                m = max(x for _, x in s)
                w = [(j, (x - m).exp()) for j, x in s]
                l = sum(x for _, x in w)
                for c in range(d):
                    o[b, i, h, c] = float(sum(x * D(float(v[b, j, hk, c])) for j, x in w) / l)
                lse[b, h, i] = float(m + l.ln())
    return o, lse


def check_variants_decimal_brute_force(orc):
    rng = np.random.default_rng(870)
    for seed, (B, Sq, Sk, Hq, Hkv, d, causal, win, cap) in enumerate(
            ((1, 5, 7, 2, 1, 3, False, (1, 2), 1.2), (1, 6, 6, 2, 2, 2, True, (2, -1), 0.0),
             (2, 4, 3, 2, 1, 3, False, (-1, 0), 2.5), (1, 7, 5, 1, 1, 3, False, (0, 1), 0.7))):
        q, k, v = _rand(880 + seed, B, Sq, Sk, Hq, Hkv, d)
        slopes = rng.uniform(0.1, 1.5, (B, Hq))
        od, ld = decimal_attention_variants(q, k, v, causal, 0.6, win, slopes, cap)
        o, lse = orc.fwd(q, k, v, causal, 0.6, window=win, alibi=slopes, softcap=cap)
        _same((o, lse), (od, ld))


def check_variants_through_cache_and_varlen(orc):
    # The per-batch helpers hand each batch its own slopes and the options.
    rng = np.random.default_rng(890)
    B, Sq, Hq, Hkv, d, page, nblk = 2, 3, 4, 2, 3, 4, 3
    q = rng.standard_normal((B, Sq, Hq, d))
    kc = rng.standard_normal((B * nblk, page, Hkv, d))
    vc = rng.standard_normal((B * nblk, page, Hkv, d))
    table = rng.permutation(B * nblk).reshape(B, nblk)
    slopes = rng.uniform(0.1, 0.9, (B, Hq))
    opts = dict(window=(4, 0), alibi=slopes, softcap=2.0)
    o, lse = orc.kvcache(q, kc, vc, table, [10, 7], [1, 0], True, 0.7, **opts)
    for b, (n, lp) in enumerate(((10, 1), (7, 0))):
        kb, vb = orc.kv_gather(kc, vc, table, n, lp, b)
        ob, lb = orc.fwd(q[b:b + 1], kb[None], vb[None], True, 0.7, window=(4, 0),
                         alibi=slopes[b], softcap=2.0)
        assert np.array_equal(o[b], ob[0]) and np.array_equal(lse[b], lb[0])
    qv, kv, vv = (rng.standard_normal((9, Hq, d)), rng.standard_normal((11, Hkv, d)),
                  rng.standard_normal((11, Hkv, d)))
    o, lse = orc.varlen(qv, kv, vv, [0, 4, 9], [0, 5, 11], True, 0.7, **opts)
    ob, lb = orc.fwd(qv[None, 4:9], kv[None, 5:11], vv[None, 5:11], True, 0.7, window=(4, 0),
                     alibi=slopes[1], softcap=2.0)
    assert np.array_equal(o[4:9], ob[0]) and np.array_equal(lse[:, 4:9], lb[0])


# ---------------------------------------------------------------------------
# FP8: the E4M3 format, block quantization, rotation, FP8 attention


def check_e4m3_format(orc):
    g = golden("fp8_e4m3.json")
    codes = np.arange(256, dtype=np.uint8)
    val = orc.e4m3_decode(codes)
    for c, want in g["values"].items():
        got = val[int(c, 16)]
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (c, got)
    nan = [int(c, 16) for c in g["nan_codes"]]
    assert np.isnan(val[nan]).all() and np.isnan(val).sum() == 2
    pos = val[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[-1] == g["max_finite"]
    assert np.array_equal(val[0x80:0xFF], -pos)
    assert pos[1] == g["min_subnormal"] and pos[8] == g["min_normal"]
    # each binade [2^e, 2^(e+1)) of normals holds 8 values spaced 2^(e-3)
    for e in range(-6, 9):
        binade = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(binade) == (8 if e < 8 else 7), e
        assert np.allclose(np.diff(binade), 2.0 ** (e - 3), rtol=0, atol=0)


def check_e4m3_rounding(orc):
    codes = np.arange(256, dtype=np.uint8)
    val = orc.e4m3_decode(codes)
    fin = ~np.isnan(val)
    assert np.array_equal(orc.e4m3_encode(val[fin].astype(np.float32)), codes[fin])  # round trip
    pos = val[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2                 # exactly representable in fp32
    enc = orc.e4m3_encode(mids.astype(np.float32))
    lo = np.arange(0, 0x7E)
    assert np.array_equal(enc, np.where(lo % 2 == 0, lo, lo + 1)), "ties go to the even code"
    below = np.nextafter(mids.astype(np.float32), np.float32(0))
    above = np.nextafter(mids.astype(np.float32), np.float32(1e9))
    assert np.array_equal(orc.e4m3_encode(below), lo) and np.array_equal(orc.e4m3_encode(above), lo + 1)
    sat = orc.e4m3_encode(np.array([448.0, 463.9, 464.0, 1e6, -1e6], np.float32))
    assert list(sat) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    tiny = orc.e4m3_encode(np.array([2.0 ** -10, 2.0 ** -10 + 2.0 ** -20, -2.0 ** -11, 0.0], np.float32))
    assert list(tiny) == [0x00, 0x01, 0x80, 0x00]
    assert orc.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def _sylvester(d):
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def check_fwht(orc):
    rng = np.random.default_rng(1000)
    for d in (2, 8, 64, 128):
        x = rng.standard_normal((5, d)).astype(np.float32)
        y = orc.fwht(x)
        ref = x.astype(np.float64) @ _sylvester(d) / math.sqrt(d)   # H is symmetric
        assert np.allclose(y, ref, rtol=0, atol=1e-5 * math.sqrt(d)), d
        assert np.allclose(orc.fwht(y), x, rtol=0, atol=1e-5 * math.sqrt(d))    # H H / d = I
        e0 = np.zeros((1, d), np.float32)
        e0[0, 0] = 1.0
        assert np.allclose(orc.fwht(e0), 1 / math.sqrt(d), rtol=0, atol=1e-7)
    # an orthogonal transform of both q and k keeps every dot product
    q = rng.standard_normal((6, 128)).astype(np.float32)
    k = rng.standard_normal((9, 128)).astype(np.float32)
    assert np.allclose(orc.fwht(q).astype(np.float64) @ orc.fwht(k).T.astype(np.float64),
                       q.astype(np.float64) @ k.T.astype(np.float64), rtol=0, atol=1e-4)


def check_quantize_blocks(orc):
    rng = np.random.default_rng(1001)
    B, S, H, d = 2, 300, 3, 16
    x = (rng.standard_normal((B, S, H, d)) * np.exp(rng.uniform(-3, 3, (B, 1, H, 1)))).astype(np.float32)
    x[1, 128:256, 2] = 0.0                                 # an all-zero block
    codes, scales = orc.quantize_fp8(x)
    assert scales.shape == (B, H, 3)
    val = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    for b in range(B):
        for h in range(H):
            for blk in range(3):
                rows = slice(128 * blk, min(128 * blk + 128, S))
                xb = x[b, rows, h]
                amax = np.abs(xb).max()
                sc = np.float32(amax) / np.float32(448) if amax > 0 else np.float32(1)
                assert scales[b, h, blk] == sc, (b, h, blk)
                cb = codes[b, rows, h]
                if amax == 0:
                    assert np.all(cb == 0)
                    continue
                # the largest magnitude lands on the top code, and every value is within
                # half a code spacing of its code (relative 2^-4, absolute 2^-10 near 0)
                assert (cb & 0x7F).max() == 0x7E
                y = (xb / sc).astype(np.float64)
                err = np.abs(val[cb] - y)
                assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(y), 2.0 ** -10) + 1e-12)
                assert np.all(np.signbit(val[cb]) == np.signbit(y))
    # blocks are independent: changing block 1 leaves block 0 and 2 alone
    x2 = x.copy()
    x2[0, 130, 0] *= 50.0
    c2, s2 = orc.quantize_fp8(x2)
    assert np.array_equal(c2[0, :128], codes[0, :128]) and np.array_equal(c2[0, 256:], codes[0, 256:])
    assert s2[0, 0, 1] != scales[0, 0, 1] and np.array_equal(s2[0, 0, [0, 2]], scales[0, 0, [0, 2]])
    # bf16 inputs are widened exactly; rotation is the quantization of the rotated rows
    bits = synth_bits(rng, (1, 200, 2, 64))
    cb, sb = orc.quantize_fp8(bits)
    cf, sf = orc.quantize_fp8(((bits.astype(np.uint32) << 16).view(np.float32)))
    assert np.array_equal(cb, cf) and np.array_equal(sb, sf)
    cr, sr = orc.quantize_fp8(bits, rotate=True)
    rot = orc.fwht((bits.astype(np.uint32) << 16).view(np.float32))
    c3, s3 = orc.quantize_fp8(rot)
    assert np.array_equal(cr, c3) and np.array_equal(sr, s3)


def synth_bits(rng, shape):
    """bf16 bit patterns of N(0,1) values (the top half of their float32 bits)."""
    f = rng.standard_normal(shape).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def check_fp8_attention(orc):
    rng = np.random.default_rng(1002)
    for causal, (B, Sq, Sk, Hq, Hkv, d) in ((True, (1, 200, 200, 2, 1, 16)),
                                           (False, (2, 130, 260, 4, 2, 8))):
        q = rng.standard_normal((B, Sq, Hq, d)).astype(np.float32)
        k = rng.standard_normal((B, Sk, Hkv, d)).astype(np.float32)
        v = rng.standard_normal((B, Sk, Hkv, d)).astype(np.float32)
        (q8, qs), (k8, ks), (v8, vs) = (orc.quantize_fp8(x) for x in (q, k, v))
        o, lse, o_abs, inv_l = orc.fwd_fp8(q8, k8, v8, qs, ks, vs, causal, 0.3)
        # the dequantized tensors, built here from the pinned decode table and the
        # per-(batch, head, 128-row) scales
        table = orc.e4m3_decode(np.arange(256, dtype=np.uint8))

        def deq(c, sc):
            blk = np.arange(c.shape[1]) // 128
            return table[c] * sc[:, :, blk].transpose(0, 2, 1)[..., None].astype(np.float64)

        qd, kd, vd = deq(q8, qs), deq(k8, ks), deq(v8, vs)
        o2, l2 = orc.fwd(qd, kd, vd, causal, 0.3)
        assert np.array_equal(o, o2) and np.array_equal(lse, l2)
        # the dequantized tensors are close to the originals (half a code spacing)
        assert np.abs(vd - v).max() <= 2.0 ** -4 * np.abs(v).max() + 1e-12
        g = Hq // Hkv
        for b, h, i in ((0, 0, 0), (B - 1, Hq - 1, Sq - 1), (0, Hq // 2, Sq // 2)):
            p = orc.probs(qd, kd, vd, causal, 0.3, b, h, i)
            assert np.allclose(o_abs[b, i, h], p @ np.abs(vd[b, :, h // g]), rtol=0, atol=TIGHT)
            s = 0.3 * (kd[b, :, h // g] @ qd[b, i, h])
            vis = np.arange(Sk) <= i + Sk - Sq if causal else np.ones(Sk, bool)
            l = np.exp(s[vis] - s[vis].max()).sum()
            assert abs(inv_l[b, h, i] - 1 / l) < TIGHT


ALL_CHECKS = [
    check_online_softmax_example, check_one_query_two_keys, check_exercise_1, check_exercise_2,
    check_causal_mask_pictures, check_tail_tile_case, check_special_cases,
    check_probability_rows, check_shift_invariance, check_key_permutation, check_gqa_grouping,
    check_online_and_split_agree, check_rows_match_full, check_bf16_widening,
    check_decimal_brute_force, check_backward_worked_example, check_backward_exercise_2,
    check_backward_finite_differences, check_backward_invariants, check_backward_units,
    check_backward_bf16_widening, check_varlen_printed_prefix_sums,
    check_varlen_equal_lengths_and_independence, check_paged_cache_gather, check_cache_append,
    check_window_reductions, check_window_printed_range, check_alibi_derived_examples,
    check_alibi_as_extra_feature, check_softcap_closed_forms, check_variants_online_split_agree,
    check_variants_decimal_brute_force, check_variants_through_cache_and_varlen,
    check_e4m3_format, check_e4m3_rounding, check_fwht, check_quantize_blocks, check_fp8_attention,
]


def failing_checks(orc):
    failed = []
    for chk in ALL_CHECKS:
        try:
            chk(orc)
        except AssertionError:
            failed.append(chk.__name__)
    return failed
