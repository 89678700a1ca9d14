"""attn_fwd_ex and attn_fwd_kvcache_ex (the sliding window, ALiBi and soft-cap variants)
against the fp64 CPU oracle, element by element, through the C ABI.

Small shapes span several key tiles with ragged tails and windows that start and end
inside tiles; the full-size cases are compared on sampled rows.  ALiBi slopes are the
usual geometric sequence 2^(-8(h+1)/H), as fp32 on the device and the same values widened
on the oracle side."""
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


def slopes_for(B, Hq, per_batch):
    s = np.array([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=np.float32)
    if per_batch:
        s = np.stack([s * (1.0 + 0.25 * b) for b in range(B)]).astype(np.float32)
    return s


def run_ex(ff, q, k, v, causal, scale, window=(-1, -1), slopes=None, softcap=0.0):
    import torch
    al = None if slopes is None else torch.from_numpy(slopes).to("cuda:0")
    o, lse = ff.forward(to_dev(q), to_dev(k), to_dev(v), causal, scale, window=window,
                        alibi_slopes=al, softcap=softcap)
    torch.cuda.synchronize()
    return host(o), host(lse)


def oracle_opts(window, slopes, softcap):
    return dict(window=window, alibi=None if slopes is None else slopes.astype(np.float64),
                softcap=float(np.float32(softcap)))


WINDOW_CASES = [
    # B, Sq, Sk, Hq, Hkv, d, causal, (wl, wr)
    (1, 333, 333, 2, 1, 64, False, (64, 0)),
    (1, 333, 333, 2, 1, 64, False, (100, 37)),
    (2, 300, 300, 4, 2, 128, False, (0, 0)),
    (1, 300, 300, 2, 2, 128, True, (150, -1)),
    (1, 300, 300, 2, 2, 128, False, (-1, 50)),
    (1, 450, 450, 2, 1, 64, False, (1, 1)),
    (1, 300, 300, 2, 2, 128, True, (500, 500)),     # wider than the sequence
    (1, 200, 517, 4, 1, 128, True, (129, 7)),       # Sq < Sk
    (1, 300, 77, 2, 2, 64, False, (10, 3)),         # Sq > Sk: early rows see nothing
    (1, 1, 1000, 4, 2, 128, False, (255, 0)),       # one query row
    (2, 260, 190, 6, 3, 128, False, (63, 64)),
    (1, 700, 700, 2, 1, 64, True, (200, 0)),        # many unmasked middle tiles
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "B%d_Sq%d_Sk%d_Hq%d_Hkv%d_d%d_%s_w%d_%d" % (
    *c[:6], "causal" if c[6] else "full", *c[7]))
def test_window(ff, oracle, case):
    B, Sq, Sk, Hq, Hkv, d, causal, win = case
    say(f"window case {case}")
    q, k, v = make_inputs(B, Sq, Sk, Hq, Hkv, d, seed=900 + Sq + Sk + win[0])
    scale = synth.f32(1 / math.sqrt(d))
    o, lse = run_ex(ff, q, k, v, causal, scale, window=win)
    o_ref, lse_ref = oracle.fwd(q, k, v, causal, scale, window=win)
    check_outputs(o, lse, o_ref, lse_ref, str(case))


def test_window_minus1_0_is_causal(ff):
    # The window (-1, 0) on the non-causal kernel is the causal mask.
    q, k, v = make_inputs(2, 333, 333, 4, 2, 128, seed=901)
    o1, l1 = run_ex(ff, q, k, v, False, 0.09, window=(-1, 0))
    o2, l2 = run_ex(ff, q, k, v, True, 0.09)
    assert np.allclose(o1, o2, rtol=0, atol=1e-6) and np.allclose(l1, l2, rtol=0, atol=1e-6)


ALIBI_CASES = [
    # B, Sq, Sk, Hq, Hkv, d, causal, window, per-batch slopes, softcap
    (2, 300, 300, 4, 2, 128, True, (-1, -1), False, 0.0),
    (2, 300, 300, 4, 2, 128, False, (-1, -1), True, 0.0),
    (1, 333, 400, 4, 1, 64, True, (120, -1), True, 0.0),
    (1, 257, 257, 2, 2, 64, False, (40, 40), False, 0.0),
    (2, 300, 300, 4, 2, 128, True, (-1, -1), False, 5.0),
    (1, 333, 333, 2, 1, 64, False, (-1, -1), False, 0.5),     # strong cap
    (1, 300, 300, 2, 2, 128, False, (80, 10), False, 30.0),
    (2, 300, 300, 4, 2, 128, True, (100, -1), True, 2.0),     # all three
    (1, 150, 77, 2, 2, 64, False, (-1, -1), True, 1.5),       # Sq > Sk
]


@pytest.mark.parametrize("case", ALIBI_CASES, ids=lambda c: "B%d_Sq%d_Sk%d_d%d_%s_w%d_%d_%s_cap%g" % (
    c[0], c[1], c[2], c[5], "causal" if c[6] else "full", *c[7],
    ("alibiBH" if c[8] else "alibiH"), c[9]))
def test_alibi_softcap(ff, oracle, case):
    B, Sq, Sk, Hq, Hkv, d, causal, win, per_batch, cap = case
    say(f"alibi/softcap case {case}")
    q, k, v = make_inputs(B, Sq, Sk, Hq, Hkv, d, seed=950 + Sq + Sk)
    scale = synth.f32(1 / math.sqrt(d))
    slopes = slopes_for(B, Hq, per_batch)
    o, lse = run_ex(ff, q, k, v, causal, scale, win, slopes, cap)
    o_ref, lse_ref = oracle.fwd(q, k, v, causal, scale, **oracle_opts(win, slopes, cap))
    check_outputs(o, lse, o_ref, lse_ref, str(case))


@pytest.mark.parametrize("d", [64, 128])
def test_softcap_closed_form_on_gpu(ff, d):
    # q = e0, scores [0, ln 3] through k = [0, 1] and scale = ln 3; cap 2 turns them into
    # the logits [0, 1]: O = (2 + 6e)/(1 + e), LSE = ln(1 + e).
    n = 2
    q = np.zeros((1, 1, 1, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, n, 1, d), np.float32)
    k[0, :, 0, 0] = [0.0, 1.0]
    v = np.zeros((1, n, 1, d), np.float32)
    v[0, :, 0, 0] = [2.0, 6.0]
    q, k, v = (synth.f32_to_bf16_bits(x) for x in (q, k, v))
    o, lse = run_ex(ff, q, k, v, False, synth.f32(math.log(3.0)), softcap=2.0)
    e = math.e
    assert abs(o[0, 0, 0, 0] - (2 + 6 * e) / (1 + e)) < 2e-2
    assert abs(lse[0, 0, 0] - math.log(1 + e)) < 1e-3


def test_sliding_window_full_size_every_tile(ff, oracle):
    import torch
    w = synth.WORKLOADS["sliding_window_gqa"]
    say(f"full-size workload sliding_window_gqa: {w}")
    q, k, v = synth.make_qkv(w)
    win = (w["window_left"], w["window_right"])
    o_d, lse_d = ff.forward(to_dev(q), to_dev(k), to_dev(v), w["causal"], w["scale"],
                            window=win)
    torch.cuda.synchronize()
    assert torch.isfinite(o_d).all().item() and torch.isfinite(lse_d).all().item()
    rows = tile_edge_rows(w["B"], w["Sq"], w["Hq"], seed=31)
    say(f"  comparing {len(rows)} rows (first and last of every query tile)")
    o_ref, lse_ref = oracle.rows(q, k, v, w["causal"], w["scale"], rows, window=win)
    idx = torch.tensor(rows, dtype=torch.long)
    check_outputs(host(o_d[idx[:, 0], idx[:, 2], idx[:, 1]]),
                  host(lse_d[idx[:, 0], idx[:, 1], idx[:, 2]]), o_ref, lse_ref,
                  "sliding_window_gqa")


def test_variants_are_deterministic(ff):
    import torch
    q, k, v = make_inputs(1, 500, 500, 4, 2, 128, seed=960)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    al = torch.from_numpy(slopes_for(1, 4, False)).to("cuda:0")
    r1 = ff.forward(qd, kd, vd, True, 0.09, window=(100, 0), alibi_slopes=al, softcap=3.0)
    r2 = ff.forward(qd, kd, vd, True, 0.09, window=(100, 0), alibi_slopes=al, softcap=3.0)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


# ---------------------------------------------------------------------------
# attn_fwd_kvcache_ex

def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


CACHE_CASES = [
    # B, Sq, Hq, Hkv, d, page, max_blocks, seqlens, leftpad, causal, window, alibi, cap, splits
    (3, 1, 8, 2, 128, 64, 8, [300, 1, 512], None, False, (100, -1), False, 0.0, 1),
    (3, 1, 8, 2, 128, 64, 8, [300, 1, 512], None, False, (100, -1), False, 0.0, 3),
    (3, 1, 8, 2, 128, 64, 8, [300, 7, 512], [5, 0, 100], False, (-1, -1), True, 0.0, 4),
    (3, 4, 8, 2, 128, 64, 8, [300, 7, 512], [5, 0, 33], True, (60, 0), True, 4.0, 2),
    (2, 4, 8, 8, 64, 32, 20, [640, 130], [0, 127], True, (31, -1), False, 1.0, 3),
    (2, 16, 4, 1, 64, 128, 3, [384, 200], [50, 190], False, (20, 5), True, 0.0, 2),
    (4, 1, 32, 8, 128, 256, 4, [0, 1000, 1024, 17], None, False, (511, 0), True, 8.0, 4),
]


@pytest.mark.parametrize("case", CACHE_CASES, ids=lambda c: "B%d_Sq%d_d%d_page%d_%s_w%d_%d_%s_cap%g_S%d" % (
    c[0], c[1], c[4], c[5], "causal" if c[9] else "full", *c[10],
    "alibi" if c[11] else "noalibi", c[12], c[13]))
def test_kvcache_variants(ff, oracle, case):
    import torch
    B, Sq, Hq, Hkv, d, page, mb, seqlens, leftpad, causal, win, use_alibi, cap, S = case
    say(f"kvcache variant case {case}")
    nb = B * mb + 3
    kc = synth.normal_bf16(970 + d, 1, (nb, page, Hkv, d))
    vc = synth.normal_bf16(970 + d, 2, (nb, page, Hkv, d))
    table = np.random.default_rng(971).permutation(nb)[:B * mb].reshape(B, mb).astype(np.int32)
    q = synth.normal_bf16(970 + d, 0, (B, Sq, Hq, d))
    scale = synth.f32(1 / math.sqrt(d))
    slopes = slopes_for(B, Hq, True) if use_alibi else None
    al = None if slopes is None else torch.from_numpy(slopes).to("cuda:0")
    o, lse = ff.forward_kvcache(to_dev(q), to_dev(kc), to_dev(vc), dev_i32(seqlens), causal,
                                scale, block_table=dev_i32(table),
                                cache_leftpad=None if leftpad is None else dev_i32(leftpad),
                                num_splits=S, window=win, alibi_slopes=al, softcap=cap)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.kvcache(q, kc, vc, table, seqlens, leftpad, causal, scale,
                                    **oracle_opts(win, slopes, cap))
    check_outputs(host(o), host(lse), o_ref, lse_ref, str(case))


def test_kvcache_window_full_size(ff, oracle):
    # paged_decode's cache with a 4096-key window: the splits share only the window, and
    # every row is compared with the oracle on the gathered keys.
    import torch
    w = synth.WORKLOADS["paged_decode"]
    B, Sk, Hq, Hkv, d, page = w["B"], w["Sk"], w["Hq"], w["Hkv"], w["d"], w["page"]
    q, k, v = synth.make_qkv(w)
    mb = Sk // page
    table = np.random.default_rng(w["seed"]).permutation(B * mb).astype(np.int32)
    kc = np.empty((B * mb, page, Hkv, d), np.uint16)
    vc = np.empty_like(kc)
    kc[table] = k.reshape(B * mb, page, Hkv, d)
    vc[table] = v.reshape(B * mb, page, Hkv, d)
    seqlens = np.full(B, Sk, np.int32)
    win = (4095, 0)
    S = ff.attn_splitkv_num_splits(B, 1, 4096, Hq, Hkv, d)
    say(f"paged decode with window {win}, {S} splits")
    o, lse = ff.forward_kvcache(to_dev(q), to_dev(kc), to_dev(vc), dev_i32(seqlens), False,
                                w["scale"], block_table=dev_i32(table.reshape(B, mb)),
                                num_splits=S, window=win)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(q, k[:, Sk - 4096:], v[:, Sk - 4096:], False, w["scale"])
    check_outputs(host(o), host(lse), o_ref, lse_ref, "paged_decode window 4096")
