"""attn_quantize_fp8 and attn_fwd_fp8 against the fp64 oracle, through the C ABI.

The quantizer is byte work: its codes and scales must equal the oracle's bit for bit.
The FP8 attention is compared with the oracle's attention on the same codes and scales.
Its error comes from rounding each probability to E4M3 for the PV product: half a code
spacing, at most 2^-4 relative for normal values and 2^-10 absolute for subnormal ones,
in units where the reference point keeps every probability at most 2^8.  The kernel rounds
p~_j = 2^(s_j c - m) r_j, with r_j = sv_t / sv_max the ratio of key j's V block scale to
the largest and m at most the row's maximum, so p~_j >= e^(s_j - max s) r_j, and its row
sum l' is at least the oracle's l = sum_j e^(s_j - max s).  Per output element:

  |dO_c| <= 2^-4 sum_j P_j |v_jc| + 2^-10 sum_{j in Z} |v_jc| / (r_j l) + 2e-3

where Z holds the keys that may round as subnormals (e^(s_j - max s) r_j < 2^-6) and the
last term covers the fp32 arithmetic (as the 2e-2 bar does for bf16, here tighter since
the products of fp8 values are exact in fp32).  The LSE is computed from unrounded
probabilities: within 1e-3, as for bf16."""
import math

import numpy as np
import pytest

import synth
from gpu_helpers import LSE_TOL, host, make_inputs, say, tile_edge_rows, to_dev

pytestmark = pytest.mark.gpu

U8 = 2.0 ** -4      # half spacing of normal E4M3 values, relative
SUB = 2.0 ** -10    # half spacing of subnormal E4M3 values, absolute
SLACK = 2e-3


@pytest.fixture(scope="module")
def ff():
    import torch
    from io_aware_attention_amd import flashfwd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    flashfwd.load()
    return flashfwd


def dev_u8(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda:0")


def dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def block_scaled_bf16(seed, tid, shape, factors):
    """N(0,1) times a factor per 128-row block (cycling through `factors`), as bf16 bits."""
    x = synth.bf16_bits_to_f32(synth.normal_bf16(seed, tid, shape))
    f = np.asarray(factors, np.float32)[(np.arange(shape[1]) // 128) % len(factors)]
    return synth.f32_to_bf16_bits(x * f[None, :, None, None])


def quantize_both(ff, oracle, bits, rotate=False):
    """GPU and oracle quantization of bf16 bits; asserts they agree bit for bit."""
    import torch
    codes, scales = ff.quantize_fp8(to_dev(bits), rotate=rotate)
    torch.cuda.synchronize()
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    c_ref, s_ref = oracle.quantize_fp8(bits, rotate=rotate)
    assert np.array_equal(scales.view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    diff = np.count_nonzero(codes != c_ref)
    assert diff == 0, f"{diff} codes differ"
    return codes, scales


@pytest.mark.parametrize("shape,rotate", [
    ((2, 300, 3, 128), False), ((2, 300, 3, 128), True),
    ((1, 129, 2, 64), False), ((1, 129, 2, 64), True),
    ((1, 1, 1, 128), False), ((3, 256, 1, 64), True),
], ids=lambda x: str(x))
def test_quantize_bit_exact(ff, oracle, shape, rotate):
    say(f"quantize {shape} rotate={rotate}")
    B, S, H, d = shape
    rng = np.random.default_rng(S + d)
    x = synth.bf16_bits_to_f32(synth.normal_bf16(1100 + S, 0, shape))
    x = x * np.exp(rng.uniform(-6, 6, (B, 1, H, 1))).astype(np.float32)   # scales apart
    if S > 128:
        x[0, 128:256, 0] = 0.0                    # an all-zero block
        x[-1, 0:128, -1] = 0.0
        x[-1, 5, -1, 3] = 3e-3                    # a block with one nonzero element
    quantize_both(ff, oracle, synth.f32_to_bf16_bits(x), rotate)


def fp8_row_bound(s_row, vis, va, r):
    """Tolerance of one output row: s_row scaled scores [Sk], vis the visible keys, va |V|
    [Sk, d], r the per-key V scale ratio [Sk]."""
    if not vis.any():
        return np.full(va.shape[1], SLACK)
    e = np.exp(s_row[vis] - s_row[vis].max())
    l = e.sum()
    P = e / l
    sub = e * r[vis] < 2.0 ** -6
    return (U8 * (P @ va[vis]) + SUB * ((sub / r[vis]) @ va[vis]) / l + SLACK)


def fp8_bound(qd, kd, vd, vs, causal, scale):
    """Per-element tolerance of the FP8 attention (see the module docstring)."""
    B, Sq, Hq, d = qd.shape
    Sk, Hkv = kd.shape[1], kd.shape[2]
    g = Hq // Hkv
    tol = np.empty((B, Sq, Hq, d))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            r = (vs[b, hk] / vs[b, hk].max())[np.arange(Sk) // 128].astype(np.float64)
            S = scale * (qd[b, :, h] @ kd[b, :, hk].T)
            va = np.abs(vd[b, :, hk])
            for i in range(Sq):
                vis = (np.arange(Sk) <= i + Sk - Sq) if causal else np.ones(Sk, bool)
                tol[b, i, h] = fp8_row_bound(S[i], vis, va, r)
    return tol


def check_fp8(o, lse, o_ref, lse_ref, tol, what):
    assert not np.isnan(o).any() and not np.isnan(lse).any(), f"{what}: NaN"
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ninf), f"{what}: -inf pattern differs"
    err = np.abs(o - o_ref)
    worst = float((err / tol).max()) if err.size else 0.0
    lerr = float(np.abs(lse[~ninf] - lse_ref[~ninf]).max()) if (~ninf).any() else 0.0
    say(f"  {what}: max|dO| = {err.max():.3e}  worst |dO|/bound = {worst:.3f}  "
        f"max|dLSE| = {lerr:.3e}")
    assert worst <= 1.0, f"{what}: O error over the bound ({worst:.3f})"
    assert lerr <= LSE_TOL, f"{what}: LSE error {lerr}"


CASES = [
    # B, Sq, Sk, Hq, Hkv, d, causal, rotate Q and K
    (1, 300, 300, 2, 1, 128, True, False),
    (2, 260, 190, 4, 2, 64, False, False),
    (1, 200, 517, 4, 1, 128, True, True),
    (1, 300, 77, 2, 2, 64, True, False),     # the first rows see no key
    (1, 1, 1000, 4, 2, 128, False, False),
    (2, 129, 129, 2, 2, 128, False, True),
    (1, 700, 700, 2, 1, 64, True, False),
    # more than 64 key scale blocks: the kernel holds the block scales 64 at a time
    (1, 130, 8500, 2, 1, 128, True, False),
    (1, 64, 16500, 2, 2, 64, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_Sq%d_Sk%d_Hq%d_Hkv%d_d%d_%s%s" % (
    *c[:6], "causal" if c[6] else "full", "_rot" if c[7] else ""))
def test_fp8_attention(ff, oracle, case):
    import torch
    B, Sq, Sk, Hq, Hkv, d, causal, rotate = case
    say(f"fp8 case {case}")
    seed = 1200 + Sq + Sk
    q = block_scaled_bf16(seed, 0, (B, Sq, Hq, d), [1.0, 2.0])
    k = block_scaled_bf16(seed, 1, (B, Sk, Hkv, d), [1.0, 0.5, 3.0])
    v = block_scaled_bf16(seed, 2, (B, Sk, Hkv, d), [1.0, 4.0, 0.25])   # V scales differ
    q8, qs = quantize_both(ff, oracle, q, rotate)
    k8, ks = quantize_both(ff, oracle, k, rotate)
    v8, vs = quantize_both(ff, oracle, v, False)
    scale = synth.f32(1 / math.sqrt(d))
    o, lse = ff.forward_fp8(dev_u8(q8), dev_u8(k8), dev_u8(v8), dev_f32(qs), dev_f32(ks),
                            dev_f32(vs), causal, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref, o_abs, inv_l = oracle.fwd_fp8(q8, k8, v8, qs, ks, vs, causal, scale)
    qd, kd, vd = (oracle.dequantize_fp8(c, x) for c, x in ((q8, qs), (k8, ks), (v8, vs)))
    tol = fp8_bound(qd, kd, vd, vs, causal, scale)
    check_fp8(host(o), host(lse), o_ref, lse_ref, tol, str(case))


def test_fp8_full_size_every_tile(ff, oracle):
    # causal_prefill's tensors quantized on the GPU; one seeded row of every (batch, head,
    # 128-row query tile) against the oracle on the dequantized tensors (the FP8
    # attention's definition)
    import torch
    w = synth.WORKLOADS["causal_prefill"]
    say(f"full-size fp8 on causal_prefill: {w}")
    q, k, v = synth.make_qkv(w)
    q8, qs = ff.quantize_fp8(to_dev(q))
    k8, ks = ff.quantize_fp8(to_dev(k))
    v8, vs = ff.quantize_fp8(to_dev(v))
    o_d, lse_d = ff.forward_fp8(q8, k8, v8, qs, ks, vs, True, w["scale"])
    torch.cuda.synchronize()
    assert torch.isfinite(o_d).all().item() and torch.isfinite(lse_d).all().item()
    q8, k8, v8 = (x.cpu().numpy() for x in (q8, k8, v8))
    qs, ks, vs = (x.cpu().numpy() for x in (qs, ks, vs))
    qd, kd, vd = (oracle.dequantize_fp8(c, s) for c, s in ((q8, qs), (k8, ks), (v8, vs)))
    rows = tile_edge_rows(w["B"], w["Sq"], w["Hq"], seed=41, per_tile=1)
    say(f"  comparing {len(rows)} rows (one in every query tile)")
    o_ref, lse_ref = oracle.rows(qd, kd, vd, True, w["scale"], rows)
    idx = torch.tensor(rows, dtype=torch.long)
    o_s = host(o_d[idx[:, 0], idx[:, 2], idx[:, 1]])
    lse_s = host(lse_d[idx[:, 0], idx[:, 1], idx[:, 2]])
    tol = np.empty_like(o_ref)
    Sk = w["Sk"]
    for n_, (b, h, i) in enumerate(rows):
        r = (vs[b, h] / vs[b, h].max())[np.arange(Sk) // 128].astype(np.float64)
        s_row = w["scale"] * (kd[b, :, h] @ qd[b, i, h])
        tol[n_] = fp8_row_bound(s_row, np.arange(Sk) <= i, np.abs(vd[b, :, h]), r)
    check_fp8(o_s, lse_s, o_ref, lse_ref, tol, "causal_prefill fp8 (sampled)")


def test_fp8_close_to_bf16(ff, oracle):
    # How far the FP8 path lands from exact attention on the original bf16 inputs: the
    # quantization error of Q, K, V plus the rounding of P.  A loose property check (the
    # parity bar is the oracle on the same codes, above); printed for the record.
    import torch
    q, k, v = make_inputs(1, 512, 512, 4, 2, 128, seed=1300)
    scale = synth.f32(1 / math.sqrt(128))
    o_ref, _ = oracle.fwd(q, k, v, True, scale)
    errs = {}
    for rotate in (False, True):
        q8, qs = ff.quantize_fp8(to_dev(q), rotate=rotate)
        k8, ks = ff.quantize_fp8(to_dev(k), rotate=rotate)
        v8, vs = ff.quantize_fp8(to_dev(v))
        o, _ = ff.forward_fp8(q8, k8, v8, qs, ks, vs, True, scale)
        torch.cuda.synchronize()
        e = np.abs(host(o) - o_ref)
        errs[rotate] = (float(e.max()), float(e.mean()))
        say(f"  fp8 vs exact bf16-input attention, rotate={rotate}: max {e.max():.3e}, "
            f"mean {e.mean():.3e}")
        assert e.mean() < 2e-2 and e.max() < 0.25


def test_fp8_is_deterministic(ff):
    import torch
    q, k, v = make_inputs(1, 400, 400, 4, 2, 128, seed=1301)
    q8, qs = ff.quantize_fp8(to_dev(q))
    k8, ks = ff.quantize_fp8(to_dev(k))
    v8, vs = ff.quantize_fp8(to_dev(v))
    r1 = ff.forward_fp8(q8, k8, v8, qs, ks, vs, True, 0.09)
    r2 = ff.forward_fp8(q8, k8, v8, qs, ks, vs, True, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])
