"""attn_fwd_kvcache (split-KV attention against a paged or contiguous key/value cache, with
left padding) and attn_kvcache_append against the fp64 oracle.  Cache slots that no batch
owns are filled with NaN, so a read outside a batch's keys shows up in O.  The append is
byte work and is compared bit for bit.  Calls go through the C ABI."""
import math

import numpy as np
import pytest

import synth
from gpu_helpers import check_outputs, host, say, to_dev

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module")
def ff():
    import torch
    from io_aware_attention_amd import flashfwd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    flashfwd.load()
    return flashfwd


def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


def paged_cache(B, Hkv, d, page, max_blocks, spare, seed):
    """Caches [num_blocks, page, Hkv, d] with num_blocks = B * max_blocks + spare and a
    block table that deals the blocks to the batches in a seeded random order."""
    nb = B * max_blocks + spare
    kc = synth.normal_bf16(seed, 1, (nb, page, Hkv, d))
    vc = synth.normal_bf16(seed, 2, (nb, page, Hkv, d))
    perm = np.random.default_rng(seed).permutation(nb)[:B * max_blocks]
    return kc, vc, perm.reshape(B, max_blocks).astype(np.int32)


def poison_unowned(kc, vc, table, seqlens, leftpad):
    """NaN in every cache row outside positions leftpad[b] .. seqlens[b]-1 of some batch."""
    page = kc.shape[1]
    owned = np.zeros(kc.shape[:2], dtype=bool)
    for b in range(table.shape[0]):
        lp = 0 if leftpad is None else int(leftpad[b])
        pos = np.arange(lp, int(seqlens[b]))
        owned[table[b, pos // page], pos % page] = True
    kc, vc = kc.copy(), vc.copy()
    kc[~owned] = NAN_BF16
    vc[~owned] = NAN_BF16
    return kc, vc


def run_kvcache(ff, q, kc, vc, seqlens, causal, scale, table=None, leftpad=None, new_keys=0,
                num_splits=1):
    import torch
    o, lse = ff.forward_kvcache(to_dev(q), to_dev(kc), to_dev(vc), dev_i32(seqlens), causal,
                                scale, block_table=None if table is None else dev_i32(table),
                                cache_leftpad=None if leftpad is None else dev_i32(leftpad),
                                new_keys=new_keys, num_splits=num_splits)
    torch.cuda.synchronize()
    return host(o), host(lse)


CASES = [
    # B, Sq, Hq, Hkv, d, page, max_blocks, seqlens, leftpad, causal
    (3, 1, 8, 2, 128, 64, 8, [300, 1, 512], None, False),
    (3, 1, 8, 2, 128, 64, 8, [300, 1, 512], [5, 0, 100], False),
    (3, 4, 8, 2, 128, 64, 8, [300, 7, 512], [5, 0, 33], True),     # a few queries, causal
    (2, 4, 8, 8, 64, 32, 20, [640, 130], [0, 127], True),
    (2, 16, 4, 1, 64, 128, 3, [384, 200], [50, 190], True),        # queries that see nothing
    (4, 1, 32, 8, 128, 256, 4, [0, 1000, 1024, 17], [0, 999, 0, 17], False),  # empty batches
    (1, 3, 4, 2, 128, 96, 5, [479], [1], False),                    # page 96
]


def ids(c):
    return "B%d_Sq%d_Hq%d_Hkv%d_d%d_page%d_mb%d_len%s_lp%s_%s" % (
        *c[:7], "-".join(map(str, c[7])), "none" if c[8] is None else "-".join(map(str, c[8])),
        "causal" if c[9] else "full")


@pytest.mark.parametrize("num_splits", [1, 3])
@pytest.mark.parametrize("case", CASES, ids=ids)
def test_paged_matches_oracle(ff, oracle, case, num_splits):
    B, Sq, Hq, Hkv, d, page, mb, seqlens, leftpad, causal = case
    say(f"kvcache {ids(case)} splits={num_splits}")
    kc, vc, table = paged_cache(B, Hkv, d, page, mb, 3, seed=61 + page)
    kc, vc = poison_unowned(kc, vc, table, seqlens, leftpad)
    q = synth.normal_bf16(61 + page, 0, (B, Sq, Hq, d))
    scale = synth.f32(1 / math.sqrt(d))
    o, lse = run_kvcache(ff, q, kc, vc, seqlens, causal, scale, table, leftpad,
                         num_splits=num_splits)
    o_ref, lse_ref = oracle.kvcache(q, kc, vc, table, seqlens, leftpad, causal, scale)
    check_outputs(o, lse, o_ref, lse_ref, ids(case))


@pytest.mark.parametrize("num_splits", [1, 4])
def test_contiguous_cache_matches_oracle(ff, oracle, num_splits):
    B, Sq, Hq, Hkv, d, cap = 3, 2, 8, 4, 128, 700
    seqlens, leftpad = [700, 333, 2], [0, 30, 1]
    kc = synth.normal_bf16(62, 1, (B, cap, Hkv, d))
    vc = synth.normal_bf16(62, 2, (B, cap, Hkv, d))
    table = np.arange(B, dtype=np.int32)[:, None]   # the oracle's view: one block per batch
    kc, vc = poison_unowned(kc, vc, table, seqlens, leftpad)
    q = synth.normal_bf16(62, 0, (B, Sq, Hq, d))
    o, lse = run_kvcache(ff, q, kc, vc, seqlens, True, 0.09, None, leftpad,
                         num_splits=num_splits)
    o_ref, lse_ref = oracle.kvcache(q, kc, vc, table, seqlens, leftpad, True, 0.09)
    check_outputs(o, lse, o_ref, lse_ref, f"contiguous splits={num_splits}")


@pytest.mark.parametrize("paged", [True, False])
def test_append_then_attend(ff, oracle, paged):
    import torch
    B, S_new, Hq, Hkv, d = 3, 5, 8, 2, 64
    if paged:
        page, mb = 32, 6
        kc, vc, table = paged_cache(B, Hkv, d, page, mb, 2, seed=63)
    else:
        cap = 150
        kc = synth.normal_bf16(63, 1, (B, cap, Hkv, d))
        vc = synth.normal_bf16(63, 2, (B, cap, Hkv, d))
        table = np.arange(B, dtype=np.int32)[:, None]
    capacity = table.shape[1] * kc.shape[1]
    seqlens = np.array([0, 61, capacity - 2], dtype=np.int32)   # the last one overflows
    k_new = synth.normal_bf16(63, 3, (B, S_new, Hkv, d))
    v_new = synth.normal_bf16(63, 4, (B, S_new, Hkv, d))
    kd, vd = to_dev(kc), to_dev(vc)
    tbl = dev_i32(table) if paged else None
    sl = dev_i32(seqlens)
    ff.kvcache_append(to_dev(k_new), to_dev(v_new), kd, vd, sl, tbl)
    q = synth.normal_bf16(63, 0, (B, S_new, Hq, d))
    o, lse = ff.forward_kvcache(to_dev(q), kd, vd, sl, True, 0.125, block_table=tbl,
                                new_keys=S_new, num_splits=2)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.append(k_new, v_new, kc, vc, table, seqlens)
    got_k = kd.view(torch.int16).cpu().numpy().view(np.uint16)
    got_v = vd.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_k, k_ref) and np.array_equal(got_v, v_ref)
    ends = np.minimum(seqlens + S_new, capacity)
    o_ref, lse_ref = oracle.kvcache(q, k_ref, v_ref, table, ends, None, True, 0.125)
    check_outputs(host(o), host(lse), o_ref, lse_ref, f"append paged={paged}")


def test_full_size_paged_decode(ff, oracle):
    # gqa_decode's shape (B=8, 32768 keys, Hq=32, Hkv=8, d=128) in 256-position blocks dealt
    # in a random order.  With full caches the splits cut the keys where the dense split
    # kernel does, so the outputs must equal attn_fwd_splitkv's bit for bit; sampled rows
    # are checked against the oracle as well.
    import torch
    w = synth.WORKLOADS["gqa_decode"]
    B, Sk, Hq, Hkv, d = (w[x] for x in ("B", "Sk", "Hq", "Hkv", "d"))
    page = 256
    mb = Sk // page
    q, k, v = synth.make_qkv(w)
    perm = np.random.default_rng(64).permutation(B * mb).astype(np.int32)
    table = perm.reshape(B, mb)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    kc = torch.empty((B * mb, page, Hkv, d), dtype=torch.bfloat16, device="cuda:0")
    vc = torch.empty_like(kc)
    tb = torch.from_numpy(table).long().cuda()
    kc[tb.flatten()] = kd.view(B * mb, page, Hkv, d)
    vc[tb.flatten()] = vd.view(B * mb, page, Hkv, d)
    seqlens = dev_i32(np.full(B, Sk))
    S = ff.attn_splitkv_num_splits(B, 1, Sk, Hq, Hkv, d)
    o_p, l_p = ff.forward_kvcache(qd, kc, vc, seqlens, False, w["scale"], block_table=dev_i32(table),
                                  num_splits=S)
    o_d, l_d = ff.forward_splitkv(qd, kd, vd, False, w["scale"], num_splits=S)
    torch.cuda.synchronize()
    say(f"  paged vs dense split-KV, {S} splits: max|diff| = {(o_p - o_d).abs().max().item():.3e}")
    assert torch.equal(o_p, o_d) and torch.equal(l_p, l_d)
    rows = [(0, 0, 0), (B - 1, Hq - 1, 0), (3, 17, 0), (5, 8, 0)]
    o_ref, lse_ref = oracle.rows(q, k, v, False, w["scale"], rows)
    idx = torch.tensor(rows, dtype=torch.long)
    check_outputs(host(o_p[idx[:, 0], idx[:, 2], idx[:, 1]]),
                  host(l_p[idx[:, 0], idx[:, 1], idx[:, 2]]), o_ref, lse_ref, "paged gqa_decode")
