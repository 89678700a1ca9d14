"""Shared helpers for the GPU parity tests: device transfer, the error bar, row sampling."""
import sys

import numpy as np

import synth

# Error bar for fp32-accumulated bf16 attention against the fp64 oracle.
O_TOL = 2e-2     # max-abs on O
LSE_TOL = 1e-3   # max-abs on LSE


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits):
    """bf16 bit patterns (numpy uint16) -> contiguous torch bf16 tensor on cuda:0."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda:0")


def host(t):
    return t.detach().cpu().double().numpy()


def check_outputs(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    """Element-wise comparison at the error bar; -inf must match -inf, no NaN anywhere."""
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in LSE"
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), ninf), f"{what}: -inf pattern differs"
    fin = ~ninf
    lerr = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    oerr = float(np.abs(o_gpu - o_ref).max()) if o_ref.size else 0.0
    say(f"  {what}: max|dO| = {oerr:.3e}  max|dLSE| = {lerr:.3e}")
    assert oerr <= O_TOL, f"{what}: O error {oerr}"
    assert lerr <= LSE_TOL, f"{what}: LSE error {lerr}"
    return oerr, lerr


def sample_rows(B, Sq, Hq, n, seed, boundaries=(127, 128, 255, 256)):
    """(b, h, i) triples: first and last rows, tile boundaries, then random rows."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0, 0), (B - 1, Hq - 1, Sq - 1), (0, Hq - 1, Sq - 1), (B - 1, 0, 0)}
    for i in boundaries:
        if i < Sq:
            rows.add((int(rng.integers(B)), int(rng.integers(Hq)), i))
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(Sq))))
    return sorted(rows)


def tile_edge_rows(B, Sq, Hq, seed, bm=128, per_tile=2):
    """(b, h, i) triples covering every (batch, head, bm-row query tile): its first and
    last row (per_tile=2), or one seeded row inside it (per_tile=1).  bm is the prefill
    kernel's query-tile height, so every workgroup of a launch is checked."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(B):
        for h in range(Hq):
            for m0 in range(0, Sq, bm):
                last = min(m0 + bm, Sq) - 1
                if per_tile == 2:
                    rows.append((b, h, m0))
                    if last != m0:
                        rows.append((b, h, last))
                else:
                    rows.append((b, h, int(rng.integers(m0, last + 1))))
    return rows


def make_inputs(B, Sq, Sk, Hq, Hkv, d, seed, mult=1.0):
    q = synth.normal_bf16(seed, 0, (B, Sq, Hq, d), mult)
    k = synth.normal_bf16(seed, 1, (B, Sk, Hkv, d), mult)
    v = synth.normal_bf16(seed, 2, (B, Sk, Hkv, d), mult)
    return q, k, v
