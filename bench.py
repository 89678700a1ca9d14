#!/usr/bin/env python3
"""Benchmark of the attention forward path on one MI355X.

A step is one call of the path over one batch of synthetic bf16 input already resident in
HBM.  The headline line is the causal-prefill workload (B=4, Hq=Hkv=16, Sq=Sk=4096,
d=128): ``value`` is its algorithmic TFLOP/s (4*d flops per visible query/key pair).  The
same JSON line carries the split-KV GQA decode workload (K/V bytes per second over
attn_fwd_splitkv + attn_splitkv_combine) and the other workloads, each with the
roofline fraction of its dominant kernel, and the fp64 CPU oracle timed on this host's
cores on a bounded sample of each configuration.

    python bench.py [--steps K] [--warmup W] [--workloads a,b] [--no-cpu-baseline]

Each workload runs W untimed warm-up steps, then exactly K steps between HIP events on
the launch stream.  Under sustained load the prefill kernels run at the board's power
limit, and the clock controller takes ~50 ms to settle: coming out of idle, the first
causal_prefill launches run at ~280 us, the power controller then pulls the clock down
(~345 us per launch 3-5 ms in) and lets it recover to ~270 us over the next ~50 ms.  With
a short warm-up (W = 5, K = 20) the timed steps fall in that dip.  The default W = 300
times the settled clock; the headline workload also reports a separately labelled
`steady_clock` figure, taken after its timed steps, whatever W is.

Progress goes to stderr; stdout gets exactly one JSON line.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

METRIC = "attn fwd TFLOP/s (bf16 causal prefill) + decode KV GB/s, % of roofline"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 (E4M3) MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE = "causal_prefill"
DECODE = "gqa_decode"
BACKWARD = "causal_prefill_bwd"   # attn_bwd over causal_prefill's inputs
# backward workloads and the forward workloads whose inputs (and options) they take
BWD_SOURCES = {BACKWARD: "causal_prefill", "sliding_window_gqa_bwd": "sliding_window_gqa"}
PROFILES = os.path.join(ROOT, "profiles")
# The device sources each kernel is compiled from (its template code and the shared
# building blocks); a change to any of them makes its committed counter summary stale.
KERNEL_SOURCES = {k: [os.path.join(ROOT, "io_aware_attention_amd", "csrc", f) for f in v]
                  for k, v in {"attn_fwd_prefill": ("device.h", "tiles.h", "worklist.h", "prefill.h"),
                               "attn_fwd_splitkv": ("device.h", "splitkv.h"),
                               "attn_bwd_dkdv": ("device.h", "worklist.h", "backward.h"),
                               "attn_fwd_fp8": ("device.h", "worklist.h", "fp8.h"),
                               "attn_kvcache_append": ("device.h", "append.h")}.items()}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(Sq, Sk, causal, wl=-1, wr=-1):
    """(query, key) pairs with j <= diag (causal) and diag - wl <= j <= diag + wr (window
    limits >= 0), diag = i + Sk - Sq."""
    if not causal and wl < 0 and wr < 0:
        return Sq * Sk
    total = 0
    for i in range(Sq):
        diag = i + Sk - Sq
        hi = Sk - 1
        if causal:
            hi = min(hi, diag)
        if wr >= 0:
            hi = min(hi, diag + wr)
        lo = max(0, diag - wl) if wl >= 0 else 0
        total += max(0, hi - lo + 1)
    return total


def window_of(w):
    return w.get("window_left", -1), w.get("window_right", -1)


def prefill_flops(w):
    return 4 * w["d"] * visible_pairs(w["Sq"], w["Sk"], w["causal"], *window_of(w)) * \
        w["B"] * w["Hq"]


def decode_bytes(w):
    kv = 2 * w["B"] * w["Sk"] * w["Hkv"] * w["d"] * 2
    q = w["B"] * w["Sq"] * w["Hq"] * w["d"] * 2
    o = w["B"] * w["Sq"] * w["Hq"] * w["d"] * 4
    lse = w["B"] * w["Hq"] * w["Sq"] * 4
    return kv, q, o, lse


def sources_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter summary
    profiles/<kernel>_<workload>_traffic.txt, or None when the summary is missing or the
    kernel sources changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    if kernel not in KERNEL_SOURCES or kv.get("kernel_sources_sha256") != sources_digest(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events on the stream the kernels are launched on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record(self.stream)

    def stop_ms(self):
        self.b.record(self.stream)
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def to_dev(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


# The clock settles after ~50 ms of sustained load (the power controller first lowers it
# below its steady value).  The steady-clock figure reported beside the headline is taken
# after the timed steps, so it never changes `value`.
STEADY_SETTLE, STEADY_STEPS = 300, 100


def run_prefill(torch, ff, name, steps, warmup, steady=False):
    w = synth.WORKLOADS[name]
    q, k, v = synth.make_qkv(w)
    qd, kd, vd = (to_dev(torch, x) for x in (q, k, v))
    B, Sq, Sk, Hq, Hkv, d = (w[x] for x in ("B", "Sq", "Sk", "Hq", "Hkv", "d"))
    o = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    wl, wr = window_of(w)

    def step():
        if wl < 0 and wr < 0:
            ff.attn_fwd(qd, kd, vd, o, lse, B, Sq, Sk, Hq, Hkv, d, w["causal"], w["scale"],
                        stream)
        else:
            ff.attn_fwd_ex(qd, kd, vd, o, lse, B, Sq, Sk, Hq, Hkv, d, w["causal"], wl, wr, None,
                           0, 0.0, w["scale"], stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t = Timer(torch, stream)
    wall0 = time.perf_counter()
    t.start()
    for _ in range(steps):
        step()
    ms = t.stop_ms() / steps
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3 / steps
    assert torch.isfinite(o).all().item(), f"{name}: non-finite output"
    flops = prefill_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    res = {
        "workload": name, "metric": "TFLOP/s", "value": round(tflops, 2),
        "ms_per_step": round(ms, 4), "wall_ms_per_step": round(wall_ms, 4),
        "kernel": "attn_fwd_prefill", "algorithmic_flop_per_launch": flops,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4)},
    }
    log(f"[bench] {name}: {ms:.4f} ms/step, {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of dense bf16 peak)")
    if steady:
        for _ in range(STEADY_SETTLE):
            step()
        t.start()
        for _ in range(STEADY_STEPS):
            step()
        sms = t.stop_ms() / STEADY_STEPS
        torch.cuda.synchronize()
        stf = flops / (sms * 1e-3) / 1e12
        res["steady_clock"] = {
            "note": f"{STEADY_SETTLE} more untimed steps after the timed ones, then "
                    f"{STEADY_STEPS} timed: the rate once the clock has settled; not `value`",
            "ms_per_step": round(sms, 4), "value": round(stf, 2),
            "frac": round(stf / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench] {name} (steady clock, after {STEADY_SETTLE} more steps): {sms:.4f} ms/step, "
            f"{stf:.1f} TFLOP/s ({100 * stf / PEAK_BF16_TFLOPS:.1f}%)")
    return res, (q, k, v)


def run_fp8(torch, ff, name, steps, warmup):
    """attn_fwd_fp8 on the workload's tensors quantized by attn_quantize_fp8 (outside the
    timed region; its own time is reported beside).  Flops as for the bf16 forward."""
    w = synth.WORKLOADS[name]
    q, k, v = synth.make_qkv(w)
    qd, kd, vd = (to_dev(torch, x) for x in (q, k, v))
    del q, k, v
    B, Sq, Sk, Hq, Hkv, d = (w[x] for x in ("B", "Sq", "Sk", "Hq", "Hkv", "d"))
    stream = torch.cuda.current_stream()
    q8, qs = ff.quantize_fp8(qd, stream=stream)
    k8, ks = ff.quantize_fp8(kd, stream=stream)
    v8, vs = ff.quantize_fp8(vd, stream=stream)
    o = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda:0")

    def step():
        ff.attn_fwd_fp8(q8, k8, v8, qs, ks, vs, o, lse, B, Sq, Sk, Hq, Hkv, d, w["causal"],
                        w["scale"], stream)

    def quant():
        ff.attn_quantize_fp8(qd, q8, qs, B, Sq, Hq, d, 0, stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t = Timer(torch, stream)
    t.start()
    for _ in range(steps):
        step()
    ms = t.stop_ms() / steps
    t.start()
    for _ in range(steps):
        quant()
    q_ms = t.stop_ms() / steps
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item(), f"{name}: non-finite output"
    flops = prefill_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    qbytes = B * Sq * Hq * d * 3   # bf16 read, fp8 written
    log(f"[bench] {name}: {ms:.4f} ms/step, {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_FP8_TFLOPS:.1f}% of dense fp8 peak); quantizing Q takes "
        f"{q_ms * 1e3:.1f} us ({qbytes / (q_ms * 1e-3) / 1e9:.0f} GB/s)")
    return {"workload": name, "metric": "TFLOP/s", "value": round(tflops, 2),
            "ms_per_step": round(ms, 4), "kernel": "attn_fwd_fp8", "dtype": "fp8 e4m3",
            "algorithmic_flop_per_launch": flops,
            "quantize_q_ms": round(q_ms, 4),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP8_TFLOPS, 4)}}


def run_varlen(torch, ff, name, steps, warmup):
    """attn_fwd_varlen over a packed batch: the flops are those of each sequence on its own."""
    w = synth.WORKLOADS[name]
    q, k, v, lens = synth.make_varlen_qkv(w)
    cu = torch.from_numpy(synth.prefix_sums(lens)).to("cuda:0")
    qd, kd, vd = (to_dev(torch, x) for x in (q, k, v))
    del q, k, v
    T, Hq, Hkv, d = w["total"], w["Hq"], w["Hkv"], w["d"]
    o = torch.empty((T, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def step():
        ff.attn_fwd_varlen(qd, kd, vd, o, lse, cu, cu, len(lens), max(lens), T, T, Hq, Hkv, d,
                           w["causal"], w["scale"], stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t = Timer(torch, stream)
    t.start()
    for _ in range(steps):
        step()
    ms = t.stop_ms() / steps
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item(), f"{name}: non-finite output"
    flops = sum(4 * d * visible_pairs(n, n, w["causal"]) * Hq for n in lens)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {name}: {len(lens)} sequences, {ms:.4f} ms/step, {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of dense bf16 peak)")
    return {"workload": name, "metric": "TFLOP/s", "value": round(tflops, 2),
            "ms_per_step": round(ms, 4), "kernel": "attn_fwd_prefill",
            "sequence_lengths": lens, "algorithmic_flop_per_launch": flops,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}}


def run_backward(torch, ff, name, steps, warmup):
    """The backward over a forward workload's inputs (causal_prefill, or sliding_window_gqa
    through attn_bwd_ex with its window): dO is tensor 3 of the workload's seed, O and LSE
    come from the forward with the same options.  A step is the two backward kernels (dQ,
    which also computes each row's D and base-2 LSE, then dK/dV)."""
    w = synth.WORKLOADS[BWD_SOURCES[name]]
    q, k, v = synth.make_qkv(w)
    dout = synth.normal_bf16(w["seed"], 3, q.shape)
    qd, kd, vd, dod = (to_dev(torch, x) for x in (q, k, v, dout))
    del q, k, v, dout
    B, Sq, Sk, Hq, Hkv, d = (w[x] for x in ("B", "Sq", "Sk", "Hq", "Hkv", "d"))
    win = window_of(w)
    o, lse = ff.forward(qd, kd, vd, w["causal"], w["scale"], window=win)
    dq = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device="cuda:0")
    dk = torch.empty((B, Sk, Hkv, d), dtype=torch.float32, device="cuda:0")
    dv = torch.empty((B, Sk, Hkv, d), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(ff.attn_bwd_workspace_floats(B, Sq, Hq), dtype=torch.float32,
                     device="cuda:0")
    stream = torch.cuda.current_stream()

    def step():
        if win == (-1, -1):
            ff.attn_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, ws, B, Sq, Sk, Hq, Hkv, d,
                        w["causal"], w["scale"], stream)
        else:
            ff.attn_bwd_ex(qd, kd, vd, o, lse, dod, dq, dk, dv, ws, B, Sq, Sk, Hq, Hkv, d,
                           w["causal"], win[0], win[1], None, 0, 0.0, w["scale"], stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t = Timer(torch, stream)
    t.start()
    for _ in range(steps):
        step()
    ms = t.stop_ms() / steps
    torch.cuda.synchronize()
    assert all(torch.isfinite(x).all().item() for x in (dq, dk, dv)), "non-finite gradient"
    flops = 2.5 * prefill_flops(w)   # 10*d per visible pair: S, dP, dV, dQ, dK
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {name}: {ms:.4f} ms/step, {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of dense bf16 peak)")
    return {"workload": name, "metric": "TFLOP/s", "value": round(tflops, 2),
            "ms_per_step": round(ms, 4), "kernel": "attn_bwd_dkdv",
            "kernels": ["attn_bwd_dq", "attn_bwd_dkdv"],
            "algorithmic_flop_per_launch": flops,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}}


def run_decode(torch, ff, name, steps, warmup):
    w = synth.WORKLOADS[name]
    q, k, v = synth.make_qkv(w)
    qd, kd, vd = (to_dev(torch, x) for x in (q, k, v))
    del k, v
    B, Sq, Sk, Hq, Hkv, d = (w[x] for x in ("B", "Sq", "Sk", "Hq", "Hkv", "d"))
    S = ff.attn_splitkv_num_splits(B, Sq, Sk, Hq, Hkv, d)
    page = w.get("page")
    if page:
        # the same keys and values moved into blocks of `page` positions in a random order
        mb = Sk // page
        table = np.random.default_rng(w["seed"]).permutation(B * mb).astype(np.int32)
        tb = torch.from_numpy(table).long().to("cuda:0")
        kc = torch.empty((B * mb, page, Hkv, d), dtype=torch.bfloat16, device="cuda:0")
        vc = torch.empty_like(kc)
        kc[tb] = kd.view(B * mb, page, Hkv, d)
        vc[tb] = vd.view(B * mb, page, Hkv, d)
        kd, vd = kc, vc
        table_d = torch.from_numpy(table.reshape(B, mb)).to("cuda:0")
        seqlens = torch.full((B,), Sk, dtype=torch.int32, device="cuda:0")
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    o = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda:0")
    oa = torch.empty((S, B, Hq, Sq, d), dtype=torch.float32, device="cuda:0")
    la = torch.empty((S, B, Hq, Sq), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]

    def split():
        if page:
            ff.attn_fwd_kvcache(qd, kd, vd, seqlens, None, table_d, oa if S > 1 else None,
                                la if S > 1 else None, o, lse, B, Sq, Hq, Hkv, d, B * mb, page,
                                mb, 0, w["causal"], w["scale"], S, stream)
        elif S == 1:
            ff.attn_fwd_splitkv(qd, kd, vd, None, None, o, lse, B, Sq, Sk, Hq, Hkv, d,
                                w["causal"], w["scale"], 1, stream)
        else:
            ff.attn_fwd_splitkv(qd, kd, vd, oa, la, None, None, B, Sq, Sk, Hq, Hkv, d,
                                w["causal"], w["scale"], S, stream)

    def step(i=None):
        if i is not None:
            ev[i][0].record(stream)
        split()
        if i is not None:
            ev[i][1].record(stream)
        if S > 1:
            ff.attn_splitkv_combine(oa, la, o, lse, B, Sq, Hq, d, S, stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the step: split kernel and combine, back to back, nothing else in the timed region
    t = Timer(torch, stream)
    t.start()
    for _ in range(steps):
        step()
    ms = t.stop_ms() / steps
    torch.cuda.synchronize()
    # the split kernel's own time (the roofline's launch duration): a second pass with an
    # event pair around each split launch
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    split_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    assert torch.isfinite(o).all().item(), f"{name}: non-finite output"
    kvb, qb, ob, lb = decode_bytes(w)
    step_gbs = (kvb + qb + ob + lb) / (ms * 1e-3) / 1e9
    kern_bytes = kvb + qb
    kern_gbs = kern_bytes / (split_ms * 1e-3) / 1e9
    res = {
        "workload": name, "metric": "GB/s", "value": round(step_gbs, 1),
        "ms_per_step": round(ms, 4), "num_splits": S,
        "kernel": "attn_fwd_splitkv", "kernel_ms": round(split_ms, 4),
        "kv_layout": f"paged, {page}-position blocks" if page else "dense",
        "algorithmic_bytes_per_step": kvb + qb + ob + lb,
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(kern_gbs / PEAK_HBM_GBS, 4),
                     "traffic": None},
    }
    log(f"[bench] {name}: {ms:.4f} ms/step (split-KV kernel {split_ms:.4f} ms, S={S}), "
        f"{step_gbs:.0f} GB/s step, kernel {kern_gbs:.0f} GB/s "
        f"({100 * kern_gbs / PEAK_HBM_GBS:.1f}% of HBM peak)")
    return res


def omp_threads():
    try:
        return int(ctypes.CDLL("libgomp.so.1").omp_get_max_threads())
    except OSError:
        return os.cpu_count()


def host_description():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "omp_max_threads": omp_threads(), "cpu_model": model}


# The workloads the oracle is timed on: the five configurations of the metric (the ragged
# one run non-causal and causal).
CPU_CONFIGS = ("tiny_mha", "causal_prefill", "ragged_noncausal", "ragged_causal", DECODE,
               "long_causal_gqa")


def cpu_oracle(name, seconds, inputs=None):
    """The fp64 oracle, as it stands, on a bounded sample of rows of workload `name`,
    sized from a pilot of 64 rows to take about `seconds`.  Prefill workloads report
    algorithmic TFLOP/s (4 d per visible pair of the sampled rows), the decode workload
    algorithmic key/value GB/s (its rows' share of the step's bytes)."""
    import oracle
    w = synth.WORKLOADS[name]
    q, k, v = inputs if inputs is not None else synth.make_qkv(w)
    orc = oracle.get()
    B, Sq, Sk, Hq, d = (w[x] for x in ("B", "Sq", "Sk", "Hq", "d"))
    n_all = B * Hq * Sq

    def rows_for(n):
        idx = np.linspace(0, n_all - 1, n).astype(np.int64)
        return [(int(r // (Hq * Sq)), int((r // Sq) % Hq), int(r % Sq)) for r in idx]

    def timed(rows):
        t0 = time.perf_counter()
        orc.rows(q, k, v, w["causal"], w["scale"], rows)
        return time.perf_counter() - t0

    pilot = rows_for(min(64, n_all))
    per_row = timed(pilot) / len(pilot)
    n = int(max(min(64, n_all), min(n_all, seconds / max(per_row, 1e-9))))
    rows = rows_for(n)
    secs = timed(rows)
    sample = (f"{n} of the {n_all} query rows of {name}, evenly spaced over (batch, head, "
              f"position); {secs:.2f} s wall")
    if name == DECODE:
        kvb, qb, ob, lb = decode_bytes(w)
        gbs = (kvb + qb + ob + lb) * (n / n_all) / secs / 1e9
        return {"value": round(gbs, 4), "unit": "GB/s", "seconds": round(secs, 3),
                "rows": n, "sample": sample + "; algorithmic bytes of the sampled share"}
    vis = sum(max(0, min(Sk, i + Sk - Sq + 1)) if w["causal"] else Sk for _, _, i in rows)
    tf = 4 * d * vis / secs / 1e12
    return {"value": round(tf, 6), "unit": "TFLOP/s", "seconds": round(secs, 3), "rows": n,
            "sample": sample + "; algorithmic flops of their visible keys"}


def run_append(torch, ff, steps, warmup):
    """attn_kvcache_append alone: a 2048-position chunk per sequence appended to the paged
    cache of the paged_decode shape (B=8, Hkv=8, d=128, 256-position blocks, capacity 32768,
    blocks in a seeded random order), starting at position 15384 (mid-block).  HBM-bound:
    the new K and V rows are read once and written once."""
    B, Hkv, d, page, S_new, cap, start = 8, 8, 128, 256, 2048, 32768, 15384
    mb = cap // page
    g = torch.Generator(device="cuda:0").manual_seed(5)
    kn = torch.randn((B, S_new, Hkv, d), generator=g, device="cuda:0").to(torch.bfloat16)
    vn = torch.randn((B, S_new, Hkv, d), generator=g, device="cuda:0").to(torch.bfloat16)
    kc = torch.zeros((B * mb, page, Hkv, d), dtype=torch.bfloat16, device="cuda:0")
    vc = torch.zeros_like(kc)
    table = torch.from_numpy(np.random.default_rng(5).permutation(B * mb).astype(np.int32)
                             .reshape(B, mb)).to("cuda:0")
    seqlens = torch.full((B,), start, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def step():
        ff.attn_kvcache_append(kn, vn, kc, vc, seqlens, table, B, S_new, Hkv, d, B * mb, page, mb,
                               stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t = Timer(torch, stream)
    t.start()
    for _ in range(steps):
        step()
    ms = t.stop_ms() / steps
    torch.cuda.synchronize()
    # spot check: the first new row of batch 0 landed at its logical position
    blk, row = divmod(start, page)
    assert torch.equal(kc[int(table[0, blk])][row], kn[0, 0]), "append check failed"
    nbytes = 4 * B * S_new * Hkv * d * 2  # read k_new, v_new; write both into the cache
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] attn_kvcache_append: {ms * 1e3:.1f} us per launch, {gbs:.0f} GB/s "
        f"({100 * gbs / PEAK_HBM_GBS:.1f}% of HBM peak)")
    return {"kernel": "attn_kvcache_append", "workload": "B=8 Hkv=8 d=128, 2048 new positions "
            "per sequence into 256-position blocks", "us_per_launch": round(ms * 1e3, 2),
            "algorithmic_bytes_per_launch": nbytes, "GB/s": round(gbs, 1),
            "frac": round(gbs / PEAK_HBM_GBS, 4), "steps": steps, "warmup": warmup}


def cpu_baseline(headline_inputs, seconds):
    """The oracle on every configuration (`seconds` split evenly), the headline's entry
    first-class in the JSON line, the host it ran on described."""
    per = {}
    for name in CPU_CONFIGS:
        inputs = headline_inputs if name == HEADLINE else None
        per[name] = cpu_oracle(name, seconds / len(CPU_CONFIGS), inputs)
        log(f"[bench] cpu oracle {name}: {per[name]['rows']} rows in {per[name]['seconds']:.1f} s"
            f" = {per[name]['value']} {per[name]['unit']}")
    head = per[HEADLINE]
    host = host_description()
    log(f"[bench] cpu oracle host: {host}")
    return {"value": head["value"], "unit": head["unit"], "cores": host["omp_max_threads"],
            "kind": "oracle", "sample": head["sample"], "host": host, "per_config": per}


def describe(name):
    """The JSON line's config object for workload `name`."""
    w = synth.WORKLOADS.get(name, synth.WORKLOADS[HEADLINE])
    kind = "causal" if w["causal"] else "non-causal"
    if "total" in w:
        return {"workload": f"{name}: {w['total']} tokens packed in sequences of length "
                            f"uniform on [1, {w['max_len']}], Hq={w['Hq']} Hkv={w['Hkv']} "
                            f"d={w['d']} {kind}",
                "total_tokens": w["total"], "Hq": w["Hq"], "Hkv": w["Hkv"], "d": w["d"],
                "causal": w["causal"], "parallelism": "none (1 GPU)"}
    label = name if name in synth.WORKLOADS else f"{name} (on {HEADLINE})"
    wl, wr = window_of(w)
    if wl >= 0 or wr >= 0:
        kind += f" window ({wl}, {wr})"
    return {"workload": f"{label}: B={w['B']} Hq={w['Hq']} Hkv={w['Hkv']} Sq={w['Sq']} "
                        f"Sk={w['Sk']} d={w['d']} {kind}",
            "B": w["B"], "Sq": w["Sq"], "Sk": w["Sk"], "Hq": w["Hq"], "Hkv": w["Hkv"],
            "d": w["d"], "causal": w["causal"], "parallelism": "none (1 GPU)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workloads", default="all",
                    help="comma list of " + ",".join(list(synth.WORKLOADS) + list(BWD_SOURCES)) + " (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=24.0,
                    help="oracle time budget, split over the configurations")
    ap.add_argument("--append", action="store_true",
                    help="time attn_kvcache_append alone (a measurement mode, like --copy-mib)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from io_aware_attention_amd import flashfwd as ff
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ff.load()

    if args.copy_mib:
        n = args.copy_mib << 20
        x = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        y = torch.empty_like(x)
        for _ in range(args.steps):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": args.steps}), flush=True)
        return

    if args.append:
        print(json.dumps(run_append(torch, ff, args.steps, args.warmup)), flush=True)
        return

    names = list(synth.WORKLOADS) + list(BWD_SOURCES) if args.workloads == "all" else \
        args.workloads.split(",")
    results = {}
    headline_inputs = None
    for name in names:
        log(f"[bench] running {name} ...")
        if name in (DECODE, "paged_decode"):
            results[name] = run_decode(torch, ff, name, args.steps, args.warmup)
        elif name in BWD_SOURCES:
            results[name] = run_backward(torch, ff, name, args.steps, args.warmup)
        elif "total" in synth.WORKLOADS[name]:
            results[name] = run_varlen(torch, ff, name, args.steps, args.warmup)
        elif synth.WORKLOADS[name].get("fp8"):
            results[name] = run_fp8(torch, ff, name, args.steps, args.warmup)
        else:
            results[name], inputs = run_prefill(torch, ff, name, args.steps, args.warmup,
                                                steady=(name == HEADLINE))
            if name == HEADLINE:
                headline_inputs = inputs
        torch.cuda.empty_cache()

    main_name = HEADLINE if HEADLINE in results else names[0]
    main = results[main_name]
    for name, res in results.items():
        res["roofline"]["traffic"] = measured_traffic(res["kernel"], name)
    cpu = None
    if not args.no_cpu_baseline and headline_inputs is not None:
        cpu = cpu_baseline(headline_inputs, args.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": main["value"],
        "unit": main["metric"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": describe(main_name),
        "roofline": main["roofline"],
        "cpu_baseline": cpu,
        "steady_clock": main.get("steady_clock"),
        "workloads": {k: v for k, v in results.items()},
    }
    if DECODE in results:
        line["decode_kv_gbs"] = results[DECODE]["value"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
