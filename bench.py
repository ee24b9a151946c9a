#!/usr/bin/env python3
"""Benchmark of the HLA2 hot path on one MI355X.

A step is one hla2_forward over the headline forward workload (decay_8k:
B=8, H=16, n=8192, d=64, dv=128, bf16, decay 0.99, chunk 64) with inputs
resident in HBM.  The same JSON line also carries the decode workload
(decode_256x32: 256 sequences x 32 heads, d = dv = 64, one hla2_decode_step
per step, fp32 state) because the metric names both.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  Timing uses HIP events on the stream the kernels are
launched on (torch's current stream), bracketed by device synchronisation.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_MFMA = 2.5e15      # dense bf16 MFMA, MI355X, FLOP/s
PEAK_HBM = 8.0e12            # HBM3E, B/s
METRIC = "masked HLA2 fwd tokens/s + % bf16 MFMA peak (d=64); decode tokens/s + % HBM BW"


def canonical_flops_per_head_token(d, dv, C, normalize):
    """Algorithmic work of the chunked forward per head-token: chunk summaries
    + scan combines + masked chunk outputs, every product counted as 2mnk at
    full chunk tiles of the requested chunk C (dv' = dv + 1 when normalised)."""
    dvp = dv + (1 if normalize else 0)
    return 4 * d * d + 6 * d * dvp + 6 * C * d + 4 * C * dvp + 2 * C * C + 6 * d * d * dvp / C


def output_kernel_flops_per_head_token(d, dv, C, normalize):
    """Algorithmic work of the chunk-output step alone (masked chunk-local
    block A, W and the carried-state terms Q S0, Q U0) per head-token, at full
    chunk tiles of the requested chunk C."""
    dvp = dv + (1 if normalize else 0)
    return 4 * C * d + 2 * C * C + 2 * d * d + 2 * C * dvp + 2 * d * dvp


def summary_kernel_flops_per_head_token(d, dv, C, normalize):
    """Algorithmic work of forming a chunk's summaries (S, C, m, G, h) per
    head-token, at full chunk tiles of the requested chunk C."""
    dvp = dv + (1 if normalize else 0)
    return 2 * d * d + 4 * d * dvp + 2 * C * d + 2 * C * dvp


def min_bytes_forward(w, esize):
    """q, k, v read once and out written once."""
    return w.B * w.H * w.n * (2 * w.d + 2 * w.dv) * esize


def min_bytes_backward(w, esize):
    """q, k, v, dout read once (out and the fp32 den too under the ratio), dq, dk, dv written once."""
    per = (2 * w.d + 2 * w.dv) * esize + (2 * w.d + w.dv) * esize
    if w.normalize:
        per += w.dv * esize + 4
    return w.B * w.H * w.n * per


def output_launch_tokens(w, plan):
    """Tokens per head that the chunk-output launch walks: every token under a
    plain plan; under a lead plan those after segment 0 (walked, with its
    outputs, in the launch before the scan)."""
    nseg, c0, _, lead = plan
    return max(w.n - c0 * 64, 0) if lead else w.n


# Lead plans at d <= 64 with at most this many summaries to fold fold them in the output launch's
# prologue instead of a scan launch (the library's rule).
MAX_PROLOGUE_FOLDS = 1


def prologue_folds(w, plan):
    """Summaries per head that the output launch folds in its workgroups' prologues: segment s of a
    lead plan without a scan launch folds s - 1 of them (none when the plan launches the scan)."""
    nseg, _, _, lead = plan
    if not (lead and w.dtype == "bf16" and w.d <= 64 and 2 < nseg <= 2 + MAX_PROLOGUE_FOLDS):
        return 0
    return (nseg - 2) * (nseg - 1) // 2


def output_kernel_bytes(w, esize, plan):
    """Algorithmic HBM bytes of one chunk-output launch: q, k, v of its tokens
    read once, their outputs written once, the incoming state (S0, U0, u0) of
    every segment after the first read once, and the summaries (S, C, U, m, u)
    folded in the prologue read once each."""
    state = (w.d * w.d + w.d * w.dv + w.d) * 4
    summary = (w.d * w.d + 2 * w.d * w.dv + 2 * w.d) * 4
    return w.B * w.H * output_launch_tokens(w, plan) * (2 * w.d + 2 * w.dv) * esize + \
        w.B * w.H * (plan[0] - 1) * state + w.B * w.H * prologue_folds(w, plan) * summary


def roofline(flops, nbytes, seconds):
    """The binding roofline of a kernel that does `flops` and moves `nbytes` in
    `seconds`: HBM when its arithmetic intensity is below the ridge
    (peak FLOP/s over peak B/s), else the bf16 MFMA peak."""
    hbm = nbytes / PEAK_HBM >= flops / PEAK_BF16_MFMA
    out = {"bound": "hbm" if hbm else "mfma"}
    if hbm:
        out.update(achieved=nbytes / seconds / 1e9, peak=PEAK_HBM / 1e9, unit="GB/s", frac=nbytes / seconds / PEAK_HBM)
    else:
        out.update(achieved=flops / seconds / 1e12, peak=PEAK_BF16_MFMA / 1e12, unit="TFLOP/s",
                   frac=flops / seconds / PEAK_BF16_MFMA)
    out["arithmetic_intensity"] = flops / nbytes
    out["ridge"] = PEAK_BF16_MFMA / PEAK_HBM
    return out


def decode_bytes_per_step(N, H, d, dv, esize=2):
    state = N * H * (d * d + 2 * d * dv + 2 * d) * 4
    return 2 * state + N * H * (2 * d + dv) * esize + N * H * dv * esize


def sources_digest():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "causal_prefix_scan_hla2_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(key):
    """HBM traffic per call measured with rocprofv3 counters (profiles/traffic.json),
    or None when the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(key)
    if not ent or ent.get("sources") != sources_digest():
        return None
    return ent.get("bytes_per_call")


# Untimed calls before each timed region run for at least this long (whatever --warmup says):
# after the host-side input generation the device idles and its clocks drop, and a few
# warm-up calls do not bring them back (5 warm-up and 20 timed forward calls read about 25%
# slower than steady clocks).  Set with --min-warm-ms.
MIN_WARM_S = 0.5


def warm(fn, warmup, torch, min_seconds=None):
    """`warmup` untimed calls, then more in batches of 10 until `min_seconds` of wall time
    have passed.  Returns the number of untimed calls made."""
    min_seconds = MIN_WARM_S if min_seconds is None else min_seconds
    t0 = time.perf_counter()
    calls = 0
    for _ in range(warmup):
        fn()
        calls += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(10):
            fn()
        calls += 10
        torch.cuda.synchronize()
    return calls


def load_counters(key):
    """SQ counter figures of one kernel (profiles/counters.json: MFMA busy, VALU busy, ...), or None
    when the kernel sources changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("sources") != sources_digest():
        return None
    return data.get(key)


def time_calls(fn, steps, warmup, torch):
    warm(fn, warmup, torch)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / 1e3 / steps, wall


def bench_forward(w, steps, warmup, torch, H, I):
    """Time `steps` forward calls back to back (plain hla2_forward: the step
    time and `value`), then `steps` calls of hla2_forward_timed, which records
    four HIP events between its kernels on the stream they run on: the average
    duration of every kernel.  The event records widen the gaps between the
    kernels (about 13 us per call at the decay workload), so they stay out of
    the step time."""
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in I.make_qkv(w))
    out = torch.empty_like(v)
    need = H.hla2_forward_workspace_bytes(w.B, w.H, w.n, w.d, w.dv, w.chunk)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(max(steps, 1))]
    for row in evs:      # create the underlying HIP events
        for e in row:
            e.record()
    it = [0]

    def fn():
        H.hla2_forward(q, k, v, out, decay=w.decay, normalize=w.normalize, chunk=w.chunk, workspace=ws)

    def fn_timed():
        row = evs[it[0] % len(evs)]
        it[0] += 1
        H.hla2_forward(q, k, v, out, decay=w.decay, normalize=w.normalize, chunk=w.chunk, workspace=ws,
                       events=row)

    warm_calls = warm(fn, warmup, torch)
    t, wall = time_calls(fn, steps, 0, torch)
    time_calls(fn_timed, steps, 0, torch)
    plan = H.hla2_forward_plan(w.B, w.H, w.n, w.d, w.dv, w.chunk)
    nseg = plan[0]
    # the launch before the scan: segment summaries, plus segment 0's outputs under a lead plan
    first = "lead" if plan[3] else "summary"
    phases = {first: 0.0, "scan": 0.0, "output": 0.0}
    for row in evs[:steps]:
        phases[first] += row[0].elapsed_time(row[1]) / 1e3
        phases["scan"] += row[1].elapsed_time(row[2]) / 1e3
        phases["output"] += row[2].elapsed_time(row[3]) / 1e3
    phases = {key: val / max(steps, 1) for key, val in phases.items()}
    esize = 4 if w.dtype == "f32" else 2
    flops = canonical_flops_per_head_token(w.d, w.dv, w.chunk, w.normalize) * w.head_tokens
    return {
        "seconds": t,
        "wall": wall,
        "warm_calls": warm_calls,
        "phases": phases,
        "plan": {"segments": nseg, "lead_chunks": plan[1], "seg_chunks": plan[2], "lead": plan[3]},
        "output_flops_per_call": output_kernel_flops_per_head_token(w.d, w.dv, w.chunk, w.normalize)
                                 * w.B * w.H * output_launch_tokens(w, plan)
                                 + w.B * w.H * prologue_folds(w, plan) * 2 * w.d * w.d * (w.dv + int(w.normalize)),
        "tokens_per_s": w.B * w.n / t,
        "head_tokens_per_s": w.head_tokens / t,
        "tflops": flops / t / 1e12,
        "mfma_frac": flops / t / PEAK_BF16_MFMA,
        "flops_per_call": flops,
        "min_bytes": min_bytes_forward(w, esize),
        "output_bytes_per_call": output_kernel_bytes(w, esize, plan),
        "segments": nseg,
    }


def bench_decode(dw, steps, warmup, torch, H, prefill_tokens):
    """Build every head's state from a random prefix with the chunk-parallel
    forward pass and its final-state export, then time single-token steps."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(dw.seed)
    L = H.hla2_state_floats(dw.d, dw.dv)
    state = torch.zeros(dw.N, dw.H, L, dtype=torch.float32, device=dev)
    s = 1.0 / math.sqrt(dw.d)
    out = torch.empty(dw.N, dw.H, dw.dv, dtype=torch.bfloat16, device=dev)
    if prefill_tokens > 0:
        shp = (dw.N, dw.H, prefill_tokens)
        pq = (torch.randn(*shp, dw.d, generator=g, device=dev) * s).to(torch.bfloat16)
        pk = (torch.randn(*shp, dw.d, generator=g, device=dev) * s).to(torch.bfloat16)
        pv = (torch.randn(*shp, dw.dv, generator=g, device=dev) * s).to(torch.bfloat16)
        po = torch.empty_like(pv)
        H.hla2_forward_state(pq, pk, pv, po, state, decay=dw.decay, normalize=dw.normalize, chunk=64)
        del pq, pk, pv, po
    nsteps = dw.steps
    qs = (torch.randn(nsteps, dw.N, dw.H, dw.d, generator=g, device=dev) * s).to(torch.bfloat16)
    ks = (torch.randn(nsteps, dw.N, dw.H, dw.d, generator=g, device=dev) * s).to(torch.bfloat16)
    vs = (torch.randn(nsteps, dw.N, dw.H, dw.dv, generator=g, device=dev) * s).to(torch.bfloat16)
    torch.cuda.synchronize()
    it = [0]

    def fn():
        i = it[0] % nsteps
        it[0] += 1
        H.hla2_decode_step(state, qs[i], ks[i], vs[i], out, decay=dw.decay, normalize=dw.normalize)

    t, wall = time_calls(fn, steps, warmup, torch)
    byts = decode_bytes_per_step(dw.N, dw.H, dw.d, dw.dv)
    return {
        "seconds": t,
        "wall": wall,
        "tokens_per_s": dw.N / t,
        "head_tokens_per_s": dw.N * dw.H / t,
        "gbps": byts / t / 1e9,
        "hbm_frac": byts / t / PEAK_HBM,
        "bytes_per_call": byts,
    }


def bench_backward(w, steps, warmup, torch, H, I):
    """Time `steps` backward calls (gradients w.r.t. q, k, v) on the workload,
    with the forward's out and den (from one forward call) and a random dout."""
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in I.make_qkv(w))
    g = torch.Generator(device=dev).manual_seed(w.seed + 7)
    dout = torch.randn(w.B, w.H, w.n, w.dv, generator=g, device=dev).to(q.dtype)
    out = den = None
    if w.normalize:
        out = torch.empty_like(v)
        den = torch.empty(w.B, w.H, w.n, dtype=torch.float32, device=dev)
        H.hla2_forward(q, k, v, out, decay=w.decay, normalize=True, chunk=w.chunk, den_out=den)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    code = H.HLA2_BF16 if q.dtype == torch.bfloat16 else H.HLA2_F32
    ws = torch.empty(H.hla2_backward_workspace_bytes(w.B, w.H, w.n, w.d, w.dv, w.normalize, code),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def fn():
        H.hla2_backward(q, k, v, dout, gq, gk, gv, decay=w.decay, normalize=w.normalize, out=out, den=den,
                        workspace=ws)

    t, wall = time_calls(fn, steps, warmup, torch)
    return {"seconds": t, "wall": wall, "tokens_per_s": w.B * w.n / t, "head_tokens_per_s": w.B * w.H * w.n / t,
            "workspace_bytes": ws.numel()}


def ahla_flops_per_head_token(w):
    """AHLA chunk outputs per head-token at chunk C: Ad 2Cd, Y and O 2(2d dv' + 2C dv'), the P' and E'
    updates 4 d dv' (dv' = dv + 1 under the ratio)."""
    C, d, dv = w.chunk, w.d, w.dv + (1 if w.normalize else 0)
    return 2 * C * d + 8 * d * dv + 4 * C * dv


def ho3_flops_per_head_token(w):
    """Third-order chunk outputs per head-token at chunk C: Ad 2Cd, Z 2d^2 + 2Cd, Y 2d dv' + 2C dv',
    the masked Q Z^T 2Cd, O 2d dv' + 2C dv', the S, P', W' updates 2d^2 + 4d dv'."""
    C, d, dv = w.chunk, w.d, w.dv + (1 if w.normalize else 0)
    return 6 * C * d + 4 * d * d + 8 * d * dv + 4 * C * dv


def bench_variant(fn_name, w, steps, warmup, torch, H, I, flops_per_head_token):
    """Time `steps` calls of a variant's forward (AHLA or third order) on the workload's shape."""
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in I.make_qkv(w))
    out = torch.empty_like(v)
    code = H.HLA2_BF16 if q.dtype == torch.bfloat16 else H.HLA2_F32
    fwd = getattr(H, fn_name)
    ws = torch.empty(max(getattr(H, fn_name + "_workspace_bytes")(w.B, w.H, w.n, w.d, w.dv, code), 1),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def fn():
        fwd(q, k, v, out, decay=w.decay, normalize=w.normalize, workspace=ws)

    t, wall = time_calls(fn, steps, warmup, torch)
    fl = flops_per_head_token * w.B * w.H * w.n
    return {"workload": w.name + " shape", "ms_per_step": t * 1e3, "tokens_per_s": w.B * w.n / t,
            "tflops": fl / t / 1e12, "mfma_frac": fl / t / PEAK_BF16_MFMA, "flops_per_head_token": flops_per_head_token}


def cpu_single_thread(w, I):
    """The fp64 oracle (as it stands) on one host thread over every head of a (small) workload."""
    from oracle import oracle as O
    q, k, v = (x.double().numpy() for x in I.make_qkv(w))
    t0 = time.perf_counter()
    O.serial(q, k, v, w.decay, threads=1)
    dt = time.perf_counter() - t0
    return {"workload": w.name, "value": w.B * w.n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "all %d heads of %d tokens, fp64 serial recurrence on 1 thread, %.2f s wall"
                      % (w.B * w.H, w.n, dt)}


def cpu_baseline(w, heads_sample, I):
    """The fp64 oracle (as it stands) on a bounded sample of the workload's
    heads: the serial recurrence, threaded over heads."""
    from oracle import oracle as O
    q, k, v = I.make_qkv(w)
    q, k, v = (x.reshape(w.B * w.H, w.n, -1)[:heads_sample].double().numpy() for x in (q, k, v))
    threads = min(O.default_threads(), 16)  # the host share of one GPU
    t0 = time.perf_counter()
    O.serial(q, k, v, w.decay, threads=threads)
    dt = time.perf_counter() - t0
    head_tokens = heads_sample * w.n
    return {
        "value": head_tokens / dt / w.H,   # sequence tokens/s: H head-tokens make one token
        "unit": "tokens/s",
        "cores": min(threads, heads_sample),
        "kind": "oracle",
        "sample": "%d of the %d heads of one step (%d tokens each, the step's own inputs), fp64 serial "
                  "recurrence on %d threads, %.1f s wall" % (heads_sample, w.B * w.H, w.n,
                                                              min(threads, heads_sample), dt),
    }


def copy_calibration(torch, gib=1):
    """Two plain device-to-device copies of `gib` GiB, after the timed work:
    the reference kernel against which rocprofv3's FETCH_SIZE / WRITE_SIZE
    counters are scaled (each copy reads and writes gib GiB)."""
    src = torch.empty(gib << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()


def main(argv=None):
    global MIN_WARM_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults reach steady clocks: 50 untimed steps, then 200 timed ones (about 70 ms of forward work)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decay_8k")
    ap.add_argument("--decode-prefill", type=int, default=None, help="prefix tokens (default: the workload's)")
    ap.add_argument("--cpu-heads", type=int, default=128, help="heads in the oracle's timed sample (0: skip)")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-backward", action="store_true")
    ap.add_argument("--skip-variants", action="store_true", help="skip the AHLA and third-order legs")
    ap.add_argument("--skip-workloads", action="store_true",
                    help="skip the other forward workloads (normalised 2k, long 64k)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="finish with two 1 GiB device copies (reference for HBM byte counters)")
    ap.add_argument("--min-warm-ms", type=float, default=MIN_WARM_S * 1e3,
                    help="untimed calls before each timed region last at least this long (0: only --warmup)")
    args = ap.parse_args(argv)
    MIN_WARM_S = max(args.min_warm_ms, 0.0) / 1e3

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the forward shards over (b, h) with no communication; see the design notes).", file=sys.stderr)
        return 2

    import torch
    from causal_prefix_scan_hla2_amd import build as Bld
    if not os.path.exists(os.path.join(ROOT, "causal_prefix_scan_hla2_amd", "libhla2.so")):
        Bld.build()
    from causal_prefix_scan_hla2_amd import hla2 as H
    from causal_prefix_scan_hla2_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    fw = bench_forward(w, args.steps, args.warmup, torch, H, I)
    line = {
        "metric": METRIC,
        "value": fw["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls": fw["warm_calls"],
        "warmup_min_ms": MIN_WARM_S * 1e3,
        "ms_per_step": fw["seconds"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) draws with the workload's scaling, rounded to the element type)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "n": w.n, "d": w.d, "dv": w.dv, "chunk": w.chunk,
                   "decay": w.decay, "normalize": w.normalize, "segments": fw["segments"], "plan": fw["plan"],
                   "global_batch": w.B, "seq_len": w.n, "parallelism": "single GPU"},
        "head_tokens_per_s": fw["head_tokens_per_s"],
        "tflops": fw["tflops"],
        "mfma_frac": fw["mfma_frac"],
        "hbm_min_bytes_frac": fw["min_bytes"] / fw["seconds"] / PEAK_HBM,
        "kernel_ms": {key: val * 1e3 for key, val in fw["phases"].items()},
        "roofline": dict(
            roofline(fw["output_flops_per_call"], fw["output_bytes_per_call"], fw["phases"]["output"]),
            kernel="walk8_kernel<%d,%d,out,decay=%d,den=%d> (chunk outputs%s)" % (
                64 if w.d <= 64 else 128, 64 if w.dv <= 64 else 128, int(w.decay < 1), int(w.normalize),
                " of segments 1 .. %d" % (fw["segments"] - 1) if fw["plan"]["lead"] else ""),
            traffic=load_traffic("output_" + w.name),
            avg_launch_ms=fw["phases"]["output"] * 1e3,
            algorithmic_bytes_per_launch=fw["output_bytes_per_call"],
            algorithmic_flops_per_launch=fw["output_flops_per_call"],
            mfma_tflops=fw["output_flops_per_call"] / fw["phases"]["output"] / 1e12,
            mfma_frac=fw["output_flops_per_call"] / fw["phases"]["output"] / PEAK_BF16_MFMA,
            # measured share of time the MFMA units were busy in this kernel (rocprofv3
            # SQ_VALU_MFMA_BUSY_CYCLES over busy cycles x SIMDs; null when the kernels changed since)
            mfma_busy_counter=(load_counters(w.name + ":output walk") or {}).get("mfma_busy"),
        ),
    }
    if not args.skip_workloads:
        # the other forward workloads, timed like the step (reported beside it, not in `value`)
        line["forward_workloads"] = {}
        for name in ("norm_2k", "long_64k"):
            ow = I.WORKLOADS[name]
            if ow.name == w.name:
                continue
            of = bench_forward(ow, args.steps, args.warmup, torch, H, I)
            line["forward_workloads"][name] = {
                "B": ow.B, "H": ow.H, "n": ow.n, "d": ow.d, "dv": ow.dv, "chunk": ow.chunk, "decay": ow.decay,
                "normalize": ow.normalize, "plan": of["plan"], "ms_per_step": of["seconds"] * 1e3,
                "tokens_per_s": of["tokens_per_s"], "head_tokens_per_s": of["head_tokens_per_s"],
                "tflops": of["tflops"], "mfma_frac": of["mfma_frac"],
                "hbm_min_bytes_frac": of["min_bytes"] / of["seconds"] / PEAK_HBM,
                "kernel_ms": {key: val * 1e3 for key, val in of["phases"].items()},
            }
    if not args.skip_decode:
        dw = I.DECODE
        pre = dw.prefix if args.decode_prefill is None else args.decode_prefill
        dc = bench_decode(dw, max(args.steps, 1) * 4, args.warmup, torch, H, pre)
        line["decode"] = {
            "workload": dw.name, "N": dw.N, "H": dw.H, "d": dw.d, "dv": dw.dv, "prefix": pre,
            "tokens_per_s": dc["tokens_per_s"], "head_tokens_per_s": dc["head_tokens_per_s"],
            "ms_per_step": dc["seconds"] * 1e3,
            "roofline": {"bound": "hbm", "kernel": "hla2_decode_step", "achieved": dc["gbps"],
                         "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": dc["hbm_frac"],
                         "traffic": load_traffic("decode_" + dw.name)},
        }
    if not args.skip_backward:
        bw = bench_backward(w, args.steps, args.warmup, torch, H, I)
        line["backward"] = {
            "workload": w.name, "ms_per_step": bw["seconds"] * 1e3, "tokens_per_s": bw["tokens_per_s"],
            "head_tokens_per_s": bw["head_tokens_per_s"], "vs_forward_time": bw["seconds"] / fw["seconds"],
            "workspace_bytes": bw["workspace_bytes"],
            "hbm_min_bytes_frac": min_bytes_backward(w, 2 if w.dtype == "bf16" else 4) / bw["seconds"] / PEAK_HBM,
        }
    if not args.skip_variants:
        line["ahla"] = bench_variant("hla2_ahla_forward", w, args.steps, args.warmup, torch, H, I,
                                     ahla_flops_per_head_token(w))
        if w.d <= 64:
            line["third_order"] = bench_variant("hla2_ho3_forward", w, args.steps, args.warmup, torch, H, I,
                                                ho3_flops_per_head_token(w))
    if args.cpu_heads > 0:
        line["cpu_baseline"] = cpu_baseline(w, min(args.cpu_heads, w.B * w.H), I)
        line["cpu_baseline"]["single_thread"] = cpu_single_thread(I.WORKLOADS["norm_2k"], I)
    if args.copy_calibration:
        copy_calibration(torch)
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
