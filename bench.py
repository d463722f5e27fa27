#!/usr/bin/env python3
"""Benchmark of the FlashAttention forward on one MI355X.

A step is one fa_fwd call: the whole forward (tile scheduling, Q/K/V loads,
S = QK^T, masking, online softmax with conditional rescale, O += PV, epilogue)
runs in one kernel launch on inputs already resident in HBM.  The default
workload is causal attention, B=2, H=32, Nq=Nk=4096, d=128, bf16 in, bf16 O,
fp32 LSE, scale 1/sqrt(128), seeded N(0,1) inputs.

Timing: first a settle phase of back-to-back launches until --settle-ms of
wall time have passed (the shader clock of a cold GPU takes a few hundred
milliseconds of load to reach its steady value, whatever --warmup says), then
--warmup untimed steps, then exactly --steps timed steps between two
synchronisations.  Right after them the same launches run once more, now with
a one-wavefront probe on a second stream sampling the shader clock against the
constant-rate clock (fa_clock_probe), so the line states the clock the
throughput was measured at.  (The probe holds registers on one compute unit,
where a workgroup of the d = 128 kernel then no longer fits; beside the timed
loop it slowed it by about 6%, so it samples an adjacent window of the same
load instead.)

Prints one JSON line:
  value        TFLOP/s = 4*B*H*Nq*Nk*d/2 (causal) / ms_per_step
  roofline     the kernel's achieved TFLOP/s from the average launch duration
               over the timed region (two HIP events on the launch stream
               bracketing the K launches), against the bf16
               dense MFMA peak (2.5 PFLOP/s, nominal at 2.4 GHz), and against
               CUs x 4096 flop/clk x the measured shader clock (peak_at_sclk);
               launch_ms_median / launch_ms_min: median and minimum of K more
               launches, each between its own pair of events (the mean is
               avg_launch_ms);
               traffic = HBM bytes per launch from the committed rocprofv3
               FETCH_SIZE / WRITE_SIZE summary (null unless it was taken on the
               kernel source as it is now)
  cpu_baseline the fp64 CPU oracle timed on a bounded sample of the same
               workload (whole (batch, head) slices until ~10 s have passed)

With --backward a step is one fa_bwd call (two launches: the dQ kernel, which
also forms the row terms D = rowsum(dO*O), then the dK/dV kernel) on the forward's O and LSE
and a seeded dO; its flops are counted as 2.5x the forward's (the five
products of the gradient), the events bracket the whole call, and traffic is
null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA (256 CUs at 2.4 GHz)
MFMA_BF16_FLOP_PER_CLK_CU = 4096  # dense bf16 matrix-core flops per clock per CU
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["flashattention_forward_fa_amd/csrc/fa_fwd_kernel.hip",
                  "flashattention_forward_fa_amd/csrc/fa_device.h",
                  "flashattention_forward_fa_amd/csrc/fa_internal.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch from profiles/<workload>.pmc.txt, or None when the
    counters were taken on another kernel source."""
    path = os.path.join(ROOT, "profiles", f"fa_fwd_{workload}.pmc.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    fields = dict(re.findall(r"^([a-z0-9_]+):\s*(\S+)\s*$", text, flags=re.M))
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float, backward: bool = False):
    """Time the oracle on whole (sequence, head) slices of the workload until budget_s
    (the backward: gradients of one slice's O for the seeded dO)."""
    import oracle
    from flashattention_forward_fa_amd import workloads as wl
    orc = oracle.default()
    d = w.d
    group = w.H // w.kv_heads
    dout_bits = wl.make_dout(w, seed=w.seed + 500) if backward else None
    if w.varlen:
        units = [(b, h) for h in range(w.H) for b in range(len(w.lengths))]
    else:
        units = [(b, h) for h in range(w.H) for b in range(w.B)]
    flops = 0.0
    spent = 0.0
    done = 0
    for (b, h) in units:
        hk = h // group
        if w.varlen:
            sl = slice(int(w.offsets[b]), int(w.offsets[b + 1]))
            pick = lambda x, j: wl.bf16_to_f64(x[sl, j:j + 1])[None]
            Nq = Nk = int(w.lengths[b])
        else:
            pick = lambda x, j: wl.bf16_to_f64(x[b:b + 1, :, j:j + 1])
            Nq, Nk = w.Nq, w.Nk
        q, k, v = pick(w.q, h), pick(w.k, hk), pick(w.v, hk)
        if backward:
            dout = pick(dout_bits, h)
            t0 = time.perf_counter()
            orc.attention_bwd(q, k, v, dout, w.scale, w.causal)
        else:
            t0 = time.perf_counter()
            orc.attention(q, k, v, w.scale, w.causal)
        spent += time.perf_counter() - t0
        per = 4.0 * Nq * Nk * d * (2.5 if backward else 1.0)
        flops += per / 2.0 if w.causal else per
        done += 1
        if spent >= budget_s:
            break
    what = "fp64 backward (forward recomputed, then dQ, dK, dV)" if backward else \
        "fp64 three-pass"
    # The backward's parallel loop runs over (batch, K/V head): one slice per call is
    # one thread.  The forward's runs over query rows and uses every thread.
    cores = 1 if backward else orc.num_threads()
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": cores, "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{done} of {len(units)} (sequence, head) slices, every query row of each, "
                      f"{what}, {spent:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps after the settle phase")
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="launch back to back for at least this long before the warm-up (clocks)")
    ap.add_argument("--config", type=int, default=3, help="workload 1-5 (3 = the headline)")
    ap.add_argument("--tau", type=float, default=8.0, help="rescale threshold")
    ap.add_argument("--exp2-poly", type=int, default=0,
                    help="exponentials per 16 by the FMA polynomial (0 = all by v_exp_f32, or 8)")
    ap.add_argument("--backward", action="store_true",
                    help="time fa_bwd (dQ, dK, dV for the forward's outputs) instead of fa_fwd")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="grouped K/V heads for workloads 2-4 (0 = as many as query heads)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the oracle CPU baseline (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of attention, time a plain device copy of 1 GiB (used to "
                         "scale the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the forward shards over (batch, head) with no exchange; run one process per GPU)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import flashattention_forward_fa_amd as fa
    from flashattention_forward_fa_amd import workloads as wl
    from tests import parity

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = 1 << 29                                   # 2^29 bf16 = 1 GiB each way
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n,
                          "ms_per_copy": round(ms, 4),
                          "GB_per_s": round(4 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return
    fa.load()
    w = wl.grouped(args.config, args.kv_heads) if args.kv_heads else wl.config(args.config)
    q, k, v, off = parity.to_device(w)
    odt = fa.FA_DTYPE_F32 if w.o_dtype == "f32" else fa.FA_DTYPE_BF16
    o = torch.empty(q.shape, dtype=torch.float32 if odt else torch.bfloat16, device="cuda")
    if w.varlen:
        lse = torch.empty((w.H, w.total_tokens), dtype=torch.float32, device="cuda")
    else:
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    opts = fa.fa_fwd_opts_default()
    opts.o_dtype = odt
    opts.rescale_threshold = args.tau
    opts.kv_heads = w.kv_heads
    opts.exp2_poly = args.exp2_poly
    stream = torch.cuda.current_stream()

    def step():
        st = fa.fa_fwd_ex(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal),
                          off, stream, opts)
        if st != fa.FA_OK:
            raise fa.FaError(st)

    if args.backward:
        # The backward's inputs: the forward's O (bf16) and LSE, a seeded dO.
        if odt != fa.FA_DTYPE_BF16:
            raise SystemExit("the backward takes a bf16 O: use a workload with bf16 output")
        step()
        dout = torch.from_numpy(wl.make_dout(w, seed=w.seed + 500).view(np.int16)).view(
            torch.bfloat16).to("cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty((fa.fa_bwd_workspace_size(w.B, w.H, w.Nq) // 4,), dtype=torch.float32,
                         device="cuda")

        def step():  # noqa: F811 -- the timed step is the backward
            st = fa.fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, w.B, w.H, w.Nq, w.Nk, w.d,
                           w.scale, int(w.causal), off, w.kv_heads, stream)
            if st != fa.FA_OK:
                raise fa.FaError(st)

    # Settle: back-to-back launches until settle_ms of wall time have passed.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    settle_launches = 0
    while True:
        for _ in range(10):
            step()
        settle_launches += 10
        torch.cuda.synchronize()
        settle_ms = (time.perf_counter() - t0) * 1e3
        if settle_ms >= args.settle_ms:
            break

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The whole job: K steps back to back, wall clock between two syncs, and
    # two HIP events on the launch stream bracketing the same K launches (the
    # kernel's average launch duration back to back, for the roofline).
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    avg_launch_ms = ev0.elapsed_time(ev1) / args.steps

    # The shader clock under the same load: K more launches with the probe
    # sampling beside them for about 90% of their expected duration.
    probe_interval_us = 10
    n_probe = max(2, min(1000000, int(0.9 * ms_per_step * args.steps * 1e3 / probe_interval_us)))
    samples = torch.zeros(2 * n_probe, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    st_probe, ref_hz = fa.fa_clock_probe(samples, n_probe, probe_interval_us, side)
    if st_probe != fa.FA_OK:
        raise fa.FaError(st_probe, "fa_clock_probe")
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    sm = samples.cpu().numpy().astype(np.float64).reshape(-1, 2)
    sclk_ghz = float((sm[-1, 0] - sm[0, 0]) / (sm[-1, 1] - sm[0, 1]) * ref_hz / 1e9)
    probe_ms = float((sm[-1, 1] - sm[0, 1]) / ref_hz * 1e3)

    # Per-launch durations: K more launches, each between its own pair of
    # events on the launch stream (the launches still queue back to back);
    # their median and minimum beside the mean above.
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e0, e1 in pairs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    per_launch = np.array([e0.elapsed_time(e1) for e0, e1 in pairs])
    launch_ms_median = float(np.median(per_launch))
    launch_ms_min = float(per_launch.min())

    flops = w.flops() * (2.5 if args.backward else 1.0)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    peak_at_sclk = cus * MFMA_BF16_FLOP_PER_CLK_CU * sclk_ghz * 1e9 / 1e12
    traffic = None if args.backward else traffic_from_profile(w.name)
    # The headline metric names its workload; another --config or --kv-heads names its own.
    metric = "attention fwd TFLOP/s and % of bf16 MFMA peak (d=128, N=4096 causal)"
    if args.config != 3 or args.kv_heads or args.exp2_poly:
        poly = f", exp2 polynomial {args.exp2_poly}/16" if args.exp2_poly else ""
        metric = f"attention fwd TFLOP/s and % of bf16 MFMA peak ({w.name}{poly})"
    if args.backward:
        metric = ("attention bwd TFLOP/s (algorithmic flops 2.5x the forward's: five products) "
                  f"and % of bf16 MFMA peak ({w.name})")
    result = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": round(settle_ms, 1),
        "settle_launches": settle_launches,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 Q/K/V",
        "config": {**w.describe(), "rescale_threshold": args.tau, "exp2_poly": args.exp2_poly,
                   "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "sclk_ghz": round(sclk_ghz, 4),
                     "sclk_window_ms": round(probe_ms, 3),
                     "peak_at_sclk": round(peak_at_sclk, 1),
                     "frac_at_sclk": round(achieved / peak_at_sclk, 4),
                     "cus": cus,
                     "avg_launch_ms": round(avg_launch_ms, 5),
                     "launch_ms_median": round(launch_ms_median, 5),
                     "launch_ms_min": round(launch_ms_min, 5),
                     "achieved_at_median": round(flops / (launch_ms_median * 1e-3) / 1e12, 2),
                     "algorithmic_hbm_bytes": w.io_bytes()},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, args.backward)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
