#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one S6 selective-scan forward (softplus step, per-token
discretisation, state update, readout, skip, silu gate, segment carry) over the
Mamba-130M-shaped layer workload B=8 L=2048 D=1536 N=16 with bf16 activations
and fp32 state; inputs are seeded synthetic tensors resident in HBM before the
timed region.  Before every step a 512 MiB buffer is rewritten (outside the
timed interval) so that the 203 MB working set is not served from the 256 MB
Infinity Cache.  Each step is bracketed by HIP events recorded by the library
itself on the stream it launches on, at its phase boundaries (segment reduce,
carry scan, segment scan); `value` is the algorithmic bytes of the step
divided by the mean step time.  The default 60 untimed warm-up steps bring the
GPU to its steady clock first (the first ~40 calls of a cold process run up to
~10% slower).

The same run also measures, under "paths", the other calls of the library on
their own workloads (each flushed and timed the same way): the SSD chunked
forward (Mamba-2, B=4 L=8192 H=64 P=64 N=128, chunk 256), the decode step
(64 sequences, D=5120 N=16), the backward pass with recomputation, the
causal conv1d + SiLU, and the conv1d fused in front of the scan (all three on
the Mamba-130M layer shape), and it times the
fp64 CPU oracle on the host cores over the whole S6 workload.

`--only PART` runs one part alone and prints its result (for profiling).
Prints one JSON line.  Only one GPU is used; --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
FP32_VECTOR_PEAK_TFLOPS = 157.3

# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per
# dispatch), scaled by what the same counters read for a 256 MiB copy
# (fetch x2.000, write x1.000); profiles/s6_scan_mamba130m_layer_bf16.md and
# profiles/s6_split_mamba130m_layer_bf16.md, profiles/ssd_chunk_mamba2_bf16.md.  Valid for the kernels as profiled: to be
# re-taken (or set to None) when those kernels change.
S6_LANES_TRAFFIC_BYTES = int((75527.0 * 2.0 + 50814.0) * 1024)
S6_SCAN_TRAFFIC_BYTES = int((83273.4 * 2.0 + 49920.0) * 1024)
SSD_CHUNK_TRAFFIC_BYTES = int((153721.0 * 2.0 + 275968.0) * 1024)


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return lib


def _events(hip, n):
    evs = (ctypes.c_void_p * n)()
    for i in range(n):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs[i] = e
    return evs


def _elapsed(hip, a, b):
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
    return ms.value


def bench_s6(args, torch, ssm, W, native, hip):
    w = W.S6_MAMBA130M
    t = W.make_s6_inputs(w, seed=0)
    dev = torch.device("cuda:0")
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    y = torch.empty_like(d["u"])
    h_last = torch.empty((w.B, w.D, w.N), dtype=torch.float32, device=dev)
    ws_bytes = ssm.selective_scan_workspace_bytes(w.B, w.L, w.D, w.N, torch.bfloat16)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    lanes = ssm.selective_scan_lanes(w.B, w.L, w.D, w.N)
    segments = 1 if lanes else ssm.selective_scan_segments(w.B, w.L, w.D, w.N)
    flush = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=dev)
    lib = native.load()
    stream = torch.cuda.current_stream(dev)
    evs = _events(hip, 4)

    def step(events):
        rc = lib.ssm_selective_scan_fwd_timed(
            d["u"].data_ptr(), d["delta"].data_ptr(), d["A"].data_ptr(), d["B"].data_ptr(),
            d["C"].data_ptr(), d["D"].data_ptr(), d["z"].data_ptr(), d["delta_bias"].data_ptr(),
            native.FLAG_DELTA_SOFTPLUS, None, y.data_ptr(), h_last.data_ptr(),
            w.B, w.L, w.D, w.N, native.SSM_BF16, ws.data_ptr(), ws_bytes, stream.cuda_stream,
            events)
        native.check(rc, "ssm_selective_scan_fwd_timed")

    for i in range(args.warmup):
        flush.fill_(float(i))
        step(None)
    torch.cuda.synchronize()
    # the call as a whole, between two events on its stream
    total = 0.0
    per_step = []
    wall0 = time.perf_counter()
    for i in range(args.steps):
        flush.fill_(float(i))                      # evict the Infinity Cache (untimed)
        hip.hipEventRecord(evs[0], stream.cuda_stream)
        step(None)
        hip.hipEventRecord(evs[1], stream.cuda_stream)
        torch.cuda.synchronize()
        per_step.append(_elapsed(hip, evs[0], evs[1]))
        total += per_step[-1]
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    # the split path's phases (the library records an event at each boundary;
    # a recorded event costs a few microseconds, so this loop is kept apart)
    phases = [0.0, 0.0, 0.0]
    for i in range(args.steps):
        flush.fill_(float(i))
        step(evs)
        torch.cuda.synchronize()
        for k in range(3):
            phases[k] += _elapsed(hip, evs[k], evs[k + 1])
    # back-to-back steps without the flush (working set may sit in the MALL)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(None)
    torch.cuda.synchronize()
    hot_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    ms = total / args.steps
    nbytes = W.s6_algorithmic_bytes(w)
    gbs = nbytes / (ms * 1e-3) / 1e9
    elems = w.B * w.L * w.D * w.N
    # the state-per-lane call is one kernel: its time is the call's
    scan_ms = ms if lanes else phases[2] / args.steps
    reduce_ms = phases[0] / args.steps
    carry_ms = phases[1] / args.steps
    scan_gbs = nbytes / (scan_ms * 1e-3) / 1e9
    flops = 6.0 * elems                            # mul, mul, fma, fma per state update
    return dict(
        ms_median=sorted(per_step)[len(per_step) // 2], ms_min=min(per_step),
        w=w, t=t, ms=ms, gbs=gbs, nbytes=nbytes, segments=segments, lanes=lanes, wall=wall,
        hot_ms=hot_ms,
        phases_ms=(dict(state_per_lane=scan_ms) if lanes else
                   dict(segment_reduce=reduce_ms, carry_scan=carry_ms, segment_scan=scan_ms)),
        scan_gbs=scan_gbs, scan_tflops=flops / (scan_ms * 1e-3) / 1e12,
        gtokch=w.tok_ch / (ms * 1e-3) / 1e9, elems=elems)


def bench_ssd(args, torch, ssm, W):
    s = W.SSD_MAMBA2
    t = W.make_ssd_inputs(s, seed=0)
    dev = torch.device("cuda:0")
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    Y = torch.empty_like(d["X"])
    flush = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=dev)

    def step():
        ssm.ssd_chunk_fwd(d["X"], d["delta"], d["A"], d["B"], d["C"], chunk=s.chunk, out=Y)

    try:
        step()
    except ssm.SSMError as e:
        return dict(status=f"unavailable: {e}")
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    total = 0.0
    for i in range(args.steps):
        flush.fill_(float(i))
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        total += a.elapsed_time(b)
    ms = total / args.steps
    nbytes = W.ssd_algorithmic_bytes(s)
    Q = s.chunk
    nchunks = -(-s.L // Q)
    # causal chunked-SSD MACs: the scores C B^T (lower triangle, Q(Q+1)/2 * N)
    # once per (b, group, chunk), as they depend on the group only; per (b, h,
    # chunk) the masked Y_diag (Q(Q+1)/2 * P), chunk state (P*N*Q) and Y_off
    # (Q*P*N).  The kernel forms the scores per head, so it executes more.
    tri = Q * (Q + 1) / 2
    per_head = tri * s.P + 2 * s.P * s.N * Q
    macs = s.B * nchunks * (s.G * tri * s.N + s.H * per_head)
    macs_exec = s.B * nchunks * s.H * (tri * s.N + per_head)
    return dict(status="ok", workload=s.name, ms=round(ms, 5),
                gbs=round(nbytes / (ms * 1e-3) / 1e9, 2),
                pct_hbm_peak=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS * 100, 2),
                tflops=round(2 * macs / (ms * 1e-3) / 1e12, 2),
                mfma_util=round(2 * macs / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                gtokch=round(s.tok_ch / (ms * 1e-3) / 1e9, 3), algorithmic_bytes=nbytes,
                causal_gflop=round(2 * macs / 1e9, 3),
                executed_gflop=round(2 * macs_exec / 1e9, 3),
                executed_tflops=round(2 * macs_exec / (ms * 1e-3) / 1e12, 2),
                hbm_traffic_bytes=SSD_CHUNK_TRAFFIC_BYTES)


def _time_flushed(torch, fn, steps, warmup):
    """Mean ms of fn() over `steps` calls, each after rewriting a 512 MiB
    buffer (untimed), bracketed by events on the current stream."""
    flush = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device="cuda:0")
    for _ in range(max(1, warmup)):
        fn()
    torch.cuda.synchronize()
    total = 0.0
    for i in range(steps):
        flush.fill_(float(i))
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        total += a.elapsed_time(b)
    return total / steps


def bench_decode(args, torch, ssm, W):
    w = W.S6_DECODE_2P8B
    t = W.make_step_inputs(w, seed=0)
    d = {k: (v.to("cuda:0") if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    y = torch.empty((w.B, w.D), dtype=torch.bfloat16, device="cuda:0")

    def step():
        ssm.selective_state_update(d["state"], d["u"], d["delta"], d["A"], d["B"], d["C"],
                                   D=d["D"], z=d["z"], delta_bias=d["delta_bias"], out=y)

    ms = _time_flushed(torch, step, args.steps, args.warmup)
    nbytes = W.step_algorithmic_bytes(w)
    return dict(status="ok", workload=w.name, ms=round(ms, 5), algorithmic_bytes=nbytes,
                gbs=round(nbytes / (ms * 1e-3) / 1e9, 2),
                pct_hbm_peak=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS * 100, 2),
                state_updates_per_s=round(w.B * w.D * w.N / (ms * 1e-3), 1))


def bench_bwd(args, torch, ssm, W):
    w = W.S6_MAMBA130M
    t = W.make_s6_inputs(w, seed=0)
    d = {k: (v.to("cuda:0") if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    g = torch.Generator().manual_seed(1)
    dy = torch.randn(w.B, w.L, w.D, generator=g).to(torch.bfloat16).to("cuda:0")
    need = int(ssm._native.load().ssm_selective_scan_bwd_workspace_bytes(w.B, w.L, w.D, w.N, 1))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")

    def step():
        ssm.selective_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], dy, D=d["D"],
                               z=d["z"], delta_bias=d["delta_bias"], workspace=ws)

    ms = _time_flushed(torch, step, args.steps, args.warmup)
    e = 2
    # inputs u, delta, z, dy, B, C read and du, ddelta, dz written once (bf16);
    # dB, dC fp32; A, dA and the per-channel vectors are negligible
    nbytes = 7 * w.B * w.L * w.D * e + 2 * w.B * w.L * w.N * (e + 4)
    return dict(status="ok", workload=w.name, ms=round(ms, 5), algorithmic_bytes=nbytes,
                gbs=round(nbytes / (ms * 1e-3) / 1e9, 2),
                gtokch=round(w.tok_ch / (ms * 1e-3) / 1e9, 3), workspace_bytes=need)


def bench_conv(args, torch, ssm, W):
    w = W.CONV_MAMBA130M
    t = W.make_conv_inputs(w, seed=0)
    d = {k: v.to("cuda:0") for k, v in t.items()}
    u = torch.empty_like(d["x"])

    def step():
        ssm.causal_conv1d_silu(d["x"], d["weight"], d["bias"], out=u)

    ms = _time_flushed(torch, step, args.steps, args.warmup)
    nbytes = W.conv_algorithmic_bytes(w)
    return dict(status="ok", workload=w.name, ms=round(ms, 5), algorithmic_bytes=nbytes,
                gbs=round(nbytes / (ms * 1e-3) / 1e9, 2),
                pct_hbm_peak=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS * 100, 2))


def bench_conv_scan(args, torch, ssm, W):
    """The conv1d + SiLU fused in front of the S6 scan, on the Mamba-130M layer
    shape with a K = 4 convolution: x replaces u as the input, so the
    algorithmic bytes are those of the scan plus the convolution weights."""
    w = W.S6_MAMBA130M
    t = W.make_s6_inputs(w, seed=0)
    cv = W.make_conv_inputs(W.CONV_MAMBA130M, seed=1)
    d = {k: (v.to("cuda:0") if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    x, cw, cb = (cv[k].to("cuda:0") for k in ("x", "weight", "bias"))
    y = torch.empty_like(d["u"])
    ws = torch.empty(max(1, ssm.selective_scan_workspace_bytes(w.B, w.L, w.D, w.N)),
                     dtype=torch.uint8, device="cuda:0")

    def step():
        ssm.selective_scan_conv_fwd(x, cw, cb, d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                    z=d["z"], delta_bias=d["delta_bias"], out=y, workspace=ws)

    ms = _time_flushed(torch, step, args.steps, args.warmup)
    nbytes = W.s6_algorithmic_bytes(w) + W.CONV_MAMBA130M.D * (W.CONV_MAMBA130M.K + 1) * 4
    return dict(status="ok", workload=w.name + "+conv1d_k4", ms=round(ms, 5),
                algorithmic_bytes=nbytes, gbs=round(nbytes / (ms * 1e-3) / 1e9, 2),
                gtokch=round(w.tok_ch / (ms * 1e-3) / 1e9, 3))


def cpu_baseline(r, torch, min_seconds=10.0):
    """The fp64 oracle over the whole S6 workload on the host cores, repeated
    until at least `min_seconds` of wall time (the workload alone takes well
    under a second); value = algorithmic bytes per workload / mean seconds."""
    import oracle
    w, t = r["w"], r["t"]
    f64 = {k: (oracle._f64(v) if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    threads = oracle.default_threads()
    runs = 0
    t0 = time.perf_counter()
    while True:
        oracle.s6_fwd(f64["u"], f64["delta"], f64["A"], f64["B"], f64["C"], D=f64["D"],
                      z=f64["z"], delta_bias=f64["delta_bias"], threads=threads)
        runs += 1
        total = time.perf_counter() - t0
        if total >= min_seconds:
            break
    sec = total / runs
    return {"value": round(r["nbytes"] / sec / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole {w.name} workload (B={w.B} L={w.L} D={w.D} N={w.N}), run "
                      f"{runs} times ({total:.1f} s wall); fp64 sequential loop per channel, "
                      f"channels over {threads} OpenMP threads; algorithmic bytes of the "
                      f"workload / mean seconds per run",
            "seconds_per_run": round(sec, 4),
            "gtokch_per_s": round(w.tok_ch / sec / 1e9, 6)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU reaches its steady clock after ~30-40 back-to-back calls
    # (~15 ms): the first calls of a cold process run ~10% slower
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ssd", action="store_true", help="skip every path but the S6 scan")
    ap.add_argument("--only", choices=["s6", "ssd", "decode", "bwd", "conv", "conv_scan"],
                    help="run one part alone and print its result")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a plain 256 MiB device copy three times, the "
                         "reference for scaling FETCH_SIZE/WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the scan is data-parallel over channels and would shard with no "
              "communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_21_amd as ssm
    from selective_state_space_21_amd import _native as native
    from selective_state_space_21_amd import workloads as W

    hip = _hip()
    if args.calibration_copy:
        src = torch.ones(64 * 2**20, dtype=torch.float32, device="cuda:0")   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only and args.only != "s6":
        fn = {"ssd": bench_ssd, "decode": bench_decode, "bwd": bench_bwd, "conv": bench_conv,
              "conv_scan": bench_conv_scan}
        res = fn[args.only](args, torch, ssm, W)
        print(json.dumps({"part": args.only, **{k: v for k, v in res.items()}}), flush=True)
        return
    r = bench_s6(args, torch, ssm, W, native, hip)
    paths = {}
    if not args.no_ssd and not args.only:
        paths["ssd_chunk_fwd"] = bench_ssd(args, torch, ssm, W)
        paths["selective_state_update"] = bench_decode(args, torch, ssm, W)
        paths["selective_scan_bwd"] = bench_bwd(args, torch, ssm, W)
        paths["causal_conv1d_silu"] = bench_conv(args, torch, ssm, W)
        paths["selective_scan_conv_fwd"] = bench_conv_scan(args, torch, ssm, W)
    w = r["w"]
    line = {
        "metric": "selective-scan fwd achieved HBM GB/s (% of peak) + Gtoken·channels/s",
        "value": round(r["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "L": w.L, "D": w.D, "N": w.N,
            "io_dtype": "bf16", "state_dtype": "f32",
            "path": "state_per_lane" if r["lanes"] else "split", "segments": r["segments"],
            "pct_of_hbm_peak": round(r["gbs"] / HBM_PEAK_GBS * 100, 2),
            "gtoken_channels_per_s": round(r["gtokch"], 3),
            "algorithmic_bytes": r["nbytes"],
            "phases_ms": {k: round(v, 5) for k, v in r["phases_ms"].items()},
            "ms_median": round(r["ms_median"], 5), "ms_min": round(r["ms_min"], 5),
            "ms_per_step_without_cache_flush": round(r["hot_ms"], 5),
        },
        "roofline": {
            "kernel": ("s6_lanes (state per lane, the only kernel of the call)" if r["lanes"]
                       else "s6_fast segment scan (dominant phase)"),
            "bound": "hbm",
            "achieved": round(r["scan_gbs"], 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["scan_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": S6_LANES_TRAFFIC_BYTES if r["lanes"] else S6_SCAN_TRAFFIC_BYTES,
            "alu_view": {"achieved_tflops": round(r["scan_tflops"], 3),
                         "peak_tflops": FP32_VECTOR_PEAK_TFLOPS,
                         "flops_per_state_update": 6, "transcendentals_per_state_update": 1},
        },
    }
    if paths:
        line["paths"] = paths
    if not args.no_cpu_baseline and not args.only:
        line["cpu_baseline"] = cpu_baseline(r, torch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
