#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one S6 selective-scan forward (softplus step, per-token
discretisation, state update, readout, skip, silu gate, segment carry) over the
Mamba-130M-shaped layer workload B=8 L=2048 D=1536 N=16 with bf16 activations
and fp32 state; inputs are seeded synthetic tensors resident in HBM before the
timed region.  `value` is the algorithmic bytes of the step (every input read
once, y and the final state written once) divided by the mean step time
between two HIP events on the stream the library launches on.

Cache: the 203 MB working set fits the 256 MB Infinity Cache, so before every
timed call a 512 MiB buffer is read (outside the timed interval).  A read pass
leaves clean lines behind; the previous protocol rewrote the buffer instead,
which left the cache full of dirty lines whose write-back then landed inside
the timed call.  Both are reported for the headline workload
(`ms_per_step_dirty_flush`), as is the time of back-to-back calls without any
flush.

The same run measures, under "paths", the other workloads and calls of the
library, each flushed and timed the same way: the Mamba-2.8B-shaped layer
scan, the long fp32 sequence (131072 tokens, split over the sequence with a
segment carry), the SSD chunked forward (Mamba-2), the decode step, the
backward pass with recomputation, the causal conv1d + SiLU and the conv1d
fused in front of the scan.  It also times a plain device copy of the same
byte count as the practical bandwidth ceiling.

The CPU leg (`cpu_baseline`) times the fp64 oracle on the host, on one thread
and on all cores, and checks sampled outputs of every timed S6 and SSD call
against it before the line is printed (the line carries `verified`; a failed
check exits with status 1 after printing).

`--only PART` runs one part alone and prints its result (for profiling).
Prints one JSON line.  Only one GPU is used; --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
CSRC = os.path.join(ROOT, "selective_state_space_21_amd", "csrc")

HBM_PEAK_GBS = 8000.0           # MI355X published HBM3E bandwidth
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
# MI355X published fp32 vector peak: 256 CUs x 2.4 GHz x 256 flop/clk, i.e. a
# wave64 FMA every 2 cycles per SIMD.  Plain (non-packed) v_fma_f32 is priced
# against it: instruction counters on the issue-rate probe show one
# non-packed FMA per lane and instruction retiring at 24.6 lanes per
# SIMD-cycle, above the 16 a 78.6 TFLOP/s reading would allow
# (profiles/issue_rates_gfx950.md).
FP32_VECTOR_PEAK_TFLOPS = 157.3
# The bare per-element pattern of the scan (dt*A, exp2, dt*u*B, state FMA,
# readout FMA) measured on its own at 8 waves per SIMD: the rate a scan kernel
# cannot exceed while it evaluates one v_exp_f32 per state update
# (profiles/issue_rates_gfx950.md).
ISSUE_PEAK_ELEMS_PER_S = 6.52e12

# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per
# dispatch), scaled by what the same counters read for a 256 MiB copy (fetch
# x2.000, write x1.000), with the hash of the sources the kernel was built from
# when the counters were taken.  A kernel whose sources changed since then
# reports traffic null until its counters are taken again.
COUNTER_TRAFFIC = {
    # kernel@workload: (bytes, sources, sha1 of the sources)
    "s6_lanes@s6_mamba130m_layer_bf16": (205222194, ['s6_fwd.hip', 's6_plan.cpp', 'device_math.h', 'lane_ops.h', 'ssm_internal.h'], "42494928e818"),
    "s6_lanes@s6_mamba2.8b_layer_bf16": (687235652, ['s6_fwd.hip', 's6_plan.cpp', 'device_math.h', 'lane_ops.h', 'ssm_internal.h'], "42494928e818"),
    "s6_lanes@s6_long_fp32": (3523984132, ['s6_fwd.hip', 's6_plan.cpp', 'device_math.h', 'lane_ops.h', 'ssm_internal.h'], "42494928e818"),
    "ssd@ssd_mamba2_bf16": (600585033, ['ssd_fwd.hip', 'device_math.h', 'lane_ops.h', 'ssm_internal.h'], "744bff51c7ed"),
}


def sources_sha1(files) -> str:
    h = hashlib.sha1()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def counter_traffic(key: str):
    """(bytes or None, note) for a kernel@workload key."""
    ent = COUNTER_TRAFFIC.get(key)
    if ent is None:
        return None, "no counter run for this kernel"
    nbytes, srcs, sha = ent
    if sources_sha1(srcs) != sha:
        return None, "kernel sources changed since the counters were taken"
    return nbytes, "rocprofv3 FETCH_SIZE/WRITE_SIZE scaled by a 256 MiB copy"


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


class Flusher:
    """Evicts the 256 MB Infinity Cache before a timed call (untimed): `clean`
    reads a 512 MiB buffer (the lines it leaves are clean), `dirty` rewrites it
    (the old protocol: the dirty lines are written back during the next call)."""

    def __init__(self, torch):
        self.torch = torch
        self.buf = torch.zeros(512 * 2**20 // 4, dtype=torch.float32, device="cuda:0")
        self.i = 0

    def clean(self):
        self.torch.sum(self.buf)

    def dirty(self):
        self.i += 1
        self.buf.fill_(float(self.i))


class Timer:
    """Mean/median/min ms of a call between two HIP events recorded on the
    stream the call launches on, each call preceded by `flush` (untimed)."""

    def __init__(self, torch, hip):
        self.torch, self.hip = torch, hip
        self.ev = _events(hip, 2)

    def run(self, fn, steps, warmup, flush=None):
        torch, hip = self.torch, self.hip
        stream = torch.cuda.current_stream().cuda_stream
        for _ in range(warmup):
            if flush:
                flush()
            fn()
        torch.cuda.synchronize()
        per = []
        for _ in range(steps):
            if flush:
                flush()
            hip.hipEventRecord(self.ev[0], stream)
            fn()
            hip.hipEventRecord(self.ev[1], stream)
            torch.cuda.synchronize()
            per.append(_elapsed(hip, self.ev[0], self.ev[1]))
        per.sort()
        return dict(mean=sum(per) / len(per), median=per[len(per) // 2], min=per[0])


def roofline(kind, achieved, peak, unit, traffic=None, note=None, **extra):
    r = {"bound": kind, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic}
    if note:
        r["traffic_note"] = note
    r.update(extra)
    return r


# ------------------------------------------------------------------ S6
def bench_s6(args, ctx, w, headline=False):
    torch, ssm, W, native, hip = ctx["torch"], ctx["ssm"], ctx["W"], ctx["native"], ctx["hip"]
    t = W.make_s6_inputs(w, seed=0)
    dev = torch.device("cuda:0")
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    y = torch.empty_like(d["u"])
    h_last = torch.empty((w.B, w.D, w.N), dtype=torch.float32, device=dev)
    dtc = native.SSM_BF16 if w.dtype == "bf16" else native.SSM_F32
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    ws_bytes = ssm.selective_scan_workspace_bytes(w.B, w.L, w.D, w.N, tdt)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    lanes = ssm.selective_scan_lanes(w.B, w.L, w.D, w.N)
    segments = ssm.selective_scan_segments(w.B, w.L, w.D, w.N)
    lib = native.load()
    stream = torch.cuda.current_stream(dev)
    evs = _events(hip, 4)
    ptr = lambda k: None if d[k] is None else d[k].data_ptr()

    def step(events=None):
        rc = lib.ssm_selective_scan_fwd_timed(
            ptr("u"), ptr("delta"), ptr("A"), ptr("B"), ptr("C"), ptr("D"), ptr("z"),
            ptr("delta_bias"), native.FLAG_DELTA_SOFTPLUS, None, y.data_ptr(), h_last.data_ptr(),
            w.B, w.L, w.D, w.N, dtc, ws.data_ptr(), ws_bytes, stream.cuda_stream, events)
        native.check(rc, "ssm_selective_scan_fwd_timed")

    fl = ctx["flusher"]
    tm = ctx["timer"]
    wall0 = time.perf_counter()
    res = tm.run(step, args.steps, args.warmup, fl.clean)
    wall = time.perf_counter() - wall0
    # phases (the library records an event at each boundary; recording costs a
    # few microseconds, so this loop is kept apart from the timed one)
    phases = [0.0, 0.0, 0.0]
    n_ph = max(3, args.steps // 4)
    for _ in range(n_ph):
        fl.clean()
        step(evs)
        torch.cuda.synchronize()
        for k in range(3):
            phases[k] += _elapsed(hip, evs[k], evs[k + 1])
    phases = [p / n_ph for p in phases]
    extra = {}
    if headline:
        extra["dirty"] = tm.run(step, args.steps, 0, fl.dirty)
        extra["hot"] = tm.run(step, args.steps, 0, None)
    torch.cuda.synchronize()
    ms = res["mean"]
    nbytes = W.s6_algorithmic_bytes(w)
    elems = w.B * w.L * w.D * w.N
    # library events: state-per-lane path [scan of every segment | carry |
    # fix-up of the later segments]; split path [segment reduce | carry |
    # segment rescan]
    if lanes:
        ph = {"scan": phases[0]}
        if segments > 1:
            ph.update(carry=phases[1], fixup=phases[2])
        dom_name, dom_ms = "s6_lanes (scan of every segment)", phases[0]
    else:
        ph = {"segment_reduce": phases[0], "carry": phases[1], "segment_rescan": phases[2]}
        dom_name, dom_ms = "s6_fast segment rescan", phases[2]
    # the dominant kernel reads every input and writes y
    dom_gbs = nbytes / (dom_ms * 1e-3) / 1e9
    key = f"{'s6_lanes' if lanes else 's6_split'}@{w.name}"
    traffic, note = counter_traffic(key)
    out = dict(
        status="ok", workload=w.name, B=w.B, L=w.L, D=w.D, N=w.N, io_dtype=w.dtype,
        path="state_per_lane" if lanes else "split", segments=segments,
        ms=round(ms, 5), ms_median=round(res["median"], 5), ms_min=round(res["min"], 5),
        gbs=round(nbytes / (ms * 1e-3) / 1e9, 2),
        pct_hbm_peak=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS * 100, 2),
        gtokch=round(w.tok_ch / (ms * 1e-3) / 1e9, 3), algorithmic_bytes=nbytes,
        phases_ms={k: round(v, 5) for k, v in ph.items()},
        roofline=roofline("hbm", dom_gbs, HBM_PEAK_GBS, "GB/s", traffic, note,
                          kernel=dom_name),
        issue=roofline("issue", elems / (ms * 1e-3) / 1e9, ISSUE_PEAK_ELEMS_PER_S / 1e9,
                       "G state updates/s",
                       peak_source="the bare per-element pattern (4 VALU + 1 v_exp_f32) "
                                   "measured alone at 8 waves per SIMD"),
        alu_view={"achieved_tflops": round(6.0 * elems / (ms * 1e-3) / 1e12, 3),
                  "peak_tflops": FP32_VECTOR_PEAK_TFLOPS, "flops_per_state_update": 6,
                  "transcendentals_per_state_update": 1},
        wall_s=round(wall, 3))
    if headline:
        out["ms_dirty_flush"] = round(extra["dirty"]["mean"], 5)
        out["ms_no_flush"] = round(extra["hot"]["mean"], 5)
    import numpy as np
    samples = _sample_channels(w, np.random.default_rng(123))
    ctx["verify"].append(("s6", w, t, samples,
                          [y[b][:, ds].float().cpu() for b, ds in samples],
                          [h_last[b][ds].cpu() for b, ds in samples]))
    return out


# ------------------------------------------------------------------ SSD
def bench_ssd(args, ctx):
    torch, ssm, W = ctx["torch"], ctx["ssm"], ctx["W"]
    s = W.SSD_MAMBA2
    t = W.make_ssd_inputs(s, seed=0)
    dev = torch.device("cuda:0")
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    Y = torch.empty_like(d["X"])

    def step():
        ssm.ssd_chunk_fwd(d["X"], d["delta"], d["A"], d["B"], d["C"], chunk=s.chunk, out=Y)

    try:
        ssm.ssd_chunk_fwd(d["X"], d["delta"], d["A"], d["B"], d["C"], chunk=s.chunk, out=Y)
    except ssm.SSMError as e:
        return dict(status=f"unavailable: {e}")
    res = ctx["timer"].run(step, args.steps, args.warmup, ctx["flusher"].clean)
    _, h_last = ssm.ssd_chunk_fwd(d["X"], d["delta"], d["A"], d["B"], d["C"], chunk=s.chunk,
                                  out=Y)
    torch.cuda.synchronize()
    ms = res["mean"]
    nbytes = W.ssd_algorithmic_bytes(s)
    Q = s.chunk
    nchunks = -(-s.L // Q)
    # causal chunked-SSD MACs: the scores C B^T (lower triangle, Q(Q+1)/2 * N)
    # once per (b, group, chunk), as they depend on the group only; per (b, h,
    # chunk) the masked Y_diag (Q(Q+1)/2 * P), chunk state (P*N*Q) and Y_off
    # (Q*P*N).
    tri = Q * (Q + 1) / 2
    per_head = tri * s.P + 2 * s.P * s.N * Q
    macs = s.B * nchunks * (s.G * tri * s.N + s.H * per_head)
    macs_exec = s.B * nchunks * s.H * (tri * s.N + per_head)
    traffic, note = counter_traffic(f"ssd@{s.name}")
    gbs = nbytes / (ms * 1e-3) / 1e9
    pairs = [(0, 0), (s.B - 1, s.H - 1)]
    ctx["verify"].append(("ssd", s, t, pairs, [Y[b, :, hh].float().cpu() for b, hh in pairs],
                          [h_last[b, hh].cpu() for b, hh in pairs]))
    return dict(status="ok", workload=s.name, ms=round(ms, 5), ms_median=round(res["median"], 5),
                ms_min=round(res["min"], 5), gbs=round(gbs, 2),
                pct_hbm_peak=round(gbs / HBM_PEAK_GBS * 100, 2),
                tflops=round(2 * macs / (ms * 1e-3) / 1e12, 2),
                mfma_util=round(2 * macs / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                gtokch=round(s.tok_ch / (ms * 1e-3) / 1e9, 3), algorithmic_bytes=nbytes,
                causal_gflop=round(2 * macs / 1e9, 3),
                executed_gflop=round(2 * macs_exec / 1e9, 3),
                executed_tflops=round(2 * macs_exec / (ms * 1e-3) / 1e12, 2),
                roofline=roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", traffic, note,
                                  kernel="ssd_chunk_kernel (the only kernel of the call)"),
                mfma_view=roofline("mfma", 2 * macs / (ms * 1e-3) / 1e12, BF16_MFMA_PEAK_TFLOPS,
                                   "TFLOP/s"))


def bench_decode(args, ctx):
    torch, ssm, W = ctx["torch"], ctx["ssm"], ctx["W"]
    w = W.S6_DECODE_2P8B
    t = W.make_step_inputs(w, seed=0)
    d = {k: (v.to("cuda:0") if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    y = torch.empty((w.B, w.D), dtype=torch.bfloat16, device="cuda:0")

    def step():
        ssm.selective_state_update(d["state"], d["u"], d["delta"], d["A"], d["B"], d["C"],
                                   D=d["D"], z=d["z"], delta_bias=d["delta_bias"], out=y)

    ms = ctx["timer"].run(step, args.steps, args.warmup, ctx["flusher"].clean)["mean"]
    nbytes = W.step_algorithmic_bytes(w)
    return dict(status="ok", workload=w.name, ms=round(ms, 5), algorithmic_bytes=nbytes,
                gbs=round(nbytes / (ms * 1e-3) / 1e9, 2),
                pct_hbm_peak=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS * 100, 2),
                state_updates_per_s=round(w.B * w.D * w.N / (ms * 1e-3), 1))


def bench_bwd(args, ctx, long=False):
    """The backward at the Mamba-130M layer, or (long) at the long fp32
    sequence, where the planner cuts the sequence into segments."""
    torch, ssm, W = ctx["torch"], ctx["ssm"], ctx["W"]
    w = W.S6_LONG_FP32 if long else W.S6_MAMBA130M
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    t = W.make_s6_inputs(w, seed=0)
    d = {k: (v.to("cuda:0") if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    g = torch.Generator().manual_seed(1)
    dy = torch.randn(w.B, w.L, w.D, generator=g).to(dt).to("cuda:0")
    lib = ssm._native.load()
    code = 0 if dt == torch.float32 else 1
    need = int(lib.ssm_selective_scan_bwd_workspace_bytes(w.B, w.L, w.D, w.N, code))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")

    def step():
        ssm.selective_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], dy, D=d["D"],
                               z=d["z"], delta_bias=d["delta_bias"], workspace=ws)

    ms = ctx["timer"].run(step, args.steps, args.warmup, ctx["flusher"].clean)["mean"]
    e = 2 if dt == torch.bfloat16 else 4
    # inputs u, delta, (z,) dy, B, C read and du, ddelta, (dz) written once;
    # dB, dC fp32; A, dA and the per-channel vectors are negligible
    acts = 7 if w.gate else 5
    nbytes = acts * w.B * w.L * w.D * e + 2 * w.B * w.L * w.N * (e + 4)
    return dict(status="ok", workload=w.name, ms=round(ms, 5), algorithmic_bytes=nbytes,
                gbs=round(nbytes / (ms * 1e-3) / 1e9, 2),
                gtokch=round(w.tok_ch / (ms * 1e-3) / 1e9, 3), workspace_bytes=need,
                segments=int(lib.ssm_selective_scan_bwd_segments(w.B, w.L, w.D, w.N)))


def bench_train(args, ctx, long=False):
    """Forward and backward of one training step at the Mamba-130M layer (or,
    long, at the long fp32 sequence), two ways: the plain forward then the
    self-contained backward (which starts with its own forward sweep), and the
    forward that saves the 16-token checkpoints then the backward that takes
    them.  Each call alone and each pair as one timed step."""
    torch, ssm, W = ctx["torch"], ctx["ssm"], ctx["W"]
    w = W.S6_LONG_FP32 if long else W.S6_MAMBA130M
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    code = 0 if dt == torch.float32 else 1
    t = W.make_s6_inputs(w, seed=0)
    d = {k: (v.to("cuda:0") if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    g = torch.Generator().manual_seed(1)
    dy = torch.randn(w.B, w.L, w.D, generator=g).to(dt).to("cuda:0")
    lib = ssm._native.load()
    y = torch.empty_like(d["u"])
    ck = torch.empty((w.B, w.D, (w.L + 15) // 16, w.N), dtype=torch.float32, device="cuda:0")
    ws_full = torch.empty(int(lib.ssm_selective_scan_bwd_workspace_bytes(w.B, w.L, w.D, w.N, code)),
                          dtype=torch.uint8, device="cuda:0")
    ws_part = torch.empty(int(lib.ssm_selective_scan_bwd_ckpt_workspace_bytes(w.B, w.L, w.D, w.N, code)),
                          dtype=torch.uint8, device="cuda:0")
    ws_fwd = torch.empty(max(1, int(lib.ssm_selective_scan_workspace_bytes(w.B, w.L, w.D, w.N, code))),
                         dtype=torch.uint8, device="cuda:0")
    kw = dict(D=d["D"], z=d["z"], delta_bias=d["delta_bias"])
    args_in = (d["u"], d["delta"], d["A"], d["B"], d["C"])

    def fwd():
        ssm.selective_scan_fwd(*args_in, **kw, return_last_state=False, out=y, workspace=ws_fwd)

    def fwd_ckpt():
        ssm.selective_scan_fwd_ckpt(*args_in, **kw, return_last_state=False, out=y, ckpt=ck,
                                    workspace=ws_fwd)

    def bwd():
        ssm.selective_scan_bwd(*args_in, dy, **kw, workspace=ws_full)

    def bwd_ckpt():
        ssm.selective_scan_bwd(*args_in, dy, **kw, workspace=ws_part, ckpt=ck)

    def run(fn):
        return round(ctx["timer"].run(fn, args.steps, args.warmup, ctx["flusher"].clean)["mean"], 5)

    res = dict(status="ok", workload=w.name, ckpt_bytes=ck.numel() * 4)
    res["ms_fwd_ckpt"] = run(fwd_ckpt)
    res["ms_bwd_ckpt"] = run(bwd_ckpt)
    res["ms_fwd_then_bwd_ckpt"] = run(lambda: (fwd_ckpt(), bwd_ckpt()))
    res["ms_fwd_then_bwd"] = run(lambda: (fwd(), bwd()))
    res["ms"] = res["ms_fwd_then_bwd_ckpt"]
    return res


def bench_conv(args, ctx):
    torch, ssm, W = ctx["torch"], ctx["ssm"], ctx["W"]
    w = W.CONV_MAMBA130M
    t = W.make_conv_inputs(w, seed=0)
    d = {k: v.to("cuda:0") for k, v in t.items()}
    u = torch.empty_like(d["x"])

    def step():
        ssm.causal_conv1d_silu(d["x"], d["weight"], d["bias"], out=u)

    ms = ctx["timer"].run(step, args.steps, args.warmup, ctx["flusher"].clean)["mean"]
    nbytes = W.conv_algorithmic_bytes(w)
    return dict(status="ok", workload=w.name, ms=round(ms, 5), algorithmic_bytes=nbytes,
                gbs=round(nbytes / (ms * 1e-3) / 1e9, 2),
                pct_hbm_peak=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS * 100, 2))


def bench_conv_scan(args, ctx):
    """The conv1d + SiLU fused in front of the S6 scan, on the Mamba-130M layer
    shape with a K = 4 convolution: x replaces u as the input, so the
    algorithmic bytes are those of the scan plus the convolution weights."""
    torch, ssm, W = ctx["torch"], ctx["ssm"], ctx["W"]
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

    ms = ctx["timer"].run(step, args.steps, args.warmup, ctx["flusher"].clean)["mean"]
    nbytes = W.s6_algorithmic_bytes(w) + W.CONV_MAMBA130M.D * (W.CONV_MAMBA130M.K + 1) * 4
    return dict(status="ok", workload=w.name + "+conv1d_k4", ms=round(ms, 5),
                algorithmic_bytes=nbytes, gbs=round(nbytes / (ms * 1e-3) / 1e9, 2),
                gtokch=round(w.tok_ch / (ms * 1e-3) / 1e9, 3))


def bench_copy(args, ctx, nbytes):
    """A plain device copy moving `nbytes` in total (nbytes/2 read, nbytes/2
    written), flushed and timed like the scan: the practical ceiling."""
    torch = ctx["torch"]
    n = nbytes // 8
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    res = ctx["timer"].run(lambda: dst.copy_(src), args.steps, max(3, args.warmup // 4),
                           ctx["flusher"].clean)
    del src, dst
    return dict(bytes_moved=8 * n, ms=round(res["mean"], 5),
                gbs=round(8 * n / (res["mean"] * 1e-3) / 1e9, 2))


# ------------------------------------------------------------------ CPU leg
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _sample_channels(w, rng, per_b=16):
    bs = sorted(set([0, w.B - 1]))
    return [(b, sorted(set([0, w.D - 1] + list(rng.choice(w.D, size=per_b, replace=False)))))
            for b in bs]


def verify_outputs(ctx):
    """Sampled channels (S6) or (batch, head) pairs (SSD) of each timed call's
    output against the fp64 oracle, normwise max relative error."""
    import numpy as np
    import oracle
    out = {}
    for kind, w, t, samples, ys, hs in ctx["verify"]:
        yr, hr = [], []
        if kind == "s6":
            for b, ds in samples:
                yo, ho = oracle.s6_fwd(
                    t["u"][b:b + 1, :, ds], t["delta"][b:b + 1, :, ds], t["A"][ds],
                    t["B"][b:b + 1], t["C"][b:b + 1],
                    D=None if t["D"] is None else t["D"][ds],
                    z=None if t["z"] is None else t["z"][b:b + 1, :, ds],
                    delta_bias=None if t["delta_bias"] is None else t["delta_bias"][ds])
                yr.append(yo[0]); hr.append(ho[0])
            g, r = np.concatenate([v.numpy() for v in ys], 1), np.concatenate(yr, 1)
            gh, rh = np.concatenate([v.numpy() for v in hs], 0), np.concatenate(hr, 0)
            what = f"{sum(len(ds) for _, ds in samples)} sampled channels"
        else:
            for b, hh in samples:
                gg = hh // (w.H // w.G)
                Yo, ho = oracle.ssd_fwd(t["X"][b:b + 1, :, hh:hh + 1],
                                        t["delta"][b:b + 1, :, hh:hh + 1], t["A"][hh:hh + 1],
                                        t["B"][b:b + 1, :, gg:gg + 1],
                                        t["C"][b:b + 1, :, gg:gg + 1])
                yr.append(Yo[0, :, 0]); hr.append(ho[0, 0])
            g, r = np.stack([v.numpy() for v in ys]), np.stack(yr)
            gh, rh = np.stack([v.numpy() for v in hs]), np.stack(hr)
            what = f"{len(samples)} sampled (batch, head) pairs"
        err_y = float(np.max(np.abs(g - r)) / np.max(np.abs(r)))
        err_h = float(np.max(np.abs(gh - rh)) / np.max(np.abs(rh)))
        tol = 1e-5 if w.dtype == "f32" else 2e-2
        out[w.name] = {"sample": what, "err_y": float(f"{err_y:.3e}"),
                       "err_h_last": float(f"{err_h:.3e}"), "tol": tol,
                       "ok": bool(err_y <= tol and err_h <= max(tol, 1e-5))}
    return out


def cpu_baseline(r, ctx, seconds=8.0):
    """The fp64 oracle (as it stands, untuned) on the host: on all cores over
    the whole headline workload, and on one thread over a slice of it, each
    repeated until `seconds` of wall time; value = algorithmic bytes per
    workload / mean seconds per workload (the slice scaled to the whole)."""
    import oracle
    torch = ctx["torch"]
    W = ctx["W"]
    w, t = r["w"], r["t"]
    f64 = {k: (oracle._f64(v) if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    threads = oracle.default_threads()

    def run(sub, th):
        runs, t0 = 0, time.perf_counter()
        while True:
            oracle.s6_fwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], D=sub["D"],
                          z=sub["z"], delta_bias=sub["delta_bias"], threads=th)
            runs += 1
            if time.perf_counter() - t0 >= seconds:
                return runs, time.perf_counter() - t0

    runs, total = run(f64, threads)
    sec_all = total / runs
    nd = 256
    sl = {"u": f64["u"][:1, :, :nd], "delta": f64["delta"][:1, :, :nd], "A": f64["A"][:nd],
          "B": f64["B"][:1], "C": f64["C"][:1], "D": f64["D"][:nd], "z": f64["z"][:1, :, :nd],
          "delta_bias": f64["delta_bias"][:nd]}
    sl = {k: (v.copy() if hasattr(v, "copy") else v) for k, v in sl.items()}
    runs1, total1 = run(sl, 1)
    frac = (1 * w.L * nd) / w.tok_ch
    sec_one = total1 / runs1 / frac
    nbytes = r["nbytes"]
    return {"value": round(nbytes / sec_all / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole {w.name} workload (B={w.B} L={w.L} D={w.D} N={w.N}), run "
                      f"{runs} times ({total:.1f} s wall); fp64 sequential loop per channel, "
                      f"channels over {threads} OpenMP threads",
            "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(),
            "seconds_per_workload": round(sec_all, 4),
            "gtokch_per_s": round(w.tok_ch / sec_all / 1e9, 6),
            "single_thread": {"value": round(nbytes / sec_one / 1e9, 4), "unit": "GB/s",
                              "cores": 1,
                              "sample": f"batch row 0, channels 0..{nd - 1} (1/{round(1 / frac)} "
                                        f"of the workload), run {runs1} times "
                                        f"({total1:.1f} s); scaled to the whole workload",
                              "seconds_per_workload": round(sec_one, 3)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU reaches its steady clock after ~30-40 back-to-back calls: the
    # first calls of a cold process run ~10% slower
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-paths", action="store_true", help="the headline S6 workload only")
    ap.add_argument("--only", choices=["s6", "s6_2p8b", "s6_long", "ssd", "decode", "bwd",
                                       "bwd_long", "train", "train_long", "conv", "conv_scan",
                                       "copy"],
                    help="run one part alone and print its result")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a plain 256 MiB device copy three times, the "
                         "reference for scaling FETCH_SIZE/WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the scan is data-parallel over channels and would shard with no "
              "communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_21_amd as ssm
    from selective_state_space_21_amd import _native as native
    from selective_state_space_21_amd import workloads as W

    hip = _hip()
    ctx = dict(torch=torch, ssm=ssm, W=W, native=native, hip=hip, verify=[])
    ctx["flusher"] = Flusher(torch)
    ctx["timer"] = Timer(torch, hip)
    if args.calibration_copy:
        src = torch.ones(64 * 2**20, dtype=torch.float32, device="cuda:0")   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    parts = {"s6": lambda: bench_s6(args, ctx, W.S6_MAMBA130M, headline=True),
             "s6_2p8b": lambda: bench_s6(args, ctx, W.S6_MAMBA2P8B),
             "s6_long": lambda: bench_s6(args, ctx, W.S6_LONG_FP32),
             "ssd": lambda: bench_ssd(args, ctx), "decode": lambda: bench_decode(args, ctx),
             "bwd": lambda: bench_bwd(args, ctx), "bwd_long": lambda: bench_bwd(args, ctx, True),
             "train": lambda: bench_train(args, ctx),
             "train_long": lambda: bench_train(args, ctx, True),
             "conv": lambda: bench_conv(args, ctx),
             "conv_scan": lambda: bench_conv_scan(args, ctx),
             "copy": lambda: bench_copy(args, ctx, W.s6_algorithmic_bytes(W.S6_MAMBA130M))}
    if args.only:
        res = parts[args.only]()
        print(json.dumps({"part": args.only, **res}), flush=True)
        return
    w = W.S6_MAMBA130M
    r = bench_s6(args, ctx, w, headline=True)
    copy_same = bench_copy(args, ctx, r["algorithmic_bytes"])
    copy_big = bench_copy(args, ctx, 2 * 2**30)
    paths = {}
    if not args.no_paths:
        for name, key in [("s6_mamba2.8b_layer", "s6_2p8b"), ("s6_long_fp32", "s6_long"),
                          ("ssd_chunk_fwd", "ssd"), ("selective_state_update", "decode"),
                          ("selective_scan_bwd", "bwd"), ("selective_scan_bwd_long_fp32", "bwd_long"),
                          ("training_step_fwd_bwd", "train"),
                          ("training_step_fwd_bwd_long_fp32", "train_long"),
                          ("causal_conv1d_silu", "conv"),
                          ("selective_scan_conv_fwd", "conv_scan")]:
            paths[name] = parts[key]()
            torch.cuda.empty_cache()
    line = {
        "metric": "selective-scan fwd achieved HBM GB/s (% of peak) + Gtoken·channels/s",
        "value": r["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "L": w.L, "D": w.D, "N": w.N,
            "io_dtype": "bf16", "state_dtype": "f32", "path": r["path"],
            "segments": r["segments"], "pct_of_hbm_peak": r["pct_hbm_peak"],
            "gtoken_channels_per_s": r["gtokch"], "algorithmic_bytes": r["algorithmic_bytes"],
            "phases_ms": r["phases_ms"], "ms_median": r["ms_median"], "ms_min": r["ms_min"],
            "cache_flush": "read of a 512 MiB buffer before every timed call (clean lines)",
            "ms_per_step_dirty_flush": r["ms_dirty_flush"],
            "ms_per_step_without_cache_flush": r["ms_no_flush"],
            "copy_ceiling": {"same_bytes": copy_same, "2_GiB": copy_big,
                             "pct_of_copy_same_bytes": round(r["gbs"] / copy_same["gbs"] * 100, 2)},
        },
        "roofline": {**r["roofline"], "issue_view": r["issue"], "alu_view": r["alu_view"]},
    }
    if paths:
        line["paths"] = paths
    ok = True
    if not args.no_cpu_baseline:
        rr = dict(w=w, t=W.make_s6_inputs(w, seed=0), nbytes=r["algorithmic_bytes"])
        line["verified"] = verify_outputs(ctx)
        ok = all(v["ok"] for v in line["verified"].values())
        line["cpu_baseline"] = cpu_baseline(rr, ctx)
    print(json.dumps(line), flush=True)
    if not ok:
        sys.exit(1)


if __name__ == "__main__":
    main()
