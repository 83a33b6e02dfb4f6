"""Helpers shared by the GPU parity tests: move inputs to the device, call the
HIP path through the C ABI, call the oracle (possibly on a sample of
channels), and the normwise error metric.

Metric: err = max_i |gpu_i - ref_i| / max_i |ref_i| over the compared
elements.  Elementwise relative error is unbounded where y crosses zero, so
the bar is normwise: 1e-5 for fp32 storage, 2e-2 for bf16 storage with fp32
state.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import selective_state_space_21_amd as ssm

TOL = {"f32": 1e-5, torch.float32: 1e-5, "bf16": 2e-2, torch.bfloat16: 2e-2}


def normwise_err(gpu, ref) -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    scale = np.max(np.abs(r))
    diff = np.max(np.abs(g - r))
    if scale == 0.0:
        return float(diff)
    return float(diff / scale)


def to_dev(inp: dict, device="cuda") -> dict:
    out = {}
    for k, v in inp.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


def s6_gpu(inp: dict, zoh=False, **kw):
    d = to_dev(inp)
    y, h = ssm.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                  z=d["z"], delta_bias=d["delta_bias"],
                                  delta_softplus=d["delta_softplus"], zoh=zoh, h0=d["h0"], **kw)
    torch.cuda.synchronize()
    return y, h


def s6_oracle(inp: dict, zoh=False):
    return oracle.s6_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                         z=inp["z"], delta_bias=inp["delta_bias"],
                         delta_softplus=inp["delta_softplus"], zoh=zoh, h0=inp["h0"])


def s6_oracle_sampled(inp: dict, samples):
    """Oracle on a list of (b, [d...]) channel groups; returns a list of
    (b, ds, y [L, nd], h_last [nd, N])."""
    res = []
    for b, ds in samples:
        ds = list(ds)
        sub = dict(
            u=inp["u"][b:b + 1, :, ds], delta=inp["delta"][b:b + 1, :, ds],
            A=inp["A"][ds], B=inp["B"][b:b + 1], C=inp["C"][b:b + 1],
            D=None if inp["D"] is None else inp["D"][ds],
            z=None if inp["z"] is None else inp["z"][b:b + 1, :, ds],
            delta_bias=None if inp["delta_bias"] is None else inp["delta_bias"][ds],
            h0=None if inp["h0"] is None else inp["h0"][b:b + 1, ds],
            delta_softplus=inp["delta_softplus"])
        y, h = s6_oracle(sub)
        res.append((b, ds, y[0], h[0]))
    return res


def ssd_gpu(inp: dict, chunk=None, **kw):
    d = to_dev(inp)
    Y, h = ssm.ssd_chunk_fwd(d["X"], d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                             delta_bias=d["delta_bias"], delta_softplus=d["delta_softplus"],
                             h0=d["h0"], chunk=chunk or d["chunk"], **kw)
    torch.cuda.synchronize()
    return Y, h


def ssd_oracle(inp: dict):
    return oracle.ssd_fwd(inp["X"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                          z=inp["z"], delta_bias=inp["delta_bias"],
                          delta_softplus=inp["delta_softplus"], h0=inp["h0"])


def ssd_oracle_sampled(inp: dict, pairs):
    """Oracle on selected (b, h) pairs; returns list of (b, h, Y [L, P], h_last [P, N])."""
    H = inp["X"].shape[2]
    G = inp["B"].shape[2]
    res = []
    for b, h in pairs:
        g = h // (H // G)
        sub = dict(
            X=inp["X"][b:b + 1, :, h:h + 1], delta=inp["delta"][b:b + 1, :, h:h + 1],
            A=inp["A"][h:h + 1], B=inp["B"][b:b + 1, :, g:g + 1], C=inp["C"][b:b + 1, :, g:g + 1],
            D=None if inp["D"] is None else inp["D"][h:h + 1],
            z=None if inp["z"] is None else inp["z"][b:b + 1, :, h:h + 1],
            delta_bias=None if inp["delta_bias"] is None else inp["delta_bias"][h:h + 1],
            h0=None if inp["h0"] is None else inp["h0"][b:b + 1, h:h + 1],
            delta_softplus=inp["delta_softplus"])
        Y, hl = ssd_oracle(sub)
        res.append((b, h, Y[0, :, 0], hl[0, 0]))
    return res
