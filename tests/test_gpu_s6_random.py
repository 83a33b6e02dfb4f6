"""Randomised S6 parity sweep against the fp64 oracle.

A fixed list of cases drawn from one seeded generator: batch rows, sequence
length, channels (multiples of 16 for the state-per-lane path, others for the
split path), state size, storage dtype, the optional inputs (gate, skip,
bias, h0), softplus on or off, a forced segment count, and per-row lengths.
Each case is compared element by element with the oracle at the bars of the
other S6 tests (normwise 1e-5 fp32, 2e-2 bf16); rows past their length must
be left untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_21_amd as ssm
from selective_state_space_21_amd import workloads as W

from _parity import TOL, normwise_err, to_dev

pytestmark = pytest.mark.gpu


def _draw(i):
    r = np.random.default_rng(1000 + i)
    lanes = bool(r.random() < 0.7)
    D = 16 * int(r.integers(1, 13)) if lanes else int(r.integers(1, 200))
    N = 16 if lanes else int(r.choice([1, 4, 8, 16, 24, 32]))
    case = dict(
        B=int(r.integers(1, 5)), L=int(r.integers(1, 3000)), D=D, N=N,
        dtype=str(r.choice(["f32", "bf16"])), gate=bool(r.random() < 0.5),
        skip=bool(r.random() < 0.5), bias=bool(r.random() < 0.5), h0=bool(r.random() < 0.5),
        softplus=bool(r.random() < 0.8), segments=int(r.choice([0, 1, 2, 3, 7, 16, 40])),
        varlen=bool(r.random() < 0.3), a_scale=float(r.choice([0.02, 1.0, 5.0])), seed=i)
    return case


CASES = [_draw(i) for i in range(40)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{B}L{L}D{D}N{N}{dtype}S{segments}".format(**c))
def test_random_case(case, monkeypatch):
    c = case
    if c["segments"]:
        monkeypatch.setenv("SSM_S6_SEGMENTS", str(c["segments"]))
    else:
        monkeypatch.delenv("SSM_S6_SEGMENTS", raising=False)
    monkeypatch.delenv("SSM_S6_LANES", raising=False)
    w = W.S6_MAMBA130M.scaled(B=c["B"], L=c["L"], D=c["D"], N=c["N"], dtype=c["dtype"],
                              gate=c["gate"], skip="normal" if c["skip"] else None,
                              bias_range=(-4.0, -2.0) if c["bias"] else None)
    inp = W.make_s6_inputs(w, seed=c["seed"])
    g = torch.Generator().manual_seed(c["seed"])
    inp["A"] = inp["A"] * c["a_scale"]
    if not c["softplus"]:
        # delta used as the step itself: positive and small
        inp["delta"] = (0.01 + 0.05 * torch.rand(c["B"], c["L"], c["D"], generator=g)).to(inp["u"].dtype)
        inp["delta_bias"] = None
    h0 = 0.3 * torch.randn(c["B"], c["D"], c["N"], generator=g) if c["h0"] else None
    lens = ([int(x) for x in torch.randint(0, c["L"] + 1, (c["B"],), generator=g)]
            if c["varlen"] else [c["L"]] * c["B"])
    d = to_dev(inp)
    sentinel = 5.0
    y = torch.full((c["B"], c["L"], c["D"]), sentinel, device="cuda").to(d["u"].dtype)
    kw = {}
    if c["varlen"]:
        kw["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device="cuda")
    _, h = ssm.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                                  delta_bias=d["delta_bias"], delta_softplus=c["softplus"],
                                  h0=None if h0 is None else h0.cuda(), out=y, **kw)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    h = h.cpu().numpy()
    tol = TOL[c["dtype"]]
    for b, n in enumerate(lens):
        cut = lambda t: None if t is None else t[b:b + 1, :n]
        yr, hr = oracle.s6_fwd(cut(inp["u"]), cut(inp["delta"]), inp["A"], cut(inp["B"]),
                               cut(inp["C"]), D=inp["D"], z=cut(inp["z"]),
                               delta_bias=inp["delta_bias"], delta_softplus=c["softplus"],
                               h0=None if h0 is None else h0[b:b + 1])
        if n > 0:
            assert normwise_err(y[b:b + 1, :n], yr) <= tol, (b, n)
        assert normwise_err(h[b:b + 1], hr) <= max(tol, 1e-5), (b, n)
        assert np.all(y[b, n:] == sentinel), (b, n)
