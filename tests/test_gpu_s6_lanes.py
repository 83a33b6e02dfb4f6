"""GPU parity of the state-per-lane S6 forward (one lane per channel x state,
the whole sequence in one pass) against the fp64 oracle.  SSM_S6_SEGMENTS=1
keeps it in one pass at sizes the planner would cut into segments.  Bars
as for the split path: normwise 1e-5 (fp32), 2e-2 (bf16); bit-exact on the
integer-valued boundary cases."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_21_amd as ssm
from selective_state_space_21_amd import workloads as W

from _parity import TOL, normwise_err, s6_gpu, s6_oracle, to_dev
from test_gpu_s6 import _exact_case

pytestmark = pytest.mark.gpu


@pytest.fixture
def lanes(monkeypatch):
    # the state-per-lane kernel in one pass over the sequence (small shapes
    # would otherwise be cut into segments)
    monkeypatch.delenv("SSM_S6_LANES", raising=False)
    monkeypatch.setenv("SSM_S6_SEGMENTS", "1")


def _cmp(inp, tol=None):
    y, h = s6_gpu(inp)
    yr, hr = s6_oracle(inp)
    tol = tol if tol is not None else TOL[inp["u"].dtype]
    ey = normwise_err(y.float().cpu().numpy(), yr)
    eh = normwise_err(h.cpu().numpy(), hr)
    assert ey <= tol, f"y err {ey:.3e} > {tol}"
    assert eh <= max(tol, 1e-5), f"h_last err {eh:.3e}"
    return ey, eh


def test_planner_takes_lanes_at_the_layer_shapes(monkeypatch):
    monkeypatch.delenv("SSM_S6_SEGMENTS", raising=False)
    for w in (W.S6_MAMBA130M, W.S6_MAMBA2P8B):
        assert ssm.selective_scan_lanes(w.B, w.L, w.D, w.N)
        assert ssm.selective_scan_segments(w.B, w.L, w.D, w.N) == 1
    # too few channels to fill the chip: segments of whole super-tiles
    assert ssm.selective_scan_lanes(1, 131072, 2048, 16)
    assert ssm.selective_scan_segments(1, 131072, 2048, 16) == 12
    # D not a multiple of 16, N != 16: the split path
    assert not ssm.selective_scan_lanes(8, 2048, 1544, 16)
    assert not ssm.selective_scan_lanes(8, 2048, 1536, 8)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [1, 15, 16, 17, 127, 128, 129, 300, 1000])
def test_lengths(lanes, dtype, L):
    w = W.S6_MAMBA130M.scaled(B=2, L=L, D=48, dtype=dtype)
    assert ssm.selective_scan_lanes(w.B, w.L, w.D, w.N)
    _cmp(W.make_s6_inputs(w, seed=L))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate,skip,bias,softplus", [
    (True, True, True, True), (False, True, True, True), (True, False, False, True),
    (False, False, False, False), (True, True, False, False)])
def test_options(lanes, dtype, gate, skip, bias, softplus):
    w = W.S6_MAMBA130M.scaled(B=3, L=400, D=64, dtype=dtype)
    inp = W.make_s6_inputs(w, seed=11)
    if not gate: inp["z"] = None
    if not skip: inp["D"] = None
    if not bias: inp["delta_bias"] = None
    if not softplus:
        # raw steps must stay positive and moderate without the softplus
        inp["delta"] = (0.02 + 0.05 * inp["delta"].float().abs()).to(inp["delta"].dtype)
        inp["delta_softplus"] = False
    g = torch.Generator().manual_seed(5)
    inp["h0"] = 0.3 * torch.randn(3, 64, 16, generator=g)
    _cmp(inp)


@pytest.mark.parametrize("w", [
    W.S6_MAMBA130M.scaled(B=2, L=1000, D=192),
    W.S6_MAMBA2P8B.scaled(B=2, L=777, D=320),
    W.S6_LONG_FP32.scaled(L=5000, D=128),
], ids=lambda w: w.name)
def test_workloads_small(lanes, w):
    _cmp(W.make_s6_inputs(w, seed=0))


@pytest.mark.parametrize("mode", ["prefix", "reset", "mixed"])
@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 127, 128, 129, 255, 256, 257, 4099])
def test_bit_exact_boundaries(lanes, mode, L):
    for dtype in ("f32", "bf16"):
        inp = _exact_case(L, 96, 16, dtype, mode, seed=L * 5 + 1)
        y, h = s6_gpu(inp)
        yr, hr = s6_oracle(inp)
        assert np.all(np.abs(yr) < 256) and np.all(yr == np.round(yr))
        np.testing.assert_array_equal(y.float().cpu().numpy(), yr)
        np.testing.assert_array_equal(h.cpu().numpy(), hr)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lens", [[700, 1, 0, 333, 1000, 64], [1000, 999, 17, 128, 129, 1000]])
def test_varlen(lanes, dtype, lens):
    Bt, L, Dm = len(lens), 1000, 96
    w = W.S6_MAMBA130M.scaled(B=Bt, L=L, D=Dm, dtype=dtype)
    inp = W.make_s6_inputs(w, seed=lens[1])
    g = torch.Generator().manual_seed(3)
    inp["h0"] = 0.2 * torch.randn(Bt, Dm, 16, generator=g)
    d = to_dev(inp)
    sentinel = 7.0
    y = torch.full((Bt, L, Dm), sentinel, device="cuda").to(d["u"].dtype)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    _, h = ssm.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                                  delta_bias=d["delta_bias"], h0=d["h0"], out=y, seq_lens=sl)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    h = h.cpu().numpy()
    for b, n in enumerate(lens):
        cut = lambda t: None if t is None else t[b:b + 1, :n]
        yr, hr = oracle.s6_fwd(cut(inp["u"]), cut(inp["delta"]), inp["A"], cut(inp["B"]),
                               cut(inp["C"]), D=inp["D"], z=cut(inp["z"]),
                               delta_bias=inp["delta_bias"], h0=inp["h0"][b:b + 1])
        if n > 0:
            assert normwise_err(y[b:b + 1, :n], yr) <= TOL[w.dtype]
        assert normwise_err(h[b:b + 1], hr) <= max(TOL[w.dtype], 1e-5)
        assert np.all(y[b, n:] == sentinel)


def test_agrees_with_split_path(monkeypatch):
    w = W.S6_MAMBA130M.scaled(B=2, L=2048, D=256)
    d = to_dev(W.make_s6_inputs(w, seed=4))
    outs = []
    monkeypatch.setenv("SSM_S6_SEGMENTS", "1")
    for env in ("1", "0"):
        monkeypatch.setenv("SSM_S6_LANES", env)
        assert ssm.selective_scan_lanes(w.B, w.L, w.D, w.N) == (env == "1")
        outs.append(ssm.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                           z=d["z"], delta_bias=d["delta_bias"]))
    torch.cuda.synchronize()
    # same fp32 state update per element; only the readout's summation order differs
    assert torch.equal(outs[0][1], outs[1][1]) or normwise_err(outs[0][1].cpu(), outs[1][1].cpu()) <= 1e-6
    assert normwise_err(outs[0][0].float().cpu(), outs[1][0].float().cpu()) <= 8e-3


def test_deterministic_and_no_out_of_bounds_writes(lanes):
    w = W.S6_MAMBA130M.scaled(B=3, L=513, D=144)
    inp = to_dev(W.make_s6_inputs(w, seed=9))
    n = 3 * 513 * 144
    pad = 64
    guard = torch.full((n + 2 * pad,), 12345.0, device="cuda").to(torch.bfloat16)
    out = guard[pad:pad + n].view(3, 513, 144)
    y1, h1 = ssm.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                    D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"], out=out)
    y2, h2 = ssm.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                    D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    g = guard.float()
    assert torch.all(g[:pad] == 12352.0) and torch.all(g[pad + n:] == 12352.0)


def test_h0_chaining(lanes):
    w = W.S6_MAMBA130M.scaled(B=2, L=640, D=128)
    inp = W.make_s6_inputs(w, seed=6)
    inp["h0"] = torch.randn(2, 128, 16, generator=torch.Generator().manual_seed(0))
    d = to_dev(inp)
    y_all, h_all = ssm.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                          z=d["z"], delta_bias=d["delta_bias"], h0=d["h0"])
    cut = 200
    sl = lambda t, a, b: t[:, a:b].contiguous()
    y1, h1 = ssm.selective_scan_fwd(sl(d["u"], 0, cut), sl(d["delta"], 0, cut), d["A"],
                                    sl(d["B"], 0, cut), sl(d["C"], 0, cut), D=d["D"],
                                    z=sl(d["z"], 0, cut), delta_bias=d["delta_bias"], h0=d["h0"])
    y2, h2 = ssm.selective_scan_fwd(sl(d["u"], cut, 640), sl(d["delta"], cut, 640), d["A"],
                                    sl(d["B"], cut, 640), sl(d["C"], cut, 640), D=d["D"],
                                    z=sl(d["z"], cut, 640), delta_bias=d["delta_bias"], h0=h1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], 1), y_all)
    assert torch.equal(h2, h_all)


def test_full_lengths_equal_plain_call(lanes):
    w = W.S6_MAMBA130M.scaled(B=3, L=512, D=128)
    d = to_dev(W.make_s6_inputs(w, seed=2))
    y1, h1 = ssm.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                    z=d["z"], delta_bias=d["delta_bias"])
    y2, h2 = ssm.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                    z=d["z"], delta_bias=d["delta_bias"],
                                    seq_lens=torch.full((3,), 512, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_long_fp32_sequence_sampled(lanes):
    """The long fp32 shape (131072 tokens, 1024 super-tiles per row) forced onto
    the state-per-lane kernel; sampled channels against the oracle at the fp32
    bar."""
    from _parity import s6_oracle_sampled
    w = W.S6_LONG_FP32
    assert ssm.selective_scan_lanes(w.B, w.L, w.D, w.N)
    inp = W.make_s6_inputs(w, seed=0)
    y, h = s6_gpu(inp)
    y = y.float().cpu().numpy()
    h = h.cpu().numpy()
    ds = [0, 1, 15, 16, 511, 1024, 2047]
    ys, yr, hs, hr = [], [], [], []
    for b, dl, yo, ho in s6_oracle_sampled(inp, [(0, ds)]):
        ys.append(y[b][:, dl]); yr.append(yo)
        hs.append(h[b][dl]); hr.append(ho)
    ey = normwise_err(np.concatenate(ys, 1), np.concatenate(yr, 1))
    eh = normwise_err(np.concatenate(hs, 0), np.concatenate(hr, 0))
    assert ey <= TOL[w.dtype] and eh <= 1e-5, (ey, eh)
