"""The training pair ssm_selective_scan_fwd_ckpt / ssm_selective_scan_bwd_ckpt.

The forward call must return exactly what the plain forward returns and, in
ckpt[b, d, k], the state before token 16k.  Those states are checked three
ways: against the oracle run on each 16-token prefix (its h_last), between
the path where the one-pass state-per-lane scan stores them itself and the
path where the backward's own forward sweep writes them (bit for bit), and
through the backward: gradients from the checkpoints must equal those of the
self-contained backward bit for bit (where the forward is one pass: the
segmented scan's checkpoints, completed by its fix-up, round differently),
and the oracle's at the usual bars.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_21_amd as ssm
from oracle.backward import s6_bwd as oracle_bwd
from selective_state_space_21_amd import workloads as W

from _parity import TOL, normwise_err, to_dev

pytestmark = pytest.mark.gpu

FP32_OUT = {"dA", "dB", "dC", "dD", "ddelta_bias", "dh0"}


def _inputs(Bt, L, Dm, N, dtype, extras=True, softplus=True, seed=0):
    w = W.S6_MAMBA130M.scaled(B=Bt, L=L, D=Dm, N=N, dtype=dtype, gate=extras,
                              skip="normal" if extras else None,
                              bias_range=(-4.0, -2.0) if extras else None)
    inp = W.make_s6_inputs(w, seed=seed)
    g = torch.Generator().manual_seed(seed)
    inp["delta_softplus"] = softplus
    if not softplus:
        inp["delta"] = (0.02 + 0.05 * torch.rand(Bt, L, Dm, generator=g)).to(inp["u"].dtype)
        inp["delta_bias"] = None
    inp["h0"] = 0.5 * torch.randn(Bt, Dm, N, generator=g) if extras else None
    inp["dy"] = torch.randn(Bt, L, Dm, generator=g).to(inp["u"].dtype)
    inp["dh_last"] = torch.randn(Bt, Dm, N, generator=g) if extras else None
    return inp


def _fwd(d, ckpt):
    kw = dict(D=d["D"], z=d["z"], delta_bias=d["delta_bias"], delta_softplus=d["delta_softplus"],
              h0=d["h0"])
    if ckpt:
        return ssm.selective_scan_fwd_ckpt(d["u"], d["delta"], d["A"], d["B"], d["C"], **kw)
    return ssm.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], **kw)


def _bwd(d, ckpt=None):
    return ssm.selective_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["dy"], D=d["D"],
                                  z=d["z"], delta_bias=d["delta_bias"],
                                  delta_softplus=d["delta_softplus"], h0=d["h0"],
                                  dh_last=d["dh_last"], ckpt=ckpt)


# (Bt, L, Dm, N, dtype, environment): with one segment (forced for these
# small shapes) the state-per-lane scan stores the checkpoints itself;
# segmented, split-path and other state sizes get them from the backward's
# sweep
ONE = {"SSM_S6_SEGMENTS": "1"}
CASES = [
    (3, 200, 32, 16, "bf16", ONE),          # ragged last tile and super-tile
    (2, 513, 48, 16, "f32", ONE),
    (1, 1, 16, 16, "bf16", ONE),
    (2, 16, 16, 16, "f32", ONE),
    (2, 700, 32, 16, "bf16", {"SSM_S6_SEGMENTS": "3"}),
    (2, 300, 32, 16, "bf16", {}),           # the planner's segments
    (2, 300, 40, 16, "bf16", {}),           # split path: D not a multiple of 16
    (2, 300, 32, 16, "f32", {"SSM_S6_LANES": "0"}),
    (3, 150, 24, 5, "f32", {}),
]


def _env(monkeypatch, env):
    for k in ("SSM_S6_SEGMENTS", "SSM_S6_LANES"):
        monkeypatch.delenv(k, raising=False)
    for k, v in env.items():
        monkeypatch.setenv(k, v)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}L{}D{}N{}{}{}".format(*c[:5], "".join(f"_{k[7:]}{v}" for k, v in c[5].items())))
def test_fwd_ckpt_outputs_and_states(case, monkeypatch):
    Bt, L, Dm, N, dtype, env = case
    _env(monkeypatch, env)
    inp = _inputs(Bt, L, Dm, N, dtype, seed=L)
    d = to_dev(inp)
    y0, h0l = _fwd(d, False)
    y, hl, ck = _fwd(d, True)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(hl, h0l)
    nck = (L + 15) // 16
    assert tuple(ck.shape) == (Bt, Dm, nck, N)
    ck = ck.cpu().numpy()
    h0 = np.zeros((Bt, Dm, N), np.float32) if inp["h0"] is None else inp["h0"].numpy()
    assert np.array_equal(ck[:, :, 0], h0)
    tol = max(TOL[dtype], 1e-5)
    for k in range(1, nck):
        cut = lambda t: None if t is None else t[:, :16 * k]
        _, hr = oracle.s6_fwd(cut(inp["u"]), cut(inp["delta"]), inp["A"], cut(inp["B"]),
                              cut(inp["C"]), D=inp["D"], z=cut(inp["z"]),
                              delta_bias=inp["delta_bias"], delta_softplus=inp["delta_softplus"],
                              h0=inp["h0"])
        assert normwise_err(ck[:, :, k], hr) <= tol, k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("softplus", [True, False])
def test_fused_checkpoints_equal_the_sweep(dtype, softplus, monkeypatch):
    # the one-pass scan's stores and the backward's sweep give the same bits
    inp = _inputs(2, 333, 64, 16, dtype, softplus=softplus, seed=7)
    d = to_dev(inp)
    _env(monkeypatch, ONE)
    assert ssm.selective_scan_lanes(2, 333, 64, 16) and ssm.selective_scan_segments(2, 333, 64, 16) == 1
    _, _, fused = _fwd(d, True)
    _env(monkeypatch, {"SSM_S6_LANES": "0"})
    _, _, swept = _fwd(d, True)
    torch.cuda.synchronize()
    assert torch.equal(fused, swept)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}L{}D{}N{}{}{}".format(*c[:5], "".join(f"_{k[7:]}{v}" for k, v in c[5].items())))
def test_bwd_ckpt_equals_bwd_and_oracle(case, monkeypatch):
    Bt, L, Dm, N, dtype, env = case
    _env(monkeypatch, env)
    inp = _inputs(Bt, L, Dm, N, dtype, seed=L + 1)
    d = to_dev(inp)
    _, _, ck = _fwd(d, True)
    got = _bwd(d, ckpt=ck)
    ref_gpu = _bwd(d)
    torch.cuda.synchronize()
    assert set(got) == set(ref_gpu)
    # the segmented scan's checkpoints (completed by the fix-up) round
    # differently from the backward's one-pass sweep; elsewhere they agree
    if not (ssm.selective_scan_lanes(Bt, L, Dm, N) and ssm.selective_scan_segments(Bt, L, Dm, N) > 1):
        for k in got:
            assert torch.equal(got[k], ref_gpu[k]), k
    ref = oracle_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["dy"], D=inp["D"],
                     z=inp["z"], delta_bias=inp["delta_bias"],
                     delta_softplus=inp["delta_softplus"], h0=inp["h0"], dh_last=inp["dh_last"])
    for k in ref:
        tol = 1e-5 if (k in FP32_OUT or dtype == "f32") else 2e-2
        e = normwise_err(got[k].float().cpu().numpy(), ref[k].numpy())
        assert e <= tol, f"{k}: err {e:.3e} > {tol}"


def test_empty_sequence():
    inp = _inputs(2, 0, 32, 16, "bf16")
    d = to_dev(inp)
    y, hl, ck = _fwd(d, True)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 32) and ck.shape == (2, 32, 0, 16)
    assert torch.equal(hl, d["h0"])
    g = _bwd(d, ckpt=ck)
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], d["dh_last"])


def test_full_size_training_pair():
    # Mamba-130M layer: the fused checkpoints drive a backward equal bit for
    # bit to the self-contained one, and the forward's y is unchanged
    w = W.S6_MAMBA130M
    inp = W.make_s6_inputs(w, seed=3)
    g = torch.Generator().manual_seed(3)
    inp["dy"] = torch.randn(w.B, w.L, w.D, generator=g).to(torch.bfloat16)
    inp["dh_last"] = None
    d = to_dev(inp)
    assert ssm.selective_scan_lanes(w.B, w.L, w.D, w.N) and ssm.selective_scan_segments(w.B, w.L, w.D, w.N) == 1
    y0, _ = _fwd(d, False)
    y, _, ck = _fwd(d, True)
    a = _bwd(d, ckpt=ck)
    b = _bwd(d)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def _draw(i):
    r = np.random.default_rng(4000 + i)
    return dict(Bt=int(r.integers(1, 5)), L=int(r.integers(1, 1500)), Dm=16 * int(r.integers(1, 9)),
                dtype=str(r.choice(["f32", "bf16"])), extras=bool(r.random() < 0.6),
                softplus=bool(r.random() < 0.8), seed=i)


RANDOM = [_draw(i) for i in range(16)]


@pytest.mark.parametrize("c", RANDOM, ids=lambda c: "B{Bt}L{L}D{Dm}{dtype}".format(**c))
def test_random_fused_training_pair(c, monkeypatch):
    # one segment forced, so the state-per-lane scan stores the checkpoints:
    # they must equal the sweep's, and the pair must reproduce the plain
    # forward and the self-contained backward bit for bit
    inp = _inputs(c["Bt"], c["L"], c["Dm"], 16, c["dtype"], extras=c["extras"],
                  softplus=c["softplus"], seed=c["seed"])
    d = to_dev(inp)
    _env(monkeypatch, ONE)
    y0, h0l = _fwd(d, False)
    y, hl, ck = _fwd(d, True)
    got = _bwd(d, ckpt=ck)
    ref = _bwd(d)
    _env(monkeypatch, {"SSM_S6_LANES": "0"})
    _, _, swept = _fwd(d, True)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(hl, h0l)
    assert torch.equal(ck, swept)
    for k in ref:
        assert torch.equal(got[k], ref[k]), k


@pytest.mark.parametrize("softplus", [True, False])
def test_segmented_scan_checkpoints(softplus, monkeypatch):
    # the segmented state-per-lane scan stores each segment's states from
    # zero and the fix-up completes them: slow decay (A scaled down), so the
    # incoming state reaches across whole segments, fp32 at the fp32 bar
    _env(monkeypatch, {})
    Bt, L, Dm, N = 1, 2000, 32, 16
    assert ssm.selective_scan_lanes(Bt, L, Dm, N) and ssm.selective_scan_segments(Bt, L, Dm, N) > 4
    inp = _inputs(Bt, L, Dm, N, "f32", softplus=softplus, seed=13)
    inp["A"] = inp["A"] * 0.02
    d = to_dev(inp)
    y0, h0l = _fwd(d, False)
    y, hl, ck = _fwd(d, True)
    got = _bwd(d, ckpt=ck)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(hl, h0l)
    ck = ck.cpu().numpy()
    for k in range(0, (L + 15) // 16, 5):
        cut = lambda t: None if t is None else t[:, :16 * k]
        _, hr = oracle.s6_fwd(cut(inp["u"]), cut(inp["delta"]), inp["A"], cut(inp["B"]),
                              cut(inp["C"]), D=inp["D"], z=cut(inp["z"]),
                              delta_bias=inp["delta_bias"], delta_softplus=softplus,
                              h0=inp["h0"])
        assert normwise_err(ck[:, :, k], hr) <= 1e-5, k
    ref = oracle_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["dy"], D=inp["D"],
                     z=inp["z"], delta_bias=inp["delta_bias"], delta_softplus=softplus,
                     h0=inp["h0"], dh_last=inp["dh_last"])
    for k in ref:
        assert normwise_err(got[k].float().cpu().numpy(), ref[k].numpy()) <= 1e-5, k
