"""The backward split along the sequence (segments scanned in parallel from
the state and adjoint that the carry folds from the segment pairs), forced
on shapes the oracle finishes quickly with SSM_BWD_SEGMENTS, against the
fp64 autodiff oracle at the backward's bars (fp32 gradients 1e-5, bf16-stored
ones 2e-2).  Also: the planner's own split at a long single sequence
(sampled channels), the split with the checkpoints of the training pair,
with a variable-length batch, and segment counts that do not divide the
tiles evenly."""
import numpy as np
import pytest
import torch

import selective_state_space_21_amd as ssm
from oracle.backward import s6_bwd as oracle_bwd
from selective_state_space_21_amd import workloads as W

from _parity import normwise_err, to_dev

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
        inp["delta"] = (0.01 + 0.03 * torch.rand(Bt, L, Dm, generator=g)).to(inp["u"].dtype)
        inp["delta_bias"] = None
    inp["A"] = inp["A"] * 0.05          # slow decay: the carried state and adjoint matter
    inp["h0"] = 0.5 * torch.randn(Bt, Dm, N, generator=g) if extras else None
    inp["dy"] = torch.randn(Bt, L, Dm, generator=g).to(inp["u"].dtype)
    inp["dh_last"] = torch.randn(Bt, Dm, N, generator=g) if extras else None
    return inp


def _bwd(d, **kw):
    return ssm.selective_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["dy"], D=d["D"],
                                  z=d["z"], delta_bias=d["delta_bias"],
                                  delta_softplus=d["delta_softplus"], h0=d["h0"],
                                  dh_last=d["dh_last"], **kw)


def _check(got, inp, dtype):
    ref = oracle_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["dy"], D=inp["D"],
                     z=inp["z"], delta_bias=inp["delta_bias"],
                     delta_softplus=inp["delta_softplus"], h0=inp["h0"], dh_last=inp["dh_last"])
    assert set(got) == set(ref)
    for k in ref:
        tol = 1e-5 if (k in FP32_OUT or dtype == "f32") else 2e-2
        e = normwise_err(got[k].float().cpu().numpy(), ref[k].numpy())
        assert e <= tol, f"{k}: err {e:.3e} > {tol}"


# (Bt, L, Dm, N, dtype, segments, extras, softplus)
CASES = [
    (1, 1024, 32, 16, "f32", 2, True, True),
    (2, 1500, 48, 16, "bf16", 3, True, True),
    (1, 2000, 80, 16, "f32", 7, True, False),
    (2, 777, 16, 5, "f32", 4, True, True),
    (1, 300, 96, 16, "bf16", 64, False, True),     # capped at one segment per tile
    (3, 1030, 40, 8, "bf16", 5, True, True),
]


@pytest.mark.parametrize("c", CASES, ids=lambda c: "B{}L{}D{}N{}{}S{}".format(*c[:6]))
def test_segmented_backward(c, monkeypatch):
    Bt, L, Dm, N, dtype, S, extras, softplus = c
    monkeypatch.setenv("SSM_BWD_SEGMENTS", str(S))
    inp = _inputs(Bt, L, Dm, N, dtype, extras=extras, softplus=softplus, seed=L + S)
    d = to_dev(inp)
    got = _bwd(d)
    torch.cuda.synchronize()
    _check(got, inp, dtype)


def test_segmented_backward_from_checkpoints(monkeypatch):
    # the training pair with a split backward: the carry then folds only the
    # adjoint (the checkpoints come from the forward)
    inp = _inputs(1, 1400, 64, 16, "bf16", seed=9)
    d = to_dev(inp)
    monkeypatch.setenv("SSM_S6_SEGMENTS", "1")
    _, _, ck = ssm.selective_scan_fwd_ckpt(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                           z=d["z"], delta_bias=d["delta_bias"], h0=d["h0"])
    monkeypatch.setenv("SSM_BWD_SEGMENTS", "4")
    a = _bwd(d, ckpt=ck)
    b = _bwd(d)
    torch.cuda.synchronize()
    # the self-contained call rebuilds its checkpoints from carried states,
    # which round differently from the forward's own: both against the oracle
    _check(a, inp, "bf16")
    _check(b, inp, "bf16")


def test_segmented_backward_varlen(monkeypatch):
    lens = [1100, 0, 517]
    inp = _inputs(len(lens), 1100, 32, 16, "f32", seed=21)
    padded = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    for b, n in enumerate(lens):
        for k in ("u", "delta", "B", "C", "z", "dy"):
            padded[k][b, n:] = float("nan")
    monkeypatch.setenv("SSM_BWD_SEGMENTS", "3")
    d = to_dev(padded)
    got = _bwd(d, seq_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    got = {k: v.float().cpu().numpy() for k, v in got.items()}
    summed = {}
    for b, n in enumerate(lens):
        row = lambda t: None if t is None else t[b:b + 1, :n]
        ref = oracle_bwd(row(inp["u"]), row(inp["delta"]), inp["A"], row(inp["B"]), row(inp["C"]),
                         row(inp["dy"]), D=inp["D"], z=row(inp["z"]), delta_bias=inp["delta_bias"],
                         h0=inp["h0"][b:b + 1], dh_last=inp["dh_last"][b:b + 1])
        for k in ("du", "ddelta", "dz", "dB", "dC"):
            if n > 0:
                assert normwise_err(got[k][b:b + 1, :n], ref[k].numpy()) <= 1e-5, (k, b)
            assert np.all(got[k][b, n:] == 0.0), (k, b)
        assert normwise_err(got["dh0"][b:b + 1], ref["dh0"].numpy()) <= 1e-5, b
        for k in ("dA", "dD", "ddelta_bias"):
            summed[k] = summed.get(k, 0.0) + ref[k].numpy().astype(np.float64)
    for k, v in summed.items():
        assert normwise_err(got[k], v) <= 1e-5, k


def test_long_single_sequence(monkeypatch):
    # B = 1, L = 8192, D = 512 (11 adjoint-sweep workgroups): the planner's
    # own split (8 segments), sampled channels against the oracle
    monkeypatch.delenv("SSM_BWD_SEGMENTS", raising=False)
    Bt, L, Dm = 1, 8192, 512
    assert ssm.selective_scan_bwd_segments(Bt, L, Dm, 16) > 1
    inp = _inputs(Bt, L, Dm, 16, "f32", seed=5)
    d = to_dev(inp)
    got = _bwd(d)
    torch.cuda.synchronize()
    chans = [0, 100, 300, 511]
    sub = {k: (v[..., chans] if k in ("u", "delta", "z", "dy") else v) for k, v in inp.items()}
    for k in ("A",):
        sub[k] = inp[k][chans]
    for k in ("D", "delta_bias"):
        sub[k] = None if inp[k] is None else inp[k][chans]
    for k in ("h0", "dh_last"):
        sub[k] = None if inp[k] is None else inp[k][:, chans]
    ref = oracle_bwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["dy"], D=sub["D"],
                     z=sub["z"], delta_bias=sub["delta_bias"], delta_softplus=True, h0=sub["h0"],
                     dh_last=sub["dh_last"])
    pick = {"du": (..., chans), "ddelta": (..., chans), "dz": (..., chans), "dA": (chans,),
            "dD": (chans,), "ddelta_bias": (chans,), "dh0": (slice(None), chans)}
    for k, idx in pick.items():
        g = got[k].float().cpu()[idx].numpy()
        assert normwise_err(g, ref[k].numpy()) <= 1e-5, k


def _draw(i):
    r = np.random.default_rng(5000 + i)
    return dict(Bt=int(r.integers(1, 4)), L=int(r.integers(1100, 2500)), Dm=int(r.integers(1, 120)),
                N=int(r.choice([1, 4, 8, 13, 16])), dtype=str(r.choice(["f32", "bf16"])),
                S=int(r.integers(2, 21)), extras=bool(r.random() < 0.7),
                softplus=bool(r.random() < 0.8), seed=i)


RANDOM = [_draw(i) for i in range(12)]


@pytest.mark.parametrize("c", RANDOM, ids=lambda c: "B{Bt}L{L}D{Dm}N{N}{dtype}S{S}".format(**c))
def test_random_segmented_backward(c, monkeypatch):
    monkeypatch.setenv("SSM_BWD_SEGMENTS", str(c["S"]))
    inp = _inputs(c["Bt"], c["L"], c["Dm"], c["N"], c["dtype"], extras=c["extras"],
                  softplus=c["softplus"], seed=c["seed"])
    assert ssm.selective_scan_bwd_segments(c["Bt"], c["L"], c["Dm"], c["N"]) > 1
    d = to_dev(inp)
    got = _bwd(d)
    torch.cuda.synchronize()
    _check(got, inp, c["dtype"])
