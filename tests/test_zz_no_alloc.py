"""The allocation-free S6 entry point (ssm_selective_scan_fwd_noalloc) against
the ordinary one, through the C ABI: same kernels, so bit-identical results,
on two calls in a row (the second smaller) whose plans cut the sequence into
segments and so use the library's static scratch.  Both calls run in one process, the second
after the first left its pairs in the scratch."""
import ctypes

import pytest
import torch

import selective_state_space_21_amd as ssm
from selective_state_space_21_amd import _native
from selective_state_space_21_amd import workloads as W

pytestmark = pytest.mark.gpu


def _both(w, seed, monkeypatch, segments=None, split=False):
    if segments:
        monkeypatch.setenv("SSM_S6_SEGMENTS", str(segments))
    if split:
        monkeypatch.setenv("SSM_S6_LANES", "0")
    t = W.make_s6_inputs(w, seed=seed)
    d = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    assert ssm.selective_scan_lanes(w.B, w.L, w.D, w.N) == (not split)
    S = ssm.selective_scan_segments(w.B, w.L, w.D, w.N)
    assert S > 1, "the case must use the scratch (split path)"
    need = ssm.selective_scan_workspace_bytes(w.B, w.L, w.D, w.N, d["u"].dtype)
    assert 0 < need <= _native.load().ssm_selective_scan_workspace_bytes(w.B, w.L, w.D, w.N, 0) * 2
    y_ref, h_ref = ssm.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                          z=d["z"], delta_bias=d["delta_bias"])
    y = torch.full_like(y_ref, float("nan"))
    h = torch.full_like(h_ref, float("nan"))
    ssm.selective_scan_fwd_noalloc(d["u"], d["delta"], d["A"], d["B"], d["C"], y, h, D=d["D"],
                                   z=d["z"], delta_bias=d["delta_bias"])
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(h, h_ref)
    return S


def test_noalloc_matches_workspace_call_twice(monkeypatch):
    # first the state-per-lane path cut into segments (pairs, carry, fix-up),
    # then a smaller call on the split path, over what the first left behind
    s1 = _both(W.S6_LONG_FP32.scaled(L=30000, D=256), seed=1, monkeypatch=monkeypatch)
    s2 = _both(W.S6_MAMBA130M.scaled(B=1, L=3000, D=64), seed=2, monkeypatch=monkeypatch,
               segments=7, split=True)
    assert s1 > 1 and s2 > 1


def test_noalloc_rejects_sizes_beyond_the_scratch():
    lib = _native.load()
    B, L, D, N = 1, 131072, 60000, 64          # split in 4: pairs far beyond the static array
    need = lib.ssm_selective_scan_workspace_bytes(B, L, D, N, 0)
    assert need > (32 << 20)
    fake = 0x10000
    rc = lib.ssm_selective_scan_fwd_noalloc(fake, fake, fake, fake, fake, None, None, None, 1,
                                            None, fake, None, B, L, D, N, 0, None)
    assert rc == 6                             # SSM_ERR_WORKSPACE, nothing launched
