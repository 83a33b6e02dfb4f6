"""GPU parity of the causal depthwise conv1d + SiLU (ssm_causal_conv1d_silu)
against the fp64 oracle, through the C ABI.  Bar: normwise max relative
error <= 1e-5 (fp32 storage) / 2e-2 (bf16); integer cases without SiLU and
chunked calls against one call are bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_21_amd as ssm
from selective_state_space_21_amd import workloads as W

from _parity import TOL, normwise_err

pytestmark = pytest.mark.gpu


def _run(inp, state=None, silu=True, ret_state=True):
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    st = None if state is None else state.cuda()
    r = ssm.causal_conv1d_silu(d["x"], d["weight"], d["bias"], state=st, silu=silu,
                               return_state=ret_state)
    torch.cuda.synchronize()
    if ret_state:
        return r[0].float().cpu().numpy(), r[1].cpu().numpy()
    return r.float().cpu().numpy(), None


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 100, 64, 4), (1, 1, 8, 4), (3, 2, 16, 4), (2, 77, 40, 3),
                                   (2, 65, 13, 4), (1, 33, 7, 2), (2, 40, 24, 1), (2, 70, 18, 4),
                                   (1, 50, 20, 4)])
def test_conv_parity(dtype, shape):
    Bt, L, Dm, K = shape
    inp = W.make_conv_inputs(W.CONV_MAMBA130M.scaled(B=Bt, L=L, D=Dm, K=K, dtype=dtype), seed=L)
    g = torch.Generator().manual_seed(Dm)
    state = torch.randn(Bt, Dm, K - 1, generator=g) if K > 1 else None
    u, st = _run(inp, state=state)
    ur, sr = oracle.causal_conv1d_silu(inp["x"], inp["weight"], inp["bias"], state=state)
    assert normwise_err(u, ur) <= TOL[dtype]
    np.testing.assert_array_equal(st, sr)          # the carried inputs are copied exactly


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_chunks_equal_one_call(dtype):
    inp = W.make_conv_inputs(W.CONV_MAMBA130M.scaled(B=2, L=150, D=48, dtype=dtype), seed=3)
    u, st = _run(inp)
    parts, state = [], None
    for a, b in [(0, 5), (5, 6), (6, 70), (70, 150)]:
        sub = dict(inp, x=inp["x"][:, a:b].contiguous())
        ui, state = _run(sub, state=None if state is None else torch.from_numpy(state))
        parts.append(ui)
    np.testing.assert_array_equal(np.concatenate(parts, 1), u)
    np.testing.assert_array_equal(state, st)


def test_conv_integer_exact_without_silu():
    g = torch.Generator().manual_seed(0)
    x = torch.randint(-3, 4, (2, 90, 24), generator=g).float()
    w = torch.randint(-2, 3, (24, 4), generator=g).float()
    b = torch.randint(-2, 3, (24,), generator=g).float()
    for dt in (torch.float32, torch.bfloat16):
        u, _ = _run(dict(x=x.to(dt), weight=w, bias=b), silu=False)
        ur, _ = oracle.causal_conv1d_silu(x, w, b, silu=False)
        np.testing.assert_array_equal(u, ur)


def test_conv_empty_sequence_passes_state():
    st = torch.randn(2, 16, 3)
    inp = dict(x=torch.empty(2, 0, 16), weight=torch.randn(16, 4), bias=None)
    _, s = _run(inp, state=st)
    np.testing.assert_array_equal(s, st.numpy())
    _, s0 = _run(inp)
    assert np.all(s0 == 0)


def test_conv_no_out_of_bounds_writes():
    inp = W.make_conv_inputs(W.CONV_MAMBA130M.scaled(B=2, L=37, D=40), seed=5)
    n, pad = 2 * 37 * 40, 64
    guard = torch.full((n + 2 * pad,), 9.0, device="cuda").to(torch.bfloat16)
    out = guard[pad:pad + n].view(2, 37, 40)
    ssm.causal_conv1d_silu(inp["x"].cuda(), inp["weight"].cuda(), inp["bias"].cuda(), out=out)
    torch.cuda.synchronize()
    g = guard.float()
    assert torch.all(g[:pad] == 9.0) and torch.all(g[pad + n:] == 9.0)
    ur, _ = oracle.causal_conv1d_silu(inp["x"], inp["weight"], inp["bias"])
    assert normwise_err(out.float().cpu().numpy(), ur) <= 2e-2


def test_conv_full_size():
    w = W.CONV_MAMBA130M
    inp = W.make_conv_inputs(w, seed=0)
    u, _ = _run(inp, ret_state=False)
    ur, _ = oracle.causal_conv1d_silu(inp["x"], inp["weight"], inp["bias"])
    e = normwise_err(u, ur)
    print(f"{w.name}: err {e:.3e}")
    assert e <= 2e-2
