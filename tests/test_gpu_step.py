"""GPU parity of the decode step (ssm_selective_state_update) against the
fp64 oracle, through the C ABI.

Bar: normwise max relative error <= 1e-5 for fp32 storage, <= 2e-2 for bf16
storage (fp32 state either way; the state is compared at 1e-5 when the
inputs are fp32).  Integer cases where every operation is exact are compared
bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_21_amd as ssm
from selective_state_space_21_amd import workloads as W

from _parity import TOL, normwise_err, to_dev

pytestmark = pytest.mark.gpu


def _inputs(Bt, Dm, N, dtype, seed, extras=True):
    w = W.S6_DECODE_2P8B.scaled(B=Bt, D=Dm, N=N, dtype=dtype)
    inp = W.make_step_inputs(w, seed)
    if not extras:
        inp.update(D=None, z=None, delta_bias=None)
    return inp


def _gpu_step(d, zoh=False, state=None):
    st = (d["state"] if state is None else state).clone()
    y = ssm.selective_state_update(st, d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                   z=d["z"], delta_bias=d["delta_bias"],
                                   delta_softplus=d["delta_softplus"], zoh=zoh)
    torch.cuda.synchronize()
    return y, st


def _oracle_step(inp, zoh=False):
    return oracle.s6_step(inp["state"], inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                          D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                          delta_softplus=inp["delta_softplus"], zoh=zoh)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 3, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("extras", [True, False])
def test_step_parity(dtype, N, extras):
    inp = _inputs(3, 333, N, dtype, seed=N + 7 * extras, extras=extras)
    y, st = _gpu_step(to_dev(inp))
    yr, sr = _oracle_step(inp)
    assert normwise_err(y.float().cpu(), yr) <= TOL[dtype]
    assert normwise_err(st.cpu(), sr) <= 1e-5


@pytest.mark.parametrize("N", [4, 16, 5])
def test_step_zoh(N):
    inp = _inputs(2, 200, N, "f32", seed=11)
    y, st = _gpu_step(to_dev(inp), zoh=True)
    yr, sr = _oracle_step(inp, zoh=True)
    assert normwise_err(y.cpu(), yr) <= 1e-5
    assert normwise_err(st.cpu(), sr) <= 1e-5


def test_page_worked_example_as_decode():
    """The two-token worked example of "Mamba & Mamba-2 Architecture" run as
    two decode steps: h1 = 20, then 19.80 retained + 0.20 input."""
    dev = "cuda"
    st = torch.zeros(1, 1, 1, device=dev)
    one = torch.ones(1, 1, device=dev)
    A = -torch.ones(1, 1, device=dev)
    y1 = ssm.selective_state_update(st, torch.tensor([[10.0]], device=dev),
                                    torch.tensor([[2.0]], device=dev), A, one, one,
                                    delta_softplus=False)
    y2 = ssm.selective_state_update(st, torch.tensor([[20.0]], device=dev),
                                    torch.tensor([[0.01]], device=dev), A, one, one,
                                    delta_softplus=False)
    torch.cuda.synchronize()
    assert abs(y1.item() - 20.0) <= 20.0 * 1e-6
    expect = 20.0 * np.exp(-np.float32(0.01)) + np.float32(0.01) * 20.0
    assert abs(y2.item() - expect) <= expect * 1e-5
    assert round(20.0 * float(np.exp(-0.01)), 2) == 19.80
    assert st.item() == y2.item()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_chain_equals_scan(dtype):
    """L decode steps from h0 reproduce one scan over the same L tokens."""
    w = W.S6_MAMBA130M.scaled(B=2, L=40, D=130, dtype=dtype)
    inp = W.make_s6_inputs(w, seed=5)
    inp["h0"] = torch.randn(2, 130, 16, generator=torch.Generator().manual_seed(5))
    d = to_dev(inp)
    st = d["h0"].clone()
    ys = []
    for t in range(w.L):
        ys.append(ssm.selective_state_update(
            st, d["u"][:, t].contiguous(), d["delta"][:, t].contiguous(), d["A"],
            d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), D=d["D"],
            z=d["z"][:, t].contiguous(), delta_bias=d["delta_bias"]))
    torch.cuda.synchronize()
    y = torch.stack(ys, 1).float().cpu().numpy()
    yr, hr = oracle.s6_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                           z=inp["z"], delta_bias=inp["delta_bias"], h0=inp["h0"])
    assert normwise_err(y, yr) <= TOL[dtype]
    assert normwise_err(st.cpu(), hr) <= 1e-5


@pytest.mark.parametrize("N", [16, 7])
def test_bit_exact_prefix_and_reset(N):
    """A = 0, dt = 1 (softplus off): the state is an integer prefix sum and y
    an integer; A = -1e4: every decay underflows to 0 and the state is the
    current input term.  Every operation is exact in fp32."""
    g = torch.Generator().manual_seed(N)
    Bt, Dm, L = 2, 97, 9
    for mode in ("prefix", "reset"):
        A = torch.zeros(Dm, N) if mode == "prefix" else torch.full((Dm, N), -1e4)
        st = torch.zeros(Bt, Dm, N, device="cuda")
        st_ref = np.zeros((Bt, Dm, N))
        for t in range(L):
            u = torch.randint(-3, 4, (Bt, Dm), generator=g).float()
            Bm = torch.randint(-2, 3, (Bt, N), generator=g).float()
            Cm = torch.randint(-2, 3, (Bt, N), generator=g).float()
            y = ssm.selective_state_update(st, u.cuda(), torch.ones(Bt, Dm, device="cuda"),
                                           A.cuda(), Bm.cuda(), Cm.cuda(), delta_softplus=False)
            torch.cuda.synchronize()
            decay = 1.0 if mode == "prefix" else 0.0
            st_ref = decay * st_ref + u.numpy()[:, :, None] * Bm.numpy()[:, None, :]
            y_ref = np.einsum("bdn,bn->bd", st_ref, Cm.numpy())
            np.testing.assert_array_equal(st.cpu().numpy(), st_ref)
            np.testing.assert_array_equal(y.cpu().numpy(), y_ref)


def test_no_out_of_bounds_writes():
    inp = _inputs(3, 77, 16, "bf16", seed=3)
    d = to_dev(inp)
    pad = 64
    n_st, n_y = 3 * 77 * 16, 3 * 77
    gs = torch.full((n_st + 2 * pad,), 5.0, device="cuda")
    gy = torch.full((n_y + 2 * pad,), 5.0, device="cuda").to(torch.bfloat16)
    st = gs[pad:pad + n_st].view(3, 77, 16)
    st.copy_(d["state"])
    y = gy[pad:pad + n_y].view(3, 77)
    ssm.selective_state_update(st, d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                               delta_bias=d["delta_bias"], out=y)
    torch.cuda.synchronize()
    assert torch.all(gs[:pad] == 5.0) and torch.all(gs[pad + n_st:] == 5.0)
    assert torch.all(gy[:pad].float() == 5.0) and torch.all(gy[pad + n_y:].float() == 5.0)
    yr, sr = _oracle_step(inp)
    assert normwise_err(y.float().cpu(), yr) <= 2e-2


def test_full_size_decode_workload():
    w = W.S6_DECODE_2P8B
    inp = W.make_step_inputs(w, seed=0)
    y, st = _gpu_step(to_dev(inp))
    yr, sr = _oracle_step(inp)
    ey = normwise_err(y.float().cpu(), yr)
    es = normwise_err(st.cpu(), sr)
    print(f"{w.name}: y err {ey:.3e}, state err {es:.3e}")
    assert ey <= 2e-2 and es <= 1e-5
