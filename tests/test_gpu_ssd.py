"""GPU parity of the SSD (Mamba-2) chunked forward against the fp64 oracle,
through the C ABI.  Bar: normwise max relative error <= 2e-2 (bf16 storage,
fp32 state and accumulation, bf16 matrix-core operands); bit-exact on
integer-valued cases where every product is exact (decay 1 -> causal all-ones
mask; decay 0 -> identity mask)."""
import numpy as np
import pytest
import torch

import selective_state_space_21_amd as ssm
from selective_state_space_21_amd import workloads as W

from _parity import TOL, normwise_err, ssd_gpu, ssd_oracle, ssd_oracle_sampled, to_dev

pytestmark = pytest.mark.gpu


def _cmp(inp, chunk=None, tol=2e-2):
    Y, h = ssd_gpu(inp, chunk=chunk)
    Yr, hr = ssd_oracle(inp)
    ey = normwise_err(Y.float().cpu().numpy(), Yr)
    eh = normwise_err(h.cpu().numpy(), hr)
    assert ey <= tol, f"Y err {ey:.3e}"
    assert eh <= tol, f"h_last err {eh:.3e}"
    return ey, eh


@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("L", [600, 1024])
def test_workload_parity_small(chunk, L):
    w = W.SSD_MAMBA2.scaled(B=2, L=L, H=4, chunk=chunk)
    _cmp(W.make_ssd_inputs(w, seed=chunk + L))


@pytest.mark.parametrize("N", [64, 128])
def test_state_sizes(N):
    w = W.SSD_MAMBA2.scaled(B=1, L=700, H=3, N=N, chunk=128)
    _cmp(W.make_ssd_inputs(w, seed=N))


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_state64_every_chunk(chunk):
    """N = 64 at each chunk length, ragged L, with skip, gate, bias and h0."""
    w = W.SSD_MAMBA2.scaled(B=2, L=517, H=3, N=64, chunk=chunk)
    _cmp(_with_extras(W.make_ssd_inputs(w, seed=chunk + 64), chunk), chunk=chunk)


def test_groups():
    w = W.SSD_MAMBA2.scaled(B=2, L=333, H=8, G=2, chunk=64)
    _cmp(W.make_ssd_inputs(w, seed=3))
    w = W.SSD_MAMBA2.scaled(B=1, L=333, H=8, G=8, chunk=128)
    _cmp(W.make_ssd_inputs(w, seed=4))


def _with_extras(inp, seed):
    g = torch.Generator().manual_seed(seed)
    Bt, L, H, P = inp["X"].shape
    N = inp["B"].shape[-1]
    inp = dict(inp)
    inp["D"] = 1.0 + 0.1 * torch.randn(H, generator=g)
    inp["z"] = torch.randn(Bt, L, H, P, generator=g).to(torch.bfloat16)
    inp["delta_bias"] = torch.empty(H).uniform_(-1.0, 0.5, generator=g)
    inp["h0"] = 0.3 * torch.randn(Bt, H, P, N, generator=g)
    return inp


@pytest.mark.parametrize("chunk", [64, 256])
def test_skip_gate_bias_h0(chunk):
    w = W.SSD_MAMBA2.scaled(B=2, L=400, H=4, chunk=chunk)
    _cmp(_with_extras(W.make_ssd_inputs(w, seed=7), 7), chunk=chunk)


def test_chaining_two_calls_equal_one():
    w = W.SSD_MAMBA2.scaled(B=2, L=640, H=4, chunk=128)
    inp = _with_extras(W.make_ssd_inputs(w, seed=8), 8)
    d = to_dev(inp)
    kw = dict(D=d["D"], delta_bias=d["delta_bias"], chunk=128)
    Y, h = ssm.ssd_chunk_fwd(d["X"], d["delta"], d["A"], d["B"], d["C"], z=d["z"], h0=d["h0"], **kw)
    cut = 200                                   # not a chunk boundary
    sl = lambda t, a, b: t[:, a:b].contiguous()
    Y1, h1 = ssm.ssd_chunk_fwd(sl(d["X"], 0, cut), sl(d["delta"], 0, cut), d["A"], sl(d["B"], 0, cut),
                               sl(d["C"], 0, cut), z=sl(d["z"], 0, cut), h0=d["h0"], **kw)
    Y2, h2 = ssm.ssd_chunk_fwd(sl(d["X"], cut, 640), sl(d["delta"], cut, 640), d["A"],
                               sl(d["B"], cut, 640), sl(d["C"], cut, 640), z=sl(d["z"], cut, 640),
                               h0=h1, **kw)
    torch.cuda.synchronize()
    assert normwise_err(torch.cat([Y1, Y2], 1).float().cpu(), Y.float().cpu()) <= 2e-2
    assert normwise_err(h2.cpu(), h.cpu()) <= 2e-2


def test_empty_sequence_copies_h0():
    h0 = torch.randn(2, 3, 64, 128, device="cuda")
    e = torch.empty(2, 0, 3, 64, device="cuda", dtype=torch.bfloat16)
    Y, h = ssm.ssd_chunk_fwd(e, torch.empty(2, 0, 3, device="cuda", dtype=torch.bfloat16),
                             -torch.ones(3, device="cuda"),
                             torch.empty(2, 0, 1, 128, device="cuda", dtype=torch.bfloat16),
                             torch.empty(2, 0, 1, 128, device="cuda", dtype=torch.bfloat16), h0=h0)
    torch.cuda.synchronize()
    assert Y.shape == (2, 0, 3, 64) and torch.equal(h, h0)


def _exact_case(L, mode, seed, H=3, N=128, G=1, P=64):
    """Integer inputs, softplus off, dt = 1.  mode 'ones': A = 0 (every decay 1,
    the mask is causal all-ones); 'eye': A = -1e4 (every decay underflows to 0,
    the mask is the identity).  Sparse X and C keep every partial sum a small
    integer, exact in bf16 and fp32."""
    g = torch.Generator().manual_seed(seed)
    Bt = 2
    X = torch.randint(-1, 2, (Bt, L, H, P), generator=g).float()
    X = X * (torch.rand(Bt, L, H, 1, generator=g) < 3.0 / max(L, 3)).float()
    Bm = (torch.rand(Bt, L, G, N, generator=g) < 0.5).float()
    Cm = (torch.rand(Bt, L, G, N, generator=g) < 1.0 / 32).float()
    A = torch.zeros(H) if mode == "ones" else torch.full((H,), -1e4)
    if mode == "eye":
        X = torch.randint(-2, 3, (Bt, L, H, P), generator=g).float()
    bf = torch.bfloat16
    return dict(X=X.to(bf), delta=torch.ones(Bt, L, H).to(bf), A=A, B=Bm.to(bf), C=Cm.to(bf),
                D=None, z=None, delta_bias=None, h0=None, delta_softplus=False)


@pytest.mark.parametrize("mode", ["ones", "eye"])
@pytest.mark.parametrize("L", [1, 31, 64, 65, 255, 256, 257, 600])
@pytest.mark.parametrize("chunk", [64, 256])
def test_bit_exact_masks(mode, L, chunk):
    inp = _exact_case(L, mode, seed=L + chunk)
    Y, h = ssd_gpu(inp, chunk=chunk)
    Yr, hr = ssd_oracle(inp)
    assert np.all(np.abs(Yr) <= 256) and np.all(Yr == np.round(Yr))
    np.testing.assert_array_equal(Y.float().cpu().numpy(), Yr)
    np.testing.assert_array_equal(h.cpu().numpy(), hr)


def test_deterministic_and_no_out_of_bounds_writes():
    w = W.SSD_MAMBA2.scaled(B=2, L=300, H=4, chunk=128)
    d = to_dev(W.make_ssd_inputs(w, seed=9))
    n = 2 * 300 * 4 * 64
    pad = 64
    guard = torch.full((n + 2 * pad,), 7.0, device="cuda").to(torch.bfloat16)
    out = guard[pad:pad + n].view(2, 300, 4, 64)
    Y1, _ = ssm.ssd_chunk_fwd(d["X"], d["delta"], d["A"], d["B"], d["C"], chunk=128, out=out)
    Y2, _ = ssm.ssd_chunk_fwd(d["X"], d["delta"], d["A"], d["B"], d["C"], chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    g = guard.float()
    assert torch.all(g[:pad] == 7.0) and torch.all(g[pad + n:] == 7.0)


def test_full_size_sampled():
    w = W.SSD_MAMBA2
    inp = W.make_ssd_inputs(w, seed=0)
    Y, h = ssd_gpu(inp)
    Y = Y.float().cpu().numpy()
    h = h.cpu().numpy()
    pairs = [(0, 0), (1, 17), (2, 40), (3, 63), (3, 5)]
    ys, yr, hs, hr = [], [], [], []
    for b, hh, Yo, ho in ssd_oracle_sampled(inp, pairs):
        ys.append(Y[b, :, hh]); yr.append(Yo)
        hs.append(h[b, hh]); hr.append(ho)
    ey = normwise_err(np.stack(ys), np.stack(yr))
    eh = normwise_err(np.stack(hs), np.stack(hr))
    print(f"{w.name}: sampled Y err {ey:.3e}, h_last err {eh:.3e}")
    assert ey <= 2e-2 and eh <= 2e-2
    assert np.all(np.isfinite(Y))


def _block_decay_log2(inp, chunk):
    """For each (b, h, chunk): the largest decay, in log2 units, from the first
    token of a 32-token block to a later token of the same block (the cumulative
    sum of dt * A * log2(e) inside the chunk, differenced against the block's
    first token).  Plain numpy on the CPU from the inputs."""
    raw = inp["delta"].float().numpy().astype(np.float64)
    bias = inp["delta_bias"].numpy().astype(np.float64)
    A = inp["A"].numpy().astype(np.float64)
    x = raw + bias
    dt = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
    a = dt * A * np.log2(np.e)                       # [B, L, H]
    Bt, L, H = a.shape
    nch = -(-L // chunk)
    pad = np.zeros((Bt, nch * chunk, H))
    pad[:, :L] = a
    cum = np.cumsum(pad.reshape(Bt, nch, chunk, H), axis=2)
    first = cum.reshape(Bt, nch, chunk // 32, 32, H)[:, :, :, :1, :]
    rel = first - cum.reshape(Bt, nch, chunk // 32, 32, H)
    return np.abs(rel).max(axis=(2, 3))              # [B, nch, H]


def _spiked_case(L, H, N, chunk, seed, P=64):
    """Random X, B and C; steps softplus(N(-2, 0.5) + bias) with strong decays
    |A_h| in [2, 5]; in about one 32-token block in twelve, 40% of the tokens
    have their raw step raised to +2.5 (a write/flush spike), so those blocks
    decay by far more than 2^64 while the others stay well below.  Skip, gate,
    bias and h0 are on."""
    w = W.SSD_MAMBA2.scaled(B=2, L=L, H=H, N=N, P=P, chunk=chunk)
    inp = _with_extras(W.make_ssd_inputs(w, seed=seed), seed)
    rng = np.random.default_rng(seed + 1000)
    raw = inp["delta"].float().numpy().copy()
    nblk = -(-L // 32)
    hot = rng.random((2, nblk)) < 1.0 / 12.0
    for b in range(2):
        for k in np.nonzero(hot[b])[0]:
            toks = 32 * k + np.nonzero(rng.random(32) < 0.4)[0]
            raw[b, toks[toks < L], :] = 2.5
    inp["delta"] = torch.from_numpy(raw).to(torch.bfloat16)
    inp["delta_bias"] = torch.from_numpy(rng.uniform(-0.5, 0.0, size=H).astype(np.float32))
    inp["A"] = -torch.from_numpy(rng.uniform(2.0, 5.0, size=H).astype(np.float32))
    return inp


@pytest.mark.parametrize("chunk,N", [(64, 128), (256, 128), (64, 64), (128, 64), (256, 64)])
def test_wide_block_decay(chunk, N):
    """Chunks where a 32-token block decays by more than 2^64 (which the kernel
    handles with a per-element mask) next to chunks where none does, in one
    call, against the oracle at the bf16 bar."""
    inp = _spiked_case(L=1000, H=4, N=N, chunk=chunk, seed=chunk + N)
    span = _block_decay_log2(inp, chunk)
    assert np.any(span > 64.0), "no chunk reaches the wide case"
    assert np.any(span <= 64.0), "every chunk is wide"
    ey, eh = _cmp(inp, chunk=chunk)
    print(f"wide chunks {np.mean(span > 64.0):.2f}; Y err {ey:.2e}, h_last err {eh:.2e}")


@pytest.mark.parametrize("P", [32, 96, 128])
@pytest.mark.parametrize("chunk", [64, 256])
def test_head_dims(P, chunk):
    """Head dimensions other than 64: P = 32 (one 32-row slice per head), 96
    (three 32-row slices) and 128 (two 64-row slices), ragged L, with skip,
    gate, bias and h0 (whose rows each slice reads at its own offset)."""
    w = W.SSD_MAMBA2.scaled(B=2, L=419, H=3, P=P, chunk=chunk)
    _cmp(_with_extras(W.make_ssd_inputs(w, seed=P + chunk), P), chunk=chunk)


@pytest.mark.parametrize("N", [32, 96])
@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_state_dims(N, chunk):
    """State sizes 32 and 96 (one and three 32-wide k steps of the score and
    Y_off products; two and six wavefronts own state columns)."""
    w = W.SSD_MAMBA2.scaled(B=2, L=517, H=3, N=N, chunk=chunk)
    _cmp(_with_extras(W.make_ssd_inputs(w, seed=N + chunk), N), chunk=chunk)


@pytest.mark.parametrize("P,N", [(32, 32), (128, 96), (96, 128)])
def test_head_and_state_dims_groups(P, N):
    """Mixed sizes with two groups of heads (each group's B and C rows)."""
    w = W.SSD_MAMBA2.scaled(B=2, L=300, H=4, G=2, P=P, N=N, chunk=128)
    _cmp(_with_extras(W.make_ssd_inputs(w, seed=P * N), 3), chunk=128)


@pytest.mark.parametrize("P,N,chunk", [(128, 128, 64), (32, 96, 256)])
def test_wide_block_decay_sizes(P, N, chunk):
    """The per-element mask of strongly decaying blocks at other head and state
    sizes, with h0 rows read per slice."""
    inp = _spiked_case(L=700, H=3, N=N, chunk=chunk, seed=P + N + chunk, P=P)
    span = _block_decay_log2(inp, chunk)
    assert np.any(span > 64.0) and np.any(span <= 64.0)
    _cmp(inp, chunk=chunk)


@pytest.mark.parametrize("P", [32, 128])
def test_bit_exact_masks_head_dims(P):
    """The exact integer cases at other head dimensions (every slice's rows)."""
    for mode in ("ones", "eye"):
        inp = _exact_case(257, mode, seed=P, P=P)
        Y, h = ssd_gpu(inp, chunk=64)
        Yr, hr = ssd_oracle(inp)
        np.testing.assert_array_equal(Y.float().cpu().numpy(), Yr)
        np.testing.assert_array_equal(h.cpu().numpy(), hr)
