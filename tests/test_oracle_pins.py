"""Pins for the fp64 oracle: values the pages print, closed forms, brute-force
sums and library routines.  None of these re-types the oracle's own loop; each
is chosen so that a plausible slip in it (a dropped term, a wrong sign or index,
ZOH instead of first-order input, bias outside the softplus, a missed h0)
fails at least one test.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import scans

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _single_channel(u, delta, A=-1.0, B=1.0, C=1.0, h0=None, softplus=False, zoh=False):
    """Run the oracle on one channel with N = 1 and constant B, C."""
    L = len(u)
    uu = np.asarray(u, dtype=np.float64).reshape(1, L, 1)
    dd = np.asarray(delta, dtype=np.float64).reshape(1, L, 1)
    Bm = np.full((1, L, 1), B)
    Cm = np.full((1, L, 1), C)
    h = None if h0 is None else np.array([[[h0]]], dtype=np.float64)
    y, hl = oracle.s6_fwd(uu, dd, np.array([[A]]), Bm, Cm, h0=h,
                          delta_softplus=softplus, zoh=zoh)
    return y[0, :, 0], hl[0, 0, 0]


# ---------------------------------------------------------------- P1
def test_p1_page2_code_example():
    g = _golden("page2_code_example.json")
    y, _ = _single_channel(g["x"], g["delta"], A=g["a_scalar"])
    dec = g["printed_decimals"]
    assert round(y[0], dec) == g["printed_outputs"][0]
    assert round(y[1], dec) == g["printed_outputs"][1]
    # third token: the listing's arithmetic, evaluated by hand
    h2 = math.exp(-0.001) * 7.5 + 0.001 * 100.0
    h3 = math.exp(-1.0) * h2 + 1.0 * 1.0
    assert abs(y[2] - h3) < 1e-12
    assert round(y[2], 4) == 3.7931 and round(y[2], 4) != g["printed_outputs"][2]
    # the exact zero-order-hold input term would NOT reproduce the page
    yz, _ = _single_channel(g["x"], g["delta"], A=g["a_scalar"], zoh=True)
    assert round(yz[0], dec) != g["printed_outputs"][0]


# ---------------------------------------------------------------- P2
def test_p2_page2_worked_example():
    g = _golden("page2_worked_example.json")
    d1, d2 = g["delta"]
    x1, x2 = g["x"]
    y, h = _single_channel([x1, x2], [d1, d2], A=g["A"])
    assert y[0] == pytest.approx(20.0, abs=1e-12)
    # split step 2 into the retained part and the input part
    _, retained = _single_channel([0.0], [d2], A=g["A"], h0=y[0])
    y_in, _ = _single_channel([x2], [d2], A=g["A"])
    assert round(retained, 2) == g["printed_retained_h1"]
    assert round(y_in[0], 2) == g["printed_input_term_step2"]
    assert h == pytest.approx(retained + y_in[0], abs=1e-12)


def test_p2_as_two_decode_steps():
    """The worked example is itself a two-token decode: each step starts from
    the state the previous one returned."""
    g = _golden("page2_worked_example.json")
    one = np.ones((1, 1))
    st = np.zeros((1, 1, 1))
    y1, st = oracle.s6_step(st, np.array([[g["x"][0]]]), np.array([[g["delta"][0]]]),
                            g["A"] * one, one, one, delta_softplus=False)
    assert y1[0, 0] == pytest.approx(20.0, abs=1e-12) and st[0, 0, 0] == y1[0, 0]
    y2, st = oracle.s6_step(st, np.array([[g["x"][1]]]), np.array([[g["delta"][1]]]),
                            g["A"] * one, one, one, delta_softplus=False)
    retained = 20.0 * math.exp(-g["delta"][1])
    assert round(retained, 2) == g["printed_retained_h1"]
    assert round(y2[0, 0] - retained, 2) == g["printed_input_term_step2"]
    assert y2[0, 0] == pytest.approx(retained + g["delta"][1] * g["x"][1], abs=1e-12)


# ---------------------------------------------------------------- P3
def test_p3_horizon_table():
    g = _golden("page5_horizon_table.json")
    for d, printed in zip(g["delta"], g["printed_retained"]):
        _, h = _single_channel([0.0], [d], A=-1.0, h0=1.0)
        digits = 4 if printed < 0.01 else 3
        assert round(h, digits) == printed
    # horizon ~ 1/delta: after round(1/delta) steps the state is ~ 1/e
    for d in (0.01, 0.1):
        n = int(round(1 / d))
        _, h = _single_channel([0.0] * n, [d] * n, A=-1.0, h0=1.0)
        assert h == pytest.approx(math.exp(-1.0), rel=1e-9)


# ---------------------------------------------------------------- P4
def test_p4_gru_identity_softplus_and_zoh():
    s = np.linspace(-12.0, 12.0, 97)
    for si in s:
        # kept fraction with softplus on: exp(-softplus(s)) == sigmoid(-s)
        _, h = _single_channel([0.0], [si], A=-1.0, h0=1.0, softplus=True)
        assert h == pytest.approx(scipy.special.expit(-si), rel=1e-13, abs=1e-300)
        # exact ZOH input term: dB = 1 - dA = sigmoid(s) -> GRU update
        _, hz = _single_channel([3.0], [si], A=-1.0, h0=-2.0, softplus=True, zoh=True)
        g = scipy.special.expit(si)
        assert hz == pytest.approx((1 - g) * -2.0 + g * 3.0, rel=1e-12, abs=1e-14)


def test_softplus_matches_logaddexp():
    x = np.array([-80.0, -30.0, -5.0, -1e-3, 0.0, 0.7, 5.0, 19.0, 25.0, 60.0])
    y, _ = _single_channel(np.ones_like(x), x, A=-1.0, softplus=True)
    # L tokens chained: isolate each step by running them one at a time
    for xi in x:
        yi, _ = _single_channel([1.0], [xi], A=-1.0, softplus=True)
        assert yi[0] == pytest.approx(np.logaddexp(0.0, xi), rel=1e-14, abs=1e-300)


# ---------------------------------------------------------------- P5
def test_p5_lti_convolution_brute_force():
    rng = np.random.default_rng(1)
    Bt, L, Dm, N = 2, 60, 3, 5
    A = -rng.uniform(0.2, 3.0, size=(Dm, N))
    dconst = rng.uniform(0.05, 0.5, size=(Bt, Dm))
    Bc = rng.standard_normal((Bt, N))
    Cc = rng.standard_normal((Bt, N))
    Dskip = rng.standard_normal(Dm)
    u = rng.standard_normal((Bt, L, Dm))
    delta = np.broadcast_to(dconst[:, None, :], (Bt, L, Dm)).copy()
    Bm = np.broadcast_to(Bc[:, None, :], (Bt, L, N)).copy()
    Cm = np.broadcast_to(Cc[:, None, :], (Bt, L, N)).copy()
    y, _ = oracle.s6_fwd(u, delta, A, Bm, Cm, D=Dskip, delta_softplus=False)
    for b in range(Bt):
        for d in range(Dm):
            dt = dconst[b, d]
            lags = np.arange(L)
            # LTI kernel K[m] = sum_n C[n] exp(dt*A[n]*m) dt*B[n]
            K = (Cc[b][None, :] * np.exp(dt * A[d][None, :] * lags[:, None])
                 * dt * Bc[b][None, :]).sum(axis=1)
            ref = np.convolve(u[b, :, d], K)[:L] + Dskip[d] * u[b, :, d]
            np.testing.assert_allclose(y[b, :, d], ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- P6
def _brute_force_time_varying(u, delta, A, Bm, Cm, Dskip, z, bias, h0, softplus):
    Bt, L, Dm = u.shape
    N = A.shape[1]
    y = np.zeros((Bt, L, Dm))
    for b in range(Bt):
        for d in range(Dm):
            x = delta[b, :, d] + (bias[d] if bias is not None else 0.0)
            dt = np.logaddexp(0.0, x) if softplus else x          # softplus via library
            dA = np.exp(dt[:, None] * A[d][None, :])              # [L, N]
            dB = dt[:, None] * Bm[b]                              # [L, N]
            for k in range(L):
                acc = 0.0
                for j in range(k + 1):
                    prod = np.prod(dA[j + 1:k + 1], axis=0)       # empty -> ones
                    acc += np.dot(Cm[b, k], prod * dB[j]) * u[b, j, d]
                if h0 is not None:
                    acc += np.dot(Cm[b, k], np.prod(dA[:k + 1], axis=0) * h0[b, d])
                if Dskip is not None:
                    acc += Dskip[d] * u[b, k, d]
                if z is not None:
                    acc *= z[b, k, d] * scipy.special.expit(z[b, k, d])
                y[b, k, d] = acc
    return y


@pytest.mark.parametrize("with_extras", [False, True])
def test_p6_time_varying_unrolled_sum(with_extras):
    rng = np.random.default_rng(2 + with_extras)
    Bt, L, Dm, N = 2, 17, 3, 4
    u = rng.standard_normal((Bt, L, Dm))
    delta = rng.normal(-1.0, 1.0, size=(Bt, L, Dm))
    A = -rng.uniform(0.1, 4.0, size=(Dm, N))
    Bm = rng.standard_normal((Bt, L, N))
    Cm = rng.standard_normal((Bt, L, N))
    kw = {}
    Dskip = z = bias = h0 = None
    if with_extras:
        Dskip = rng.standard_normal(Dm)
        z = rng.standard_normal((Bt, L, Dm))
        bias = rng.uniform(-2, 1, size=Dm)
        h0 = rng.standard_normal((Bt, Dm, N))
    y, _ = oracle.s6_fwd(u, delta, A, Bm, Cm, D=Dskip, z=z, delta_bias=bias,
                         h0=h0, delta_softplus=True)
    ref = _brute_force_time_varying(u, delta, A, Bm, Cm, Dskip, z, bias, h0, True)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_p6_semiseparable_matrix_reproduces_scan():
    """Materialise the L x L matrix M[t,k] = C_t (prod_{j=k+1..t} dA_j) dB_k of
    one channel (exercise 3 of the temporalbook section) and multiply by u."""
    rng = np.random.default_rng(4)
    L, N = 24, 6
    u = rng.standard_normal((1, L, 1))
    delta = rng.uniform(0.01, 1.0, size=(1, L, 1))
    A = -rng.uniform(0.5, 2.0, size=(1, N))
    Bm = rng.standard_normal((1, L, N))
    Cm = rng.standard_normal((1, L, N))
    y, _ = oracle.s6_fwd(u, delta, A, Bm, Cm, delta_softplus=False)
    dt = delta[0, :, 0]
    logdA = dt[:, None] * A[0][None, :]                      # [L, N]
    cum = np.cumsum(logdA, axis=0)
    M = np.zeros((L, L))
    for t in range(L):
        for k in range(t + 1):
            decay = np.exp(cum[t] - cum[k])                  # prod over j in (k, t]
            M[t, k] = np.dot(Cm[0, t], decay * dt[k] * Bm[0, k])
    np.testing.assert_allclose(y[0, :, 0], M @ u[0, :, 0], rtol=1e-10, atol=1e-12)
    # selection makes M depend on absolute time, not only the lag
    assert not np.allclose(M[5, 2], M[6, 3])


# ---------------------------------------------------------------- P7 / P8
def test_p7_hold_when_delta_is_zero():
    rng = np.random.default_rng(5)
    Bt, L, Dm, N = 2, 9, 3, 4
    h0 = rng.standard_normal((Bt, Dm, N))
    Cm = rng.standard_normal((Bt, L, N))
    y, hl = oracle.s6_fwd(rng.standard_normal((Bt, L, Dm)), np.zeros((Bt, L, Dm)),
                          -rng.uniform(0.1, 5, (Dm, N)), rng.standard_normal((Bt, L, N)),
                          Cm, h0=h0, delta_softplus=False)
    assert np.array_equal(hl, h0)                              # bit-exact hold
    np.testing.assert_allclose(y, np.einsum("btn,bdn->btd", Cm, h0), rtol=1e-13, atol=1e-14)
    # softplus(-60) ~ 9e-27: the state moves by less than 1e-25 relative
    y2, hl2 = oracle.s6_fwd(rng.standard_normal((Bt, L, Dm)), np.full((Bt, L, Dm), -60.0),
                            -rng.uniform(0.1, 5, (Dm, N)), rng.standard_normal((Bt, L, N)),
                            Cm, h0=h0, delta_softplus=True)
    assert np.max(np.abs(hl2 - h0) / np.abs(h0)) < 1e-24


def test_p8_flush_when_decay_underflows():
    rng = np.random.default_rng(6)
    Bt, L, Dm, N = 2, 11, 3, 4
    u = rng.standard_normal((Bt, L, Dm))
    delta = rng.uniform(0.05, 2.0, size=(Bt, L, Dm))
    Bm = rng.standard_normal((Bt, L, N))
    Cm = rng.standard_normal((Bt, L, N))
    y, hl = oracle.s6_fwd(u, delta, np.full((Dm, N), -1e6), Bm, Cm,
                          h0=rng.standard_normal((Bt, Dm, N)), delta_softplus=False)
    # the state is exactly the current write delta*B_t*u_t
    expect_h = delta[:, -1, :, None] * Bm[:, -1, None, :] * u[:, -1, :, None]
    np.testing.assert_array_equal(hl, expect_h)
    expect_y = np.einsum("btn,btd->btd", Cm * Bm, delta * u)
    np.testing.assert_allclose(y, expect_y, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- skip / gate / bias
def test_skip_and_gate_special_cases():
    rng = np.random.default_rng(7)
    Bt, L, Dm, N = 2, 7, 5, 3
    u = rng.standard_normal((Bt, L, Dm))
    z = rng.normal(0, 3, (Bt, L, Dm))
    Dskip = rng.standard_normal(Dm)
    zeros = np.zeros((Bt, L, N))
    args = (u, rng.standard_normal((Bt, L, Dm)), -np.ones((Dm, N)), rng.standard_normal((Bt, L, N)), zeros)
    # C = 0: only the skip survives, then the gate silu(z)
    y, _ = oracle.s6_fwd(*args, D=Dskip)
    np.testing.assert_array_equal(y, Dskip[None, None, :] * u)
    y, _ = oracle.s6_fwd(*args, D=Dskip, z=z)
    silu = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(y, Dskip[None, None, :] * u * silu, rtol=1e-14, atol=1e-300)
    # without skip and C = 0 the output is exactly zero
    y, _ = oracle.s6_fwd(*args, z=z)
    assert np.all(y == 0.0)


def test_bias_is_inside_the_softplus():
    rng = np.random.default_rng(8)
    Bt, L, Dm, N = 1, 12, 4, 3
    u = rng.standard_normal((Bt, L, Dm))
    raw = rng.standard_normal((Bt, L, Dm))
    bias = rng.uniform(-4, -2, Dm)
    A = -rng.uniform(0.5, 3, (Dm, N))
    Bm = rng.standard_normal((Bt, L, N))
    Cm = rng.standard_normal((Bt, L, N))
    y1, h1 = oracle.s6_fwd(u, raw, A, Bm, Cm, delta_bias=bias, delta_softplus=True)
    y2, h2 = oracle.s6_fwd(u, raw + bias[None, None, :], A, Bm, Cm, delta_softplus=True)
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-15)
    # softplus(raw) + bias would be a different (wrong) reading
    y3, _ = oracle.s6_fwd(u, np.logaddexp(0, raw) + bias, A, Bm, Cm, delta_softplus=False)
    assert np.max(np.abs(y3 - y1)) > 1e-3


# ---------------------------------------------------------------- P9 / P12
def test_p9_scans_agree_and_count_combines():
    rng = np.random.default_rng(9)
    for L in (1, 2, 5, 8, 31, 64, 100):
        a = rng.uniform(0.0, 1.0, size=(L, 3))
        b = rng.standard_normal((L, 3))
        ref = scans.scan_sequential(a, b)
        hs, c_hs = scans.scan_hillis_steele(a, b)
        bl, c_bl = scans.scan_blelloch(a, b)
        np.testing.assert_allclose(hs, ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(bl, ref, rtol=1e-12, atol=1e-13)
        for ch in (1, 3, 7, 16, L):
            np.testing.assert_allclose(scans.scan_chunked(a, b, ch), ref, rtol=1e-12, atol=1e-13)
        n = 1 << max(0, (L - 1).bit_length())
        assert c_bl <= 2 * n                                  # O(L) work
        assert c_hs == sum(L - (1 << k) for k in range(max(0, (L - 1).bit_length())))
    # p1's own check: parallel scan equals the loop at atol 1e-5
    a = np.exp(rng.uniform(0, 0.5, (2, 8, 4)) * -1.0).transpose(1, 0, 2)
    b = rng.standard_normal((8, 2, 4))
    assert np.allclose(scans.scan_hillis_steele(a, b)[0], scans.scan_sequential(a, b), atol=1e-5)


def test_p9_oracle_chaining_equals_one_call():
    rng = np.random.default_rng(10)
    Bt, L, Dm, N = 2, 40, 3, 4
    u = rng.standard_normal((Bt, L, Dm))
    raw = rng.standard_normal((Bt, L, Dm))
    A = -rng.uniform(0.1, 2, (Dm, N))
    Bm = rng.standard_normal((Bt, L, N))
    Cm = rng.standard_normal((Bt, L, N))
    z = rng.standard_normal((Bt, L, Dm))
    y, hl = oracle.s6_fwd(u, raw, A, Bm, Cm, z=z)
    for cut in (1, 13, 39):
        ya, ha = oracle.s6_fwd(u[:, :cut], raw[:, :cut], A, Bm[:, :cut], Cm[:, :cut], z=z[:, :cut])
        yb, hb = oracle.s6_fwd(u[:, cut:], raw[:, cut:], A, Bm[:, cut:], Cm[:, cut:], z=z[:, cut:], h0=ha)
        np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(hb, hl, rtol=1e-13, atol=1e-14)


def test_empty_sequence_returns_h0():
    h0 = np.arange(12, dtype=np.float64).reshape(1, 3, 4)
    y, hl = oracle.s6_fwd(np.zeros((1, 0, 3)), np.zeros((1, 0, 3)), -np.ones((3, 4)),
                          np.zeros((1, 0, 4)), np.zeros((1, 0, 4)), h0=h0)
    assert y.shape == (1, 0, 3)
    assert np.array_equal(hl, h0)


# ---------------------------------------------------------------- P10 (SSD)
def _ssd_case(rng, Bt=2, L=23, H=4, P=3, G=2, N=5, extras=True):
    X = rng.standard_normal((Bt, L, H, P))
    delta = rng.normal(-1.0, 0.7, (Bt, L, H))
    A = -np.exp(rng.uniform(0, 2, H))
    Bm = rng.standard_normal((Bt, L, G, N))
    Cm = rng.standard_normal((Bt, L, G, N))
    kw = {}
    if extras:
        kw = dict(D=rng.standard_normal(H), z=rng.standard_normal((Bt, L, H, P)),
                  delta_bias=rng.uniform(-1, 0.5, H), h0=rng.standard_normal((Bt, H, P, N)))
    return X, delta, A, Bm, Cm, kw


@pytest.mark.parametrize("extras", [False, True])
def test_p10_ssd_equals_s6_with_scalar_decay(extras):
    rng = np.random.default_rng(11 + extras)
    Bt, L, H, P, G, N = 2, 23, 4, 3, 2, 5
    X, delta, A, Bm, Cm, kw = _ssd_case(rng, Bt, L, H, P, G, N, extras)
    Y, hl = oracle.ssd_fwd(X, delta, A, Bm, Cm, **kw)
    hpg = H // G
    for g in range(G):
        hs = list(range(g * hpg, (g + 1) * hpg))
        # S6 view of this group's heads: channel (h, p) with A'[., n] = A_h
        u6 = X[:, :, hs, :].reshape(Bt, L, hpg * P)
        d6 = np.repeat(delta[:, :, hs], P, axis=2)
        A6 = np.repeat(A[hs], P)[:, None] * np.ones((1, N))
        k6 = {}
        if extras:
            k6 = dict(D=np.repeat(kw["D"][hs], P), z=kw["z"][:, :, hs, :].reshape(Bt, L, hpg * P),
                      delta_bias=np.repeat(kw["delta_bias"][hs], P),
                      h0=kw["h0"][:, hs].reshape(Bt, hpg * P, N))
        y6, h6 = oracle.s6_fwd(u6, d6, A6, Bm[:, :, g], Cm[:, :, g], **k6)
        np.testing.assert_allclose(Y[:, :, hs, :].reshape(Bt, L, hpg * P), y6, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(hl[:, hs].reshape(Bt, hpg * P, N), h6, rtol=1e-12, atol=1e-13)


def test_p10_ssd_masked_attention_form():
    """Y = (M o (C B^T)) (delta o X) + decayed readout of h0, M[t,s] = prod_{k=s+1..t} a_k."""
    rng = np.random.default_rng(13)
    Bt, L, H, P, G, N = 2, 19, 4, 3, 1, 6
    X, delta, A, Bm, Cm, kw = _ssd_case(rng, Bt, L, H, P, G, N, extras=False)
    h0 = rng.standard_normal((Bt, H, P, N))
    Y, _ = oracle.ssd_fwd(X, delta, A, Bm, Cm, h0=h0)
    for b in range(Bt):
        for h in range(H):
            dt = np.logaddexp(0.0, delta[b, :, h])
            loga = dt * A[h]
            M = np.zeros((L, L))
            for t in range(L):
                for s in range(t + 1):
                    M[t, s] = np.prod(np.exp(loga[s + 1:t + 1]))
            CBt = Cm[b, :, 0, :] @ Bm[b, :, 0, :].T
            ref = (M * CBt) @ (dt[:, None] * X[b, :, h, :])
            decay0 = np.array([np.prod(np.exp(loga[:t + 1])) for t in range(L)])
            ref += decay0[:, None] * (Cm[b, :, 0, :] @ h0[b, h].T)
            np.testing.assert_allclose(Y[b, :, h, :], ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- P11
def test_p11_byte_model():
    g = _golden("page5_byte_model.json")
    elems = g["B"] * g["L"] * g["D"] * g["N"]
    assert elems == 268_435_456
    assert abs(elems - g["printed_elements_approx"]) / elems < 0.01
    assert round(elems * 2 / 1e6) == g["printed_fp16_MB_approx"]
    assert abs(g["D"] * g["N"] - g["printed_decode_fma_approx"]) / 32768 < 0.01
    assert g["D"] * g["N"] * 4 // 1024 == g["printed_state_KB_fp32"]


def test_oracle_rejects_bad_arguments():
    with pytest.raises(AssertionError):
        oracle.s6_fwd(np.zeros((1, 4, 3)), np.zeros((1, 4, 2)), -np.ones((3, 2)),
                      np.zeros((1, 4, 2)), np.zeros((1, 4, 2)))
    with pytest.raises(ValueError):
        oracle.ssd_fwd(np.zeros((1, 4, 3, 2)), np.zeros((1, 4, 3)), -np.ones(3),
                       np.zeros((1, 4, 2, 2)), np.zeros((1, 4, 2, 2)))   # H % G != 0


# ---------------------------------------------------------------- backward
def _fd_case(seed=0, Bt=2, L=5, Dm=3, N=4):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64)
    return dict(u=r(Bt, L, Dm), delta=r(Bt, L, Dm), A=-2.0 * torch.rand(Dm, N, generator=g,
                dtype=torch.float64), B=r(Bt, L, N), C=r(Bt, L, N), D=r(Dm), z=r(Bt, L, Dm),
                delta_bias=r(Dm), h0=r(Bt, Dm, N)), r(Bt, L, Dm), r(Bt, Dm, N), g


def test_backward_matches_finite_differences_of_the_c_oracle():
    """Directional derivatives of sum(dy*y) + sum(dh*h_last), by central
    differences of the C oracle (separate code), against the autodiff
    gradients, for every input."""
    from oracle.backward import s6_bwd
    inp, dy, dh, g = _fd_case()
    gr = s6_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], dy, D=inp["D"], z=inp["z"],
                delta_bias=inp["delta_bias"], h0=inp["h0"], dh_last=dh)

    def f(**kw):
        a = dict(inp)
        a.update(kw)
        y, hl = oracle.s6_fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], D=a["D"], z=a["z"],
                              delta_bias=a["delta_bias"], h0=a["h0"])
        return float((y * dy.numpy()).sum() + (hl * dh.numpy()).sum())

    eps = 1e-6
    for k, x in inp.items():
        v = torch.randn(x.shape, generator=g, dtype=torch.float64)
        fd = (f(**{k: x + eps * v}) - f(**{k: x - eps * v})) / (2 * eps)
        an = float((gr["dh0" if k == "h0" else "d" + k] * v).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (k, fd, an)


def test_backward_one_step_closed_form():
    """N = 1, L = 1, no softplus, skip or gate: y = C (e^{dt A} h0 + dt B u)."""
    from oracle.backward import s6_bwd
    u, dt, a, b, c, h0 = 0.7, 0.3, -1.5, 1.1, -0.8, 0.4
    T = lambda v: torch.tensor(v, dtype=torch.float64)
    gr = s6_bwd(T([[[u]]]), T([[[dt]]]), T([[a]]), T([[[b]]]), T([[[c]]]), T([[[1.0]]]),
                delta_softplus=False, h0=T([[[h0]]]))
    e = math.exp(dt * a)
    assert gr["du"].item() == pytest.approx(c * dt * b, rel=1e-14)
    assert gr["ddelta"].item() == pytest.approx(c * (a * e * h0 + b * u), rel=1e-14)
    assert gr["dA"].item() == pytest.approx(c * h0 * dt * e, rel=1e-14)
    assert gr["dB"].item() == pytest.approx(c * dt * u, rel=1e-14)
    assert gr["dC"].item() == pytest.approx(e * h0 + dt * b * u, rel=1e-14)
    assert gr["dh0"].item() == pytest.approx(c * e, rel=1e-14)


# ---------------------------------------------------------------- conv1d + SiLU
def test_conv1d_matches_torch_conv1d():
    """The causal depthwise convolution is torch's grouped conv1d (a
    cross-correlation) with K-1 zeros of left padding, truncated to L."""
    rng = np.random.default_rng(0)
    for (Bt, L, Dm, K) in [(2, 11, 5, 4), (1, 3, 7, 4), (3, 9, 4, 2), (1, 6, 3, 1)]:
        x = rng.standard_normal((Bt, L, Dm))
        w = rng.standard_normal((Dm, K))
        b = rng.standard_normal(Dm)
        u, _ = oracle.causal_conv1d_silu(x, w, b)
        s = torch.nn.functional.conv1d(torch.tensor(x).permute(0, 2, 1), torch.tensor(w)[:, None, :],
                                       torch.tensor(b), padding=K - 1, groups=Dm)[:, :, :L]
        ref = torch.nn.functional.silu(s).permute(0, 2, 1).numpy()
        np.testing.assert_allclose(u, ref, rtol=1e-13, atol=1e-13)


def test_conv1d_impulse_response_and_causality():
    """A unit impulse at t0 gives silu(w[d, K-1-(t-t0)]) for t0 <= t < t0+K,
    silu(0) = 0 elsewhere: the last tap multiplies the current token, and
    nothing reaches earlier times."""
    L, Dm, K, t0 = 12, 3, 4, 5
    w = np.arange(1.0, 1.0 + Dm * K).reshape(Dm, K) / 10.0
    x = np.zeros((1, L, Dm))
    x[0, t0, :] = 1.0
    u, _ = oracle.causal_conv1d_silu(x, w, silu=False)
    for t in range(L):
        expect = w[:, K - 1 - (t - t0)] if t0 <= t < t0 + K else np.zeros(Dm)
        np.testing.assert_array_equal(u[0, t], expect)


def test_conv1d_state_carries_chunks():
    """Splitting the sequence and passing the returned state reproduces one
    call (chunked prefill)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 20, 6))
    w = rng.standard_normal((6, 4))
    b = rng.standard_normal(6)
    u, st = oracle.causal_conv1d_silu(x, w, b)
    u1, s1 = oracle.causal_conv1d_silu(x[:, :7], w, b)
    u2, s2 = oracle.causal_conv1d_silu(x[:, 7:9], w, b, state=s1)
    u3, s3 = oracle.causal_conv1d_silu(x[:, 9:], w, b, state=s2)
    np.testing.assert_allclose(np.concatenate([u1, u2, u3], 1), u, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(s3, st)
    np.testing.assert_array_equal(st, np.transpose(x[:, -3:, :], (0, 2, 1)))
