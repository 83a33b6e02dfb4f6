"""fp64 CPU oracle for the selective scan (S6) and the SSD (Mamba-2) form.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check
(`__graft_entry__.smoke`) and the CPU-baseline leg of `bench.py` may import
this package.  The HIP library never loads it and shares no code with it: the
two implementations meet only through the seeded input generators, which hold
none of the method's arithmetic.

What is here:
  * `s6_fwd`  -- the selective-scan definition (plain sequential loop over
    tokens in double precision, `ssm_oracle.c`).
  * `ssd_fwd` -- the scalar-decay-per-head recurrence whose unrolled matrix is
    the 1-semiseparable SSD matrix (same file).
  * `s6_step` -- one decode step: the same recurrence over a single token,
    starting from and returning the caller's state.
  * `causal_conv1d_silu` -- the short causal depthwise convolution and SiLU
    that produce the scan input u (numpy, float64).
  * `backward.s6_bwd` -- gradients of the selective scan by fp64 reverse-mode
    differentiation of the per-token definition (plain PyTorch CPU ops).
  * `scans`   -- the affine-pair scans (sequential, Hillis-Steele doubling,
    Blelloch up/down sweep, chunked with carry) used as pins of the carry
    logic.

Every function is pinned by `tests/test_oracle_pins.py` against values the
pages print, closed forms, brute-force sums and library routines; see the
docstrings for the passages each one follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# The mutation check of the test-suite builds altered copies of ssm_oracle.c
# and points the pins at one of them through this variable.
_LIB_OVERRIDE = os.environ.get("SSM_ORACLE_LIB")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile `ssm_oracle.c` with plain gcc -O2 (OpenMP over channels)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_s6_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                      ctypes.c_int, ctypes.c_int, dp, dp, dp,
                                      i64, i64, i64, i64, ctypes.c_int]
        lib.oracle_s6_fwd.restype = ctypes.c_int
        lib.oracle_ssd_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                       ctypes.c_int, dp, dp, dp,
                                       i64, i64, i64, i64, i64, i64, ctypes.c_int]
        lib.oracle_ssd_fwd.restype = ctypes.c_int
        _lib = lib
        return lib


def _f64(x):
    """Exact conversion of a numpy array or torch tensor (f32/bf16/f64) to a
    C-contiguous float64 numpy array."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor; bf16 and f32 widen exactly
        import torch
        x = x.detach().to("cpu").to(torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
               else (os.cpu_count() or 1))


def s6_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
           delta_softplus=True, zoh=False, h0=None, threads=None):
    """Selective scan forward in fp64 (the plain definition).

    u, delta, z: [Bt, L, Dm]; A: [Dm, N]; B, C: [Bt, L, N]; D, delta_bias: [Dm];
    h0: [Bt, Dm, N].  Returns (y [Bt, L, Dm], h_last [Bt, Dm, N]) as float64.
    Follows the per-token discretisation and readout of the Transformer-math
    "Selective state space" article ("Discretization becomes a per-token
    operation") and the sequential `selective_scan` of "12. Selective State
    Space"; zoh=True switches to the exact zero-order-hold input term given in
    the same section.
    """
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, delta_bias, h0 = map(_f64, (D, z, delta_bias, h0))
    Bt, L, Dm = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (Dm, N)
    assert B.shape == (Bt, L, N) and C.shape == (Bt, L, N)
    if z is not None:
        assert z.shape == u.shape
    if D is not None:
        assert D.shape == (Dm,)
    if delta_bias is not None:
        assert delta_bias.shape == (Dm,)
    if h0 is not None:
        assert h0.shape == (Bt, Dm, N)
    y = np.empty((Bt, L, Dm), dtype=np.float64)
    h_last = np.empty((Bt, Dm, N), dtype=np.float64)
    rc = _load().oracle_s6_fwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(delta_bias), int(bool(delta_softplus)), int(bool(zoh)), _ptr(h0),
        _ptr(y), _ptr(h_last), Bt, L, Dm, N,
        int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_s6_fwd rejected its arguments")
    return y, h_last


def ssd_fwd(X, delta, A, B, C, D=None, z=None, delta_bias=None,
            delta_softplus=True, h0=None, threads=None):
    """SSD (scalar decay per head) forward in fp64.

    X, z: [Bt, L, H, P]; delta: [Bt, L, H]; A: [H]; B, C: [Bt, L, G, N];
    D, delta_bias: [H]; h0: [Bt, H, P, N].  Returns (Y, h_last).
    The recurrence with a scalar transition per head whose unrolled form is
    Y = (M o (C B^T)) X, per the SSD section of "Mamba & Mamba-2
    Architecture".
    """
    X, delta, A, B, C = map(_f64, (X, delta, A, B, C))
    D, z, delta_bias, h0 = map(_f64, (D, z, delta_bias, h0))
    Bt, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    assert delta.shape == (Bt, L, H) and A.shape == (H,)
    assert B.shape == (Bt, L, G, N) and C.shape == (Bt, L, G, N)
    if z is not None:
        assert z.shape == X.shape
    if h0 is not None:
        assert h0.shape == (Bt, H, P, N)
    Y = np.empty((Bt, L, H, P), dtype=np.float64)
    h_last = np.empty((Bt, H, P, N), dtype=np.float64)
    rc = _load().oracle_ssd_fwd(
        _ptr(X), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0), _ptr(Y),
        _ptr(h_last), Bt, L, H, P, G, N, int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_ssd_fwd rejected its arguments")
    return Y, h_last


def s6_step(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
            delta_softplus=True, zoh=False, threads=None):
    """One decode step in fp64: the recurrence of `s6_fwd` over a single token.

    Decoding runs the plain recurrence one token at a time against a constant
    D x N state per sequence (Transformer-math "Selective state space"
    article, section "What it costs at inference, and on a CPU"), so a step is
    `s6_fwd` with L = 1 and h0 = state.
    state: [Bt, Dm, N]; u, delta, z: [Bt, Dm]; A: [Dm, N]; B, C: [Bt, N];
    D, delta_bias: [Dm].  Returns (y [Bt, Dm], new_state [Bt, Dm, N]), float64.
    """
    state, u, delta, A, B, C = map(_f64, (state, u, delta, A, B, C))
    D, z, delta_bias = map(_f64, (D, z, delta_bias))
    y, h = s6_fwd(u[:, None, :], delta[:, None, :], A, B[:, None, :], C[:, None, :], D=D,
                  z=None if z is None else z[:, None, :], delta_bias=delta_bias,
                  delta_softplus=delta_softplus, zoh=zoh, h0=state, threads=threads)
    return y[:, 0, :], h


def causal_conv1d_silu(x, weight, bias=None, state=None, silu=True):
    """Causal depthwise convolution over tokens, then SiLU, in fp64.

    In the Mamba block the input of the selective SSM is first mixed over a
    few neighbouring tokens, channel by channel and looking only backwards,
    then put through SiLU (temporalbook "Selective State-Space Models
    (Mamba)", section 4; width d_conv = 4 in the block constructor of
    section 5).  Reading: per channel d,
        s[b,t,d] = bias[d] + sum_{k<K} weight[d,k] * x[b, t-(K-1)+k, d]
    (the last tap multiplies the current token), with x at negative times taken
    from `state` [B, D, K-1] (oldest first) or zero; u = s * sigmoid(s).
    x: [B, L, D]; weight: [D, K].  Returns (u [B, L, D], new_state [B, D, K-1]),
    the new state being the last K-1 inputs (with the old state before them).
    """
    x, weight, bias, state = map(_f64, (x, weight, bias, state))
    Bt, L, Dm = x.shape
    K = weight.shape[1]
    hist = np.zeros((Bt, K - 1, Dm)) if state is None else np.transpose(state, (0, 2, 1))
    xe = np.concatenate([hist, x], axis=1)             # [B, K-1+L, D]
    s = np.zeros((Bt, L, Dm)) if bias is None else np.broadcast_to(bias, (Bt, L, Dm)).copy()
    for k in range(K):
        s += weight[:, k][None, None, :] * xe[:, k:k + L, :]
    u = s * (1.0 / (1.0 + np.exp(-s))) if silu else s
    new_state = np.transpose(xe[:, L:, :], (0, 2, 1)).copy() if K > 1 else np.zeros((Bt, Dm, 0))
    return u, new_state
