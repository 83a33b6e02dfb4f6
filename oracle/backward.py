"""Gradients of the selective scan in fp64 (oracle side, TEST INFRASTRUCTURE ONLY).

The forward pass here is the plain per-token definition (the discretisation
and readout of the Transformer-math "Selective state space" article, section
"Discretization becomes a per-token operation", with the gate of section 4 of
the temporalbook "Selective State-Space Models (Mamba)" chapter), written
with PyTorch CPU tensor ops in float64 and looped over tokens; PyTorch's
reverse-mode differentiation of that loop gives the gradients.  Recomputing
the states instead of storing them (the backward pass the pages describe in
"Why the fused kernel is the real contribution" of the same article) is a
property of the GPU kernels, not of the values: the gradients are those of
the definition.

Pinned by tests/test_oracle_pins.py against central finite differences of the
C oracle (`oracle.s6_fwd`, separate code) and a one-step closed form.
"""
from __future__ import annotations

import torch


def _t(x):
    if x is None:
        return None
    if not isinstance(x, torch.Tensor):
        x = torch.as_tensor(x)
    return x.detach().to("cpu", torch.float64).clone()


def _softplus(x):
    # log(1 + e^x) = max(x, 0) + log1p(e^-|x|), no threshold switch
    return torch.clamp(x, min=0.0) + torch.log1p(torch.exp(-torch.abs(x)))


def s6_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, delta_softplus=True,
           h0=None, dh_last=None):
    """Gradients of L = sum(dy * y) + sum(dh_last * h_last) for the S6 scan.

    Shapes as `oracle.s6_fwd` (u, delta, z, dy: [Bt, L, Dm]; A: [Dm, N];
    B, C: [Bt, L, N]; D, delta_bias: [Dm]; h0, dh_last: [Bt, Dm, N]).
    Returns a dict of float64 tensors: du, ddelta, dA, dB, dC, and dD, dz,
    ddelta_bias, dh0 for the optional inputs that were given.
    """
    u, delta, A, B, C, dy = map(_t, (u, delta, A, B, C, dy))
    D, z, delta_bias, h0, dh_last = map(_t, (D, z, delta_bias, h0, dh_last))
    Bt, L, Dm = u.shape
    N = A.shape[1]
    leaves = {"u": u, "delta": delta, "A": A, "B": B, "C": C, "D": D, "z": z,
              "delta_bias": delta_bias, "h0": h0}
    for v in leaves.values():
        if v is not None:
            v.requires_grad_(True)
    h = h0 if h0 is not None else torch.zeros(Bt, Dm, N, dtype=torch.float64)
    ys = []
    for t in range(L):
        x = delta[:, t, :] + (delta_bias if delta_bias is not None else 0.0)
        dt = _softplus(x) if delta_softplus else x
        h = torch.exp(dt[:, :, None] * A[None]) * h + (dt * u[:, t, :])[:, :, None] * B[:, t, None, :]
        yv = (h * C[:, t, None, :]).sum(-1)
        if D is not None:
            yv = yv + D * u[:, t, :]
        if z is not None:
            zt = z[:, t, :]
            yv = yv * zt * torch.sigmoid(zt)
        ys.append(yv)
    loss = (torch.stack(ys, 1) * dy).sum() if L > 0 else torch.zeros((), dtype=torch.float64)
    if dh_last is not None:
        loss = loss + (h * dh_last).sum()
    names = [k for k, v in leaves.items() if v is not None]
    grads = torch.autograd.grad(loss, [leaves[k] for k in names], allow_unused=True)
    out = {}
    for k, g in zip(names, grads):
        g = torch.zeros_like(leaves[k]) if g is None else g
        out["d" + k if k != "h0" else "dh0"] = g.detach()
    return out
