"""MI355X-native selective scan (S6) and SSD chunked forward.

Python entry points with the same names as the C ABI in include/ssm.h.  They
only marshal arguments: every arithmetic step runs in the HIP kernels of
libssm_mi355x.so.  PyTorch supplies device memory and the current stream.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _native
from ._native import SSMError

__all__ = ["selective_scan_fwd", "selective_scan_conv_fwd", "selective_scan_bwd", "ssd_chunk_fwd", "selective_state_update",
           "causal_conv1d_silu",
           "selective_scan_workspace_bytes",
           "selective_scan_segments", "selective_scan_lanes", "ssd_chunk_workspace_bytes", "SSMError"]

_DT = {torch.float32: _native.SSM_F32, torch.bfloat16: _native.SSM_BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev_tensor(name, t, dtype=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def selective_scan_workspace_bytes(B: int, L: int, D: int, N: int, dtype=torch.bfloat16) -> int:
    return int(_native.load().ssm_selective_scan_workspace_bytes(B, L, D, N, _DT[dtype]))


def selective_scan_segments(B: int, L: int, D: int, N: int) -> int:
    return int(_native.load().ssm_selective_scan_segments(B, L, D, N))


def selective_scan_lanes(B: int, L: int, D: int, N: int) -> bool:
    """True if a forward call at these sizes (without ZOH; with or without the
    fused convolution) runs the state-per-lane kernel, unsplit."""
    return bool(_native.load().ssm_selective_scan_lanes(B, L, D, N))


def ssd_chunk_workspace_bytes(B, L, H, P, G, N, chunk, dtype=torch.bfloat16) -> int:
    return int(_native.load().ssm_ssd_chunk_workspace_bytes(B, L, H, P, G, N, chunk, _DT[dtype]))


def selective_scan_fwd(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                       B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                       z: Optional[torch.Tensor] = None,
                       delta_bias: Optional[torch.Tensor] = None,
                       delta_softplus: bool = True, zoh: bool = False,
                       h0: Optional[torch.Tensor] = None, return_last_state: bool = True,
                       out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       seq_lens: Optional[torch.Tensor] = None
                       ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """S6 selective scan forward (ssm_selective_scan_fwd).

    u, delta, z: [Bt, L, Dm]; A: [Dm, N] fp32; B, C: [Bt, L, N] (dtype of u);
    D, delta_bias: [Dm] fp32; h0: [Bt, Dm, N] fp32.  Returns (y, h_last).
    seq_lens: optional int32 [Bt] -- row b runs its first seq_lens[b] tokens
    (ssm_selective_scan_fwd_varlen); later positions of y are left untouched.
    """
    lib = _native.load()
    if u.dtype not in _DT:
        raise TypeError(f"u must be float32 or bfloat16 (got {u.dtype})")
    dev = u.device
    dt = u.dtype
    u = _dev_tensor("u", u, dt, dev)
    delta = _dev_tensor("delta", delta, dt, dev)
    B = _dev_tensor("B", B, dt, dev)
    C = _dev_tensor("C", C, dt, dev)
    z = _dev_tensor("z", z, dt, dev)
    A = _dev_tensor("A", A, torch.float32, dev)
    D = _dev_tensor("D", D, torch.float32, dev)
    delta_bias = _dev_tensor("delta_bias", delta_bias, torch.float32, dev)
    h0 = _dev_tensor("h0", h0, torch.float32, dev)
    if u.dim() != 3:
        raise ValueError("u must be [B, L, D]")
    Bt, L, Dm = u.shape
    N = A.shape[-1]
    shapes = {"delta": (delta, (Bt, L, Dm)), "A": (A, (Dm, N)), "B": (B, (Bt, L, N)),
              "C": (C, (Bt, L, N)), "z": (z, (Bt, L, Dm)), "D": (D, (Dm,)),
              "delta_bias": (delta_bias, (Dm,)), "h0": (h0, (Bt, Dm, N))}
    for name, (t, shp) in shapes.items():
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    y = out if out is not None else torch.empty((Bt, L, Dm), dtype=dt, device=dev)
    _dev_tensor("out", y, dt, dev)
    h_last = torch.empty((Bt, Dm, N), dtype=torch.float32, device=dev) if return_last_state else None
    ws_need = int(lib.ssm_selective_scan_workspace_bytes(Bt, L, Dm, N, _DT[dt]))
    if ws_need and (workspace is None or workspace.numel() * workspace.element_size() < ws_need):
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    flags = (_native.FLAG_DELTA_SOFTPLUS if delta_softplus else 0) | (_native.FLAG_ZOH if zoh else 0)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if seq_lens is not None:
        seq_lens = _dev_tensor("seq_lens", seq_lens, torch.int32, dev)
        if tuple(seq_lens.shape) != (Bt,):
            raise ValueError(f"seq_lens has shape {tuple(seq_lens.shape)}, expected {(Bt,)}")
        rc = lib.ssm_selective_scan_fwd_varlen(
            _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            flags, _ptr(h0), _ptr(y), _ptr(h_last), _ptr(seq_lens), Bt, L, Dm, N, _DT[dt],
            _ptr(workspace), ws_bytes, _stream_handle(dev))
        _native.check(rc, "ssm_selective_scan_fwd_varlen")
        return y, h_last
    rc = lib.ssm_selective_scan_fwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        flags, _ptr(h0), _ptr(y), _ptr(h_last), Bt, L, Dm, N, _DT[dt],
        _ptr(workspace), ws_bytes, _stream_handle(dev))
    _native.check(rc, "ssm_selective_scan_fwd")
    return y, h_last


def ssd_chunk_fwd(X: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                  C: torch.Tensor, D: Optional[torch.Tensor] = None,
                  z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                  delta_softplus: bool = True, h0: Optional[torch.Tensor] = None,
                  chunk: int = 256, return_last_state: bool = True,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Mamba-2 SSD chunked forward (ssm_ssd_chunk_fwd).

    X, z: [Bt, L, H, P]; delta: [Bt, L, H]; A: [H] fp32; B, C: [Bt, L, G, N];
    D, delta_bias: [H] fp32; h0: [Bt, H, P, N] fp32.  Returns (Y, h_last).
    """
    lib = _native.load()
    if X.dtype not in _DT:
        raise TypeError(f"X must be float32 or bfloat16 (got {X.dtype})")
    dev, dt = X.device, X.dtype
    X = _dev_tensor("X", X, dt, dev)
    delta = _dev_tensor("delta", delta, dt, dev)
    B = _dev_tensor("B", B, dt, dev)
    C = _dev_tensor("C", C, dt, dev)
    z = _dev_tensor("z", z, dt, dev)
    A = _dev_tensor("A", A, torch.float32, dev)
    D = _dev_tensor("D", D, torch.float32, dev)
    delta_bias = _dev_tensor("delta_bias", delta_bias, torch.float32, dev)
    h0 = _dev_tensor("h0", h0, torch.float32, dev)
    if X.dim() != 4 or B.dim() != 4:
        raise ValueError("X must be [B, L, H, P] and B/C [B, L, G, N]")
    Bt, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    shapes = {"delta": (delta, (Bt, L, H)), "A": (A, (H,)), "B": (B, (Bt, L, G, N)),
              "C": (C, (Bt, L, G, N)), "z": (z, (Bt, L, H, P)), "D": (D, (H,)),
              "delta_bias": (delta_bias, (H,)), "h0": (h0, (Bt, H, P, N))}
    for name, (t, shp) in shapes.items():
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    Y = out if out is not None else torch.empty((Bt, L, H, P), dtype=dt, device=dev)
    _dev_tensor("out", Y, dt, dev)
    h_last = torch.empty((Bt, H, P, N), dtype=torch.float32, device=dev) if return_last_state else None
    ws_need = int(lib.ssm_ssd_chunk_workspace_bytes(Bt, L, H, P, G, N, chunk, _DT[dt]))
    if ws_need and (workspace is None or workspace.numel() * workspace.element_size() < ws_need):
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = _native.FLAG_DELTA_SOFTPLUS if delta_softplus else 0
    rc = lib.ssm_ssd_chunk_fwd(
        _ptr(X), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        flags, _ptr(h0), _ptr(Y), _ptr(h_last), Bt, L, H, P, G, N, chunk, _DT[dt],
        _ptr(workspace), ws_bytes, _stream_handle(dev))
    _native.check(rc, "ssm_ssd_chunk_fwd")
    return Y, h_last


def selective_state_update(state: torch.Tensor, u: torch.Tensor, delta: torch.Tensor,
                           A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                           D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                           delta_bias: Optional[torch.Tensor] = None,
                           delta_softplus: bool = True, zoh: bool = False,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step of the selective scan (ssm_selective_state_update).

    state: [Bt, Dm, N] fp32, updated in place; u, delta, z: [Bt, Dm];
    A: [Dm, N] fp32; B, C: [Bt, N] (dtype of u); D, delta_bias: [Dm] fp32.
    Returns y [Bt, Dm].
    """
    lib = _native.load()
    if u.dtype not in _DT:
        raise TypeError(f"u must be float32 or bfloat16 (got {u.dtype})")
    dev, dt = u.device, u.dtype
    state = _dev_tensor("state", state, torch.float32, dev)
    u = _dev_tensor("u", u, dt, dev)
    delta = _dev_tensor("delta", delta, dt, dev)
    B = _dev_tensor("B", B, dt, dev)
    C = _dev_tensor("C", C, dt, dev)
    z = _dev_tensor("z", z, dt, dev)
    A = _dev_tensor("A", A, torch.float32, dev)
    D = _dev_tensor("D", D, torch.float32, dev)
    delta_bias = _dev_tensor("delta_bias", delta_bias, torch.float32, dev)
    if u.dim() != 2:
        raise ValueError("u must be [B, D]")
    Bt, Dm = u.shape
    N = A.shape[-1]
    shapes = {"state": (state, (Bt, Dm, N)), "delta": (delta, (Bt, Dm)), "A": (A, (Dm, N)),
              "B": (B, (Bt, N)), "C": (C, (Bt, N)), "z": (z, (Bt, Dm)), "D": (D, (Dm,)),
              "delta_bias": (delta_bias, (Dm,))}
    for name, (t, shp) in shapes.items():
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    y = out if out is not None else torch.empty((Bt, Dm), dtype=dt, device=dev)
    _dev_tensor("out", y, dt, dev)
    flags = (_native.FLAG_DELTA_SOFTPLUS if delta_softplus else 0) | (_native.FLAG_ZOH if zoh else 0)
    rc = lib.ssm_selective_state_update(
        _ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(delta_bias), flags, _ptr(y), Bt, Dm, N, _DT[dt], _stream_handle(dev))
    _native.check(rc, "ssm_selective_state_update")
    return y


def selective_scan_bwd(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                       C: torch.Tensor, dy: torch.Tensor, D: Optional[torch.Tensor] = None,
                       z: Optional[torch.Tensor] = None,
                       delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = True,
                       h0: Optional[torch.Tensor] = None, dh_last: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> dict:
    """Gradients of the S6 scan (ssm_selective_scan_bwd), states recomputed.

    Inputs as selective_scan_fwd plus dy [Bt, L, Dm] (dtype of u) and
    dh_last [Bt, Dm, N] fp32.  Returns a dict with du, ddelta (dtype of u),
    dA [Dm, N], dB, dC [Bt, L, N] (fp32), and dD, dz, ddelta_bias, dh0 for the
    optional inputs that were given.
    """
    lib = _native.load()
    if u.dtype not in _DT:
        raise TypeError(f"u must be float32 or bfloat16 (got {u.dtype})")
    dev, dt = u.device, u.dtype
    u = _dev_tensor("u", u, dt, dev)
    delta = _dev_tensor("delta", delta, dt, dev)
    B = _dev_tensor("B", B, dt, dev)
    C = _dev_tensor("C", C, dt, dev)
    z = _dev_tensor("z", z, dt, dev)
    dy = _dev_tensor("dy", dy, dt, dev)
    A = _dev_tensor("A", A, torch.float32, dev)
    D = _dev_tensor("D", D, torch.float32, dev)
    delta_bias = _dev_tensor("delta_bias", delta_bias, torch.float32, dev)
    h0 = _dev_tensor("h0", h0, torch.float32, dev)
    dh_last = _dev_tensor("dh_last", dh_last, torch.float32, dev)
    if u.dim() != 3:
        raise ValueError("u must be [B, L, D]")
    Bt, L, Dm = u.shape
    N = A.shape[-1]
    shapes = {"delta": (delta, (Bt, L, Dm)), "A": (A, (Dm, N)), "B": (B, (Bt, L, N)),
              "C": (C, (Bt, L, N)), "z": (z, (Bt, L, Dm)), "dy": (dy, (Bt, L, Dm)),
              "D": (D, (Dm,)), "delta_bias": (delta_bias, (Dm,)), "h0": (h0, (Bt, Dm, N)),
              "dh_last": (dh_last, (Bt, Dm, N))}
    for name, (t, shp) in shapes.items():
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    f32 = torch.float32
    out = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u),
           "dA": torch.empty((Dm, N), dtype=f32, device=dev),
           "dB": torch.empty((Bt, L, N), dtype=f32, device=dev),
           "dC": torch.empty((Bt, L, N), dtype=f32, device=dev)}
    if D is not None:
        out["dD"] = torch.empty((Dm,), dtype=f32, device=dev)
    if z is not None:
        out["dz"] = torch.empty_like(z)
    if delta_bias is not None:
        out["ddelta_bias"] = torch.empty((Dm,), dtype=f32, device=dev)
    if h0 is not None:
        out["dh0"] = torch.empty((Bt, Dm, N), dtype=f32, device=dev)
    need = int(lib.ssm_selective_scan_bwd_workspace_bytes(Bt, L, Dm, N, _DT[dt]))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    flags = _native.FLAG_DELTA_SOFTPLUS if delta_softplus else 0
    rc = lib.ssm_selective_scan_bwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        flags, _ptr(h0), _ptr(dy), _ptr(dh_last), _ptr(out["du"]), _ptr(out["ddelta"]),
        _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out.get("dD")),
        _ptr(out.get("dz")), _ptr(out.get("ddelta_bias")), _ptr(out.get("dh0")),
        Bt, L, Dm, N, _DT[dt], _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_handle(dev))
    _native.check(rc, "ssm_selective_scan_bwd")
    return out


def causal_conv1d_silu(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                       state: Optional[torch.Tensor] = None, silu: bool = True,
                       return_state: bool = False, out: Optional[torch.Tensor] = None):
    """Causal depthwise conv1d over tokens, then SiLU (ssm_causal_conv1d_silu).

    x: [Bt, L, Dm] (float32 or bfloat16); weight: [Dm, K] fp32; bias: [Dm]
    fp32; state: [Bt, Dm, K-1] fp32 (previous chunk's last inputs).  Returns u
    (same dtype as x), or (u, new_state) with return_state.
    """
    lib = _native.load()
    if x.dtype not in _DT:
        raise TypeError(f"x must be float32 or bfloat16 (got {x.dtype})")
    dev, dt = x.device, x.dtype
    x = _dev_tensor("x", x, dt, dev)
    weight = _dev_tensor("weight", weight, torch.float32, dev)
    bias = _dev_tensor("bias", bias, torch.float32, dev)
    state = _dev_tensor("state", state, torch.float32, dev)
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be [B, L, D] and weight [D, K]")
    Bt, L, Dm = x.shape
    K = weight.shape[1]
    shapes = {"weight": (weight, (Dm, K)), "bias": (bias, (Dm,)), "state": (state, (Bt, Dm, K - 1))}
    for name, (t, shp) in shapes.items():
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    u = out if out is not None else torch.empty_like(x)
    _dev_tensor("out", u, dt, dev)
    new_state = torch.empty((Bt, Dm, K - 1), dtype=torch.float32, device=dev) if return_state else None
    rc = lib.ssm_causal_conv1d_silu(_ptr(x), _ptr(weight), _ptr(bias), _ptr(state), int(bool(silu)),
                                    _ptr(u), _ptr(new_state), Bt, L, Dm, K, _DT[dt],
                                    _stream_handle(dev))
    _native.check(rc, "ssm_causal_conv1d_silu")
    return (u, new_state) if return_state else u


def selective_scan_conv_fwd(x: torch.Tensor, conv_weight: torch.Tensor,
                            conv_bias: Optional[torch.Tensor], delta: torch.Tensor,
                            A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                            D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                            delta_bias: Optional[torch.Tensor] = None,
                            delta_softplus: bool = True, h0: Optional[torch.Tensor] = None,
                            conv_state: Optional[torch.Tensor] = None,
                            return_u: bool = False, return_conv_state: bool = False,
                            out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None) -> dict:
    """Causal conv1d + SiLU fused in front of the S6 scan (ssm_selective_scan_conv_fwd).

    x: [Bt, L, Dm] (the convolution's input, in place of u); conv_weight:
    [Dm, K] fp32; conv_bias: [Dm] fp32; conv_state: [Bt, Dm, K-1] fp32; the
    rest as selective_scan_fwd (N = 16).  Returns a dict with y and h_last,
    plus u and conv_state when requested.
    """
    lib = _native.load()
    if x.dtype not in _DT:
        raise TypeError(f"x must be float32 or bfloat16 (got {x.dtype})")
    dev, dt = x.device, x.dtype
    x = _dev_tensor("x", x, dt, dev)
    conv_weight = _dev_tensor("conv_weight", conv_weight, torch.float32, dev)
    conv_bias = _dev_tensor("conv_bias", conv_bias, torch.float32, dev)
    conv_state = _dev_tensor("conv_state", conv_state, torch.float32, dev)
    delta = _dev_tensor("delta", delta, dt, dev)
    B = _dev_tensor("B", B, dt, dev)
    C = _dev_tensor("C", C, dt, dev)
    z = _dev_tensor("z", z, dt, dev)
    A = _dev_tensor("A", A, torch.float32, dev)
    D = _dev_tensor("D", D, torch.float32, dev)
    delta_bias = _dev_tensor("delta_bias", delta_bias, torch.float32, dev)
    h0 = _dev_tensor("h0", h0, torch.float32, dev)
    if x.dim() != 3 or conv_weight.dim() != 2:
        raise ValueError("x must be [B, L, D] and conv_weight [D, K]")
    Bt, L, Dm = x.shape
    N = A.shape[-1]
    K = conv_weight.shape[1]
    shapes = {"delta": (delta, (Bt, L, Dm)), "A": (A, (Dm, N)), "B": (B, (Bt, L, N)),
              "C": (C, (Bt, L, N)), "z": (z, (Bt, L, Dm)), "D": (D, (Dm,)),
              "delta_bias": (delta_bias, (Dm,)), "h0": (h0, (Bt, Dm, N)),
              "conv_weight": (conv_weight, (Dm, K)), "conv_bias": (conv_bias, (Dm,)),
              "conv_state": (conv_state, (Bt, Dm, K - 1))}
    for name, (t, shp) in shapes.items():
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    y = out if out is not None else torch.empty((Bt, L, Dm), dtype=dt, device=dev)
    _dev_tensor("out", y, dt, dev)
    h_last = torch.empty((Bt, Dm, N), dtype=torch.float32, device=dev)
    u = torch.empty_like(x) if return_u else None
    cs = torch.empty((Bt, Dm, K - 1), dtype=torch.float32, device=dev) if return_conv_state else None
    ws_need = int(lib.ssm_selective_scan_workspace_bytes(Bt, L, Dm, N, _DT[dt]))
    if ws_need and (workspace is None or workspace.numel() * workspace.element_size() < ws_need):
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = _native.FLAG_DELTA_SOFTPLUS if delta_softplus else 0
    rc = lib.ssm_selective_scan_conv_fwd(
        _ptr(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), _ptr(cs), K, _ptr(u),
        _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), flags,
        _ptr(h0), _ptr(y), _ptr(h_last), Bt, L, Dm, N, _DT[dt], _ptr(workspace), ws_bytes,
        _stream_handle(dev))
    _native.check(rc, "ssm_selective_scan_conv_fwd")
    res = {"y": y, "h_last": h_last}
    if return_u:
        res["u"] = u
    if return_conv_state:
        res["conv_state"] = cs
    return res
