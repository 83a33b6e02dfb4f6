"""MI355X-native selective scan (S6) and SSD chunked forward.

Python entry points with the same names as the C ABI in include/ssm.h.  They
only marshal arguments: every arithmetic step runs in the HIP kernels of
libssm_mi355x.so.  PyTorch supplies device memory and the current stream.

Every wrapper checks the shape and dtype of each tensor it passes (inputs,
caller-supplied outputs and workspace) before it checks devices and layout,
and raises before anything reaches the library: the kernels write through
bare pointers, so a wrongly sized buffer must never get that far.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _native
from ._native import SSMError

__all__ = ["selective_scan_fwd", "selective_scan_fwd_noalloc", "selective_scan_conv_fwd",
           "selective_scan_bwd", "selective_scan_fwd_ckpt", "selective_scan_ckpt_bytes",
           "ssd_chunk_fwd", "selective_state_update",
           "causal_conv1d_silu", "selective_scan_workspace_bytes",
           "selective_scan_segments", "selective_scan_lanes", "selective_scan_bwd_segments",
           "ssd_chunk_workspace_bytes",
           "SSMError"]

_DT = {torch.float32: _native.SSM_F32, torch.bfloat16: _native.SSM_BF16}
_F32 = torch.float32


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


def _check_args(device, *specs) -> None:
    """specs: (name, tensor or None, expected shape, dtype).  Types, shapes and
    dtypes of every argument are checked first, then device and contiguity."""
    for name, t, shape, dtype in specs:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    for name, t, _shape, dtype in specs:
        _dev_tensor(name, t, dtype, device)


def _check_workspace(ws, need: int, device):
    """A caller-supplied workspace: a contiguous uint8 tensor on the call's
    device holding at least `need` bytes, or None."""
    if ws is None:
        return None
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if ws.dtype != torch.uint8:
        raise TypeError(f"workspace must be uint8 (got {ws.dtype})")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, the call needs {need}")
    if ws.device.type != "cuda" or ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws


def _workspace(ws, need: int, device):
    ws = _check_workspace(ws, need, device)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, (0 if ws is None else ws.numel())


def _act_dtype(name, t):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in _DT:
        raise TypeError(f"{name} must be float32 or bfloat16 (got {t.dtype})")
    return t.dtype


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def selective_scan_workspace_bytes(B: int, L: int, D: int, N: int, dtype=torch.bfloat16) -> int:
    return int(_native.load().ssm_selective_scan_workspace_bytes(B, L, D, N, _DT[dtype]))


def selective_scan_segments(B: int, L: int, D: int, N: int) -> int:
    return int(_native.load().ssm_selective_scan_segments(B, L, D, N))


def selective_scan_bwd_segments(B: int, L: int, D: int, N: int) -> int:
    """Sequence segments a backward call uses at these sizes (1: one pass)."""
    return int(_native.load().ssm_selective_scan_bwd_segments(B, L, D, N))


def selective_scan_lanes(B: int, L: int, D: int, N: int) -> bool:
    """True if a forward call at these sizes (without ZOH; with or without the
    fused convolution) runs the state-per-lane kernel."""
    return bool(_native.load().ssm_selective_scan_lanes(B, L, D, N))


def ssd_chunk_workspace_bytes(B, L, H, P, G, N, chunk, dtype=torch.bfloat16) -> int:
    return int(_native.load().ssm_ssd_chunk_workspace_bytes(B, L, H, P, G, N, chunk, _DT[dtype]))


def _s6_prepare(u, delta, A, B, C, D, z, delta_bias, h0, out, name="u"):
    dt = _act_dtype(name, u)
    if u.dim() != 3:
        raise ValueError(f"{name} must be [B, L, D]")
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be [D, N]")
    Bt, L, Dm = u.shape
    N = A.shape[-1]
    dev = u.device
    _check_args(dev, (name, u, (Bt, L, Dm), dt), ("delta", delta, (Bt, L, Dm), dt),
                ("A", A, (Dm, N), _F32), ("B", B, (Bt, L, N), dt), ("C", C, (Bt, L, N), dt),
                ("D", D, (Dm,), _F32), ("z", z, (Bt, L, Dm), dt),
                ("delta_bias", delta_bias, (Dm,), _F32), ("h0", h0, (Bt, Dm, N), _F32),
                ("out", out, (Bt, L, Dm), dt))
    return dt, dev, Bt, L, Dm, N


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
    dt, dev, Bt, L, Dm, N = _s6_prepare(u, delta, A, B, C, D, z, delta_bias, h0, out)
    if seq_lens is not None:
        _check_args(dev, ("seq_lens", seq_lens, (Bt,), torch.int32))
    lib = _native.load()
    ws_need = int(lib.ssm_selective_scan_workspace_bytes(Bt, L, Dm, N, _DT[dt]))
    workspace, ws_bytes = _workspace(workspace, ws_need, dev)
    y = out if out is not None else torch.empty((Bt, L, Dm), dtype=dt, device=dev)
    h_last = torch.empty((Bt, Dm, N), dtype=_F32, device=dev) if return_last_state else None
    flags = (_native.FLAG_DELTA_SOFTPLUS if delta_softplus else 0) | (_native.FLAG_ZOH if zoh else 0)
    if seq_lens is not None:
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


def selective_scan_ckpt_bytes(B: int, L: int, D: int, N: int, dtype=torch.bfloat16) -> int:
    return int(_native.load().ssm_selective_scan_ckpt_bytes(B, L, D, N, _DT[dtype]))


def selective_scan_fwd_ckpt(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                            B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                            z: Optional[torch.Tensor] = None,
                            delta_bias: Optional[torch.Tensor] = None,
                            delta_softplus: bool = True, h0: Optional[torch.Tensor] = None,
                            return_last_state: bool = True, out: Optional[torch.Tensor] = None,
                            ckpt: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None):
    """S6 forward for training (ssm_selective_scan_fwd_ckpt): the forward
    call that also saves the state entering every 16-token tile, for
    selective_scan_bwd(..., ckpt=...).  Arguments as selective_scan_fwd (no
    ZOH, N <= 16); ckpt: optional fp32 [Bt, Dm, ceil(L/16), N] to fill.
    Returns (y, h_last, ckpt)."""
    dt, dev, Bt, L, Dm, N = _s6_prepare(u, delta, A, B, C, D, z, delta_bias, h0, out)
    nck = (L + 15) // 16
    _check_args(dev, ("ckpt", ckpt, (Bt, Dm, nck, N), _F32))
    lib = _native.load()
    ws_need = int(lib.ssm_selective_scan_workspace_bytes(Bt, L, Dm, N, _DT[dt]))
    workspace, ws_bytes = _workspace(workspace, ws_need, dev)
    y = out if out is not None else torch.empty((Bt, L, Dm), dtype=dt, device=dev)
    h_last = torch.empty((Bt, Dm, N), dtype=_F32, device=dev) if return_last_state else None
    if ckpt is None:
        ckpt = torch.empty((Bt, Dm, nck, N), dtype=_F32, device=dev)
    flags = _native.FLAG_DELTA_SOFTPLUS if delta_softplus else 0
    rc = lib.ssm_selective_scan_fwd_ckpt(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        flags, _ptr(h0), _ptr(y), _ptr(h_last), _ptr(ckpt), Bt, L, Dm, N, _DT[dt],
        _ptr(workspace), ws_bytes, _stream_handle(dev))
    _native.check(rc, "ssm_selective_scan_fwd_ckpt")
    return y, h_last, ckpt


def selective_scan_fwd_noalloc(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                               B: torch.Tensor, C: torch.Tensor, y: torch.Tensor,
                               h_last: Optional[torch.Tensor] = None,
                               D: Optional[torch.Tensor] = None,
                               z: Optional[torch.Tensor] = None,
                               delta_bias: Optional[torch.Tensor] = None,
                               delta_softplus: bool = True, zoh: bool = False,
                               h0: Optional[torch.Tensor] = None) -> None:
    """The S6 forward through ssm_selective_scan_fwd_noalloc, for callers that
    cannot allocate: the caller passes y (and h_last), the library takes its
    scratch from a static device array, and nothing is allocated here or there.
    Calls that overlap on one GPU share that scratch and race."""
    dt, dev, Bt, L, Dm, N = _s6_prepare(u, delta, A, B, C, D, z, delta_bias, h0, y)
    _check_args(dev, ("h_last", h_last, (Bt, Dm, N), _F32))
    lib = _native.load()
    flags = (_native.FLAG_DELTA_SOFTPLUS if delta_softplus else 0) | (_native.FLAG_ZOH if zoh else 0)
    rc = lib.ssm_selective_scan_fwd_noalloc(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        flags, _ptr(h0), _ptr(y), _ptr(h_last), Bt, L, Dm, N, _DT[dt], _stream_handle(dev))
    _native.check(rc, "ssm_selective_scan_fwd_noalloc")


def ssd_chunk_fwd(X: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                  C: torch.Tensor, D: Optional[torch.Tensor] = None,
                  z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                  delta_softplus: bool = True, h0: Optional[torch.Tensor] = None,
                  chunk: int = 256, return_last_state: bool = True,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  seq_lens: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Mamba-2 SSD chunked forward (ssm_ssd_chunk_fwd).

    X, z: [Bt, L, H, P]; delta: [Bt, L, H]; A: [H] fp32; B, C: [Bt, L, G, N];
    D, delta_bias: [H] fp32; h0: [Bt, H, P, N] fp32.  Returns (Y, h_last).
    seq_lens: optional int32 [Bt] -- row b runs its first seq_lens[b] tokens
    (ssm_ssd_chunk_fwd_varlen); later positions of Y are left untouched.
    """
    dt = _act_dtype("X", X)
    if X.dim() != 4 or not isinstance(B, torch.Tensor) or B.dim() != 4:
        raise ValueError("X must be [B, L, H, P] and B/C [B, L, G, N]")
    dev = X.device
    Bt, L, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    _check_args(dev, ("X", X, (Bt, L, H, P), dt), ("delta", delta, (Bt, L, H), dt),
                ("A", A, (H,), _F32), ("B", B, (Bt, L, G, N), dt), ("C", C, (Bt, L, G, N), dt),
                ("z", z, (Bt, L, H, P), dt), ("D", D, (H,), _F32),
                ("delta_bias", delta_bias, (H,), _F32), ("h0", h0, (Bt, H, P, N), _F32),
                ("out", out, (Bt, L, H, P), dt), ("seq_lens", seq_lens, (Bt,), torch.int32))
    lib = _native.load()
    ws_need = int(lib.ssm_ssd_chunk_workspace_bytes(Bt, L, H, P, G, N, chunk, _DT[dt]))
    workspace, ws_bytes = _workspace(workspace, ws_need, dev)
    Y = out if out is not None else torch.empty((Bt, L, H, P), dtype=dt, device=dev)
    h_last = torch.empty((Bt, H, P, N), dtype=_F32, device=dev) if return_last_state else None
    flags = _native.FLAG_DELTA_SOFTPLUS if delta_softplus else 0
    head = (_ptr(X), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            flags, _ptr(h0), _ptr(Y), _ptr(h_last))
    tail = (Bt, L, H, P, G, N, chunk, _DT[dt], _ptr(workspace), ws_bytes, _stream_handle(dev))
    if seq_lens is not None:
        rc = lib.ssm_ssd_chunk_fwd_varlen(*head, _ptr(seq_lens), *tail)
        _native.check(rc, "ssm_ssd_chunk_fwd_varlen")
    else:
        rc = lib.ssm_ssd_chunk_fwd(*head, *tail)
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
    dt = _act_dtype("u", u)
    if u.dim() != 2:
        raise ValueError("u must be [B, D]")
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be [D, N]")
    dev = u.device
    Bt, Dm = u.shape
    N = A.shape[-1]
    _check_args(dev, ("state", state, (Bt, Dm, N), _F32), ("u", u, (Bt, Dm), dt),
                ("delta", delta, (Bt, Dm), dt), ("A", A, (Dm, N), _F32),
                ("B", B, (Bt, N), dt), ("C", C, (Bt, N), dt), ("z", z, (Bt, Dm), dt),
                ("D", D, (Dm,), _F32), ("delta_bias", delta_bias, (Dm,), _F32),
                ("out", out, (Bt, Dm), dt))
    lib = _native.load()
    y = out if out is not None else torch.empty((Bt, Dm), dtype=dt, device=dev)
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
                       workspace: Optional[torch.Tensor] = None,
                       ckpt: Optional[torch.Tensor] = None,
                       seq_lens: Optional[torch.Tensor] = None) -> dict:
    """Gradients of the S6 scan (ssm_selective_scan_bwd), states recomputed.

    Inputs as selective_scan_fwd plus dy [Bt, L, Dm] (dtype of u) and
    dh_last [Bt, Dm, N] fp32.  With ckpt (fp32 [Bt, Dm, ceil(L/16), N] from
    selective_scan_fwd_ckpt over the same inputs) the call is
    ssm_selective_scan_bwd_ckpt, which skips its own forward sweep.  With
    seq_lens (int32 [Bt]) it is ssm_selective_scan_bwd_varlen: row b has its
    first seq_lens[b] tokens, and the gradients past them are zeros.  Returns a
    dict with du, ddelta (dtype of u), dA [Dm, N], dB, dC [Bt, L, N] (fp32),
    and dD, dz, ddelta_bias, dh0 for the optional inputs that were given.
    """
    dt, dev, Bt, L, Dm, N = _s6_prepare(u, delta, A, B, C, D, z, delta_bias, h0, None)
    _check_args(dev, ("dy", dy, (Bt, L, Dm), dt), ("dh_last", dh_last, (Bt, Dm, N), _F32),
                ("ckpt", ckpt, (Bt, Dm, (L + 15) // 16, N), _F32),
                ("seq_lens", seq_lens, (Bt,), torch.int32))
    if ckpt is not None and seq_lens is not None:
        raise ValueError("the backward from checkpoints takes no seq_lens")
    lib = _native.load()
    if ckpt is not None:
        need = int(lib.ssm_selective_scan_bwd_ckpt_workspace_bytes(Bt, L, Dm, N, _DT[dt]))
    else:
        need = int(lib.ssm_selective_scan_bwd_workspace_bytes(Bt, L, Dm, N, _DT[dt]))
    workspace = _check_workspace(workspace, need, dev)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    out = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u),
           "dA": torch.empty((Dm, N), dtype=_F32, device=dev),
           "dB": torch.empty((Bt, L, N), dtype=_F32, device=dev),
           "dC": torch.empty((Bt, L, N), dtype=_F32, device=dev)}
    if D is not None:
        out["dD"] = torch.empty((Dm,), dtype=_F32, device=dev)
    if z is not None:
        out["dz"] = torch.empty_like(z)
    if delta_bias is not None:
        out["ddelta_bias"] = torch.empty((Dm,), dtype=_F32, device=dev)
    if h0 is not None:
        out["dh0"] = torch.empty((Bt, Dm, N), dtype=_F32, device=dev)
    flags = _native.FLAG_DELTA_SOFTPLUS if delta_softplus else 0
    grads = (_ptr(dy), _ptr(dh_last), _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]),
             _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out.get("dD")), _ptr(out.get("dz")),
             _ptr(out.get("ddelta_bias")), _ptr(out.get("dh0")))
    tail = (Bt, L, Dm, N, _DT[dt], _ptr(workspace), workspace.numel(), _stream_handle(dev))
    head = (_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            flags, _ptr(h0))
    if ckpt is not None:
        rc = lib.ssm_selective_scan_bwd_ckpt(*head, _ptr(ckpt), *grads, *tail)
        _native.check(rc, "ssm_selective_scan_bwd_ckpt")
    elif seq_lens is not None:
        rc = lib.ssm_selective_scan_bwd_varlen(*head, *grads, _ptr(seq_lens), *tail)
        _native.check(rc, "ssm_selective_scan_bwd_varlen")
    else:
        rc = lib.ssm_selective_scan_bwd(*head, *grads, *tail)
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
    dt = _act_dtype("x", x)
    if x.dim() != 3 or not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise ValueError("x must be [B, L, D] and weight [D, K]")
    dev = x.device
    Bt, L, Dm = x.shape
    K = weight.shape[1]
    _check_args(dev, ("x", x, (Bt, L, Dm), dt), ("weight", weight, (Dm, K), _F32),
                ("bias", bias, (Dm,), _F32), ("state", state, (Bt, Dm, K - 1), _F32),
                ("out", out, (Bt, L, Dm), dt))
    lib = _native.load()
    u = out if out is not None else torch.empty_like(x)
    new_state = torch.empty((Bt, Dm, K - 1), dtype=_F32, device=dev) if return_state else None
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
    dt, dev, Bt, L, Dm, N = _s6_prepare(x, delta, A, B, C, D, z, delta_bias, h0, out, name="x")
    if not isinstance(conv_weight, torch.Tensor) or conv_weight.dim() != 2:
        raise ValueError("conv_weight must be [D, K]")
    K = conv_weight.shape[1]
    _check_args(dev, ("conv_weight", conv_weight, (Dm, K), _F32),
                ("conv_bias", conv_bias, (Dm,), _F32),
                ("conv_state", conv_state, (Bt, Dm, K - 1), _F32))
    lib = _native.load()
    ws_need = int(lib.ssm_selective_scan_workspace_bytes(Bt, L, Dm, N, _DT[dt]))
    workspace, ws_bytes = _workspace(workspace, ws_need, dev)
    y = out if out is not None else torch.empty((Bt, L, Dm), dtype=dt, device=dev)
    h_last = torch.empty((Bt, Dm, N), dtype=_F32, device=dev)
    u = torch.empty_like(x) if return_u else None
    cs = torch.empty((Bt, Dm, K - 1), dtype=_F32, device=dev) if return_conv_state else None
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
