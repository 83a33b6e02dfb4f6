"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/ssm.h declares, and rejects bad arguments before any
HIP call (only invalid calls are made here; nothing is launched)."""
import ctypes
import math
import os
import re

import pytest

from selective_state_space_21_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")

# never dereferenced: validation fails before any use
FAKE = 0x10000
FAKE_MIS = 0x10002


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _native.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n
        assert n in _native.SIGNATURES, n


def test_version_and_status_strings(lib):
    assert lib.ssm_abi_version() == 1
    for s in range(0, 8):
        assert lib.ssm_status_string(s)
    assert b"unknown" in lib.ssm_status_string(99)


def s6(lib, **kw):
    a = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None,
             flags=1, h0=None, y=FAKE, h_last=None, Bt=2, L=64, Dm=128, N=16, dtype=1,
             ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.ssm_selective_scan_fwd(
        a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["flags"],
        a["h0"], a["y"], a["h_last"], a["Bt"], a["L"], a["Dm"], a["N"], a["dtype"],
        a["ws"], a["ws_bytes"], a["stream"])


def test_s6_validation_errors(lib):
    assert s6(lib, u=None) == 1
    assert s6(lib, A=None) == 1
    assert s6(lib, y=None) == 1
    assert s6(lib, Bt=0) == 2
    assert s6(lib, Dm=-1) == 2
    assert s6(lib, N=0) == 2
    assert s6(lib, L=-5) == 2
    assert s6(lib, Bt=1 << 40, L=1 << 20, Dm=1 << 20) == 2        # overflow
    assert s6(lib, dtype=7) == 3
    assert s6(lib, N=65) == 4
    assert s6(lib, flags=8) == 4
    assert s6(lib, u=FAKE_MIS) == 5
    assert s6(lib, h0=FAKE + 1) == 5
    need = lib.ssm_selective_scan_workspace_bytes(2, 4096, 128, 16, 1)
    assert need > 0
    assert s6(lib, L=4096, ws=None) == 6
    assert s6(lib, L=4096, ws_bytes=need - 1) == 6


def test_s6_workspace_and_plan(lib):
    # one segment when there are plenty of channels
    assert lib.ssm_selective_scan_segments(64, 2048, 4096, 16) == 1
    assert lib.ssm_selective_scan_workspace_bytes(64, 2048, 4096, 16, 1) == 0
    # few channels, long sequence: split into up to 256 segments; the
    # workspace holds the pairs of whichever path is larger (the query has
    # no flags, and ZOH calls take the split path)
    S = lib.ssm_selective_scan_segments(1, 131072, 2048, 16)
    assert 2 <= S <= 256
    import os
    old = os.environ.get("SSM_S6_LANES")
    os.environ["SSM_S6_LANES"] = "0"
    try:
        S_split = lib.ssm_selective_scan_segments(1, 131072, 2048, 16)
    finally:
        if old is None:
            del os.environ["SSM_S6_LANES"]
        else:
            os.environ["SSM_S6_LANES"] = old
    assert 2 <= S_split <= 256
    # lanes: pairs plus one dt checkpoint per (segment, 1024-token chunk, channel)
    seg = math.ceil(math.ceil(131072 / S) / 128) * 128
    lanes_bytes = 2 * 4 * 2048 * 16 * S + 4 * S * math.ceil(seg / 1024) * 2048
    assert (lib.ssm_selective_scan_workspace_bytes(1, 131072, 2048, 16, 0)
            == max(2 * 4 * 2048 * 16 * S_split, lanes_bytes))
    # the same forced segment count on both paths: the checkpoints make the
    # lanes workspace the larger (3 chunks per segment of 2176 tokens here)
    old_seg = os.environ.get("SSM_S6_SEGMENTS")
    os.environ["SSM_S6_SEGMENTS"] = "4"
    try:
        assert lib.ssm_selective_scan_segments(2, 8700, 64, 16) == 4
        assert (lib.ssm_selective_scan_workspace_bytes(2, 8700, 64, 16, 0)
                == 2 * 4 * 2 * 64 * 16 * 4 + 4 * 4 * 3 * 2 * 64)
    finally:
        if old_seg is None:
            del os.environ["SSM_S6_SEGMENTS"]
        else:
            os.environ["SSM_S6_SEGMENTS"] = old_seg
    # never more segments than ceil(L / 32)
    assert lib.ssm_selective_scan_segments(1, 40, 64, 16) <= 2
    assert lib.ssm_selective_scan_segments(1, 0, 64, 16) == 1
    assert lib.ssm_selective_scan_workspace_bytes(0, 10, 10, 16, 1) == 0   # invalid -> 0


def test_s6_plan_env_override(lib, monkeypatch):
    # split path: any count up to 256, segments of at least 32 tokens
    monkeypatch.setenv("SSM_S6_LANES", "0")
    monkeypatch.setenv("SSM_S6_SEGMENTS", "7")
    assert lib.ssm_selective_scan_segments(1, 7000, 64, 16) == 7
    monkeypatch.setenv("SSM_S6_SEGMENTS", "500")
    assert lib.ssm_selective_scan_segments(1, 70000, 64, 16) == 256
    # state-per-lane path: segments are whole 128-token super-tiles
    monkeypatch.delenv("SSM_S6_LANES")
    monkeypatch.setenv("SSM_S6_SEGMENTS", "7")
    assert lib.ssm_selective_scan_segments(1, 7000, 64, 16) == 7
    monkeypatch.setenv("SSM_S6_SEGMENTS", "500")
    seg = -(-(-(-70000 // 256)) // 128) * 128
    assert lib.ssm_selective_scan_segments(1, 70000, 64, 16) == -(-70000 // seg)
    # the fix-up's one-dimensional grid stays under 2^24 workgroups: 128 groups
    # x 512 rows x 244 later segments x 2 chunks is 32M, so the split path
    # takes that call; 64 rows (4M workgroups) stay on the state-per-lane path
    monkeypatch.setenv("SSM_S6_SEGMENTS", "256")
    assert lib.ssm_selective_scan_lanes(512, 500000, 2048, 16) == 0
    assert lib.ssm_selective_scan_lanes(64, 500000, 2048, 16) == 1
    assert lib.ssm_selective_scan_segments(64, 500000, 2048, 16) == 245


def test_s6_lanes_plan(lib, monkeypatch):
    # The planner balances over 1024 SIMDs (256 CUs), device or not: the state-per-lane
    # kernel needs N = 16 and D % 16 == 0; below 2048 wavefronts (B*D/4) it cuts the
    # sequence into segments of whole super-tiles for six wavefronts per SIMD
    monkeypatch.delenv("SSM_S6_LANES", raising=False)
    monkeypatch.delenv("SSM_S6_SEGMENTS", raising=False)
    assert lib.ssm_selective_scan_lanes(8, 2048, 1536, 16) == 1
    assert lib.ssm_selective_scan_segments(8, 2048, 1536, 16) == 1
    assert lib.ssm_selective_scan_lanes(4, 4096, 5120, 16) == 1
    assert lib.ssm_selective_scan_lanes(1, 131072, 2048, 16) == 1      # few channels: segments
    assert lib.ssm_selective_scan_segments(1, 131072, 2048, 16) == 12
    assert lib.ssm_selective_scan_lanes(8, 2048, 1544, 16) == 0        # D % 16 != 0
    assert lib.ssm_selective_scan_lanes(8, 2048, 1536, 32) == 0        # N != 16
    assert lib.ssm_selective_scan_lanes(0, 2048, 1536, 16) == 0        # invalid sizes
    # offsets of one batch row (plus a super-tile) must fit 32 bits at 4 B per element
    assert lib.ssm_selective_scan_lanes(2, 2**20, 1024, 16) == 0
    # the split plan (segments, workspace) is unchanged: ZOH calls still use it
    monkeypatch.setenv("SSM_S6_LANES", "0")
    assert lib.ssm_selective_scan_lanes(8, 2048, 1536, 16) == 0
    assert lib.ssm_selective_scan_segments(8, 2048, 1536, 16) > 1
    monkeypatch.delenv("SSM_S6_LANES")
    assert lib.ssm_selective_scan_lanes(1, 40, 64, 16) == 1
    assert lib.ssm_selective_scan_lanes(1, 40, 72, 16) == 0
    assert lib.ssm_selective_scan_lanes(1, 40, 64, 8) == 0


def ssd(lib, **kw):
    a = dict(X=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, flags=1,
             h0=None, Y=FAKE, h_last=None, Bt=1, L=256, H=8, P=64, G=1, N=128, chunk=256,
             dtype=1, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.ssm_ssd_chunk_fwd(
        a["X"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["flags"],
        a["h0"], a["Y"], a["h_last"], a["Bt"], a["L"], a["H"], a["P"], a["G"], a["N"],
        a["chunk"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


def test_ssd_validation_errors(lib):
    assert ssd(lib, X=None) == 1
    assert ssd(lib, A=None) == 1
    assert ssd(lib, H=6, G=4) == 2
    assert ssd(lib, P=0) == 2
    assert ssd(lib, dtype=5) == 3
    assert ssd(lib, chunk=100) == 4
    assert ssd(lib, P=48) == 4
    assert ssd(lib, P=16) == 4
    assert ssd(lib, N=48) == 4
    assert ssd(lib, N=160) == 4
    assert ssd(lib, N=16) == 4
    assert ssd(lib, dtype=0) == 4
    assert ssd(lib, flags=2) == 4
    assert ssd(lib, Y=FAKE_MIS) == 5
    assert lib.ssm_ssd_chunk_workspace_bytes(4, 8192, 64, 64, 1, 128, 256, 1) == 0


def test_ssd_grid_limit(lib):
    # one workgroup per (b, h, slice of 64 head-dim rows; 32 when P % 64 != 0):
    # the count must stay below 2^31
    # (row offsets stay small here, so only the grid count can refuse these)
    assert ssd(lib, Bt=2**20, L=0, H=2**10, P=128) == 4
    assert ssd(lib, Bt=2**20, L=0, H=700, P=96) == 4


def test_ssd_offset_limit(lib):
    # a batch row of X with two chunks of 256 tokens to spare must fit 32-bit
    # byte offsets: H=64, P=64 is 8192 bytes per token, so L + 512 <= 524287
    assert ssd(lib, L=524288 - 512, H=64) == 4
    assert ssd(lib, L=2**20, H=64) == 4


def step(lib, **kw):
    a = dict(state=FAKE, u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None,
             flags=1, y=FAKE, Bt=4, Dm=256, N=16, dtype=1, stream=None)
    a.update(kw)
    return lib.ssm_selective_state_update(
        a["state"], a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"],
        a["flags"], a["y"], a["Bt"], a["Dm"], a["N"], a["dtype"], a["stream"])


def test_step_validation_errors(lib):
    assert step(lib, state=None) == 1
    assert step(lib, A=None) == 1
    assert step(lib, y=None) == 1
    assert step(lib, Bt=0) == 2
    assert step(lib, N=-1) == 2
    assert step(lib, Dm=1 << 40, N=1 << 30) == 2
    assert step(lib, dtype=7) == 3
    assert step(lib, N=65) == 4
    assert step(lib, flags=8) == 4
    assert step(lib, state=FAKE_MIS) == 5
    assert step(lib, A=FAKE + 4) == 5
    assert step(lib, D=FAKE + 2) == 5


def bwd(lib, **kw):
    a = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, flags=1,
             h0=None, dy=FAKE, dh=None, du=FAKE, dd=FAKE, dA=FAKE, dB=FAKE, dC=FAKE, dD=None,
             dz=None, dbias=None, dh0=None, Bt=2, L=64, Dm=128, N=16, dtype=1, ws=0x100000,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.ssm_selective_scan_bwd(
        a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["flags"],
        a["h0"], a["dy"], a["dh"], a["du"], a["dd"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"],
        a["dbias"], a["dh0"], a["Bt"], a["L"], a["Dm"], a["N"], a["dtype"], a["ws"],
        a["ws_bytes"], a["stream"])


def test_bwd_validation_errors(lib):
    assert bwd(lib, dy=None) == 1
    assert bwd(lib, dA=None) == 1
    assert bwd(lib, z=FAKE, dz=None) == 1
    assert bwd(lib, Bt=0) == 2
    assert bwd(lib, dtype=9) == 3
    assert bwd(lib, N=17) == 4
    assert bwd(lib, flags=3) == 4
    assert bwd(lib, du=FAKE_MIS) == 5
    assert bwd(lib, ws=0x100010) == 5
    assert bwd(lib, ws_bytes=16) == 6
    assert bwd(lib, ws=None) == 6
    need = lib.ssm_selective_scan_bwd_workspace_bytes(8, 2048, 1536, 16, 1)
    assert need > 8 * 1536 * 128 * 16 * 4          # the state checkpoints alone
    assert lib.ssm_selective_scan_bwd_workspace_bytes(8, 2048, 1536, 17, 1) == 0


def fwd_ckpt(lib, **kw):
    a = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None,
             flags=1, h0=None, y=FAKE, h_last=None, ck=FAKE, Bt=2, L=64, Dm=128, N=16, dtype=1,
             ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.ssm_selective_scan_fwd_ckpt(
        a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["flags"],
        a["h0"], a["y"], a["h_last"], a["ck"], a["Bt"], a["L"], a["Dm"], a["N"], a["dtype"],
        a["ws"], a["ws_bytes"], a["stream"])


def bwd_ckpt(lib, **kw):
    a = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, flags=1,
             h0=None, ck=FAKE, dy=FAKE, dh=None, du=FAKE, dd=FAKE, dA=FAKE, dB=FAKE, dC=FAKE,
             dD=None, dz=None, dbias=None, dh0=None, Bt=2, L=64, Dm=128, N=16, dtype=1,
             ws=0x100000, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.ssm_selective_scan_bwd_ckpt(
        a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["flags"],
        a["h0"], a["ck"], a["dy"], a["dh"], a["du"], a["dd"], a["dA"], a["dB"], a["dC"], a["dD"],
        a["dz"], a["dbias"], a["dh0"], a["Bt"], a["L"], a["Dm"], a["N"], a["dtype"], a["ws"],
        a["ws_bytes"], a["stream"])


def test_ckpt_validation_errors(lib):
    # the forward for training takes the backward's sizes and flags
    assert fwd_ckpt(lib, ck=None) == 1
    assert fwd_ckpt(lib, y=None) == 1
    assert fwd_ckpt(lib, Bt=0) == 2
    assert fwd_ckpt(lib, dtype=7) == 3
    assert fwd_ckpt(lib, N=17) == 4
    assert fwd_ckpt(lib, flags=3) == 4          # ZOH
    assert fwd_ckpt(lib, ck=FAKE + 4) == 5
    assert fwd_ckpt(lib, y=FAKE_MIS) == 5
    assert fwd_ckpt(lib, ws=None) == 6
    assert bwd_ckpt(lib, ck=None) == 1
    assert bwd_ckpt(lib, dy=None) == 1
    assert bwd_ckpt(lib, N=17) == 4
    assert bwd_ckpt(lib, flags=2) == 4
    assert bwd_ckpt(lib, ck=FAKE + 8) == 5
    assert bwd_ckpt(lib, du=FAKE_MIS) == 5
    assert bwd_ckpt(lib, ws_bytes=16) == 6


def test_ckpt_sizes(lib):
    for (Bt, L, Dm, N) in [(8, 2048, 1536, 16), (3, 513, 40, 5), (1, 1, 16, 1), (2, 0, 16, 16)]:
        nck = (L + 15) // 16
        assert lib.ssm_selective_scan_ckpt_bytes(Bt, L, Dm, N, 1) == Bt * Dm * nck * N * 4
        full = lib.ssm_selective_scan_bwd_workspace_bytes(Bt, L, Dm, N, 1)
        part = lib.ssm_selective_scan_bwd_ckpt_workspace_bytes(Bt, L, Dm, N, 1)
        # the checkpoints are the last region of the self-contained call's workspace
        assert full - part == (Bt * Dm * nck * N * 4 + 255) // 256 * 256
    assert lib.ssm_selective_scan_ckpt_bytes(8, 2048, 1536, 17, 1) == 0
    assert lib.ssm_selective_scan_bwd_ckpt_workspace_bytes(8, 2048, 1536, 17, 1) == 0


def conv(lib, **kw):
    a = dict(x=FAKE, w=FAKE, b=None, si=None, silu=1, u=FAKE, so=None, Bt=2, L=64, Dm=128, K=4,
             dtype=1, stream=None)
    a.update(kw)
    return lib.ssm_causal_conv1d_silu(a["x"], a["w"], a["b"], a["si"], a["silu"], a["u"], a["so"],
                                      a["Bt"], a["L"], a["Dm"], a["K"], a["dtype"], a["stream"])


def test_conv_validation_errors(lib):
    assert conv(lib, w=None) == 1
    assert conv(lib, x=None) == 1
    assert conv(lib, K=0) == 2
    assert conv(lib, L=-1) == 2
    assert conv(lib, dtype=3) == 3
    assert conv(lib, K=5) == 4
    assert conv(lib, u=FAKE_MIS) == 5
    assert conv(lib, b=FAKE + 2) == 5


def conv_scan(lib, **kw):
    a = dict(x=FAKE, w=FAKE, cb=None, si=None, so=None, K=4, uo=None, delta=FAKE, A=FAKE, B=FAKE,
             C=FAKE, D=None, z=None, bias=None, flags=1, h0=None, y=FAKE, hl=None, Bt=2, L=64,
             Dm=128, N=16, dtype=1, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.ssm_selective_scan_conv_fwd(
        a["x"], a["w"], a["cb"], a["si"], a["so"], a["K"], a["uo"], a["delta"], a["A"], a["B"],
        a["C"], a["D"], a["z"], a["bias"], a["flags"], a["h0"], a["y"], a["hl"], a["Bt"], a["L"],
        a["Dm"], a["N"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


def test_conv_scan_validation_errors(lib):
    assert conv_scan(lib, w=None) == 1
    assert conv_scan(lib, x=None) == 1
    assert conv_scan(lib, K=0) == 2
    assert conv_scan(lib, K=5) == 4
    assert conv_scan(lib, N=8) == 4
    assert conv_scan(lib, flags=3) == 4
    assert conv_scan(lib, uo=FAKE_MIS) == 5
    assert conv_scan(lib, si=FAKE + 2) == 5


def test_varlen_validation_errors(lib):
    def call(sl, **kw):
        a = dict(Bt=2, L=64, Dm=128, N=16, dtype=1)
        a.update(kw)
        return lib.ssm_selective_scan_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 1,
                                                 None, FAKE, None, sl, a["Bt"], a["L"], a["Dm"],
                                                 a["N"], a["dtype"], FAKE, 1 << 30, None)
    assert call(None) == 1
    assert call(FAKE + 2) == 5
    assert call(FAKE, Bt=0) == 2

    def ssd_call(sl, **kw):
        a = dict(Bt=1, L=256, H=8, P=64, G=1, N=128, chunk=256, dtype=1, Y=FAKE)
        a.update(kw)
        return lib.ssm_ssd_chunk_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 1,
                                            None, a["Y"], None, sl, a["Bt"], a["L"], a["H"],
                                            a["P"], a["G"], a["N"], a["chunk"], a["dtype"], None,
                                            0, None)
    def bwd_call(sl, **kw):
        a = dict(Bt=2, L=64, Dm=128, N=16, dtype=1, du=FAKE)
        a.update(kw)
        return lib.ssm_selective_scan_bwd_varlen(
            FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 1, None, FAKE, None, a["du"], FAKE,
            FAKE, FAKE, FAKE, None, None, None, None, sl, a["Bt"], a["L"], a["Dm"], a["N"],
            a["dtype"], 0x100000, 1 << 40, None)
    assert bwd_call(None) == 1
    assert bwd_call(FAKE + 2) == 5
    assert bwd_call(FAKE, N=17) == 4
    assert bwd_call(FAKE, du=FAKE_MIS) == 5
    assert ssd_call(None) == 1
    assert ssd_call(FAKE + 2) == 5
    assert ssd_call(FAKE, Bt=0) == 2
    assert ssd_call(FAKE, dtype=0) == 4          # fp32 storage: not implemented
    assert ssd_call(FAKE, N=48) == 4
    assert ssd_call(FAKE, Y=FAKE_MIS) == 5


def test_python_wrapper_rejects_host_tensors():
    import torch
    import selective_state_space_21_amd as ssm
    u = torch.zeros(1, 4, 64)
    with pytest.raises(ValueError):
        ssm.selective_scan_fwd(u, u, torch.zeros(64, 16), torch.zeros(1, 4, 16), torch.zeros(1, 4, 16))


def test_python_wrappers_check_out_shapes_before_devices():
    """A caller-supplied output buffer of the wrong shape (or dtype) is
    rejected, by every wrapper, before any device check, so these host tensors
    never get near the library."""
    import torch
    import selective_state_space_21_amd as ssm
    bf = torch.bfloat16
    u = torch.zeros(2, 8, 64, dtype=bf)
    A = torch.zeros(64, 16)
    Bm = torch.zeros(2, 8, 16, dtype=bf)
    with pytest.raises(ValueError, match="out has shape"):
        ssm.selective_scan_fwd(u, u, A, Bm, Bm, out=torch.zeros(2, 7, 64, dtype=bf))
    with pytest.raises(TypeError, match="out must be"):
        ssm.selective_scan_fwd(u, u, A, Bm, Bm, out=torch.zeros(2, 8, 64))
    with pytest.raises(ValueError, match="out has shape"):
        ssm.selective_scan_conv_fwd(u, torch.zeros(64, 4), None, u, A, Bm, Bm,
                                    out=torch.zeros(1, 8, 64, dtype=bf))
    X = torch.zeros(1, 8, 2, 64, dtype=bf)
    Bg = torch.zeros(1, 8, 1, 128, dtype=bf)
    with pytest.raises(ValueError, match="out has shape"):
        ssm.ssd_chunk_fwd(X, torch.zeros(1, 8, 2, dtype=bf), torch.zeros(2), Bg, Bg,
                          out=torch.zeros(1, 8, 2, 32, dtype=bf))
    st = torch.zeros(2, 64, 16)
    v = torch.zeros(2, 64, dtype=bf)
    with pytest.raises(ValueError, match="out has shape"):
        ssm.selective_state_update(st, v, v, A, torch.zeros(2, 16, dtype=bf),
                                   torch.zeros(2, 16, dtype=bf), out=torch.zeros(2, 63, dtype=bf))
    with pytest.raises(ValueError, match="out has shape"):
        ssm.causal_conv1d_silu(u, torch.zeros(64, 4), out=torch.zeros(2, 8, 32, dtype=bf))
    # an input of the wrong shape is caught the same way
    with pytest.raises(ValueError, match="C has shape"):
        ssm.selective_scan_fwd(u, u, A, Bm, torch.zeros(2, 8, 8, dtype=bf))


def test_python_workspace_checks():
    """A workspace must be a contiguous uint8 tensor on the call's device, at
    least as large as the query."""
    import torch
    from selective_state_space_21_amd import _check_workspace
    dev = torch.device("cuda:0")
    assert _check_workspace(None, 100, dev) is None
    with pytest.raises(ValueError, match="expected cuda:0"):
        _check_workspace(torch.empty(128, dtype=torch.uint8), 100, dev)
    with pytest.raises(TypeError, match="uint8"):
        _check_workspace(torch.empty(128, dtype=torch.float32), 100, dev)
    with pytest.raises(ValueError, match="needs 100"):
        _check_workspace(torch.empty(64, dtype=torch.uint8), 100, dev)
    with pytest.raises(TypeError):
        _check_workspace(12345, 100, dev)
