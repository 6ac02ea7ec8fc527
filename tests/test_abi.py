"""CPU tests of the C ABI: the library loads, exports every function that
include/lora4.h declares, and rejects bad arguments with the documented status
before any HIP call (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

import lora_fine_tuning_amd as L
from lora_fine_tuning_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, ENULL, ESHAPE, EALIGN, EFORMAT, EWS = 0, -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        B.build()
    return L.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "lora4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"sizeof"})


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "lora4_forward" in names and "quant_pack_mxfp4" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


def test_status_strings_and_version(lib):
    assert L.status_string(0) == "ok"
    for s in range(-7, 0):
        assert L.status_string(s) and L.status_string(s) != "unknown status"
    assert "gfx950" in L.version()


def _W(fmt=1, block=64, N=1024, K=1024, groups=1, codes=256, scales=512, scales2=None):
    return L.lora4_W(fmt, block, N, K, groups, codes, scales, scales2)


def test_format_and_block_validation(lib):
    assert L.lora4_workspace_bytes(0, _W(fmt=9), 16, 16) == 0
    ws = 1 << 30
    args = dict(X=4096, M=16, A=4096, B=4096, r=16, s=2.0, offs=None, Y=4096, Z=None, Yb=None, Yl=None,
                ws=8192, nbytes=ws, stream=None)

    def fwd(W, **kw):
        a = dict(args, **kw)
        return L.lora4_forward(W, a["X"], a["M"], a["A"], a["B"], a["r"], a["s"], a["offs"], a["Y"], a["Z"],
                               a["Yb"], a["Yl"], a["ws"], a["nbytes"], a["stream"])

    assert fwd(_W(fmt=9)) == EFORMAT
    assert fwd(_W(fmt=3, block=64)) == EFORMAT            # MXFP4 needs block 32
    assert fwd(_W(fmt=1, block=32)) == EFORMAT
    assert fwd(_W(K=96)) == ESHAPE                        # K % 64
    assert fwd(_W(fmt=3, block=32, K=48)) == ESHAPE
    assert fwd(_W(fmt=4, block=32)) == EFORMAT            # NVFP4 needs block 16
    assert fwd(_W(fmt=4, block=16, K=48)) == ESHAPE       # ... and K % 32 == 0
    assert fwd(_W(N=0)) == ESHAPE
    assert fwd(_W(fmt=2)) == ENULL                        # DQ needs scales2
    assert fwd(_W(codes=None)) == ENULL
    assert fwd(_W(codes=250)) == EALIGN
    assert fwd(_W(fmt=2, scales2=4098)) == EALIGN          # DQ scales2: 4-byte alignment
    assert fwd(_W(), r=0) == ESHAPE
    assert fwd(_W(), r=257) == ESHAPE
    assert fwd(_W(), s=float("nan")) == ESHAPE
    assert fwd(_W(), M=-1) == ESHAPE
    assert fwd(_W(), X=None) == ENULL
    assert fwd(_W(), Y=None) == ENULL
    assert fwd(_W(), X=4100) == EALIGN
    assert fwd(_W(), ws=None) == EWS
    assert fwd(_W(), nbytes=16) == EWS
    assert fwd(_W(groups=4)) == ENULL                     # grouped needs offsets
    assert fwd(_W(), offs=4096) == ESHAPE                 # single group takes no offsets
    assert fwd(_W(), M=0) == OK                           # nothing to launch


def test_backward_validation(lib):
    W = _W()

    def bwd(**kw):
        a = dict(X=4096, dY=4096, M=16, A=4096, B=4096, r=16, s=2.0, offs=None, Z=None, dX=4096, dA=4096,
                 dB=4096, ws=8192, nbytes=1 << 30, stream=None)
        a.update(kw)
        return L.lora4_backward(W, a["X"], a["dY"], a["M"], a["A"], a["B"], a["r"], a["s"], a["offs"], a["Z"],
                                a["dX"], a["dA"], a["dB"], a["ws"], a["nbytes"], a["stream"])

    assert bwd(dY=None) == ENULL
    assert bwd(dA=None) == ENULL
    assert bwd(dB=4104) == EALIGN
    assert bwd(nbytes=100) == EWS
    assert bwd(r=300) == ESHAPE


def test_quant_pack_validation(lib):
    assert L.quant_pack_nf4(None, 16, 64, 0, 4096, 4096, None, None) == ENULL
    assert L.quant_pack_nf4(4096, 16, 96, 0, 4096, 4096, None, None) == ESHAPE
    assert L.quant_pack_nf4(4096, 16, 64, 1, 4096, 4096, None, None) == ENULL
    assert L.quant_pack_nf4(4100, 16, 64, 0, 4096, 4096, None, None) == EALIGN
    assert L.quant_pack_nf4(4096, 16, 64, 1, 4096, 4096, 4098, None) == EALIGN   # scales2: 4-byte alignment
    assert L.quant_pack_mxfp4(4096, 16, 48, 4096, 4096, None) == ESHAPE
    assert L.quant_pack_mxfp4(4096, 0, 64, 4096, 4096, None) == ESHAPE


def test_workspace_sizes(lib):
    W = _W()
    f = L.lora4_workspace_bytes(0, W, 4096, 16)
    b = L.lora4_workspace_bytes(1, W, 4096, 16)
    assert f >= 4096 * 16 * 2 and b >= f
    assert L.lora4_workspace_bytes(0, W, 8192, 16) >= f
    assert L.lora4_workspace_bytes(2, W, 4096, 16) == 0
    assert L.lora4_workspace_bytes(0, W, 4096, 0) == 0
    # the workspace stays small next to the activations
    assert b < 4096 * 1024 * 2 * 8


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", "/nonexistent/liblora4.so")
    with pytest.raises(RuntimeError):
        L.lib()


def test_packed_bytes(lib):
    # 64 x 64 tiles: 2048 code bytes and 64 (NF4: fp32, DQ: u8) or 128 (MXFP4) scale entries per tile
    assert L.lora4_packed_bytes(L.LORA4_NF4, 1024, 1024, 0) == 16 * 16 * 2048
    assert L.lora4_packed_bytes(L.LORA4_NF4, 1024, 1024, 1) == 16 * 16 * 64 * 4
    assert L.lora4_packed_bytes(L.LORA4_NF4, 1024, 1024, 2) == 0
    assert L.lora4_packed_bytes(L.LORA4_NF4_DQ, 37, 192, 0) == 1 * 3 * 2048
    assert L.lora4_packed_bytes(L.LORA4_NF4_DQ, 37, 192, 1) == 1 * 3 * 64
    assert L.lora4_packed_bytes(L.LORA4_NF4_DQ, 37, 192, 2) == 4 * -(-(37 * 3) // 256)
    assert L.lora4_packed_bytes(L.LORA4_MXFP4, 65, 96, 0) == 2 * 2 * 2048
    assert L.lora4_packed_bytes(L.LORA4_MXFP4, 65, 96, 1) == 2 * 2 * 128
    assert L.lora4_packed_bytes(L.LORA4_NVFP4, 65, 96, 0) == 2 * 2 * 2048
    assert L.lora4_packed_bytes(L.LORA4_NVFP4, 65, 96, 1) == 2 * 2 * 256
    assert L.lora4_packed_bytes(L.LORA4_NVFP4, 65, 48, 0) == 0      # K % 32 != 0
    for bad in [(L.LORA4_NF4, 10, 96, 0), (L.LORA4_MXFP4, 0, 64, 0), (L.LORA4_MXFP4, 8, 48, 0), (9, 64, 64, 0),
                (L.LORA4_NF4, 64, 64, 3)]:
        assert L.lora4_packed_bytes(*bad) == 0, bad


def test_multi_adapter_validation(lib):
    """Several adapters over one shared base: W must be one group, adapters in
    range, offsets required for more than one adapter (nothing is launched)."""
    args = dict(X=4096, M=16, A=4096, B=4096, r=16, s=2.0, offs=None, Y=4096, Z=None, Yb=None, Yl=None,
                ws=8192, nbytes=1 << 30, stream=None)

    def fwd(W, adapters, **kw):
        a = dict(args, **kw)
        return L.lora4_forward_multi(W, adapters, a["X"], a["M"], a["A"], a["B"], a["r"], a["s"], a["offs"],
                                     a["Y"], a["Z"], a["Yb"], a["Yl"], a["ws"], a["nbytes"], a["stream"])

    def bwd(W, adapters, **kw):
        a = dict(X=4096, dY=4096, M=16, A=4096, B=4096, r=16, s=2.0, offs=None, Z=None, dX=4096, dA=4096,
                 dB=4096, ws=8192, nbytes=1 << 30, stream=None)
        a.update(kw)
        return L.lora4_backward_multi(W, adapters, a["X"], a["dY"], a["M"], a["A"], a["B"], a["r"], a["s"],
                                      a["offs"], a["Z"], a["dX"], a["dA"], a["dB"], a["ws"], a["nbytes"],
                                      a["stream"])

    assert fwd(_W(groups=2), 4, offs=4096) == ESHAPE       # the base is one shared group
    assert fwd(_W(), 0) == ESHAPE
    assert fwd(_W(), 70000, offs=4096) == ESHAPE
    assert fwd(_W(), 4) == ENULL                           # several adapters need offsets
    assert fwd(_W(), 1, offs=4096) == ESHAPE               # one adapter takes none
    assert fwd(_W(), 4, offs=4096, M=0) == OK              # nothing to launch
    assert bwd(_W(groups=3), 2, offs=4096) == ESHAPE
    assert bwd(_W(), 3) == ENULL
    assert bwd(_W(), 3, offs=4096, dA=None) == ENULL
    W = _W()
    assert L.lora4_workspace_bytes_multi(0, W, 4, 1024, 16) > 0
    assert L.lora4_workspace_bytes_multi(1, W, 4, 1024, 16) > 0
    assert L.lora4_workspace_bytes_multi(0, W, 0, 1024, 16) == 0
    assert L.lora4_workspace_bytes_multi(0, _W(groups=2), 4, 1024, 16) == 0


def test_mx_forward_validation(lib):
    """MX-native forward: MXFP4 base only, one group, the workspace it asks
    for; the MXFP8 packer wants K % 32 == 0 (nothing is launched)."""
    W = _W(fmt=L.LORA4_MXFP4, block=32, N=1024, K=1024)
    need = L.lora4_workspace_bytes_mx(W, 4096, 16)
    # the MXFP8 codes [M, K] and their scales are part of the workspace
    assert need >= 4096 * 1024 + 4096 * 1024 // 32
    assert L.lora4_workspace_bytes_mx(_W(), 4096, 16) == 0                    # NF4 base
    assert L.lora4_workspace_bytes_mx(_W(fmt=L.LORA4_MXFP4, block=32, groups=2), 16, 16) == 0

    def fwd(Wd, **kw):
        a = dict(X=4096, M=16, A=4096, B=4096, r=16, s=2.0, Y=4096, Z=None, ws=8192, nbytes=need, stream=None)
        a.update(kw)
        return L.lora4_forward_mx(Wd, a["X"], a["M"], a["A"], a["B"], a["r"], a["s"], a["Y"], a["Z"], a["ws"],
                                  a["nbytes"], a["stream"])

    assert fwd(_W()) == EFORMAT
    assert fwd(_W(fmt=L.LORA4_MXFP4, block=32, groups=2)) == ESHAPE
    assert fwd(W, r=0) == ESHAPE
    assert fwd(W, s=float("nan")) == ESHAPE
    assert fwd(W, A=None) == ENULL
    assert fwd(W, Y=None) == ENULL
    assert fwd(W, X=4100) == EALIGN
    assert fwd(W, ws=None) == EWS
    assert fwd(W, nbytes=need - 1, M=4096) == EWS
    assert fwd(W, M=0, X=None, Y=None) == OK
    assert L.quant_pack_mxfp8(4096, 16, 48, 4096, 4096, None) == ESHAPE
    assert L.quant_pack_mxfp8(4096, 16, 16, 4096, 4096, None) == ESHAPE
    assert L.quant_pack_mxfp8(4096, -1, 64, 4096, 4096, None) == ESHAPE
    assert L.quant_pack_mxfp8(None, 16, 64, 4096, 4096, None) == ENULL
    assert L.quant_pack_mxfp8(4096, 16, 64, 4104, 4096, None) == EALIGN
    assert L.quant_pack_mxfp8(None, 0, 64, None, None, None) == OK


def test_nvfp4_packer_validation(lib):
    assert L.quant_pack_nvfp4(4096, 64, 48, 4096, 4096, None) == ESHAPE    # K % 32
    assert L.quant_pack_nvfp4(4096, 0, 64, 4096, 4096, None) == ESHAPE
    assert L.quant_pack_nvfp4(None, 64, 64, 4096, 4096, None) == ENULL
    assert L.quant_pack_nvfp4(4096, 64, 64, 4100, 4096, None) == EALIGN


def test_loftq_validation(lib):
    assert L.lora4_loftq_workspace_bytes(256, 512, 16) >= 256 * 512 * 6
    assert L.lora4_loftq_workspace_bytes(256, 500, 16) == 0              # K % 64
    assert L.lora4_loftq_workspace_bytes(256, 512, 129) == 0             # r <= 128
    assert L.lora4_loftq_workspace_bytes(20, 512, 16) == 0               # r + 8 <= N
    need = L.lora4_loftq_workspace_bytes(256, 512, 16)

    def init(**kw):
        a = dict(W=4096, N=256, K=512, r=16, iters=5, s=2.0, dq=0, codes=4096, scales=4096, scales2=None,
                 A=4096, B=4096, ws=8192, nbytes=need, stream=None)
        a.update(kw)
        return L.lora4_loftq_init(a["W"], a["N"], a["K"], a["r"], a["iters"], a["s"], a["dq"], a["codes"],
                                  a["scales"], a["scales2"], a["A"], a["B"], a["ws"], a["nbytes"], a["stream"])

    assert init(W=None) == ENULL
    assert init(dq=1) == ENULL                                            # DQ needs scales2
    assert init(K=500) == ESHAPE
    assert init(r=0) == ESHAPE
    assert init(iters=0) == ESHAPE
    assert init(s=0.0) == ESHAPE
    assert init(A=4100) == EALIGN
    assert init(ws=None) == EWS
    assert init(nbytes=need - 1) == EWS


def test_import_rowmajor_validation(lib):
    imp = L.lora4_import_rowmajor
    assert imp(9, 64, 64, 1, 256, 256, 256, 256, None) == EFORMAT
    assert imp(1, 64, 96, 1, 256, 256, 256, 256, None) == ESHAPE        # NF4: K % 64
    assert imp(3, 64, 48, 1, 256, 256, 256, 256, None) == ESHAPE        # MXFP4: K % 32
    assert imp(3, 0, 64, 1, 256, 256, 256, 256, None) == ESHAPE
    assert imp(3, 64, 64, 0, 256, 256, 256, 256, None) == ESHAPE
    assert imp(1, 64, 64, 1, None, 256, 256, 256, None) == ENULL
    assert imp(1, 64, 64, 1, 256, 256, 256, None, None) == ENULL
    assert imp(1, 64, 64, 1, 256, 258, 256, 256, None) == EALIGN
    assert imp(4, 64, 64, 1, 256, 256, 264, 256, None) == EALIGN
