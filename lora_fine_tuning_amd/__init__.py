"""Python binding of liblora4 (include/lora4.h): the unmerged-LoRA linear over
a frozen 4-bit base (NF4, NF4 with double-quantized scales, MXFP4) on MI355X.

This module only marshals arguments: it takes device pointers and the current
stream from torch tensors and calls the C ABI through ctypes. Every step of the
computation runs in the library's HIP kernels. If the library is not built,
every call raises; there is no fallback.

Low-level functions carry the ABI's names and signatures (pointers as ints):
``lora4_forward``, ``lora4_backward``, ``lora4_workspace_bytes``,
``lora4_packed_bytes``, ``quant_pack_nf4``, ``quant_pack_mxfp4``. The torch-level helpers ``pack_nf4``,
``pack_mxfp4``, ``forward`` and ``backward`` allocate outputs with torch and call
them.
"""

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblora4.so")

LORA4_NF4, LORA4_NF4_DQ, LORA4_MXFP4, LORA4_NVFP4 = 1, 2, 3, 4
FORMATS = {"nf4": LORA4_NF4, "nf4_dq": LORA4_NF4_DQ, "mxfp4": LORA4_MXFP4, "nvfp4": LORA4_NVFP4}
BLOCK = {LORA4_NF4: 64, LORA4_NF4_DQ: 64, LORA4_MXFP4: 32, LORA4_NVFP4: 16}

EXPORTS = ["lora4_forward", "lora4_forward_noalloc", "lora4_backward", "lora4_workspace_bytes", "lora4_packed_bytes",
           "lora4_forward_multi", "lora4_backward_multi", "lora4_workspace_bytes_multi", "quant_pack_nf4",
           "quant_pack_mxfp4", "quant_pack_nvfp4", "quant_pack_mxfp8", "lora4_workspace_bytes_mx", "lora4_forward_mx",
           "lora4_loftq_workspace_bytes", "lora4_loftq_init", "lora4_import_rowmajor",
           "lora4_status_string", "lora4_timing_enable", "lora4_timing_collect", "lora4_version"]


class Lora4Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


class lora4_W(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("block", ctypes.c_int32), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("groups", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("scales2", ctypes.c_void_p)]


class lora4_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


_lib = None


def lib():
    """The loaded liblora4 (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m lora_fine_tuning_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        Wp = ctypes.POINTER(lora4_W)
        L.lora4_forward.argtypes = [Wp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lora4_forward.restype = ctypes.c_int
        L.lora4_forward_noalloc.argtypes = [Wp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, vp, vp]
        L.lora4_forward_noalloc.restype = ctypes.c_int
        L.lora4_backward.argtypes = [Wp, vp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lora4_backward.restype = ctypes.c_int
        L.lora4_workspace_bytes.argtypes = [ctypes.c_int, Wp, i64, i32]
        L.lora4_workspace_bytes.restype = sz
        L.lora4_packed_bytes.argtypes = [i32, i64, i64, i32]
        L.lora4_packed_bytes.restype = sz
        L.lora4_forward_multi.argtypes = [Wp, i64, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lora4_forward_multi.restype = ctypes.c_int
        L.lora4_backward_multi.argtypes = [Wp, i64, vp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lora4_backward_multi.restype = ctypes.c_int
        L.lora4_workspace_bytes_multi.argtypes = [ctypes.c_int, Wp, i64, i64, i32]
        L.lora4_workspace_bytes_multi.restype = sz
        L.quant_pack_nf4.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp]
        L.quant_pack_nf4.restype = ctypes.c_int
        L.quant_pack_mxfp4.argtypes = [vp, i64, i64, vp, vp, vp]
        L.quant_pack_mxfp4.restype = ctypes.c_int
        L.quant_pack_nvfp4.argtypes = [vp, i64, i64, vp, vp, vp]
        L.quant_pack_nvfp4.restype = ctypes.c_int
        L.quant_pack_mxfp8.argtypes = [vp, i64, i64, vp, vp, vp]
        L.quant_pack_mxfp8.restype = ctypes.c_int
        L.lora4_workspace_bytes_mx.argtypes = [Wp, i64, i32]
        L.lora4_workspace_bytes_mx.restype = sz
        L.lora4_forward_mx.argtypes = [Wp, vp, i64, vp, vp, i32, f32, vp, vp, vp, sz, vp]
        L.lora4_forward_mx.restype = ctypes.c_int
        L.lora4_loftq_workspace_bytes.argtypes = [i64, i64, i32]
        L.lora4_loftq_workspace_bytes.restype = sz
        L.lora4_loftq_init.argtypes = [vp, i64, i64, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lora4_loftq_init.restype = ctypes.c_int
        L.lora4_import_rowmajor.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp]
        L.lora4_import_rowmajor.restype = ctypes.c_int
        L.lora4_status_string.argtypes = [ctypes.c_int]
        L.lora4_status_string.restype = ctypes.c_char_p
        L.lora4_timing_enable.argtypes = [ctypes.c_int]
        L.lora4_timing_enable.restype = ctypes.c_int
        L.lora4_timing_collect.argtypes = [ctypes.POINTER(lora4_kernel_time), ctypes.c_int]
        L.lora4_timing_collect.restype = ctypes.c_int
        L.lora4_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status):
    return lib().lora4_status_string(int(status)).decode()


def _check(status, what):
    if status != 0:
        raise Lora4Error(status, what)


# ---------------------------------------------------------------------------
# ABI-named calls (pointers as ints; stream as an int handle or None)
# ---------------------------------------------------------------------------

def lora4_workspace_bytes(which, W, M, r):
    return lib().lora4_workspace_bytes(which, ctypes.byref(W), M, r)


def lora4_packed_bytes(fmt, N, K, part):
    return lib().lora4_packed_bytes(fmt, N, K, part)


def lora4_forward(W, X, M, A, B, r, s, group_offsets, Y, Z, Y_base, Y_lora, workspace, workspace_bytes,
                  stream):
    return lib().lora4_forward(ctypes.byref(W), X, M, A, B, r, s, group_offsets, Y, Z, Y_base, Y_lora,
                               workspace, workspace_bytes, stream)


def lora4_forward_noalloc(W, X, M, A, B, r, s, group_offsets, Y, Z, Y_base, Y_lora, stream):
    return lib().lora4_forward_noalloc(ctypes.byref(W), X, M, A, B, r, s, group_offsets, Y, Z, Y_base, Y_lora,
                                       stream)


def lora4_backward(W, X, dY, M, A, B, r, s, group_offsets, Z, dX, dA, dB, workspace, workspace_bytes,
                   stream):
    return lib().lora4_backward(ctypes.byref(W), X, dY, M, A, B, r, s, group_offsets, Z, dX, dA, dB,
                                workspace, workspace_bytes, stream)


def lora4_forward_multi(W, adapters, X, M, A, B, r, s, adapter_offsets, Y, Z, Y_base, Y_lora, workspace,
                        workspace_bytes, stream):
    return lib().lora4_forward_multi(ctypes.byref(W), adapters, X, M, A, B, r, s, adapter_offsets, Y, Z, Y_base,
                                     Y_lora, workspace, workspace_bytes, stream)


def lora4_backward_multi(W, adapters, X, dY, M, A, B, r, s, adapter_offsets, Z, dX, dA, dB, workspace,
                         workspace_bytes, stream):
    return lib().lora4_backward_multi(ctypes.byref(W), adapters, X, dY, M, A, B, r, s, adapter_offsets, Z, dX,
                                      dA, dB, workspace, workspace_bytes, stream)


def lora4_workspace_bytes_multi(which, W, adapters, M, r):
    return lib().lora4_workspace_bytes_multi(which, ctypes.byref(W), adapters, M, r)


def quant_pack_nf4(W_bf16, N, K, double_quant, codes, scales, scales2, stream):
    return lib().quant_pack_nf4(W_bf16, N, K, double_quant, codes, scales, scales2, stream)


def quant_pack_mxfp4(W_bf16, N, K, codes, scales_e8m0, stream):
    return lib().quant_pack_mxfp4(W_bf16, N, K, codes, scales_e8m0, stream)


def quant_pack_nvfp4(W_bf16, N, K, codes, scales_e4m3, stream):
    return lib().quant_pack_nvfp4(W_bf16, N, K, codes, scales_e4m3, stream)


def quant_pack_mxfp8(X, M, K, codes, scales_e8m0, stream):
    return lib().quant_pack_mxfp8(X, M, K, codes, scales_e8m0, stream)


def lora4_workspace_bytes_mx(W, M, r):
    return lib().lora4_workspace_bytes_mx(ctypes.byref(W), M, r)


def lora4_loftq_workspace_bytes(N, K, r):
    return lib().lora4_loftq_workspace_bytes(N, K, r)


def lora4_loftq_init(W, N, K, r, iters, s, double_quant, codes, scales, scales2, A, B, workspace,
                     workspace_bytes, stream):
    return lib().lora4_loftq_init(W, N, K, r, iters, s, double_quant, codes, scales, scales2, A, B, workspace,
                                  workspace_bytes, stream)


def lora4_import_rowmajor(fmt, N, K, groups, codes_rm, scales_rm, codes, scales, stream):
    return lib().lora4_import_rowmajor(fmt, N, K, groups, codes_rm, scales_rm, codes, scales, stream)


def lora4_forward_mx(W, X, M, A, B, r, s, Y, Z, workspace, workspace_bytes, stream):
    return lib().lora4_forward_mx(ctypes.byref(W), X, M, A, B, r, s, Y, Z, workspace, workspace_bytes, stream)


def timing_enable(on=True):
    _check(lib().lora4_timing_enable(1 if on else 0), "lora4_timing_enable")


def timing_collect():
    """{kernel name: (launches, total_ms)} since the last collect."""
    buf = (lora4_kernel_time * 64)()
    n = lib().lora4_timing_collect(buf, 64)
    if n < 0:
        raise Lora4Error(n, "lora4_timing_collect")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n, 64))}


def version():
    return lib().lora4_version().decode()


# ---------------------------------------------------------------------------
# torch-level helpers (allocation + marshalling)
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _need(t, name, shape, dtype, device=None):
    """Raises ValueError unless t is a dense tensor of this shape and dtype (on
    `device` when given). The C ABI receives raw pointers only, so a short or
    mis-typed buffer would be read or written past its end by the kernels."""
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def check_layer_args(base, X, A, B, dY=None, Z=None, offsets=None, adapters=None, outputs=()):
    """Validates the tensors of one layer call before any pointer reaches the
    library: bf16, contiguous, on X's device, X [M, K], A [(G,) r, K],
    B [(G,) N, r], dY [M, N], Z [M, r], offsets int64 [G + 1]; G is the
    base's expert count, or `adapters` for several adapters over one base.
    `outputs` holds (name, tensor, shape) triples of caller-given outputs.
    Returns (M, r, G). Pure host logic (CPU tensors work)."""
    import torch
    bf = torch.bfloat16
    if X is None or X.dim() != 2:
        raise ValueError("X must be a 2-D tensor [M, K]")
    dev = X.device
    M = X.shape[0]
    _need(X, "X", (M, base.K), bf, dev)
    G = base.groups if adapters is None else int(adapters)
    if adapters is not None and base.groups != 1:
        raise ValueError("several adapters need a base with one group")
    if A is None or A.dim() not in (2, 3):
        raise ValueError("A must be [r, K] or [groups, r, K]")
    if A.dim() == 2 and G != 1:
        raise ValueError(f"A must be [groups={G}, r, K]")
    r = A.shape[-2]
    a_shape = (r, base.K) if A.dim() == 2 else (G, r, base.K)
    b_shape = (base.N, r) if A.dim() == 2 else (G, base.N, r)
    _need(A, "A", a_shape, bf, dev)
    _need(B, "B", b_shape, bf, dev)
    if dY is not None:
        _need(dY, "dY", (M, base.N), bf, dev)
    if Z is not None:
        _need(Z, "Z", (M, r), bf, dev)
    if G > 1:
        _need(offsets, "group offsets", (G + 1,), torch.int64, dev)
    elif offsets is not None:
        raise ValueError("group offsets are only taken with several groups")
    for name, t, shape in outputs:
        if t is not None:
            _need(t, name, shape, bf, dev)
    for name, t in (("codes", base.codes), ("scales", base.scales), ("scales2", base.scales2)):
        if t is not None and (t.device != dev or not t.is_contiguous()):
            raise ValueError(f"base {name} must be contiguous on {dev}")
    return M, r, G


def _check_workspace(ws, need, dev):
    import torch
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous() or ws.device != dev:
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor on the layer's device")
    if ws.numel() < need:
        raise ValueError(f"workspace has {ws.numel()} bytes, {need} needed")


def _check_pack_input(W):
    import torch
    if W is None or W.dim() not in (2, 3):
        raise ValueError("W must be [N, K] or [E, N, K]")
    if W.dtype != torch.bfloat16 or not W.is_contiguous():
        raise ValueError("W must be a contiguous bf16 tensor")


@dataclass
class PackedBase:
    """A frozen 4-bit base on the device, [groups][N][K] logically, stored in
    the library's 64 x 64 tiles (include/lora4.h, lora4_W)."""
    fmt: int
    N: int
    K: int
    groups: int
    codes: "object"            # torch uint8 [groups, packed_bytes(part 0)]
    scales: "object"           # float32 or uint8 [groups, scale entries]
    scales2: Optional["object"] = None

    def abi(self):
        return lora4_W(self.fmt, BLOCK[self.fmt], self.N, self.K, self.groups, _ptr(self.codes),
                       _ptr(self.scales), _ptr(self.scales2))


def pack_nf4(W, double_quant=False):
    """Quantize bf16 W ([N, K] or [E, N, K], on the GPU) to NF4 on the GPU."""
    import torch
    _check_pack_input(W)
    Ws = W if W.dim() == 3 else W.unsqueeze(0)
    E, N, K = Ws.shape
    dev = W.device
    fmt = LORA4_NF4_DQ if double_quant else LORA4_NF4
    sizes = [lora4_packed_bytes(fmt, N, K, part) for part in range(3)]
    if sizes[0] == 0:
        raise ValueError("invalid shape for NF4 packing")
    codes = torch.empty((E, sizes[0]), dtype=torch.uint8, device=dev)
    if double_quant:
        scales = torch.empty((E, sizes[1]), dtype=torch.uint8, device=dev)
        scales2 = torch.empty((E, sizes[2] // 4), dtype=torch.float32, device=dev)
    else:
        scales = torch.empty((E, sizes[1] // 4), dtype=torch.float32, device=dev)
        scales2 = None
    for e in range(E):
        st = quant_pack_nf4(_ptr(Ws[e]), N, K, 1 if double_quant else 0, _ptr(codes[e]), _ptr(scales[e]),
                            _ptr(scales2[e]) if double_quant else None, _stream())
        _check(st, "quant_pack_nf4")
    return PackedBase(fmt, N, K, E, codes, scales, scales2)


def pack_mxfp4(W):
    """Quantize bf16 W ([N, K] or [E, N, K], on the GPU) to MXFP4 on the GPU."""
    import torch
    _check_pack_input(W)
    Ws = W if W.dim() == 3 else W.unsqueeze(0)
    E, N, K = Ws.shape
    dev = W.device
    sizes = [lora4_packed_bytes(LORA4_MXFP4, N, K, part) for part in range(2)]
    if sizes[0] == 0:
        raise ValueError("invalid shape for MXFP4 packing")
    codes = torch.empty((E, sizes[0]), dtype=torch.uint8, device=dev)
    scales = torch.empty((E, sizes[1]), dtype=torch.uint8, device=dev)
    for e in range(E):
        _check(quant_pack_mxfp4(_ptr(Ws[e]), N, K, _ptr(codes[e]), _ptr(scales[e]), _stream()),
               "quant_pack_mxfp4")
    return PackedBase(LORA4_MXFP4, N, K, E, codes, scales, None)


def pack_nvfp4(W):
    """Quantize bf16 W ([N, K] or [E, N, K], on the GPU) to NVFP4 on the GPU."""
    import torch
    _check_pack_input(W)
    Ws = W if W.dim() == 3 else W.unsqueeze(0)
    E, N, K = Ws.shape
    dev = W.device
    sizes = [lora4_packed_bytes(LORA4_NVFP4, N, K, part) for part in range(2)]
    if sizes[0] == 0:
        raise ValueError("invalid shape for NVFP4 packing")
    codes = torch.empty((E, sizes[0]), dtype=torch.uint8, device=dev)
    scales = torch.empty((E, sizes[1]), dtype=torch.uint8, device=dev)
    for e in range(E):
        _check(quant_pack_nvfp4(_ptr(Ws[e]), N, K, _ptr(codes[e]), _ptr(scales[e]), _stream()),
               "quant_pack_nvfp4")
    return PackedBase(LORA4_NVFP4, N, K, E, codes, scales, None)


def import_rowmajor(fmt, codes_rm, scales_rm, scales2=None):
    """A base already packed row-major (codes uint8 [(E,) N, K/2], scales
    [(E,) N, K/block]: float32 for NF4, uint8 otherwise; NF4-DQ second-level
    scales float32 [(E,) ceil(N K/64/256)]) -> a PackedBase in the library's
    tiled storage (rearranged on the GPU, bit for bit)."""
    import torch
    fmt = FORMATS.get(fmt, fmt)
    if fmt not in BLOCK:
        raise ValueError("unknown format")
    c = codes_rm if codes_rm.dim() == 3 else codes_rm.unsqueeze(0)
    sc = scales_rm if scales_rm.dim() == 3 else scales_rm.unsqueeze(0)
    E, N, half = c.shape
    K = 2 * half
    dev = c.device
    _need(c, "codes", (E, N, half), torch.uint8, dev)
    _need(sc, "scales", (E, N, K // BLOCK[fmt]), torch.float32 if fmt == LORA4_NF4 else torch.uint8, dev)
    sizes = [lora4_packed_bytes(fmt, N, K, part) for part in range(3)]
    if sizes[0] == 0:
        raise ValueError("invalid shape for this format")
    codes = torch.empty((E, sizes[0]), dtype=torch.uint8, device=dev)
    if fmt == LORA4_NF4:
        scales = torch.empty((E, sizes[1] // 4), dtype=torch.float32, device=dev)
    else:
        scales = torch.empty((E, sizes[1]), dtype=torch.uint8, device=dev)
    s2 = None
    if fmt == LORA4_NF4_DQ:
        if scales2 is None:
            raise ValueError("NF4-DQ needs its second-level scales")
        s2 = scales2 if scales2.dim() == 2 else scales2.unsqueeze(0)
        _need(s2, "scales2", (E, sizes[2] // 4), torch.float32, dev)
    _check(lora4_import_rowmajor(fmt, N, K, E, _ptr(c), _ptr(sc), _ptr(codes), _ptr(scales), _stream()),
           "lora4_import_rowmajor")
    return PackedBase(fmt, N, K, E, codes, scales, s2)


def workspace_for(which, base, M, r):
    import torch
    n = lora4_workspace_bytes(which, base.abi(), M, r)
    if n == 0:
        raise ValueError("invalid arguments for lora4_workspace_bytes")
    return torch.empty((n,), dtype=torch.uint8, device=base.codes.device)


def _out(t, shape, dev):
    import torch
    return torch.empty(shape, dtype=torch.bfloat16, device=dev) if t is None else t


def forward(base, X, A, B, s, group_offsets=None, want_z=True, want_parts=False, workspace=None, out=None):
    """Y (and Z, Y_base, Y_lora) for bf16 X [M, K], A [(E,) r, K], B [(E,) N, r].
    `out` may hold caller-allocated outputs under the keys Y, Z, Y_base, Y_lora."""
    out = out or {}
    M, r, _ = check_layer_args(base, X, A, B, offsets=group_offsets, outputs=[
        ("Y", out.get("Y"), (X.shape[0], base.N)), ("Z", out.get("Z"), (X.shape[0], A.shape[-2])),
        ("Y_base", out.get("Y_base"), (X.shape[0], base.N)), ("Y_lora", out.get("Y_lora"), (X.shape[0], base.N))])
    dev = X.device
    Y = _out(out.get("Y"), (M, base.N), dev)
    Z = _out(out.get("Z"), (M, r), dev) if want_z or out.get("Z") is not None else None
    Yb = _out(out.get("Y_base"), (M, base.N), dev) if want_parts or out.get("Y_base") is not None else None
    Yl = _out(out.get("Y_lora"), (M, base.N), dev) if want_parts or out.get("Y_lora") is not None else None
    W = base.abi()
    need = lora4_workspace_bytes(0, W, M, r)
    if need == 0:
        raise ValueError("invalid arguments for lora4_workspace_bytes")
    if workspace is None:
        workspace = workspace_for(0, base, M, r)
    _check_workspace(workspace, need, dev)
    st = lora4_forward(W, _ptr(X), M, _ptr(A), _ptr(B), r, float(s), _ptr(group_offsets), _ptr(Y), _ptr(Z),
                       _ptr(Yb), _ptr(Yl), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "lora4_forward")
    return {"Y": Y, "Z": Z, "Y_base": Yb, "Y_lora": Yl}


def forward_noalloc(base, X, A, B, s, group_offsets=None, want_z=True, want_parts=False, out=None):
    """lora4_forward through the entry point that allocates nothing (its
    scratch is the library's static device array): same arguments as
    forward() without the workspace."""
    out = out or {}
    M, r, _ = check_layer_args(base, X, A, B, offsets=group_offsets, outputs=[
        ("Y", out.get("Y"), (X.shape[0], base.N)), ("Z", out.get("Z"), (X.shape[0], A.shape[-2])),
        ("Y_base", out.get("Y_base"), (X.shape[0], base.N)), ("Y_lora", out.get("Y_lora"), (X.shape[0], base.N))])
    dev = X.device
    Y = _out(out.get("Y"), (M, base.N), dev)
    Z = _out(out.get("Z"), (M, r), dev) if want_z or out.get("Z") is not None else None
    Yb = _out(out.get("Y_base"), (M, base.N), dev) if want_parts or out.get("Y_base") is not None else None
    Yl = _out(out.get("Y_lora"), (M, base.N), dev) if want_parts or out.get("Y_lora") is not None else None
    st = lora4_forward_noalloc(base.abi(), _ptr(X), M, _ptr(A), _ptr(B), r, float(s), _ptr(group_offsets),
                               _ptr(Y), _ptr(Z), _ptr(Yb), _ptr(Yl), _stream())
    _check(st, "lora4_forward_noalloc")
    return {"Y": Y, "Z": Z, "Y_base": Yb, "Y_lora": Yl}


def forward_multi(base, X, A, B, s, adapter_offsets=None, want_z=True, want_parts=False, workspace=None, out=None):
    """Several adapters over one shared base: A [adapters, r, K], B [adapters, N, r]
    (rows of X pre-sorted by adapter, adapter_offsets a device int64 [adapters+1])."""
    out = out or {}
    if A is None or A.dim() != 3:
        raise ValueError("A must be [adapters, r, K]")
    adapters = A.shape[0]
    M, r, _ = check_layer_args(base, X, A, B, offsets=adapter_offsets, adapters=adapters, outputs=[
        ("Y", out.get("Y"), (X.shape[0], base.N)), ("Z", out.get("Z"), (X.shape[0], A.shape[-2])),
        ("Y_base", out.get("Y_base"), (X.shape[0], base.N)), ("Y_lora", out.get("Y_lora"), (X.shape[0], base.N))])
    dev = X.device
    Y = _out(out.get("Y"), (M, base.N), dev)
    Z = _out(out.get("Z"), (M, r), dev) if want_z or out.get("Z") is not None else None
    Yb = _out(out.get("Y_base"), (M, base.N), dev) if want_parts or out.get("Y_base") is not None else None
    Yl = _out(out.get("Y_lora"), (M, base.N), dev) if want_parts or out.get("Y_lora") is not None else None
    W = base.abi()
    n = lora4_workspace_bytes_multi(0, W, adapters, M, r)
    if n == 0:
        raise ValueError("invalid arguments for lora4_workspace_bytes_multi")
    if workspace is None:
        import torch
        workspace = torch.empty((n,), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, n, dev)
    st = lora4_forward_multi(W, adapters, _ptr(X), M, _ptr(A), _ptr(B), r, float(s), _ptr(adapter_offsets),
                             _ptr(Y), _ptr(Z), _ptr(Yb), _ptr(Yl), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "lora4_forward_multi")
    return {"Y": Y, "Z": Z, "Y_base": Yb, "Y_lora": Yl}


def backward_multi(base, X, dY, A, B, s, Z=None, adapter_offsets=None, workspace=None, out=None):
    """dX, dA [adapters, r, K], dB [adapters, N, r] for several adapters over one base."""
    import torch
    out = out or {}
    if A is None or A.dim() != 3:
        raise ValueError("A must be [adapters, r, K]")
    adapters = A.shape[0]
    M, r, _ = check_layer_args(base, X, A, B, dY=dY, Z=Z, offsets=adapter_offsets, adapters=adapters, outputs=[
        ("dX", out.get("dX"), (X.shape[0], base.K)), ("dA", out.get("dA"), tuple(A.shape)),
        ("dB", out.get("dB"), tuple(B.shape))])
    dev = X.device
    dX = _out(out.get("dX"), (M, base.K), dev)
    dA = out.get("dA") if out.get("dA") is not None else torch.empty_like(A)
    dB = out.get("dB") if out.get("dB") is not None else torch.empty_like(B)
    W = base.abi()
    n = lora4_workspace_bytes_multi(1, W, adapters, M, r)
    if n == 0:
        raise ValueError("invalid arguments for lora4_workspace_bytes_multi")
    if workspace is None:
        workspace = torch.empty((n,), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, n, dev)
    st = lora4_backward_multi(W, adapters, _ptr(X), _ptr(dY), M, _ptr(A), _ptr(B), r, float(s),
                              _ptr(adapter_offsets), _ptr(Z), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(workspace),
                              workspace.numel(), _stream())
    _check(st, "lora4_backward_multi")
    return {"dX": dX, "dA": dA, "dB": dB}


def backward(base, X, dY, A, B, s, Z=None, group_offsets=None, workspace=None, out=None):
    """dX, dA, dB for bf16 inputs (Z from forward, or None to recompute).
    `out` may hold caller-allocated outputs under the keys dX, dA, dB."""
    import torch
    out = out or {}
    M, r, _ = check_layer_args(base, X, A, B, dY=dY, Z=Z, offsets=group_offsets, outputs=[
        ("dX", out.get("dX"), (X.shape[0], base.K)), ("dA", out.get("dA"), tuple(A.shape)),
        ("dB", out.get("dB"), tuple(B.shape))])
    dev = X.device
    dX = _out(out.get("dX"), (M, base.K), dev)
    dA = out.get("dA") if out.get("dA") is not None else torch.empty_like(A)
    dB = out.get("dB") if out.get("dB") is not None else torch.empty_like(B)
    W = base.abi()
    need = lora4_workspace_bytes(1, W, M, r)
    if need == 0:
        raise ValueError("invalid arguments for lora4_workspace_bytes")
    if workspace is None:
        workspace = workspace_for(1, base, M, r)
    _check_workspace(workspace, need, dev)
    st = lora4_backward(W, _ptr(X), _ptr(dY), M, _ptr(A), _ptr(B), r, float(s), _ptr(group_offsets), _ptr(Z),
                        _ptr(dX), _ptr(dA), _ptr(dB), _ptr(workspace), workspace.numel(), _stream())
    _check(st, "lora4_backward")
    return {"dX": dX, "dA": dA, "dB": dB}


def mxfp8(X):
    """bf16 X [M, K] (K % 32 == 0, on the GPU) -> MXFP8 E4M3 codes [M, K] and
    E8M0 scales [M, K / 32], both uint8."""
    import torch
    if X is None or X.dim() != 2:
        raise ValueError("X must be [M, K]")
    M, K = X.shape
    _need(X, "X", (M, K), torch.bfloat16)
    codes = torch.empty((M, K), dtype=torch.uint8, device=X.device)
    scales = torch.empty((M, K // 32), dtype=torch.uint8, device=X.device)
    _check(quant_pack_mxfp8(_ptr(X), M, K, _ptr(codes), _ptr(scales), _stream()), "quant_pack_mxfp8")
    return codes, scales


def forward_mx(base, X, A, B, s, want_z=True, workspace=None):
    """MX-native forward of a plain MXFP4 layer: Y (and Z) for bf16 X [M, K],
    A [r, K], B [N, r]; the base product takes X as MXFP8."""
    import torch
    M, r, _ = check_layer_args(base, X, A, B)
    dev = X.device
    Y = torch.empty((M, base.N), dtype=torch.bfloat16, device=dev)
    Z = torch.empty((M, r), dtype=torch.bfloat16, device=dev) if want_z else None
    W = base.abi()
    if workspace is None:
        n = lora4_workspace_bytes_mx(W, M, r)
        if n == 0:
            raise ValueError("invalid arguments for lora4_workspace_bytes_mx")
        workspace = torch.empty((n,), dtype=torch.uint8, device=dev)
    st = lora4_forward_mx(W, _ptr(X), M, _ptr(A), _ptr(B), r, float(s), _ptr(Y), _ptr(Z), _ptr(workspace),
                          workspace.numel(), _stream())
    _check(st, "lora4_forward_mx")
    return {"Y": Y, "Z": Z}


def loftq_init(W, r, iters=5, s=1.0, double_quant=False):
    """LoftQ initialisation of a bf16 W [N, K] on the GPU: returns the NF4
    (or NF4-DQ) PackedBase of the base and the adapter A [r, K], B [N, r]
    (B divided by the layer scale s)."""
    import torch
    if W is None or W.dim() != 2:
        raise ValueError("W must be [N, K]")
    _check_pack_input(W)
    N, K = W.shape
    dev = W.device
    fmt = LORA4_NF4_DQ if double_quant else LORA4_NF4
    sizes = [lora4_packed_bytes(fmt, N, K, part) for part in range(3)]
    if sizes[0] == 0:
        raise ValueError("invalid shape for NF4 packing")
    codes = torch.empty((1, sizes[0]), dtype=torch.uint8, device=dev)
    if double_quant:
        scales = torch.empty((1, sizes[1]), dtype=torch.uint8, device=dev)
        scales2 = torch.empty((1, sizes[2] // 4), dtype=torch.float32, device=dev)
    else:
        scales = torch.empty((1, sizes[1] // 4), dtype=torch.float32, device=dev)
        scales2 = None
    A = torch.empty((r, K), dtype=torch.bfloat16, device=dev)
    B = torch.empty((N, r), dtype=torch.bfloat16, device=dev)
    n = lora4_loftq_workspace_bytes(N, K, r)
    if n == 0:
        raise ValueError("invalid arguments for lora4_loftq_workspace_bytes")
    ws = torch.empty((n,), dtype=torch.uint8, device=dev)
    _check(lora4_loftq_init(_ptr(W), N, K, r, iters, float(s), 1 if double_quant else 0, _ptr(codes), _ptr(scales),
                            _ptr(scales2), _ptr(A), _ptr(B), _ptr(ws), ws.numel(), _stream()), "lora4_loftq_init")
    return PackedBase(fmt, N, K, 1, codes, scales, scales2), A, B
