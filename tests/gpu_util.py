"""Helpers shared by the GPU tests: moving bf16 bit patterns between numpy and
torch, packing on the GPU through the C ABI, and oracle references."""

import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import lora_fine_tuning_amd as L
import synth
from oracle import codecs, lora, mxfp4, nf4, nvfp4

DEV = "cuda:0"
TOL = 5e-3   # relative Frobenius error bar for float outputs


def to_dev(u16):
    """numpy uint16 bf16 bits -> torch bf16 on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_host(t):
    """torch bf16 -> numpy uint16 bits."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(u16):
    return codecs.bf16_to_f32(u16).astype(np.float64)


def pack_gpu(W_u16, fmt):
    """Pack bf16 W ([N,K] or [E,N,K]) on the GPU with the library."""
    Wd = to_dev(W_u16)
    if fmt == synth.MXFP4:
        return L.pack_mxfp4(Wd)
    if fmt == synth.NVFP4:
        return L.pack_nvfp4(Wd)
    return L.pack_nf4(Wd, double_quant=(fmt == synth.NF4_DQ))


def _blocks(x):
    return -(-x // 64)


# NF4 code words in the library's storage: element i of each 8-element word
# (row-major: nibble i) sits at nibble NF4_NIBBLE[i] (include/lora4.h: byte j
# holds elements j and j + 4).
NF4_NIBBLE = [0, 2, 4, 6, 1, 3, 5, 7]


def _nf4_words(codes, inverse=False):
    """Row-major NF4 code bytes (rows of whole 4-byte words) <-> the storage's
    nibble order, word by word."""
    w = np.ascontiguousarray(codes).view(np.uint32)
    out = np.zeros_like(w)
    for i, pos in enumerate(NF4_NIBBLE):
        src, dst = (pos, i) if inverse else (i, pos)
        out |= ((w >> np.uint32(4 * src)) & np.uint32(15)) << np.uint32(4 * dst)
    return out.view(np.uint8).reshape(codes.shape)


def tile_codes(codes, N, K, fmt):
    """Row-major codes [N, K/2] of format fmt -> the library's storage: 64 x
    64-element tiles (2048 bytes, 32 per row), tile (rb, kb) at rb * KB + kb,
    zero padding; NF4 and NF4-DQ words in the storage's nibble order."""
    RB, KB = _blocks(N), _blocks(K)
    buf = np.zeros((RB * 64, KB * 32), dtype=np.uint8)
    buf[:N, :codes.shape[1]] = codes
    if fmt in (synth.NF4, synth.NF4_DQ):
        buf = _nf4_words(buf)
    return np.ascontiguousarray(buf.reshape(RB, 64, KB, 32).transpose(0, 2, 1, 3)).reshape(-1)


def untile_codes(flat, N, K, rows, fmt):
    """Rows of the stored codes back as row-major bytes (K/2 per row)."""
    c = np.ascontiguousarray(untile_rows(flat, N, K, rows, 32))
    return _nf4_words(c, inverse=True) if fmt in (synth.NF4, synth.NF4_DQ) else c


def tile_scales(sc, N, K):
    """Row-major first-level scales [N, K/64] (NF4, NF4-DQ) or [N, K/32]
    (MXFP4) -> the library's storage: 64 (or 128) entries per tile, row i's
    entries contiguous, zero padding."""
    RB, KB = _blocks(N), _blocks(K)
    per = sc.shape[1] * 64 // K                # entries per row and tile: 1 (NF4), 2 (MXFP4), 4 (NVFP4)
    buf = np.zeros((RB * 64, KB * per), dtype=sc.dtype)
    buf[:N, :sc.shape[1]] = sc
    return np.ascontiguousarray(buf.reshape(RB, 64, KB, per).transpose(0, 2, 1, 3)).reshape(-1)


def untile_rows(flat, N, K, rows, per_row):
    """Rows of a tiled array (codes: per_row = 32 bytes per 64 elements;
    scales: 1 or 2 entries per 64 elements) back in row-major order, K-padding
    dropped."""
    RB, KB = _blocks(N), _blocks(K)
    t = flat.reshape(RB, KB, 64, per_row).transpose(0, 2, 1, 3).reshape(RB * 64, KB * per_row)
    width = K // 2 if per_row == 32 else {1: K // 64, 2: K // 32, 4: K // 16}[per_row]
    return t[rows, :width]


def oracle_pack(W_u16, fmt):
    """Oracle packing of one [N, K] matrix: (codes, scales[, scales2])."""
    if fmt == synth.MXFP4:
        return mxfp4.quantize(W_u16)
    if fmt == synth.NVFP4:
        return nvfp4.quantize(W_u16)
    codes, sc = nf4.quantize(W_u16)
    if fmt == synth.NF4_DQ:
        c8, c2 = nf4.double_quantize(sc)
        return codes, c8, c2
    return codes, sc


def oracle_dequant(packed, fmt):
    """bf16 bits of the oracle dequant of an oracle packing."""
    if fmt == synth.MXFP4:
        return mxfp4.dequantize(packed[0], packed[1])
    if fmt == synth.NVFP4:
        return nvfp4.dequantize(packed[0], packed[1])
    if fmt == synth.NF4_DQ:
        return nf4.dequantize_dq(packed[0], packed[1], packed[2])
    return nf4.dequantize(packed[0], packed[1])


def dequant_rows(W_u16, rows, fmt):
    """Oracle dequant (float64) of selected rows of W (packing is row-local
    except for double quantization, whose groups span rows: there the whole
    matrix is packed once)."""
    if fmt == synth.NF4_DQ:
        full = oracle_dequant(oracle_pack(W_u16, fmt), fmt)
        return f64(full[rows])
    sub = W_u16[rows]
    return f64(oracle_dequant(oracle_pack(sub, fmt), fmt))


def dequant_cols(W_u16, k0, k1, fmt):
    """Oracle dequant (float64) of columns k0..k1 (block aligned) of every row."""
    if fmt == synth.NF4_DQ:
        full = oracle_dequant(oracle_pack(W_u16, fmt), fmt)
        return f64(full[:, k0:k1])
    return f64(oracle_dequant(oracle_pack(np.ascontiguousarray(W_u16[:, k0:k1]), fmt), fmt))


def rel(got_u16_or_f, ref):
    g = got_u16_or_f
    if isinstance(g, np.ndarray) and g.dtype == np.uint16:
        g = f64(g)
    return lora.rel_frobenius(g, ref)


def print_case(*args):
    print("[case]", *args, flush=True)


# ---------------------------------------------------------------------------
# Full-size parity: the oracle over whole matrices, guard bands, element bounds
# ---------------------------------------------------------------------------

# Host threads for the row chunks of the oracle's packing and dequant (at
# most 16: the host share of one GPU). numpy releases the GIL inside its array
# loops, so threads run the chunks in parallel; the oracle functions are the
# same, called on row ranges (every format packs rows independently, except
# the double quantization of NF4-DQ's scales, applied to the whole matrix).
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def _row_chunks(n, k):
    rows = max(16, (1 << 20) // max(k, 1))
    return [(i, min(n, i + rows)) for i in range(0, n, rows)]


def oracle_pack_full(W_u16, fmt):
    """Oracle packing of a whole [N, K] matrix, row-major: (codes, scales[,
    scales2]) exactly as oracle_pack returns them."""
    N, K = W_u16.shape
    first = synth.NF4 if fmt == synth.NF4_DQ else fmt
    chunks = _row_chunks(N, K)
    with ThreadPoolExecutor(WORKERS) as ex:
        parts = list(ex.map(lambda ab: oracle_pack(W_u16[ab[0]:ab[1]], first), chunks))
    codes = np.concatenate([p[0] for p in parts])
    scales = np.concatenate([p[1] for p in parts])
    if fmt == synth.NF4_DQ:
        c8, c2 = nf4.double_quantize(scales)
        return codes, c8, c2
    return codes, scales


def oracle_dequant_full(packed, fmt):
    """float64 deq(W) [N, K] of an oracle packing (row chunks in threads)."""
    codes = packed[0]
    N = codes.shape[0]
    if fmt == synth.NF4_DQ:
        sc = nf4.rebuild_scales(packed[1], packed[2])     # the whole matrix's rebuilt scales
        fn = lambda a, b: nf4.dequantize(codes[a:b], sc[a:b])
    else:
        fn = lambda a, b: oracle_dequant((codes[a:b], packed[1][a:b]), fmt)
    out = np.empty((N, codes.shape[1] * 2))

    def work(ab):
        out[ab[0]:ab[1]] = f64(fn(*ab))
    with ThreadPoolExecutor(WORKERS) as ex:
        list(ex.map(work, _row_chunks(N, codes.shape[1] * 2)))
    return out


GUARD = 4096          # elements of sentinel before and after a guarded buffer
SENTINEL16 = 0x7FA5   # a bf16 NaN pattern no kernel writes
SENTINEL8 = 0xA5


def guarded(shape, dtype=torch.bfloat16):
    """A tensor of `shape` inside a larger buffer whose GUARD elements on
    each side hold a sentinel; returns (view, check) where check() asserts
    the sentinels are untouched. The view keeps 16-byte alignment."""
    n = int(np.prod(shape)) if len(shape) else 1
    buf = torch.empty((n + 2 * GUARD,), dtype=dtype, device=DEV)
    if dtype == torch.uint8:
        buf.fill_(SENTINEL8)
        raw = buf
        pat = SENTINEL8
    else:
        raw = buf.view(torch.int16)
        raw.fill_(SENTINEL16 - 0x10000 if SENTINEL16 >= 0x8000 else SENTINEL16)
        pat = SENTINEL16
    view = buf[GUARD:GUARD + n].view(shape)

    def check(name="buffer"):
        lo = raw[:GUARD].cpu().numpy().view(np.uint8 if dtype == torch.uint8 else np.uint16)
        hi = raw[GUARD + n:].cpu().numpy().view(np.uint8 if dtype == torch.uint8 else np.uint16)
        assert np.all(lo == pat) and np.all(hi == pat), f"{name}: a kernel wrote outside the buffer"
    return view, check


ELEM_U = 2.0 ** -8     # bf16 unit roundoff (8 significant bits, nearest even)
ELEM_FLOOR = 2.0 ** -9


def element_bound(ref, inter=None):
    """Per-element bound on |gpu - oracle| for a bf16 output whose exact value
    is `ref` (float64): the output's own rounding, u |ref|; the rounding of a
    bf16 intermediate feeding it (Z or dZ, rounded once to bf16), u times
    `inter` = the sum of the absolute values of the terms that intermediate
    enters (e.g. |s| |Z| |B|^T for Y); the product (1 + 1/100) covers the
    rounding of the rounded values themselves; and a floor of 2^-9 rms(ref) for
    the fp32 accumulation (measured errors are below 1e-5 rms)."""
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0
    b = np.abs(ref) if inter is None else np.abs(ref) + inter
    return ELEM_U * 1.01 * b + ELEM_FLOOR * rms


def compare_full(name, got, ref, inter=None, report=None):
    """Every element of a bf16 output against the oracle: relative Frobenius
    error <= TOL and |got - ref| <= element_bound(ref, inter) everywhere.
    Returns (rel_frobenius, max |got - ref| / rms(ref), max error / bound)."""
    g = f64(got) if isinstance(got, np.ndarray) and got.dtype == np.uint16 else np.asarray(got, np.float64)
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    err = np.abs(g - ref)
    rf = lora.rel_frobenius(g, ref)
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0
    bound = element_bound(ref, inter)
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if ref.size else 0.0
    maxrel = float(np.max(err) / rms) if rms > 0 else float(np.max(err, initial=0.0))
    if report is not None:
        report[name] = {"rel_frobenius": rf, "max_err_over_rms": maxrel, "max_err_over_bound": worst}
    assert np.all(np.isfinite(g)), f"{name}: non-finite output"
    assert rf <= TOL, (name, rf)
    assert worst <= 1.0, (name, worst, maxrel)
    return rf, maxrel, worst


def write_report(case, report):
    """Appends one JSON line per case to $LORA4_PARITY_REPORT when it is set."""
    path = os.environ.get("LORA4_PARITY_REPORT")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps({"case": case, **report}) + "\n")


# Tile paths of the library, forced through its environment switches:
#  auto     : the library's own choice
#  big      : the register-direct forward and the 256 x 256 dgrad (LORA4_BIG=1)
#  small    : the 128 x 128 LDS kernels (LORA4_BIG=0)
#  half     : big, every forward tile as two 256 x 128 halves
#  mixed    : big, the second half of the forward tiles as halves
#  fwdsmall : big, the forward on 128 x 128 register-direct tiles
TILE_PATHS = ["auto", "big", "small", "half", "mixed", "fwdsmall"]


def set_tiles(monkeypatch, name):
    monkeypatch.delenv("LORA4_BIG", raising=False)
    monkeypatch.delenv("LORA4_FWD_TILES", raising=False)
    if name == "auto":
        return name
    monkeypatch.setenv("LORA4_BIG", "0" if name == "small" else "1")
    if name in ("half", "mixed"):
        monkeypatch.setenv("LORA4_FWD_TILES", name)
    elif name == "fwdsmall":
        monkeypatch.setenv("LORA4_FWD_TILES", "small")
    return name
