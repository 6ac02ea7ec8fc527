"""Helpers shared by the GPU tests: moving bf16 bit patterns between numpy and
torch, packing on the GPU through the C ABI, and oracle references."""

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


def tile_codes(codes, N, K):
    """Row-major codes [N, K/2] -> the library's storage: 64 x 64-element tiles
    (2048 bytes, 32 per row), tile (rb, kb) at rb * KB + kb, zero padding."""
    RB, KB = _blocks(N), _blocks(K)
    buf = np.zeros((RB * 64, KB * 32), dtype=np.uint8)
    buf[:N, :codes.shape[1]] = codes
    return np.ascontiguousarray(buf.reshape(RB, 64, KB, 32).transpose(0, 2, 1, 3)).reshape(-1)


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
