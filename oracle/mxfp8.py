"""MXFP8 activations and the MX-native base product of an MXFP4 base.

Test infrastructure only (see the package docstring).

Source: the Crusoe post, "Forward pass in inference" (on hardware with
MXFP4-native operations the base product of an MXFP4 base runs natively while
the adapters stay in bf16) and "Forward pass in training" (the same
operations and quantizations in the training forward). The pages do not say
in which format the activations enter that operation. Reading taken: the OCP
Microscaling v1.0 MXFP8 format, as for the MXFP4 base -- E4M3 elements with one
E8M0 scale per 32 consecutive elements of a row of X (along K):

* shared exponent ``Xe = floor(log2(amax)) - 8`` (8 is the largest E4M3
  exponent: 448 = 1.75 * 2^8), clamped to [-127, 127], stored as
  ``E = Xe + 127``; an all-zero block stores E = 0;
* element ``v = x * 2^-Xe`` (exact); ``|v|`` rounded to the nearest E4M3 value,
  ties to the even code, saturating at 448 (0x7E); the sign bit is copied from
  x, so -0 encodes as 0x80;
* value of a code: ``e4m3(code) * 2^(E-127)``.

The base product is ``sum_k deq8(x)[k] * deq4(w)[k]`` (every product exact,
summed in float64 here). Only the base product sees the quantized X:
Z = X A^T and s Z B^T use the bf16 X and bf16 adapters, as in the plain
forward.
"""

import numpy as np

from .codecs import bf16_to_f32, e4m3_decode, e4m3_encode_rne, e8m0_decode
from . import lora, mxfp4

BLOCK = 32
EMAX_E4M3 = 8          # 448 = 1.75 * 2^8
MAX_E4M3 = 448.0


def shared_exponents(x_bf16, block=BLOCK):
    """E8M0 code per block of ``block`` consecutive elements of each row."""
    x = bf16_to_f32(x_bf16).astype(np.float64)
    m, k = x.shape
    if k % block:
        raise ValueError("K must be a multiple of the block size")
    amax = np.abs(x.reshape(m, k // block, block)).max(axis=2)
    _, e = np.frexp(amax)            # amax = f * 2^e with f in [0.5, 1)
    Xe = (e - 1) - EMAX_E4M3         # floor(log2 amax) - emax(E4M3)
    Xe = np.where(amax == 0, -127, Xe)
    Xe = np.clip(Xe, -127, 127)
    return (Xe + 127).astype(np.uint8)


def encode(x_bf16, e8m0, block=BLOCK):
    """E4M3 codes [M, K] of x scaled by the given block exponents."""
    x = bf16_to_f32(x_bf16).astype(np.float64)
    Xe = np.repeat(e8m0.astype(np.int64) - 127, block, axis=1)
    v = np.ldexp(x, -Xe)                      # exact: a power-of-two scaling
    mag = np.minimum(np.abs(v), MAX_E4M3)     # saturate
    codes = e4m3_encode_rne(mag)
    sign = np.signbit(x).astype(np.uint8) << 7
    return (codes | sign).astype(np.uint8)


def quantize(x_bf16, block=BLOCK):
    """bf16 X [M, K] -> (E4M3 codes [M, K] uint8, E8M0 scales [M, K/32] uint8)."""
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    e = shared_exponents(x_bf16, block)
    return encode(x_bf16, e, block), e


def dequantize(codes, e8m0, block=BLOCK):
    """E4M3 codes + E8M0 scales -> float64 values e4m3(code) * 2^(E-127)."""
    return e4m3_decode(codes) * np.repeat(e8m0_decode(e8m0), block, axis=1)


def forward(X, W_codes, W_scales, A, B, s):
    """MX-native forward of one layer (float64).

    X [M, K], A [r, K], B [N, r]: bf16 bit patterns; W_codes [N, K/2] and
    W_scales [N, K/32]: the MXFP4 base in the oracle's row-major packing.
    Returns Y, Z, Y_base (float64) and the quantized X (codes, scales).
    """
    xc, xs = quantize(X)
    Xq = dequantize(xc, xs)
    Wd = lora.as_f64(mxfp4.dequantize(W_codes, W_scales))
    Xf, Af, Bf = lora.as_f64(X), lora.as_f64(A), lora.as_f64(B)
    Z = Xf @ Af.T
    Y_base = Xq @ Wd.T
    Y = Y_base + s * (Z @ Bf.T)
    return {"Y": Y, "Z": Z, "Y_base": Y_base, "X_codes": xc, "X_scales": xs}
