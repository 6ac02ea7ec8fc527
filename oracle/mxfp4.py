"""MXFP4: E2M1 element codes with one E8M0 scale per 32 consecutive elements.

Test infrastructure only (see the package docstring).

Source: "Fine-Tuning 4-Bit Models: Adapting a Base That Only Ships
Quantized", section "Case 2" (MXFP4 uses 32-element blocks with an E8M0
scale); the Crusoe post, "Forward pass in training" (a base released in 4-bit
is dequantized to bf16 in flight with no precision loss).

Readings where the pages are silent (the OCP Microscaling v1.0 conversion):
* shared exponent ``X = floor(log2(amax)) - 2`` (2 is the largest E2M1
  exponent), clamped to [-127, 127], stored as ``E = X + 127``; an all-zero
  block stores E = 0;
* element ``v = w * 2^-X`` (exact), magnitude rounded to the nearest E2M1
  value, ties to the even code, saturating at 6; the sign bit is copied from
  w, so -0 encodes as code 8;
* byte j of a row holds element 2j in its low nibble, 2j+1 in its high nibble;
* dequant ``bf16(e2m1(code) * 2^(E-127))``: exact wherever the product is a
  finite bf16 (it always is for E <= 252); larger products round to +-inf;
  E = 255 (NaN scale) gives NaN.
"""

import numpy as np

from .codecs import bf16_to_f32, e2m1_decode, e8m0_decode, f32_to_bf16
from .nf4 import pack_nibbles, unpack_nibbles

BLOCK = 32
_MAGS = e2m1_decode(np.arange(8))  # 0, .5, 1, 1.5, 2, 3, 4, 6


def shared_exponents(w_bf16, block=BLOCK):
    """E8M0 code per block of ``block`` consecutive elements of each row."""
    w = bf16_to_f32(w_bf16).astype(np.float64)
    n, k = w.shape
    if k % block:
        raise ValueError("K must be a multiple of the block size")
    amax = np.abs(w.reshape(n, k // block, block)).max(axis=2)
    _, e = np.frexp(amax)            # amax = m * 2^e with m in [0.5, 1)
    X = (e - 1) - 2                  # floor(log2 amax) - emax(E2M1)
    X = np.where(amax == 0, -127, X)
    X = np.clip(X, -127, 127)
    return (X + 127).astype(np.uint8)


def encode_codes(w_bf16, e8m0, block=BLOCK):
    """Unpacked E2M1 codes [N, K] for given E8M0 block scales."""
    w = bf16_to_f32(w_bf16).astype(np.float64)
    X = np.repeat(e8m0.astype(np.int64) - 127, block, axis=1)
    v = np.ldexp(w, -X)
    a = np.abs(v)
    d = np.abs(a[..., None] - _MAGS)
    dmin = d.min(axis=-1, keepdims=True)
    codes = np.arange(8)
    # nearest magnitude; on a tie the even code; above 6 the nearest is 6
    pref = np.where(d == dmin, codes & 1, 2)
    mag_code = np.argmin(pref, axis=-1).astype(np.uint8)
    sign = (np.signbit(w)).astype(np.uint8) << 3
    return (mag_code | sign).astype(np.uint8)


def quantize(w_bf16, block=BLOCK):
    """bf16 W [N, K] -> (packed codes [N, K/2] uint8, E8M0 scales [N, K/32] uint8)."""
    w_bf16 = np.asarray(w_bf16, dtype=np.uint16)
    e = shared_exponents(w_bf16, block)
    return pack_nibbles(encode_codes(w_bf16, e, block)), e


def dequantize(packed, e8m0, block=BLOCK):
    """Packed codes + E8M0 scales -> bf16 bit patterns of e2m1(code) * 2^(E-127)."""
    codes = unpack_nibbles(packed)
    val = e2m1_decode(codes) * np.repeat(e8m0_decode(e8m0), block, axis=1)
    return f32_to_bf16_exact_from_f64(val)


def f32_to_bf16_exact_from_f64(val):
    """float64 value -> bf16 (round to nearest even), for products that fit.

    Every e2m1 x 2^k product has at most 2 significant bits, so it is exactly
    representable in float32 unless it overflows or underflows binary32;
    those cases are handled explicitly (overflow -> +-inf, values below the
    smallest bf16 subnormal do not occur because the smallest product is
    0.5 * 2^-127 = 2^-128).
    """
    v = np.asarray(val, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        f = v.astype(np.float32)
    return f32_to_bf16(f)
