"""Scalar number formats used by the path, written from their definitions.

Test infrastructure only (see the package docstring).

* bf16: the top 16 bits of an IEEE binary32; fp32 -> bf16 rounds to nearest,
  ties to even. The pages fix bf16 for activations, adapters and gradients
  (Crusoe post, "Backward pass and optimizer step in training": the
  gradients are named dL/dA_bf16, dL/dB_bf16, dL/dX_bf16).
* E4M3 ("FP8", OCP E4M3FN: bias 7, no infinities, 0x7F/0xFF are NaN): the
  first-level scale format of double quantization ("Training LLMs on a
  Budget", section 3, trick 2, "8-bit FP8").
* E2M1 (FP4) element codes and E8M0 (power-of-two) block scales of MXFP4
  ("Fine-Tuning 4-Bit Models", section "Case 2": 32-element blocks with an
  E8M0 scale).
"""

import numpy as np


# ----------------------------------------------------------------------------
# bf16
# ----------------------------------------------------------------------------

def bf16_to_f32(u16):
    """bf16 bit patterns (uint16) -> float32 values, exactly (u << 16)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f32_to_bf16(x):
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    On the integer view u of a finite binary32: add 0x7FFF plus the lowest
    kept bit, then drop the low 16 bits. Overflow carries into the exponent
    and yields +-inf, as round-to-nearest requires. NaN maps to a quiet NaN
    with the same sign.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(f)
    if nan.any():
        r = np.where(nan, (u.astype(np.uint32) >> np.uint32(16)) | np.uint32(0x0040), r)
    return r.astype(np.uint16)


def bf16_round(x):
    """Round float values to the nearest bf16 and return them as float64."""
    return bf16_to_f32(f32_to_bf16(np.asarray(x, dtype=np.float32))).astype(np.float64)


# ----------------------------------------------------------------------------
# E4M3 (OCP E4M3FN)
# ----------------------------------------------------------------------------

def e4m3_decode(code):
    """E4M3FN code (uint8) -> float64 value.

    sign = bit 7, exponent field e = bits 6..3 (bias 7), mantissa m = bits
    2..0. e = 0 is subnormal: m/8 * 2^-6; otherwise (1 + m/8) * 2^(e-7).
    Codes 0x7F and 0xFF are NaN; there is no infinity (max finite 448).
    """
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


_E4M3_POS = None


def _e4m3_positive_table():
    global _E4M3_POS
    if _E4M3_POS is None:
        codes = np.arange(0, 0x7F, dtype=np.uint8)  # 0x00..0x7E: all non-negative finite codes
        _E4M3_POS = (codes, e4m3_decode(codes))
    return _E4M3_POS


def e4m3_encode_rne(x):
    """Non-negative finite value -> E4M3FN code, nearest, ties to even code.

    Brute force over the 127 non-negative finite codes: pick the code whose
    value is nearest to x; on an exact tie pick the code with an even
    mantissa (the even code). Values above 448 saturate to 448 (0x7E). Only
    non-negative inputs are needed by double quantization (ratios of
    absolute maxima).
    """
    v = np.asarray(x, dtype=np.float64)
    if np.any(v < 0) or np.any(~np.isfinite(v)):
        raise ValueError("e4m3_encode_rne expects finite non-negative values")
    codes, vals = _e4m3_positive_table()
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    chunk = 1 << 16
    for i in range(0, flat.size, chunk):
        part = flat[i:i + chunk]
        d = np.abs(part[:, None] - vals[None, :])
        dmin = d.min(axis=1, keepdims=True)
        tie = d == dmin
        # among the nearest codes (at most two neighbours) prefer the even one
        pref = np.where(tie, (codes.astype(np.int64) & 1)[None, :], 2)
        out[i:i + chunk] = codes[np.argmin(pref, axis=1)]
    return out.reshape(v.shape)


# ----------------------------------------------------------------------------
# E2M1 and E8M0 (MXFP4)
# ----------------------------------------------------------------------------

def e2m1_decode(code):
    """E2M1 code (0..15) -> float64 value.

    sign = bit 3, exponent e = bits 2..1 (bias 1), mantissa m = bit 0.
    e = 0 is subnormal: 0.5 * m; otherwise 2^(e-1) * (1 + m/2).
    """
    c = np.asarray(code).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.exp2(e - 1.0) * (1.0 + m / 2.0))
    return np.where(s == 1, -mag, mag)


def e8m0_decode(code):
    """E8M0 code (uint8) -> float64 value 2^(E-127); code 255 is NaN."""
    E = np.asarray(code, dtype=np.uint8).astype(np.float64)
    return np.where(E == 255, np.nan, np.exp2(E - 127.0))
