"""NVFP4: E2M1 element codes with one E4M3 (FP8) scale per 16 consecutive
elements.

Test infrastructure only (see the package docstring).

Source: "Fine-Tuning 4-Bit Models: Adapting a Base That Only Ships
Quantized", section "Case 2: An NVFP4 deployment checkpoint is what you were
handed" (NVIDIA's 4-bit float format: an FP8 scale per 16-element
micro-block, finer than MXFP4's 32-element E8M0 scaling) and the summary list
(16-element micro-blocks with an FP8 scale).

Readings where the page is silent:
* there is no per-tensor scale (the page names none);
* the block scale is ``amax / 6`` (6 is the largest E2M1 magnitude) rounded
  to E4M3 (nearest, ties to the even code, saturating at 448); an all-zero
  block gets scale 0;
* each element's code is the E2M1 value nearest to ``w / s``, with s the
  decoded E4M3 scale (ties to the even code, saturating at 6, sign copied
  from w); where s == 0 every element takes magnitude 0, sign copied;
* byte j of a row holds element 2j in its low nibble, 2j+1 in its high
  nibble (as MXFP4);
* dequant ``bf16(e2m1(code) * e4m3(scale))``: exact (at most 6 significant
  bits, inside bf16's range).
"""

import numpy as np

from .codecs import bf16_to_f32, e2m1_decode, e4m3_decode, e4m3_encode_rne, f32_to_bf16
from .nf4 import pack_nibbles, unpack_nibbles

BLOCK = 16
_MAGS = e2m1_decode(np.arange(8))  # 0, .5, 1, 1.5, 2, 3, 4, 6


def block_scales(w_bf16, block=BLOCK):
    """E4M3 code of amax / 6 per block of ``block`` consecutive elements of each row."""
    w = bf16_to_f32(w_bf16).astype(np.float64)
    n, k = w.shape
    if k % block:
        raise ValueError("K must be a multiple of the block size")
    amax = np.abs(w.reshape(n, k // block, block)).max(axis=2)
    return e4m3_encode_rne(np.minimum(amax / 6.0, 448.0))


def encode_codes(w_bf16, sc_e4m3, block=BLOCK):
    """Unpacked E2M1 codes [N, K] for given E4M3 block scales."""
    w = bf16_to_f32(w_bf16).astype(np.float64)
    s = np.repeat(e4m3_decode(sc_e4m3), block, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        a = np.where(s > 0, np.abs(w) / np.where(s > 0, s, 1.0), 0.0)
    # saturate first: where the scale itself saturated (amax / 6 > 448), w / s
    # can be so large that the distances to the 8 magnitudes no longer differ
    a = np.minimum(a, 6.0)
    d = np.abs(a[..., None] - _MAGS)
    dmin = d.min(axis=-1, keepdims=True)
    codes = np.arange(8)
    pref = np.where(d == dmin, codes & 1, 2)     # nearest; on a tie the even code
    mag_code = np.argmin(pref, axis=-1).astype(np.uint8)
    sign = np.signbit(w).astype(np.uint8) << 3
    return (mag_code | sign).astype(np.uint8)


def quantize(w_bf16, block=BLOCK):
    """bf16 W [N, K] -> (packed codes [N, K/2] uint8, E4M3 scales [N, K/16] uint8)."""
    w_bf16 = np.asarray(w_bf16, dtype=np.uint16)
    sc = block_scales(w_bf16, block)
    return pack_nibbles(encode_codes(w_bf16, sc, block)), sc


def dequantize(packed, sc_e4m3, block=BLOCK):
    """Packed codes + E4M3 scales -> bf16 bit patterns of e2m1(code) * e4m3(scale)."""
    codes = unpack_nibbles(packed)
    val = e2m1_decode(codes) * np.repeat(e4m3_decode(sc_e4m3), block, axis=1)
    return f32_to_bf16(val.astype(np.float32))     # exact: the products fit in bf16
