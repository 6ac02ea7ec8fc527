"""NF4 with blockwise absmax scales and optional double quantization.

Test infrastructure only (see the package docstring).

Source: "Training LLMs on a Budget: LoRA, QLoRA, and LoftQ", section 3
("The three QLoRA tricks"):
* trick 1: NF4 is 16 quantile points of a standard normal (inverse CDF),
  normalised by absmax and applied block-wise, with more bins near zero;
* trick 2: one fp32 absmax scale per block of 64 weights (0.5 bits/weight);
  double quantization stores those scales as 8-bit FP8 with a second-level
  fp32 absmax over each group of 256 first-level scales (about 0.127
  bits/weight);
* "The setup": the stored base is dequantized block by block to bf16 for the
  matmul and the dequantized tensor is never kept.

Readings where the page is silent:
* codebook: 8 positive levels at the normal quantiles of
  ``linspace(delta, 1/2, 9)`` (last point dropped), 7 negative levels at the
  negated quantiles of ``linspace(delta, 1/2, 8)`` (last point dropped), an
  exact zero, divided by the largest level; ``delta`` is the mean of
  ``1 - 1/30`` and ``1 - 1/32``. Levels are rounded to fp32.
* encoding: ``x = fp32(w / c)`` (correctly rounded), code = the nearest level,
  ties to the lower level; an all-zero block (c = 0) encodes every element as
  the zero level.
* blocks are 64 consecutive elements along K within a row; byte j of a row
  holds element 2j in its low nibble and element 2j+1 in its high nibble.
* double quantization: flatten the fp32 scales of one matrix in row-major
  order, cut them into consecutive groups of 256 (the last group may be
  shorter), ``c2 = max`` of the group, ``code8 = E4M3(c / c2)`` (nearest, ties
  to even), rebuilt scale ``c' = fp32(E4M3(code8) * c2)``. Codes are chosen
  with the exact scale first; double quantization replaces the scales after.
* dequant: ``bf16(fp32(q[code] * c))``: one fp32 product, one bf16 rounding.
"""

import statistics

import numpy as np

from .codecs import bf16_to_f32, e4m3_decode, e4m3_encode_rne, f32_to_bf16

BLOCK = 64
DQ_GROUP = 256


def codebook_float64(inv_cdf=None):
    """The 16 NF4 levels in float64, before rounding to fp32 (ascending)."""
    if inv_cdf is None:
        inv_cdf = statistics.NormalDist().inv_cdf
    delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
    pos = [inv_cdf(p) for p in np.linspace(delta, 0.5, 9)[:-1]]
    neg = [-inv_cdf(p) for p in np.linspace(delta, 0.5, 8)[:-1]]
    levels = np.array(sorted(pos + [0.0] + neg), dtype=np.float64)
    return levels / levels.max()


def codebook():
    """The 16 NF4 levels as float32, ascending: q[0] = -1, q[7] = 0, q[15] = 1."""
    return codebook_float64().astype(np.float32)


def absmax_scales(w_bf16, block=BLOCK):
    """fp32 absmax of each block of ``block`` consecutive elements of each row."""
    w = bf16_to_f32(w_bf16)
    n, k = w.shape
    if k % block:
        raise ValueError("K must be a multiple of the block size")
    return np.abs(w.reshape(n, k // block, block)).max(axis=2).astype(np.float32)


def encode_codes(w_bf16, scales, block=BLOCK):
    """Unpacked NF4 codes (uint8 0..15, shape [N, K]) for given per-block scales.

    Each element is normalised as ``x = fp32(w / c)`` and mapped to the
    nearest codebook level; on a tie the lower level wins (``argmin`` keeps the
    first minimum).
    """
    w = bf16_to_f32(w_bf16)
    c = np.repeat(np.asarray(scales, dtype=np.float32), block, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        x = np.where(c == 0, np.float32(0.0), w / c).astype(np.float32)
    return nearest_level(x)


def nearest_level(x):
    """Index of the codebook level nearest to each x (float64 distances).

    On an exact tie the lower level wins (``argmin`` keeps the first minimum).
    """
    x = np.asarray(x, dtype=np.float64)
    q = codebook().astype(np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 20
    for i in range(0, flat.size, step):
        d = np.abs(flat[i:i + step, None] - q[None, :])
        out[i:i + step] = np.argmin(d, axis=1).astype(np.uint8)
    return out.reshape(x.shape)


def pack_nibbles(codes):
    """[N, K] codes 0..15 -> [N, K/2] bytes; element 2j low nibble, 2j+1 high."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """Inverse of :func:`pack_nibbles`."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def quantize(w_bf16, block=BLOCK):
    """bf16 W [N, K] -> (packed codes [N, K/2] uint8, fp32 scales [N, K/block])."""
    w_bf16 = np.asarray(w_bf16, dtype=np.uint16)
    scales = absmax_scales(w_bf16, block)
    return pack_nibbles(encode_codes(w_bf16, scales, block)), scales


def double_quantize(scales):
    """fp32 scales (any shape) -> (E4M3 codes, same shape; fp32 second level).

    The scales are flattened row-major and cut into groups of 256; the last
    group may be shorter. A group whose maximum is 0 encodes every scale as
    code 0.
    """
    s = np.asarray(scales, dtype=np.float32)
    flat = s.reshape(-1)
    ng = -(-flat.size // DQ_GROUP)
    c2 = np.empty(ng, dtype=np.float32)
    ratio = np.empty(flat.size, dtype=np.float32)
    for g in range(ng):
        part = flat[g * DQ_GROUP:(g + 1) * DQ_GROUP]
        m = part.max() if part.size else np.float32(0)
        c2[g] = m
        if m == 0:
            ratio[g * DQ_GROUP:(g + 1) * DQ_GROUP] = 0
        else:
            ratio[g * DQ_GROUP:(g + 1) * DQ_GROUP] = (part / m).astype(np.float32)
    code8 = e4m3_encode_rne(ratio.astype(np.float64))
    return code8.reshape(s.shape), c2


def rebuild_scales(code8, scales2):
    """Double-quantized scales -> fp32 ``c' = fp32(E4M3(code8) * c2)``."""
    c8 = np.asarray(code8, dtype=np.uint8)
    flat = c8.reshape(-1)
    c2 = np.repeat(np.asarray(scales2, dtype=np.float32), DQ_GROUP)[:flat.size]
    prod = (e4m3_decode(flat).astype(np.float32) * c2).astype(np.float32)
    return prod.reshape(c8.shape)


def dequantize(packed, scales, block=BLOCK):
    """Packed codes + fp32 scales -> bf16 bit patterns of ``bf16(fp32(q[code]*c))``."""
    codes = unpack_nibbles(packed)
    q = codebook()
    c = np.repeat(np.asarray(scales, dtype=np.float32), block, axis=1)
    prod = (q[codes] * c).astype(np.float32)
    return f32_to_bf16(prod)


def dequantize_dq(packed, code8, scales2, block=BLOCK):
    """Dequant of a double-quantized NF4 matrix."""
    return dequantize(packed, rebuild_scales(code8, scales2), block)
