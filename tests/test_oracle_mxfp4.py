"""Pins for the oracle's MXFP4 quantizer and dequant.

Sources: "Fine-Tuning 4-Bit Models", section "Case 2" (32-element blocks with
an E8M0 scale); Crusoe post, "Forward pass in training" (a base that was
already 4-bit dequantizes to bf16 in flight with no precision loss).
"""

import math

import numpy as np
import torch

from oracle import codecs, mxfp4, nf4

MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # OCP E2M1 magnitudes by code


def test_dequant_exhaustive_code_times_scale():
    # every code x every finite E8M0 scale, against exact float64 products rounded by torch
    E = np.arange(255, dtype=np.uint8)
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)[None, :].repeat(255, 0)   # [255, 32]
    got = mxfp4.dequantize(nf4.pack_nibbles(codes), E[:, None])
    vals = np.array([[(-1.0 if c >= 8 else 1.0) * MAGS[c & 7] * 2.0 ** (int(e) - 127) for c in row]
                     for e, row in zip(E, codes)])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (got == ref).all()
    # lossless wherever the product is finite: decoding gives back the exact value
    back = codecs.bf16_to_f32(got).astype(np.float64)
    fin = np.isfinite(back)
    assert (back[fin] == vals[fin]).all()
    assert fin[:253].all()                       # every scale up to 2^125 is exact for all codes


def test_nan_scale_gives_nan():
    codes = np.full((1, 32), 0x22, dtype=np.uint8)[:, :16]
    got = mxfp4.dequantize(codes, np.array([[255]], dtype=np.uint8))
    assert np.isnan(codecs.bf16_to_f32(got)).all()


def test_shared_exponent_closed_form():
    rng = np.random.default_rng(11)
    w = codecs.f32_to_bf16((rng.standard_normal((16, 256)) * 0.015).astype(np.float32))
    e = mxfp4.shared_exponents(w)
    wf = codecs.bf16_to_f32(w).astype(np.float64)
    for r in range(16):
        for b in range(8):
            amax = max(abs(v) for v in wf[r, b * 32:(b + 1) * 32])
            X = math.floor(math.log2(amax)) - 2
            assert int(e[r, b]) == X + 127
            assert 4.0 <= amax * 2.0 ** -X < 8.0


def _brute_e2m1(v):
    """Pure-Python nearest E2M1 magnitude, ties to the even code, sign kept."""
    a = abs(v)
    best, bd = 0, abs(a - MAGS[0])
    for i in range(1, 8):
        d = abs(a - MAGS[i])
        if d < bd or (d == bd and i % 2 == 0 and best % 2 == 1):
            best, bd = i, d
    return best | (8 if math.copysign(1.0, v) < 0 else 0)


def test_quantize_matches_brute_force_on_tiny_inputs():
    rng = np.random.default_rng(12)
    w = codecs.f32_to_bf16((rng.standard_normal((4, 64)) * 0.015).astype(np.float32))
    packed, e = mxfp4.quantize(w)
    codes = nf4.unpack_nibbles(packed)
    wf = codecs.bf16_to_f32(w).astype(np.float64)
    for r in range(4):
        for b in range(2):
            X = int(e[r, b]) - 127
            for j in range(32):
                k = b * 32 + j
                assert codes[r, k] == _brute_e2m1(wf[r, k] * 2.0 ** -X)


def test_ties_go_to_even_code_and_saturate():
    # one block with amax = 4 (X = 0, scale 1): entries at every midpoint and above 6
    vals = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -5.0, 7.5, -7.0, 0.0, -0.0]
    vals += [0.0] * (32 - len(vals))
    # amax must stay 4 for X = 0 while 7.5 is present -> use a separate block for saturation
    blk1 = np.array(vals[:11] + [0.0] * 21, dtype=np.float32)
    blk2 = np.array([7.5, -7.0, 6.0, -0.0] + [0.0] * 28, dtype=np.float32)
    w = codecs.f32_to_bf16(np.concatenate([blk1, blk2])[None, :])
    packed, e = mxfp4.quantize(w)
    codes = nf4.unpack_nibbles(packed)[0]
    assert int(e[0, 0]) == 127 and int(e[0, 1]) == 127
    assert list(codes[:11]) == [6, 0, 2, 2, 4, 4, 6, 6, 8, 10, 14]
    assert list(codes[32:36]) == [7, 15, 7, 8]     # 7.5 and -7 saturate to +-6; -0 keeps its sign


def test_zero_block_and_subnormal_block():
    w = np.zeros((1, 64), dtype=np.uint16)
    w[0, 32:] = 0x0001                               # smallest bf16 subnormal, 2^-133
    packed, e = mxfp4.quantize(w)
    assert int(e[0, 0]) == 0                         # all-zero block
    assert int(e[0, 1]) == 0                         # X clamps to -127
    codes = nf4.unpack_nibbles(packed)[0]
    assert (codes[:32] == 0).all()
    # 2^-133 * 2^127 = 2^-6 rounds to 0
    assert (codes[32:] == 0).all()


def test_native_4bit_base_roundtrips_exactly():
    # A weight that already lies on the MXFP4 grid (a 4-bit-native release) quantizes
    # and dequantizes with no loss at all.
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 16, size=(8, 128), dtype=np.uint8)
    codes[:, ::32] = 7                                   # each block reaches magnitude 6
    E = rng.integers(100, 130, size=(8, 4)).astype(np.uint8)
    w = mxfp4.dequantize(nf4.pack_nibbles(codes), E)
    packed2, E2 = mxfp4.quantize(w)
    assert (E2 == E).all()
    c2 = nf4.unpack_nibbles(packed2)
    # -0 and +0 are the same value; compare values, then codes off zero
    assert (mxfp4.dequantize(packed2, E2) == w).all()
    nz = (codes & 7) != 0
    assert (c2[nz] == codes[nz]).all()


def test_bits_per_weight():
    N, K = 64, 1024
    packed, e = mxfp4.quantize(np.zeros((N, K), dtype=np.uint16))
    assert 8.0 * (packed.nbytes + e.nbytes) / (N * K) == 4.25
