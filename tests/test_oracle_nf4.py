"""Pins for the oracle's NF4 codebook, quantizer, double quantization and dequant.

Sources: "Training LLMs on a Budget: LoRA, QLoRA, and LoftQ", section 3 (NF4 as
16 normal quantiles with more bins near zero; one fp32 absmax per 64 weights;
double quantization with FP8 first-level and fp32 second-level scales over
256; the bits-per-weight figures and the 65B memory table).
"""

import json
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import codecs, nf4

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def test_codebook_invariants():
    q = nf4.codebook()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert (np.diff(q) > 0).all()                          # strictly increasing
    assert q[0] == -1.0 and q[7] == 0.0 and q[15] == 1.0   # absmax-normalised, exact zero
    assert (q < 0).sum() == 7 and (q > 0).sum() == 8
    # "more bins near zero": gaps grow away from zero on both sides
    gaps = np.diff(q.astype(np.float64))
    assert (np.diff(gaps[7:]) > 0).all()
    assert (np.diff(gaps[:7]) < 0).all()


def test_codebook_two_independent_inverse_cdfs_agree():
    a = nf4.codebook_float64()
    b = nf4.codebook_float64(inv_cdf=scipy.special.ndtri)
    assert (a.astype(np.float32) == b.astype(np.float32)).all()
    assert np.allclose(a, b, rtol=0, atol=1e-14)


def test_codebook_levels_are_normal_quantiles():
    # Undo the normalisation and map back through the normal CDF (scipy, a
    # third routine): the positive levels sit at the 8 probabilities
    # linspace(delta, 1/2, 9)[:-1], the negative ones mirror linspace(delta, 1/2, 8)[:-1].
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    q = nf4.codebook_float64()
    scale = scipy.stats.norm.ppf(delta)
    p_pos = scipy.stats.norm.cdf(q[8:] * scale)
    p_neg = scipy.stats.norm.cdf(-q[:7] * scale)
    assert np.allclose(np.sort(p_pos)[::-1], np.linspace(delta, 0.5, 9)[:-1], atol=1e-12)
    assert np.allclose(np.sort(p_neg)[::-1], np.linspace(delta, 0.5, 8)[:-1], atol=1e-12)


def test_codebook_spot_values():
    q = nf4.codebook()
    assert abs(q[8] - 0.0795803) < 1e-6
    assert abs(q[14] - 0.7229567) < 1e-6


def _brute_nearest(x):
    """Pure-Python nearest-level search, ties to the lower level (tiny inputs)."""
    q = [float(v) for v in nf4.codebook()]
    out = []
    for v in x:
        best, bd = 0, abs(v - q[0])
        for i in range(1, 16):
            d = abs(v - q[i])
            if d < bd:
                best, bd = i, d
        out.append(best)
    return out


def test_quantize_matches_brute_force_on_tiny_inputs():
    rng = np.random.default_rng(3)
    w = codecs.f32_to_bf16(rng.standard_normal((3, 128)).astype(np.float32) * 0.02)
    packed, scales = nf4.quantize(w)
    codes = nf4.unpack_nibbles(packed)
    wf = codecs.bf16_to_f32(w)
    for r in range(3):
        for b in range(2):
            blk = wf[r, b * 64:(b + 1) * 64]
            c = np.float32(max(abs(float(v)) for v in blk))
            assert scales[r, b] == c
            xs = [float(np.float32(v) / c) for v in blk]
            assert list(codes[r, b * 64:(b + 1) * 64]) == _brute_nearest(xs)


def test_nearest_level_ties_go_to_lower_level():
    q = nf4.codebook().astype(np.float64)
    mids = 0.5 * (q[:-1] + q[1:])             # exact in float64
    assert (nf4.nearest_level(mids) == np.arange(15)).all()
    eps = np.abs(np.spacing(mids)) * 4
    assert (nf4.nearest_level(mids + eps) == np.arange(1, 16)).all()


def test_packing_layout_and_roundtrip():
    codes = np.array([[1, 2, 3, 4, 15, 0, 7, 8]], dtype=np.uint8)
    packed = nf4.pack_nibbles(codes)
    assert list(packed[0]) == [0x21, 0x43, 0x0F, 0x87]   # element 2j low nibble
    assert (nf4.unpack_nibbles(packed) == codes).all()


def test_all_zero_block_and_signed_zero():
    w = np.zeros((2, 64), dtype=np.uint16)
    w[1, :] = 0x8000                                      # -0.0
    packed, scales = nf4.quantize(w)
    assert (scales == 0).all()
    assert (nf4.unpack_nibbles(packed) == 7).all()          # the zero level
    deq = nf4.dequantize(packed, scales)
    assert (codecs.bf16_to_f32(deq) == 0).all()


def test_dequant_every_code_times_scale_sweep():
    # all 16 codes x scales spanning many binades, against fp32 product + torch's bf16 rounding
    q = nf4.codebook()
    scales = np.float32(2.0) ** np.arange(-40, 41, dtype=np.float32)
    scales = np.concatenate([scales, scales * np.float32(1.37), np.float32([0.02, 0.0])]).astype(np.float32)
    codes = np.tile(np.arange(16, dtype=np.uint8), 4)[None, :].repeat(scales.size, 0)   # [S, 64]
    packed = nf4.pack_nibbles(codes)
    got = nf4.dequantize(packed, scales[:, None])
    prod = torch.from_numpy(q[codes]) * torch.from_numpy(scales[:, None])   # fp32 product
    ref = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (got == ref).all()


def test_quant_dequant_roundtrip_keeps_codes():
    # A block whose maximum is +-1 * c dequantizes to values that re-quantize to the same codes.
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(32, 256), dtype=np.uint8)
    codes[:, ::64] = 15                                     # each block holds the +1 level
    scales = (rng.random((32, 4)) * 0.1 + 0.01).astype(np.float32)
    scales = codecs.bf16_to_f32(codecs.f32_to_bf16(scales))  # absmax of bf16 data is a bf16 value
    w = nf4.dequantize(nf4.pack_nibbles(codes), scales)
    packed2, scales2 = nf4.quantize(w)
    assert (scales2 == scales).all()
    assert (nf4.unpack_nibbles(packed2) == codes).all()


def test_quantization_error_bound():
    # nearest level => |x - q[code]| <= half the local gap
    rng = np.random.default_rng(6)
    w = codecs.f32_to_bf16(rng.standard_normal((64, 512)).astype(np.float32) * 0.02)
    packed, scales = nf4.quantize(w)
    codes = nf4.unpack_nibbles(packed)
    q = nf4.codebook().astype(np.float64)
    x = codecs.bf16_to_f32(w).astype(np.float64) / np.repeat(scales, 64, axis=1)
    err = np.abs(x - q[codes])
    gaps = np.diff(q)
    lo = np.concatenate([[np.inf], gaps])[codes]
    hi = np.concatenate([gaps, [np.inf]])[codes]
    assert (err <= np.maximum(lo, hi) / 2 + 1e-7).all()
    assert (err <= np.where(x >= q[codes], hi, lo) / 2 + 1e-7).all()


def test_double_quant_matches_torch_e4m3_and_error_bound():
    rng = np.random.default_rng(7)
    scales = (np.abs(rng.standard_normal(1000)) * 0.05).astype(np.float32).reshape(10, 100)
    code8, c2 = nf4.double_quantize(scales)
    assert c2.shape == (4,)                                     # ceil(1000 / 256), last group short
    flat = scales.reshape(-1)
    for g in range(4):
        assert c2[g] == flat[g * 256:(g + 1) * 256].max()
    ratio = (flat / np.repeat(c2, 256)[:1000]).astype(np.float32)
    ref = torch.from_numpy(ratio).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (code8.reshape(-1) == ref).all()
    rebuilt = nf4.rebuild_scales(code8, c2).reshape(-1).astype(np.float64)
    bound = np.maximum(flat * 2.0 ** -4, np.repeat(c2, 256)[:1000] * 2.0 ** -10)
    assert (np.abs(rebuilt - flat) <= bound).all()


def test_double_quant_zero_group():
    code8, c2 = nf4.double_quantize(np.zeros(300, dtype=np.float32))
    assert (code8 == 0).all() and (c2 == 0).all()
    assert (nf4.rebuild_scales(code8, c2) == 0).all()


def _bits_per_weight(N, K, dq):
    w = np.zeros((N, K), dtype=np.uint16)
    packed, scales = nf4.quantize(w)
    nbytes = packed.nbytes
    if dq:
        code8, c2 = nf4.double_quantize(scales)
        nbytes += code8.nbytes + c2.nbytes
    else:
        nbytes += scales.nbytes
    return 8.0 * nbytes / (N * K)


def test_bits_per_weight_match_the_pages():
    N, K = 256, 4096                      # N*K/64 = 16384 scales = 64 full DQ groups
    nf4_bpw = _bits_per_weight(N, K, dq=False)
    dq_bpw = _bits_per_weight(N, K, dq=True)
    g = GOLD
    assert nf4_bpw == g["nf4_bits_per_weight"]["value"]
    assert nf4_bpw - 4 == g["nf4_bits_per_weight"]["scale_overhead_bits"]
    assert round(dq_bpw, 3) == g["nf4_dq_bits_per_weight"]["value"]
    assert round(dq_bpw - 4, 3) == g["nf4_dq_bits_per_weight"]["scale_overhead_bits"]
    assert round(nf4_bpw - dq_bpw, 3) == g["nf4_dq_bits_per_weight"]["saving_bits"]
    mem = g["memory_65b_gb"]
    assert round(mem["params"] * 16 / 8 / 1e9) == mem["fp16"]
    assert round(mem["params"] * nf4_bpw / 8 / 1e9, 1) == mem["nf4"]
    assert round(mem["params"] * dq_bpw / 8 / 1e9, 1) == mem["nf4_dq"]
    # "up to 75%": 4-bit codes alone are a quarter of bf16 storage
    assert 1 - 4 / 16 == g["base_memory_saving_4bit"]["value"]
    assert 1 - nf4_bpw / 16 < g["base_memory_saving_4bit"]["value"]


def test_quantize_rejects_ragged_k():
    with pytest.raises(ValueError):
        nf4.quantize(np.zeros((1, 96), dtype=np.uint16))
