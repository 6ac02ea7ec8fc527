"""Pins for the oracle's number formats against independent implementations.

torch's own dtype conversions (bfloat16, float8_e4m3fn, float8_e8m0fnu) are
separate code from the oracle's integer formulas, so agreement over every
code (and many random values) pins the oracle's codecs.
"""

import numpy as np
import pytest
import torch

from oracle import codecs


def test_bf16_decode_all_codes_matches_torch():
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_to_f32(u)
    ref = torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_roundtrip_all_codes():
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = codecs.bf16_to_f32(u)
    back = codecs.f32_to_bf16(f)
    finite = ~np.isnan(f)
    assert (back[finite] == u[finite]).all()
    assert np.isnan(codecs.bf16_to_f32(back[~finite])).all()


def _torch_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_random_and_edges():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # exact ties (low half == 0x8000) with both parities, overflow, subnormals
    hi = rng.integers(0, 1 << 16, size=5000, dtype=np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    edge = np.array([3.3895314e38, 3.4e38, -3.4e38, 1e-40, -1e-40, 0.0, -0.0, 1.0 + 2 ** -8,
                     1.0 + 3 * 2 ** -8, np.finfo(np.float32).max], dtype=np.float32)
    for arr in (f, ties, edge):
        assert (codecs.f32_to_bf16(arr) == _torch_bf16_bits(arr)).all()


def test_e4m3_decode_all_codes_matches_torch():
    c = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(c)
    ref = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()
    assert codecs.e4m3_decode(np.uint8(0x7E)) == 448.0
    assert codecs.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.random(20000) * 448.0,
        rng.random(20000),
        rng.random(5000) * 2 ** -6,
        # exact midpoints between neighbouring codes (ties -> even code)
        0.5 * (codecs.e4m3_decode(np.arange(0, 0x7E)) + codecs.e4m3_decode(np.arange(1, 0x7F))),
    ]).astype(np.float32)
    ours = codecs.e4m3_encode_rne(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all()


def test_e2m1_values_are_the_ocp_table():
    # The OCP MX v1.0 FP4 (E2M1) value set, listed by code 0..7; codes 8..15 are negatives.
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    v = codecs.e2m1_decode(np.arange(16))
    assert list(v[:8]) == table
    assert list(-v[8:]) == table
    assert np.signbit(v[8])  # code 8 is -0


def test_e8m0_decode_all_codes_matches_torch():
    c = np.arange(256, dtype=np.uint8)
    ours = codecs.e8m0_decode(c)
    ref = torch.from_numpy(c.copy()).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert (ours[:255] == ref[:255]).all()
    assert ours[127] == 1.0


def test_e4m3_encode_rejects_negative():
    with pytest.raises(ValueError):
        codecs.e4m3_encode_rne(np.array([-1.0]))
