"""Pins of the MXFP8 activation quantizer and the MX-native forward (CPU).

The E4M3 element codes are checked against torch's own float8_e4m3fn
conversion (an independent implementation; it rounds to nearest even and
returns NaN past the 448/480 midpoint, so it is compared where |v| <= 464 and
saturation is checked on its own). The shared exponent is checked by its
defining property, by round trips of blocks already on the MXFP8 grid and by
the all-zero and tiny-block special cases. The forward reduces to the pinned
plain forward when X is on the grid, and otherwise stays within the error
bound that the E4M3 rounding allows."""

import numpy as np
import pytest
import torch

from oracle import codecs, lora, mxfp4, mxfp8
from synth import to_bf16


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _blocks(rng, m, k, spread=30):
    """bf16 rows whose 32-element blocks span very different magnitudes."""
    x = rng.standard_normal((m, k)).astype(np.float32)
    blk = np.exp2(rng.integers(-spread, spread, (m, k // 32))).astype(np.float32)
    x *= np.repeat(blk, 32, axis=1)
    x *= np.exp2(rng.integers(-12, 1, (m, k))).astype(np.float32)   # small elements inside each block
    return to_bf16(x)


def test_elements_match_torch_e4m3():
    rng = np.random.default_rng(11)
    x = _blocks(rng, 64, 512)
    codes, e = mxfp8.quantize(x)
    xf = codecs.bf16_to_f32(x).astype(np.float64)
    v = np.ldexp(xf, -(np.repeat(e.astype(np.int64), 32, axis=1) - 127))
    ok = np.abs(v) <= 464
    ref = _torch_e4m3(v.astype(np.float32))          # v is exact in float32 (power-of-two scaling)
    assert ok.mean() > 0.99
    assert np.array_equal(codes[ok], ref[ok])


def test_saturation_past_448():
    # blocks whose largest element lands in (448, 512) after scaling
    mags = np.array([450.0, 462.0, 464.0, 466.0, 478.0, 480.0, 500.0, 510.0])   # exact in bf16
    for k, m in enumerate(mags):
        for Xe in (-20, 0, 7):
            x = np.zeros((1, 32), np.float32)
            x[0, 0] = m * 2.0 ** Xe
            x[0, 1] = -m * 2.0 ** Xe
            xb = to_bf16(x)
            codes, e = mxfp8.quantize(xb)
            mag = codecs.bf16_to_f32(xb)[0, 0] / 2.0 ** Xe     # after bf16 rounding of the input
            assert int(e[0, 0]) - 127 == Xe
            if mag >= 464:
                assert codes[0, 0] == 0x7E and codes[0, 1] == 0xFE, (m, Xe)
            else:
                assert codes[0, 0] == _torch_e4m3([mag])[0]


def test_scale_property_and_special_blocks():
    rng = np.random.default_rng(12)
    x = _blocks(rng, 32, 256)
    x[0, :32] = 0                                  # all-zero block
    x[1, :32] = 0x8000                             # all -0
    x[2, :32] = rng.integers(1, 0x80, 32)          # bf16 subnormals only (amax < 2^-126)
    codes, e = mxfp8.quantize(x)
    xf = codecs.bf16_to_f32(x).astype(np.float64)
    amax = np.abs(xf.reshape(32, -1, 32)).max(axis=2)
    Xe = e.astype(np.int64) - 127
    nz = (amax > 0) & (Xe > -127)
    r = amax[nz] * np.exp2(-Xe[nz])
    assert ((r >= 256) & (r < 512)).all()          # largest element lands in [2^8, 2^9)
    assert e[0, 0] == 0 and (codes[0, :32] == 0).all()
    assert e[1, 0] == 0 and (codes[1, :32] == 0x80).all()
    assert e[2, 0] == 0                            # clamped to 2^-127
    v = xf[2, :32] * 2.0 ** 127
    assert np.array_equal(codes[2, :32], _torch_e4m3(v))


def test_round_trip_on_grid():
    """Blocks already on the MXFP8 grid come back with the same codes and scales."""
    rng = np.random.default_rng(13)
    M, K = 16, 256
    e = rng.integers(100, 150, (M, K // 32)).astype(np.uint8)
    codes = rng.integers(0, 0x7F, (M, K)).astype(np.uint8)          # finite non-negative codes
    codes[:, ::32] = rng.integers(0x78, 0x7F, (M, K // 32))         # block max in [256, 448]
    codes |= (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    vals = mxfp8.dequantize(codes, e)
    xb = codecs.f32_to_bf16(vals.astype(np.float32))
    assert np.array_equal(codecs.bf16_to_f32(xb).astype(np.float64), vals)   # exact in bf16
    c2, e2 = mxfp8.quantize(xb)
    assert np.array_equal(e2, e)
    # -0 and +0 both decode to 0; compare values, then the codes away from zero
    assert np.array_equal(mxfp8.dequantize(c2, e2), vals)
    nz = (codes & 0x7F) != 0
    assert np.array_equal(c2[nz], codes[nz])


def _mx_layer(rng, M, K, N, r):
    X = to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    W = to_bf16(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.015))
    A = to_bf16(rng.uniform(-1, 1, (r, K)).astype(np.float32) / np.float32(np.sqrt(K)))
    B = to_bf16(rng.standard_normal((N, r)).astype(np.float32) * np.float32(0.01))
    wc, ws = mxfp4.quantize(W)
    return X, wc, ws, A, B


def test_forward_on_grid_is_the_plain_forward():
    rng = np.random.default_rng(14)
    M, K, N, r = 24, 128, 40, 8
    _, wc, ws, A, B = _mx_layer(rng, M, K, N, r)
    codes = rng.integers(0, 0x7F, (M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    codes[:, ::32] = 0x7C
    e = rng.integers(115, 125, (M, K // 32)).astype(np.uint8)
    X = codecs.f32_to_bf16(mxfp8.dequantize(codes, e).astype(np.float32))
    out = mxfp8.forward(X, wc, ws, A, B, 2.0)
    Wd = lora.as_f64(mxfp4.dequantize(wc, ws))
    ref = lora.forward(lora.as_f64(X), Wd, lora.as_f64(A), lora.as_f64(B), 2.0)
    assert np.array_equal(out["Y"], ref["Y"])
    assert np.array_equal(out["Z"], ref["Z"])


def test_forward_error_bound():
    """|Y_mx - Y| <= sum_k |x_k - q(x_k)| |w_k| elementwise, with E4M3's
    rounding error at most 2^-4 |x| (normal) or 2^-10 * 2^Xe (subnormal), or
    |x| - 448 * 2^Xe where the block maximum saturates (it lands in [256, 512)
    after scaling, so values past 448 are clamped)."""
    rng = np.random.default_rng(15)
    M, K, N, r = 32, 256, 48, 4
    X, wc, ws, A, B = _mx_layer(rng, M, K, N, r)
    out = mxfp8.forward(X, wc, ws, A, B, 1.5)
    Wd = lora.as_f64(mxfp4.dequantize(wc, ws))
    ref = lora.forward(lora.as_f64(X), Wd, lora.as_f64(A), lora.as_f64(B), 1.5)
    Xf = lora.as_f64(X)
    Xe = np.repeat(out["X_scales"].astype(np.int64) - 127, 32, axis=1)
    err = np.maximum(np.abs(Xf) * 2.0 ** -4, 2.0 ** (Xe - 10))
    err = np.maximum(err, np.abs(Xf) - 448.0 * 2.0 ** Xe)
    Xq = mxfp8.dequantize(out["X_codes"], out["X_scales"])
    assert (np.abs(Xq - Xf) <= err).all()
    bound = err @ np.abs(Wd).T
    assert (np.abs(out["Y"] - ref["Y"]) <= bound * (1 + 1e-12)).all()
    # the quantization is not a no-op: a typical relative error of a few 1e-2
    rel = lora.rel_frobenius(out["Y_base"], Xf @ Wd.T)
    assert 1e-3 < rel < 5e-2


@pytest.mark.parametrize("bad", [31, 33])
def test_block_multiple_required(bad):
    with pytest.raises(ValueError):
        mxfp8.quantize(np.zeros((2, bad), np.uint16))
