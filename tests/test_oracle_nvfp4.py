"""Pins of the NVFP4 oracle (CPU).

* the block scale against torch's float8_e4m3fn conversion of amax / 6
  (an independent E4M3 rounding);
* every element against a brute-force nearest search written here, with the
  tie rule checked on exact midpoints;
* round trips of blocks already on the NVFP4 grid;
* dequant exactness (float64 products);
* the page's claim that the 16-element FP8-scaled format loses less than
  MXFP4's 32-element E8M0 scaling on a transformer-like (Gaussian) weight
  distribution.
"""

import itertools

import numpy as np
import torch

from oracle import codecs, mxfp4, nvfp4
from oracle.nf4 import unpack_nibbles
from synth import to_bf16

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _w(rng, n, k, spread=8):
    x = rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02)
    x *= np.repeat(np.exp2(rng.integers(-spread, spread, (n, k // 16))).astype(np.float32), 16, axis=1)
    return to_bf16(x)


def test_scale_is_e4m3_of_amax_over_6():
    rng = np.random.default_rng(21)
    w = _w(rng, 64, 256, spread=20)
    w[0, :16] = 0
    sc = nvfp4.block_scales(w)
    amax = np.abs(codecs.bf16_to_f32(w).astype(np.float64).reshape(64, -1, 16)).max(axis=2)
    q = amax / 6.0
    ok = q <= 448
    ref = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # amax / 6 is exact or not a tie in float32 (see the GPU packer), so rounding it first is harmless
    assert np.array_equal(sc[ok], ref[ok])
    assert sc[0, 0] == 0


def test_elements_brute_force():
    rng = np.random.default_rng(22)
    w = _w(rng, 16, 128)
    packed, sc = nvfp4.quantize(w)
    codes = unpack_nibbles(packed)
    wf = codecs.bf16_to_f32(w).astype(np.float64)
    s = np.repeat(codecs.e4m3_decode(sc), 16, axis=1)
    for i, j in itertools.product(range(16), range(128)):
        if s[i, j] == 0:
            assert codes[i, j] & 7 == 0
            continue
        a = abs(wf[i, j]) / s[i, j]
        dist = [abs(a - m) for m in E2M1]
        best = min(dist)
        cands = [c for c in range(8) if dist[c] == best]
        want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        assert codes[i, j] & 7 == want, (i, j, a)
        assert (codes[i, j] >> 3) == (1 if np.signbit(wf[i, j]) else 0)


def test_ties_go_to_the_even_code():
    # block max 6 * s with s = 1: midpoints 0.25, 0.75, ..., 5 land exactly
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 2, 2, 4, 4, 6, 6]
    row = np.array([6.0] + mids + [-m for m in mids] + [0.0], np.float32)
    w = to_bf16(row[None, :])
    packed, sc = nvfp4.quantize(w)
    assert codecs.e4m3_decode(sc)[0, 0] == 1.0
    c = unpack_nibbles(packed)[0]
    assert list(c[1:8]) == want
    assert list(c[8:15]) == [x | 8 for x in want]


def test_round_trip_on_grid():
    rng = np.random.default_rng(23)
    N, K = 8, 128
    sc = rng.integers(0x08, 0x7E, (N, K // 16)).astype(np.uint8)   # normal E4M3 scales
    mag = rng.integers(0, 8, (N, K)).astype(np.uint8)
    mag[:, ::16] = 7                                                # block max = 6 s
    codes = mag | (rng.integers(0, 2, (N, K)) << 3).astype(np.uint8)
    packed = np.zeros((N, K // 2), np.uint8)
    packed[:] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    w = nvfp4.dequantize(packed, sc)
    p2, s2 = nvfp4.quantize(w)
    assert np.array_equal(s2, sc)
    nz = (codes & 7) != 0
    assert np.array_equal(unpack_nibbles(p2)[nz], codes[nz])
    assert np.array_equal(nvfp4.dequantize(p2, s2), w)


def test_dequant_exact():
    rng = np.random.default_rng(24)
    packed = rng.integers(0, 256, (4, 64)).astype(np.uint8)
    sc = rng.integers(0, 0x7F, (4, 8)).astype(np.uint8)
    got = codecs.bf16_to_f32(nvfp4.dequantize(packed, sc)).astype(np.float64)
    want = codecs.e2m1_decode(unpack_nibbles(packed)) * np.repeat(codecs.e4m3_decode(sc), 16, axis=1)
    assert np.array_equal(got, want)


def test_finer_than_mxfp4_on_gaussian_weights():
    rng = np.random.default_rng(25)
    w = to_bf16(rng.standard_normal((256, 1024)).astype(np.float32) * np.float32(0.02))
    wf = codecs.bf16_to_f32(w).astype(np.float64)

    def err(deq):
        return np.linalg.norm(codecs.bf16_to_f32(deq).astype(np.float64) - wf) / np.linalg.norm(wf)

    e_nv = err(nvfp4.dequantize(*nvfp4.quantize(w)))
    e_mx = err(mxfp4.dequantize(*mxfp4.quantize(w)))
    assert e_nv < e_mx, (e_nv, e_mx)


def test_saturation_of_scale_and_elements():
    """Blocks whose amax / 6 exceeds 448: the scale saturates at 448 and every
    element past 6 * 448 takes the largest magnitude, sign kept."""
    row = np.array([3e38, -3e38, 1e30, -5000.0, 2688.0, 2689.0, 100.0, -1.0] * 2, np.float32)
    w = to_bf16(row[None, :])
    packed, sc = nvfp4.quantize(w)
    assert sc[0, 0] == 0x7E
    c = unpack_nibbles(packed)[0]
    wf = codecs.bf16_to_f32(w)[0].astype(np.float64)
    for j in range(16):
        a = min(abs(wf[j]) / 448.0, 6.0)
        want = min(range(8), key=lambda m: (abs(a - E2M1[m]), m % 2))
        assert c[j] & 7 == want, (j, wf[j])
        assert c[j] >> 3 == (1 if wf[j] < 0 else 0)
    assert c[0] == 7 and c[1] == 15 and c[2] == 7 and c[3] == 15
