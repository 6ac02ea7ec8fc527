"""GPU parity of the MX-native forward of an MXFP4 base (the Crusoe post,
"Forward pass in inference": the base product runs natively on MXFP4 while the
adapters stay in bf16; activations as MXFP8, the reading the oracle's mxfp8
module states).

* the MXFP8 activation packer, bit for bit against the oracle (codes and
  scales), over rows that exercise every rounding path;
* the base product with one-hot activations (X = I on 256 columns): each output
  is one dequantized W element, so Y must equal deq(W)^T bit for bit -- this
  pins the operand lane layouts, the nibble order and both block scales;
* Y and Z against the oracle within the relative Frobenius bar on ragged
  shapes (M, N off the tiles, K % 64 == 32, several ranks), few-tile outputs
  (split reduction) and long reductions (rank-r range partials in the GEMM);
* every layer of the 70B set at full size, every element.
"""

import numpy as np
import pytest
import torch

import lora_fine_tuning_amd as L
import synth
from oracle import codecs, lora, mxfp4, mxfp8
from gpu_util import (DEV, TOL, compare_full, f64, guarded, oracle_pack_full, pack_gpu, print_case, rel,
                      to_dev, to_host, write_report)

pytestmark = pytest.mark.gpu


def _wide_rows(rng, M, K):
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= np.repeat(np.exp2(rng.integers(-40, 40, (M, K // 32))).astype(np.float32), 32, axis=1)
    x *= np.exp2(rng.integers(-12, 1, (M, K))).astype(np.float32)
    u = synth.to_bf16(x)
    u[0, :32] = 0                                       # all-zero block
    u[0, 32:64] = 0x8000                                # all -0
    if M > 1:
        u[1, :32] = rng.integers(1, 0x80, 32)           # bf16 subnormals (exponent clamped to -127)
    if M > 2 and K >= 64:
        # largest element in (448, 512) after scaling: saturation; and ties
        blk = np.float32(2.0 ** 5) * np.array([500, 466, 464, 462, 450, 17, 19, 18] * 4, np.float32)
        u[2, :32] = synth.to_bf16(blk)
        u[2, 32:64] = synth.to_bf16(np.float32(2.0 ** -30) * np.array([448, 9, 11, 13, 15, 0.5, 1.5, 2.5] * 4,
                                                                       np.float32))
    return u


@pytest.mark.parametrize("M,K", [(1, 32), (37, 96), (256, 1024), (130, 4096)])
def test_mxfp8_packer_bit_exact(M, K):
    print_case("mxfp8 pack", M, K)
    rng = np.random.default_rng(M * 7 + K)
    u = _wide_rows(rng, M, K)
    codes, scales = L.mxfp8(to_dev(u))
    torch.cuda.synchronize()
    ref_c, ref_s = mxfp8.quantize(u)
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def _layer(M, K, N, r, seed, wscale=0.015):
    rng = np.random.default_rng(seed)
    X = synth.to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    W = synth.to_bf16(rng.standard_normal((N, K)).astype(np.float32) * np.float32(wscale))
    A = synth.to_bf16(rng.uniform(-1, 1, (r, K)).astype(np.float32) / np.float32(np.sqrt(K)))
    B = synth.to_bf16(rng.standard_normal((N, r)).astype(np.float32) * np.float32(0.01))
    return X, W, A, B


def test_one_hot_gives_the_dequantized_base():
    """X = I (256 x 256, one 1.0 per row: an exact MXFP8 value) and B = 0:
    Y[i, n] = deq(W)[n, i] exactly, for a base whose block scales span a wide
    range (every row block of W gets its own magnitude)."""
    K, N, r = 256, 320, 16
    rng = np.random.default_rng(61)
    w = rng.standard_normal((N, K)).astype(np.float32)
    w *= np.repeat(np.exp2(rng.integers(-30, 30, (N, K // 32))).astype(np.float32), 32, axis=1)
    W = synth.to_bf16(w)
    X = synth.to_bf16(np.eye(K, dtype=np.float32))
    A = synth.to_bf16(rng.standard_normal((r, K)).astype(np.float32))
    B = np.zeros((N, r), np.uint16)
    print_case("mx one-hot", K, N)
    base = pack_gpu(W, synth.MXFP4)
    out = L.forward_mx(base, to_dev(X), to_dev(A), to_dev(B), 1.0)
    torch.cuda.synchronize()
    Y = to_host(out["Y"])
    wc, ws = mxfp4.quantize(W)
    ref = mxfp4.dequantize(wc, ws).T                   # bf16 bits [K, N]
    # the base product has one non-zero term per output; signed zeros may differ
    same = (Y == ref) | (((Y | ref) & 0x7FFF) == 0)
    assert same.all(), np.argwhere(~same)[:8]


CASES = [
    # M, K, N, r
    (256, 256, 256, 16),       # one tile
    (300, 1056, 380, 24),      # ragged rows and columns, K % 64 == 32
    (513, 2048, 1024, 1),      # rank 1
    (128, 4096, 512, 64),      # few tiles: split reduction
    (1024, 8192, 768, 16),     # long reduction: rank-r range partials summed in the GEMM
    (64, 96, 40, 128),         # tiny, r = 128
    (300, 512, 384, 256),      # the largest rank accepted: two 128-wide rank blocks in the Z pass
    (200, 1024, 264, 136),     # rank above 128, not a multiple of 64
]


@pytest.mark.parametrize("M,K,N,r", CASES)
def test_mx_forward_matches_oracle(M, K, N, r):
    print_case("mx forward", M, K, N, r)
    X, W, A, B = _layer(M, K, N, r, seed=M + K + N + r)
    s = 32.0 / r
    base = pack_gpu(W, synth.MXFP4)
    out = L.forward_mx(base, to_dev(X), to_dev(A), to_dev(B), s)
    torch.cuda.synchronize()
    wc, ws = mxfp4.quantize(W)
    ref = mxfp8.forward(X, wc, ws, A, B, s)
    Y, Z = to_host(out["Y"]), to_host(out["Z"])
    assert rel(Y, ref["Y"]) <= TOL
    assert rel(Z, ref["Z"]) <= TOL
    # the MX product differs from the bf16-activation product by the MXFP8
    # rounding of X (a few 1e-2): the comparison above is not the bf16 forward's
    Wd = lora.as_f64(mxfp4.dequantize(wc, ws))
    plain = f64(X) @ Wd.T + s * (ref["Z"] @ f64(B).T)
    assert rel(Y, plain) > 2 * TOL


def test_mx_forward_repeatable_and_m0():
    X, W, A, B = _layer(300, 1024, 384, 16, seed=5)
    base = pack_gpu(W, synth.MXFP4)
    a = L.forward_mx(base, to_dev(X), to_dev(A), to_dev(B), 2.0)
    b = L.forward_mx(base, to_dev(X), to_dev(A), to_dev(B), 2.0)
    torch.cuda.synchronize()
    assert torch.equal(a["Y"], b["Y"]) and torch.equal(a["Z"], b["Z"])
    e = L.forward_mx(base, to_dev(X[:0]), to_dev(A), to_dev(B), 2.0)
    assert e["Y"].shape == (0, 384)


@pytest.mark.parametrize("i", [0, 1, 2])
def test_mx_forward_full_size(i):
    """Every layer of the Llama-70B-shaped MXFP4 set (8192 tokens) through the
    MX-native forward, every element of Y and Z against the MX oracle (the
    element bound of gpu_util), outputs and workspace between guard bands."""
    lay = synth.layers(3)[i]
    t = synth.inputs(lay, names=("X", "W", "A", "B"))
    M, K, N, r = lay.M, lay.K, lay.N, lay.r
    print_case("mx full", lay.name, M, K, N, r)
    base = pack_gpu(t["W"], synth.MXFP4)
    nws = L.lora4_workspace_bytes_mx(base.abi(), M, r)
    ws, chk_ws = guarded((nws,), torch.uint8)
    Y, chk_y = guarded((M, N))
    Z, chk_z = guarded((M, r))
    # (the inputs stay referenced until the kernels have run: a tensor freed
    # after its pointer is taken could be refilled by the next copy)
    Xd, Ad, Bd = to_dev(t["X"]), to_dev(t["A"]), to_dev(t["B"])
    st = L.lora4_forward_mx(base.abi(), Xd.data_ptr(), M, Ad.data_ptr(), Bd.data_ptr(), r, lay.s, Y.data_ptr(),
                            Z.data_ptr(), ws.data_ptr(), nws, torch.cuda.current_stream().cuda_stream)
    assert st == 0, L.status_string(st)
    torch.cuda.synchronize()
    for chk, nm in ((chk_ws, "workspace"), (chk_y, "Y"), (chk_z, "Z")):
        chk(nm)
    Yh, Zh = to_host(Y), to_host(Z)
    del Y, Z, ws, base, Xd, Ad, Bd
    torch.cuda.empty_cache()
    wc, ws_ = oracle_pack_full(t["W"], synth.MXFP4)
    ref = mxfp8.forward(t["X"], wc, ws_, t["A"], t["B"], lay.s)
    report = {}
    compare_full("Y", Yh, ref["Y"], abs(lay.s) * (np.abs(ref["Z"]) @ np.abs(f64(t["B"])).T), report)
    compare_full("Z", Zh, ref["Z"], None, report)
    print("[parity] mx", lay.name, report, flush=True)
    write_report(f"llama70b-mx {lay.name} M={M} K={K} N={N} r={r}", report)
