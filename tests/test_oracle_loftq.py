"""Pins of the LoftQ oracle (CPU): the page's 3 x 3 worked example (integer
rounding standing in for NF4), its 256 x 256 rank-8 rounding setup, the
Eckart-Young optimum on a matrix with known singular values, and the NF4
variant against plain NF4."""

import numpy as np

from oracle import loftq, nf4
from oracle.codecs import bf16_to_f32
from synth import to_bf16


def test_worked_example_3x3():
    """"Training LLMs on a Budget", section 4, "A worked example: 3 x 3"."""
    W = np.array([[1.1, 0.1, 0.2], [0.2, 1.2, 0.4], [0.1, 0.1, 1.2]])
    Q0 = np.rint(W)
    assert np.array_equal(Q0, np.eye(3))
    naive = np.linalg.norm(W - Q0)
    assert abs(naive - 0.6) < 1e-12                         # the table's QLoRA row
    Q, B, A, errs = loftq.loftq(W, 1, 1, np.rint)
    assert np.array_equal(Q, np.eye(3))
    assert errs[0] < 1e-12                                  # "LoftQ, 1 iteration": 0.000
    assert np.allclose(B @ A, W - Q0, atol=1e-12)           # B0 A0 = R0 (rank 1)
    _, _, _, errs5 = loftq.loftq(W, 1, 5, np.rint)
    assert max(errs5) < 1e-12                               # "further iterations": 0.000


def test_rounding_loop_never_increases_the_error():
    """The page's synthetic setup (256 x 256, rank-8 adapter, rounding as the
    quantizer): rounding is the exact minimizer over the integer grid and the
    SVD the exact minimizer over rank r, so no step can raise the error, and
    one SVD step already beats the naive error."""
    rng = np.random.default_rng(31)
    W = rng.standard_normal((256, 256)) * 0.6 + rng.standard_normal((256, 8)) @ rng.standard_normal((8, 256)) * 0.3
    naive = np.linalg.norm(W - np.rint(W))
    _, _, _, errs = loftq.loftq(W, 8, 6, np.rint)
    assert errs[0] < naive
    assert all(b <= a + 1e-9 for a, b in zip(errs, errs[1:]))
    assert errs[-1] < errs[0]


def test_rank_r_is_the_eckart_young_optimum():
    rng = np.random.default_rng(32)
    n, k, r = 40, 30, 5
    U, _ = np.linalg.qr(rng.standard_normal((n, k)))
    V, _ = np.linalg.qr(rng.standard_normal((k, k)))
    sig = np.sort(rng.uniform(0.1, 3.0, k))[::-1]
    R = (U * sig) @ V.T
    B, A = loftq.rank_r(R, r)
    assert abs(np.linalg.norm(R - B @ A) ** 2 - np.sum(sig[r:] ** 2)) < 1e-9
    # B and A share the singular values evenly: B^T B = A A^T = diag(sig_r)
    assert np.allclose(B.T @ B, np.diag(sig[:r]), atol=1e-9)
    assert np.allclose(A @ A.T, np.diag(sig[:r]), atol=1e-9)


def test_nf4_loftq_beats_plain_nf4_and_scales_b():
    rng = np.random.default_rng(33)
    w = rng.standard_normal((128, 256)).astype(np.float32) * np.float32(0.02)
    w += (rng.standard_normal((128, 4)) @ rng.standard_normal((4, 256))).astype(np.float32) * np.float32(0.01)
    Wb = to_bf16(w)
    W = bf16_to_f32(Wb).astype(np.float64)
    codes, sc = nf4.quantize(Wb)
    naive = np.linalg.norm(W - bf16_to_f32(nf4.dequantize(codes, sc)).astype(np.float64))
    packed, B, A, err = loftq.loftq_nf4(Wb, 8, iters=5)
    Q = bf16_to_f32(nf4.dequantize(*packed)).astype(np.float64)
    assert abs(np.linalg.norm(W - Q - B @ A) - err) < 1e-9
    assert err < 0.97 * naive
    # one iteration: the base is plain NF4 of W
    p1, B1, A1, _ = loftq.loftq_nf4(Wb, 8, iters=1)
    assert np.array_equal(p1[0], codes) and np.array_equal(p1[1].view(np.uint32), sc.view(np.uint32))
    # a layer scale s divides B
    p2, B2, A2, _ = loftq.loftq_nf4(Wb, 8, iters=1, s=4.0)
    assert np.allclose(4.0 * B2 @ A2, B1 @ A1, atol=1e-12)
