"""LoftQ initialisation: alternate quantization of the base and a rank-r SVD
of the quantization residual.

Test infrastructure only (see the package docstring).

Source: "Training LLMs on a Budget: LoRA, QLoRA, and LoftQ", section 4
("The algorithm: alternating quantization and SVD", "A worked example:
3 x 3"). The goal is a small ||W - (Q + B A)||_F at step 0; the loop:
* Q_0 = quant(W), R_0 = W - Q_0;
* top-r SVD R_t = U S V^T: B_t = U_r sqrt(S_r), A_t = sqrt(S_r) V_r^T (the best
  rank-r approximation of R_t, Eckart-Young);
* Q_{t+1} = quant(W - B_t A_t), R_{t+1} = W - Q_{t+1}; repeat (5 times by
  default).

Readings where the page leaves a step open:
* one iteration is one SVD step; the loop ends after an SVD step, so the
  returned (Q_t, B_t, A_t) belong together (Q_t + B_t A_t ~ W): iters = 1 is
  the page's "LoftQ, 1 iteration" row;
* with NF4 as the quantizer the shifted matrix W - B A is rounded to bf16
  first (the NF4 packer quantizes a bf16 matrix); the SVD works on the exact
  float64 residual;
* for a layer that scales its adapter by s, B is returned divided by s, so
  that s B A is the rank-r correction.
"""

import numpy as np

from . import nf4
from .codecs import bf16_to_f32, f32_to_bf16


def rank_r(R, r):
    """Best rank-r factors of R (float64): B = U_r sqrt(S_r), A = sqrt(S_r) V_r^T."""
    U, S, Vt = np.linalg.svd(R, full_matrices=False)
    sq = np.sqrt(S[:r])
    return U[:, :r] * sq, sq[:, None] * Vt[:r]


def loftq(W, r, iters, quant):
    """The alternating loop on a float64 W with a quantize-dequantize function
    quant(matrix) -> matrix. Returns (Q, B, A) of the last SVD step and the
    error ||W - Q - B A||_F after every step."""
    Q = quant(W)
    errs = []
    for t in range(iters):
        B, A = rank_r(W - Q, r)
        errs.append(float(np.linalg.norm(W - Q - B @ A)))
        if t + 1 < iters:
            Q = quant(W - B @ A)
    return Q, B, A, errs


def nf4_quant(double_quant=False):
    """quant() for NF4: bf16(matrix) -> NF4 packing -> dequantized float64."""
    def q(M):
        u = f32_to_bf16(np.asarray(M, dtype=np.float32))
        codes, sc = nf4.quantize(u)
        if double_quant:
            c8, c2 = nf4.double_quantize(sc)
            return bf16_to_f32(nf4.dequantize_dq(codes, c8, c2)).astype(np.float64)
        return bf16_to_f32(nf4.dequantize(codes, sc)).astype(np.float64)
    return q


def loftq_nf4(W_bf16, r, iters=5, s=1.0, double_quant=False):
    """LoftQ with NF4 on a bf16 W [N, K]: returns the NF4 packing of the last
    quantization (codes, scales[, second level]), B / s [N, r] and A [r, K]
    (float64) and the errors per step."""
    W = bf16_to_f32(W_bf16).astype(np.float64)
    shift = np.zeros_like(W)
    for t in range(iters):
        u = f32_to_bf16((W - shift).astype(np.float32))
        codes, sc = nf4.quantize(u)
        if double_quant:
            c8, c2 = nf4.double_quantize(sc)
            packed = (codes, c8, c2)
            Q = bf16_to_f32(nf4.dequantize_dq(codes, c8, c2)).astype(np.float64)
        else:
            packed = (codes, sc)
            Q = bf16_to_f32(nf4.dequantize(codes, sc)).astype(np.float64)
        B, A = rank_r(W - Q, r)
        shift = B @ A
    err = float(np.linalg.norm(W - Q - B @ A))
    return packed, B / s, A, err
