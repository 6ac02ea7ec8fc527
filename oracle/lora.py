"""Unmerged-LoRA linear over a frozen base: forward and backward, plain float64.

Test infrastructure only (see the package docstring).

Sources:
* "Training LLMs on a Budget: LoRA, QLoRA, and LoftQ", section 2: W is
  ``[d_out, d_in]``, ``A`` is ``[r, d_in]`` (down), ``B`` is ``[d_out, r]``
  (up); ``y = W x + (alpha/r) B A x`` ("The math"); with ``z = A x`` the chain
  rule gives ``dL/dz = B^T dL/dy``, ``dL/dA = dL/dz x^T`` and
  ``dL/dB = dL/dy z^T`` ("Initialization matters"). The page states that the
  scale alpha/r is part of the layer and reappears wherever BA does, so it is
  applied in every gradient too.
* Crusoe post, "LoRA operations and quantization" / "Terminology": Y is split
  into Y^base and Y^LoRA and the adapter stays separate from W (unmerged);
  "Backward pass and optimizer step in training": gradients for X, A and B,
  none for the frozen W.

Row-major batched form with tokens as rows (X is ``[M, K]``):
    Z      = X A^T                      [M, r]
    Y^base = X W~^T                     [M, N]
    Y^LoRA = s Z B^T                    [M, N]
    Y      = Y^base + Y^LoRA
    dZ     = s dY B                     [M, r]
    dX     = dY W~ + dZ A               [M, K]
    dA     = dZ^T X                     [r, K]
    dB     = s dY^T Z                   [N, r]
where W~ is the dequantized base and s = alpha / r. Every input is an exact
bf16 value; all products and sums are float64 (no intermediate rounding).
"""

import numpy as np

from .codecs import bf16_to_f32


def as_f64(u16):
    """bf16 bit patterns -> float64 values (exact)."""
    return bf16_to_f32(u16).astype(np.float64)


def forward(X, W, A, B, s):
    """Float64 forward. X [M,K], W [N,K] (dequantized values), A [r,K], B [N,r]."""
    X, W, A, B = (np.asarray(t, dtype=np.float64) for t in (X, W, A, B))
    Z = X @ A.T
    Y_base = X @ W.T
    Y_lora = s * (Z @ B.T)
    return {"Y": Y_base + Y_lora, "Y_base": Y_base, "Y_lora": Y_lora, "Z": Z}


def backward(X, W, A, B, s, dY, Z=None):
    """Float64 backward: returns dX [M,K], dA [r,K], dB [N,r] (and dZ)."""
    X, W, A, B, dY = (np.asarray(t, dtype=np.float64) for t in (X, W, A, B, dY))
    if Z is None:
        Z = X @ A.T
    dZ = s * (dY @ B)
    dX = dY @ W + dZ @ A
    dA = dZ.T @ X
    dB = s * (dY.T @ np.asarray(Z, dtype=np.float64))
    return {"dX": dX, "dA": dA, "dB": dB, "dZ": dZ}


def merged_forward(X, W, A, B, s):
    """Merged form ``X (W~ + s B A)^T`` ("Deployment: keep or merge"), float64."""
    X, W, A, B = (np.asarray(t, dtype=np.float64) for t in (X, W, A, B))
    return X @ (W + s * (B @ A)).T


def grouped_forward(X, Ws, As, Bs, s, offsets):
    """Grouped (per-expert) forward: rows offsets[e]:offsets[e+1] use expert e.

    Ws[e] is expert e's dequantized W, As[e] / Bs[e] its adapters. The rows of
    X are already sorted by expert; routing and gating are outside the layer.
    """
    X = np.asarray(X, dtype=np.float64)
    M = X.shape[0]
    N = Ws[0].shape[0]
    r = As[0].shape[0]
    Y = np.zeros((M, N))
    Z = np.zeros((M, r))
    for e in range(len(Ws)):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            out = forward(X[a:b], Ws[e], As[e], Bs[e], s)
            Y[a:b] = out["Y"]
            Z[a:b] = out["Z"]
    return {"Y": Y, "Z": Z}


def grouped_backward(X, Ws, As, Bs, s, dY, offsets):
    """Grouped backward; dA, dB are per expert (zero for an expert with no rows)."""
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    E = len(Ws)
    dX = np.zeros_like(X)
    dA = [np.zeros_like(np.asarray(As[e], dtype=np.float64)) for e in range(E)]
    dB = [np.zeros_like(np.asarray(Bs[e], dtype=np.float64)) for e in range(E)]
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            g = backward(X[a:b], Ws[e], As[e], Bs[e], s, dY[a:b])
            dX[a:b] = g["dX"]
            dA[e] = g["dA"]
            dB[e] = g["dB"]
    return {"dX": dX, "dA": dA, "dB": dB}


def rel_frobenius(got, ref):
    """||got - ref||_F / ||ref||_F in float64 (0 when both are zero)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(r)
    num = np.linalg.norm(g - r)
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)
