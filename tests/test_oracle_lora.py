"""Pins for the oracle's LoRA forward and backward.

Sources: "Training LLMs on a Budget: LoRA, QLoRA, and LoftQ", section 2 (the
forward y = Wx + (alpha/r) BAx; the gradient derivation through z = Ax; the
step-0 gradient table for B = 0 and A = 0; the merge W' = W + (alpha/r) BA;
the worked parameter count). Crusoe post, "Backward pass and optimizer step in
training" (gradients for X, A and B; none for the frozen W).
"""

import json
import os

import numpy as np

import synth
from oracle import codecs, lora, nf4

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def _loss(X, W, A, B, s, dY):
    return float(np.sum(dY * lora.forward(X, W, A, B, s)["Y"]))


def test_finite_differences_float64():
    # L = sum(dY * Y) is affine in each single entry of X, A and B, so a central
    # difference is exact up to float64 rounding.
    rng = np.random.default_rng(21)
    M, K, N, r, s = 3, 8, 5, 2, 1.75
    X, W, A, B, dY = (_rand(sh, rng) for sh in [(M, K), (N, K), (r, K), (N, r), (M, N)])
    g = lora.backward(X, W, A, B, s, dY)
    h = 1e-3
    for name, T, G in [("X", X, g["dX"]), ("A", A, g["dA"]), ("B", B, g["dB"])]:
        num = np.zeros_like(T)
        for idx in np.ndindex(T.shape):
            old = T[idx]
            T[idx] = old + h
            lp = _loss(X, W, A, B, s, dY)
            T[idx] = old - h
            lm = _loss(X, W, A, B, s, dY)
            T[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert np.allclose(num, G, rtol=1e-9, atol=1e-9), name


def test_pure_python_loops_agree():
    rng = np.random.default_rng(22)
    M, K, N, r, s = 2, 4, 3, 2, 2.0
    X, W, A, B, dY = (_rand(sh, rng) for sh in [(M, K), (N, K), (r, K), (N, r), (M, N)])
    out = lora.forward(X, W, A, B, s)
    g = lora.backward(X, W, A, B, s, dY)
    for m in range(M):
        z = [sum(A[j][k] * X[m][k] for k in range(K)) for j in range(r)]
        for n in range(N):
            yb = sum(W[n][k] * X[m][k] for k in range(K))
            yl = s * sum(B[n][j] * z[j] for j in range(r))
            assert abs(out["Y"][m, n] - (yb + yl)) < 1e-12
        dz = [s * sum(dY[m][n] * B[n][j] for n in range(N)) for j in range(r)]
        for k in range(K):
            dx = sum(dY[m][n] * W[n][k] for n in range(N)) + sum(dz[j] * A[j][k] for j in range(r))
            assert abs(g["dX"][m, k] - dx) < 1e-12
    for j in range(r):
        for k in range(K):
            da = sum(s * sum(dY[m][n] * B[n][j] for n in range(N)) * X[m][k] for m in range(M))
            assert abs(g["dA"][j, k] - da) < 1e-12
    for n in range(N):
        for j in range(r):
            db = s * sum(dY[m][n] * sum(A[j][k] * X[m][k] for k in range(K)) for m in range(M))
            assert abs(g["dB"][n, j] - db) < 1e-12


def test_scalar_closed_form():
    x, w, a, b, s, dy = 0.7, -1.3, 0.4, 2.5, 3.0, -0.9
    out = lora.forward([[x]], [[w]], [[a]], [[b]], s)
    assert out["Y"][0, 0] == w * x + s * b * a * x
    g = lora.backward([[x]], [[w]], [[a]], [[b]], s, [[dy]])
    assert np.isclose(g["dX"][0, 0], dy * (w + s * b * a), rtol=1e-15)
    assert np.isclose(g["dA"][0, 0], s * b * dy * x, rtol=1e-15)
    assert np.isclose(g["dB"][0, 0], s * dy * a * x, rtol=1e-15)


def test_b_zero_is_the_frozen_base_and_kills_dA():
    # B = 0: the forward is bit-identical to the base and dL/dA = 0 (step-0 table).
    rng = np.random.default_rng(23)
    M, K, N, r, s = 6, 64, 7, 4, 2.0
    X, W, A, dY = (_rand(sh, rng) for sh in [(M, K), (N, K), (r, K), (M, N)])
    B = np.zeros((N, r))
    out = lora.forward(X, W, A, B, s)
    assert (out["Y"] == out["Y_base"]).all()
    g = lora.backward(X, W, A, B, s, dY)
    assert (g["dA"] == 0).all() and np.abs(g["dB"]).max() > 0


def test_a_zero_kills_dB():
    rng = np.random.default_rng(24)
    M, K, N, r, s = 6, 64, 7, 4, 2.0
    X, W, B, dY = (_rand(sh, rng) for sh in [(M, K), (N, K), (N, r), (M, N)])
    A = np.zeros((r, K))
    g = lora.backward(X, W, A, B, s, dY)
    assert (g["dB"] == 0).all() and np.abs(g["dA"]).max() > 0
    assert (lora.forward(X, W, A, B, s)["Y_lora"] == 0).all()


def test_merged_equals_unmerged():
    rng = np.random.default_rng(25)
    M, K, N, r, s = 9, 128, 33, 8, 2.0
    X, W, A, B = (_rand(sh, rng) for sh in [(M, K), (N, K), (r, K), (N, r)])
    un = lora.forward(X, W, A, B, s)["Y"]
    me = lora.merged_forward(X, W, A, B, s)
    assert np.allclose(un, me, rtol=1e-12, atol=1e-12)


def test_adapter_gradient_shapes_match_parameter_count():
    g = GOLD["lora_params_r8_4096"]
    r, K, N = g["r"], g["d_in"], g["d_out"]
    rng = np.random.default_rng(26)
    X = _rand((1, K), rng)
    out = lora.backward(X, np.zeros((N, K)), _rand((r, K), rng), _rand((N, r), rng), 1.0, _rand((1, N), rng))
    assert out["dA"].shape == (r, K) and out["dB"].shape == (N, r)
    assert out["dA"].size + out["dB"].size == g["value"]


def test_grouped_matches_per_expert_calls_and_empty_group():
    rng = np.random.default_rng(27)
    K, N, r, s = 64, 12, 4, 2.0
    offs = [0, 3, 3, 10, 11]                          # expert 1 has no rows
    E = 4
    X = _rand((offs[-1], K), rng)
    dY = _rand((offs[-1], N), rng)
    Ws = [_rand((N, K), rng) for _ in range(E)]
    As = [_rand((r, K), rng) for _ in range(E)]
    Bs = [_rand((N, r), rng) for _ in range(E)]
    f = lora.grouped_forward(X, Ws, As, Bs, s, offs)
    b = lora.grouped_backward(X, Ws, As, Bs, s, dY, offs)
    for e in range(E):
        a, c = offs[e], offs[e + 1]
        if c == a:
            assert (b["dA"][e] == 0).all() and (b["dB"][e] == 0).all()
            continue
        ref = lora.forward(X[a:c], Ws[e], As[e], Bs[e], s)
        assert np.array_equal(f["Y"][a:c], ref["Y"])
        g = lora.backward(X[a:c], Ws[e], As[e], Bs[e], s, dY[a:c])
        assert np.array_equal(b["dX"][a:c], g["dX"])
        assert np.array_equal(b["dA"][e], g["dA"])


def test_moe_routing_invariants():
    order, counts, offs = synth.moe_routing()
    assert counts.sum() == 4096 * 8 == offs[-1]
    assert all(len(set(row)) == 8 for row in order.tolist())     # 8 distinct experts per token
    assert counts.min() > 0


def test_rel_frobenius():
    a = np.array([[3.0, 4.0]])
    assert lora.rel_frobenius(a, a) == 0.0
    assert abs(lora.rel_frobenius(a * 1.01, a) - 0.01) < 1e-12


def test_end_to_end_small_workload_tolerance_budget():
    # bf16 rounding of the outputs alone stays well inside the 5e-3 bar
    lay = synth.layers(1)[0]
    t = synth.inputs(lay)
    packed, sc = nf4.quantize(t["W"])
    Wd = lora.as_f64(nf4.dequantize(packed, sc))
    out = lora.forward(lora.as_f64(t["X"]), Wd, lora.as_f64(t["A"]), lora.as_f64(t["B"]), lay.s)
    yb = codecs.bf16_round(out["Y"])
    assert lora.rel_frobenius(yb, out["Y"]) < 2.5e-3
