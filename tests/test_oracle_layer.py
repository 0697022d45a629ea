"""Pins of the oracle's gate and layer output (CPU only).

Layer: Y = X . dequant(Wq, s) + g (.) ((X . A) . B), g = sigmoid(X . w_g + b_g)
(SPEAR page, abstract: error compensators scaled per token by a gate, their
second half computed inside the low-bit GEMM).  Every pin below comes from outside the oracle: a
closed form, a special case that reduces to a textbook product, a library
routine, brute force, or an exactly rounded sum.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle


def grid_layer(M, K, N, r, seed):
    """Inputs whose quantized weight is known exactly: W = s q, s = 2^e."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-7, 8, size=(K, N))
    q[rng.integers(0, K, N), np.arange(N)] = rng.choice([-7, 7], N)
    s = np.ldexp(1.0, rng.integers(-9, -5, size=N))
    W64 = q * s[None, :]
    W = W64.astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    A = (rng.standard_normal((K, r)) * 0.05).astype(np.float16)
    B = (rng.standard_normal((r, N)) * 0.05).astype(np.float16)
    w_g = (rng.standard_normal(K) * 0.05).astype(np.float16)
    return X, W, W64, A, B, w_g


# ---------------------------------------------------------------- gate

def test_gate_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 3.5, -20.0, 40.0])
    g, g_eff, amb = oracle.gate(z)
    assert g[0] == 0.5
    assert np.allclose(g[1] + g[2], 1.0, rtol=0, atol=1e-15)
    assert abs(g[1] - 1.0 / (1.0 + math.e ** -1)) < 1e-15
    assert np.array_equal(g, g_eff) and not amb.any()


def test_gate_matches_scipy_expit():
    z = np.linspace(-60, 60, 10001)
    g, _, _ = oracle.gate(z)
    assert np.max(np.abs(g - scipy.special.expit(z))) < 1e-15


def test_gate_saturates_to_exact_zero_and_one():
    g, _, _ = oracle.gate(np.array([-1e4, 1e4]))
    assert g[0] == 0.0 and g[1] == 1.0
    with np.errstate(over="ignore"):
        g32 = np.float32(1) / (np.float32(1) + np.exp(np.float32(1e4)))
    assert g32 == 0.0


def test_gate_threshold_and_ambiguity_band():
    tau = 0.05
    lt = math.log(tau / (1 - tau))
    z = np.array([lt - 1.0, lt + 1.0, lt + 1e-4, lt - 1e-4, 5.0])
    g, g_eff, amb = oracle.gate(z, tau)
    assert g_eff[0] == 0.0 and g_eff[1] == g[1] and g_eff[4] == g[4]
    assert list(amb) == [False, False, True, True, False]


def test_gate_logits_is_dot_plus_bias():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((5, 40)).astype(np.float16)
    w = rng.standard_normal(40).astype(np.float16)
    z = oracle.gate_logits(X, w, -0.75)
    for m in range(5):
        ref = math.fsum(float(X[m, k]) * float(w[k]) for k in range(40)) - 0.75
        assert abs(z[m] - ref) <= 1e-13 * (1 + abs(ref))


# ---------------------------------------------------------------- layer

def test_gate_zero_reduces_to_plain_w4_gemm():
    X, W, W64, A, B, w_g = grid_layer(7, 96, 48, 5, seed=1)
    Wq, s = oracle.pack_w4(W)
    Y, info = oracle.w4ec_linear(X, Wq, s, A, B, w_g, -1e4)
    assert np.all(info["g_eff"] == 0.0)
    ref = X.astype(np.float64) @ W64
    assert np.max(np.abs(Y - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_gate_one_reduces_to_static_dense_correction():
    X, W, W64, A, B, w_g = grid_layer(9, 64, 40, 6, seed=2)
    Wq, s = oracle.pack_w4(W)
    Y, info = oracle.w4ec_linear(X, Wq, s, A, B, w_g, 1e4)
    assert np.all(info["g_eff"] == 1.0)
    merged = W64 + A.astype(np.float64) @ B.astype(np.float64)
    ref = X.astype(np.float64) @ merged
    assert np.max(np.abs(Y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_rank_zero_has_no_ec_term():
    X, W, W64, A, B, w_g = grid_layer(3, 32, 16, 4, seed=3)
    Wq, s = oracle.pack_w4(W)
    Y, _ = oracle.w4ec_linear(X, Wq, s, None, None, None, 0.0)
    assert np.max(np.abs(Y - X.astype(np.float64) @ W64)) <= 1e-13 * np.max(np.abs(Y))


@pytest.mark.parametrize("M,K,N,r,b_g", [(3, 16, 8, 2, 0.3), (5, 24, 12, 3, -1.0), (1, 8, 20, 1, 0.0)])
def test_brute_force_scalar_loops(M, K, N, r, b_g):
    """Pure-Python loops over the definition, weights known exactly."""
    X, W, W64, A, B, w_g = grid_layer(M, K, N, r, seed=M * 100 + K)
    Wq, s = oracle.pack_w4(W)
    Y, _ = oracle.w4ec_linear(X, Wq, s, A, B, w_g, b_g)
    x = X.astype(float).tolist()
    a = A.astype(float).tolist()
    b = B.astype(float).tolist()
    wg = w_g.astype(float).tolist()
    w = W64.tolist()
    bias = float(np.float32(b_g))          # the bias argument is a float32
    for m in range(M):
        z = sum(x[m][k] * wg[k] for k in range(K)) + bias
        g = 1.0 / (1.0 + math.exp(-z))
        p = [sum(x[m][k] * a[k][j] for k in range(K)) for j in range(r)]
        for n in range(N):
            main = sum(x[m][k] * w[k][n] for k in range(K))
            ec = sum(p[j] * b[j][n] for j in range(r))
            ref = main + g * ec
            assert abs(Y[m, n] - ref) <= 1e-12 * (1 + abs(ref))


def test_main_term_exactly_rounded_at_sampled_outputs():
    """fp16 x (int4 * power-of-two) products are exact in float64, so
    math.fsum gives the exactly rounded main term."""
    X, W, W64, A, B, w_g = grid_layer(16, 512, 64, 4, seed=4)
    Wq, s = oracle.pack_w4(W)
    Y, _ = oracle.w4ec_linear(X, Wq, s, None, None, None, 0.0)
    rng = np.random.default_rng(0)
    for _ in range(200):
        m, n = int(rng.integers(16)), int(rng.integers(64))
        terms = [float(X[m, k]) * W64[k, n] for k in range(512)]
        exact = math.fsum(terms)
        scale = math.fsum(abs(t) for t in terms)
        assert abs(Y[m, n] - exact) <= 512 * 2.0 ** -53 * scale


def test_linearity_in_gate():
    X, W, W64, A, B, w_g = grid_layer(6, 64, 32, 4, seed=5)
    Wq, s = oracle.pack_w4(W)
    Y1, i1 = oracle.w4ec_linear(X, Wq, s, A, B, w_g, 0.5)
    Y2, i2 = oracle.w4ec_linear(X, Wq, s, A, B, w_g, -2.0)
    PB = (X.astype(np.float64) @ A.astype(np.float64)) @ B.astype(np.float64)
    diff = (i1["g"] - i2["g"])[:, None] * PB
    assert np.max(np.abs((Y1 - Y2) - diff)) <= 1e-13 * (1 + np.max(np.abs(Y1)))
    assert np.any(np.abs(diff) > 1e-3)


def test_transposed_operands_are_caught_by_shapes():
    X, W, W64, A, B, w_g = grid_layer(3, 40, 24, 5, seed=6)
    Wq, s = oracle.pack_w4(W)
    with pytest.raises(ValueError):
        oracle.w4ec_linear(X, Wq, s, B.T, A.T, w_g, 0.0)


def test_skip_threshold_zeroes_only_low_gate_tokens():
    X, W, W64, A, B, w_g = grid_layer(12, 64, 32, 4, seed=8)
    Wq, s = oracle.pack_w4(W)
    Yt, it = oracle.w4ec_linear(X, Wq, s, A, B, w_g, 0.0, tau=0.5)
    Y0, i0 = oracle.w4ec_linear(X, Wq, s, A, B, w_g, 0.0, tau=0.0)
    Yoff, _ = oracle.w4ec_linear(X, Wq, s, A, B, w_g, -1e4)
    low = i0["g"] < 0.5
    assert low.any() and (~low).any()
    assert np.allclose(Yt[low], Yoff[low], rtol=0, atol=1e-13)
    assert np.allclose(Yt[~low], Y0[~low], rtol=0, atol=1e-13)


def test_metrics():
    ref = np.array([[3.0, 4.0]])
    assert oracle.rel_l2(ref, ref) == 0.0
    assert abs(oracle.rel_l2(ref * 1.001, ref) - 1e-3) < 1e-12
    rms = math.sqrt(12.5)
    assert abs(oracle.max_abs_over_rms(ref + [[0.0, 0.5]], ref) - 0.5 / rms) < 1e-12
