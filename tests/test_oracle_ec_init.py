"""Pins of the oracle's data-free EC initialisation (CPU only): the rank-r
truncated SVD of the quantization residual.  Each pin comes from outside the
function: the Eckart-Young error, an independent route through the
eigenvectors of E^T E, a residual of known singular structure, the factor
split, and the reduction of the output error at gate 1."""
import numpy as np
import pytest

import oracle
from oracle import spear_ec_init as eci


def random_orthonormal(rng, n, k):
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))[None, :]


def test_eckart_young_error_and_rank():
    rng = np.random.default_rng(1)
    E = rng.standard_normal((60, 40))
    for r in (1, 5, 17, 40):
        A, B, S = eci.truncated_svd_factors(E, r)
        err = np.linalg.norm(E - A @ B) ** 2
        assert abs(err - np.sum(S[r:] ** 2)) <= 1e-10 * np.sum(S ** 2)
        assert np.linalg.matrix_rank(A @ B) == r


def test_projection_matches_eigenvectors_of_gram():
    """A B = E V_r V_r^T with V_r the top-r eigenvectors of E^T E (numpy.linalg.eigh,
    a different algorithm)."""
    rng = np.random.default_rng(2)
    E = rng.standard_normal((50, 30)) @ np.diag(np.linspace(3.0, 0.1, 30))
    r = 7
    A, B, _ = eci.truncated_svd_factors(E, r)
    lam, V = np.linalg.eigh(E.T @ E)
    Vr = V[:, np.argsort(lam)[::-1][:r]]
    assert np.allclose(A @ B, E @ Vr @ Vr.T, rtol=0, atol=1e-10 * np.abs(E).max())


def test_known_singular_structure():
    """E = U diag(sigma) V^T with chosen orthonormal U, V: A B is its leading r
    terms, and the sigma come back."""
    rng = np.random.default_rng(3)
    K, N, r = 64, 48, 6
    U, V = random_orthonormal(rng, K, N), random_orthonormal(rng, N, N)
    sigma = np.concatenate([np.linspace(10.0, 5.0, r), np.linspace(1.0, 0.01, N - r)])
    E = U @ np.diag(sigma) @ V.T
    A, B, S = eci.truncated_svd_factors(E, r)
    assert np.allclose(S, sigma, rtol=1e-12)
    assert np.allclose(A @ B, U[:, :r] @ np.diag(sigma[:r]) @ V[:, :r].T, atol=1e-12)


def test_balanced_split_and_sign_convention():
    rng = np.random.default_rng(4)
    E = rng.standard_normal((30, 20))
    A, B, S = eci.truncated_svd_factors(E, 5)
    assert np.allclose(A.T @ A, np.diag(S[:5]), atol=1e-12)
    assert np.allclose(B @ B.T, np.diag(S[:5]), atol=1e-12)
    idx = np.argmax(np.abs(A), axis=0)
    assert np.all(A[idx, np.arange(5)] > 0)


def test_residual_is_weight_minus_dequant_and_reduces_gate_one_error():
    """On a quantized weight: E = W - q s exactly (a grid weight has E = 0); at
    gate 1 the layer's error against the fp16 weight drops, and falls as the
    rank grows (the compensator's purpose)."""
    rng = np.random.default_rng(5)
    K, N, M = 256, 96, 32
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    Wq, s = oracle.pack_w4(W)
    E = eci.residual(W, Wq, s, K, N)
    assert np.array_equal(E, W.astype(np.float64) - oracle.dequant(Wq, s, K, N))
    X = rng.standard_normal((M, K))
    base = np.linalg.norm(X @ E)
    prev = base
    for r in (4, 16, 64):
        A, B, _ = eci.ec_init(W, Wq, s, r)
        err = np.linalg.norm(X @ (E - A @ B))
        assert err < prev
        prev = err
    assert prev < 0.9 * base
    # grouped scales: the residual uses the group dequantization
    Wq_g, s_g = oracle.pack_w4_grouped(W, 128)
    Eg = eci.residual(W, Wq_g, s_g, K, N, group=128)
    assert np.array_equal(Eg, W.astype(np.float64) - oracle.dequant_grouped(Wq_g, s_g, K, N, 128))
    # a weight on its own grid (power-of-two scales, every column reaching 7):
    # the residual and the factors are exactly zero
    q = rng.integers(-7, 8, size=(K, N))
    q[0, :] = 7
    grid = (q * np.power(2.0, rng.integers(-10, -5, size=N))[None, :]).astype(np.float16)
    Wq2, s2 = oracle.pack_w4(grid)
    assert not np.any(eci.residual(grid, Wq2, s2, K, N))
    A0, B0, S0 = eci.ec_init(grid, Wq2, s2, 4)
    assert not np.any(A0 @ B0) and not np.any(S0)
