"""Pins of the oracle's group-wise quantizer (CPU only).

Reading (SPEAR page, abstract: per-channel quantization named as the
challenging setting, so the group-wise one is its counterpart): one scale per
group of 128 consecutive input rows of each column, s[g, n] =
fp16(max |w| / 7) over the group, q = clamp(rint(w / s), -7, 7); the codes
use the same packed layout as the per-channel weights.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def fp16_round(fr):
    """Round a non-negative Fraction to the nearest fp16 (ties to even), by
    exhaustive bracketing over the fp16 grid (independent of numpy casts)."""
    grid = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    x = float(fr)
    i = int(np.searchsorted(grid, x))
    if i == 0:
        return 0.0
    if i >= grid.size:
        return float(grid[-1])
    lo, hi = Fraction(float(grid[i - 1])), Fraction(float(grid[i]))
    d_lo, d_hi = fr - lo, hi - fr
    if d_lo < d_hi:
        return float(lo)
    if d_hi < d_lo:
        return float(hi)
    # tie: even mantissa (the fp16 bit pattern's last bit)
    return float(lo) if (i - 1) % 2 == 0 else float(hi)


def brute_force_grouped(W, group):
    """Per element, with exact rationals and Python's round-half-even."""
    K, N = W.shape
    G = -(-K // group)
    s = np.zeros((G, N))
    q = np.zeros((K, N), dtype=np.int64)
    for n in range(N):
        for g in range(G):
            rows = range(g * group, min(K, (g + 1) * group))
            m = max(abs(Fraction(float(W[k, n]))) for k in rows)
            sg = fp16_round(m / 7)
            s[g, n] = sg
            for k in rows:
                if sg == 0:
                    q[k, n] = 0
                else:
                    v = round(Fraction(float(W[k, n])) / Fraction(sg))   # half to even
                    q[k, n] = max(-7, min(7, v))
    return s, q


@pytest.mark.parametrize("K,N,group", [(20, 3, 8), (136, 4, 128), (64, 2, 16), (7 * 8, 5, 24)])
def test_brute_force_per_element(K, N, group):
    rng = np.random.default_rng(K + N + group)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    W[0, 0] = np.float16(0.0)
    s_bf, q_bf = brute_force_grouped(W, group)
    s = oracle.group_scales(W, group)
    q = oracle.quantize_grouped(W, s, group)
    assert s.shape == (-(-K // group), N)
    assert np.array_equal(s.astype(np.float64), s_bf)
    assert np.array_equal(q.astype(np.int64), q_bf)


def test_one_group_spanning_k_is_the_per_channel_quantizer():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((256, 40)) * 0.02).astype(np.float16)
    for group in (256, 300, 4096):
        s = oracle.group_scales(W, group)
        assert s.shape == (1, 40)
        assert np.array_equal(s[0].view(np.uint16), oracle.channel_scales(W).view(np.uint16))
        q = oracle.quantize_grouped(W, s, group)
        assert np.array_equal(q, oracle.quantize(W, oracle.channel_scales(W)))
        Wq, s2 = oracle.pack_w4_grouped(W, group)
        Wq1, s1 = oracle.pack_w4(W)
        assert np.array_equal(Wq, Wq1)


def test_groups_are_independent_half_step_bound():
    rng = np.random.default_rng(5)
    K, N, group = 512, 32, 128
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    W[128:256, 3] *= np.float16(50.0)          # one loud group
    s = oracle.group_scales(W, group).astype(np.float64)
    q = oracle.quantize_grouped(W, oracle.group_scales(W, group), group).astype(np.float64)
    rows = np.arange(K) // group
    err = np.abs(W.astype(np.float64) - q * s[rows])
    assert np.all(err <= s[rows] / 2 * (1 + 1e-12))
    # the loud group does not change its neighbours' scales
    quiet = oracle.group_scales(np.delete(W, 3, axis=1), group)
    assert np.array_equal(np.delete(oracle.group_scales(W, group), 3, axis=1).view(np.uint16), quiet.view(np.uint16))


def test_grid_weights_per_group_round_trip_exactly():
    K, N, group = 384, 16, 128
    rng = np.random.default_rng(11)
    q = rng.integers(-7, 8, size=(K, N))
    q[0::group, :] = 7                             # each group's max maps to 7
    exps = rng.integers(-12, -4, size=(K // group, N)).astype(np.float64)
    s = np.power(2.0, exps)
    W = (q * s[np.arange(K) // group]).astype(np.float16)
    assert np.array_equal(W.astype(np.float64), q * s[np.arange(K) // group])
    Wq, s16 = oracle.pack_w4_grouped(W, group)
    assert np.array_equal(s16.astype(np.float64), s)
    assert np.array_equal(oracle.unpack_w4(Wq, K, N).astype(np.int64), q)
    assert np.array_equal(oracle.dequant_grouped(Wq, s16, K, N, group), W.astype(np.float64))


def test_zero_group_has_zero_scale_and_codes():
    W = (np.random.default_rng(2).standard_normal((256, 8)) * 0.02).astype(np.float16)
    W[128:, 5] = 0
    s = oracle.group_scales(W, 128)
    assert s[1, 5] == 0 and s[0, 5] != 0
    q = oracle.quantize_grouped(W, s, 128)
    assert np.all(q[128:, 5] == 0)


def test_layer_main_term_exactly_rounded_with_group_scales():
    """With the gate at 0 the layer is X dequant(Wq, s); each product
    x * q * s_g is exact in fp64 (11 + 4 + 11 bits), so math.fsum over k is
    the exactly rounded sum, which the oracle must match to a few ulp."""
    rng = np.random.default_rng(9)
    M, K, N, r = 6, 392, 24, 8
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    A = (rng.standard_normal((K, r)) * 0.01).astype(np.float16)
    B = (rng.standard_normal((r, N)) * 0.01).astype(np.float16)
    wg = (rng.standard_normal(K) * 0.05).astype(np.float16)
    Wq, s = oracle.pack_w4_grouped(W, 128)
    Y, info = oracle.w4ec_linear(X, Wq, s, A, B, wg, -1e4, K=K, N=N, group=128)
    assert np.all(info["g_eff"] == 0)
    q = oracle.unpack_w4(Wq, K, N)
    for m in range(M):
        for n in range(N):
            terms = [float(X[m, k]) * int(q[k, n]) * float(s[k // 128, n]) for k in range(K)]
            exact = math.fsum(terms)
            assert abs(Y[m, n] - exact) <= 4 * np.spacing(abs(exact)) + 1e-300


def test_layer_with_group_scales_keeps_the_ec_term():
    rng = np.random.default_rng(10)
    M, K, N, r = 4, 256, 16, 4
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    A = (rng.standard_normal((K, r)) * 0.01).astype(np.float16)
    B = (rng.standard_normal((r, N)) * 0.01).astype(np.float16)
    wg = (rng.standard_normal(K) * 0.05).astype(np.float16)
    Wq, s = oracle.pack_w4_grouped(W, 128)
    Y0, _ = oracle.w4ec_linear(X, Wq, s, A, B, wg, -1e4, K=K, N=N, group=128)
    Y1, _ = oracle.w4ec_linear(X, Wq, s, A, B, wg, 1e4, K=K, N=N, group=128)
    # g = 1 minus g = 0 is the whole EC term (X A) B
    ec = X.astype(np.float64) @ A.astype(np.float64) @ B.astype(np.float64)
    assert np.allclose(Y1 - Y0, ec, rtol=1e-12, atol=1e-15)
