"""Pins of the scheduler oracle (brute force over subsets) and parity of the
library's selection step (spear_schedule_ec_costs, host code) with it; the
cost model's structure.  CPU only."""
import os

import numpy as np
import pytest

from oracle import spear_sched as osch

try:
    import w4_gemm_gated_amd as sp
    from w4_gemm_gated_amd import _binding
    HAVE_LIB = os.path.exists(_binding.LIB_PATH)
except Exception:  # noqa: BLE001
    HAVE_LIB = False

needs_lib = pytest.mark.skipif(not HAVE_LIB, reason="libspear_w4ec.so not built")


def test_hand_worked_instance():
    # added times 2, 3, 4 us, weights 3, 4, 5, slack 5.5: {0, 1} (5 us, weight 7)
    # fits, {0, 2} and {1, 2} do not; weight 7 beats every single layer.
    sub, w, u = osch.best_subset([2.0, 3.0, 4.0], [3.0, 4.0, 5.0], 5.5)
    assert sub == (0, 1) and w == 7.0
    # slack exactly 5: rounding up (2 -> 26215 units, 3 -> 39322) puts {0, 1} one
    # unit over 65536, so the best is the single layer of weight 5.
    sub, w, u = osch.best_subset([2.0, 3.0, 4.0], [3.0, 4.0, 5.0], 5.0)
    assert sub == (2,) and w == 5.0


def test_special_cases():
    assert osch.best_subset([1.0, 2.0], [1.0, 1.0], -0.1)[0] == ()
    assert osch.best_subset([1.0, 2.0, 0.5], [1.0, 1.0, 1.0], 100.0)[0] == (0, 1, 2)   # everything fits
    assert osch.best_subset([0.0, 1.0], [1.0, 1.0], 0.0)[0] == (0,)                    # only free layers
    assert osch.best_subset([-1.0, 1.0], [9.0, 1.0], 10.0)[0] == (1,)                  # no EC: never
    assert osch.best_subset([1.0, 1.0], [0.0, 2.0], 10.0)[0] == (1,)                   # weight 0: never
    # equal weights: the cheaper set
    assert osch.best_subset([3.0, 1.0], [1.0, 1.0], 3.5)[0] == (1,)


def test_optimum_matches_an_independent_integer_program():
    """scipy's MILP solver on the same integer knapsack finds the same best weight."""
    from scipy.optimize import LinearConstraint, Bounds, milp
    rng = np.random.default_rng(5)
    for trial in range(30):
        n = int(rng.integers(1, 11))
        extra = rng.uniform(0.0, 6.0, n)
        weights = rng.integers(1, 20, n).astype(float)
        slack = float(rng.uniform(0.0, 20.0))
        unit, cap = osch.grid(slack)
        units = np.array([osch.units_of(e, unit) for e in extra], dtype=float)
        res = milp(c=-weights, constraints=LinearConstraint(units[None, :], -np.inf, cap),
                   integrality=np.ones(n), bounds=Bounds(0, 1))
        sub, w, u = osch.best_subset(list(extra), list(weights), slack)
        assert res.status == 0
        assert abs(-res.fun - w) < 1e-9, (trial, sub, w, -res.fun)


def test_monotone_in_slack():
    rng = np.random.default_rng(8)
    extra = list(rng.uniform(0.5, 4.0, 8))
    weights = list(rng.uniform(0.1, 3.0, 8))
    prev = -1.0
    for slack in np.linspace(0.0, 30.0, 31):
        w = osch.best_subset(extra, weights, float(slack))[1]
        assert w >= prev - 1e-12
        prev = w


@needs_lib
def test_library_selection_matches_oracle():
    rng = np.random.default_rng(11)
    for trial in range(60):
        n = int(rng.integers(0, 13))
        extra = list(np.where(rng.random(n) < 0.2, -1.0, rng.uniform(0.0, 8.0, n)))
        weights = list(np.float32(np.where(rng.random(n) < 0.1, 0.0, rng.uniform(0.0, 5.0, n))))
        if trial % 7 == 0:
            weights = [np.float32(1.0)] * n                       # many ties
        slack = float(rng.uniform(-2.0, 25.0))
        on, added = sp.spear_schedule_ec_costs(extra, weights, slack)
        sub, w, u = osch.best_subset(extra, weights, slack)
        got = tuple(i for i in range(n) if on[i])
        unit, cap = osch.grid(max(slack, 0.0))
        got_w = 0.0
        for i in got:
            got_w += float(weights[i])
        got_u = sum(osch.units_of(extra[i], unit) for i in got)
        assert got_w == w and got_u == u, (trial, got, sub)
        assert got_u <= cap or slack < 0
        assert abs(added - sum(extra[i] for i in got)) < 1e-9
        assert added <= max(slack, 0.0) + 1e-9


@needs_lib
def test_library_selection_on_the_coarse_grid():
    """Beyond 256 layers the grid coarsens with n; the library's choice is
    still an optimum of that grid's knapsack (scipy's MILP on the same integer
    costs), fits the slack, and 4096 layers take a fraction of a second."""
    import time
    from scipy.optimize import LinearConstraint, Bounds, milp
    assert osch.grid_steps(256) == 65536 and osch.grid_steps(512) == 32768 and osch.grid_steps(4096) == 4096
    rng = np.random.default_rng(23)
    for n in (300, 600):
        extra = rng.uniform(0.0, 2.0, n)
        weights = rng.integers(1, 50, n).astype(np.float32)
        slack = float(rng.uniform(50.0, 200.0))
        on, added = sp.spear_schedule_ec_costs(list(extra), list(weights), slack)
        unit, cap = osch.grid(slack, n)
        units = np.array([osch.units_of(e, unit) for e in extra], dtype=float)
        res = milp(c=-weights.astype(float), constraints=LinearConstraint(units[None, :], -np.inf, cap),
                   integrality=np.ones(n), bounds=Bounds(0, 1))
        assert res.status == 0
        got = [i for i in range(n) if on[i]]
        assert sum(units[i] for i in got) <= cap and added <= slack + 1e-9
        assert abs(sum(float(weights[i]) for i in got) - (-res.fun)) < 1e-6, n
    extra = list(rng.uniform(0.0, 1.0, 4096))
    weights = list(rng.uniform(0.1, 1.0, 4096).astype(np.float32))
    t0 = time.perf_counter()
    on, added = sp.spear_schedule_ec_costs(extra, weights, 1000.0)
    assert time.perf_counter() - t0 < 2.0 and added <= 1000.0 + 1e-9 and 0 < sum(on) < 4096


@needs_lib
def test_selection_argument_checks():
    with pytest.raises(sp.SpearError):
        sp.spear_schedule_ec_costs([1.0], [-1.0], 5.0)
    with pytest.raises(sp.SpearError):
        sp.spear_schedule_ec_costs([float("nan")], [1.0], 5.0)
    with pytest.raises(sp.SpearError):
        sp.spear_schedule_ec_costs([1.0], [1.0], float("inf"))


STACK = [(2048, 2048, 32), (2048, 2048, 0), (2048, 2048, 0), (2048, 2048, 32),
         (2048, 8192, 0), (2048, 8192, 32), (8192, 2048, 32)]


@needs_lib
def test_cost_model_structure():
    for M in (1, 4, 16, 64, 256, 2048):
        for (K, N, r) in STACK + [(4096, 4096, 32), (4096, 14336, 64), (14336, 4096, 64)]:
            for g in (0, 128):
                p = sp.spear_dispatch_plan(M, K, N, r, 0.0, device_cus=256, group_size=g)
                assert np.isfinite(p.predicted_us) and p.predicted_us > 0
                if r == 0:
                    assert p.predicted_us == p.predicted_no_ec_us
                else:
                    assert p.predicted_us >= p.predicted_no_ec_us
                po = sp.spear_dispatch_plan(M, K, N, r, 0.0, variant="no_ec", device_cus=256, group_size=g)
                assert po.predicted_us == p.predicted_no_ec_us
    # more tokens never predict less time on one kernel family and tile
    prev = 0.0
    for M in (1, 2, 4, 8, 16):
        p = sp.spear_dispatch_plan(M, 4096, 4096, 0, 0.0, device_cus=256)
        assert p.predicted_us >= prev
        prev = p.predicted_us


@needs_lib
def test_schedule_on_the_layer_stack():
    """The small-model stack (EC on q, o, up, down; equal weights): a generous
    SLO keeps every EC, one below the all-off time keeps none, one in between
    keeps a subset whose predicted time fits, and the choice is the selection
    step's on the same plan costs."""
    layers = [(K, N, r, 0, 1.0 if r else 0.0) for (K, N, r) in STACK]
    for M in (8, 256):
        on_all, t_all = sp.spear_schedule_ec(layers, M, 1e9, device_cus=256)
        assert on_all == [r > 0 for (_, _, r) in STACK]
        off = sum(sp.spear_dispatch_plan(M, K, N, r, 0.0, device_cus=256).predicted_no_ec_us for (K, N, r) in STACK)
        on_none, t_none = sp.spear_schedule_ec(layers, M, off * 0.9, device_cus=256)
        assert not any(on_none) and abs(t_none - off) < 1e-3 * off
        slo = off + 0.5 * (t_all - off)
        on_mid, t_mid = sp.spear_schedule_ec(layers, M, slo, device_cus=256)
        assert 0 < sum(on_mid) < 4 and t_mid <= slo + 1e-9
        extra = []
        for (K, N, r) in STACK:
            p = sp.spear_dispatch_plan(M, K, N, r, 0.0, device_cus=256)
            extra.append(max(0.0, float(p.predicted_us) - float(p.predicted_no_ec_us)) if r else -1.0)
        sel, _ = sp.spear_schedule_ec_costs(extra, [l[4] for l in layers], slo - sum(
            float(sp.spear_dispatch_plan(M, K, N, r, 0.0, device_cus=256).predicted_no_ec_us) for (K, N, r) in STACK))
        assert sel == on_mid
