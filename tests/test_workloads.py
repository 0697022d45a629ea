"""Seeded synthetic workloads: determinism, shapes, stated distributions and
the stored gate bias of the mixed-gate down_proj workload (CPU only)."""
import json
import math
import os
import sys

import numpy as np
import pytest

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def test_determinism_and_prefix_rows():
    a = workloads.draw((0, 2), 16, 256, 64, 8, outliers=True)
    b = workloads.draw((0, 2), 16, 256, 64, 8, outliers=True)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()
    c = workloads.draw((1, 2), 16, 256, 64, 8, outliers=True)
    assert a[1].tobytes() != c[1].tobytes()


def test_decode_workload_shapes_and_outliers():
    w = workloads.workload(2)
    assert w["X"].shape == (16, 4096) and w["W"].shape == (4096, 4096)
    assert w["A"].shape == (4096, 32) and w["B"].shape == (32, 4096) and w["w_g"].shape == (4096,)
    assert all(t.dtype == np.float16 for t in (w["X"], w["W"], w["A"], w["B"], w["w_g"]))
    col_rms = np.sqrt(np.mean(w["X"].astype(np.float64) ** 2, axis=0))
    assert int(np.sum(col_rms > 8.0)) == 41          # round(0.01 * 4096) channels x 20
    assert w["b_g"] == {1: -1.0, 4: -1.0, 16: -1.0}
    assert abs(np.std(w["W"].astype(np.float64)) - 0.02) < 0.0005


def test_tiny_workload_moments():
    w = workloads.workload(1)
    assert abs(np.std(w["X"].astype(np.float64)) - 1.0) < 0.02
    assert abs(np.std(w["A"].astype(np.float64)) - 0.01) < 0.0005
    assert abs(np.std(w["w_g"].astype(np.float64)) - 0.05) < 0.005


def test_stack_layers():
    assert sum(workloads.STACK_REQUESTS) == workloads.STACK_TOKENS == 256
    ranks = [l[3] for l in workloads.STACK_LAYERS]
    assert sum(1 for r in ranks if r > 0) == 4
    lay = workloads.stack_layer(6)
    assert lay["X"].shape == (256, 8192) and lay["W"].shape == (8192, 2048)
    lay = workloads.stack_layer(1)
    assert lay["A"] is None and lay["r"] == 0


@pytest.mark.slow
def test_stored_gate_bias_reproduces_and_splits_70_percent():
    sys.path.insert(0, os.path.join(HERE, "golden"))
    import make_gate_bias
    b, margins = make_gate_bias.compute()
    stored = workloads.gate_bias_table()
    assert {int(k): v for k, v in b.items()} == stored
    w = workloads.workload(4)
    for M, expect in ((64, 45), (512, 359)):
        z = oracle.gate_logits(w["X"][:M], w["w_g"], stored[M])
        g, g_eff, amb = oracle.gate(z, 0.05)
        assert int(np.sum(g < 0.05)) == expect == math.ceil(0.7 * M)
        assert not amb.any()
        assert margins[str(M)] > 1e-3


def test_accounting_formulas():
    # tiny workload: 198,656 bytes with the EC, 164,864 without
    assert workloads.algorithmic_bytes(16, 512, 512, 16) == 198656
    assert workloads.algorithmic_bytes(16, 512, 512, 0) == 164864
    main, ec = workloads.algorithmic_flops(2048, 4096, 14336, 64)
    assert main == 2 * 2048 * 4096 * 14336 and ec == 2 * 2048 * (4096 * 65 + 64 * 14336)
