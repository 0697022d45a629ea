"""Seeded synthetic inputs for the W4+EC linear layer (shared by tests and bench).

This module only draws random numbers and casts them to fp16; it holds none of
the layer's arithmetic.  Shapes follow Llama-class linear layers; values are
synthetic (no dataset or checkpoint is used or needed).

Recipe (the same for every workload):
  * generator: numpy ``default_rng(SeedSequence([seed, workload_id, tensor_id]))``
    (``[seed, 5, layer, tensor_id]`` for the layer stack), tensor ids
    X=0, W=1, A=2, B=3, w_g=4, outlier channels=5;
  * values are drawn in float64 as standard normals times the stated standard
    deviation and rounded to fp16 (round to nearest even);
  * X ~ N(0, 1); W ~ N(0, 0.02); A, B ~ N(0, 0.01); w_g ~ N(0, 0.05)
    (second parameter = standard deviation);
  * outliers: round(0.01 K) distinct input channels, drawn without
    replacement, are multiplied by 20 before the fp16 cast;
  * X is drawn at the largest token count of a workload; smaller token counts
    take the leading rows.
"""

import json
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_REPO = os.path.dirname(_HERE)
GATE_BIAS_FILE = os.path.join(_REPO, "tests", "golden", "downproj_gate_bias.json")

X_ID, W_ID, A_ID, B_ID, WG_ID, OUTLIER_ID = range(6)

STD_X, STD_W, STD_AB, STD_WG = 1.0, 0.02, 0.01, 0.05

# Workload table.  ``ms`` lists the token counts; ``taus`` the skip thresholds.
WORKLOADS = {
    1: dict(name="tiny", ms=(16,), K=512, N=512, r=16, outliers=False, b_g=0.0, taus=(0.0,)),
    2: dict(name="decode_q_proj_4096x4096", ms=(1, 4, 16), K=4096, N=4096, r=32,
            outliers=True, b_g=-1.0, taus=(0.0,)),
    3: dict(name="prefill_up_proj_4096x14336", ms=(2048,), K=4096, N=14336, r=64,
            outliers=True, b_g=0.0, taus=(0.0,)),
    4: dict(name="mixed_gate_down_proj_14336x4096", ms=(64, 512), K=14336, N=4096, r=64,
            outliers=False, b_g=None, taus=(0.0, 0.05)),
}

# Small-model layer stack: hidden 2048, intermediate 8192, 16 heads of 128
# (k and v as wide as q: no grouped-query sharing is stated), 256 tokens from
# 8 requests; ECs of rank 32 on q, o, up and down only.
STACK_HIDDEN, STACK_INTER, STACK_TOKENS = 2048, 8192, 256
STACK_REQUESTS = (96, 64, 40, 24, 16, 8, 6, 2)
STACK_LAYERS = (
    ("q_proj", 2048, 2048, 32),
    ("k_proj", 2048, 2048, 0),
    ("v_proj", 2048, 2048, 0),
    ("o_proj", 2048, 2048, 32),
    ("gate_proj", 2048, 8192, 0),
    ("up_proj", 2048, 8192, 32),
    ("down_proj", 8192, 2048, 32),
)


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def _normal16(rng, shape, std):
    return (rng.standard_normal(shape) * std).astype(np.float16)


def draw(key, M, K, N, r, outliers=False):
    """Draw (X, W, A, B, w_g) for a layer; ``key`` is the SeedSequence prefix."""
    x = _rng(*key, X_ID).standard_normal((M, K)) * STD_X
    if outliers:
        idx = _rng(*key, OUTLIER_ID).choice(K, int(round(0.01 * K)), replace=False)
        x[:, idx] *= 20.0
    X = x.astype(np.float16)
    W = _normal16(_rng(*key, W_ID), (K, N), STD_W)
    if r > 0:
        A = _normal16(_rng(*key, A_ID), (K, r), STD_AB)
        B = _normal16(_rng(*key, B_ID), (r, N), STD_AB)
        w_g = _normal16(_rng(*key, WG_ID), (K,), STD_WG)
    else:
        A = B = w_g = None
    return X, W, A, B, w_g


def gate_bias_table():
    """Stored gate biases of the mixed-gate down_proj workload, keyed by M."""
    with open(GATE_BIAS_FILE) as f:
        data = json.load(f)
    return {int(k): float(v) for k, v in data["b_g"].items()}


def workload(wid, seed=0):
    """Inputs of workload ``wid`` (1..4) at its largest token count.

    Returns a dict with X [M_max, K], W, A, B, w_g (fp16 numpy), and K, N, r,
    ms, taus, name, b_g (a dict M -> float32 bias).
    """
    spec = WORKLOADS[wid]
    M = max(spec["ms"])
    X, W, A, B, w_g = draw((seed, wid), M, spec["K"], spec["N"], spec["r"], spec["outliers"])
    if spec["b_g"] is None:
        table = gate_bias_table() if seed == 0 else {}
        b_g = {m: table.get(m) for m in spec["ms"]}
    else:
        b_g = {m: float(np.float32(spec["b_g"])) for m in spec["ms"]}
    out = dict(spec)
    out.update(X=X, W=W, A=A, B=B, w_g=w_g, b_g=b_g)
    return out


def stack_layer(index, seed=0, tokens=STACK_TOKENS):
    """Inputs of layer ``index`` (0..6) of the small-model stack."""
    name, K, N, r = STACK_LAYERS[index]
    X, W, A, B, w_g = draw((seed, 5, index), tokens, K, N, r, False)
    return dict(name=name, K=K, N=N, r=r, ms=(tokens,), taus=(0.0,), b_g={tokens: 0.0},
                X=X, W=W, A=A, B=B, w_g=w_g, requests=STACK_REQUESTS)


def random_layer(M, K, N, r, seed, outliers=False):
    """Arbitrary-shape layer with the same distributions (parity and edge cases)."""
    return draw((seed, 1000 + M, K, N, r), M, K, N, r, outliers)


# --------------------------------------------------------------------------
# Accounting used by the benchmark (algorithmic bytes and flops of one call).
# Bytes: K N / 2 (Wq) + 2 N (s) + 2 M K (X) + 2 M N (Y) + [2 r (K + N) (A, B)
# + 2 K (w_g) when the EC is on].  Flops: 2 M K N + [2 M (K (r + 1) + r N)].
# --------------------------------------------------------------------------

def algorithmic_bytes(M, K, N, r):
    b = K * N // 2 + 2 * N + 2 * M * K + 2 * M * N
    if r > 0:
        b += 2 * r * (K + N) + 2 * K
    return b


def algorithmic_flops(M, K, N, r):
    main = 2 * M * K * N
    ec = 2 * M * (K * (r + 1) + r * N) if r > 0 else 0
    return main, ec
