"""GPU parity of the data-free EC initialisation (spear_ec_init) against the
fp64 oracle (rank-r truncated SVD of the quantization residual).

Where the residual's spectrum has a gap after r, A B is unique and the GPU's
fp16 factors are compared with the oracle's element by element: relative L2
of A B <= 2e-3 (the fp16 rounding of A and B alone gives about 7e-4; the
subspace iteration converges as (s_{r+16} / s_r)^(2 iterations + 1)), and A and
B themselves (their sign convention fixed) <= 2e-3.  On real quantization
residuals, whose spectrum is nearly flat at the top, A B is not unique; there
the bar is Eckart-Young's: the captured energy and the remaining error within
1 % of the optimum, and a smaller output error at gate 1."""
import numpy as np
import pytest
import torch

import oracle
from oracle import spear_ec_init as eci
import workloads
import w4_gemm_gated_amd as sp

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def note(msg):
    print(f"[gpu-ec-init] {msg}", flush=True)


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_factors(W, Wq, s, r, iterations=0):
    A, B = sp.spear_ec_init(cuda(W), cuda(Wq.view(np.uint8)), cuda(s), r, iterations)
    torch.cuda.synchronize()
    return A.cpu().numpy().astype(np.float64), B.cpu().numpy().astype(np.float64)


def gapped_weight(K, N, r, seed, group=None):
    """W = fp16(dequant(Wq0, s0) + U diag(sigma) V^T + small noise), with
    sigma_1..r in [2e-3, 4e-3] and the tail below 6e-4 (a gap of 3 or more):
    the residual W - dequant(Wq0, s0) then has a unique rank-r truncation."""
    rng = np.random.default_rng(seed)
    W0 = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    Wq0, s0 = oracle.pack_w4(W0) if group is None else oracle.pack_w4_grouped(W0, group)
    base = oracle.dequant(Wq0, s0, K, N) if group is None else oracle.dequant_grouped(Wq0, s0, K, N, group)
    U = np.linalg.qr(rng.standard_normal((K, r)))[0]
    V = np.linalg.qr(rng.standard_normal((N, r)))[0]
    sig = np.linspace(4e-3, 2e-3, r) * np.sqrt(K * N) / 8
    low = U @ np.diag(sig) @ V.T
    noise = rng.standard_normal((K, N)) * 6e-4 * np.sqrt(K * N) / 8 / np.sqrt(max(K, N)) / 4
    W = (base + low + noise).astype(np.float16)
    return W, Wq0, s0


@pytest.mark.parametrize("K,N,r,group", [(512, 512, 16, None), (1024, 768, 32, None), (768, 1024, 8, 128),
                                         (2048, 2048, 64, None), (264, 200, 4, None)])
def test_gapped_residual_matches_oracle(K, N, r, group):
    W, Wq, s = gapped_weight(K, N, r, seed=K + N + r, group=group)
    A_o, B_o, S = eci.ec_init(W, Wq, s, r, K, N, group)
    assert S[r - 1] > 2.5 * S[r]
    A, B = gpu_factors(W, Wq, s, r)
    rl = oracle.rel_l2(A @ B, A_o @ B_o)
    ra, rb = oracle.rel_l2(A, A_o), oracle.rel_l2(B, B_o)
    note(f"gapped K={K} N={N} r={r} group={group}: relL2 AB={rl:.2e} A={ra:.2e} B={rb:.2e} "
         f"gap s_r/s_r+1={S[r - 1] / S[r]:.2f}")
    assert rl <= 2e-3 and ra <= 2e-3 and rb <= 2e-3


@pytest.mark.parametrize("which", ["tiny", "stack_q_proj", "decode_q_proj_4096"])
def test_quantization_residual_is_near_optimal(which):
    if which == "tiny":
        w = workloads.workload(1)
        W, r = w["W"], 16
    elif which == "stack_q_proj":
        w = workloads.stack_layer(0)
        W, r = w["W"], 32
    else:
        w = workloads.workload(2)
        W, r = w["W"], 32
    K, N = W.shape
    Wq, s = oracle.pack_w4(W)
    E = eci.residual(W, Wq, s, K, N)
    S = np.linalg.svd(E, compute_uv=False)
    A, B = gpu_factors(W, Wq, s, r)
    top, tail = np.sum(S[:r] ** 2), np.sum(S[r:] ** 2)
    got = np.linalg.norm(A @ B) ** 2
    err = np.linalg.norm(E - A @ B) ** 2
    note(f"{which} K={K} N={N} r={r}: captured {got / top:.4f} of the optimum, residual error "
         f"{err / tail:.5f} of the optimum; s_r/s_r+1={S[r - 1] / S[r]:.3f}")
    # A B = E V V^T is a projection, so captured + remaining = ||E||^2 and a
    # shortfall of the captured energy equals the remaining error's excess: with
    # a flat spectrum the top-r energy is a few percent of the tail, so 1 % on
    # the error (the Eckart-Young bar) allows a few percent on the energy.
    assert err <= 1.01 * tail
    assert got >= 0.95 * top
    assert abs((top - got) - (err - tail)) <= 1e-3 * (top + tail)
    X = w["X"][:16].astype(np.float64)
    assert np.linalg.norm(X @ (E - A @ B)) < np.linalg.norm(X @ E)


def test_grid_weight_gives_zero_factors():
    rng = np.random.default_rng(7)
    K, N = 256, 128
    q = rng.integers(-7, 8, size=(K, N))
    q[0, :] = 7
    W = (q * np.power(2.0, rng.integers(-10, -5, size=N))[None, :]).astype(np.float16)
    Wq, s = oracle.pack_w4(W)
    A, B = gpu_factors(W, Wq, s, 8)
    assert np.all(np.isfinite(A)) and np.all(np.isfinite(B))
    assert not np.any(A @ B)
