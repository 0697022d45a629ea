"""The allocation-free entry point (spear_w4ec_linear_noalloc) through the C
ABI, against the workspace entry point (spear_w4ec_linear) on the same inputs
and plans: identical bits (same kernels, fixed-order sums), and within the
oracle's bar.  Two calls in a row on the shared device array, the second with
a smaller input; a plan beyond the array's size is refused before anything is
enqueued."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import w4_gemm_gated_amd as sp

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def note(msg):
    print(f"[no-alloc] {msg}", flush=True)


def cuda(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def case(M, K, N, r, b_g, variant, seed):
    X, W, A, B, w_g = workloads.random_layer(M, K, N, r, seed=seed, outliers=True)
    Wq_d, s_d = sp.spear_pack_w4(cuda(W))
    args = (cuda(X), Wq_d, s_d, cuda(A), cuda(B), cuda(w_g), b_g)
    p = sp.spear_dispatch_plan(M, K, N, r, b_g, variant=variant)
    note(f"M={M} K={K} N={N} r={r} {variant}: variant={p.variant} kernel={p.kernel} "
         f"workspace={p.workspace_bytes} B")
    Y_ws = sp.spear_w4ec_linear(*args, variant=variant, N=N, plan=p).clone()
    Y_na = sp.spear_w4ec_linear_noalloc(*args, variant=variant, N=N, plan=p)
    torch.cuda.synchronize()
    assert torch.equal(Y_ws, Y_na), "no-alloc output differs from the workspace entry point"
    Wq_o, s_o = oracle.pack_w4(W)
    Y_ref, _ = oracle.w4ec_linear(X, Wq_o, s_o, A, B, w_g, b_g, 0.0, K=K, N=N)
    Yg = Y_na.cpu().numpy().astype(np.float64)
    assert oracle.rel_l2(Yg, Y_ref) <= 1e-3 and oracle.max_abs_over_rms(Yg, Y_ref) <= 1e-2
    return p


@pytest.mark.parametrize("first,second", [
    # large fused tiled call (mid M, K split), then a decode call with the hand-off
    ((512, 14336, 4096, 64, -5.9, "fused"), (16, 4096, 4096, 32, -1.0, "fused")),
    # split variant, then a smaller split call
    ((300, 1000, 100, 20, -0.5, "split"), (17, 264, 40, 4, -0.5, "split")),
    # decode hand-off (K split), then the tiny workload's shape
    ((5, 8192, 256, 64, 0.3, "auto"), (3, 136, 20, 4, 0.3, "auto")),
])
def test_noalloc_matches_workspace_entry_two_calls(first, second):
    p1 = case(*first, seed=sum(first[:4]))
    p2 = case(*second, seed=sum(second[:4]) + 1)
    assert p2.workspace_bytes <= p1.workspace_bytes
    assert sp.spear_take_error_noalloc() == 0


def test_noalloc_refuses_a_plan_beyond_its_array():
    M, K, N, r = 65536, 256, 64, 256
    p = sp.spear_dispatch_plan(M, K, N, r, 0.0, variant="split")
    assert p.workspace_bytes > 64 << 20
    X = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    Wq = torch.zeros(sp.spear_packed_bytes(K, N), dtype=torch.uint8, device=DEV)
    s = torch.zeros(N, dtype=torch.float16, device=DEV)
    A = torch.zeros((K, r), dtype=torch.float16, device=DEV)
    B = torch.zeros((r, N), dtype=torch.float16, device=DEV)
    wg = torch.zeros(K, dtype=torch.float16, device=DEV)
    with pytest.raises(sp.SpearError) as ei:
        sp.spear_w4ec_linear_noalloc(X, Wq, s, A, B, wg, 0.0, variant="split", N=N, plan=p)
    assert ei.value.status == 5
