"""GPU parity of the group-wise (g128) W4 variant through the C ABI against
the fp64 oracle: packing bit-exact (codes and scales), the in-register decode
bit-exact on both kernel families, and outputs within relative L2 <= 1e-3 and
max-abs <= 1e-2 rms(Y) over every element on the decode and prefill
workloads and on ragged shapes that reach every tile path."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import w4_gemm_gated_amd as sp

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
G = 128


def note(msg):
    print(f"[gpu-grouped] {msg}", flush=True)


def cuda(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def pack_both(W):
    K, N = W.shape
    Wq_o, s_o = oracle.pack_w4_grouped(W, G)
    Wq_d, s_d = sp.spear_pack_w4_grouped(cuda(W))
    torch.cuda.synchronize()
    return Wq_o, s_o, Wq_d, s_d


@pytest.mark.parametrize("K,N", [(8, 1), (136, 20), (1000, 100), (4096, 4096), (14336, 4096)])
def test_grouped_pack_bit_exact(K, N):
    note(f"grouped pack K={K} N={N}")
    X, W, A, B, w_g = workloads.random_layer(1, K, N, 0, seed=23)
    W[: min(K, 128), 0] = 0.0                       # a group of zeros
    Wq_o, s_o, Wq_d, s_d = pack_both(W)
    s_g = s_d.cpu().numpy()
    assert s_g.shape == (-(-K // 128), -(-N // 16) * 16)
    assert np.array_equal(s_g[:, :N].view(np.uint16), s_o.view(np.uint16))
    assert np.all(s_g[:, N:] == 0)
    assert np.array_equal(Wq_d.cpu().numpy().view(np.uint32), Wq_o)


def run(X, Wq_d, s_d, A, B, w_g, b_g, variant, N, tau=0.0):
    Y = sp.spear_w4ec_linear(cuda(X), Wq_d, s_d, cuda(A), cuda(B), cuda(w_g), b_g, tau, variant, N=N)
    torch.cuda.synchronize()
    return Y.cpu().numpy().astype(np.float64)


def check(Y, X, Wq_o, s_o, A, B, w_g, b_g, K, N, where, tau=0.0):
    Y_ref, info = oracle.w4ec_linear(X, Wq_o, s_o, A, B, w_g, b_g, tau, K=K, N=N, group=G)
    rl, ma = oracle.rel_l2(Y, Y_ref), oracle.max_abs_over_rms(Y, Y_ref)
    note(f"{where}: relL2={rl:.3e} maxabs/rms={ma:.3e}")
    assert np.all(np.isfinite(Y))
    assert rl <= 1e-3 and ma <= 1e-2, where


@pytest.mark.parametrize("M,K,N", [(16, 4096, 4096), (5, 1000, 100), (256, 392, 200), (300, 1000, 100),
                                   (2100, 520, 300)])
def test_grouped_identity_input_is_exact_dequant(M, K, N):
    """One-hot rows of X: Y[i, n] = fp16(q[k_i, n] s[k_i / 128, n]) exactly, on
    the decode kernel (M <= 16: fp32 group sums scaled in fp32) and on the tile
    kernels (fp16 fragments times the fp16 scale, one rounding)."""
    X0, W, A, B, w_g = workloads.random_layer(1, K, N, 0, seed=M + K + N)
    ks = np.resize(np.unique(np.concatenate([[0, K - 1], np.linspace(1, K - 2, M).astype(int)])), M)
    X = np.zeros((M, K), dtype=np.float16)
    X[np.arange(M), ks] = 1.0
    Wq_o, s_o, Wq_d, s_d = pack_both(W)
    Y = run(X, Wq_d, s_d, None, None, None, 0.0, "auto", N)
    expect = oracle.dequant_grouped(Wq_o, s_o, K, N, G)[ks].astype(np.float16).astype(np.float64)
    p = sp.spear_dispatch_plan(M, K, N, 0, 0.0, group_size=G)
    note(f"grouped identity M={M} K={K} N={N}: kernel={p.kernel} tile_m={p.tile_m} split_k={p.split_k}")
    assert np.array_equal(Y, expect)


@pytest.mark.parametrize("variant", ["auto", "split", "no_ec"])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_grouped_decode_workload(M, variant):
    w = workloads.workload(2)
    K, N = w["K"], w["N"]
    Wq_o, s_o, Wq_d, s_d = pack_both(w["W"])
    A, B, w_g = (w["A"], w["B"], w["w_g"]) if variant != "no_ec" else (None, None, None)
    Y = run(w["X"][:M], Wq_d, s_d, A, B, w_g, w["b_g"][M], variant, N)
    check(Y, w["X"][:M], Wq_o, s_o, A, B, w_g, w["b_g"][M], K, N, f"g128 decode M={M} {variant}")


@pytest.mark.parametrize("variant", ["auto", "split", "no_ec"])
def test_grouped_prefill_workload(variant):
    w = workloads.workload(3)
    K, N = w["K"], w["N"]
    Wq_o, s_o, Wq_d, s_d = pack_both(w["W"])
    A, B, w_g = (w["A"], w["B"], w["w_g"]) if variant != "no_ec" else (None, None, None)
    Y = run(w["X"], Wq_d, s_d, A, B, w_g, w["b_g"][2048], variant, N)
    check(Y, w["X"], Wq_o, s_o, A, B, w_g, w["b_g"][2048], K, N, f"g128 prefill M=2048 {variant} (all rows)")


@pytest.mark.parametrize("variant", ["fused", "split"])
@pytest.mark.parametrize("M,K,N,r", [(3, 136, 20, 4), (16, 2056, 4096, 32), (5, 8192, 256, 64), (1, 1000, 100, 20),
                                     (17, 264, 40, 4), (130, 392, 200, 32), (300, 1000, 100, 20),
                                     (520, 2056, 300, 36), (2100, 1000, 7000, 36), (64, 14336, 4096, 64),
                                     (1000, 200, 10750, 64)])
def test_grouped_ragged_shapes(M, K, N, r, variant):
    """K tails (the last group shorter than 128), partial column panels, every
    tile path: decode (local EC and hand-off), 64-row tiles with K split (three
    stages, scales through LDS), 128 x 256 tiles, 256-row tiles, 128 x 448
    tiles (four waves fused, eight waves split)."""
    X, W, A, B, w_g = workloads.random_layer(M, K, N, r, seed=11 * M + K + N + r, outliers=True)
    if variant == "fused" and r % 4 != 0:
        pytest.skip("the fused variant needs rank % 4 == 0")
    Wq_o, s_o, Wq_d, s_d = pack_both(W)
    p = sp.spear_dispatch_plan(M, K, N, r, -0.5, variant=variant, group_size=G)
    note(f"g128 ragged M={M} K={K} N={N} r={r} {variant}: kernel={p.kernel} tile_m={p.tile_m} "
         f"split_k={p.split_k} ec_local={p.ec_local}")
    Y = run(X, Wq_d, s_d, A, B, w_g, -0.5, variant, N)
    check(Y, X, Wq_o, s_o, A, B, w_g, -0.5, K, N, f"g128 ragged M={M} K={K} N={N} r={r} {variant}")


def test_grouped_layer_stack_down_proj():
    lay = workloads.stack_layer(6)
    K, N = lay["K"], lay["N"]
    Wq_o, s_o, Wq_d, s_d = pack_both(lay["W"])
    Y = run(lay["X"], Wq_d, s_d, lay["A"], lay["B"], lay["w_g"], 0.0, "auto", N)
    check(Y, lay["X"], Wq_o, s_o, lay["A"], lay["B"], lay["w_g"], 0.0, K, N, "g128 stack down_proj")
