"""Data-free initialisation of the Error Compensator (test infrastructure only).

Sources: the SPEAR page, Abstract ("lightweight Error Compensators" that
recover the quantization error), and, for how such a low-rank compensator is
set up without data, the page "SERQ: Saliency-Aware Low-Rank Error
Reconstruction for LLM Quantization", Figure 1 (a low-rank reconstruction of
the quantization error from its singular value decomposition) and Table 8
(the quality of that decomposition at ranks 128 / 64 / 32).

Reading taken here: with E = W - dequant(Wq, s) the residual of the 4-bit
weight (float64, exact), A B is the rank-r truncated SVD of E, the best rank-r
approximation in the Frobenius norm (Eckart-Young), and the singular values
are split evenly between the factors: A = U_r diag(sqrt(sigma_r)),
B = diag(sqrt(sigma_r)) V_r^T.  The product A B is unique when
sigma_r > sigma_{r+1}; the split is a convention (A^T A = B B^T =
diag(sigma_r)), and each singular pair's sign is fixed so the largest-magnitude
entry of the column of U is positive.

Library primitive used as a step: numpy.linalg.svd (float64).
"""

import numpy as np

from .spear_oracle import dequant, dequant_grouped


def residual(W, Wq, s, K, N, group=None):
    """E [K, N] float64 = W - dequant(Wq, s)."""
    Wd = dequant(Wq, s, K, N) if group is None else dequant_grouped(Wq, s, K, N, group)
    return np.asarray(W, dtype=np.float16).astype(np.float64) - Wd


def truncated_svd_factors(E, rank):
    """(A [K, r], B [r, N], sigma [min(K, N)]) of the rank-r truncated SVD of E."""
    U, S, Vt = np.linalg.svd(np.asarray(E, dtype=np.float64), full_matrices=False)
    U, S, Vt = U[:, :rank].copy(), S, Vt[:rank].copy()
    for j in range(rank):
        i = int(np.argmax(np.abs(U[:, j])))
        if U[i, j] < 0:
            U[:, j] = -U[:, j]
            Vt[j] = -Vt[j]
    root = np.sqrt(S[:rank])
    return U * root[None, :], root[:, None] * Vt, S


def ec_init(W, Wq, s, rank, K=None, N=None, group=None):
    """(A, B, sigma): the EC factors of the weight's quantization residual."""
    W = np.asarray(W, dtype=np.float16)
    K = W.shape[0] if K is None else K
    N = W.shape[1] if N is None else N
    return truncated_svd_factors(residual(W, Wq, s, K, N, group), rank)
