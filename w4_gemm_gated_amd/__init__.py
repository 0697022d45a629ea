"""MI355X (gfx950) W4 linear layer with a per-token-gated low-rank Error
Compensator, after "SPEAR: A System for Post-Quantization Error-Adaptive
Recovery Enabling Efficient Low-Bit LLM Serving" (arXiv 2606.11244), Abstract.

    Y = X . dequant(Wq, s) + g' (.) ((X . A) . B),   g = sigmoid(X . w_g + b_g)

Python names mirror the C ABI in include/spear_w4ec.h.  This module only
marshals arguments: tensors must already live on the GPU, every step runs in
the HIP kernels of libspear_w4ec.so, and PyTorch supplies memory and the
current stream.
"""
import ctypes

import torch

from . import _binding
from ._binding import LinearDesc, Plan, SpearError, VARIANTS, EXPORTS  # noqa: F401

__all__ = [
    "spear_packed_bytes",
    "spear_pack_w4",
    "spear_dispatch_plan",
    "spear_w4ec_linear",
    "spear_ec_project",
    "spear_debug_unpack_w4",
    "spear_abi_version",
    "library",
    "SpearError",
]


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _binding.load()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, dims=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions")


def spear_abi_version():
    return int(library().spear_abi_version())


def spear_packed_bytes(K, N):
    out = ctypes.c_size_t(0)
    _binding.check(library().spear_packed_bytes(int(K), int(N), ctypes.byref(out)), "spear_packed_bytes")
    return int(out.value)


def spear_pack_w4(W):
    """W fp16 [K, N] on the GPU -> (Wq uint8 [packed bytes], scales fp16 [N])."""
    _need(W, "W", torch.float16, 2)
    K, N = W.shape
    Wq = torch.empty(spear_packed_bytes(K, N), dtype=torch.uint8, device=W.device)
    s = torch.empty(N, dtype=torch.float16, device=W.device)
    st = library().spear_pack_w4(_ptr(W), K, N, _ptr(Wq), _ptr(s), _stream(W.device))
    _binding.check(st, "spear_pack_w4")
    return Wq, s


def spear_debug_unpack_w4(Wq, K, N):
    """Packed weight -> int8 codes q [K, N] (same decode as the GEMM kernels)."""
    _need(Wq, "Wq", torch.uint8, 1)
    q = torch.empty((K, N), dtype=torch.int8, device=Wq.device)
    st = library().spear_debug_unpack_w4(_ptr(Wq), int(K), int(N), _ptr(q), _stream(Wq.device))
    _binding.check(st, "spear_debug_unpack_w4")
    return q


def _desc(M, K, N, rank, gate_bias, skip_tau, variant, device_cus):
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    return LinearDesc(int(M), int(K), int(N), int(rank), float(gate_bias), float(skip_tau), v, int(device_cus))


def spear_dispatch_plan(M, K, N, rank, gate_bias=0.0, skip_tau=0.0, variant="auto", device_cus=0):
    """Plan a call; returns the Plan structure (see Plan.as_dict())."""
    d = _desc(M, K, N, rank, gate_bias, skip_tau, variant, device_cus)
    p = Plan()
    _binding.check(library().spear_dispatch_plan(ctypes.byref(d), ctypes.byref(p)), "spear_dispatch_plan")
    return p


# Zero-filled workspaces, one per (device, stream); every call leaves its
# workspace zero-filled, so they are reused as they are.
_workspaces = {}


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    dev = torch.device(device)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def spear_w4ec_linear(X, Wq, scales, A, B, w_g, gate_bias, skip_tau=0.0, variant="auto",
                      N=None, plan=None, Y=None, workspace=None):
    """Y fp16 [M, N] = X . dequant(Wq, s) + g' (.) ((X . A) . B).

    X fp16 [M, K]; Wq/scales from spear_pack_w4; A fp16 [K, r]; B fp16 [r, N];
    w_g fp16 [K].  A, B, w_g may be None (rank 0).  `plan` may come from
    spear_dispatch_plan for the same shape; `workspace` (uint8, zero-filled
    before first use) defaults to a cached one for the current stream.
    """
    _need(X, "X", torch.float16, 2)
    _need(Wq, "Wq", torch.uint8, 1)
    _need(scales, "scales", torch.float16, 1)
    M, K = X.shape
    N = scales.shape[0] if N is None else int(N)
    rank = 0
    if A is not None:
        _need(A, "A", torch.float16, 2)
        _need(B, "B", torch.float16, 2)
        _need(w_g, "w_g", torch.float16, 1)
        rank = A.shape[1]
        if A.shape[0] != K or B.shape != (rank, N) or w_g.shape[0] != K:
            raise ValueError("EC shapes must be A [K, r], B [r, N], w_g [K]")
    if Wq.numel() != spear_packed_bytes(K, N):
        raise ValueError("Wq size does not match K and N")
    d = _desc(M, K, N, rank, gate_bias, skip_tau, variant, 0)
    if plan is None:
        plan = Plan()
        _binding.check(library().spear_dispatch_plan(ctypes.byref(d), ctypes.byref(plan)),
                       "spear_dispatch_plan")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    else:
        _need(Y, "Y", torch.float16, 2)
    if workspace is None:
        workspace = _workspace(plan.workspace_bytes, X.device)
    ws_bytes = workspace.numel() if workspace is not None else 0
    st = library().spear_w4ec_linear(ctypes.byref(d), ctypes.byref(plan), _ptr(X), _ptr(Wq), _ptr(scales),
                                     _ptr(A), _ptr(B), _ptr(w_g), _ptr(Y), _ptr(workspace), ws_bytes,
                                     _stream(X.device))
    _binding.check(st, "spear_w4ec_linear")
    return Y


def spear_ec_project(X, A, w_g, gate_bias, skip_tau=0.0):
    """(P fp32 [M, r], g' fp32 [M]) = EC projection and gate in one pass over X."""
    _need(X, "X", torch.float16, 2)
    _need(A, "A", torch.float16, 2)
    _need(w_g, "w_g", torch.float16, 1)
    M, K = X.shape
    rank = A.shape[1]
    nb = ctypes.c_size_t(0)
    _binding.check(library().spear_ec_workspace_bytes(M, K, rank, ctypes.byref(nb)), "spear_ec_workspace_bytes")
    ws = _workspace(int(nb.value), X.device)
    P = torch.empty((M, rank), dtype=torch.float32, device=X.device)
    g = torch.empty(M, dtype=torch.float32, device=X.device)
    st = library().spear_ec_project(M, K, rank, _ptr(X), _ptr(A), _ptr(w_g), float(gate_bias), float(skip_tau),
                                    _ptr(P), _ptr(g), _ptr(ws), ws.numel() if ws is not None else 0,
                                    _stream(X.device))
    _binding.check(st, "spear_ec_project")
    return P, g
