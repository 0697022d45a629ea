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
    "spear_pack_w4_grouped",
    "spear_dispatch_plan",
    "spear_schedule_ec",
    "spear_schedule_ec_costs",
    "spear_w4ec_linear",
    "spear_ec_project",
    "spear_debug_unpack_w4",
    "spear_ec_init",
    "spear_abi_version",
    "spear_take_error",
    "spear_w4ec_linear_noalloc",
    "spear_debug_set_spin_limit",
    "spear_debug_fail_waits",
    "spear_debug_stream_read",
    "spear_debug_mfma_rate",
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


def _need(t, name, dtype, dims=None):  # noqa: D401 - argument check
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


def spear_pack_w4_grouped(W, group_size=128):
    """W fp16 [K, N] on the GPU -> (Wq uint8 [packed bytes], scales fp16
    [ceil(K/128), N rounded up to 16]; columns >= N hold 0)."""
    _need(W, "W", torch.float16, 2)
    K, N = W.shape
    Wq = torch.empty(spear_packed_bytes(K, N), dtype=torch.uint8, device=W.device)
    s = torch.empty((-(-K // 128), -(-N // 16) * 16), dtype=torch.float16, device=W.device)
    st = library().spear_pack_w4_grouped(_ptr(W), K, N, int(group_size), _ptr(Wq), _ptr(s), _stream(W.device))
    _binding.check(st, "spear_pack_w4_grouped")
    return Wq, s


def spear_ec_init(W, Wq, scales, rank, iterations=0):
    """(A fp16 [K, r], B fp16 [r, N]): the rank-r truncated SVD of W's
    quantization residual, on the GPU.  scales 1-D: per channel; 2-D: the
    group scales of spear_pack_w4_grouped."""
    _need(W, "W", torch.float16, 2)
    _need(Wq, "Wq", torch.uint8, 1)
    K, N = W.shape
    group = 0 if scales.dim() == 1 else 128
    nb = ctypes.c_size_t(0)
    _binding.check(library().spear_ec_init_workspace_bytes(K, N, int(rank), ctypes.byref(nb)),
                   "spear_ec_init_workspace_bytes")
    ws = torch.empty(int(nb.value), dtype=torch.uint8, device=W.device)
    A = torch.empty((K, rank), dtype=torch.float16, device=W.device)
    B = torch.empty((rank, N), dtype=torch.float16, device=W.device)
    st = library().spear_ec_init(_ptr(W), _ptr(Wq), _ptr(scales), K, N, group, int(rank), int(iterations), _ptr(A),
                                 _ptr(B), _ptr(ws), ws.numel(), _stream(W.device))
    _binding.check(st, "spear_ec_init")
    return A, B


def spear_debug_unpack_w4(Wq, K, N):
    """Packed weight -> int8 codes q [K, N] (same decode as the GEMM kernels)."""
    _need(Wq, "Wq", torch.uint8, 1)
    q = torch.empty((K, N), dtype=torch.int8, device=Wq.device)
    st = library().spear_debug_unpack_w4(_ptr(Wq), int(K), int(N), _ptr(q), _stream(Wq.device))
    _binding.check(st, "spear_debug_unpack_w4")
    return q


def _desc(M, K, N, rank, gate_bias, skip_tau, variant, device_cus, group_size=0):
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    return LinearDesc(int(M), int(K), int(N), int(rank), float(gate_bias), float(skip_tau), v, int(device_cus),
                      int(group_size))


def spear_dispatch_plan(M, K, N, rank, gate_bias=0.0, skip_tau=0.0, variant="auto", device_cus=0, group_size=0):
    """Plan a call; returns the Plan structure (see Plan.as_dict())."""
    d = _desc(M, K, N, rank, gate_bias, skip_tau, variant, device_cus, group_size)
    p = Plan()
    _binding.check(library().spear_dispatch_plan(ctypes.byref(d), ctypes.byref(p)), "spear_dispatch_plan")
    return p


def spear_schedule_ec(layers, M, slo_us, device_cus=0):
    """layers: sequence of (K, N, rank, group_size, weight).  Returns (ec_on
    list of bools, predicted batch latency in us) for a batch of M tokens."""
    n = len(layers)
    arr = (_binding.SchedLayer * max(n, 1))()
    for i, (K, N, r, g, wt) in enumerate(layers):
        arr[i] = _binding.SchedLayer(int(K), int(N), int(r), int(g), float(wt))
    on = (ctypes.c_uint8 * max(n, 1))()
    pred = ctypes.c_double(0.0)
    st = library().spear_schedule_ec(arr, n, int(M), float(slo_us), int(device_cus), on, ctypes.byref(pred))
    _binding.check(st, "spear_schedule_ec")
    return [bool(on[i]) for i in range(n)], float(pred.value)


def spear_schedule_ec_costs(extra_us, weights, slack_us):
    """The scheduler's selection step on given costs: (ec_on list, added us)."""
    n = len(extra_us)
    ex = (ctypes.c_double * max(n, 1))(*[float(x) for x in extra_us])
    wt = (ctypes.c_float * max(n, 1))(*[float(x) for x in weights])
    on = (ctypes.c_uint8 * max(n, 1))()
    added = ctypes.c_double(0.0)
    st = library().spear_schedule_ec_costs(ex, wt, n, float(slack_us), on, ctypes.byref(added))
    _binding.check(st, "spear_schedule_ec_costs")
    return [bool(on[i]) for i in range(n)], float(added.value)


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


def _scales_shape(scales, K, N):
    """(N, group_size) from the scale tensor: [N] per channel, or the group
    scales [ceil(K/128), N_pad] of spear_pack_w4_grouped (N then required)."""
    _need(scales, "scales", torch.float16)
    if scales.dim() == 1:
        return (scales.shape[0] if N is None else int(N)), 0
    if N is None:
        raise ValueError("N must be given with group scales")
    N = int(N)
    if scales.dim() != 2 or scales.shape != (-(-K // 128), -(-N // 16) * 16):
        raise ValueError("group scales must be [ceil(K/128), N rounded up to 16]")
    return N, 128


def spear_w4ec_linear(X, Wq, scales, A, B, w_g, gate_bias, skip_tau=0.0, variant="auto",
                      N=None, plan=None, Y=None, workspace=None):
    """Y fp16 [M, N] = X . dequant(Wq, s) + g' (.) ((X . A) . B).

    X fp16 [M, K]; Wq/scales from spear_pack_w4 (scales [N]) or
    spear_pack_w4_grouped (scales [ceil(K/128), N_pad]; N required); A fp16
    [K, r]; B fp16 [r, N]; w_g fp16 [K].  A, B, w_g may be None (rank 0).
    `plan` may come from spear_dispatch_plan for the same shape; `workspace`
    (uint8, zero-filled before first use) defaults to a cached one for the
    current stream.
    """
    _need(X, "X", torch.float16, 2)
    _need(Wq, "Wq", torch.uint8, 1)
    M, K = X.shape
    N, group = _scales_shape(scales, K, N)
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
    d = _desc(M, K, N, rank, gate_bias, skip_tau, variant, 0, group)
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


def spear_w4ec_linear_noalloc(X, Wq, scales, A, B, w_g, gate_bias, skip_tau=0.0, variant="auto", N=None,
                              plan=None, Y=None):
    """spear_w4ec_linear on the library's own device workspace (no workspace
    argument; the library call allocates nothing).  Y is allocated here when
    not given."""
    _need(X, "X", torch.float16, 2)
    _need(Wq, "Wq", torch.uint8, 1)
    M, K = X.shape
    N, group = _scales_shape(scales, K, N)
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
    d = _desc(M, K, N, rank, gate_bias, skip_tau, variant, 0, group)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    else:
        _need(Y, "Y", torch.float16, 2)
    st = library().spear_w4ec_linear_noalloc(ctypes.byref(d), ctypes.byref(plan) if plan is not None else None,
                                             _ptr(X), _ptr(Wq), _ptr(scales), _ptr(A), _ptr(B), _ptr(w_g),
                                             _ptr(Y), _stream(X.device))
    _binding.check(st, "spear_w4ec_linear_noalloc")
    return Y


def spear_take_error_noalloc(device=None):
    """Read and clear the sticky error word of the allocation-free entry
    point's workspace on the current device; synchronizes the stream."""
    dev = torch.device(device if device is not None else "cuda")
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    st = library().spear_take_error(None, 0, _ptr(out), _stream(dev))
    _binding.check(st, "spear_take_error")
    return int(out.item()) & 0xFFFFFFFF


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


def spear_take_error(workspace=None, device=None):
    """Read and clear the sticky error word of a workspace (the cached one of
    the current stream when None); synchronizes the current stream.  Returns
    0, or the bits of the waits that gave up (1: fused decode hand-off, 2:
    fused tiled ready flag)."""
    if workspace is None:
        dev = torch.device(device if device is not None else "cuda")
        key = (dev.index if dev.index is not None else torch.cuda.current_device(),
               torch.cuda.current_stream(dev).cuda_stream)
        workspace = _workspaces.get(key)
        if workspace is None:
            return 0
    _need(workspace, "workspace", torch.uint8, 1)
    out = torch.zeros(1, dtype=torch.int32, device=workspace.device)
    st = library().spear_take_error(_ptr(workspace), workspace.numel(), _ptr(out), _stream(workspace.device))
    _binding.check(st, "spear_take_error")
    return int(out.item()) & 0xFFFFFFFF


def spear_debug_set_spin_limit(polls):
    """Bound of cross-workgroup waits in later calls (negative: the default)."""
    library().spear_debug_set_spin_limit(int(polls))


def spear_debug_fail_waits(on):
    """Test hook: fused waits of later calls look for a tag nobody writes."""
    library().spear_debug_fail_waits(1 if on else 0)


def spear_debug_stream_read(src, grid, sink):
    """Enqueue a plain streaming read of the bytes of `src` (a measurement aid)."""
    _need(sink, "sink", torch.int32, 1)
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    if sink.numel() < grid:
        raise ValueError("sink needs one word per workgroup")
    st = library().spear_debug_stream_read(_ptr(src), src.numel() * src.element_size(), int(grid), _ptr(sink),
                                           _stream(src.device))
    _binding.check(st, "spear_debug_stream_read")


def spear_debug_mfma_rate(shape, waves_per_simd, iterations, sink):
    """Enqueue back-to-back matrix instructions on every CU (a measurement
    aid); returns the launch's floating-point operations.  shape 0:
    v_mfma_f32_16x16x32_f16, 1: v_mfma_f32_32x32x16_f16; sink: float32, one
    per CU."""
    _need(sink, "sink", torch.float32, 1)
    flops = ctypes.c_double(0.0)
    st = library().spear_debug_mfma_rate(int(shape), int(waves_per_simd), int(iterations), _ptr(sink),
                                         _stream(sink.device), ctypes.byref(flops))
    _binding.check(st, "spear_debug_mfma_rate")
    return flops.value
