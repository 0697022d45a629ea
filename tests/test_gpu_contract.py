"""GPU tests of the library's device-side contract: the sticky error word of
a workspace (a cross-workgroup wait that gives up is reported, not silent),
the call epoch's wrap-around, and the streaming-read measurement aid.

The failure path is forced from the host (spear_debug_fail_waits makes the
fused waits look for a tag nobody writes; spear_debug_set_spin_limit bounds
them to a few polls), so every kernel still ends normally."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import w4_gemm_gated_amd as sp

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
EPOCH_WORD = 32 * 1024 // 4 + 96     # GEMM counter region at 32 KiB, word 96
ERROR_WORD = 32 * 1024 // 4 + 64


def note(msg):
    print(f"[gpu-contract] {msg}", flush=True)


def cuda(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# Four fused shapes: decode calls that take the producers' hand-off (one of
# few rows on a K=8192 layer, one on a square 4096 layer, one whose entries
# fill most of the hand-off region), and a tiled call whose EC workgroups
# raise ready flags.
HANDOFF = (2, 8192, 1024, 64)
HANDOFF_SQUARE = (2, 4096, 4096, 32)
HANDOFF_LARGE = (16, 8192, 1024, 64)
TILED = (130, 392, 200, 32)


def fused_case(shape, seed):
    M, K, N, r = shape
    X, W, A, B, w_g = workloads.random_layer(M, K, N, r, seed=seed, outliers=True)
    Wq_d, s_d = sp.spear_pack_w4(cuda(W))
    p = sp.spear_dispatch_plan(M, K, N, r, -0.5, variant="fused")
    assert p.variant == 1 and p.ec_local == 0 and p.producers > 0
    ws = torch.zeros(p.workspace_bytes, dtype=torch.uint8, device=DEV)
    args = (cuda(X), Wq_d, s_d, cuda(A), cuda(B), cuda(w_g), -0.5)
    Wq_o, s_o = oracle.pack_w4(W)
    Y_ref, _ = oracle.w4ec_linear(X, Wq_o, s_o, A, B, w_g, -0.5, 0.0, K=K, N=N)

    def call():
        Y = sp.spear_w4ec_linear(*args, variant="fused", N=N, plan=p, workspace=ws)
        torch.cuda.synchronize()
        return Y.cpu().numpy().astype(np.float64)
    return call, ws, Y_ref


def within(Y, Y_ref):
    return oracle.rel_l2(Y, Y_ref) <= 1e-3 and oracle.max_abs_over_rms(Y, Y_ref) <= 1e-2


@pytest.mark.parametrize("shape,bit", [(HANDOFF, 1), (HANDOFF_SQUARE, 1), (HANDOFF_LARGE, 1), (TILED, 2)])
def test_wait_give_up_is_reported(shape, bit):
    note(f"forced give-up on fused shape {shape}")
    call, ws, Y_ref = fused_case(shape, seed=sum(shape))
    assert sp.spear_take_error(ws) == 0
    try:
        sp.spear_debug_set_spin_limit(16)
        sp.spear_debug_fail_waits(True)
        call()
    finally:
        sp.spear_debug_fail_waits(False)
        sp.spear_debug_set_spin_limit(-1)
    code = sp.spear_take_error(ws)
    note(f"error word after the forced give-up: {code}")
    assert code & bit
    assert sp.spear_take_error(ws) == 0          # read-and-clear
    Y = call()                                   # normal again
    assert within(Y, Y_ref)
    assert sp.spear_take_error(ws) == 0
    words = ws[:64 * 1024].view(torch.int32).cpu().numpy()
    assert words[32 * 1024 // 4 + 32] == 0       # finisher count back at zero


@pytest.mark.parametrize("shape", [HANDOFF, HANDOFF_SQUARE, HANDOFF_LARGE, TILED])
def test_epoch_wrap(shape):
    """The epoch word set to 2^32 - 2 (as after that many calls): the next call
    carries the largest tag, clears the header's tagged words and restarts the
    epoch at 0; the call after it carries tag 1.  Both are correct."""
    note(f"epoch wrap on fused shape {shape}")
    call, ws, Y_ref = fused_case(shape, seed=3 * sum(shape))
    call()                                       # leaves tagged words of tag 1 behind
    w = ws.view(torch.int32)
    w[EPOCH_WORD] = -2                           # 0xFFFFFFFE
    torch.cuda.synchronize()
    Y1 = call()
    e1 = int(w[EPOCH_WORD].item()) & 0xFFFFFFFF
    Y2 = call()
    e2 = int(w[EPOCH_WORD].item()) & 0xFFFFFFFF
    note(f"epochs after the wrap: {e1}, {e2}")
    assert e1 == 0 and e2 == 1
    assert within(Y1, Y_ref) and within(Y2, Y_ref)
    assert np.array_equal(Y1, Y2)
    assert sp.spear_take_error(ws) == 0


def test_take_error_argument_checks():
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(sp.SpearError):
        sp.spear_take_error(ws[: 64 * 1024])     # smaller than the header
    assert sp.spear_take_error(ws) == 0


def test_mfma_rate_counts_and_runs():
    """The matrix-rate aid reports the flops of its launch (instructions x
    multiply-adds x 2 over every wave of one workgroup per CU) and the
    measured rate lies below the published dense fp16 peak of 2.5 PF/s."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(cus, dtype=torch.float32, device=DEV)
    for shape, per in ((0, 8 * 8192 * 2), (1, 4 * 16384 * 2)):
        flops = sp.spear_debug_mfma_rate(shape, 2, 2000, sink)
        assert flops == per * 2000 * 4 * 2 * cus
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        sp.spear_debug_mfma_rate(shape, 2, 2000, sink)
        e.record()
        torch.cuda.synchronize()
        rate = flops / (s.elapsed_time(e) * 1e-3)
        note(f"mfma shape {shape}: {rate / 1e12:.0f} TFLOP/s")
        assert 2e14 < rate < 2.6e15
    assert not sink.any()


def test_stream_read_runs():
    src = torch.ones(1 << 20, dtype=torch.int32, device=DEV)
    sink = torch.zeros(512, dtype=torch.int32, device=DEV)
    sp.spear_debug_stream_read(src, 512, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum().item()) == 0
