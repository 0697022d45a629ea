"""The layer call captured in a HIP graph and replayed, as the benchmark times
it: every replay must give the eager call's output bit for bit (same
kernels, fixed-order sums), with the program's own eager work (fills, other
layer calls, synchronizations) between the replays.  Covers both entry points
(caller workspace and the allocation-free one), the decode kernel with the
producers' hand-off and with the local EC, and the fused tiled launch; the
fused calls advance the workspace's call epoch on every replay, so this also
checks that replays and eager calls interleave on one workspace."""
import numpy as np
import pytest
import torch

import workloads
import w4_gemm_gated_amd as sp

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def note(msg):
    print(f"[gpu-graph] {msg}", flush=True)


def cuda(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("M,K,N,r", [(4, 4096, 4096, 32), (16, 8192, 1024, 64), (3, 1024, 4096, 16),
                                     (130, 392, 200, 32), (512, 2048, 2048, 64), (1000, 256, 10752, 64)])
def test_graph_replay_matches_eager(M, K, N, r, noalloc):
    X, W, A, B, w_g = workloads.random_layer(M, K, N, r, seed=M + K + N + r + 17, outliers=True)
    Wq, s = sp.spear_pack_w4(cuda(W))
    args = (cuda(X), Wq, s, cuda(A), cuda(B), cuda(w_g), -0.5)
    plan = sp.spear_dispatch_plan(M, K, N, r, -0.5, 0.0, "auto")
    note(f"M={M} K={K} N={N} r={r} noalloc={noalloc}: variant={plan.variant} kernel={plan.kernel} "
         f"ec_local={plan.ec_local} producers={plan.producers}")
    ws = None if noalloc else torch.zeros(max(plan.workspace_bytes, 1 << 20), dtype=torch.uint8, device=DEV)

    def call(Y):
        if noalloc:
            return sp.spear_w4ec_linear_noalloc(*args, N=N, plan=plan, Y=Y)
        return sp.spear_w4ec_linear(*args, N=N, plan=plan, Y=Y, workspace=ws)

    Y_eager = call(torch.empty((M, N), dtype=torch.float16, device=DEV)).clone()
    torch.cuda.synchronize()
    Y = torch.empty((M, N), dtype=torch.float16, device=DEV)
    Y_other = torch.empty_like(Y)
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            call(Y)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(4):
        Y.fill_(float("nan"))                      # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_eager), f"replay {rep} differs from the eager call"
        call(Y_other)                              # an eager call on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(Y_other, Y_eager), f"eager call after replay {rep} differs"
    if noalloc:
        assert sp.spear_take_error_noalloc() == 0
    else:
        assert sp.spear_take_error(ws) == 0
    del g


FIRST_CALL_SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import workloads, w4_gemm_gated_amd as sp
M, K, N, r = 4, 1024, 2048, 32
X, W, A, B, w_g = workloads.random_layer(M, K, N, r, seed=3, outliers=True)
t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
Wq, s = sp.spear_pack_w4(t(W))
args = (t(X), Wq, s, t(A), t(B), t(w_g), -0.5)
plan = sp.spear_dispatch_plan(M, K, N, r, -0.5, 0.0, "fused")
assert plan.workspace_bytes > 0
Y = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
refused = False
try:
    with torch.cuda.graph(g):
        sp.spear_w4ec_linear_noalloc(*args, N=N, plan=plan, Y=Y)
except Exception as e:   # the library's refusal (ending an empty capture may raise on top of it)
    refused = any("SPEAR_ERR_HIP" in str(x) for x in (e, e.__context__) if x is not None)
assert refused, "the first call under capture was not refused"
del g
torch.cuda.synchronize()
Y_eager = sp.spear_w4ec_linear_noalloc(*args, N=N, plan=plan).clone()
Y_ws = sp.spear_w4ec_linear(*args, N=N, plan=plan)
torch.cuda.synchronize()
assert torch.equal(Y_eager, Y_ws)
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):
    sp.spear_w4ec_linear_noalloc(*args, N=N, plan=plan, Y=Y)
for _ in range(3):
    Y.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_eager)
print("first-call capture check passed", flush=True)
"""


def test_noalloc_first_call_under_capture_is_refused():
    """In a fresh process (no earlier call has set up the library's array):
    the first allocation-free call made under graph capture is refused with
    nothing enqueued, the next eager call sets the array up and matches the
    workspace entry point, and captured calls after it replay correctly."""
    import os
    import subprocess
    import sys
    repo = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    note("fresh process: first allocation-free call under capture")
    res = subprocess.run([sys.executable, "-c", FIRST_CALL_SCRIPT, repo], capture_output=True, text=True,
                         timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "first-call capture check passed" in out
