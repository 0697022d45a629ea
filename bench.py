"""Benchmark of the W4+EC linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: decode, Llama-3-8B q_proj shape (K = N = 4096, EC rank 32,
gate bias -1, 1% outlier input channels x20), token counts M = 1, 4 and 16.
One step = one call of the layer (EC projection and gate, W4 GEMM, gated EC
epilogue) for each of the three token counts.  `value` is HBM GB/s: the
algorithmic bytes of the three calls (packed weight, scales, X, Y, A, B, w_g)
over their measured time, inputs resident in HBM, weights cold: every call
reads one of R copies of the weights, R x bytes >= 512 MiB (twice the
last-level cache).  Timing uses HIP events on the stream the library launches
on (torch's current stream).

Also reported on the same line: per-token-count times and the EC overhead
(same calls with the EC switched off), the read rate a plain streaming read
of the same bytes gets in one launch (the practical ceiling for a stream of
this size), the prefill workload (M = 2048, K = 4096, N = 14336, rank 64) in
TFLOP/s against the fp16 matrix-core peak, and the fp64 oracle timed on the
host cores on a bounded sample (all threads, and one thread).  Under
"mid_m", the mid-size token counts: the mixed-gate down_proj (M = 64 and
512, K = 14336, N = 4096, rank 64; FUSED, SPLIT and EC off, skip threshold
0 and 0.05; the FUSED/SPLIT crossover and the fraction of the binding
roofline) and the small-model layer stack (256 tokens, seven linears, the EC
on four of them; per-layer latency with the EC on and off).  These are
reported beside the headline, never as `value`.
"""
import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_FP16_PEAK_TFS = 2500.0    # MI355X dense fp16 matrix cores, published
COLD_BYTES = 512 << 20
METRIC = "W4+EC linear TFLOP/s and HBM GB/s (% roofline) at decode M=1–16 and prefill M=2048"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=30)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mid", action="store_true", help="skip the mid-size-M configurations")
    ap.add_argument("--mid-steps", type=int, default=20)
    ap.add_argument("--no-grouped", action="store_true", help="skip the group-wise (g128) variant")
    ap.add_argument("--no-ec-init", action="store_true", help="skip timing the data-free EC initialisation")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle timing")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph replay")
    ap.add_argument("--pmc-mode", action="store_true",
                    help="for hardware-counter runs: a few eager decode calls (M=16), one plain device copy "
                         "of 256 MiB and one streaming read of 64 MiB (the counters' calibrations), no timing line")
    ap.add_argument("--pmc-prefill", action="store_true",
                    help="for hardware-counter runs: a few eager prefill calls (AUTO variant, then EC off), no timing line")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Layer:
    """R device copies of one layer's weights (same values, distinct addresses);
    grouped: group-wise scales (one per 128 input rows) instead of per channel."""

    def __init__(self, torch, sp, w, copies, grouped=False):
        dev = "cuda:0"
        t = lambda a: None if a is None else torch.from_numpy(a).to(dev)  # noqa: E731
        W = t(w["W"])
        Wq, s = sp.spear_pack_w4_grouped(W) if grouped else sp.spear_pack_w4(W)
        del W
        A, B, wg = t(w["A"]), t(w["B"]), t(w["w_g"])
        self.sets = []
        for i in range(copies):
            if i == 0:
                self.sets.append((Wq, s, A, B, wg))
            else:
                self.sets.append(tuple(None if x is None else x.clone() for x in (Wq, s, A, B, wg)))
        self.X = t(w["X"])
        self.K, self.N, self.r = w["K"], w["N"], w["r"]


def time_calls(torch, calls, steps, warmup, graph=True):
    """calls: list of callables forming one step.  Returns seconds per step,
    measured with events on the current stream.  With graph=True the steps
    are captured once into a HIP graph and the graph is replayed, so the
    figure is the GPU's back-to-back rate, free of Python launch overhead."""
    for i in range(warmup):
        for c in calls:
            c(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(steps):
                    for c in calls:
                        c(warmup + i)
        torch.cuda.current_stream().wait_stream(s)
        g.replay()                       # one untimed replay
        torch.cuda.synchronize()
        start.record()
        g.replay()
        stop.record()
        torch.cuda.synchronize()
        del g
    else:
        start.record()
        for i in range(steps):
            for c in calls:
                c(warmup + i)
        stop.record()
        torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3 / steps


def make_call(sp, layer, M, b_g, variant, Ys, plans, workspace, slot=0, stride=1):
    """One call of the layer; call(i) reads weight copy (stride i + slot) mod R,
    so the `stride` calls of one step (slots 0 .. stride-1) each read their own
    copy and no call finds its weights in a cache."""
    plan = plans[(M, variant)]
    X = layer.X[:M]

    def call(i):
        Wq, s, A, B, wg = layer.sets[(stride * i + slot) % len(layer.sets)]
        if variant == "no_ec":
            A = B = wg = None
        sp.spear_w4ec_linear(X, Wq, s, A, B, wg, b_g, 0.0, variant, N=layer.N, plan=plan,
                             Y=Ys[i % len(Ys)][:M], workspace=workspace)
    return call


def _oracle_rate(w, ms, budget_s, W_deq):
    """Decode steps of the oracle (the M of `ms` each) until `budget_s` passes:
    (GB/s of algorithmic bytes, steps, seconds)."""
    import oracle
    import workloads
    Wq, s = oracle.pack_w4(w["W"])
    t0 = time.perf_counter()
    steps, nbytes = 0, 0
    while True:
        for M in ms:
            oracle.w4ec_linear(w["X"][:M], Wq, s, w["A"], w["B"], w["w_g"], w["b_g"][M], K=w["K"], N=w["N"],
                               W_deq=W_deq)
            nbytes += workloads.algorithmic_bytes(M, w["K"], w["N"], w["r"])
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return nbytes / el / 1e9, steps, el


def cpu_baseline(w, ms, budget_s):
    """The oracle as it stands, on a bounded sample of the decode step: weight
    preparation (quantize, pack, fp64 dequantization) timed once and apart;
    then calls on the prepared weight with every BLAS thread, and with one
    thread for the decode step and the tiny workload."""
    import oracle
    import workloads
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    blas = ",".join(sorted({p.get("internal_api", "?") for p in threadpool_info()}))
    t0 = time.perf_counter()
    Wq, s = oracle.pack_w4(w["W"])
    W_deq = oracle.dequant(Wq, s, w["K"], w["N"])
    prep_s = time.perf_counter() - t0
    rate, steps, el = _oracle_rate(w, ms, budget_s, W_deq)
    one = {}
    with threadpool_limits(limits=1):
        r1, st1, el1 = _oracle_rate(w, ms, max(2.0, budget_s / 4), W_deq)
        one["decode_q_proj_4096"] = {"GB/s": round(r1, 4), "steps": st1, "s": round(el1, 2)}
        tiny = workloads.workload(1)
        tq, ts = oracle.pack_w4(tiny["W"])
        tW = oracle.dequant(tq, ts, tiny["K"], tiny["N"])
        t1, n1 = time.perf_counter(), 0
        while time.perf_counter() - t1 < 1.0:
            oracle.w4ec_linear(tiny["X"], tq, ts, tiny["A"], tiny["B"], tiny["w_g"], tiny["b_g"][16],
                               K=tiny["K"], N=tiny["N"], W_deq=tW)
            n1 += 1
        tel = time.perf_counter() - t1
        one["tiny_16x512x512"] = {"us_per_call": round(tel / n1 * 1e6, 1), "calls": n1,
                                  "GB/s": round(n1 * workloads.algorithmic_bytes(16, 512, 512, 16) / tel / 1e9, 4)}
    return {"value": round(rate, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "blas": blas, "host_cpus": len(os.sched_getaffinity(0)),
            "weight_prep_s": round(prep_s, 3),
            "single_thread": one,
            "sample": f"{steps} decode step(s) (M=1,4,16 on K=N=4096, r=32) of the numpy float64 oracle on its "
                      f"dequantized weight (prepared once, {prep_s:.2f} s, not in the rate), {el:.1f} s"}


def read_ceiling(torch, sp, nbytes, steps, graph):
    """Best rate of a plain streaming read of `nbytes` bytes per launch
    (spear_debug_stream_read), cold: each launch reads another copy of
    R x nbytes >= 512 MiB, launches back to back (graph replay) as the layer's
    calls are timed.  Returns (GB/s, grid, us per launch)."""
    nb = -(-nbytes // 256) * 256
    copies = max(2, -(-COLD_BYTES // nb))
    buf = torch.ones(copies * nb // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda:0")
    best = None
    for grid in (256, 512, 1024, 2048):
        def call(i, grid=grid):
            off = (i % copies) * (nb // 4)
            sp.spear_debug_stream_read(buf[off: off + nbytes // 4], grid, sink)
        t = time_calls(torch, [call], steps, 5, graph)
        rate = nbytes / t / 1e9
        if best is None or rate > best[0]:
            best = (rate, grid, t * 1e6)
    del buf
    return best


def mfma_ceiling(torch, sp):
    """Practical ceiling of the matrix cores: back-to-back independent fp16
    matrix instructions on register operands on every CU
    (spear_debug_mfma_rate), right after the prefill timing (clocks settled).
    Returns, per instruction, the best TFLOP/s over 1, 2 and 4 waves per SIMD
    (median of three launches each)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(cus, dtype=torch.float32, device="cuda:0")
    out = {}
    for shape, name in ((0, "v_mfma_f32_16x16x32_f16"), (1, "v_mfma_f32_32x32x16_f16")):
        best = None
        for wps in (1, 2, 4):
            iters = 20000 // wps
            ts = []
            for _ in range(3):
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                flops = sp.spear_debug_mfma_rate(shape, wps, iters, sink)
                e.record()
                torch.cuda.synchronize()
                ts.append(s.elapsed_time(e) * 1e-3)
            rate = flops / sorted(ts)[1] / 1e12
            if best is None or rate > best[0]:
                best = (rate, wps)
        out[name] = {"TFLOP/s": round(best[0], 1), "waves_per_simd": best[1]}
    return out


PMC_COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "decode_m16_hbm_traffic.json")


# The sources that decide the decode call's code and launch: its kernel, the
# headers it includes and the planner.
DECODE_SOURCES = ("w4_gemm_gated_amd/csrc/skinny.hip", "w4_gemm_gated_amd/csrc/device_common.h",
                  "w4_gemm_gated_amd/csrc/internal.h", "w4_gemm_gated_amd/csrc/plan.cpp",
                  "include/spear_w4ec.h")


def _code_only(text):
    """Source text without C/C++ comments and blank-line differences (what
    the compiler sees), so edits to comments do not change the digest."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_digest(read=None):
    """Digest of the decode kernel's sources (code only), to tell whether
    stored counter readings still describe the library as built.  read(name)
    returns a file's text (default: the working tree)."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    if read is None:
        def read(name):
            with open(os.path.join(root, name), encoding="utf-8") as f:
                return f.read()
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        h.update(name.encode() + b"\0" + _code_only(read(name)).encode())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch of the decode call at M=16 from the committed
    counter readings (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known
    size), or None if they were taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def pmc_prefill(torch, sp, workloads):
    """Eager prefill calls for rocprofv3 --pmc runs: 6 of the AUTO variant,
    then 6 with the EC off (each dispatch reported apart)."""
    wp = workloads.workload(3)
    pre = Layer(torch, sp, wp, 2)
    Ys = [torch.empty((2048, wp["N"]), dtype=torch.float16, device="cuda:0")]
    plans = {(2048, "auto"): sp.spear_dispatch_plan(2048, wp["K"], wp["N"], wp["r"], 0.0, 0.0, "auto"),
             (2048, "no_ec"): sp.spear_dispatch_plan(2048, wp["K"], wp["N"], 0, 0.0, 0.0, "no_ec")}
    ws = torch.zeros(max(max(p.workspace_bytes for p in plans.values()), 1 << 20), dtype=torch.uint8,
                     device="cuda:0")
    for v in ("auto", "no_ec"):
        call = make_call(sp, pre, 2048, 0.0, v, Ys, plans, ws)
        for i in range(6):
            call(i)
        torch.cuda.synchronize()
    main_f, ec_f = workloads.algorithmic_flops(2048, wp["K"], wp["N"], wp["r"])
    print(json.dumps({"pmc_prefill": True, "calls": 6, "main_flops": main_f, "ec_flops": ec_f,
                      "source_digest": source_digest()}), flush=True)


PMC_READ_BYTES = 64 << 20


def pmc_mode(torch, sp, workloads):
    """Eager calls for rocprofv3 --pmc runs (each dispatch reported apart)."""
    w = workloads.workload(2)
    dec = Layer(torch, sp, w, 4)
    Ys = [torch.empty((16, w["N"]), dtype=torch.float16, device="cuda:0")]
    plans = {(16, "auto"): sp.spear_dispatch_plan(16, w["K"], w["N"], w["r"], w["b_g"][16], 0.0, "auto")}
    ws = torch.zeros(max(plans[(16, "auto")].workspace_bytes, 1 << 20), dtype=torch.uint8, device="cuda:0")
    call = make_call(sp, dec, 16, w["b_g"][16], "auto", Ys, plans, ws)
    for i in range(8):
        call(i)
    torch.cuda.synchronize()
    src = torch.empty(PMC_COPY_BYTES // 2, dtype=torch.float16, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda:0")
    sp.spear_debug_stream_read(dst[: PMC_READ_BYTES // 2], 1024, sink)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_mode": True, "decode_calls": 8, "copy_bytes": PMC_COPY_BYTES,
                      "stream_read_bytes": PMC_READ_BYTES, "source_digest": source_digest()}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this layer runs on a "
              "single GPU; multi-GPU sharding is not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    import w4_gemm_gated_amd as sp
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    sp.library()
    if args.pmc_mode:
        pmc_mode(torch, sp, workloads)
        return
    if args.pmc_prefill:
        pmc_prefill(torch, sp, workloads)
        return

    # ------------------------------------------------------------ decode
    w = workloads.workload(2)
    ms = w["ms"]
    per_set = workloads.algorithmic_bytes(16, w["K"], w["N"], w["r"])
    copies = max(2, -(-COLD_BYTES // per_set))
    log(f"decode: K=N=4096 r=32, {copies} weight copies")
    dec = Layer(torch, sp, w, copies)
    Ys = [torch.empty((16, w["N"]), dtype=torch.float16, device="cuda:0") for _ in range(8)]
    plans = {}
    for M in ms:
        for v in ("auto", "no_ec"):
            plans[(M, v)] = sp.spear_dispatch_plan(M, w["K"], w["N"], w["r"] if v == "auto" else 0,
                                                   w["b_g"][M], 0.0, v)
    ws_bytes = max(p.workspace_bytes for p in plans.values())
    ws = torch.zeros(max(ws_bytes, 1 << 20), dtype=torch.uint8, device="cuda:0")
    graph = not args.eager
    step_calls = [make_call(sp, dec, M, w["b_g"][M], "auto", Ys, plans, ws, slot=j, stride=len(ms))
                  for j, M in enumerate(ms)]
    t_step = time_calls(torch, step_calls, args.steps, args.warmup, graph)
    step_bytes = sum(workloads.algorithmic_bytes(M, w["K"], w["N"], w["r"]) for M in ms)
    value = step_bytes / t_step / 1e9
    # Secondary figure, the other timing mode: eager launches from Python
    # (each call's argument marshalling and launch on the host) when the
    # headline is a graph replay, or the graph replay when it is eager.
    t_other = time_calls(torch, step_calls, args.steps, args.warmup, not graph)
    other = {"timing": "eager launches" if graph else "hip graph replay of back-to-back calls",
             "ms_per_step": round(t_other * 1e3, 6), "GB/s": round(step_bytes / t_other / 1e9, 1)}
    per_m, overhead = {}, {}
    for M in ms:
        b = workloads.algorithmic_bytes(M, w["K"], w["N"], w["r"])
        t_on = time_calls(torch, [make_call(sp, dec, M, w["b_g"][M], "auto", Ys, plans, ws)], args.steps,
                          args.warmup, graph)
        t_off = time_calls(torch, [make_call(sp, dec, M, 0.0, "no_ec", Ys, plans, ws)], args.steps,
                           args.warmup, graph)
        b_off = workloads.algorithmic_bytes(M, w["K"], w["N"], 0)
        per_m[str(M)] = {"us": round(t_on * 1e6, 3), "GB/s": round(b / t_on / 1e9, 1),
                         "frac_hbm": round(b / t_on / 1e9 / HBM_PEAK_GBS, 4),
                         "variant": _binding_variant(plans[(M, "auto")]),
                         "no_ec_us": round(t_off * 1e6, 3), "no_ec_GB/s": round(b_off / t_off / 1e9, 1)}
        overhead[str(M)] = round(t_on / t_off - 1.0, 4)
        log(f"decode M={M}: {t_on * 1e6:.2f} us ({b / t_on / 1e9:.0f} GB/s), EC off {t_off * 1e6:.2f} us")
    dom_m = "16"
    b16 = workloads.algorithmic_bytes(16, w["K"], w["N"], w["r"])
    achieved = b16 / (per_m[dom_m]["us"] * 1e-6) / 1e9
    del dec
    ceil_rate, ceil_grid, ceil_us = read_ceiling(torch, sp, b16 // 16 * 16, args.steps, graph)
    log(f"read ceiling for {b16 // 16 * 16} B per launch: {ceil_rate:.0f} GB/s ({ceil_us:.2f} us, grid {ceil_grid})")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(),
                "kernel": "skinny_kernel (fused decode call at M=16, one launch per call)",
                "bytes_per_launch": b16,
                "launch_us": per_m[dom_m]["us"],
                "read_ceiling": {"GB/s": round(ceil_rate, 1), "us": round(ceil_us, 3), "grid": ceil_grid,
                                 "what": "plain streaming read of the same bytes per launch, cold, back to back"},
                "frac_of_read_ceiling": round(achieved / ceil_rate, 4)}

    # ------------------------------------------------------------ prefill
    prefill = None
    if not args.no_prefill:
        wp = workloads.workload(3)
        pb = workloads.algorithmic_bytes(2048, wp["K"], wp["N"], wp["r"])
        pcopies = max(2, -(-COLD_BYTES // pb))
        log(f"prefill: M=2048 K=4096 N=14336 r=64, {pcopies} weight copies")
        pre = Layer(torch, sp, wp, pcopies)
        pYs = [torch.empty((2048, wp["N"]), dtype=torch.float16, device="cuda:0") for _ in range(2)]
        pplans = {(2048, "auto"): sp.spear_dispatch_plan(2048, wp["K"], wp["N"], wp["r"], 0.0, 0.0, "auto"),
                  (2048, "no_ec"): sp.spear_dispatch_plan(2048, wp["K"], wp["N"], 0, 0.0, 0.0, "no_ec")}
        pws = torch.zeros(max(max(p.workspace_bytes for p in pplans.values()), 1 << 20), dtype=torch.uint8,
                          device="cuda:0")
        on_call = make_call(sp, pre, 2048, 0.0, "auto", pYs, pplans, pws)
        off_call = make_call(sp, pre, 2048, 0.0, "no_ec", pYs, pplans, pws)
        # The GPU takes a few hundred milliseconds of dense matrix work to
        # settle its clocks: run the layer for about 0.3 s first, then time
        # EC on and off alternately and keep the medians.
        t0 = time.time()
        i = 0
        while time.time() - t0 < 0.3:
            on_call(i)
            i += 1
            if i % 64 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ons, offs = [], []
        for _ in range(3):
            ons.append(time_calls(torch, [on_call], args.prefill_steps, 3, graph))
            offs.append(time_calls(torch, [off_call], args.prefill_steps, 3, graph))
        t_on, t_off = sorted(ons)[1], sorted(offs)[1]
        ceiling = mfma_ceiling(torch, sp)
        main_f, ec_f = workloads.algorithmic_flops(2048, wp["K"], wp["N"], wp["r"])
        tf = main_f / t_on / 1e12
        c16 = ceiling["v_mfma_f32_16x16x32_f16"]["TFLOP/s"]
        prefill = {"us": round(t_on * 1e6, 2), "TFLOP/s": round(tf, 1),
                   "frac_mfma_fp16": round(tf / MFMA_FP16_PEAK_TFS, 4),
                   "mfma_ceiling": ceiling, "frac_of_mfma_ceiling": round(tf / c16, 4),
                   "TFLOP/s_incl_ec": round((main_f + ec_f) / t_on / 1e12, 1),
                   "no_ec_us": round(t_off * 1e6, 2), "ec_overhead": round(t_on / t_off - 1.0, 4),
                   "variant": _binding_variant(pplans[(2048, "auto")])}
        log(f"prefill: {t_on * 1e6:.1f} us, {tf:.1f} TFLOP/s; EC off {t_off * 1e6:.1f} us")
        del pre, pYs

    # ------------------------------------------------------------ mid-size M
    mid = None
    if not args.no_mid:
        mid = mid_size(torch, sp, workloads, args.mid_steps, graph)

    # ------------------------------------------------------------ EC scheduler
    scheduler = None
    if not args.no_mid:
        scheduler = ec_scheduler_section(torch, sp, workloads, args.mid_steps, graph)

    # ------------------------------------------------------------ EC initialisation
    ec_init = None
    if not args.no_ec_init:
        ec_init = ec_init_section(torch, sp, workloads)

    # ------------------------------------------------------------ group-wise scales
    grouped = None
    if not args.no_grouped:
        grouped = grouped_section(torch, sp, workloads, args.steps, args.prefill_steps, graph, not args.no_prefill)

    # ------------------------------------------------------------ oracle on the host
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(w, ms, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "timing": "hip graph replay of back-to-back calls" if graph else "eager launches",
        "secondary_timing": other,
        "data": "synthetic",
        "config": {"workload": "decode q_proj 4096x4096, W4 per-channel + EC rank 32, gate bias -1, "
                               "1% outlier channels x20, M=1,4,16 per step, cold weights",
                   "K": w["K"], "N": w["N"], "rank": w["r"], "tokens": list(ms), "weight_copies": copies},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_m": per_m,
        "ec_overhead": overhead,
        "prefill": prefill,
        "mid_m": mid,
        "g128": grouped,
        "ec_scheduler": scheduler,
        "ec_init": ec_init,
        "cost_model": cost_model_report(sp, per_m, prefill, mid),
    }
    print(json.dumps(line), flush=True)


def mid_size(torch, sp, workloads, steps, graph):
    """Mid-size M: the mixed-gate down_proj (config of M = 64 and 512) and the
    layer stack (M = 256), cold weights (R copies, R x bytes >= 512 MiB)."""
    dev = "cuda:0"

    def timed(layer, M, variant, b_g, tau, plan, Ys, ws):
        X = layer.X[:M]

        def call(i):
            Wq, s, A, B, wg = layer.sets[i % len(layer.sets)]
            if variant == "no_ec" or A is None:
                A = B = wg = None
            sp.spear_w4ec_linear(X, Wq, s, A, B, wg, b_g, tau, variant, N=layer.N, plan=plan,
                                 Y=Ys[i % len(Ys)][:M], workspace=ws)
        return time_calls(torch, [call], steps, 3, graph)

    out = {}
    w = workloads.workload(4)
    per_set = workloads.algorithmic_bytes(64, w["K"], w["N"], w["r"])
    copies = max(2, -(-COLD_BYTES // per_set))
    log(f"mid-size M: mixed-gate down_proj, {copies} weight copies")
    lay = Layer(torch, sp, w, copies)
    Ys = [torch.empty((max(w["ms"]), w["N"]), dtype=torch.float16, device=dev) for _ in range(2)]
    rows = {}
    for M in w["ms"]:
        b_g = w["b_g"][M]
        plans = {v: sp.spear_dispatch_plan(M, w["K"], w["N"], w["r"] if v != "no_ec" else 0, b_g, 0.0, v)
                 for v in ("fused", "split", "no_ec")}
        ws = torch.zeros(max(max(p.workspace_bytes for p in plans.values()), 1 << 20), dtype=torch.uint8,
                         device=dev)
        r = {}
        for tau in w["taus"]:
            for v in ("fused", "split"):
                r[f"{v}_us" + ("" if tau == 0.0 else f"_tau{tau:g}")] = round(
                    timed(lay, M, v, b_g, tau, plans[v], Ys, ws) * 1e6, 2)
        r["no_ec_us"] = round(timed(lay, M, "no_ec", 0.0, 0.0, plans["no_ec"], Ys, ws) * 1e6, 2)
        # The skip threshold's departure from the exact definition, on the GPU:
        # Y at tau = 0.05 against Y at tau = 0 (same inputs, first weight copy).
        Wq, s, A, B, wg = lay.sets[0]
        Ye = sp.spear_w4ec_linear(lay.X[:M], Wq, s, A, B, wg, b_g, 0.0, "auto", N=lay.N).float()
        Yt = sp.spear_w4ec_linear(lay.X[:M], Wq, s, A, B, wg, b_g, 0.05, "auto", N=lay.N).float()
        torch.cuda.synchronize()
        rms = float(Ye.pow(2).mean().sqrt())
        r["tau0.05_deviation"] = {"relL2": round(float((Yt - Ye).norm() / Ye.norm()), 7),
                                  "maxabs_over_rms": round(float((Yt - Ye).abs().max()) / rms, 6)}
        best = min(r["fused_us"], r["split_us"])
        r["faster"] = "fused" if r["fused_us"] <= r["split_us"] else "split"
        r["ec_overhead"] = round(best / r["no_ec_us"] - 1.0, 4)
        nbytes = workloads.algorithmic_bytes(M, w["K"], w["N"], w["r"])
        main_f, _ = workloads.algorithmic_flops(M, w["K"], w["N"], w["r"])
        if M == 64:
            r["bound"] = "hbm"
            r["frac"] = round(nbytes / (best * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        else:
            r["bound"] = "mfma"
            r["frac"] = round(main_f / (best * 1e-6) / 1e12 / MFMA_FP16_PEAK_TFS, 4)
        rows[str(M)] = r
        log(f"mid-size M={M}: fused {r['fused_us']} us, split {r['split_us']} us, EC off {r['no_ec_us']} us")
    out["mixed_gate_down_proj"] = {"K": w["K"], "N": w["N"], "rank": w["r"], "weight_copies": copies,
                                   "per_m": rows}
    del lay

    layers = [workloads.stack_layer(i) for i in range(7)]
    per_set = sum(workloads.algorithmic_bytes(256, L["K"], L["N"], L["r"] if L["A"] is not None else 0)
                  for L in layers)
    copies = max(2, -(-COLD_BYTES // per_set))
    log(f"mid-size M: layer stack (256 tokens), {copies} weight copies")
    st = {}
    total_on = total_off = 0.0
    for L in layers:
        lay = Layer(torch, sp, L, copies)
        M, ec = 256, L["A"] is not None
        Ys = [torch.empty((M, L["N"]), dtype=torch.float16, device=dev) for _ in range(2)]
        p_on = sp.spear_dispatch_plan(M, L["K"], L["N"], L["r"] if ec else 0, 0.0, 0.0, "auto")
        p_off = sp.spear_dispatch_plan(M, L["K"], L["N"], 0, 0.0, 0.0, "no_ec")
        ws = torch.zeros(max(p_on.workspace_bytes, p_off.workspace_bytes, 1 << 20), dtype=torch.uint8, device=dev)
        t_off = timed(lay, M, "no_ec", 0.0, 0.0, p_off, Ys, ws)
        t_on = timed(lay, M, "auto", 0.0, 0.0, p_on, Ys, ws) if ec else t_off
        total_on += t_on
        total_off += t_off
        st[L["name"]] = {"K": L["K"], "N": L["N"], "ec": ec, "us": round(t_on * 1e6, 2),
                         "no_ec_us": round(t_off * 1e6, 2),
                         "variant": _binding_variant(p_on) if ec else "no_ec",
                         "ec_overhead": round(t_on / t_off - 1.0, 4) if ec else 0.0}
        del lay
    out["layer_stack"] = {"tokens": 256, "weight_copies": copies, "layers": st,
                          "stack_us": round(total_on * 1e6, 2), "stack_no_ec_us": round(total_off * 1e6, 2)}
    log(f"mid-size M: layer stack {total_on * 1e6:.1f} us, EC off {total_off * 1e6:.1f} us")
    return out


def grouped_section(torch, sp, workloads, steps, prefill_steps, graph, do_prefill):
    """The group-wise (g128) variant on the decode step's calls (M = 1, 4, 16 of
    the q_proj shape) and on the prefill workload, fused, cold weights; bytes
    count the group scales (ceil(K/128) x N_pad x 2) in place of the per-channel
    ones."""
    out = {}
    w = workloads.workload(2)
    K, N, r = w["K"], w["N"], w["r"]
    scale_extra = -(-K // 128) * (-(-N // 16) * 16) * 2 - 2 * N
    per_set = workloads.algorithmic_bytes(16, K, N, r) + scale_extra
    copies = max(2, -(-COLD_BYTES // per_set))
    lay = Layer(torch, sp, w, copies, grouped=True)
    Ys = [torch.empty((16, N), dtype=torch.float16, device="cuda:0") for _ in range(8)]
    dec = {}
    for M in w["ms"]:
        plans = {(M, v): sp.spear_dispatch_plan(M, K, N, r if v == "auto" else 0, w["b_g"][M], 0.0, v,
                                                group_size=128) for v in ("auto", "no_ec")}
        ws = torch.zeros(max(max(p.workspace_bytes for p in plans.values()), 1 << 20), dtype=torch.uint8,
                         device="cuda:0")
        t_on = time_calls(torch, [make_call(sp, lay, M, w["b_g"][M], "auto", Ys, plans, ws)], steps, 5, graph)
        t_off = time_calls(torch, [make_call(sp, lay, M, 0.0, "no_ec", Ys, plans, ws)], steps, 5, graph)
        b = workloads.algorithmic_bytes(M, K, N, r) + scale_extra
        dec[str(M)] = {"us": round(t_on * 1e6, 3), "GB/s": round(b / t_on / 1e9, 1),
                       "frac_hbm": round(b / t_on / 1e9 / HBM_PEAK_GBS, 4), "no_ec_us": round(t_off * 1e6, 3)}
        log(f"g128 decode M={M}: {t_on * 1e6:.2f} us, EC off {t_off * 1e6:.2f} us")
    out["decode_q_proj_4096"] = dec
    del lay
    if do_prefill:
        wp = workloads.workload(3)
        K, N, r = wp["K"], wp["N"], wp["r"]
        pb = workloads.algorithmic_bytes(2048, K, N, r)
        pre = Layer(torch, sp, wp, max(2, -(-COLD_BYTES // pb)), grouped=True)
        pYs = [torch.empty((2048, N), dtype=torch.float16, device="cuda:0") for _ in range(2)]
        plans = {(2048, v): sp.spear_dispatch_plan(2048, K, N, r if v == "auto" else 0, 0.0, 0.0, v, group_size=128)
                 for v in ("auto", "no_ec")}
        ws = torch.zeros(max(max(p.workspace_bytes for p in plans.values()), 1 << 20), dtype=torch.uint8,
                         device="cuda:0")
        t_on = min(time_calls(torch, [make_call(sp, pre, 2048, 0.0, "auto", pYs, plans, ws)], prefill_steps, 3, graph)
                   for _ in range(2))
        t_off = min(time_calls(torch, [make_call(sp, pre, 2048, 0.0, "no_ec", pYs, plans, ws)], prefill_steps, 3,
                               graph) for _ in range(2))
        main_f, _ = workloads.algorithmic_flops(2048, K, N, r)
        out["prefill_up_proj_2048"] = {"us": round(t_on * 1e6, 2), "TFLOP/s": round(main_f / t_on / 1e12, 1),
                                       "frac_mfma_fp16": round(main_f / t_on / 1e12 / MFMA_FP16_PEAK_TFS, 4),
                                       "no_ec_us": round(t_off * 1e6, 2)}
        log(f"g128 prefill: {t_on * 1e6:.1f} us, EC off {t_off * 1e6:.1f} us")
        del pre, pYs
    return out


def ec_init_section(torch, sp, workloads):
    """Time of the data-free EC initialisation (spear_ec_init, a weight-
    preparation step) on the decode and prefill weights at their ranks: one
    warm call, then the median of three; each call streams the fp32 residual
    (4 K N bytes) twice per iteration (10) and once more, which gives the
    effective rate beside the time."""
    out = {}
    for name, wid in (("decode_q_proj_4096x4096_r32", 2), ("prefill_up_proj_4096x14336_r64", 3)):
        w = workloads.workload(wid)
        W = torch.from_numpy(w["W"]).to("cuda:0")
        Wq, s = sp.spear_pack_w4(W)
        sp.spear_ec_init(W, Wq, s, w["r"])
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            sp.spear_ec_init(W, Wq, s, w["r"])
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        t = sorted(ts)[1]
        streamed = (2 * 10 + 1) * 4 * w["K"] * w["N"]
        out[name] = {"ms": round(t * 1e3, 2), "residual_stream_GB/s": round(streamed / t / 1e9, 1)}
        log(f"ec_init {name}: {t * 1e3:.1f} ms")
        del W, Wq, s
    return out


def cost_model_report(sp, per_m, prefill, mid):
    """The planner's predicted time (predicted_us, predicted_no_ec_us) beside
    each measured call of this run: the decode step's calls, prefill, and the
    mixed-gate and layer-stack calls."""
    rows = []

    def add(name, M, K, N, r, b_g, meas_on, meas_off):
        p = sp.spear_dispatch_plan(M, K, N, r, b_g)
        rows.append({"call": name, "predicted_us": round(float(p.predicted_us), 2), "measured_us": meas_on,
                     "predicted_no_ec_us": round(float(p.predicted_no_ec_us), 2), "measured_no_ec_us": meas_off})
    for M, d in per_m.items():
        add(f"decode q_proj M={M}", int(M), 4096, 4096, 32, -1.0, d["us"], d["no_ec_us"])
    if prefill:
        add("prefill up_proj M=2048", 2048, 4096, 14336, 64, 0.0, prefill["us"], prefill["no_ec_us"])
    if mid:
        for M, d in mid["mixed_gate_down_proj"]["per_m"].items():
            add(f"mixed-gate down_proj M={M}", int(M), 14336, 4096, 64, -5.9, d["fused_us"], d["no_ec_us"])
        for name, d in mid["layer_stack"]["layers"].items():
            if d["ec"]:
                add(f"stack {name} M=256", 256, d["K"], d["N"], 32, 0.0, d["us"], d["no_ec_us"])
    errs = [abs(r["predicted_us"] / r["measured_us"] - 1) for r in rows if r["measured_us"]]
    errs += [abs(r["predicted_no_ec_us"] / r["measured_no_ec_us"] - 1) for r in rows if r["measured_no_ec_us"]]
    errs.sort()
    return {"rows": rows, "median_abs_rel_error": round(errs[len(errs) // 2], 4) if errs else None,
            "max_abs_rel_error": round(errs[-1], 4) if errs else None}


def ec_scheduler_section(torch, sp, workloads, steps, graph):
    """The SLO-constrained EC scheduler (spear_schedule_ec) on the small-model
    layer stack (7 linears, ECs on q, o, up, down, equal weights): a trace of
    the 8 requests of the stack workload (a prefill of their 256 prompt tokens,
    then decode steps of one token per unfinished request, each request
    generating as many tokens as its prompt holds, a reading) under per-step
    SLOs halfway between the stack's predicted time with every EC off and every
    EC on (at M = 256 for the prefill step, M = 8 for decode steps); reported:
    the steps whose predicted time fits, the share of EC layer-steps kept on,
    and for the prefill step and an M = 8 decode step the measured time of the
    chosen configuration beside the model's prediction."""
    dev = "cuda:0"
    layers = [workloads.stack_layer(i) for i in range(7)]
    sched = [(L["K"], L["N"], L["r"], 0, 1.0 if L["r"] else 0.0) for L in layers]
    prompts = list(workloads.STACK_REQUESTS)
    gen = list(prompts)                                   # tokens each request generates

    def bounds(M):
        on, t_on = sp.spear_schedule_ec(sched, M, 1e12)
        off = sum(float(sp.spear_dispatch_plan(M, L["K"], L["N"], L["r"], 0.0).predicted_no_ec_us) for L in layers)
        return off, t_on

    off_p, on_p = bounds(sum(prompts))
    off_d, on_d = bounds(len(prompts))
    slo_p, slo_d = off_p + 0.5 * (on_p - off_p), off_d + 0.5 * (on_d - off_d)
    trace = [sum(prompts)] + [sum(1 for g in gen if g > t) for t in range(max(gen))]
    fit, kept, ec_steps, choices = 0, 0, 0, {}
    for i, M in enumerate(trace):
        slo = slo_p if i == 0 else slo_d
        on, t = sp.spear_schedule_ec(sched, M, slo)
        fit += t <= slo + 1e-9
        kept += sum(on)
        ec_steps += sum(1 for L in layers if L["r"])
        choices.setdefault(M, (on, t))
    out = {"slo_us": {"prefill_M256": round(slo_p, 2), "decode_M8": round(slo_d, 2)},
           "predicted_all_off_us": {"prefill_M256": round(off_p, 2), "decode_M8": round(off_d, 2)},
           "predicted_all_on_us": {"prefill_M256": round(on_p, 2), "decode_M8": round(on_d, 2)},
           "steps": len(trace), "steps_within_slo": int(fit), "ec_kept_share": round(kept / ec_steps, 4)}
    # measured: the chosen configurations of the prefill step and an M = 8 step
    meas = {}
    per_set = sum(workloads.algorithmic_bytes(256, L["K"], L["N"], L["r"]) for L in layers)
    copies = max(2, -(-COLD_BYTES // per_set))
    lays = [Layer(torch, sp, L, copies) for L in layers]
    ws = torch.zeros(32 << 20, dtype=torch.uint8, device=dev)
    for name, M in (("prefill_M256", trace[0]), ("decode_M8", len(prompts))):
        on, t_pred = choices[M]
        calls = []
        for L, lay, keep in zip(layers, lays, on):
            v = "auto" if keep else "no_ec"
            plan = sp.spear_dispatch_plan(M, L["K"], L["N"], L["r"] if keep else 0, 0.0, 0.0, v)
            Ys = [torch.empty((M, L["N"]), dtype=torch.float16, device=dev) for _ in range(2)]
            calls.append(make_call(sp, lay, M, 0.0, v, Ys, {(M, v): plan}, ws))
        t = time_calls(torch, calls, steps, 5, graph)
        meas[name] = {"ec_on": [L["name"] for L, k in zip(layers, on) if k], "predicted_us": round(t_pred, 2),
                      "measured_us": round(t * 1e6, 2)}
        log(f"scheduler {name}: ECs kept {meas[name]['ec_on']}, predicted {t_pred:.1f} us, measured {t * 1e6:.1f} us")
    out["chosen"] = meas
    del lays
    return out


def _binding_variant(plan):
    return {1: "fused", 2: "split", 3: "no_ec"}.get(plan.variant, "?")


if __name__ == "__main__":
    main()
