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
(same calls with the EC switched off), the prefill workload (M = 2048,
K = 4096, N = 14336, rank 64) in TFLOP/s against the fp16 matrix-core peak,
and the fp64 oracle timed on the host cores on a bounded sample.  Under
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
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle timing")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph replay")
    ap.add_argument("--pmc-mode", action="store_true",
                    help="for hardware-counter runs: a few eager decode (M=16) and prefill calls and one "
                         "plain device copy of 256 MiB (the counters' calibration), no timing line")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Layer:
    """R device copies of one layer's weights (same values, distinct addresses)."""

    def __init__(self, torch, sp, w, copies):
        dev = "cuda:0"
        t = lambda a: None if a is None else torch.from_numpy(a).to(dev)  # noqa: E731
        W = t(w["W"])
        Wq, s = sp.spear_pack_w4(W)
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


def make_call(sp, layer, M, b_g, variant, Ys, plans, workspace):
    plan = plans[(M, variant)]
    X = layer.X[:M]

    def call(i):
        Wq, s, A, B, wg = layer.sets[i % len(layer.sets)]
        if variant == "no_ec":
            A = B = wg = None
        sp.spear_w4ec_linear(X, Wq, s, A, B, wg, b_g, 0.0, variant, N=layer.N, plan=plan,
                             Y=Ys[i % len(Ys)][:M], workspace=workspace)
    return call


def cpu_baseline(w, ms, budget_s):
    """The oracle as it stands, on a bounded sample of the decode step."""
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
        blas = ",".join(sorted({p.get("internal_api", "?") for p in threadpool_info()}))
    except Exception:  # noqa: BLE001 - informational only
        threads, blas = os.cpu_count() or 1, "?"
    Wq, s = oracle.pack_w4(w["W"])
    t0 = time.perf_counter()
    steps, nbytes = 0, 0
    while True:
        for M in ms:
            oracle.w4ec_linear(w["X"][:M], Wq, s, w["A"], w["B"], w["w_g"], w["b_g"][M], K=w["K"], N=w["N"])
            nbytes += workloads.algorithmic_bytes(M, w["K"], w["N"], w["r"])
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "blas": blas, "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{steps} decode step(s) (M=1,4,16 on K=N=4096, r=32), numpy float64 oracle incl. "
                      f"dequantizing the packed weight each call, {el:.1f} s"}


PMC_COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "decode_m16_hbm_traffic.json")


def source_digest():
    """Digest of the kernel sources, to tell whether stored counter readings
    still describe the library as built."""
    import hashlib
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "w4_gemm_gated_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(root)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(root, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
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
    print(json.dumps({"pmc_mode": True, "decode_calls": 8, "copy_bytes": PMC_COPY_BYTES,
                      "source_digest": source_digest()}), flush=True)


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
    step_calls = [make_call(sp, dec, M, w["b_g"][M], "auto", Ys, plans, ws) for M in ms]
    t_step = time_calls(torch, step_calls, args.steps, args.warmup, graph)
    step_bytes = sum(workloads.algorithmic_bytes(M, w["K"], w["N"], w["r"]) for M in ms)
    value = step_bytes / t_step / 1e9
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
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(),
                "kernel": "skinny_kernel (fused decode call at M=16, one launch per call)",
                "bytes_per_launch": b16,
                "launch_us": per_m[dom_m]["us"]}
    del dec

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
        main_f, ec_f = workloads.algorithmic_flops(2048, wp["K"], wp["N"], wp["r"])
        tf = main_f / t_on / 1e12
        prefill = {"us": round(t_on * 1e6, 2), "TFLOP/s": round(tf, 1),
                   "frac_mfma_fp16": round(tf / MFMA_FP16_PEAK_TFS, 4),
                   "TFLOP/s_incl_ec": round((main_f + ec_f) / t_on / 1e12, 1),
                   "no_ec_us": round(t_off * 1e6, 2), "ec_overhead": round(t_on / t_off - 1.0, 4),
                   "variant": _binding_variant(pplans[(2048, "auto")])}
        log(f"prefill: {t_on * 1e6:.1f} us, {tf:.1f} TFLOP/s; EC off {t_off * 1e6:.1f} us")
        del pre, pYs

    # ------------------------------------------------------------ mid-size M
    mid = None
    if not args.no_mid:
        mid = mid_size(torch, sp, workloads, args.mid_steps, graph)

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


def _binding_variant(plan):
    return {1: "fused", 2: "split", 3: "no_ec"}.get(plan.variant, "?")


if __name__ == "__main__":
    main()
