#!/usr/bin/env python3
"""Throughput of one MoE FFN layer (moe_layer) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--tokens N]
                    [--no-flush] [--fp8 | --micro-batches M | --cost-model]

A step is one moe_layer call over one batch of synthetic, seeded input that is
already resident in HBM: router -> top-k -> dispatch/permutation -> grouped
SwiGLU (gate+up, down) -> shared experts -> combine.  The default workload is
the Qwen3-235B-shaped skewed layer (N=8192 tokens, M=4096, E=128, top-8,
H=1536, a Zipf-shaped router bias that gives the hottest expert 4x the mean
load), the largest workload that fits one GPU and the one where the expert
GEMMs are bound by the matrix cores.  Other workloads: --workload tiny,
mixtral, dsv2, qwen30 (with --tokens), qwen235_node.

Timing: W untimed warm-up calls, then K timed calls; before each call a 1 GiB
buffer is read (outside the events), so that L2 and the Infinity Cache hold
nothing of the layer, and each call is bracketed by two events on the layer's
stream.  The step time is the median call; p10/p90 are reported beside it.
A further K calls record events at the layer's stage boundaries; the gate+up
launch's mean time from them gives the dominant kernel's roofline.  The
oracle is timed on the host cores as the CPU baseline.  Prints ONE JSON line.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
METRIC = "MoE-layer tokens/s + achieved TFLOP/s or HBM GB/s vs roofline, 1xMI355X"
STAGES = ("route", "permute", "shared", "gate_up", "down", "combine")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_work(w, active: int, fp8: bool = False):
    """Algorithmic flops/bytes of one layer call: three GEMMs of m_e x M x H
    per expert (6*M*H flops per assignment), router, shared experts; bytes =
    weights of experts that received rows + router + shared weights + x + out.
    FP8 weights: one byte per weight plus a float32 scale per output channel."""
    A = w.N * w.k
    has_router = not w.pre_routed
    wb = 1.0 if fp8 else 2.0
    F = 6.0 * w.M * w.H * A + (2.0 * w.N * w.M * w.E if has_router else 0) + 6.0 * w.M * w.S * w.Hs * w.N
    B = (active * 3.0 * w.M * w.H * wb + w.S * 3.0 * w.M * w.Hs * wb + (w.M * w.E * 2.0 if has_router else 0)
         + 2.0 * w.N * w.M * 2)
    if fp8:
        B += (active * (2.0 * w.H + w.M) + (2.0 * w.S * w.Hs + w.M if w.S else 0)) * 4
    return F, B


def gateup_work(w, active: int, fp8: bool = False):
    """Algorithmic bytes/flops of one gate+up launch: W_gate and W_up rows of
    every active expert (and their scales with FP8 weights), the token rows
    read once each, h written."""
    A = w.N * w.k
    wb = 1.0 if fp8 else 2.0
    B = active * 2.0 * w.H * w.M * wb + w.N * w.M * 2.0 + A * w.H * 2.0
    if fp8:
        B += active * 2.0 * w.H * 4
    F = 4.0 * w.M * w.H * A
    return F, B


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    """Cores this process may run on (its affinity mask), capped by
    OMP_NUM_THREADS where that is set (the host's share of cores per GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(w, d, budget_s: float = 20.0, max_runs: int = 5):
    """The oracle on the host cores over the same inputs: runs of the whole
    layer while they fit in about 20 s (at least one, at most five), median
    reported.  The BLAS pool is limited to the cores the process may use, and
    that count is reported."""
    import threadpoolctl
    from oracle import moe_oracle as O
    cores = host_cores()
    times = []
    with threadpoolctl.threadpool_limits(limits=cores):
        while len(times) < max_runs and sum(times) < budget_s:
            t0 = time.perf_counter()
            if w.pre_routed:
                O.expert_node(d["x"], d["topk_ids"], d["topk_weights"], d["w_gate"], d["w_up"], d["w_down"])
            else:
                O.moe_layer(d, w.k, w.S, w.Hs)
            times.append(time.perf_counter() - t0)
        used = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    dt = float(np.median(times))
    return {"value": w.N / dt, "unit": "tokens/s", "cores": int(min(used, cores)), "kind": "oracle",
            "cpu_model": _cpu_model(), "runs": len(times),
            "sample": f"the whole {w.title} layer (N={w.N}) through the CPU oracle (float64 expert math, "
                      f"float32 routing), {'median of ' + str(len(times)) + ' runs' if len(times) > 1 else 'one run'}"
                      f": {dt:.2f} s"}


def dense_reference(args) -> int:
    """hipBLASLt (torch.matmul) on dense GEMMs holding the workload's total
    expert work: [A x M].[M x 2H] (gate+up) and [A x H].[H x M] (down), A =
    N*k rows, both operands contraction-contiguous as the expert weights are.
    A reference point for the grouped kernels' MFMA rate: the same flops with
    no grouping, gathering, padding or SwiGLU.  Flushed medians, one JSON line."""
    import statistics
    import torch
    from datagen import configs

    w = configs.get(args.workload, args.tokens)
    A = w.N * w.k
    dev = torch.device("cuda:0")
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    res = {"metric": "dense bf16 GEMM reference (torch.matmul / hipBLASLt)", "workload": w.title, "rows": A}
    for name, (K, Nc) in (("gate_up", (w.M, 2 * w.H)), ("down", (w.H, w.M))):
        a = torch.randn(A, K, device=dev).to(torch.bfloat16)
        b = torch.randn(Nc, K, device=dev).to(torch.bfloat16)
        a @ b.t()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(args.steps, 5)):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            a @ b.t()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        us = statistics.median(ts)
        res[name] = {"shape": [A, K, Nc], "us": us, "tflops": 2.0 * A * K * Nc / us / 1e6}
        del a, b
    print(json.dumps(res), flush=True)
    return 0


def cost_model(args) -> int:
    """FinDEP's per-expert cost model (review page, section 核心公式: an expert's
    time is linear in its batch, t_e(m) = alpha_e + beta_e * m).  For each
    workload's (M, H, E) it times moe_grouped_ffn (gate+up and down GEMMs)
    with every one of the E experts given m rows, m = 1, 2, 4, ..., 4096,
    caches flushed before every call (a 1 GiB read), and fits alpha and beta to the
    per-expert time (launch time / E) by least squares.  Also reports where a
    two-line fit (flat weight-streaming part, rising compute part) bends.
    Weights and rows are seeded normal values drawn on the device (their
    values do not matter for the timing)."""
    import torch
    import expert_ffn_dispatch_amd as moe

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)    # read (not written) before each call
    shapes = [("mixtral", 6144, 16384, 8), ("dsv2", 5120, 1536, 160), ("qwen30", 2048, 768, 128),
              ("qwen235", 4096, 1536, 128)]
    rows = [1 << i for i in range(13)]
    reps = 5
    for i, (name, M, H, E) in enumerate(shapes):
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + i)

        def normal(shape, std):
            return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)

        wg = normal((E, H, M), 0.02)
        wu = normal((E, H, M), 0.02)
        wd = normal((E, M, H), 0.02)
        base = normal((rows[-1], M), 1.0)
        t_us = []
        for m in rows:
            A = E * m
            d = moe.dims(A, M, E, 1, H)
            off = torch.arange(0, A + 1, m, dtype=torch.int32, device=dev)
            xs = base[:m].repeat(E, 1)
            y = torch.empty((A, M), dtype=torch.bfloat16, device=dev)
            ws = moe.workspace(moe.moe_grouped_ffn_workspace_bytes(d), dev)
            times = []
            for r in range(reps):
                flush.sum()
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record()
                moe.moe_grouped_ffn(d, xs, off, wg, wu, wd, y_sorted=y, ws=ws)
                ev1.record()
                torch.cuda.synchronize()
                times.append(ev0.elapsed_time(ev1) * 1e3)
            t_us.append(float(np.median(times[1:])) / E)
            del xs, y, ws
        mm = np.array(rows, dtype=np.float64)
        tt = np.array(t_us)
        beta, alpha = np.polyfit(mm, tt, 1)
        pred = alpha + beta * mm
        r2 = 1.0 - float(((tt - pred) ** 2).sum() / ((tt - tt.mean()) ** 2).sum())
        # bend: where the compute line through the last four points reaches
        # the flat streaming time of the first five
        flat = float(tt[:5].mean())
        b1, a1 = np.polyfit(mm[-4:], tt[-4:], 1)
        knee = (flat - a1) / b1 if b1 > 0 else None
        wbytes = 3 * M * H * 2
        print(json.dumps({"cost_model": name, "M": M, "H": H, "E": E, "rows_per_expert": rows,
                          "t_us_per_expert": t_us, "alpha_us": float(alpha), "beta_us_per_row": float(beta),
                          "r2": r2, "flat_us": flat, "knee_rows": float(knee) if knee is not None else None,
                          "weight_gbs_at_1_row": wbytes / (t_us[0] * 1e-6) / 1e9,
                          "tflops_at_4096_rows": 6.0 * M * H * rows[-1] / (t_us[-1] * 1e-6) / 1e12}),
              flush=True)
        del wg, wu, wd, base
        torch.cuda.empty_cache()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen235")
    ap.add_argument("--tokens", type=int, default=None, help="token count for the decode sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30,
                    help="size of the plain device copy timed after the layer (0 = skip); its GB/s is "
                         "the practical bandwidth ceiling and its counters scale FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--no-flush", dest="flush", action="store_false",
                    help="skip the 1 GiB read before every call (by default it runs, outside the call's "
                         "events, so that weights come from HBM); the step time is then the wall clock "
                         "over K back-to-back calls")
    ap.add_argument("--fp8", action="store_true",
                    help="run moe_layer_fp8: expert weights quantised once (moe_quantize_fp8, OCP E4M3 "
                         "with per-channel scales) before timing; activations and h stay bf16; no CPU "
                         "baseline in this mode")
    ap.add_argument("--micro-batches", type=int, default=1,
                    help="run moe_layer_pipelined with this many micro-batches overlapped on two streams "
                         "(per-stage events are not available in this mode; the roofline is the layer's)")
    ap.add_argument("--cost-model", action="store_true",
                    help="instead of the layer: time one expert's SwiGLU FFN over per-expert batches "
                         "1..4096 at each workload's (M, H) and fit t(m) = alpha + beta*m (one JSON "
                         "line per shape)")
    ap.add_argument("--dense-reference", action="store_true",
                    help="instead of the layer: time hipBLASLt (torch.matmul) on dense GEMMs with the "
                         "workload's total gate+up and down work, as a reference MFMA rate")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs one MoE layer on ONE GPU; --gpus {args.gpus} is not supported "
              f"(the expert-parallel exchange across GPUs is not built)", file=sys.stderr)
        return 2
    if args.cost_model:
        return cost_model(args)
    if args.dense_reference:
        return dense_reference(args)

    import torch
    import expert_ffn_dispatch_amd as moe
    from expert_ffn_dispatch_amd import profiling
    from datagen import configs, gen

    w = configs.get(args.workload, args.tokens)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: generating {w.title} N={w.N}")
    t = time.perf_counter()
    d = gen.generate(w)
    log(f"bench: inputs generated in {time.perf_counter() - t:.1f} s")

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    T = {k: up(v) for k, v in d.items() if isinstance(v, np.ndarray) and v.ndim > 0}
    dm = moe.dims(w.N, w.M, w.E, w.k, w.H, w.S, w.Hs)
    flags = moe.MOE_FLAG_IDS_IN if w.pre_routed else 0
    ws = moe.workspace(moe.moe_layer_workspace_bytes(dm, flags), dev)
    out = torch.empty((w.N, w.M), dtype=torch.bfloat16, device=dev)
    if w.pre_routed:
        ids, wts = T["topk_ids"], T["topk_weights"]
    else:
        ids = torch.empty((w.N, w.k), dtype=torch.int32, device=dev)
        wts = torch.empty((w.N, w.k), dtype=torch.float32, device=dev)
    # cache flush: a reduction over 1 GiB that the layer never touches; it reads
    # (an overwrite would leave L2 and the Infinity Cache full of dirty lines
    # whose write-back the timed call would then pay)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev) if args.flush else None

    def flush():
        flush_buf.sum()
    if args.fp8:
        W8 = moe.quantize_ffn_fp8(T["w_gate"], T["w_up"], T["w_down"])
        S8 = moe.quantize_ffn_fp8(T["ws_gate"], T["ws_up"], T["ws_down"]) if w.S > 0 else None
        for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
            T.pop(n, None)       # the bf16 expert weights are not used in this mode
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    pipelined = args.micro_batches > 1
    if pipelined:
        if args.fp8:
            raise SystemExit("bench.py: --micro-batches runs the bf16 layer only")
        ws = moe.workspace(moe.moe_layer_pipelined_workspace_bytes(dm, args.micro_batches, flags), dev)

    def step(events=None):
        if pipelined:
            moe.moe_layer_pipelined(dm, args.micro_batches, T["x"], T["w_gate"], T["w_up"], T["w_down"],
                                    w_router=T.get("w_router"), router_bias=T.get("router_bias"),
                                    ws_gate=T.get("ws_gate"), ws_up=T.get("ws_up"), ws_down=T.get("ws_down"),
                                    topk_ids=ids, topk_weights=wts, ids_in=w.pre_routed, out=out, ws=ws)
            return
        if events is not None:
            moe.moe_set_stage_events(events)
        if args.fp8:
            moe.moe_layer_fp8(dm, T["x"], W8, S8, w_router=T.get("w_router"), router_bias=T.get("router_bias"),
                              topk_ids=ids, topk_weights=wts, ids_in=w.pre_routed, out=out, ws=ws)
            return
        moe.moe_layer(dm, T["x"], T["w_gate"], T["w_up"], T["w_down"], w_router=T.get("w_router"),
                      router_bias=T.get("router_bias"), ws_gate=T.get("ws_gate"), ws_up=T.get("ws_up"),
                      ws_down=T.get("ws_down"), topk_ids=ids, topk_weights=wts, ids_in=w.pre_routed,
                      out=out, ws=ws)

    for _ in range(args.warmup):
        if flush_buf is not None:
            flush()
        step()
    torch.cuda.synchronize()
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(K)]
    call_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for row in evs + call_ev:    # torch creates the HIP event on first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    # pass 1, timed steps: back-to-back layer calls with nothing else on the
    # stream (skipped with --flush, whose value is the per-call median)
    wall = 0.0
    if flush_buf is None:
        t0 = time.perf_counter()
        for i in range(K):
            step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    # pass 2, per call: each call between two events on the layer's stream;
    # with --flush a 1 GiB buffer is read before each call, outside the events,
    # so no weight is served from L2 or the Infinity Cache
    for i in range(K):
        if flush_buf is not None:
            flush()
        call_ev[i][0].record()
        step()
        call_ev[i][1].record()
    torch.cuda.synchronize()
    call_ms = np.array([call_ev[i][0].elapsed_time(call_ev[i][1]) for i in range(K)])
    # pass 3, stages: events recorded inside the layer at its stage boundaries
    # (each costs the stream a few us); the micro-batched layer records its
    # whole call between two events instead
    for i in range(K):
        if flush_buf is not None:
            flush()
        if pipelined:
            evs[i][0].record()
            step()
            for e in evs[i][1:]:
                e.record()
        else:
            step(evs[i])
    torch.cuda.synchronize()

    stage_ms = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(6)] for i in range(K)])
    ms_per_step = float(np.median(call_ms)) if args.flush else wall * 1e3 / K
    value = w.N / (ms_per_step * 1e-3)

    hid = ids.cpu().numpy().reshape(-1)
    counts = np.bincount(hid, minlength=w.E)
    active = int((counts > 0).sum())
    F, B = layer_work(w, active, args.fp8)
    Fg, Bg = gateup_work(w, active, args.fp8)
    t_gu = stage_ms[:, 3].mean() * 1e-3
    t_layer = ms_per_step * 1e-3
    if pipelined:
        # the launches of several micro-batches interleave: report the layer
        Fg, Bg, t_gu = F, B, t_layer
    # the gate+up launch is bound by MFMA when its flops per algorithmic
    # byte exceed the ridge point (peak flops / peak bandwidth), else by HBM
    mfma_bound = Fg / Bg > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    achieved = Fg / t_gu / 1e12 if mfma_bound else Bg / t_gu / 1e9
    peak = BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS
    t_roof = max(F / (BF16_PEAK_TFLOPS * 1e12), B / (HBM_PEAK_GBS * 1e9))
    res = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.title, "N": w.N, "M": w.M, "E": w.E, "k": w.k, "H": w.H, "S": w.S, "Hs": w.Hs,
                   "expert_weights": "fp8 e4m3, per-channel fp32 scales" if args.fp8 else "bf16",
                   "micro_batches": args.micro_batches,
                   "parallelism": "single GPU",
                   "timing": "median of per-call event times, L2 and Infinity Cache flushed before each call"
                   if args.flush else "wall clock over back-to-back steps"},
        "roofline": {"bound": "mfma" if mfma_bound else "hbm",
                     "kernel": ("whole layer, micro-batched" if pipelined else
                                "grouped SwiGLU gate+up GEMM (ffn_stream_kernel at decode-sized experts, "
                                "ffn_tile_kernel otherwise)"),
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s" if mfma_bound else "GB/s",
                     "frac": achieved / peak, "traffic": None, "algorithmic_bytes": Bg, "algorithmic_flops": Fg,
                     "avg_us": t_gu * 1e6},
        "layer": {"flops": F, "bytes": B, "tflops": F / t_layer / 1e12, "hbm_gbs": B / t_layer / 1e9,
                  "mfma_frac": F / t_layer / (BF16_PEAK_TFLOPS * 1e12), "hbm_frac": B / t_layer / (HBM_PEAK_GBS * 1e9),
                  "roofline_frac": t_roof / t_layer, "t_roof_us": t_roof * 1e6,
                  # per-call times, each call between two events (caches flushed with --flush)
                  "event_layer_us": float(call_ms.mean() * 1e3),
                  "event_layer_us_p10_p50_p90": [float(np.percentile(call_ms, q) * 1e3) for q in (10, 50, 90)]},
        "stages_us": None if pipelined else {s: float(stage_ms[:, j].mean() * 1e3) for j, s in enumerate(STAGES)},
        "routing": {"active_experts": active, "max_rows": int(counts.max()), "mean_rows": float(counts.mean()),
                    "empty_experts": int((counts == 0).sum())},
    }
    if args.copy_bytes > 0:
        # a plain elementwise copy of known size: reads and writes copy_bytes
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.add(src, 0.0, out=dst)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            torch.add(src, 0.0, out=dst)
        c1.record()
        torch.cuda.synchronize()
        res["copy_gbs"] = 2.0 * n * 4 * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del src, dst
    tr = None if pipelined else profiling.read_traffic(os.path.join(ROOT, "profiles",
                                             f"traffic_{w.name}_N{w.N}{'_fp8' if args.fp8 else ''}.txt"))
    if tr is not None:
        res["roofline"]["traffic"] = float(tr["traffic_bytes"])
    if not args.no_cpu_baseline and not args.fp8:
        log("bench: timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(w, d)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
