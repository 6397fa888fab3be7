"""Benchmark of the 4-bit weight-streaming matmul and the A8 prefill route on one MI355X.

Prints ONE JSON line on stdout.  A "step" is one pass of the hot path over
one batch: one skinny decode GEMV (M = 1, K = 5120, N = 17408, the FFN
gate/up shape) streaming one of >= 2 GB of distinct packed weight copies, so
the 256 MB Infinity Cache cannot serve it.  `value` is the effective
weight-stream bandwidth of those K steps (algorithmic bytes / time).

The timed region replays a HIP graph holding exactly K captured launches
(launch-bound inner loops belong in graphs); the same K launches issued
eagerly from Python are reported beside it.  Extra sections, each timed the
same way, cover the rest of the path:
  verify_down_per_M      K = 17408, N = 5120, M = 1..16 (speculative verify)
  decode_step_64L        64 layers x {qkv, out, gate, up, down} at M = 5
  a8w4_prefill           M = 2048, K = 5120, N = 17408 (activation quant + int8 MFMA GEMM)
  a8w4_prefill_pass_64L  the 64-layer A8 pass at M = 512, 1024 and 2048 (section "pass")
plus `roofline` for the dominant kernel and `cpu_baseline` (the oracle).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0       # MI355X dense int8 MFMA, published
ROTATE_BYTES = 2 * 1024 ** 3  # distinct weight bytes cycled through per series
BYTES_PER_WEIGHT = 0.5625     # 4 bits + one fp16 scale per 32 weights


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemv_bytes(m, k, n):
    """Algorithmic bytes of one skinny GEMV: packed weights + X + Y."""
    return int(n * k * BYTES_PER_WEIGHT) + 2 * m * k + 2 * m * n


# --------------------------------------------------------------------------
# timing helpers
# --------------------------------------------------------------------------

def time_region(torch, fn):
    """Run fn() between two synchronizations, timed with events on the current stream."""
    s = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(s)
    fn()
    stop.record(s)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3


def capture(torch, fn):
    """Capture fn() into a HIP graph (through torch's graph API) and return it."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # warm the side stream (allocations, code objects)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# --------------------------------------------------------------------------
# skinny GEMV series over rotating weight copies
# --------------------------------------------------------------------------

def make_copies(torch, q4w, synthetic, n, k, base_seed):
    per = int(n * k * BYTES_PER_WEIGHT)
    count = max(2, -(-ROTATE_BYTES // per))
    copies = []
    for i in range(count):
        w = synthetic.weights_device(n, k, base_seed + i)
        copies.append(q4w.pack(w))
        del w
    torch.cuda.synchronize()
    return copies


def gemv_series(torch, q4w, copies, x, y, steps, warmup, series=1):
    """Returns (graph seconds, eager seconds) for `steps` launches rotating over
    copies; with series > 1 the graph of `steps` launches is timed that many
    times and the median is returned (and the list as a third value)."""
    m, k = x.shape
    n = copies[0][0].shape[0]
    ws = torch.zeros(max(q4w.gemv_ws_bytes(m, n, k, 0), 1), dtype=torch.uint8, device="cuda")

    def launches(count, offset=0):
        for i in range(count):
            c, s = copies[(offset + i) % len(copies)]
            q4w.q4_gemv_skinny_raw(x, c, s, y, 0, ws)

    launches(warmup)
    t_eager = time_region(torch, lambda: launches(steps))
    g = capture(torch, lambda: launches(steps))
    g.replay()
    times = [time_region(torch, g.replay) for _ in range(series)]
    del g
    if series == 1:
        return times[0], t_eager
    return sorted(times)[series // 2], t_eager, times


# --------------------------------------------------------------------------
# sections
# --------------------------------------------------------------------------

def bench_decode(torch, q4w, synthetic, steps, warmup):
    wl = synthetic.WORKLOADS["decode_gate_up"]
    m, k, n = wl["M"], wl["K"], wl["N"]
    copies = make_copies(torch, q4w, synthetic, n, k, 10_000)
    x = synthetic.activations_device(m, k, synthetic.ACT_SEED)
    y = torch.empty((m, n), dtype=torch.float16, device="cuda")
    tg, te = gemv_series(torch, q4w, copies, x, y, steps, warmup)
    b = gemv_bytes(m, k, n)
    out = dict(M=m, K=k, N=n, copies=len(copies), bytes_per_launch=b,
               t_graph_s=tg, t_eager_s=te,
               gbs_graph=b * steps / tg / 1e9, gbs_eager=b * steps / te / 1e9,
               us_per_launch_graph=tg / steps * 1e6, us_per_launch_eager=te / steps * 1e6)
    del copies
    torch.cuda.empty_cache()
    return out


def bench_verify(torch, q4w, synthetic, steps, warmup):
    wl = synthetic.WORKLOADS["verify_down"]
    k, n = wl["K"], wl["N"]
    copies = make_copies(torch, q4w, synthetic, n, k, 20_000)
    res = {}
    for m in (1, 2, 3, 4, 5, 8, 13, 16):      # 1..5: the verify workload; 8..16: wide drafts
        # median of three timed graph replays of `steps` launches (min and max kept)
        x = synthetic.activations_device(m, k, synthetic.ACT_SEED)
        y = torch.empty((m, n), dtype=torch.float16, device="cuda")
        tg, te, ts = gemv_series(torch, q4w, copies, x, y, steps, warmup, series=3)
        b = gemv_bytes(m, k, n)
        res[str(m)] = dict(gbs_graph=b * steps / tg / 1e9, gbs_eager=b * steps / te / 1e9,
                           us_per_launch_graph=tg / steps * 1e6,
                           us_per_launch_graph_min_max=[min(ts) / steps * 1e6, max(ts) / steps * 1e6],
                           frac_of_peak=b * steps / tg / 1e9 / HBM_PEAK_GBS)
    del copies
    torch.cuda.empty_cache()
    return dict(K=k, N=n, per_M=res)


def bench_decode_step(torch, q4w, synthetic, reps, m=5):
    """64 layers x 5 projections at M = 5, back to back on one stream."""
    from bit_quantized_weight_amd.decode import DecodeStep
    step = DecodeStep(m)
    torch.cuda.synchronize()
    for _ in range(2):
        step.run()
    t_eager = time_region(torch, lambda: [step.run() for _ in range(reps)]) / reps
    g = capture(torch, step.run)
    g.replay()
    t_graph = time_region(torch, lambda: [g.replay() for _ in range(reps)]) / reps
    # the same step as one persistent launch over all 320 matmuls
    step.plan_batched()
    for _ in range(2):
        step.run_batched()
    t_batched = time_region(torch, lambda: [step.run_batched() for _ in range(reps)]) / reps
    total = step.weight_bytes + step.io_bytes
    out = dict(M=m, layers=len(step.layers), launches_per_step=step.launches,
               weight_bytes_per_step=step.weight_bytes, ms_graph=t_graph * 1e3,
               ms_eager=t_eager * 1e3, gbs_graph=total / t_graph / 1e9,
               gbs_eager=total / t_eager / 1e9,
               ms_batched=t_batched * 1e3, gbs_batched=total / t_batched / 1e9,
               batched_grid=step.batch.plan.grid, batched_items=step.batch.plan.total_items)
    del g, step
    torch.cuda.empty_cache()
    return out


def bench_prefill_pass(torch, q4w, synthetic, reps, ms=(512, 1024, 2048)):
    """64 layers x 5 projections on the A8 route at M = 512, 1024 and 2048
    tokens (one packed weight set): per layer three activation quantizations
    and five GEMMs, as a HIP graph."""
    from bit_quantized_weight_amd.prefill import PrefillPass
    weights = None
    per_m = {}
    for m in ms:
        p = PrefillPass(m, weights=weights)
        weights = p.layers
        torch.cuda.synchronize()
        p.run()
        t_eager = time_region(torch, lambda: [p.run() for _ in range(reps)]) / reps
        g = capture(torch, p.run)
        g.replay()
        t_graph = time_region(torch, lambda: [g.replay() for _ in range(reps)]) / reps
        per_m[str(m)] = dict(int_ops_per_pass=p.int_ops, ms_graph=t_graph * 1e3, ms_eager=t_eager * 1e3,
                             tok_s=m / t_graph, tops=p.int_ops / t_graph / 1e12)
        layers = len(p.layers)
        del g, p
        torch.cuda.empty_cache()
    del weights
    torch.cuda.empty_cache()
    return dict(layers=layers, launches_per_pass=8 * layers, per_M=per_m)


def bench_prefill(torch, q4w, synthetic, reps):
    """A8 route at M = 2048: the whole route per launch pair (activation
    quantization + GEMM), and the GEMM alone from prepared activations."""
    wl = synthetic.WORKLOADS["prefill_a8"]
    m, k, n = wl["M"], wl["K"], wl["N"]
    w = synthetic.weights_device(n, k, synthetic.WEIGHT_SEED)
    codes, scales = q4w.pack(w)
    del w
    x = synthetic.activations_device(m, k, synthetic.ACT_SEED)
    y = torch.empty((m, n), dtype=torch.float16, device="cuda")
    for _ in range(3):
        q4w.a8w4_gemm(x, codes, scales, y)
    t_route = time_region(torch, lambda: [q4w.a8w4_gemm(x, codes, scales, y) for _ in range(reps)]) / reps
    ws = q4w.a8w4_prepare(x)
    for _ in range(3):
        q4w.a8w4_gemm_prepared(ws, m, k, codes, scales, y)
    t_gemm = time_region(torch, lambda: [q4w.a8w4_gemm_prepared(ws, m, k, codes, scales, y)
                                          for _ in range(reps)]) / reps
    ops = 2 * m * n * k
    return dict(M=m, K=k, N=n, ms_route=t_route * 1e3, ms_gemm=t_gemm * 1e3,
                tok_s=m / t_route, tops_gemm=ops / t_gemm / 1e12, tops_route=ops / t_route / 1e12)


# --------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on the host cores
# --------------------------------------------------------------------------

def cpu_baseline(synthetic, budget_s=15.0):
    from oracle import q4
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    wl = synthetic.WORKLOADS["decode_gate_up"]
    m, k, n = wl["M"], wl["K"], wl["N"]
    w = synthetic.weights(n, k, synthetic.WEIGHT_SEED)
    q, d = q4.quantize(w)          # preparation, not timed (as on the GPU)
    del w
    x = synthetic.activations(m, k, synthetic.ACT_SEED)
    q4.matmul(x, q, d)             # warm-up
    reps, t0 = 0, time.perf_counter()
    while True:
        q4.matmul(x, q, d)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    b = gemv_bytes(m, k, n)
    return dict(value=b * reps / el / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
                sample=f"oracle q4.matmul (dequantize to fp64, then fp64 matvec) on the full "
                       f"decode_gate_up matrix M={m} K={k} N={n}, {reps} calls in {el:.1f} s; "
                       f"host has {os.cpu_count()} logical CPUs")


# --------------------------------------------------------------------------
# traffic counters recorded under profiles/ (valid only for the same kernel source)
# --------------------------------------------------------------------------

def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("q4_gemv.hip", "q4w_internal.h"):
        with open(os.path.join(ROOT, "bit_quantized_weight_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    path = os.path.join(ROOT, "profiles", "skinny_decode_gate_up_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sections", default="decode,verify,step,prefill,pass",
                    help="comma list of extra sections (decode is always run)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 5 plain 512 MiB device copies (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build targets a single MI355X; sharding is described in the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_weight_amd as q4w
    from bit_quantized_weight_amd import synthetic

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    q4w.lib()  # fail loudly if the HIP library is missing
    sections = set(args.sections.split(","))

    if args.copy_calibration:
        src = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    log(f"[bench] decode_gate_up: {args.steps} steps, {args.warmup} warmup")
    dec = bench_decode(torch, q4w, synthetic, args.steps, args.warmup)
    log(f"[bench] decode_gate_up: {dec['gbs_graph']:.0f} GB/s graph, {dec['gbs_eager']:.0f} GB/s eager")
    extra = {}
    if "verify" in sections:
        extra["verify_down"] = bench_verify(torch, q4w, synthetic, max(args.steps // 3, 50), args.warmup)
        log("[bench] verify_down:", {mm: round(v["gbs_graph"]) for mm, v in extra["verify_down"]["per_M"].items()})
    if "step" in sections:
        extra["decode_step_64L"] = bench_decode_step(torch, q4w, synthetic, reps=10)
        log(f"[bench] decode_step_64L: {extra['decode_step_64L']['ms_graph']:.3f} ms graph")
    if "prefill" in sections:
        extra["a8w4_prefill"] = bench_prefill(torch, q4w, synthetic, reps=20)
        log(f"[bench] a8w4_prefill: route {extra['a8w4_prefill']['ms_route']:.3f} ms "
            f"({extra['a8w4_prefill']['tok_s']:.0f} tok/s), GEMM {extra['a8w4_prefill']['ms_gemm']:.3f} ms")
    if "pass" in sections:
        extra["a8w4_prefill_pass_64L"] = bench_prefill_pass(torch, q4w, synthetic, reps=3)
        for m_, r_ in extra["a8w4_prefill_pass_64L"]["per_M"].items():
            log(f"[bench] a8w4_prefill_pass_64L M={m_}: {r_['ms_graph']:.2f} ms ({r_['tok_s']:.0f} tok/s)")

    steps = args.steps
    t = dec["t_graph_s"]
    b = dec["bytes_per_launch"]
    achieved = b / (t / steps) / 1e9
    traffic = recorded_traffic()
    result = {
        "metric": "effective weight-stream GB/s (% of HBM peak) at M=1..5; A8W4 prefill tok/s",
        "value": round(b * steps / t / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(t / steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode_gate_up", "M": dec["M"], "K": dec["K"], "N": dec["N"],
                   "weight_format": "4-bit codes, fp16 scale per 32 weights",
                   "weight_copies_rotated": dec["copies"], "timing": "HIP graph of K launches"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "eager": {"gbs": round(dec["gbs_eager"], 2), "us_per_launch": round(dec["us_per_launch_eager"], 3)},
        "us_per_launch": round(dec["us_per_launch_graph"], 3),
        "kernel_source_hash": kernel_source_hash(),
    }
    result.update(extra)
    if "a8w4_prefill" in extra:
        p = extra["a8w4_prefill"]
        result["a8w4_prefill"]["roofline"] = {
            "bound": "mfma", "achieved": round(p["tops_gemm"], 2), "peak": INT8_PEAK_TOPS,
            "unit": "TOP/s", "frac": round(p["tops_gemm"] / INT8_PEAK_TOPS, 4), "traffic": None,
            "kernel": "a8w4 int8 GEMM (activations prepared once, timed per launch)"}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(synthetic)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
