"""Benchmark of the 4-bit weight-streaming matmul and the A8 prefill route on one MI355X.

Prints ONE JSON line on stdout.  A "step" is one pass of the hot path over
one batch: one skinny decode GEMV (M = 1, K = 5120, N = 17408, the FFN
gate/up shape) streaming one of >= 2 GB of distinct packed weight copies, so
the 256 MB Infinity Cache cannot serve it.  `value` is the effective
weight-stream bandwidth of those K steps (algorithmic bytes / time).

Timing.  The GPU is first run for about half a second so that its clocks
have left their idle state (the first timed region of a cold process reads
10-15% slow).  The timed region is the K launches issued on one stream
between two events; an untimed batch of K launches is queued in front, so
the GPU is already executing when the start event is reached and the host's
launch latency is not counted as GPU time.  The region is synchronized on
both sides.  The same K launches as one HIP graph replay are reported
beside it: a replay carries a fixed cost of about 12 us on this runtime (its
own start and completion), 5% of the region at K = 20, so the stream timing
is the one that measures the GEMVs.  Longer regions (a decode step, a
prefill pass, the A8 GEMM) replay their graph with one untimed replay in
front.  Extra sections, each timed the same way, cover the rest of the path:
  verify_down            K = 17408, N = 5120, M = 1..16 (speculative verify)
  decode_step_64L        64 layers x {qkv, out, gate, up, down}: M = 5 as a
                         320-launch graph, and M = 1, 4, 5 as one persistent launch
  attn_decode_256k       the K/V reads of a step's 16 attention layers at a 262,144-token
                         4-bit cache, M = 1..5
  decode_step_256k       a whole step at that context: the 64 layers' weights (one
                         persistent launch) plus the 16 layers' K/V reads, M = 5 and 1
  a8w4_prefill           M = 2048, K = 5120, N = 17408 (activation quant + int8 MFMA GEMM)
  a8w4_prefill_pass_64L  the 64-layer A8 pass at M = 512, 1024 and 2048
  read_ceiling           a plain streaming read (q4w_stream_read) of the same byte
                         counts: what this GPU reaches, beside the 8 TB/s peak
plus `roofline` for the dominant kernel and `cpu_baseline` (the oracle).
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0       # MI355X dense int8 MFMA, published
ROTATE_BYTES = 2 * 1024 ** 3  # distinct weight bytes cycled through per series
BYTES_PER_WEIGHT = 0.5625     # 4 bits + one fp16 scale per 32 weights
CLOCK_WARMUP_S = 0.5          # GPU time spent before anything is timed


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemv_bytes(m, k, n):
    """Algorithmic bytes of one skinny GEMV: packed weights + X + Y."""
    return int(n * k * BYTES_PER_WEIGHT) + 2 * m * k + 2 * m * n


# --------------------------------------------------------------------------
# timing helpers
# --------------------------------------------------------------------------

def time_region(torch, fn, preroll=None):
    """GPU seconds of fn(), between events on the current stream.  preroll
    (untimed) is enqueued first so the GPU is busy when the start event is
    reached; the region is synchronized on both sides."""
    s = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if preroll is not None:
        preroll()
    start.record(s)
    fn()
    stop.record(s)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3


def warm_clocks(torch, fn, seconds=CLOCK_WARMUP_S):
    """Run fn() (untimed work) until about `seconds` of GPU time have passed."""
    t = time_region(torch, fn)
    reps = max(1, int(seconds / max(t, 1e-6)))
    time_region(torch, lambda: [fn() for _ in range(reps)])


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


def time_graph(torch, g, reps=1):
    """GPU seconds of `reps` replays of g, with one untimed replay in front."""
    return time_region(torch, lambda: [g.replay() for _ in range(reps)], preroll=g.replay) / reps


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
    """Returns (stream seconds, graph seconds) for `steps` launches rotating
    over copies: the launches issued on the stream (an untimed batch of
    `steps` launches queued in front), and the same launches as one HIP
    graph replay.  With series > 1 each is timed that many times and the
    medians are returned (and the stream times as a third value)."""
    m, k = x.shape
    n = copies[0][0].shape[0]
    ws = torch.zeros(max(q4w.gemv_ws_bytes(m, n, k, 0), 1), dtype=torch.uint8, device="cuda")

    def launches(count, offset=0):
        for i in range(count):
            c, s = copies[(offset + i) % len(copies)]
            q4w.q4_gemv_skinny_raw(x, c, s, y, 0, ws)

    launches(warmup)
    t_stream = [time_region(torch, lambda: launches(steps), preroll=lambda: launches(steps))
                for _ in range(series)]
    g = capture(torch, lambda: launches(steps))
    g.replay()
    t_graph = [time_graph(torch, g) for _ in range(series)]
    del g
    med = lambda v: sorted(v)[len(v) // 2]   # noqa: E731
    if series == 1:
        return t_stream[0], t_graph[0]
    return med(t_stream), med(t_graph), t_stream


# --------------------------------------------------------------------------
# sections
# --------------------------------------------------------------------------

def bench_decode(torch, q4w, synthetic, steps, warmup):
    wl = synthetic.WORKLOADS["decode_gate_up"]
    m, k, n = wl["M"], wl["K"], wl["N"]
    copies = make_copies(torch, q4w, synthetic, n, k, 10_000)
    x = synthetic.activations_device(m, k, synthetic.ACT_SEED)
    y = torch.empty((m, n), dtype=torch.float16, device="cuda")
    ws = torch.zeros(max(q4w.gemv_ws_bytes(m, n, k, 0), 1), dtype=torch.uint8, device="cuda")
    warm_clocks(torch, lambda: [q4w.q4_gemv_skinny_raw(x, c, s, y, 0, ws) for c, s in copies])
    ts, tg = gemv_series(torch, q4w, copies, x, y, steps, warmup)
    # two more series of the same `steps` stream launches, for the spread (the
    # line's value is the first series)
    more = [gemv_series(torch, q4w, copies, x, y, steps, 0)[0] for _ in range(2)]
    b = gemv_bytes(m, k, n)
    out = dict(M=m, K=k, N=n, copies=len(copies), bytes_per_launch=b,
               t_stream_s=ts, t_graph_s=tg,
               gbs_stream=b * steps / ts / 1e9, gbs_graph=b * steps / tg / 1e9,
               us_per_launch_stream=ts / steps * 1e6, us_per_launch_graph=tg / steps * 1e6,
               us_per_launch_series=[t / steps * 1e6 for t in [ts] + more])
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
        # the previous M's graph capture left the GPU idle: warm the clock first
        ws = torch.zeros(max(q4w.gemv_ws_bytes(m, n, k, 0), 1), dtype=torch.uint8, device="cuda")
        warm_clocks(torch, lambda: [q4w.q4_gemv_skinny_raw(x, c, s, y, 0, ws) for c, s in copies])
        t, tg, ts = gemv_series(torch, q4w, copies, x, y, steps, warmup, series=3)
        b = gemv_bytes(m, k, n)
        res[str(m)] = dict(gbs=b * steps / t / 1e9, us_per_launch=t / steps * 1e6,
                           us_per_launch_min_max=[min(ts) / steps * 1e6, max(ts) / steps * 1e6],
                           frac_of_peak=b * steps / t / 1e9 / HBM_PEAK_GBS,
                           gbs_graph=b * steps / tg / 1e9)
    del copies
    torch.cuda.empty_cache()
    return dict(K=k, N=n, per_M=res)


def bench_decode_step(torch, q4w, synthetic, reps, ms=(5, 1, 4)):
    """64 layers x 5 projections, back to back on one stream: at M = 5 as a
    graph of 320 launches and as one persistent launch; at M = 1 and 4 as one
    persistent launch (the same packed weights)."""
    from bit_quantized_weight_amd.decode import DecodeStep
    out = {}
    base = None
    for m in ms:
        step = DecodeStep(m, weights=None if base is None else base.layers)
        torch.cuda.synchronize()
        total = step.weight_bytes + step.io_bytes
        r = dict(M=m, layers=len(step.layers), weight_bytes_per_step=step.weight_bytes)
        if base is None:
            for _ in range(2):
                step.run()
            warm_clocks(torch, step.run)
            t_eager = time_region(torch, lambda: [step.run() for _ in range(reps)], preroll=step.run) / reps
            g = capture(torch, step.run)
            g.replay()
            t_graph = time_graph(torch, g, reps)
            del g
            r.update(launches_per_step=step.launches, ms_graph=t_graph * 1e3, ms_eager=t_eager * 1e3,
                     gbs_graph=total / t_graph / 1e9, gbs_eager=total / t_eager / 1e9)
        step.plan_batched()
        # the graph capture and planning above leave the GPU idle: warm the
        # clock again on this launch before timing it
        warm_clocks(torch, step.run_batched)
        t_batched = time_region(torch, lambda: [step.run_batched() for _ in range(reps)],
                                preroll=step.run_batched) / reps
        r.update(ms_batched=t_batched * 1e3, gbs_batched=total / t_batched / 1e9,
                 frac_batched=total / t_batched / 1e9 / HBM_PEAK_GBS,
                 batched_grid=step.batch.plan.grid, batched_items=step.batch.plan.total_items)
        out[str(m)] = r
        if base is None:
            base = step
        else:
            del step
    del base
    torch.cuda.empty_cache()
    return out


def bench_attn(torch, q4w, synthetic, reps, t=262144, layers=16, ms=(1, 2, 3, 4, 5)):
    """The K/V attention read of one decode step: the 16 full-attention
    layers, each with its own 4-bit cache of t tokens (K and V rows of
    H_kv * D = 4 x 256), read back to back at M = 1..5 query tokens (20
    query heads).  Bytes per layer = both caches (codes and scales) + q + o."""
    hq, hkv, d = 20, 4, 256
    caches = []
    for layer in range(layers):
        kv = []
        for which in range(2):
            w = synthetic.weights_device(t, hkv * d, 50_000 + 2 * layer + which, std=1.0)
            kv.extend(q4w.pack(w))
            del w
        caches.append(kv)
    torch.cuda.synchronize()
    cache_bytes = 2 * int(t * hkv * d * BYTES_PER_WEIGHT)
    per_m = {}
    for m in ms:
        q = synthetic.activations_device(m * hq, d, 60_000 + m).reshape(m, hq, d)
        outs = [torch.empty_like(q) for _ in range(layers)]
        ws = torch.empty(max(q4w.attn_decode_ws_bytes(m, hq, hkv, d, t), 1), dtype=torch.uint8, device="cuda")

        def step():
            for (kc, ks, vc, vs), o in zip(caches, outs):
                q4w.attn_decode(q, kc, ks, vc, vs, hkv, out=o, ws=ws)

        if m == ms[0]:
            warm_clocks(torch, step)
        step()
        dt = time_region(torch, lambda: [step() for _ in range(reps)], preroll=step) / reps
        b = layers * (cache_bytes + 4 * m * hq * d)
        per_m[str(m)] = dict(ms_16_layers=dt * 1e3, us_per_layer=dt / layers * 1e6, gbs=b / dt / 1e9,
                             frac_of_peak=b / dt / 1e9 / HBM_PEAK_GBS)
        del outs, ws
    del caches
    torch.cuda.empty_cache()
    m1 = per_m[str(ms[0])]
    roof = {"bound": "hbm", "achieved": round(m1["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(m1["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic("attn_decode_256k_traffic.json", attn_source_hash()),
            "M": ms[0], "kernel": "attn_partial_kernel + attn_merge_kernel, one layer per launch pair",
            "kernel_source_hash": attn_source_hash()}
    return dict(T=t, layers=layers, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                cache_bytes_per_layer=cache_bytes, per_M=per_m, roofline=roof)


def bench_step_256k(torch, q4w, synthetic, reps=5, ms=(5, 1), t=262144, attn_layers=16):
    """One whole decode step at a 262,144-token context: the weights of all 64
    layers in one persistent launch, then the K/V reads of the 16
    full-attention layers (one launch pair each), back to back on one stream.
    The two HBM streams of a long-context step; the pages measure their sum as
    the drop from about 50 to 12.61 tok/s when the cache fills."""
    from bit_quantized_weight_amd.decode import DecodeStep
    hq, hkv, d = 20, 4, 256
    caches = []
    for layer in range(attn_layers):
        kv = []
        for which in range(2):
            w = synthetic.weights_device(t, hkv * d, 50_000 + 2 * layer + which, std=1.0)
            kv.extend(q4w.pack(w))
            del w
        caches.append(kv)
    cache_bytes = attn_layers * 2 * int(t * hkv * d * BYTES_PER_WEIGHT)
    out = {}
    base = None
    for m in ms:
        step = DecodeStep(m, weights=None if base is None else base.layers)
        step.plan_batched()
        q = synthetic.activations_device(m * hq, d, 60_000 + m).reshape(m, hq, d)
        outs = [torch.empty_like(q) for _ in range(attn_layers)]
        ws = torch.empty(max(q4w.attn_decode_ws_bytes(m, hq, hkv, d, t), 1), dtype=torch.uint8, device="cuda")

        def run():
            step.run_batched()
            for (kc, ks, vc, vs), o in zip(caches, outs):
                q4w.attn_decode(q, kc, ks, vc, vs, hkv, out=o, ws=ws)

        torch.cuda.synchronize()
        if base is None:
            warm_clocks(torch, run)
        run()
        dt = time_region(torch, lambda: [run() for _ in range(reps)], preroll=run) / reps
        total = step.weight_bytes + step.io_bytes + cache_bytes
        out[str(m)] = dict(M=m, ms_step=dt * 1e3, steps_per_s=1 / dt, bytes_per_step=total,
                           gbs=total / dt / 1e9, frac_of_peak=total / dt / 1e9 / HBM_PEAK_GBS,
                           weight_bytes=step.weight_bytes, kv_bytes=cache_bytes)
        del outs, ws
        if base is None:
            base = step
        else:
            del step
    del base, caches
    torch.cuda.empty_cache()
    return dict(T=t, attn_layers=attn_layers, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, per_M=out)


def bench_ceiling(torch, q4w, reps=40):
    """What a plain streaming read (q4w_stream_read) reaches on this GPU for
    the byte counts of the HBM-bound workloads: one decode_gate_up launch
    (50.2 MB), one attention layer (302 MB) and a long stream (2.4 GB), each
    rotating over copies in a 2.4 GB buffer so nothing is served from the
    256 MB Infinity Cache.  The achievable ceiling beside the 8 TB/s peak."""
    total = 2_415_919_104
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    cases = {"one_launch_50MB": (50_180_096, 200), "attn_layer_302MB": (301_989_888, reps),
             "long_stream_2400MB": (total, 5)}
    shapes = [(256, 512), (1024, 256), (2048, 256)]
    res = {}
    for name, (nbytes, n) in cases.items():
        stride = (nbytes + 255) // 256 * 256
        views = [buf[i * stride:i * stride + nbytes] for i in range(max(1, total // stride))]
        best = None
        per_shape = {}
        for grid, block in shapes:
            out = torch.empty(grid * (block // 64), dtype=torch.int32, device="cuda")

            def run():
                for i in range(n):
                    q4w.stream_read(views[i % len(views)], grid, block, out)

            warm_clocks(torch, run)
            dt_stream = time_region(torch, run, preroll=run) / n
            # Launched from Python, a ~9 us read of 50 MB is bounded by the host's
            # enqueue rate (about 10 us per call through the binding); one HIP
            # graph replay of the same n launches is not.
            g = capture(torch, run)
            g.replay()
            dt_graph = time_graph(torch, g) / n
            del g
            dt = min(dt_stream, dt_graph)
            per_shape[f"{grid}x{block}"] = dict(us_per_launch=dt * 1e6, gbs=nbytes / dt / 1e9,
                                                us_per_launch_stream=dt_stream * 1e6,
                                                us_per_launch_graph=dt_graph * 1e6)
            if best is None or dt < best[0]:
                best = (dt, f"{grid}x{block}")
        res[name] = dict(bytes=nbytes, copies=len(views), best_shape=best[1], us_per_launch=best[0] * 1e6,
                         gbs=nbytes / best[0] / 1e9, frac_of_peak=nbytes / best[0] / 1e9 / HBM_PEAK_GBS,
                         per_shape=per_shape)
    del buf
    torch.cuda.empty_cache()
    return res


def bench_prefill_pass(torch, q4w, synthetic, reps, ms=(512, 1024, 2048)):
    """64 layers x 5 projections on the A8 route at M = 512, 1024 and 2048
    tokens (one packed weight set): per layer three activation quantizations
    and four GEMMs (gate and up as one), as a HIP graph."""
    from bit_quantized_weight_amd.prefill import PrefillPass
    weights = None
    per_m = {}
    for m in ms:
        p = PrefillPass(m, weights=weights)
        weights = p.layers
        torch.cuda.synchronize()
        p.run()
        t_eager = time_region(torch, lambda: [p.run() for _ in range(reps)], preroll=p.run) / reps
        g = capture(torch, p.run)
        g.replay()
        t_graph = time_graph(torch, g, reps)
        per_m[str(m)] = dict(int_ops_per_pass=p.int_ops, ms_graph=t_graph * 1e3, ms_eager=t_eager * 1e3,
                             tok_s=m / t_graph, tops=p.int_ops / t_graph / 1e12)
        layers = len(p.layers)
        del g, p
        torch.cuda.empty_cache()
    del weights
    torch.cuda.empty_cache()
    return dict(layers=layers, launches_per_pass=7 * layers, per_M=per_m)


def bench_prefill(torch, q4w, synthetic, reps, gemm_only=False):
    """A8 route at M = 2048, one projection (K = 5120, N = 17408): the GEMM
    alone from prepared activations (the dominant kernel), then the whole
    route per call (activation quantization + GEMM).  gemm_only: the GEMM
    alone (one activation quantization in front), for profiling that kernel."""
    wl = synthetic.WORKLOADS["prefill_a8"]
    m, k, n = wl["M"], wl["K"], wl["N"]
    w = synthetic.weights_device(n, k, synthetic.WEIGHT_SEED)
    codes, scales = q4w.pack(w)
    del w
    x = synthetic.activations_device(m, k, synthetic.ACT_SEED)
    y = torch.empty((m, n), dtype=torch.float16, device="cuda")
    ws = q4w.a8w4_prepare(x)
    gemm = lambda: q4w.a8w4_gemm_prepared(ws, m, k, codes, scales, y)   # noqa: E731
    warm_clocks(torch, gemm)
    t_gemm = time_region(torch, lambda: [gemm() for _ in range(reps)], preroll=gemm) / reps
    ops = 2 * m * n * k
    if gemm_only:
        return dict(M=m, K=k, N=n, ms_gemm=t_gemm * 1e3, tops_gemm=ops / t_gemm / 1e12)
    route = lambda: q4w.a8w4_gemm(x, codes, scales, y)                   # noqa: E731
    route()
    t_route = time_region(torch, lambda: [route() for _ in range(reps)], preroll=route) / reps
    t_quant = time_region(torch, lambda: [q4w.a8w4_prepare(x, ws) for _ in range(reps)],
                          preroll=lambda: q4w.a8w4_prepare(x, ws)) / reps
    return dict(M=m, K=k, N=n, ms_route=t_route * 1e3, ms_gemm=t_gemm * 1e3, ms_act_quant=t_quant * 1e3,
                one_projection_tokens_per_s=m / t_route,
                tops_gemm=ops / t_gemm / 1e12, tops_route=ops / t_route / 1e12)


# --------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on the host cores
# --------------------------------------------------------------------------

def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def _timed_calls(fn, budget_s):
    fn()                                     # warm-up
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            return reps, el


def cpu_baseline(synthetic, budget_s=4.0):
    """The oracle, untuned, on the host, each workload with all BLAS threads
    and with one: the headline GEMV, the verify down-projection at M = 5 and
    the exact A8 route on a token sample of the M = 2048 projection; plus one
    layer of the 64-layer decode step at M = 5 (its five projections),
    extrapolated to the whole step."""
    from oracle import a8, q4
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    threads = _blas_threads()

    def both(fn):
        """(reps, seconds) with all threads, and with one thread (or None)."""
        r = _timed_calls(fn, budget_s)
        if threadpool_limits is None:
            return r, None
        with threadpool_limits(limits=1):
            return r, _timed_calls(fn, budget_s)

    out = {}
    # headline: decode_gate_up, M = 1
    wl = synthetic.WORKLOADS["decode_gate_up"]
    m, k, n = wl["M"], wl["K"], wl["N"]
    w = synthetic.weights(n, k, synthetic.WEIGHT_SEED)
    q, d = q4.quantize(w)          # preparation, not timed (as on the GPU)
    del w
    x = synthetic.activations(m, k, synthetic.ACT_SEED)
    b = gemv_bytes(m, k, n)
    (reps, el), one = both(lambda: q4.matmul(x, q, d))
    out.update(value=b * reps / el / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
               sample=f"oracle q4.matmul (dequantize to fp64, then fp64 matvec) on the full "
                      f"decode_gate_up matrix M={m} K={k} N={n}, {reps} calls in {el:.1f} s; "
                      f"{threads} BLAS threads; host has {os.cpu_count()} logical CPUs")
    if one:
        out["single_thread"] = dict(value=b * one[0] / one[1] / 1e9, unit="GB/s", cores=1,
                                    sample=f"same, {one[0]} calls in {one[1]:.1f} s, 1 BLAS thread")
    del q, d
    # verify down-projection, M = 5 (K = 17408, N = 5120)
    wl = synthetic.WORKLOADS["verify_down"]
    k, n, m = wl["K"], wl["N"], 5
    w = synthetic.weights(n, k, synthetic.WEIGHT_SEED)
    q, d = q4.quantize(w)
    del w
    x = synthetic.activations(m, k, synthetic.ACT_SEED)
    b = gemv_bytes(m, k, n)
    (reps, el), one = both(lambda: q4.matmul(x, q, d))
    out["verify_down_m5"] = dict(value=b * reps / el / 1e9, unit="GB/s", cores=int(threads),
                                 sample=f"q4.matmul M={m} K={k} N={n}, {reps} calls in {el:.1f} s")
    if one:
        out["verify_down_m5"]["single_thread"] = dict(value=b * one[0] / one[1] / 1e9, unit="GB/s", cores=1,
                                                      sample=f"same, {one[0]} calls in {one[1]:.1f} s")
    del q, d
    # A8 route, M = 2048, K = 5120, N = 17408: the exact oracle on 64 of the tokens
    wl = synthetic.WORKLOADS["prefill_a8"]
    m, k, n = wl["M"], wl["K"], wl["N"]
    w = synthetic.weights(n, k, synthetic.WEIGHT_SEED)
    q, d = q4.quantize(w)
    del w
    tokens = 64
    x = synthetic.activations(tokens, k, synthetic.ACT_SEED)
    (reps, el), one = both(lambda: a8.prefill(x, q, d))
    out["a8_prefill"] = dict(value=tokens * reps / el, unit="tokens/s", cores=int(threads),
                             tops=2 * tokens * n * k * reps / el / 1e12,
                             sample=f"a8.prefill (int8 quantization, 160 fp64 K=32 GEMMs of exact block "
                                    f"sums, fp64 rescale) on {tokens} tokens x K={k} x N={n}, "
                                    f"{reps} calls in {el:.1f} s")
    if one:
        out["a8_prefill"]["single_thread"] = dict(value=tokens * one[0] / one[1], unit="tokens/s", cores=1,
                                                  tops=2 * tokens * n * k * one[0] / one[1] / 1e12,
                                                  sample=f"same, {one[0]} calls in {one[1]:.1f} s")
    del q, d
    # decode step, M = 5: layer 0's five projections, one at a time, scaled to 64 layers
    m = 5
    layer = []
    for pi, (_, k, n) in enumerate(synthetic.LAYER_PROJECTIONS):
        w = synthetic.weights(n, k, synthetic.layer_weight_seed(0, pi))
        q, d = q4.quantize(w)
        del w
        layer.append((synthetic.activations(m, k, synthetic.ACT_SEED), q, d))
    step_layer = lambda: [q4.matmul(x, q, d) for x, q, d in layer]
    reps, el = _timed_calls(step_layer, budget_s)
    t_layer = el / reps
    wbytes = sum(int(n * k * BYTES_PER_WEIGHT) for _, k, n in synthetic.LAYER_PROJECTIONS) * synthetic.N_LAYERS
    out["decode_step_m5"] = dict(value=wbytes / (t_layer * synthetic.N_LAYERS) / 1e9, unit="GB/s",
                                 cores=int(threads), ms_per_step=t_layer * synthetic.N_LAYERS * 1e3,
                                 sample=f"q4.matmul over layer 0's five projections at M={m} "
                                        f"(qkv, out, gate, up, down), {reps} layer passes in {el:.1f} s, "
                                        f"times {synthetic.N_LAYERS} layers")
    del layer
    return out


# --------------------------------------------------------------------------
# traffic counters recorded under profiles/ (valid only for the same kernel source)
# --------------------------------------------------------------------------

def code_text(text):
    """Source text with comments and blank lines removed: a change to the
    comments alone leaves the compiled kernel, and so its counters, as they were."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.split("\n") if line.strip()) + "\n"


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "bit_quantized_weight_amd", "csrc", f)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def kernel_source_hash():
    """The skinny kernel's own sources (the kernel, its plan and split-K fixup)."""
    return source_hash(("q4_gemv.hip", "splitk.h"))


def a8_source_hash():
    return source_hash(("a8w4.hip",))


def attn_source_hash():
    return source_hash(("q4_attn.hip",))


def recorded_traffic(name, current_hash):
    path = os.path.join(ROOT, "profiles", name)
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != current_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sections", default="decode,verify,step,attn,step256k,prefill,pass,ceiling",
                    help="comma list of extra sections (decode is always run)")
    ap.add_argument("--only", default=None,
                    help="run only this section (decode, verify, step, attn, step256k, prefill, gemm (the A8 GEMM "
                         "alone), pass, ceiling) and print its "
                         "result; for profiling one kernel")
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

    if args.copy_calibration:
        src = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    if args.only:
        fn = {"decode": lambda: bench_decode(torch, q4w, synthetic, args.steps, args.warmup),
              "verify": lambda: bench_verify(torch, q4w, synthetic, max(args.steps // 3, 50), args.warmup),
              "step": lambda: bench_decode_step(torch, q4w, synthetic, reps=10),
              "prefill": lambda: bench_prefill(torch, q4w, synthetic, reps=max(args.steps, 5)),
              "attn": lambda: bench_attn(torch, q4w, synthetic, reps=max(args.steps // 10, 3)),
              "pass": lambda: bench_prefill_pass(torch, q4w, synthetic, reps=3),
              "gemm": lambda: bench_prefill(torch, q4w, synthetic, reps=max(args.steps, 5), gemm_only=True),
              "ceiling": lambda: bench_ceiling(torch, q4w),
              "step256k": lambda: bench_step_256k(torch, q4w, synthetic)}[args.only]
        print(json.dumps({args.only: fn()}), flush=True)
        return

    sections = set(args.sections.split(","))
    log(f"[bench] decode_gate_up: {args.steps} steps, {args.warmup} warmup")
    dec = bench_decode(torch, q4w, synthetic, args.steps, args.warmup)
    log(f"[bench] decode_gate_up: {dec['gbs_stream']:.0f} GB/s, {dec['gbs_graph']:.0f} GB/s as one graph")
    extra = {}
    if "verify" in sections:
        extra["verify_down"] = bench_verify(torch, q4w, synthetic, max(args.steps // 3, 50), args.warmup)
        log("[bench] verify_down:", {mm: round(v["gbs"]) for mm, v in extra["verify_down"]["per_M"].items()})
    if "step" in sections:
        extra["decode_step_64L"] = bench_decode_step(torch, q4w, synthetic, reps=10)
        log("[bench] decode_step_64L:",
            {mm: round(v["ms_batched"], 3) for mm, v in extra["decode_step_64L"].items()},
            f"ms batched; M=5 graph {extra['decode_step_64L']['5']['ms_graph']:.3f} ms")
    if "attn" in sections:
        extra["attn_decode_256k"] = bench_attn(torch, q4w, synthetic, reps=5)
        log("[bench] attn_decode_256k:", {mm: round(v["gbs"]) for mm, v in extra["attn_decode_256k"]["per_M"].items()},
            "GB/s")
    if "prefill" in sections:
        extra["a8w4_prefill"] = bench_prefill(torch, q4w, synthetic, reps=20)
        p = extra["a8w4_prefill"]
        log(f"[bench] a8w4_prefill: GEMM {p['ms_gemm']:.3f} ms, route {p['ms_route']:.3f} ms, "
            f"act quant {p['ms_act_quant']:.4f} ms")
    if "step256k" in sections:
        extra["decode_step_256k"] = bench_step_256k(torch, q4w, synthetic)
        log("[bench] decode_step_256k:", {k_: round(v_["ms_step"], 3) for k_, v_ in extra["decode_step_256k"]["per_M"].items()},
            "ms per step")
    if "ceiling" in sections:
        extra["read_ceiling"] = bench_ceiling(torch, q4w)
        log("[bench] read_ceiling:", {k_: round(v_["gbs"]) for k_, v_ in extra["read_ceiling"].items()}, "GB/s")
    if "pass" in sections:
        extra["a8w4_prefill_pass_64L"] = bench_prefill_pass(torch, q4w, synthetic, reps=3)
        for m_, r_ in extra["a8w4_prefill_pass_64L"]["per_M"].items():
            log(f"[bench] a8w4_prefill_pass_64L M={m_}: {r_['ms_graph']:.2f} ms ({r_['tok_s']:.0f} tok/s)")

    steps = args.steps
    t = dec["t_stream_s"]
    b = dec["bytes_per_launch"]
    achieved = b / (t / steps) / 1e9
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
                   "weight_copies_rotated": dec["copies"],
                   "timing": "K launches on one stream between two events, an untimed batch of K "
                             "launches queued in front, after clock warm-up"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("skinny_decode_gate_up_traffic.json", kernel_source_hash())},
        "graph": {"gbs": round(dec["gbs_graph"], 2), "us_per_launch": round(dec["us_per_launch_graph"], 3),
                  "note": "the same K launches as one HIP graph replay, which adds a fixed cost per replay"},
        "us_per_launch": round(dec["us_per_launch_stream"], 3),
        "us_per_launch_series": [round(t, 3) for t in dec["us_per_launch_series"]],
        "kernel_source_hash": kernel_source_hash(),
    }
    result.update(extra)
    if "a8w4_prefill" in extra:
        p = extra["a8w4_prefill"]
        result["a8w4_prefill"]["roofline"] = {
            "bound": "mfma", "achieved": round(p["tops_gemm"], 2), "peak": INT8_PEAK_TOPS,
            "unit": "TOP/s", "frac": round(p["tops_gemm"] / INT8_PEAK_TOPS, 4),
            "traffic": recorded_traffic("a8w4_prefill_gemm_traffic.json", a8_source_hash()),
            "kernel": "a8w4 int8 GEMM (activations prepared once, timed per launch)",
            "kernel_source_hash": a8_source_hash()}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(synthetic)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
