"""Throughput of the H2O chunk path: attention + summed weights + score update +
eviction/insert, over a whole synthetic sequence, on one MI355X.

A step is one full sequence of the workload pushed through the path chunk by chunk
(h2o_chunk_attn, then h2o_update_evict_and_insert: the score update, selection and
insertion, with the update inside the selection kernel) from an empty cache (default: Qwen3-4B attention shape, 32 query /
8 KV heads, head_dim 128, bf16, chunk 1024, cache 8192, recent window 256, 64k
tokens = 64 chunks).  Inputs are resident in HBM before the timed region.

Prints one JSON line.  `value` is F6 TFLOP/s: 6*d*Hq*(visible query/key pairs),
i.e. QK^T and PV for the output plus the QK^T recompute for the summed weights.

`--workload 4` runs the 36-layer stack of the same attention shape (cache 8192,
chunk 1k, 128k tokens): each step pushes one chunk through all 36 layers, each
layer from its own full cache with its own seeded inputs; `value` is ms per
chunk across the layers.

`--policy lastrec` runs the same sequence under the lastrec policy (attention
without summed weights, eviction by position keeping the first `--sink`
tokens); its `value` is F4 TFLOP/s, the work that policy does.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "H2O chunk-attn+score+evict TFLOP/s & tokens/s (chunk 1k, 64k ctx), % roofline"
METRIC_CHUNK2K = "H2O chunk-attn+score+evict TFLOP/s & tokens/s (chunk 2k, 128k ctx), % roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_chunk1k_ctx64k_traffic.txt")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_b16_cache16k_traffic.txt")


def pairs_per_head(n_before: int, S: int) -> int:
    """Visible (query, key) pairs of one chunk for one query head."""
    return S * n_before + S * (S + 1) // 2


def chunk_schedule(wl):
    n = 0
    out = []
    for _ in range(wl.n_chunks):
        out.append(n)
        n = min(wl.capacity, n + wl.chunk)
    return out


def read_traffic(path: str):
    """HBM bytes per launch of the dominant kernel from a committed rocprofv3
    counter summary, or None unless it was taken on the current kernel source."""
    try:
        fields = {}
        for line in open(path):
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                fields[k.strip()] = v.strip()
        src = os.path.join(ROOT, fields["kernel_source"])
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        if fields.get("kernel_source_sha256_16") != digest:
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(wl, budget_s: float):
    """The fp64 oracle on steady (full-cache) chunks of the same workload."""
    import oracle
    import workloads as W
    threads = blas_threads()
    c = 16
    s = W.steady_state(wl, 0, start=c * wl.chunk, seed=0)
    x = W.chunk_inputs(wl, 0, c)
    flops = 0.0
    chunks = 0
    t0 = time.perf_counter()
    while True:
        st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
        oracle.h2o_step(st, x["q"], x["k"], x["v"], wl.sm_scale, wl.recent_window)
        chunks += 1
        flops += 6.0 * wl.head_dim * wl.n_q_heads * pairs_per_head(wl.capacity, wl.chunk)
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{chunks} steady chunk(s) of {wl.name} (full cache, "
                     f"{wl.capacity}+{wl.chunk} keys, fp64 NumPy), {dt:.1f} s",
           "tokens_per_s": chunks * wl.chunk / dt, "ms_per_chunk": dt / chunks * 1e3}
    # The same oracle on one thread, one chunk.
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"],
                                             s["start"])
            t1 = time.perf_counter()
            oracle.h2o_step(st, x["q"], x["k"], x["v"], wl.sm_scale, wl.recent_window)
            d1 = time.perf_counter() - t1
        f1 = 6.0 * wl.head_dim * wl.n_q_heads * pairs_per_head(wl.capacity, wl.chunk)
        out["one_thread"] = {"value": f1 / d1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                             "ms_per_chunk": d1 * 1e3, "sample": "1 steady chunk"}
    except ImportError:  # pragma: no cover
        out["one_thread"] = None
    return out


def copy_probe(mib: int) -> None:
    """Plain device copies of a known size (mib MiB read, mib MiB written), run
    before the workload so that HBM byte counters read for the path's kernels
    can be scaled by what the same counters read for a copy."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    print(f"[bench] copy probe: 3 x copy_ and 3 x neg of {mib} MiB", file=sys.stderr,
          flush=True)


DECODE_METRIC = "H2O decode step (attn+score+evict) tokens/s, % HBM roofline"
LASTREC_METRIC = "lastrec chunk-attn+evict TFLOP/s & tokens/s (chunk 1k, 64k ctx), % roofline"
LASTREC_DECODE_METRIC = "lastrec decode step (attn+evict) tokens/s, % HBM roofline"
BUFFER_METRIC = ("H2O insert-first buffer chunk-attn+score+evict TFLOP/s & tokens/s "
                 "(chunk 1k, 64k ctx), % roofline")
BUFFER_DECODE_METRIC = "H2O insert-first buffer decode step tokens/s, % HBM roofline"


def decode_slot_bytes(wl, policy="h2o") -> int:
    """Algorithmic HBM bytes per cache slot per decode step: K and V rows read,
    the position read, and under h2o the score read and written."""
    return 2 * wl.head_dim * 2 + 4 + (8 if policy == "h2o" else 0)


def capture(fn, reset):
    """Capture fn (a whole sequence of library calls) into a HIP graph after one
    warm run on the capturing stream, as torch requires."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def check_replay(name, pairs):
    """Graph replays must give the eager results bit for bit (the kernels are
    deterministic); a mismatch is reported and fails the run."""
    import torch
    for got, want in pairs:
        if not torch.equal(got, want):
            print(f"[bench] ERROR: {name} graph replay differs from the eager run",
                  file=sys.stderr, flush=True)
            sys.exit(3)


SPIN_CYCLES = 2_000_000      # torch.cuda._sleep: at least ~1 ms at any shader clock


def steady_chunk(wl, dims, step_kw, bufs, reps: int = 10):
    """One chunk of the path (all its calls) on a full cache, replayed from a captured HIP
    graph and timed alone with HIP events on the replay stream: the cache is reloaded from
    a snapshot before each repetition, outside the events.  Returns the median in
    microseconds."""
    import torch

    import h2o_sparse_attention_amd as h2o
    import workloads as W

    dev = torch.device("cuda:0")
    dt = dims.torch_dtype
    c = wl.n_chunks // 2
    s = W.steady_state(wl, 0, start=c * wl.chunk)
    x = W.chunk_inputs(wl, 0, c)
    snap = [torch.from_numpy(s[k]).to(dev, dt if k in ("k", "v") else None)
            for k in ("k", "v", "pos", "phi")]
    q, k, v = (torch.from_numpy(x[key]).to(dev, dt) for key in ("q", "k", "v"))
    cache = h2o.H2OCache(dims, dev)

    def reset():
        cache.load(*snap, s["n"], s["start"])

    graph = capture(lambda: h2o.step(cache, q, k, v, wl.sm_scale, bufs=bufs, **step_kw), reset)
    times = []
    for r in range(reps + 2):
        reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # A device-side spin ahead of the start event keeps the GPU busy while the
        # host submits the event and the graph, so the interval holds the chunk's
        # GPU work and not the host's submission latency.
        torch.cuda._sleep(SPIN_CYCLES)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        if r >= 2:
            times.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(times))


def measured_peaks():
    """Achievable rates on this GPU for comparison with the datasheet peaks: a large bf16
    GEMM through torch (hipBLASLt), a 1 GiB device copy and a 1 GiB read (torch's sum)."""
    import torch
    dev = torch.device("cuda:0")
    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy = 2.0 * src.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del dst
    for _ in range(3):
        src.sum()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        src.sum()
    e1.record()
    torch.cuda.synchronize()
    read = src.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src
    return {"gemm_bf16_8192_tflops": round(gemm, 1), "copy_1gib_gbs": round(copy, 1),
            "read_1gib_gbs": round(read, 1)}


def blas_threads() -> int:
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        return max((i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"),
                   default=1)
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def decode_cpu_baseline(wl, st0, budget_s: float, max_steps: int = 8):
    """The fp64 oracle on the first decode steps of the workload (at most max_steps,
    or fewer if budget_s runs out), from the same initial cache; per-step time
    extrapolated linearly to the whole run."""
    import oracle
    import workloads as W
    st = oracle.H2OState.from_arrays(st0["k"], st0["v"], st0["pos"], st0["phi"], st0["n"],
                                     st0["start"])
    t0 = time.perf_counter()
    steps = 0
    while steps < max_steps:
        x = W.decode_step_inputs(wl, steps)
        oracle.h2o_step(st, x["q"], x["k"], x["v"], wl.sm_scale, wl.recent_window)
        steps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    per_step = dt / steps
    return {"value": round(wl.batch * steps / dt, 2), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{steps} decode step(s) of {wl.name} ({wl.batch} sequences x "
                      f"{wl.n_kv_heads} KV heads x {wl.capacity} slots, fp64 NumPy), "
                      f"{dt:.1f} s; linear extrapolation to the {wl.seq_len}-step run: "
                      f"{per_step * wl.seq_len:.0f} s",
            "us_per_decode_step": round(per_step * 1e6, 1)}


def run_decode(args):
    import torch

    import h2o_sparse_attention_amd as h2o
    import workloads as W

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    dims = h2o.H2ODims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.capacity,
                       wl.recent_window, wl.dtype)
    dt = dims.torch_dtype
    t_gen = time.perf_counter()
    st = W.decode_initial_state(wl)
    snap = {k: torch.from_numpy(st[k]).to(dev, dt if k in ("k", "v") else None)
            for k in ("k", "v", "pos", "phi")}
    st_host = st if (args.cpu_budget > 0 and args.policy == "h2o") else None
    del st
    steps_in = []
    for t in range(wl.seq_len):
        x = W.decode_step_inputs(wl, t)
        steps_in.append(tuple(torch.from_numpy(x[k]).to(dev, dt) for k in ("q", "k", "v")))
    print(f"[bench] decode state + {wl.seq_len} steps generated in "
          f"{time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    cache = h2o.H2OCache(dims, dev)
    B, Hq, Hkv, D, NC = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.capacity
    bufs = {"out": torch.empty(B, Hq, 1, D, dtype=dt, device=dev),
            "lse": torch.empty(B, Hq, 1, dtype=torch.float32, device=dev),
            "colsum_cache": torch.empty(B, Hkv, NC, dtype=torch.float32, device=dev),
            "colsum_new": torch.empty(B, Hkv, 1, dtype=torch.float32, device=dev),
            "freed_slots": torch.empty(B, Hkv, 1, dtype=torch.int32, device=dev),
            "workspace": torch.zeros(h2o.workspace_bytes(dims, 1), dtype=torch.uint8, device=dev)}

    step_kw = dict(policy=args.policy, sink_tokens=args.sink)

    def reset():
        cache.load(snap["k"], snap["v"], snap["pos"].to(torch.int32), snap["phi"].float(),
                   NC, NC)

    def run(nsteps):
        for t in range(nsteps):
            q, k, v = steps_in[t % len(steps_in)]
            h2o.step(cache, q, k, v, wl.sm_scale, bufs=bufs, **step_kw)

    for _ in range(args.warmup):
        reset()
        run(wl.seq_len)
    reset()
    torch.cuda.synchronize()
    # Per-kernel means: one eager pass with the library's kernel timers.
    n_launch = args.steps * wl.seq_len
    kernels = ("decode", "decode_finish", "update", "select", "insert")
    if args.policy == "lastrec":
        kernels = ("decode", "decode_finish", "select", "insert")
    timers = {k: h2o.KernelTimer(k, n_launch) for k in kernels}
    for t_ in timers.values():
        t_.__enter__()
    eager_s = 0.0
    for _ in range(args.steps):
        reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(wl.seq_len)
        torch.cuda.synchronize()
        eager_s += time.perf_counter() - t0
    for t_ in timers.values():
        t_.__exit__(None, None, None)
    ref_out = bufs["out"].clone()
    ref_score = cache.score.clone()
    ref_pos = cache.pos.clone()
    # Timed region: the 512 steps replayed from one captured HIP graph (the
    # snapshot reload between replays is outside the timed region).
    total_s = eager_s
    if not args.no_graph:
        graph = capture(lambda: run(wl.seq_len), reset)
        total_s = 0.0
        for _ in range(args.steps):
            reset()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            graph.replay()
            torch.cuda.synchronize()
            total_s += time.perf_counter() - t0
        check_replay("decode", [(bufs["out"], ref_out), (cache.score, ref_score),
                                (cache.pos, ref_pos)])
    n_tok = args.steps * wl.seq_len * B
    us_per_step = total_s / (args.steps * wl.seq_len) * 1e6
    slot_bytes = decode_slot_bytes(wl, args.policy)
    step_bytes = B * Hkv * NC * slot_bytes
    dec = timers["decode"]
    # Algorithmic bytes per slot of the attention launch: K and V rows and the
    # position read; with summed weights, their write; under h2o the score read and
    # written as well (the score update and eviction keys are formed in this launch).
    kern_slot_bytes = (2 * D * 2 + 4 + (0 if args.policy == "lastrec" else 4)
                       + (8 if args.policy == "h2o" else 0))
    achieved = B * Hkv * NC * kern_slot_bytes / (dec.mean_ms * 1e-3) / 1e9
    kernel_name = {"h2o": "decode_attn4_kernel<128, 3>", "h2o_buffer": "decode_attn4_kernel<128, 2>",
                   "lastrec": "decode_attn4_kernel<128, 0>"}[args.policy]
    peaks = measured_peaks()
    cpu = None
    if st_host is not None:
        print("[bench] cpu baseline ...", file=sys.stderr, flush=True)
        cpu = decode_cpu_baseline(wl, st_host, args.cpu_budget)
    line = {
        "metric": {"h2o": DECODE_METRIC, "h2o_buffer": BUFFER_DECODE_METRIC,
                   "lastrec": LASTREC_DECODE_METRIC}[args.policy],
        "value": round(n_tok / total_s, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(total_s / args.steps * 1e3, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "capacity": NC, "recent_window": wl.recent_window,
                   "decode_steps": wl.seq_len, "policy": args.policy,
                   **({"sink_tokens": args.sink} if args.policy == "lastrec" else {}),
                   "parallelism": "single-gpu"},
        "timing": "hip_graph" if not args.no_graph else "eager",
        "us_per_decode_step": round(us_per_step, 2),
        "us_per_decode_step_eager": round(eager_s / (args.steps * wl.seq_len) * 1e6, 2),
        "step_hbm_gbs": round(step_bytes / (us_per_step * 1e-6) / 1e9, 1),
        "frac_hbm_peak_step": round(step_bytes / (us_per_step * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "kernel_mean_us": {k: round(t_.mean_ms * 1e3, 2) for k, t_ in timers.items()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": (read_traffic(DECODE_TRAFFIC_FILE) if args.policy == "h2o"
                                 else None),
                     "kernel": kernel_name, "bytes_per_slot": kern_slot_bytes,
                     "launches": dec.launches,
                     "mean_launch_us": round(dec.mean_ms * 1e3, 2)},
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


BACKWARD_METRIC = "H2O chunk-attn backward TFLOP/s (chunk 1k, cache 8192, steady chunk), % roofline"


def run_backward(args):
    """Backward of one steady chunk (full cache) repeated: the gradients of the chunk
    attention w.r.t. q, the chunk's k/v and the cached slots' k/v."""
    import torch

    import h2o_sparse_attention_amd as h2o
    import workloads as W

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    dims = h2o.H2ODims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.capacity,
                       wl.recent_window, wl.dtype)
    dt = dims.torch_dtype
    c = 16
    s = W.steady_state(wl, 0, start=c * wl.chunk)
    x = W.chunk_inputs(wl, 0, c)
    cache = h2o.H2OCache(dims, dev)
    cache.load(torch.from_numpy(s["k"]).to(dev, dt), torch.from_numpy(s["v"]).to(dev, dt),
               torch.from_numpy(s["pos"]).to(dev), torch.from_numpy(s["phi"]).to(dev),
               s["n"], s["start"])
    q, k, v = (torch.from_numpy(x[key]).to(dev, dt) for key in ("q", "k", "v"))
    B, Hq, Hkv, D, NC, S = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.capacity, wl.chunk
    P = s["start"]
    out, lse, _, _ = h2o.chunk_attn(cache, P, q, k, v, wl.sm_scale, summed_weights=False)
    g = torch.Generator(device="cpu").manual_seed(7)
    dout = torch.randn(B, Hq, S, D, generator=g).to(dev, dt)
    grads = {"dq": torch.empty(B, Hq, S, D, device=dev), "dk_new": torch.empty(B, Hkv, S, D, device=dev),
             "dv_new": torch.empty(B, Hkv, S, D, device=dev),
             "dk_cache": torch.empty(B, Hkv, NC, D, device=dev),
             "dv_cache": torch.empty(B, Hkv, NC, D, device=dev)}
    ws = torch.empty(int(h2o.lib.h2o_backward_workspace_bytes(ctypes_byref(dims), S)),
                     dtype=torch.uint8, device=dev)

    def step():
        h2o.chunk_attn_backward(cache, P, q, k, v, out, lse, dout, wl.sm_scale, grads=grads,
                                workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer = h2o.KernelTimer("backward", args.steps)
    with timer:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    pairs = pairs_per_head(NC, S)
    flops = 10.0 * D * Hq * B * pairs         # QK^T recompute, dP, dQ, dK, dV
    ms = elapsed / args.steps * 1e3
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        print("[bench] cpu baseline ...", file=sys.stderr, flush=True)
        st = oracle.H2OState.from_arrays(s["k"], s["v"], s["pos"], s["phi"], s["n"], s["start"])
        dout_h = dout.float().cpu().numpy()
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.attend_chunk_backward(st, x["q"], x["k"], x["v"], dout_h, wl.sm_scale)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_budget:
                break
        dtc = time.perf_counter() - t0
        cpu = {"value": round(flops * reps / dtc / 1e12, 4), "unit": "TFLOP/s",
               "cores": blas_threads(), "kind": "oracle",
               "sample": f"{reps} steady chunk backward(s) of {wl.name} ({NC}+{S} keys, "
                         f"fp64 NumPy), {dtc:.1f} s",
               "ms_per_chunk": round(dtc / reps * 1e3, 1)}
    tflops = flops / (ms * 1e-3) / 1e12
    achieved = flops / (timer.mean_ms * 1e-3) / 1e12
    line = {
        "metric": BACKWARD_METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name + " steady chunk backward", "batch": B, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "capacity": NC, "chunk": S,
                   "parallelism": "single-gpu"},
        "timing": "eager",
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "h2o_chunk_attn_backward (row-dot, dQ, dK/dV)",
                     "launches": timer.launches, "mean_launch_us": round(timer.mean_ms * 1e3, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


STACK_METRIC = "H2O 36-layer stack ms per chunk across layers (chunk 1k, cache 8192, 128k ctx)"


def run_stack(args):
    """The layer stack: each timed step pushes one chunk through every layer (chunk-major,
    as a model runs it), each layer with its own full cache and its own seeded inputs.
    The caches start as steady full caches before the middle chunk of the sequence."""
    from concurrent.futures import ThreadPoolExecutor

    import torch

    import h2o_sparse_attention_amd as h2o
    import workloads as W

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    dims = h2o.H2ODims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.capacity,
                       wl.recent_window, wl.dtype)
    dt = dims.torch_dtype
    L = wl.layers
    B, Hq, Hkv, D, NC, S = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.capacity, wl.chunk
    c0 = wl.n_chunks // 2
    n_chunk = args.warmup + args.steps
    assert c0 + n_chunk <= wl.n_chunks
    t_gen = time.perf_counter()

    def gen_layer(layer):
        s = W.steady_state(wl, layer, start=c0 * S, seed=layer)
        xs = [W.chunk_inputs(wl, layer, c0 + i) for i in range(n_chunk)]
        return s, xs

    caches, inputs = [], [[None] * L for _ in range(n_chunk)]
    with ThreadPoolExecutor(8) as pool:
        for layer, (s, xs) in enumerate(pool.map(gen_layer, range(L))):
            cache = h2o.H2OCache(dims, dev)
            cache.load(torch.from_numpy(s["k"]).to(dev, dt), torch.from_numpy(s["v"]).to(dev, dt),
                       torch.from_numpy(s["pos"]).to(dev), torch.from_numpy(s["phi"]).to(dev),
                       s["n"], s["start"])
            caches.append(cache)
            for i, x in enumerate(xs):
                inputs[i][layer] = tuple(torch.from_numpy(x[k]).to(dev, dt) for k in ("q", "k", "v"))
    print(f"[bench] {L} layer caches + {n_chunk} chunks per layer generated in "
          f"{time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    bufs = {"out": torch.empty(B, Hq, S, D, dtype=dt, device=dev),
            "lse": torch.empty(B, Hq, S, dtype=torch.float32, device=dev),
            "colsum_cache": torch.empty(B, Hkv, NC, dtype=torch.float32, device=dev),
            "colsum_new": torch.empty(B, Hkv, S, dtype=torch.float32, device=dev),
            "freed_slots": torch.empty(B, Hkv, S, dtype=torch.int32, device=dev),
            "workspace": torch.empty(max(1, h2o.workspace_bytes(dims, S)), dtype=torch.uint8,
                                     device=dev)}

    def chunk_through_stack(i):
        for layer in range(L):
            q, k, v = inputs[i][layer]
            h2o.step(caches[layer], q, k, v, wl.sm_scale, bufs=bufs)

    for i in range(args.warmup):
        chunk_through_stack(i)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    snap = [(c.k.clone(), c.v.clone(), c.pos.clone(), c.score.clone(), c.n_valid, c.next_pos)
            for c in caches]
    # Per-kernel means: the timed chunks run eagerly once with the library's kernel timers.
    kernels = ("attn", "colsum", "update", "select", "insert")
    timers = {k: h2o.KernelTimer(k, args.steps * L) for k in kernels}
    for t_ in timers.values():
        t_.__enter__()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, n_chunk):
        chunk_through_stack(i)
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t0
    for t_ in timers.values():
        t_.__exit__(None, None, None)
    elapsed = eager_s
    if not args.no_graph:
        # Timed region: the same chunks again from the same cache states, each chunk's
        # pass through the stack replayed from a HIP graph captured beforehand.
        ref = [bufs["out"].clone()] + [t for c in caches for t in (c.score.clone(), c.pos.clone())]
        for c, sn in zip(caches, snap):
            c.load(*sn)
        graphs = []
        for i in range(args.warmup, n_chunk):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                chunk_through_stack(i)
            graphs.append(g)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        got = [bufs["out"]] + [t for c in caches for t in (c.score, c.pos)]
        check_replay("layer stack", zip(got, ref))
    ms_chunk = elapsed / args.steps * 1e3
    pairs = pairs_per_head(NC, S)
    f6 = 6.0 * D * Hq * B * pairs * L
    attn = timers["attn"]
    attn_flops = 4.0 * D * Hq * B * pairs
    achieved = attn_flops / (attn.mean_ms * 1e-3) / 1e12
    kernel_us = {k: round(t_.mean_ms * 1e3, 2) for k, t_ in timers.items()}
    cpu = None
    if args.cpu_budget > 0:
        print("[bench] cpu baseline ...", file=sys.stderr, flush=True)
        c = cpu_baseline(wl, args.cpu_budget)
        cpu = {"value": round(c["ms_per_chunk"] * L, 1), "unit": "ms per chunk across layers",
               "cores": c["cores"], "kind": "oracle",
               "sample": c["sample"] + f"; per-chunk time x {L} layers",
               "tflops": c["value"]}
    line = {
        "metric": STACK_METRIC, "value": round(ms_chunk, 3), "unit": "ms",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_chunk, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "batch": B, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "capacity": NC,
                   "recent_window": wl.recent_window, "chunk": S, "seq_len": wl.seq_len,
                   "timed_chunks": f"{c0 + args.warmup}..{c0 + n_chunk - 1} (full caches)",
                   "policy": "h2o", "parallelism": "single-gpu"},
        "timing": "hip_graph" if not args.no_graph else "eager",
        "ms_per_step_eager": round(eager_s / args.steps * 1e3, 3),
        "tokens_per_s": round(B * S / (ms_chunk * 1e-3), 1),
        "tflops_f6": round(f6 / (ms_chunk * 1e-3) / 1e12, 3),
        "kernel_mean_us": kernel_us,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "attn_bf16_kernel<128>",
                     "launches": attn.launches, "mean_launch_us": round(attn.mean_ms * 1e3, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def ctypes_byref(dims):
    import ctypes
    return ctypes.byref(dims.c())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 10 whole sequences; 50 with --backward, whose "
                         "step is one call)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 3; 100 with --backward: the clocks take "
                         "some tens of calls under 1 ms to settle)")
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of replaying a captured HIP graph")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run plain copies of this size first (HBM counter calibration)")
    ap.add_argument("--policy", choices=("h2o", "h2o_buffer", "lastrec"), default="h2o",
                    help="h2o: attend, then evict; h2o_buffer: the insert-first buffer form; "
                         "lastrec: keep the first --sink and the most recent tokens")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward of a steady chunk instead of the forward sequence")
    ap.add_argument("--sink", type=int, default=64,
                    help="lastrec: leading tokens kept (beta); the pages give no value")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 50 if args.backward else 10
    if args.warmup is None:
        args.warmup = 100 if args.backward else 3
    if args.gpus != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch

    import h2o_sparse_attention_amd as h2o
    import workloads as W

    wl = W.WORKLOADS[args.workload]
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
    if args.backward:
        return run_backward(args)
    if wl.decode:
        return run_decode(args)
    if wl.layers > 1:
        return run_stack(args)
    assert wl.layers == 1, "bench runs a single-layer prefill workload"
    dev = torch.device("cuda:0")
    dims = h2o.H2ODims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.capacity,
                       wl.recent_window, wl.dtype)
    dt = dims.torch_dtype
    t_gen = time.perf_counter()
    inputs = []
    for c in range(wl.n_chunks):
        x = W.chunk_inputs(wl, 0, c)
        inputs.append(tuple(torch.from_numpy(x[k]).to(dev, dt) for k in ("q", "k", "v")))
    print(f"[bench] generated {wl.n_chunks} chunks in {time.perf_counter() - t_gen:.1f}s",
          file=sys.stderr, flush=True)
    cache = h2o.H2OCache(dims, dev)
    B, Hq, Hkv, D, NC, S = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.capacity, wl.chunk
    bufs = {"out": torch.empty(B, Hq, S, D, dtype=dt, device=dev),
            "lse": torch.empty(B, Hq, S, dtype=torch.float32, device=dev),
            "colsum_cache": torch.empty(B, Hkv, NC, dtype=torch.float32, device=dev),
            "colsum_new": torch.empty(B, Hkv, S, dtype=torch.float32, device=dev),
            "freed_slots": torch.empty(B, Hkv, S, dtype=torch.int32, device=dev),
            "workspace": torch.empty(max(1, h2o.workspace_bytes(dims, S)), dtype=torch.uint8,
                                     device=dev)}

    step_kw = dict(policy=args.policy, sink_tokens=args.sink)
    lastrec = args.policy == "lastrec"

    def run_sequence():
        cache.reset()
        for q, k, v in inputs:
            h2o.step(cache, q, k, v, wl.sm_scale, bufs=bufs, **step_kw)

    for _ in range(args.warmup):
        run_sequence()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # Per-kernel means: one eager pass with the library's kernel timers.
    n_launch = args.steps * wl.n_chunks
    kernels = ("attn", "select", "insert") if lastrec else ("attn", "colsum", "update",
                                                             "select", "insert")
    timers = {k: h2o.KernelTimer(k, n_launch) for k in kernels}
    for t in timers.values():
        t.__enter__()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_sequence()
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t0
    for t in timers.values():
        t.__exit__(None, None, None)
    checked = [bufs["out"], cache.score, cache.pos] + ([] if lastrec else [bufs["colsum_cache"]])
    ref = [t.clone() for t in checked]
    # Timed region: whole sequences replayed from one captured HIP graph.
    elapsed = eager_s
    if not args.no_graph:
        graph = capture(lambda: [h2o.step(cache, q, k, v, wl.sm_scale, bufs=bufs, **step_kw)
                                 for q, k, v in inputs], cache.reset)
        graph.replay()
        torch.cuda.synchronize()
        check_replay("prefill", zip(checked, ref))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        check_replay("prefill", zip(checked, ref))
    ms_per_step = elapsed / args.steps * 1e3

    # sanity on the last chunk: every query row's weights sum to 1
    if not lastrec:
        total = bufs["colsum_cache"].sum().item() + bufs["colsum_new"].sum().item()
        expect = B * Hkv * S * (Hq // Hkv)
        if abs(total - expect) > 1e-3 * expect:
            print(f"[bench] WARNING: summed weights {total} != {expect}", file=sys.stderr)

    sched = chunk_schedule(wl)
    # keys per row: the filled slots (minus those the buffer form overwrites first)
    # and the chunk's own causal keys
    if args.policy == "h2o_buffer":
        pairs = sum(pairs_per_head(n - max(0, n + S - NC), S) for n in sched)
    else:
        pairs = sum(pairs_per_head(n, S) for n in sched)
    f6 = 6.0 * D * Hq * B * pairs
    f4 = 4.0 * D * Hq * B * pairs
    tflops = (f4 if lastrec else f6) / (ms_per_step * 1e-3) / 1e12
    tokens_per_s = B * wl.seq_len / (ms_per_step * 1e-3)

    attn = timers["attn"]
    attn_flops_per_launch = f4 / wl.n_chunks          # QK^T + PV, averaged over the chunks
    attn_ms = attn.mean_ms
    achieved = attn_flops_per_launch / (attn_ms * 1e-3) / 1e12
    # counters were taken on the headline h2o sequence only
    traffic = read_traffic(TRAFFIC_FILE) if (wl.key == 2 and args.policy == "h2o") else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": "attn_bf16_kernel<128>",
                "launches": attn.launches, "mean_launch_us": round(attn_ms * 1e3, 2)}
    kernel_us = {k: round(t.mean_ms * 1e3, 2) for k, t in timers.items()}
    steady_n = [i for i, n in enumerate(sched) if n == NC]
    # One full-cache chunk alone, and the rates this GPU reaches on a GEMM and a copy.
    steady_us = steady_chunk(wl, dims, step_kw, bufs)
    if args.policy == "h2o_buffer":
        steady_pairs = pairs_per_head(NC - S, S)
    else:
        steady_pairs = pairs_per_head(NC, S)
    steady_f = (4.0 if lastrec else 6.0) * D * Hq * B * steady_pairs
    steady = {"us": round(steady_us, 1),
              "tflops": round(steady_f / (steady_us * 1e-6) / 1e12, 1),
              "frac_bf16_peak": round(steady_f / (steady_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
              "flops": "F4" if lastrec else "F6"}
    peaks = measured_peaks()
    roofline["frac_of_measured_gemm"] = round(achieved / peaks["gemm_bf16_8192_tflops"], 4)

    cpu = None
    if args.cpu_budget > 0 and args.policy == "h2o":
        print("[bench] cpu baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_budget)

    line = {
        "metric": LASTREC_METRIC if lastrec else (
            BUFFER_METRIC if args.policy == "h2o_buffer" else
            (METRIC_CHUNK2K if wl.chunk == 2048 else METRIC)), "value": round(tflops, 3),
        "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "capacity": NC, "recent_window": wl.recent_window,
                   "chunk": S, "seq_len": wl.seq_len, "chunks": wl.n_chunks,
                   "policy": args.policy,
                   **({"sink_tokens": args.sink} if lastrec else {}),
                   "parallelism": "single-gpu"},
        "timing": "hip_graph" if not args.no_graph else "eager",
        "ms_per_step_eager": round(eager_s / args.steps * 1e3, 4),
        "tokens_per_s": round(tokens_per_s, 1),
        "tflops_f4": round(f4 / (ms_per_step * 1e-3) / 1e12, 3),
        "frac_bf16_peak_f6": None if lastrec else round(tflops / PEAK_BF16_TFLOPS, 4),
        "kernel_mean_us": kernel_us,
        "steady_chunks": len(steady_n),
        "steady_chunk": steady,
        "measured_peaks": peaks,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
