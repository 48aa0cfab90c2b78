"""Decode-step benchmark: append + paged decode attention on one MI355X.

A step is one pass of the decode hot path over one batch of synthetic input
already resident in HBM: this step's K/V rows go into their slots, the
split-KV partials kernel reads every visible position, and the log-sum-exp
merge kernel writes the output.  The default workload is the
Llama-3-8B-shaped GQA batch (H_q = 32, H_kv = 8, d_head = 128, batch 64,
lengths uniform in [512, 8192], bf16, 16-token blocks randomly placed).

Prints ONE JSON line.  ``value`` is KV GB/s: the K and V bytes of every
visible position (the algorithmic bytes of the step) divided by the measured
time per step (K replays of the step captured in a HIP graph).  The line also
carries decode-attention tokens/s (sequences per second for one layer
call); the roofline of the dominant kernel (the partials kernel, timed with
HIP events around each of at least 100 eager launches on the launch stream:
mean, median and 10th / 90th percentiles); the device's streaming-read rate
measured in the same run (the practical ceiling of a cache-reading step);
and the fp64 CPU oracle timed on a bounded sample of the same workload on
this host, with all BLAS threads and with one (a reported baseline, not the
target).

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload NAME]
"""

import argparse
import contextlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "decode-attn KV GB/s (% of HBM peak) + tokens/s, GQA 8:1 paged, 1 MI355X"
MIN_KERNEL_SAMPLES = 100
STREAM_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa_llama3_8b",
                    choices=["gqa_llama3_8b", "mha_llama2_7b", "long_gqa_split", "tiny",
                             "mla_deepseek_v2", "gqa_llama3_8b_int8", "gqa_llama3_8b_fp8",
                             "prefill_llama3_8b", "stream_read", "lds_read"])
    ap.add_argument("--replicas", type=int, default=4,
                    help="MLA: rotate over this many copies of the latent cache so the "
                         "timed reads come from HBM, not the 256 MB Infinity Cache")
    ap.add_argument("--separate-append", action="store_true",
                    help="run kv_append_paged as its own kernel instead of fused into the attention pass")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of a captured HIP graph of the step")
    ap.add_argument("--partition", type=int, default=-1,
                    help="partition tokens (-1: the workload's own, 0: library auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target CPU time of each oracle leg (all threads, then one thread)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read measurement")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the decode step, time a plain device copy of MIB MiB "
                         "(reference kernel for scaling HBM traffic counters)")
    return ap.parse_args()


def calibrate_copy(mib, steps, warmup):
    """Plain copy of a known size: reads and writes exactly mib MiB per launch."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "ms_per_copy": round(ms, 5),
                      "copy_GBps_read_plus_write": round(2 * n / (ms / 1e3) / 1e9, 1)}),
          flush=True)


def up(a, dev):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


# --- GPU timing ---------------------------------------------------------------------

_SPIN_CYCLES_PER_MS = None


def queue_ahead(torch, stream, ms):
    """Keep the device busy for about ``ms`` before timed eager launches (a
    bounded spin kernel, not part of any step), so that the host enqueues the
    steps ahead of the device and no host-side gap falls between a kernel's
    timing events and the kernel itself.  Returns a function giving the
    seconds the spin held the device (read after synchronising), which the
    callers take out of their wall-clock figure."""
    global _SPIN_CYCLES_PER_MS
    if _SPIN_CYCLES_PER_MS is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        torch.cuda._sleep(1 << 22)
        b.record(stream)
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_MS = (1 << 22) / max(a.elapsed_time(b), 1e-3)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(int(_SPIN_CYCLES_PER_MS * ms))
    b.record(stream)
    return lambda: a.elapsed_time(b) / 1e3  # seconds the spin held the device


def time_eager(torch, stream, step, n, spin_ms_per_step):
    """n eager steps, step(i, ev) recording ev[0] / ev[1] around the dominant
    kernel.  Returns (ms per step, per-launch kernel ms list, wall seconds)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    spin_s = queue_ahead(torch, stream, spin_ms_per_step * n)
    start.record(stream)
    for i in range(n):
        step(i, evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0 - spin_s()
    return start.elapsed_time(end) / n, [a.elapsed_time(b) for a, b in evs], wall


def kernel_stats(name, ms):
    """Mean, median, 10th / 90th percentile, min and max of per-launch times."""
    a = np.asarray(ms, dtype=np.float64)
    return {f"{name}_avg": round(float(a.mean()), 5),
            f"{name}_median": round(float(np.median(a)), 5),
            f"{name}_p10": round(float(np.percentile(a, 10)), 5),
            f"{name}_p90": round(float(np.percentile(a, 90)), 5),
            f"{name}_min": round(float(a.min()), 5), f"{name}_max": round(float(a.max()), 5),
            "launches": int(a.size)}


def time_graph(torch, step, out, args, variants=1):
    """Capture the step (append, partials, merge) in HIP graphs, check that
    replays give the eager step's output bit for bit (with eager work between
    replays), then time args.steps replays.  ``step(i)`` takes the step's index;
    with ``variants`` > 1 the steps differ with i % variants (e.g. rotating
    cache copies), so one graph is captured per variant and step i replays
    graph i % variants.  Returns (ms per step, True)."""
    stream = torch.cuda.current_stream()
    graphs, refs = [], []
    for v in range(variants):
        step(v)
        torch.cuda.synchronize()
        refs.append(out.clone())
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(v)  # first run on the capture stream outside the capture
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step(v)
        graphs.append(g)
    for _ in range(3):
        for v, g in enumerate(graphs):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(out, refs[v]):
                raise RuntimeError("graph replay differs from the eager step")
            step(v)  # eager work between replays
            torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % variants].replay()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        graphs[i % variants].replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / args.steps, True


def stream_ceiling(torch, kvd, launches=20):
    """The library's streaming-read probe over 1 GiB (four times the 256 MB
    Infinity Cache): launches back to back between two events."""
    stream = torch.cuda.current_stream()
    src = torch.ones(STREAM_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(kvd.stream_read_sink_bytes(), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        kvd.stream_read(src, sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    spin_s = queue_ahead(torch, stream, 0.2 * launches)
    a.record(stream)
    for _ in range(launches):
        kvd.stream_read(src, sink)
    b.record(stream)
    torch.cuda.synchronize()
    spin_s()
    ms = a.elapsed_time(b) / launches
    gbs = STREAM_BYTES / (ms / 1e3) / 1e9
    del src, sink
    return {"kernel": "stream_read_kernel", "bytes": STREAM_BYTES, "ms_per_launch": round(ms, 5),
            "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def with_ceiling(res, torch, kvd, args):
    """Adds the streaming-read rate and the dominant kernel's share of it."""
    if args.no_ceiling:
        return
    c = stream_ceiling(torch, kvd)
    res["stream_read_ceiling"] = c
    if res["roofline"]["unit"] == "GB/s":
        res["roofline"]["frac_of_stream_read"] = round(res["roofline"]["achieved"] / c["GBps"], 4)


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None.

    profiles/<kernel>__<workload>.md carries the scaled FETCH_SIZE + WRITE_SIZE
    bytes and the SHA-256 of the kernel sources they were taken with; the
    figure is only returned while the current sources hash the same.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    tag = "```json traffic"
    if tag not in text:
        return None
    rec = json.loads(text.split(tag, 1)[1].split("```", 1)[0])
    h = hashlib.sha256()
    for f in rec["source_files"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return int(rec["traffic_bytes_per_launch"])


# --- CPU oracle baseline ----------------------------------------------------------

def host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        cfg = np.__config__.CONFIG["Build Dependencies"]["blas"]
        blas = f"{cfg.get('name')} {cfg.get('version', '')}".strip()
    except Exception:  # pragma: no cover - numpy without the config dict
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "numpy": np.__version__,
            "blas": blas}


def _cpu_leg(work, target_s, threads, max_units):
    """Calls work(i) (one unit of oracle work; returns the amount of the
    metric it covers) until ~target_s; ``threads`` limits the BLAS / OpenMP
    pools (None: as configured).  Returns units, amount, seconds, the pool
    size and the effective cores (process CPU time / wall time)."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        ctx = threadpool_limits(limits=threads) if threads else contextlib.nullcontext()
    except Exception:  # pragma: no cover - threadpoolctl missing
        threadpool_info, ctx = None, contextlib.nullcontext()
    with ctx:
        pool = (max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
                if threadpool_info else (threads or 1))
        t0, c0 = time.perf_counter(), time.process_time()
        n = 0
        amount = 0.0
        while time.perf_counter() - t0 < target_s and n < max_units:
            amount += work(n)
            n += 1
        dt = time.perf_counter() - t0
        cpu = time.process_time() - c0
    return {"units": n, "amount": amount, "seconds": dt, "pool": int(pool),
            "effective_cores": round(cpu / dt, 2) if dt > 0 else None}


def cpu_baseline_legs(work, target_s, max_units, unit, scale, describe):
    """The oracle timed with every BLAS thread and with one.  ``scale``
    turns an amount per second into the metric's unit; ``describe(leg)``
    words the sample."""
    legs = [_cpu_leg(work, target_s, None, max_units), _cpu_leg(work, target_s, 1, max_units)]
    out = []
    for leg in legs:
        out.append({"value": leg["amount"] / leg["seconds"] * scale, "cores": leg["pool"],
                    "effective_cores": leg["effective_cores"],
                    "sample": f"{describe(leg)} in {leg['seconds']:.1f} s; fp64 numpy, BLAS pool "
                              f"of {leg['pool']} thread(s)",
                    "units_per_s": leg["units"] / leg["seconds"]})
    res = {"value": out[0]["value"], "unit": unit, "cores": out[0]["cores"], "kind": "oracle",
           "sample": out[0]["sample"], "effective_cores": out[0]["effective_cores"],
           "units_per_s": out[0]["units_per_s"], "one_thread": out[1], "host": host_info()}
    return res


def cpu_baseline(inp, target_s):
    """The fp64 oracle on whole sequences of the workload, in a fixed random
    order over repeated passes."""
    import oracle
    order = np.random.default_rng(0).permutation(inp.B)
    elem = 2 if inp.dtype == "bf16" else 4

    def work(i):
        b = int(order[i % inp.B])
        sl = slice(b, b + 1)
        oracle.decode_attn_paged(inp.q[sl], inp.k_pool, inp.v_pool, inp.block_table[sl],
                                 inp.seq_lens[sl], inp.dtype, inp.k_new[sl], inp.v_new[sl])
        return 2 * int(inp.seq_lens[b]) * inp.H_kv * inp.d * elem

    return cpu_baseline_legs(
        work, target_s, 50 * inp.B, "GB/s", 1e-9,
        lambda leg: f"{leg['units']} sequence decodes ({leg['units'] / inp.B:.2f} passes over "
                    f"the {inp.B} sequences, all heads)")


def cpu_baseline_mla(inp, target_s, scale):
    import oracle
    order = np.random.default_rng(0).permutation(inp.B)

    def work(i):
        b = int(order[i % inp.B])
        sl = slice(b, b + 1)
        oracle.mla_decode_paged(inp.q[sl], inp.c_pool, inp.block_table[sl], inp.seq_lens[sl],
                                inp.d_c, scale, c_new=inp.c_new[sl])
        return int(inp.seq_lens[b]) * inp.width * 2

    return cpu_baseline_legs(
        work, target_s, 50 * inp.B, "GB/s", 1e-9,
        lambda leg: f"{leg['units']} sequence decodes ({leg['units'] / inp.B:.2f} passes over "
                    f"the {inp.B} sequences, all {inp.H} heads)")


def cpu_baseline_int8(inp, target_s):
    """The oracle's quantising append and decode over the one-byte cache (INT8
    or FP8), one whole sequence at a time."""
    import oracle
    order = np.random.default_rng(0).permutation(inp.B)
    fp8 = inp.codes == "fp8"
    append = oracle.append_paged_fp8 if fp8 else oracle.append_paged_int8
    decode = oracle.decode_attn_paged_fp8 if fp8 else oracle.decode_attn_paged_int8

    def work(i):
        b = int(order[i % inp.B])
        sl = slice(b, b + 1)
        n = int(inp.seq_lens[b])
        # the sequence's own blocks, appended to and read as one small pool
        blocks = inp.block_table[b, :-(-n // 16)]
        table = np.arange(len(blocks), dtype=np.int32)[None, :]
        kq, vq, vs = append(inp.kq_pool[blocks], inp.vq_pool[blocks], inp.vs_pool[blocks],
                            inp.k_new[sl], inp.v_new[sl], "bf16", inp.k_scale, table,
                            inp.seq_lens[sl])
        decode(inp.q[sl], kq, vq, vs, inp.k_scale, table, inp.seq_lens[sl], "bf16")
        return n * inp.H_kv * (2 * inp.d + 4)

    return cpu_baseline_legs(
        work, target_s, 50 * inp.B, "GB/s", 1e-9,
        lambda leg: f"{leg['units']} sequence decodes ({leg['units'] / inp.B:.2f} passes over "
                    f"the {inp.B} sequences, all heads)")


def cpu_baseline_prefill(inp, target_s):
    """The oracle on prefill rows, in order, sequence by sequence; FLOP/s on
    the same count as the GPU figure."""
    import oracle
    k2, v2 = oracle.append_paged_multi(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                       inp.cu_rows, inp.block_table, inp.seq_lens)
    rows = [(b, i) for b in range(inp.B) for i in range(int(inp.cu_rows[b + 1] - inp.cu_rows[b]))]
    cache = {}

    def work(j):
        b, i = rows[j % len(rows)]
        if b not in cache:
            cache.clear()
            L = int(inp.seq_lens[b])
            cache[b] = (oracle.to_f64(oracle.gather_logical(k2, inp.block_table, b, L), inp.dtype),
                        oracle.to_f64(oracle.gather_logical(v2, inp.block_table, b, L), inp.dtype))
        K, V = cache[b]
        n = int(inp.cu_rows[b + 1] - inp.cu_rows[b])
        p = int(inp.seq_lens[b]) - n + i
        q = oracle.to_f64(inp.q[inp.cu_rows[b] + i], inp.dtype)
        oracle.decode_attention(q, K[:p + 1], V[:p + 1])
        return (p + 1) * inp.H_q * inp.d * 4

    return cpu_baseline_legs(
        work, target_s, len(rows), "TFLOP/s", 1e-12,
        lambda leg: f"{leg['units']} prefill rows (all {inp.H_q} heads)")


# --- workloads ------------------------------------------------------------------------

def _base(args, value, unit, ms_step, ms_eager, graph_check, dtype, kernels, config):
    return {"metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "step_launch": "hip graph" if not args.no_graph else "eager",
            "step_kernels": kernels, "ms_per_step_eager": round(ms_eager, 5),
            "graph_replays_match_eager": graph_check, "data": "synthetic", "config": config}


def main_int8(args, kvd, make_config_inputs):
    """One decode step over a one-byte cache (INT8 or FP8 E4M3 codes): the
    quantising append, the partial kernel and the merge, timed like the bf16
    step (graph replay)."""
    import torch
    dev = torch.device("cuda:0")
    inp = make_config_inputs(args.workload, sentinel="zero")[0]
    pt = args.partition if args.partition >= 0 else 0
    q = up(inp.q, dev)
    kq, vq, vs, ks = up(inp.kq_pool, dev), up(inp.vq_pool, dev), up(inp.vs_pool, dev), up(inp.k_scale, dev)
    kn, vn = up(inp.k_new, dev), up(inp.v_new, dev)
    table, seq = up(inp.block_table, dev), up(inp.seq_lens, dev)
    H_q, H_kv, d, L = inp.H_q, inp.H_kv, inp.d, inp.max_seq_len
    pt_used = kvd.decode_attn_partition_tokens(inp.B, H_q, H_kv, d, L, pt)
    ws = kvd.alloc_workspace(inp.B, H_q, H_kv, d, L, pt)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    fp8 = inp.codes == "fp8"
    append = kvd.kv_append_paged_fp8 if fp8 else kvd.kv_append_paged_int8
    partials = kvd.decode_attn_paged_fp8_partials if fp8 else kvd.decode_attn_paged_int8_partials

    def step(i=0, ev=None):
        append(kq, vq, vs, kn, vn, ks, table, seq)
        if ev is not None:
            ev[0].record(stream)
        partials(q, kq, vq, ks, vs, table, seq, L, ws, partition_tokens=pt)
        if ev is not None:
            ev[1].record(stream)
        kvd.decode_attn_merge(out, seq, H_kv, L, ws, partition_tokens=pt)

    for _ in range(args.warmup):
        step()
    ms_eager, part_ms, wall = time_eager(torch, stream, step, max(args.steps, MIN_KERNEL_SAMPLES), 0.3)
    ms_step, graph_check = ms_eager, None
    if not args.no_graph:
        ms_step, graph_check = time_graph(torch, step, out, args)
    kv_bytes = inp.kv_bytes_read
    kernel = "paged_balanced" if pt_used == 0 else "paged_partials"
    part_avg = float(np.mean(part_ms))
    value = kv_bytes / (ms_step / 1e3) / 1e9
    achieved = kv_bytes / (part_avg / 1e3) / 1e9
    name = "fp8" if fp8 else "int8"
    res = _base(args, value, "GB/s", ms_step, ms_eager, graph_check,
                "fp8 e4m3" if fp8 else "int8", f"kv_append_paged_{name}, partials, merge",
                {"workload": args.workload, "batch": inp.B, "num_q_heads": H_q,
                 "num_kv_heads": H_kv, "head_dim": d, "block_size": 16,
                 "sum_seq_len": int(inp.seq_lens.astype(np.int64).sum()), "max_seq_len": L,
                 "partition_tokens": pt_used,
                 "cache": f"{'fp8 e4m3' if fp8 else 'int8'} codes, per-channel K and "
                 "per-token V fp32 scales; bf16 queries and output"})
    res.update({
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(inp.B / (ms_step / 1e3), 1),
        "kv_bytes_per_step": kv_bytes,
        "wall_s_timed": round(wall, 4),
        "kernel_ms": kernel_stats("partials", part_ms),
        "roofline": {"bound": "hbm", "kernel": kernel + "_kernel",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(kernel, args.workload)},
        "cpu_baseline": None,
    })
    with_ceiling(res, torch, kvd, args)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_int8(inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def prefill_flops(inp):
    """Algorithmic FLOPs of the causal prefill: every row's q.K and P.V over
    the positions it sees (2 d multiply-adds per position and head each)."""
    n = np.diff(inp.cu_rows).astype(np.int64)
    past = inp.seq_lens.astype(np.int64) - n
    seen = int(np.sum(n * past + n * (n + 1) // 2))
    return seen * inp.H_q * inp.d * 4


def prefill_min_bytes(inp):
    """Least HBM bytes the prefill kernel can move: K and V of every cached
    position once per KV head, the queries read and the outputs written."""
    kv = int(inp.seq_lens.astype(np.int64).sum()) * inp.H_kv * inp.d * 2 * 2
    return kv + 2 * inp.num_rows * inp.H_q * inp.d * 2


def main_prefill(args, kvd, make_config_inputs):
    """One chunked-prefill call: the many-slot append and the causal MFMA
    kernel, timed like the decode step (graph replay, events around the
    attention kernel)."""
    import torch
    dev = torch.device("cuda:0")
    inp = make_config_inputs(args.workload, sentinel="zero")[0]
    q, kc, vc = up(inp.q, dev), up(inp.k_pool, dev), up(inp.v_pool, dev)
    kn, vn = up(inp.k_new, dev), up(inp.v_new, dev)
    cu, table, seq = up(inp.cu_rows, dev), up(inp.block_table, dev), up(inp.seq_lens, dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    L, R = inp.max_seq_len, inp.max_rows

    def step(i=0, ev=None):
        kvd.kv_append_paged_multi(kc, vc, kn, vn, cu, table, seq, R)
        if ev is not None:
            ev[0].record(stream)
        kvd.prefill_attn_paged(q, kc, vc, cu, table, seq, L, R, out=out)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    ms_eager, part_ms, wall = time_eager(torch, stream, step, max(args.steps, MIN_KERNEL_SAMPLES), 1.2)
    ms_step, graph_check = ms_eager, None
    if not args.no_graph:
        ms_step, graph_check = time_graph(torch, step, out, args)
    flops = prefill_flops(inp)
    part_avg = float(np.mean(part_ms))
    value = flops / (ms_step / 1e3) / 1e12
    achieved = flops / (part_avg / 1e3) / 1e12
    res = _base(args, value, "TFLOP/s", ms_step, ms_eager, graph_check, "bf16",
                "kv_append_paged_multi, prefill",
                {"workload": args.workload, "batch": inp.B, "num_q_heads": inp.H_q,
                 "num_kv_heads": inp.H_kv, "head_dim": inp.d, "block_size": 16,
                 "new_rows": inp.num_rows, "seq_lens": inp.seq_lens.tolist()})
    res["metric"] = "chunked-prefill attention TFLOP/s (bf16 MFMA), paged GQA, 1 MI355X"
    res.update({
        "tokens_per_s": round(inp.num_rows / (ms_step / 1e3), 1),
        "flops_per_step": flops,
        "min_bytes_per_step": prefill_min_bytes(inp),
        "wall_s_timed": round(wall, 4),
        "kernel_ms": kernel_stats("prefill", part_ms),
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(achieved, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic("prefill", args.workload)},
        "cpu_baseline": None,
    })
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def main_mla(args, kvd, make_config_inputs):
    import torch
    dev = torch.device("cuda:0")
    inp = make_config_inputs(args.workload, sentinel="zero")[0]
    pt = args.partition if args.partition > 0 else 0
    q = up(inp.q, dev)
    caches = [up(inp.c_pool, dev) for _ in range(max(1, args.replicas))]
    c_new = up(inp.c_new[:, None, :], dev)
    table, seq = up(inp.block_table, dev), up(inp.seq_lens, dev)
    H, L = inp.H, inp.max_seq_len
    pt_used = kvd.decode_attn_partition_tokens(inp.B, H, 1, inp.d_c, L, pt)
    ws = kvd.alloc_workspace(inp.B, H, 1, inp.d_c, L, pt)
    out = torch.empty((inp.B, H, inp.d_c), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        # The default step is the partials kernel with the append fused in (it
        # takes the new rows from c_new and writes them into their slots),
        # then the merge; --separate-append runs kv_append_paged first.
        c = caches[i % len(caches)]
        if args.separate_append:
            kvd.kv_append_paged(c[:, :, None, :], None, c_new, None, table, seq)
        if ev is not None:
            ev[0].record(stream)
        if args.separate_append:
            kvd.decode_attn_mla_partials(q, c, table, seq, L, ws, partition_tokens=pt)
        else:
            kvd.decode_attn_mla_append_partials(q, c, c_new[:, 0], table, seq, L, ws,
                                                partition_tokens=pt)
        if ev is not None:
            ev[1].record(stream)
        kvd.decode_attn_merge(out, seq, 1, L, ws, partition_tokens=pt)

    for i in range(args.warmup):
        step(i)
    ms_eager, part_ms, wall = time_eager(torch, stream, step, max(args.steps, MIN_KERNEL_SAMPLES), 0.3)
    ms_step, graph_check = ms_eager, None
    if not args.no_graph:
        # one graph per cache copy; step i replays the graph of copy i % copies
        ms_step, graph_check = time_graph(torch, step, out, args, variants=len(caches))
    kv_bytes = inp.kv_bytes_read
    positions = int(inp.seq_lens.astype(np.int64).sum())
    flops = positions * H * (inp.width + inp.d_c) * 2
    part_avg = float(np.mean(part_ms))
    achieved = kv_bytes / (part_avg / 1e3) / 1e9
    tflops = flops / (part_avg / 1e3) / 1e12
    value = kv_bytes / (ms_step / 1e3) / 1e9
    res = _base(args, value, "GB/s", ms_step, ms_eager, graph_check, "bf16",
                ("kv_append_paged, decode_attn_mla_partials, merge" if args.separate_append
                 else "decode_attn_mla_append_partials (append fused), merge"),
                {"workload": args.workload, "batch": inp.B, "num_q_heads": H, "d_c": inp.d_c,
                 "d_rope": inp.d_rope, "block_size": 16, "sum_seq_len": positions,
                 "max_seq_len": L, "partition_tokens": pt_used, "cache_replicas": len(caches)})
    res.update({
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(inp.B / (ms_step / 1e3), 1),
        "kv_bytes_per_step": kv_bytes,
        "flops_per_step": flops,
        "wall_s_timed": round(wall, 4),
        "kernel_ms": kernel_stats("partials", part_ms),
        "roofline": {"bound": "hbm", "kernel": "mla_partials_kernel", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("mla_partials", args.workload)},
        "mfma": {"achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
        "cpu_baseline": None,
    })
    with_ceiling(res, torch, kvd, args)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_mla(inp, args.cpu_seconds, kvd.mla_default_scale())
    print(json.dumps(res), flush=True)


def main_stream(args, kvd):
    """The streaming-read probe alone (its own profile leg)."""
    import torch
    c = stream_ceiling(torch, kvd, launches=max(args.steps, 20))
    print(json.dumps({"metric": "streaming read GB/s, 1 MI355X", "value": c["GBps"], "unit": "GB/s",
                      "n_gpus": 1, "steps": max(args.steps, 20), "warmup": 3,
                      "ms_per_step": c["ms_per_launch"], "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "u8",
                      "data": "synthetic", "config": {"workload": "stream_read",
                                                      "bytes": STREAM_BYTES},
                      "roofline": {"bound": "hbm", "kernel": c["kernel"], "achieved": c["GBps"],
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": c["frac_of_peak"], "traffic": None}}), flush=True)


def main_lds(args, kvd):
    """The LDS-read probe alone: one workgroup of eight waves per compute unit
    reading its LDS, for 16-byte and for transposing 8-byte reads."""
    import torch
    groups = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 4096
    cycles = torch.zeros(groups, dtype=torch.int64, device="cuda")
    sink = torch.zeros(kvd.lds_read_sink_bytes(groups), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    launches = max(args.steps, 20)
    legs = {}
    for mode, name in ((0, "b128"), (1, "tr_b64")):
        for _ in range(3):
            kvd.lds_read(mode, groups, iters, cycles, sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(launches):
            kvd.lds_read(mode, groups, iters, cycles, sink)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / launches
        nbytes = kvd.lds_read_bytes(mode, groups, iters)
        cyc = float(cycles.double().mean())
        legs[name] = {"bytes_per_launch": nbytes, "ms_per_launch": round(ms, 5),
                      "TBps_all_cus": round(nbytes / (ms / 1e3) / 1e12, 2),
                      "bytes_per_cycle_per_cu": round(nbytes / groups / cyc, 1),
                      "loop_cycles_per_cu": round(cyc, 0)}
    print(json.dumps({"metric": "LDS read bytes per cycle and compute unit, 1 MI355X",
                      "value": legs["b128"]["bytes_per_cycle_per_cu"], "unit": "B/cycle/CU",
                      "n_gpus": 1, "steps": launches, "warmup": 3,
                      "ms_per_step": legs["b128"]["ms_per_launch"], "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
                      "config": {"workload": "lds_read", "groups": groups, "iters": iters,
                                 "threads_per_group": 512},
                      "legs": legs}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path would shard by sequence or KV head, with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, args.steps, args.warmup)
        return

    import torch
    import kv_cache_decode_02_amd as kvd
    from workloads import make_config_inputs, config

    if args.workload == "stream_read":
        main_stream(args, kvd)
        return
    if args.workload == "lds_read":
        main_lds(args, kvd)
        return
    cfg = config(args.workload)
    if cfg["kind"] == "mla":
        main_mla(args, kvd, make_config_inputs)
        return
    if cfg["kind"] in ("paged_int8", "paged_fp8"):
        main_int8(args, kvd, make_config_inputs)
        return
    if cfg["kind"] == "prefill":
        main_prefill(args, kvd, make_config_inputs)
        return
    dev = torch.device("cuda:0")
    inp = make_config_inputs(args.workload, sentinel="zero")[0]
    pt = cfg["partition"] if args.partition < 0 else args.partition
    q, kc, vc = up(inp.q, dev), up(inp.k_pool, dev), up(inp.v_pool, dev)
    kn, vn = up(inp.k_new, dev), up(inp.v_new, dev)
    table, seq = up(inp.block_table, dev), up(inp.seq_lens, dev)
    H_q, H_kv, d, L = inp.H_q, inp.H_kv, inp.d, inp.max_seq_len
    pt_used = kvd.decode_attn_partition_tokens(inp.B, H_q, H_kv, d, L, pt)
    ws = kvd.alloc_workspace(inp.B, H_q, H_kv, d, L, pt)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(i=0, ev=None):
        # One decode step: append this step's K/V, attend, merge.  By default
        # the append is fused into the attention pass (one kernel reads the
        # history and writes the new rows); --separate-append runs
        # kv_append_paged first.
        if args.separate_append:
            kvd.kv_append_paged(kc, vc, kn, vn, table, seq)
        if ev is not None:
            ev[0].record(stream)
        if args.separate_append:
            kvd.decode_attn_paged_partials(q, kc, vc, table, seq, L, ws, partition_tokens=pt)
        else:
            kvd.decode_attn_paged_append_partials(q, kc, vc, kn, vn, table, seq, L, ws,
                                                  partition_tokens=pt)
        if ev is not None:
            ev[1].record(stream)
        kvd.decode_attn_merge(out, seq, H_kv, L, ws, partition_tokens=pt)

    for _ in range(args.warmup):
        step()
    # Eager steps, with events around the partials kernel (the roofline).
    ms_eager, part_ms, wall = time_eager(torch, stream, step, max(args.steps, MIN_KERNEL_SAMPLES), 0.3)
    ms_step, graph_check = ms_eager, None
    if not args.no_graph:
        ms_step, graph_check = time_graph(torch, step, out, args)

    kv_bytes = inp.kv_bytes_read
    step_s = ms_step / 1e3
    part_avg = float(np.mean(part_ms))
    # The automatic mode (partition 0) runs the balanced split.
    kernel = "paged_balanced" if pt_used == 0 else "paged_partials"
    value = kv_bytes / step_s / 1e9
    achieved = kv_bytes / (part_avg / 1e3) / 1e9
    res = _base(args, value, "GB/s", ms_step, ms_eager, graph_check, inp.dtype,
                ("kv_append_paged, partials, merge" if args.separate_append
                 else "append fused into partials, merge"),
                {"workload": args.workload, "batch": inp.B, "num_q_heads": H_q,
                 "num_kv_heads": H_kv, "head_dim": d, "block_size": 16,
                 "sum_seq_len": int(inp.seq_lens.astype(np.int64).sum()),
                 "max_seq_len": L, "partition_tokens": pt_used})
    res.update({
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(inp.B / step_s, 1),
        "kv_bytes_per_step": kv_bytes,
        "wall_s_timed": round(wall, 4),
        "kernel_ms": kernel_stats("partials", part_ms),
        "roofline": {"bound": "hbm", "kernel": kernel + "_kernel",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(kernel, args.workload)},
        "cpu_baseline": None,
    })
    with_ceiling(res, torch, kvd, args)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
