"""Benchmark of paged-KV batch decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The default workload is the largest one that fits one GPU, gemma2_decode
(256 requests, head_dim 256, soft cap 50, window 4096; 4.99 GB per call).

One step is one pkd_run (one kernel launch: decode, with the merge of split
requests fused in) over one batch whose inputs already sit in HBM; the plan
is built once before timing, as plan() is amortised over layers and steps.
Successive steps alternate between distinct K/V pools so that no step finds
the previous step's data in the 256 MB Infinity Cache. The class example
(worked_example) runs the page's layer loop instead: one step is a pass over
32 layers, each with its own cache, q and output, and the figures are per
call.

Prints one JSON line. ``value`` is the achieved HBM bandwidth of the whole
call: algorithmic bytes / wall time per call, with the K timed calls replayed
from one HIP graph (the way a serving loop issues its decode steps; pkd_run
allocates nothing and never synchronises, so it captures unchanged); the
graph is replayed R times, after 0.2 s of untimed replays that bring the
GPU's clocks to their steady state, and the median replay is reported, with
the fastest and slowest beside it. ``--eager`` times K host launches instead.
Algorithmic bytes = K and V rows of the attended tokens (each read once per
kv head) + q + o + fp32 lse + the page indices of the touched pages + indptr
+ last_page_len. ``roofline`` is that kernel, timed with HIP events on the
stream it runs on, around each timed region. ``cpu_baseline`` times the fp64 CPU oracle on a bounded
sample: the median of three runs over the same requests, and for the two
small workloads also a run limited to one thread. ``per_call_events`` gives
single calls timed with HIP events, median and p10/p90 of 100: "cold", each
after an untimed 1 GiB fill that evicts the caches, and "hot", without it.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_kv_decode_09_amd as pkd  # noqa: E402
from paged_kv_decode_09_amd import workloads as wl  # noqa: E402

PEAK_HBM_GBS = 8000.0
WARM_S = 0.2
MALL_BYTES = 256 << 20
ELEM = {"f16": 2, "bf16": 2, "e4m3": 1}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_decode_09_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, pt):
    """Bytes one call must move: K and V rows of the attended tokens (each
    read once per kv head), q, o, fp32 lse, the page indices of the touched
    pages, indptr and last_page_len."""
    B, nq, nkv, hd = w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim
    ps, Q = w.page_size, w.q_len_per_req
    attended, touched = 0, 0
    for i in range(B):
        L = int(pt.lengths[i])
        # the union of the Q query tokens' windows (the first token's is widest)
        s0 = 0 if w.window_left < 0 else max(0, L - Q - w.window_left)
        attended += L - s0
        touched += (L - 1) // ps - s0 // ps + 1
    kv = attended * nkv * hd * 2 * ELEM[w.kv_dtype]
    q = B * Q * nq * hd * ELEM[w.q_dtype]
    out = B * Q * nq * (hd * ELEM[w.o_dtype] + 4)
    meta = touched * 4 + (B + 1) * 4 + B * 4
    return kv + q + out + meta


def _sub_pool(case, requests):
    pt = case.pt
    pages = np.concatenate([pt.indices[pt.indptr[i]:pt.indptr[i + 1]]
                            for i in requests]).astype(np.int64)
    indptr = np.concatenate([[0], np.cumsum(
        [pt.indptr[i + 1] - pt.indptr[i] for i in requests])]).astype(np.int32)
    host = case.pool[torch.from_numpy(pages).to(case.pool.device)].cpu()
    return host, indptr, np.arange(len(pages), dtype=np.int32), \
        pt.last_page_len[list(requests)].astype(np.int32)


def _oracle_call(w, case, i):
    """The oracle on request i alone (argument marshalling only)."""
    import oracle
    kw = dict(logits_soft_cap=w.logits_soft_cap, window_left=w.window_left,
              k_scale=w.k_scale, v_scale=w.v_scale)
    if w.pos_encoding_mode == "ROPE_LLAMA":
        kw["rope"] = (w.rope_theta, w.rope_scale)
    elif w.pos_encoding_mode == "ALIBI":
        kw["alibi"] = True
    Q = w.q_len_per_req
    pool, indptr, indices, last = _sub_pool(case, [i])
    qn = wl.raw_numpy(case.q[i * Q:(i + 1) * Q], w.q_dtype)
    pn = wl.raw_numpy(pool, w.kv_dtype)
    common = (qn, pn, w.layout, indptr, indices, last, w.page_size)
    if Q > 1 or w.pos_encoding_mode != "NONE":
        return lambda: oracle.batch_decode_multi(*common, Q, w.q_dtype, w.kv_dtype,
                                                 w.sm_scale, **kw)
    if w.fixed_split_size:
        return lambda: oracle.batch_decode_split(*common, w.q_dtype, w.kv_dtype,
                                                 w.sm_scale, w.fixed_split_size, **kw)
    return lambda: oracle.batch_decode(*common, w.q_dtype, w.kv_dtype, w.sm_scale, **kw)


def _timed(calls):
    """(wall seconds, process CPU seconds) of running every call once."""
    c0, t0 = time.process_time(), time.perf_counter()
    for f in calls:
        f()
    return time.perf_counter() - t0, time.process_time() - c0


def run_cpu_baseline(w, case, budget_s=5.0, one_thread=False):
    """The fp64 oracle as it stands on a bounded sample of the batch: the
    requests in batch order until `budget_s` seconds of oracle time have
    passed (or all), then the same requests twice more; the median of the
    three runs. ``cores`` is the parallelism the runs actually had (process
    CPU time / wall time, rounded up), next to the BLAS thread count."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threadpool_limits, blas = None, 1
    Q = w.q_len_per_req
    calls, tokens, spent = [], 0, 0.0
    for i in range(w.batch):
        f = _oracle_call(w, case, i)
        dt, _ = _timed([f])
        spent += dt
        calls.append(f)
        L = int(case.pt.lengths[i])
        s0 = 0 if w.window_left < 0 else max(0, L - Q - w.window_left)
        tokens += L - s0
        if spent >= budget_s:
            break
    n = len(calls)
    nbytes = tokens * w.num_kv_heads * w.head_dim * 2 * ELEM[w.kv_dtype] + \
        n * Q * w.num_qo_heads * (w.head_dim * (ELEM[w.q_dtype] + ELEM[w.o_dtype]) + 4)
    runs = [_timed(calls) for _ in range(3)]
    wall = sorted(r[0] for r in runs)[1]
    cores = max(1, math.ceil(max(r[1] / r[0] for r in runs) - 0.05))
    out = {"value": round(nbytes / wall / 1e9, 4), "unit": "GB/s", "cores": int(cores),
           "kind": "oracle",
           "sample": f"{n} of {w.batch} requests ({tokens} attended tokens), fp64 "
                     f"NumPy, median of 3 runs of {wall:.2f} s (spread "
                     f"{runs_spread(runs)}); host has {os.cpu_count()} cpus, BLAS "
                     f"threads {blas}"}
    if one_thread and threadpool_limits is not None:
        with threadpool_limits(limits=1):
            r1 = sorted(_timed(calls)[0] for _ in range(3))[1]
        out["value_1thread"] = round(nbytes / r1 / 1e9, 4)
        out["sample"] += f"; one thread: median of 3 runs of {r1:.2f} s"
    return out


def runs_spread(runs):
    w = [r[0] for r in runs]
    return f"{min(w):.2f}-{max(w):.2f} s"


def profiled_traffic(workload: str, src_hash: str, launch_bytes: int):
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_hash:\s*(\w+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != src_hash:
        return None
    return float(t.group(1))


def per_call_protocol(call, first, n, dev, warm=10, flush_bytes=1 << 30):
    """Median / p10 / p90 µs of n single calls, each bracketed by HIP events
    on the current stream: "cold" with an untimed fill of flush_bytes before
    every call (more than the L2s and the 256 MB Infinity Cache hold), "hot"
    with no fill and the same pool every call. The fill keeps the GPU busy
    between calls, so the clocks stay up."""
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device=dev)
    out = {"calls": n, "warmup_calls": warm, "flush_bytes": flush_bytes}
    for label, flush in (("cold", True), ("hot", False)):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i in range(warm + n):
            if flush:
                scratch.fill_(i & 0xFF)
            # hot: call `first` on its pool every time; cold: rotate as usual
            k = first + i if flush else first
            call(k, evs[i - warm] if i >= warm else None)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        out[label] = {"median_us": round(float(np.median(us)), 2),
                      "p10_us": round(float(np.percentile(us, 10)), 2),
                      "p90_us": round(float(np.percentile(us, 90)), 2)}
    del scratch
    torch.cuda.synchronize()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gemma2_decode",
                    choices=sorted(wl.WORKLOADS))
    ap.add_argument("--replays", type=int, default=5,
                    help="timed replays of the graph holding the K calls")
    ap.add_argument("--layers", type=int, default=None,
                    help="calls per step, each on a cache of its own (default: "
                         "32 for the class example, whose loop runs over 32 "
                         "layers, else 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-calls", type=int, default=100,
                    help="single calls timed with HIP events, each after an untimed "
                         "1 GiB cache-evicting fill (and as many without it); 0 skips")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (for counter scaling)")
    ap.add_argument("--eager", action="store_true",
                    help="time host launches of the K calls instead of one "
                         "replay of a HIP graph holding them")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU "
              "path (the decode shards by request or kv head with no "
              "exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = wl.make_case(w, device=dev)
    layers = args.layers or (32 if w.name == "worked_example" else 1)
    used_bytes = int(case.pt.indptr[-1]) * 2 * w.page_size * w.num_kv_heads * \
        w.head_dim * ELEM[w.kv_dtype]
    # Distinct K/V pools: one per layer, and at least enough that a step
    # never finds the previous step's rows in the Infinity Cache.
    n_pools = max(layers, 2, math.ceil(2 * MALL_BYTES / max(used_bytes * layers, 1)) * layers)
    pools = [case.pool] + [wl.make_pool(w, case.pt.pool_pages, dev,
                                        seed=w.seed + 1000 * k)
                           for k in range(1, n_pools)]
    indices = torch.from_numpy(case.pt.indices).to(dev)
    plan = pkd.PagedDecodePlan(
        case.pt.indptr, indices, case.pt.last_page_len, w.num_qo_heads,
        w.num_kv_heads, w.head_dim, w.page_size, kv_layout=w.layout,
        window_left=w.window_left, logits_soft_cap=w.logits_soft_cap or None,
        q_data_type=w.q_dtype, kv_data_type=w.kv_dtype, o_data_type=w.o_dtype,
        sm_scale=w.sm_scale, fixed_split_size=w.fixed_split_size or None,
        q_len_per_req=w.q_len_per_req, pos_encoding_mode=w.pos_encoding_mode,
        rope_theta=w.rope_theta, rope_scale=w.rope_scale)
    info = plan.info
    rows = w.batch * w.q_len_per_req
    # per layer: its own q and outputs (the class example's loop)
    qs = [case.q] + [wl.make_q(w, np.random.default_rng(w.seed + 7 * k), device=dev)
                     for k in range(1, layers)]
    outs = [(torch.empty((rows, w.num_qo_heads, w.head_dim),
                         dtype=wl.TORCH_DTYPES[w.o_dtype], device=dev),
             torch.empty((rows, w.num_qo_heads), dtype=torch.float32, device=dev))
            for _ in range(layers)]
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8,
                     device=dev)
    total_bytes = algorithmic_bytes(w, case.pt)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def call(k, evs=None):
        """Call k: layer k % layers on pool k % n_pools."""
        li = k % layers
        if evs is not None:
            evs[0].record()
        plan.run(qs[li], pools[k % n_pools], k_scale=w.k_scale, v_scale=w.v_scale,
                 out=outs[li][0], lse=outs[li][1], workspace=ws)
        if evs is not None:
            evs[1].record()

    calls = args.steps * layers
    base = args.warmup * layers
    for k in range(base):
        call(k)
    torch.cuda.synchronize()
    def warm_eager():
        """WARM_S seconds of back-to-back eager passes: the GPU's clocks drop
        while it idles and take tens of milliseconds of work to come back."""
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < WARM_S:
            for k in range(calls):
                call(base + k)
            torch.cuda.synchronize()

    warm_eager()
    # Per-call protocol: HIP events around each single call, every call
    # preceded by an untimed 1 GiB fill that evicts the L2 and the Infinity
    # Cache ("cold"), and the same without the fill on one pool ("hot"). The
    # fills keep the GPU busy between calls, so the clocks stay up. Taken
    # before the graph so that the graph's replays stay the last launches of
    # a run.
    flushed = per_call_protocol(call, base, args.flush_calls, dev) if args.flush_calls > 0 else None
    # Eager pass: K steps launched from the host (the eager per-call figure).
    warm_eager()
    t0 = time.perf_counter()
    for k in range(calls):
        call(base + k)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) * 1e6 / calls
    launch = "eager"
    stream = torch.cuda.current_stream()
    if args.eager:
        graph = None
    else:
        # Whole-job throughput: the K steps' calls (the same pool rotation)
        # captured once in a HIP graph, replayed once untimed, then R times.
        # pkd_run allocates nothing and never synchronises, so it captures
        # as is.
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            call(0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for k in range(calls):
                call(base + k)
        graph.replay()
        torch.cuda.synchronize()
        launch = "hip_graph"
    # Steady state: the GPU's clocks drop while it idles (the capture above)
    # and take tens of milliseconds of back-to-back work to ramp up again, so
    # the timed regions follow at least WARM_S seconds of untimed ones.
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < WARM_S:
        if graph is not None:
            graph.replay()
        else:
            for k in range(calls):
                call(base + k)
        torch.cuda.synchronize()
    # Each timed region (one graph replay, or K eager launches) runs on
    # torch's current stream, where the kernels run, bracketed by two HIP
    # events (the kernel time, K launches back to back, and the gaps between
    # them) and by the host clock around synchronisations (the whole call).
    replay_us, kernel_us = [], []
    for _ in range(max(1, args.replays)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for k in range(calls):
                call(base + k)
        e1.record(stream)
        torch.cuda.synchronize()
        replay_us.append((time.perf_counter() - t0) * 1e6 / calls)
        kernel_us.append(e0.elapsed_time(e1) * 1e3 / calls)
    dec_avg = float(np.median(kernel_us)) / 1e3          # ms per launch
    us_call = float(np.median(replay_us))
    ms_step = us_call * layers / 1e3
    value = total_bytes / (us_call * 1e-6) / 1e9
    achieved = total_bytes / (dec_avg * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = profiled_traffic(w.name, src_hash, total_bytes)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(w, case, one_thread=w.name in ("worked_example",
                                                              "serving_batch"))

    line = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) and "
                  "μs/call",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_call": round(us_call, 2),
        "us_per_call_min_max": [round(min(replay_us), 2), round(max(replay_us), 2)],
        "replays": len(replay_us),
        "us_per_call_eager": round(eager_us, 2),
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype if w.kv_dtype == "e4m3" else w.q_dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.batch, "num_qo_heads": w.num_qo_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "page_size": w.page_size, "layout": w.layout,
            "q_dtype": w.q_dtype, "kv_dtype": w.kv_dtype,
            "logits_soft_cap": w.logits_soft_cap,
            "window_left": w.window_left,
            "fixed_split_size": w.fixed_split_size,
            "q_len_per_req": w.q_len_per_req,
            "pos_encoding_mode": w.pos_encoding_mode,
            "layers_per_step": layers,
            "split_pages_used": info.split_pages,
            "work_items": info.num_items,
            "attended_tokens": int(info.attended_tokens),
            "algorithmic_bytes_per_call": int(total_bytes),
            "kv_pools_rotated": n_pools,
            "launch": launch,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": "decode_kernel",
            "algorithmic_bytes_per_launch": int(total_bytes),
            "avg_launch_us": round(dec_avg * 1e3, 2),
            "avg_launch_us_min_max": [round(min(kernel_us), 2), round(max(kernel_us), 2)],
            "timing": "HIP events on the kernels' stream around each timed "
                      "region (K launches), median over the regions",
            "kernel_source_hash": src_hash,
        },
        "cpu_baseline": cpu,
        "per_call_events": flushed,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
