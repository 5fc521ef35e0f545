"""Benchmark of paged-KV batch decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pkd_run (one kernel launch: decode, with the merge of split
requests fused in) over one batch whose inputs already sit in HBM; the plan is built once before timing,
as plan() is amortised over layers and steps. Successive steps alternate
between distinct K/V pools so that no step finds the previous step's data in
the 256 MB Infinity Cache.

Prints one JSON line. ``value`` is the achieved HBM bandwidth of the whole
call: algorithmic bytes / wall time per call, with the K timed calls replayed
from one HIP graph (the way a serving loop issues its decode steps; pkd_run
allocates nothing and never synchronises, so it captures unchanged);
``--eager`` times K host launches instead. Algorithmic bytes = K and V rows
of the attended tokens (each read once per kv head) + q + o + fp32 lse + the
page indices of the touched pages + indptr + last_page_len.
``roofline`` is that kernel, timed with HIP events on the stream it runs on. ``cpu_baseline`` times the fp64 CPU oracle on a bounded sample.
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


def run_cpu_baseline(w, case, budget_s=10.0):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()]
                      or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    order = list(range(w.batch))
    done, elapsed, nbytes, tokens = [], 0.0, 0, 0
    kw = dict(logits_soft_cap=w.logits_soft_cap, window_left=w.window_left,
              k_scale=w.k_scale, v_scale=w.v_scale)
    rope = (w.rope_theta, w.rope_scale) \
        if w.pos_encoding_mode == "ROPE_LLAMA" else None
    alibi = w.pos_encoding_mode == "ALIBI"
    if rope or alibi:
        # only the one-token / multi-token oracle entry takes these
        kw.update(rope=rope, alibi=alibi)
    Q = w.q_len_per_req
    for i in order:
        pool, indptr, indices, last = _sub_pool(case, [i])
        qn = wl.raw_numpy(case.q[i * Q:(i + 1) * Q], w.q_dtype)
        pn = wl.raw_numpy(pool, w.kv_dtype)
        t = time.perf_counter()
        if Q > 1 or "rope" in kw:
            oracle.batch_decode_multi(qn, pn, w.layout, indptr, indices, last,
                                      w.page_size, Q, w.q_dtype, w.kv_dtype,
                                      w.sm_scale, **kw)
        elif w.fixed_split_size:
            oracle.batch_decode_split(qn, pn, w.layout, indptr, indices, last,
                                      w.page_size, w.q_dtype, w.kv_dtype,
                                      w.sm_scale, w.fixed_split_size, **kw)
        else:
            oracle.batch_decode(qn, pn, w.layout, indptr, indices, last,
                                w.page_size, w.q_dtype, w.kv_dtype, w.sm_scale,
                                **kw)
        elapsed += time.perf_counter() - t
        L = int(case.pt.lengths[i])
        s0 = 0 if w.window_left < 0 else max(0, L - Q - w.window_left)
        tokens += L - s0
        done.append(i)
        if elapsed >= budget_s:
            break
    kvb = tokens * w.num_kv_heads * w.head_dim * 2 * ELEM[w.kv_dtype]
    other = len(done) * Q * w.num_qo_heads * (w.head_dim * (
        ELEM[w.q_dtype] + ELEM[w.o_dtype]) + 4)
    gbs = (kvb + other) / elapsed / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(done)} of {w.batch} requests ({tokens} attended "
                      f"tokens), fp64 NumPy, {elapsed:.1f} s; host has "
                      f"{os.cpu_count()} cpus, BLAS threads {threads}"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="serving_batch",
                    choices=sorted(wl.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    used_bytes = int(case.pt.indptr[-1]) * 2 * w.page_size * w.num_kv_heads * \
        w.head_dim * ELEM[w.kv_dtype]
    n_pools = max(2, math.ceil(2 * MALL_BYTES / max(used_bytes, 1)))
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
    o = torch.empty((rows, w.num_qo_heads, w.head_dim),
                    dtype=wl.TORCH_DTYPES[w.o_dtype], device=dev)
    lse = torch.empty((rows, w.num_qo_heads), dtype=torch.float32,
                      device=dev)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8,
                     device=dev)
    total_bytes = algorithmic_bytes(w, case.pt)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(k, evs=None):
        pool = pools[k % n_pools]
        if evs is not None:
            evs[0].record()
        plan.run(case.q, pool, k_scale=w.k_scale, v_scale=w.v_scale, out=o,
                 lse=lse, workspace=ws)
        if evs is not None:
            evs[1].record()

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # Per-launch kernel time (the roofline): each call launched from the
    # host between two events on the stream it runs on.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k, events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_avg = float(np.mean(dec_ms))
    eager_us = wall * 1e6 / args.steps
    launch = "eager"
    if not args.eager:
        # Whole-job throughput: the K calls (the same pool rotation) captured
        # once in a HIP graph, replayed once untimed and once timed. pkd_run
        # allocates nothing and never synchronises, so it captures as is.
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for k in range(args.steps):
                step(args.warmup + k)
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        launch = "hip_graph"
    ms_step = wall * 1e3 / args.steps
    value = total_bytes / (ms_step * 1e-3) / 1e9
    achieved = total_bytes / (dec_avg * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = profiled_traffic(w.name, src_hash, total_bytes)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(w, case)

    line = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) and "
                  "μs/call",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_call": round(ms_step * 1e3, 2),
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
            "kernel_source_hash": src_hash,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
