"""Shared test helpers: run the library and the oracle on the same inputs."""
import numpy as np
import torch

import oracle
import paged_kv_decode_09_amd as pkd
from paged_kv_decode_09_amd import workloads as wl

# max-abs tolerances on o by stored KV dtype (f16 / bf16 / fp8 E4M3 KV), and
# on the natural-log lse.
O_TOL = {"f16": 2e-3, "bf16": 1e-2, "e4m3": 3e-2}
LSE_TOL = 1e-3


def o_tol(w):
    return O_TOL["e4m3"] if w.kv_dtype == "e4m3" else O_TOL[w.o_dtype]


def plan_for(w, case, **overrides):
    kw = dict(kv_layout=w.layout, window_left=w.window_left,
              logits_soft_cap=w.logits_soft_cap or None,
              q_data_type=w.q_dtype, kv_data_type=w.kv_dtype,
              o_data_type=w.o_dtype, sm_scale=w.sm_scale,
              fixed_split_size=w.fixed_split_size or None,
              q_len_per_req=w.q_len_per_req,
              pos_encoding_mode=w.pos_encoding_mode, rope_theta=w.rope_theta,
              rope_scale=w.rope_scale)
    kw.update(overrides)
    indices = torch.from_numpy(case.pt.indices).to("cuda")
    return pkd.PagedDecodePlan(case.pt.indptr, indices, case.pt.last_page_len,
                               w.num_qo_heads, w.num_kv_heads, w.head_dim,
                               w.page_size, **kw)


def run_gpu(w, case, plan=None, cache=None, q=None, **overrides):
    plan = plan or plan_for(w, case, **overrides)
    o, lse = plan.run(case.q if q is None else q,
                      case.pool if cache is None else cache,
                      k_scale=w.k_scale, v_scale=w.v_scale, return_lse=True)
    torch.cuda.synchronize()
    return o, lse, plan


def sub_pool(case, requests):
    """The pages of the selected requests as a compact host pool with a
    renumbered page table (so the oracle does not copy the whole pool)."""
    pt = case.pt
    pages, indptr, last = [], [0], []
    for i in requests:
        pg = pt.indices[pt.indptr[i]:pt.indptr[i + 1]]
        pages.append(pg)
        indptr.append(indptr[-1] + len(pg))
        last.append(int(pt.last_page_len[i]))
    pages = np.concatenate(pages).astype(np.int64)
    host = case.pool[torch.from_numpy(pages).to(case.pool.device)].cpu()
    return host, np.array(indptr, np.int32), np.arange(len(pages),
                                                        dtype=np.int32), \
        np.array(last, np.int32)


def rows_of(w, requests):
    """Rows of q / o / lse that hold the given requests' query tokens."""
    Q = w.q_len_per_req
    return [i * Q + j for i in requests for j in range(Q)]


def oracle_for(w, case, requests=None, split_pages=None, q=None):
    """fp64 oracle o [len(requests) * Q, nq, hd] and lse for the case's
    inputs (Q query tokens per request)."""
    reqs = list(range(w.batch)) if requests is None else list(requests)
    pool, indptr, indices, last = sub_pool(case, reqs)
    qq = (case.q if q is None else q)[torch.tensor(rows_of(w, reqs))]
    qn = wl.raw_numpy(qq, w.q_dtype)
    pn = wl.raw_numpy(pool, w.kv_dtype)
    args = (qn, pn, w.layout, indptr, indices, last, w.page_size, w.q_dtype,
            w.kv_dtype, w.sm_scale)
    kw = dict(logits_soft_cap=w.logits_soft_cap, window_left=w.window_left,
              k_scale=w.k_scale, v_scale=w.v_scale)
    if w.pos_encoding_mode != "NONE":
        assert not split_pages, "the split oracle has no positional encoding"
        pos = dict(rope=(w.rope_theta, w.rope_scale)) if w.pos_encoding_mode == "ROPE_LLAMA" \
            else dict(alibi=True)
        return oracle.batch_decode_multi(qn, pn, w.layout, indptr, indices, last,
                                         w.page_size, w.q_len_per_req, w.q_dtype,
                                         w.kv_dtype, w.sm_scale, **kw, **pos)
    if w.q_len_per_req > 1:
        return oracle.batch_decode_multi(qn, pn, w.layout, indptr, indices, last,
                                         w.page_size, w.q_len_per_req, w.q_dtype,
                                         w.kv_dtype, w.sm_scale, **kw)
    if split_pages:
        return oracle.batch_decode_split(*args, split_pages, **kw)
    return oracle.batch_decode(*args, **kw)


def max_abs(gpu: torch.Tensor, ref: np.ndarray) -> float:
    g = gpu.detach().float().cpu().double().numpy()
    return float(np.max(np.abs(g - ref))) if ref.size else 0.0
