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


def oracle_all(w, case, chunk=32, q=None):
    """oracle_for over every request of the batch, `chunk` requests at a
    time (bounds the host copy of the pages)."""
    outs, lses = [], []
    for r0 in range(0, w.batch, chunk):
        o, l = oracle_for(w, case, range(r0, min(w.batch, r0 + chunk)), q=q)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)


def _rne_error_var(x, dtype):
    """Variance of the error of rounding x (fp64) to nearest-even in `dtype`,
    with the error taken as uniform over one unit in the last place:
    ulp(x)^2 / 12, ulp(x) = 2^(floor(log2|x|) - (p - 1)) with p = 8
    significant bits (bf16) or 11 (f16), and the format's smallest
    spacing below its normal range."""
    p, emin = (8, -126) if dtype == "bf16" else (11, -14)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, emin)
    ulp = np.exp2(e - (p - 1))
    return np.where(ax > 0, ulp * ulp / 12.0, 0.0)


def rope_lse_bounds(w, case, requests, theta, scale, base=LSE_TOL, sigmas=6.0):
    """Per-row lse bound for ROPE_LLAMA runs, [len(requests) * Q, nq].

    With ROPE_LLAMA the kernel rounds the rotated q (once per unit) and each
    rotated key element to the MFMA operand type (the q dtype) before the
    dot product; the unrotated path never rounds its operands. Rounding
    error delta of an element x is modelled as independent, zero-mean,
    variance ulp(x)^2/12 (round to nearest even). A logit's error is then
    dx_t = sm * sum_d (dq_d k'_td + q'_d dk_td), and to first order the lse
    moves by sum_t p_t dx_t (p the softmax weights), whose variance is
        sm^2 [ sum_d var(dq_d) (sum_t p_t k'_td)^2
               + sum_t p_t^2 sum_d q'_d^2 var(dk_td) ]
    (the q error is shared by every token, the key errors are not). The
    bound is the plain path's lse tolerance plus `sigmas` standard
    deviations of that error; q', k' and p are the exact fp64 values (the
    soft cap's derivative, at most 1, is left out, which only widens the
    bound)."""
    import oracle as orc
    Q = w.q_len_per_req
    reqs = list(requests)
    pool, indptr, indices, last = sub_pool(case, reqs)
    rows = torch.tensor(rows_of(w, reqs))
    qn = orc.widen(wl.raw_numpy(case.q[rows], w.q_dtype), w.q_dtype)
    pn = wl.raw_numpy(pool, w.kv_dtype)
    kc = pn[:, 0]
    lens = orc.kv_lengths(indptr, last, w.page_size)
    nq, nkv, hd = w.num_qo_heads, w.num_kv_heads, w.head_dim
    G = nq // nkv
    sm = w.sm_scale
    out = np.zeros((len(reqs) * Q, nq))
    for r in range(len(reqs)):
        i = r
        L = int(lens[i])
        K, _ = orc.gather_request(kc, kc, w.layout, indices, indptr, i, L, w.page_size)
        Kf = orc.widen(K, w.kv_dtype, w.k_scale)                 # [L, nkv, hd]
        for j in range(Q):
            pos = L - Q + j
            s0 = 0 if w.window_left < 0 else max(0, pos - w.window_left)
            Kr = orc.rope_rotate(Kf[s0:pos + 1].transpose(1, 0, 2),
                                 np.arange(s0, pos + 1), theta, scale)  # [nkv, n, hd]
            vk = _rne_error_var(Kr / w.k_scale, w.q_dtype) * w.k_scale ** 2
            qr = orc.rope_rotate(qn[r * Q + j][:, None, :], [pos], theta, scale)[:, 0, :]
            vq = _rne_error_var(qr, w.q_dtype)
            for h in range(nkv):
                # the G q heads of kv head h at once: columns of [n, G]
                hs = slice(h * G, (h + 1) * G)
                x = sm * (Kr[h] @ qr[hs].T)
                if w.logits_soft_cap > 0:
                    x = w.logits_soft_cap * np.tanh(x / w.logits_soft_cap)
                p = np.exp(x - x.max(axis=0))
                p /= p.sum(axis=0)
                kbar = p.T @ Kr[h]                                # [G, hd]
                var = sm * sm * (np.sum(vq[hs] * kbar * kbar, axis=1) +
                                 np.sum(p * p * (vk[h] @ (qr[hs] * qr[hs]).T), axis=0))
                out[r * Q + j, hs] = base + sigmas * np.sqrt(var)
    return out


def rope_o_bounds(w, case, requests, theta, scale, ref_o, sigmas=6.0, base=True,
                  parts=("operands", "p")):
    """Elementwise o bound for ROPE_LLAMA runs, shaped like ref_o
    [len(requests) * Q, nq, hd]: o_bounds (the tolerance, or the output's own
    rounding) plus `sigmas` standard deviations of the error that the RoPE
    instances' roundings add to o. Besides the rotated q and keys rounded to
    the q dtype (the logit errors dx_t of rope_lse_bounds), these instances
    take P into P.V as a single operand term: p rounded to the q dtype, with
    relative error e_t. To first order
        do_j = sum_t p_t (dx_t - sum_s p_s dx_s) v_tj + sum_t p_t e_t v_tj,
    and with all rounding errors independent and zero-mean
        var(do_j) = sm^2 [ sum_d var(dq_d) (sum_t p_t k'_td (v_tj - o_j))^2
                           + sum_t p_t^2 (v_tj - o_j)^2 sum_d q'_d^2 var(dk_td) ]
                    + sum_t var(p_t e_t) v_tj^2,
    the last from rounding p_t / max_s p_s (the kernel rounds p against its
    running maximum) scaled back. q', k', p, v and o are exact fp64 values;
    the soft cap's derivative (at most 1) is left out, which only widens the
    bound. base=False returns the sigmas-standard-deviation term alone;
    `parts` selects the error sources ("operands": q and keys, "p": P)."""
    import oracle as orc
    Q = w.q_len_per_req
    reqs = list(requests)
    pool, indptr, indices, last = sub_pool(case, reqs)
    rows = torch.tensor(rows_of(w, reqs))
    qn = orc.widen(wl.raw_numpy(case.q[rows], w.q_dtype), w.q_dtype)
    pn = wl.raw_numpy(pool, w.kv_dtype)
    lens = orc.kv_lengths(indptr, last, w.page_size)
    nq, nkv, hd = w.num_qo_heads, w.num_kv_heads, w.head_dim
    G = nq // nkv
    sm = w.sm_scale
    out = np.array(o_bounds(w, ref_o), dtype=np.float64) if base else \
        np.zeros(np.shape(ref_o))
    for r in range(len(reqs)):
        L = int(lens[r])
        K, V = orc.gather_request(pn[:, 0], pn[:, 1], w.layout, indices, indptr, r, L,
                                  w.page_size)
        Kf = orc.widen(K, w.kv_dtype, w.k_scale)                 # [L, nkv, hd]
        Vf = orc.widen(V, w.kv_dtype, w.v_scale)
        for j in range(Q):
            pos = L - Q + j
            s0 = 0 if w.window_left < 0 else max(0, pos - w.window_left)
            Kr = orc.rope_rotate(Kf[s0:pos + 1].transpose(1, 0, 2),
                                 np.arange(s0, pos + 1), theta, scale)  # [nkv, n, hd]
            vk = _rne_error_var(Kr / w.k_scale, w.q_dtype) * w.k_scale ** 2
            qr = orc.rope_rotate(qn[r * Q + j][:, None, :], [pos], theta, scale)[:, 0, :]
            vq = _rne_error_var(qr, w.q_dtype)
            for h in range(nkv):
                # the G q heads of kv head h at once (columns of [n, G]); the
                # sums over tokens t of terms in (v_tj - o_j) are expanded in
                # powers of o_j, so that each is a product with V or V*V
                hs = slice(h * G, (h + 1) * G)
                Vh = Vf[s0:pos + 1, h]                            # [n, hd]
                V2 = Vh * Vh
                x = sm * (Kr[h] @ qr[hs].T)                       # [n, G]
                if w.logits_soft_cap > 0:
                    x = w.logits_soft_cap * np.tanh(x / w.logits_soft_cap)
                p = np.exp(x - x.max(axis=0))
                p /= p.sum(axis=0)
                o = p.T @ Vh                                      # [G, hd]
                kp = Kr[h].T @ p                                  # [d, G]: sum_t p_t k'_td
                for g in range(G):
                    # A_dj = sum_t p_t k'_td (v_tj - o_j)
                    A = (Kr[h] * p[:, g:g + 1]).T @ Vh - np.outer(kp[:, g], o[g])
                    t1 = vq[h * G + g] @ (A * A)
                    s = vk[h] @ (qr[h * G + g] * qr[h * G + g])   # [n]
                    wt = p[:, g] * p[:, g] * s
                    t2 = wt @ V2 - 2.0 * o[g] * (wt @ Vh) + o[g] * o[g] * wt.sum()
                    pg = p[:, g]
                    pm = pg.max()
                    # (the maximum, p / pm = 1, is exact in any format: no error)
                    vp = np.where(pg == pm, 0.0, _rne_error_var(pg / pm, w.q_dtype) * pm * pm)
                    t3 = vp @ V2
                    var = (sm * sm * (t1 + t2) if "operands" in parts else 0.0) + \
                        (t3 if "p" in parts else 0.0)
                    out[r * Q + j, h * G + g] += sigmas * np.sqrt(np.maximum(var, 0.0))
    return out


def o_bounds(w, ref):
    """Elementwise bound on |o - ref| for an output of dtype w.o_dtype: the
    max-abs tolerance, or, where the exact value is too large in magnitude
    for that tolerance to be reachable, half a unit in the last place of the
    exact value in the output dtype (the error of rounding it to nearest)
    plus 1e-4 for the fp32 arithmetic before the rounding. For bf16 that
    widens the 1e-2 bound only where |o| >= 4 (a half ulp of 2^-6 there);
    for f16 the 2e-3 bound where |o| >= 8."""
    p = 8 if w.o_dtype == "bf16" else 11
    ax = np.abs(np.asarray(ref, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    half_ulp = np.where(ax > 0, np.exp2(e - (p - 1)) / 2, 0.0)
    return np.maximum(o_tol(w), half_ulp + 1e-4)
