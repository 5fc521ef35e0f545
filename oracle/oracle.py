"""Plain fp64 CPU oracle: batch decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring). Slow on purpose: every
request is gathered page by page into dense K/V and attended with a dense
softmax in float64. No blocking, fusion or reordering beyond what the
definition states.

What is computed, and where the pages define it ("FlashInfer attention
kernels" page, section flashinfer.decode › BatchDecodeWithPagedKVCacheWrapper,
unless stated otherwise):

* Page table (plan() parameters indptr / indices / last_page_len, and the
  class example's comment that 1 <= last_page_len <= page_size): request i owns
  pages indices[indptr[i]:indptr[i+1]]; every page but the last is full.
* Sequence length: kv_len = page_size*(indptr[i+1]-indptr[i]-1) +
  last_page_len[i] (the kv_len expression in the custom-mask part of the
  BatchPrefillWithPagedKVCacheWrapper example on the same page).
* Cache layouts (run() parameter paged_kv_cache): NHD pages are
  [page_size, num_kv_heads, head_dim], HND pages are
  [num_kv_heads, page_size, head_dim]; the 5-D form stacks K at index 0 and V
  at index 1 of dimension 1.
* Grouped heads (plan() notes): num_qo_heads is a multiple of num_kv_heads.
  Reading taken: q head hq uses kv head hq // (num_qo_heads // num_kv_heads).
* Logits: x = sm_scale * q.k (sm_scale default 1/sqrt(head_dim), stated in the
  prefill plan() parameters); q_scale / k_scale / v_scale are the calibration
  scales of run(), applied to q, K and V.
* Soft cap (plan() parameter logits_soft_cap): if cap > 0 the logit x is
  replaced by cap * tanh(x / cap). Reading taken: x is the scaled logit.
* Window (plan() parameter window_left): a left window that includes its
  edge; -1 means the whole sequence. Reading taken: the single query sits at
  position kv_len-1 (the causal diagonal kv_len - qo_len of the prefill mask
  example with qo_len = 1), so it sees tokens t >= kv_len-1-window_left.
* Output (run() returns): o [batch, num_qo_heads, head_dim] and, on request,
  lse [batch, num_qo_heads], the log-sum-exp of the final logits. Reading
  taken: natural logarithm.
* Split-KV (plan() parameter fixed_split_size, a count of pages): the sequence is
  cut into chunks of that many pages; per-chunk states are combined by a
  log-sum-exp merge (the merge_states step named there).
* Positional encoding ALIBI (plan() parameter pos_encoding_mode; the
  encoding happens within the attention kernel). Readings taken: the slopes of the ALiBi
  paper over the num_qo_heads q heads (for n a power of two, head h gets
  2^(-8(h+1)/n); otherwise the n' = 2^floor(log2 n) slopes of that rule,
  then the odd powers of 2^(-4/n') for the remaining heads), and the bias
  slope * (t - query position) is added to the scaled logit before the soft
  cap.
* Positional encoding ROPE_LLAMA (same parameter; rope_scale, the RoPE
  interpolation factor, default 1; rope_theta default 1e4). Readings taken: the
  Llama-style rotary embedding rotates each pair (x[i], x[i + head_dim/2]),
  i < head_dim/2, of q (at its query position) and of every key (at its
  token index) by the angle position / rope_scale * rope_theta^(-2i/head_dim);
  values are not rotated; the rotation comes before q_scale/k_scale-scaled
  logits, the ALiBi bias and the cap as the kernel applies it to stored K.
* Several query tokens per request (run() parameter q_len_per_req, default
  1). Readings taken: q, o and lse hold q_len_per_req consecutive rows per
  request, in token order; query token j of a request sits at position
  kv_len - q_len_per_req + j, the causal diagonal kv_len - qo_len of the
  prefill mask example, so it attends tokens t <= that position (and, with a
  window, t >= that position - window_left). Each query token is therefore
  exactly a one-token decode over the prefix that ends at its position.
"""
import math

import numpy as np

from .fp8 import e4m3_to_f64

DTYPES = ("f16", "bf16", "e4m3", "f32", "f64")


def widen(a, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Exact float64 values of stored data, times a calibration scale.

    ``f16`` arrays are np.float16; ``bf16`` arrays are the raw uint16 bit
    patterns (numpy has no bfloat16); ``e4m3`` arrays are uint8 codes.
    """
    a = np.asarray(a)
    if dtype == "f16":
        if a.dtype != np.float16:
            raise TypeError("f16 data must be np.float16")
        out = a.astype(np.float64)
    elif dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be raw np.uint16 bit patterns")
        with np.errstate(invalid="ignore"):
            out = (a.astype(np.uint32) << 16).view(np.float32).astype(
                np.float64)
    elif dtype == "e4m3":
        out = e4m3_to_f64(a)
    elif dtype in ("f32", "f64"):
        out = a.astype(np.float64)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    return out * float(scale) if scale != 1.0 else out


def kv_lengths(indptr, last_page_len, page_size: int) -> np.ndarray:
    """Per-request KV length from the CSR page table."""
    indptr = np.asarray(indptr, dtype=np.int64)
    last = np.asarray(last_page_len, dtype=np.int64)
    npages = indptr[1:] - indptr[:-1]
    if np.any(npages < 1):
        raise ValueError("every request needs at least one page")
    if np.any(last < 1) or np.any(last > page_size):
        raise ValueError("last_page_len must lie in [1, page_size]")
    return page_size * (npages - 1) + last


def csr_from_block_table(seq_lens, block_tables, page_size: int):
    """CSR page table (indptr, indices, last_page_len) of a block table.

    The XQA decode on the API page takes page_table [batch, nb_pages_per_seq]
    (K and V share it) and seq_lens; request i owns the pages
    block_tables[i, 0 : ceil(seq_lens[i] / page_size)], and its last page
    holds seq_lens[i] - page_size * (pages - 1) tokens.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    block_tables = np.asarray(block_tables)
    if np.any(seq_lens < 1):
        raise ValueError("every request needs at least one token")
    npages = (seq_lens + page_size - 1) // page_size
    if np.any(npages > block_tables.shape[1]):
        raise ValueError("a request needs more pages than its row holds")
    indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
    indices = np.concatenate([block_tables[i, :n] for i, n in
                              enumerate(npages)]).astype(np.int32)
    last = (seq_lens - page_size * (npages - 1)).astype(np.int32)
    return indptr, indices, last


def rope_rotate(x, positions, rope_theta: float = 1e4, rope_scale: float = 1.0):
    """Llama-style rotary embedding of rows x [..., n, head_dim] at the
    given positions [n] (fp64): pair (i, i + head_dim/2) turns by
    position / rope_scale * rope_theta^(-2i/head_dim)."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = rope_theta ** (-2.0 * np.arange(half) / hd) / rope_scale
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def alibi_slopes(num_heads: int) -> np.ndarray:
    """ALiBi slopes of num_heads heads (the geometric sequence of the ALiBi
    paper; the closest power of two below n, then interleaved extra slopes)."""
    n2 = 2 ** int(math.floor(math.log2(num_heads)))
    base = [2.0 ** (-8.0 * (h + 1) / n2) for h in range(n2)]
    extra = [2.0 ** (-4.0 * (2 * k + 1) / n2) for k in range(num_heads - n2)]
    return np.array(base + extra, dtype=np.float64)


def window_start(kv_len: int, window_left: int) -> int:
    """First attended token of a request whose query sits at kv_len-1."""
    if window_left < 0:
        return 0
    return max(0, kv_len - 1 - window_left)


def gather_request(k_cache, v_cache, layout: str, indices, indptr, i: int,
                   kv_len: int, page_size: int):
    """Dense K and V [kv_len, num_kv_heads, head_dim] of request i, bit-exact.

    ``k_cache`` / ``v_cache`` are the 4-D per-tensor caches (for the 5-D form
    pass cache[:, 0] and cache[:, 1]). The stored dtype is kept unchanged.
    """
    t = np.arange(kv_len)
    pages = np.asarray(indices)[int(indptr[i]) + t // page_size]
    slots = t % page_size
    if layout == "NHD":
        return k_cache[pages, slots], v_cache[pages, slots]
    if layout == "HND":
        # [page, head, slot, dim] -> pick (page, slot) per token, keep heads.
        return (k_cache[pages, :, slots, :], v_cache[pages, :, slots, :])
    raise ValueError(f"unknown layout {layout!r}")


def attention_state(q, K, V, sm_scale: float, logits_soft_cap: float = 0.0,
                    return_weights: bool = False, sinks=None, bias=None):
    """Dense softmax attention of one query row per q head over n tokens.

    q: [num_qo_heads, head_dim]; K, V: [n, num_kv_heads, head_dim]; all fp64.
    Returns (o [num_qo_heads, head_dim], lse [num_qo_heads]) and, if asked,
    the weights p [num_qo_heads, n]. With n == 0 the state is empty:
    o = 0, lse = -inf.

    ``bias`` (optional, [num_qo_heads, n]): added to the scaled logits before
    the soft cap (the ALiBi bias).

    ``sinks`` (optional, [num_qo_heads]): the attention-sink values of the
    XQA decode on the API page ("sinks" [num_kv_heads, head_group_ratio]
    float32, flattened in q-head order). Reading taken: sink s of a q head
    is one more logit in that head's softmax, compared with the final
    (scaled, capped) logits, that carries no value row: o = sum_t e^x_t v_t /
    (sum_t e^x_t + e^s), and lse = ln(sum_t e^x_t + e^s).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    nq, hd = q.shape
    n, nkv, _ = K.shape
    if nq % nkv:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    group = nq // nkv
    o = np.zeros((nq, hd))
    lse = np.full(nq, -np.inf)
    p_all = np.zeros((nq, n))
    if n == 0:
        return (o, lse, p_all) if return_weights else (o, lse)
    for hq in range(nq):
        h = hq // group
        x = sm_scale * (K[:, h, :] @ q[hq])
        if bias is not None:
            x = x + bias[hq]
        if logits_soft_cap > 0:
            x = logits_soft_cap * np.tanh(x / logits_soft_cap)
        m = x.max()
        if sinks is not None:
            m = max(m, float(sinks[hq]))
        p = np.exp(x - m)
        z = p.sum()
        if sinks is not None:
            z += math.exp(float(sinks[hq]) - m)
        o[hq] = (p @ V[:, h, :]) / z
        lse[hq] = m + math.log(z)
        p_all[hq] = p / z
    return (o, lse, p_all) if return_weights else (o, lse)


def _request_f64(q_i, K, V, q_dtype, kv_dtype, q_scale, k_scale, v_scale):
    return (widen(q_i, q_dtype, q_scale), widen(K, kv_dtype, k_scale),
            widen(V, kv_dtype, v_scale))


def decode_request(q_i, K, V, q_dtype: str, kv_dtype: str, sm_scale: float,
                   logits_soft_cap: float = 0.0, window_left: int = -1,
                   q_scale: float = 1.0, k_scale: float = 1.0,
                   v_scale: float = 1.0, sinks=None, alibi: bool = False,
                   rope=None):
    """Decode attention of one request from its gathered (stored-dtype) K/V.

    ``rope`` = (rope_theta, rope_scale) applies ROPE_LLAMA to q (at position
    kv_len - 1) and to each key (at its token index)."""
    kv_len = K.shape[0]
    s0 = window_start(kv_len, window_left)
    qf, Kf, Vf = _request_f64(q_i, K[s0:], V[s0:], q_dtype, kv_dtype,
                              q_scale, k_scale, v_scale)
    if rope is not None:
        theta, scale = rope
        qf = rope_rotate(qf[:, None, :], [kv_len - 1], theta, scale)[:, 0, :]
        Kf = rope_rotate(Kf.transpose(1, 0, 2), np.arange(s0, kv_len), theta,
                         scale).transpose(1, 0, 2)
    bias = None
    if alibi:
        # the query sits at kv_len - 1; token t is (kv_len - 1 - t) behind it
        dist = np.arange(s0, kv_len, dtype=np.float64) - (kv_len - 1)
        bias = alibi_slopes(qf.shape[0])[:, None] * dist[None, :]
    return attention_state(qf, Kf, Vf, sm_scale, logits_soft_cap, sinks=sinks,
                           bias=bias)


def _cache_pair(paged_kv_cache):
    if isinstance(paged_kv_cache, (tuple, list)):
        return paged_kv_cache[0], paged_kv_cache[1]
    return paged_kv_cache[:, 0], paged_kv_cache[:, 1]


def batch_decode(q, paged_kv_cache, layout: str, indptr, indices,
                 last_page_len, page_size: int, q_dtype: str, kv_dtype: str,
                 sm_scale: float, logits_soft_cap: float = 0.0,
                 window_left: int = -1, q_scale: float = 1.0,
                 k_scale: float = 1.0, v_scale: float = 1.0, requests=None,
                 sinks=None, alibi: bool = False, rope=None):
    """o [len(requests), num_qo_heads, head_dim] and lse, both fp64.

    ``q`` is [batch, num_qo_heads, head_dim] in its stored dtype;
    ``paged_kv_cache`` is the 5-D cache or a (k_cache, v_cache) pair.
    ``requests`` selects a subset of the batch (default: all).
    """
    k_cache, v_cache = _cache_pair(paged_kv_cache)
    lens = kv_lengths(indptr, last_page_len, page_size)
    reqs = range(len(lens)) if requests is None else list(requests)
    nq, hd = q.shape[1], q.shape[2]
    o = np.zeros((len(reqs), nq, hd))
    lse = np.zeros((len(reqs), nq))
    for r, i in enumerate(reqs):
        K, V = gather_request(k_cache, v_cache, layout, indices, indptr, i,
                              int(lens[i]), page_size)
        o[r], lse[r] = decode_request(q[i], K, V, q_dtype, kv_dtype, sm_scale,
                                      logits_soft_cap, window_left, q_scale,
                                      k_scale, v_scale, sinks, alibi, rope)
    return o, lse


def chunk_bounds(kv_len: int, page_size: int, split_pages: int,
                 window_left: int = -1):
    """Token ranges [begin, end) of the fixed-size chunks of one request.

    Chunk c covers pages [c*split_pages, (c+1)*split_pages) counted from the
    request's first page, cut to the attended range [window start, kv_len).
    Chunks with nothing to attend are dropped. split_pages <= 0 means one
    chunk.
    """
    s0 = window_start(kv_len, window_left)
    if split_pages <= 0:
        return [(s0, kv_len)]
    step = split_pages * page_size
    out = []
    for b in range(0, kv_len, step):
        lo, hi = max(b, s0), min(b + step, kv_len)
        if lo < hi:
            out.append((lo, hi))
    return out


def merge_states(v, s):
    """Log-sum-exp merge of attention states, chunk by chunk.

    v: [rows, n, head_dim] per-chunk normalised outputs; s: [rows, n] per-chunk
    natural-log LSE. Returns (v_merged [rows, head_dim], s_merged [rows]).
    A state with s = -inf is empty and contributes nothing; rows whose states
    are all empty give v = 0, s = -inf.
    """
    v = np.asarray(v, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    rows, n, hd = v.shape
    v_out = np.zeros((rows, hd))
    s_out = np.full(rows, -np.inf)
    for r in range(rows):
        m = s[r].max() if n else -np.inf
        if m == -np.inf:
            continue
        w = np.exp(s[r] - m)
        z = w.sum()
        v_out[r] = (w @ v[r]) / z
        s_out[r] = m + math.log(z)
    return v_out, s_out


def decode_request_split(q_i, K, V, q_dtype: str, kv_dtype: str,
                         sm_scale: float, page_size: int, split_pages: int,
                         logits_soft_cap: float = 0.0, window_left: int = -1,
                         q_scale: float = 1.0, k_scale: float = 1.0,
                         v_scale: float = 1.0):
    """Split-KV decode of one request: per-chunk states, then merge_states."""
    kv_len = K.shape[0]
    qf, Kf, Vf = _request_f64(q_i, K, V, q_dtype, kv_dtype, q_scale, k_scale,
                              v_scale)
    states = [attention_state(qf, Kf[a:b], Vf[a:b], sm_scale, logits_soft_cap)
              for a, b in chunk_bounds(kv_len, page_size, split_pages,
                                       window_left)]
    v = np.stack([st[0] for st in states], axis=1)   # [nq, n, hd]
    s = np.stack([st[1] for st in states], axis=1)   # [nq, n]
    return merge_states(v, s)


def batch_decode_split(q, paged_kv_cache, layout: str, indptr, indices,
                       last_page_len, page_size: int, q_dtype: str,
                       kv_dtype: str, sm_scale: float, split_pages: int,
                       logits_soft_cap: float = 0.0, window_left: int = -1,
                       q_scale: float = 1.0, k_scale: float = 1.0,
                       v_scale: float = 1.0, requests=None):
    """batch_decode through fixed-size chunks and merge_states."""
    k_cache, v_cache = _cache_pair(paged_kv_cache)
    lens = kv_lengths(indptr, last_page_len, page_size)
    reqs = range(len(lens)) if requests is None else list(requests)
    nq, hd = q.shape[1], q.shape[2]
    o = np.zeros((len(reqs), nq, hd))
    lse = np.zeros((len(reqs), nq))
    for r, i in enumerate(reqs):
        K, V = gather_request(k_cache, v_cache, layout, indices, indptr, i,
                              int(lens[i]), page_size)
        o[r], lse[r] = decode_request_split(
            q[i], K, V, q_dtype, kv_dtype, sm_scale, page_size, split_pages,
            logits_soft_cap, window_left, q_scale, k_scale, v_scale)
    return o, lse


def batch_decode_multi(q, paged_kv_cache, layout: str, indptr, indices,
                       last_page_len, page_size: int, q_len_per_req: int,
                       q_dtype: str, kv_dtype: str, sm_scale: float,
                       logits_soft_cap: float = 0.0, window_left: int = -1,
                       q_scale: float = 1.0, k_scale: float = 1.0,
                       v_scale: float = 1.0, requests=None, sinks=None,
                       alibi: bool = False, rope=None):
    """Decode with q_len_per_req query tokens per request, fp64.

    ``q`` is [batch * q_len_per_req, num_qo_heads, head_dim] (request-major,
    tokens in order). Returns o [len(requests) * q_len_per_req, num_qo_heads,
    head_dim] and lse [len(requests) * q_len_per_req, num_qo_heads]. Query
    token j of request i is the one-token decode of the prefix of length
    kv_len - q_len_per_req + j + 1.
    """
    Q = int(q_len_per_req)
    if Q < 1:
        raise ValueError("q_len_per_req must be >= 1")
    k_cache, v_cache = _cache_pair(paged_kv_cache)
    lens = kv_lengths(indptr, last_page_len, page_size)
    if np.any(lens < Q):
        raise ValueError("every request needs kv_len >= q_len_per_req")
    reqs = range(len(lens)) if requests is None else list(requests)
    nq, hd = q.shape[1], q.shape[2]
    o = np.zeros((len(reqs) * Q, nq, hd))
    lse = np.zeros((len(reqs) * Q, nq))
    for r, i in enumerate(reqs):
        L = int(lens[i])
        K, V = gather_request(k_cache, v_cache, layout, indices, indptr, i, L,
                              page_size)
        for j in range(Q):
            pos = L - Q + j
            o[r * Q + j], lse[r * Q + j] = decode_request(
                q[i * Q + j], K[:pos + 1], V[:pos + 1], q_dtype, kv_dtype,
                sm_scale, logits_soft_cap, window_left, q_scale, k_scale,
                v_scale, sinks, alibi, rope)
    return o, lse
