"""Seeded synthetic inputs for paged-KV batch decode.

This module only draws inputs: sequence lengths, page tables, queries and
K/V pools. It holds none of the attention arithmetic, and both the library's
tests and the CPU oracle's tests take their inputs from here.

Named workloads follow the shapes of the class example on the "FlashInfer
attention kernels" page (flashinfer.decode › BatchDecodeWithPagedKVCacheWrapper)
and four decode workloads of the same kind (a serving batch, long-context
split-KV, a Gemma-2-style soft-capped windowed decode, and fp8 KV), plus the
serving batch with several query tokens per request (run()'s
q_len_per_req).

Recipe (per workload, ``rng = numpy.random.default_rng(seed)``, drawn in this
order): lengths -> page permutation -> q -> K/V pool. The pool is drawn with a
``torch.Generator`` seeded with the same number on the pool's device, in page
slices, as N(0, 1) fp32 rounded to nearest-even into the stored dtype. fp8 E4M3
pools store round(clamp(x / scale, -448, 448)) through torch's float8_e4m3fn
cast and are handed around as their uint8 codes.
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np
import torch

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16,
                "e4m3": torch.uint8}


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    q_dtype: str
    kv_dtype: str
    o_dtype: str
    layout: str
    lengths: tuple            # ("fixed", [...]) | ("uniform", lo, hi) |
                              # ("lognormal", median, sigma, lo, hi) |
                              # ("table", indptr, last_page_len)
    pages: str = "perm_used"  # "arange" | "perm_used" | "perm_pool"
    pool_pages: Optional[int] = None
    logits_soft_cap: float = 0.0
    window_left: int = -1
    fixed_split_size: int = 0
    k_scale: float = 1.0
    v_scale: float = 1.0
    q_len_per_req: int = 1    # query tokens per request (q has batch * this rows)
    pos_encoding_mode: str = "NONE"   # NONE | ALIBI | ROPE_LLAMA
    rope_theta: float = 1e4
    rope_scale: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


WORKLOADS = {
    "worked_example": Workload(
        "worked_example", 1, 7, 64, 8, 128, 16, "f16", "f16", "f16", "NHD",
        ("table", [0, 17, 29, 44, 48, 66, 100, 128], [1, 7, 14, 4, 3, 1, 16]),
        pages="arange", pool_pages=128,
        note="class example of BatchDecodeWithPagedKVCacheWrapper"),
    "serving_batch": Workload(
        "serving_batch", 2, 64, 32, 8, 128, 16, "bf16", "bf16", "bf16", "HND",
        ("uniform", 512, 4096), pages="perm_pool", pool_pages=20000,
        note="64 requests, L ~ U[512, 4096], pages drawn from a 20k pool"),
    "long_context": Workload(
        "long_context", 3, 4, 64, 8, 128, 16, "f16", "f16", "f16", "NHD",
        ("fixed", [32768, 65536, 98304, 131072]), pages="perm_used",
        fixed_split_size=256,
        note="4 long requests, fixed split of 256 pages"),
    "gemma2_decode": Workload(
        "gemma2_decode", 4, 256, 16, 8, 256, 16, "bf16", "bf16", "bf16",
        "NHD", ("lognormal", 2048, 1.0, 128, 8192), pages="perm_used",
        logits_soft_cap=50.0, window_left=4096,
        note="log-normal lengths, soft cap 50, window 4096"),
    "fp8_kv": Workload(
        "fp8_kv", 5, 128, 64, 8, 128, 16, "bf16", "e4m3", "bf16", "NHD",
        ("uniform", 2048, 16384), pages="perm_used", k_scale=1.0 / 64,
        v_scale=1.0 / 64, note="E4M3 KV with per-tensor scale 1/64"),
    "spec_decode": Workload(
        "spec_decode", 6, 64, 32, 8, 128, 16, "bf16", "bf16", "bf16", "HND",
        ("uniform", 512, 4096), pages="perm_pool", pool_pages=20000,
        q_len_per_req=4,
        note="the serving batch with 4 query tokens per request (causal)"),
    "serving_rope": Workload(
        "serving_rope", 2, 64, 32, 8, 128, 16, "bf16", "bf16", "bf16", "HND",
        ("uniform", 512, 4096), pages="perm_pool", pool_pages=20000,
        pos_encoding_mode="ROPE_LLAMA",
        note="the serving batch with Llama-style rotary embedding in the kernel"),
}


def draw_lengths(w: Workload, rng: np.random.Generator) -> np.ndarray:
    kind = w.lengths[0]
    if kind == "fixed":
        return np.asarray(w.lengths[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(w.lengths[1], w.lengths[2], w.batch,
                            endpoint=True).astype(np.int64)
    if kind == "lognormal":
        med, sigma, lo, hi = w.lengths[1:]
        x = np.rint(med * np.exp(rng.normal(0.0, sigma, w.batch)))
        return np.clip(x, lo, hi).astype(np.int64)
    if kind == "table":
        indptr = np.asarray(w.lengths[1], dtype=np.int64)
        last = np.asarray(w.lengths[2], dtype=np.int64)
        return w.page_size * (np.diff(indptr) - 1) + last
    raise ValueError(kind)


@dataclass
class PageTable:
    lengths: np.ndarray        # int64 [B], the drawn KV lengths
    indptr: np.ndarray         # int32 [B+1]
    indices: np.ndarray        # int32 [indptr[-1]]
    last_page_len: np.ndarray  # int32 [B]
    pool_pages: int


def page_table_for(lengths: Sequence[int], page_size: int, pages: str,
                   rng: np.random.Generator,
                   pool_pages: Optional[int] = None) -> PageTable:
    """A CSR page table that stores the given lengths.

    Each request gets ceil(L / page_size) pages; its last page holds the
    remainder (a full page when page_size divides L).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    if np.any(lengths < 1):
        raise ValueError("lengths must be >= 1")
    npages = (lengths + page_size - 1) // page_size
    last = lengths - page_size * (npages - 1)
    indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
    used = int(indptr[-1])
    pool = used if pool_pages is None else int(pool_pages)
    if pool < used:
        raise ValueError("pool smaller than the pages needed")
    if pages == "arange":
        indices = np.arange(used)
    elif pages == "perm_used":
        indices = rng.permutation(used)
    elif pages == "perm_pool":
        indices = rng.permutation(pool)[:used]
    else:
        raise ValueError(pages)
    return PageTable(lengths, indptr, indices.astype(np.int32),
                     last.astype(np.int32), pool)


def make_page_table(w: Workload, rng: np.random.Generator) -> PageTable:
    lengths = draw_lengths(w, rng)
    return page_table_for(lengths, w.page_size, w.pages, rng, w.pool_pages)


def make_q(w: Workload, rng: np.random.Generator, scale: float = 1.0,
           device="cpu") -> torch.Tensor:
    x = rng.standard_normal((w.batch * w.q_len_per_req, w.num_qo_heads,
                             w.head_dim), dtype=np.float32) * np.float32(scale)
    return torch.from_numpy(x).to(TORCH_DTYPES[w.q_dtype]).to(device)


def cache_shape(w: Workload, pool_pages: int, five_d: bool = True):
    if w.layout == "NHD":
        page = (w.page_size, w.num_kv_heads, w.head_dim)
    else:
        page = (w.num_kv_heads, w.page_size, w.head_dim)
    return (pool_pages, 2) + page if five_d else (pool_pages,) + page


def to_e4m3_codes(x: torch.Tensor, scale: float) -> torch.Tensor:
    """uint8 E4M3 codes of x / scale, clamped to the finite range first."""
    y = (x / scale).clamp_(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def make_pool(w: Workload, pool_pages: int, device="cpu", seed=None,
              slice_pages: int = 2048) -> torch.Tensor:
    """The 5-D paged cache [pool, 2, ...] filled with seeded N(0, 1) data."""
    shape = cache_shape(w, pool_pages)
    out = torch.empty(shape, dtype=TORCH_DTYPES[w.kv_dtype], device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    for p0 in range(0, pool_pages, slice_pages):
        p1 = min(pool_pages, p0 + slice_pages)
        x = torch.randn((p1 - p0,) + shape[1:], generator=gen,
                        dtype=torch.float32, device=device)
        if w.kv_dtype == "e4m3":
            out[p0:p1] = to_e4m3_codes(x, w.k_scale)
        else:
            out[p0:p1] = x.to(out.dtype)
        del x
    return out


NAN_CODE = {"f16": 0x7E00, "bf16": 0x7FC0, "e4m3": 0x7F}


def poison_unused(w: Workload, pool: torch.Tensor, pt: PageTable) -> None:
    """Write NaN into every slot no request may read.

    These are the slots past last_page_len in each request's last page and
    every pool page no request references.
    """
    ps = w.page_size
    used = torch.zeros(pool.shape[0], dtype=torch.bool)
    used[torch.from_numpy(pt.indices.astype(np.int64))] = True
    unused = (~used).nonzero().flatten().to(pool.device)
    raw = pool.view(torch.int16) if pool.dtype != torch.uint8 else pool
    nan = NAN_CODE[w.kv_dtype]
    if raw.dtype == torch.int16 and nan >= 0x8000:
        nan -= 0x10000
    if unused.numel():
        raw[unused] = nan
    for i in range(len(pt.last_page_len)):
        last = int(pt.last_page_len[i])
        if last == ps:
            continue
        page = int(pt.indices[int(pt.indptr[i + 1]) - 1])
        if w.layout == "NHD":
            raw[page, :, last:] = nan
        else:
            raw[page, :, :, last:] = nan


@dataclass
class Case:
    w: Workload
    pt: PageTable
    q: torch.Tensor
    pool: torch.Tensor


def make_case(w: Workload, device="cpu", poison: bool = False,
              q_scale: float = 1.0) -> Case:
    rng = np.random.default_rng(w.seed)
    pt = make_page_table(w, rng)
    q = make_q(w, rng, q_scale, device)
    pool = make_pool(w, pt.pool_pages, device)
    if poison:
        poison_unused(w, pool, pt)
    return Case(w, pt, q, pool)


def small_workload(name="small", **kw) -> Workload:
    """A small workload for tests; keyword arguments override fields."""
    base = Workload(name, 7, 3, 8, 2, 64, 16, "f16", "f16", "f16", "NHD",
                    ("uniform", 1, 200))
    return replace(base, **kw)


def raw_numpy(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Host numpy view of stored data: f16 as float16, bf16 as uint16 bits,
    e4m3 as uint8 codes."""
    t = t.detach().cpu().contiguous()
    if dtype == "f16":
        return t.numpy()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    if dtype == "e4m3":
        return t.numpy()
    raise ValueError(dtype)
