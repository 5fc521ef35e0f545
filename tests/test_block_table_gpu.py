"""GPU tests of the block-table page input (pkd_plan_create_block_table):
request i owns pages block_tables[i][0 .. ceil(L_i / P)), as the page_table /
seq_lens input of the XQA decode on the API page. Every test prints its case
before it touches the GPU."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_09_amd as pkd
from paged_kv_decode_09_amd import workloads as wl
from helpers import LSE_TOL, max_abs, o_tol, plan_for, run_gpu

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def block_table_of(case, max_blocks, filler):
    """The case's CSR page table as a block table; entries past a request's
    pages hold `filler` (a page no request owns)."""
    pt = case.pt
    B = len(pt.last_page_len)
    table = np.full((B, max_blocks), filler, dtype=np.int32)
    for i in range(B):
        pg = pt.indices[pt.indptr[i]:pt.indptr[i + 1]]
        table[i, :len(pg)] = pg
    return torch.from_numpy(table).cuda()


@pytest.mark.parametrize("layout,Q,split", [("NHD", 1, None), ("HND", 1, 2),
                                            ("NHD", 2, None), ("HND", 3, 1)])
def test_block_table_plan_gives_the_csr_bits(layout, Q, split):
    # one spare pool page, filled with NaN, fills the unused entries of every
    # row: a read past a request's pages would show up as NaN
    w = wl.small_workload(seed=67, batch=6, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                          layout=layout, q_len_per_req=Q, pages="perm_pool",
                          lengths=("fixed", [Q, 17, 100, 333, 900, 64]), pool_pages=200)
    say(w, "split", split)
    case = wl.make_case(w, device="cuda", poison=True)
    used = set(case.pt.indices.tolist())
    spare = next(p for p in range(w.pool_pages) if p not in used)
    o1, l1, _ = run_gpu(w, case, fixed_split_size=split)
    table = block_table_of(case, 64, spare)
    plan = pkd.PagedDecodePlan(
        None, None, None, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
        kv_layout=layout, q_data_type=w.q_dtype, fixed_split_size=split,
        q_len_per_req=Q, seq_lens=case.pt.lengths.astype(np.int32), block_tables=table)
    o2, l2 = plan.run(case.q, case.pool, return_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(o2).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_block_table_wrapper_matches_oracle():
    w = wl.small_workload(seed=71, batch=4, num_qo_heads=16, num_kv_heads=4, head_dim=256,
                          q_dtype="bf16", kv_dtype="bf16", o_dtype="bf16",
                          lengths=("fixed", [1, 40, 513, 1200]), pages="perm_pool",
                          pool_pages=150)
    say(w)
    case = wl.make_case(w, device="cuda")
    table = block_table_of(case, 80, 0)
    wrapper = pkd.BatchDecodeWithPagedKVCacheWrapper(
        torch.empty(1 << 20, dtype=torch.uint8, device="cuda"), kv_layout=w.layout)
    wrapper.plan(None, None, None, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                 w.page_size, q_data_type=torch.bfloat16,
                 seq_lens=torch.from_numpy(case.pt.lengths.astype(np.int32)),
                 block_tables=table)
    o, lse = wrapper.run(case.q, case.pool, return_lse=True)
    torch.cuda.synchronize()
    indptr, indices, last = oracle.csr_from_block_table(case.pt.lengths,
                                                        table.cpu().numpy(), w.page_size)
    ref_o, ref_l = oracle.batch_decode(
        wl.raw_numpy(case.q, w.q_dtype), wl.raw_numpy(case.pool, w.kv_dtype), w.layout,
        indptr, indices, last, w.page_size, w.q_dtype, w.kv_dtype, w.sm_scale)
    assert max_abs(o, ref_o) <= o_tol(w) and max_abs(lse, ref_l) <= LSE_TOL
