"""GPU parity of groups of more than 16 query rows per kv head (G * Q > 16:
multi-query models, large GQA groups, several query tokens with a large
group) against the fp64 oracle, through the C-ABI.

The pages ask only that num_qo_heads be a multiple of num_kv_heads. A unit
carries at most 16 query rows (one MFMA tile), so the planner splits each kv
head's q heads into the fewest equal blocks that fit and runs every block as
a head of its own over that kv head's K/V; the tests check every q head's
output and lse against the oracle, with ALiBi slopes and sinks (which are
per q head) and RoPE. Every test prints its case before it touches the GPU."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_09_amd import workloads as wl
from helpers import (LSE_TOL, max_abs, o_tol, oracle_for, plan_for, rope_lse_bounds,
                     rope_o_bounds, run_gpu, sub_pool)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


# (num_qo_heads, num_kv_heads, Q, head_dim, dtype): blocks per kv head in the id
GRID = [
    (32, 1, 1, 128, "bf16"),     # 2 blocks of 16
    (64, 2, 1, 128, "f16"),      # 2 blocks of 16
    (48, 1, 1, 64, "bf16"),      # 3 blocks of 16
    (34, 2, 1, 128, "bf16"),     # G = 17: 17 blocks of 1
    (16, 1, 4, 128, "bf16"),     # 4 blocks of 4 heads x 4 tokens
    (8, 1, 4, 256, "f16"),       # 2 blocks of 4 heads x 4 tokens
    (32, 1, 1, 128, "e4m3"),     # E4M3 K/V
]


@pytest.mark.parametrize("cfg", GRID, ids=lambda c: "nq{}-nkv{}-q{}-hd{}-{}".format(*c))
@pytest.mark.parametrize("split", [None, 2])
def test_large_group_matches_oracle(cfg, split):
    nq, nkv, Q, hd, kv = cfg
    qd = "bf16" if kv == "e4m3" else kv
    w = wl.small_workload(seed=131, batch=4, num_qo_heads=nq, num_kv_heads=nkv, head_dim=hd,
                          q_dtype=qd, kv_dtype=kv, o_dtype=qd, q_len_per_req=Q,
                          k_scale=1 / 64 if kv == "e4m3" else 1.0,
                          v_scale=1 / 64 if kv == "e4m3" else 1.0,
                          lengths=("fixed", [Q, 45, 300, 1200]))
    say(w, "split", split)
    case = wl.make_case(w, device="cuda")
    o, lse, plan = run_gpu(w, case, fixed_split_size=split)
    assert tuple(o.shape) == (4 * Q, nq, hd)
    ref_o, ref_l = oracle_for(w, case)
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    eo, el = max_abs(o, ref_o), max_abs(lse, ref_l)
    say("items", plan.info.num_items, "o max-abs", eo, "lse max-abs", el)
    assert eo <= o_tol(w), eo
    assert el <= LSE_TOL, el


@pytest.mark.parametrize("split", [None, 3])
def test_large_group_alibi_and_sinks(split):
    """ALiBi's slope and the sink are per q head: a block's heads must get
    their own (the oracle takes both per q head)."""
    w = wl.small_workload(seed=137, batch=3, num_qo_heads=40, num_kv_heads=2, head_dim=128,
                          q_dtype="bf16", kv_dtype="bf16", o_dtype="bf16",
                          pos_encoding_mode="ALIBI", lengths=("fixed", [7, 260, 900]))
    say(w, "split", split)
    case = wl.make_case(w, device="cuda")
    rng = np.random.default_rng(5)
    sinks = rng.uniform(-3.0, 6.0, w.num_qo_heads).astype(np.float32)
    plan = plan_for(w, case, fixed_split_size=split)
    o, lse = plan.run(case.q, case.pool, k_scale=1.0, v_scale=1.0, return_lse=True,
                      sinks=torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    reqs = list(range(w.batch))
    pool, indptr, indices, last = sub_pool(case, reqs)
    ref_o, ref_l = oracle.batch_decode_multi(
        wl.raw_numpy(case.q, w.q_dtype), wl.raw_numpy(pool, w.kv_dtype), w.layout, indptr,
        indices, last, w.page_size, 1, w.q_dtype, w.kv_dtype, w.sm_scale,
        alibi=True, sinks=sinks.astype(np.float64))
    eo, el = max_abs(o, ref_o), max_abs(lse, ref_l)
    say("items", plan.info.num_items, "o max-abs", eo, "lse max-abs", el)
    assert eo <= o_tol(w), eo
    assert el <= LSE_TOL, el


def test_large_group_rope():
    """RoPE with 32 q heads on one kv head: every block turns its own q and
    the shared keys; the lse of each row within its derived bound."""
    w = wl.small_workload(seed=139, batch=3, num_qo_heads=32, num_kv_heads=1, head_dim=128,
                          q_dtype="bf16", kv_dtype="bf16", o_dtype="bf16",
                          pos_encoding_mode="ROPE_LLAMA", lengths=("fixed", [1, 500, 2100]))
    say(w)
    case = wl.make_case(w, device="cuda")
    o, lse, plan = run_gpu(w, case)
    ref_o, ref_l = oracle_for(w, case)
    eo = np.abs(o.double().cpu().numpy() - ref_o)
    bo = rope_o_bounds(w, case, range(w.batch), w.rope_theta, w.rope_scale, ref_o)
    err = np.abs(lse.double().cpu().numpy() - ref_l)
    bound = rope_lse_bounds(w, case, range(w.batch), w.rope_theta, w.rope_scale)
    say("items", plan.info.num_items, "worst o err/bound", float(np.max(eo / bo)),
        "worst lse err/bound", float(np.max(err / bound)))
    assert np.all(eo <= bo), float(np.max(eo / bo))
    assert np.all(err <= bound), float(np.max(err / bound))
