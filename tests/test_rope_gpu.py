"""GPU parity of the Llama-style rotary embedding (plan()'s pos_encoding_mode
"ROPE_LLAMA", rope_scale, rope_theta) against the fp64 oracle, through the
C-ABI: q turned at its query position and every key at its token index,
inside the kernel. Every test prints its case before it touches the GPU."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_09_amd import workloads as wl
from helpers import (max_abs, o_tol, oracle_all, plan_for, rope_lse_bounds, rope_o_bounds,
                     run_gpu, sub_pool)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def check_rope(w, case, theta, scale, split, reqs=None):
    plan = plan_for(w, case, fixed_split_size=split, pos_encoding_mode="ROPE_LLAMA",
                    rope_theta=theta, rope_scale=scale)
    o, lse = plan.run(case.q, case.pool, k_scale=w.k_scale, v_scale=w.v_scale,
                      return_lse=True)
    torch.cuda.synchronize()
    reqs = list(range(w.batch)) if reqs is None else reqs
    Q = w.q_len_per_req
    rows = [i * Q + j for i in reqs for j in range(Q)]
    pool, indptr, indices, last = sub_pool(case, reqs)
    ref_o, ref_l = oracle.batch_decode_multi(
        wl.raw_numpy(case.q[torch.tensor(rows)], w.q_dtype), wl.raw_numpy(pool, w.kv_dtype),
        w.layout, indptr, indices, last, w.page_size, Q, w.q_dtype, w.kv_dtype, w.sm_scale,
        logits_soft_cap=w.logits_soft_cap, window_left=w.window_left, k_scale=w.k_scale,
        v_scale=w.v_scale, rope=(theta, scale))
    idx = torch.tensor(rows)
    assert not torch.isnan(o).any()
    check_rope_lse(w, case, reqs, lse[idx], ref_l, theta, scale)
    check_rope_o(w, case, reqs, o[idx], ref_o, theta, scale)


def check_rope_o(w, case, reqs, o_gpu, ref_o, theta, scale):
    """Every element of o within its derived bound (helpers.rope_o_bounds:
    the plain bound plus six standard deviations of the error that rounding
    the rotated operands and P to the q dtype adds)."""
    err = np.abs(o_gpu.double().cpu().numpy() - ref_o)
    bound = rope_o_bounds(w, case, reqs, theta, scale, ref_o)
    say("o max-abs", float(err.max()), "worst err/bound", float(np.max(err / bound)))
    assert np.all(err <= bound), float(np.max(err / bound))


def check_rope_lse(w, case, reqs, lse_gpu, ref_l, theta, scale):
    """Every row's lse error within its own derived bound (helpers.
    rope_lse_bounds: the plain tolerance plus six standard deviations of
    the error that rounding the rotated operands to the q dtype adds)."""
    err = np.abs(lse_gpu.double().cpu().numpy() - ref_l)
    bound = rope_lse_bounds(w, case, reqs, theta, scale)
    say("lse max-abs", float(err.max()), "worst err/bound", float(np.max(err / bound)),
        "bounds", float(bound.min()), "..", float(bound.max()))
    assert np.all(err <= bound), float(np.max(err / bound))


@pytest.mark.parametrize("hd,kv,Q,cap,window,layout", [
    (128, "bf16", 1, 0.0, -1, "NHD"), (128, "f16", 3, 0.0, -1, "HND"),
    (64, "f16", 1, 0.0, 40, "HND"), (256, "bf16", 1, 30.0, -1, "NHD"),
    (128, "e4m3", 2, 0.0, -1, "NHD"), (256, "e4m3", 1, 0.0, 100, "HND"),
    (64, "e4m3", 1, 0.0, -1, "NHD"), (64, "e4m3", 2, 30.0, 50, "HND")])
@pytest.mark.parametrize("theta,scale", [(1e4, 1.0), (5e5, 8.0)])
@pytest.mark.parametrize("split", [None, 3])
def test_rope_matches_oracle(hd, kv, Q, cap, window, layout, theta, scale, split):
    qd = "bf16" if kv == "e4m3" else kv
    w = wl.small_workload(seed=97, batch=5, num_qo_heads=8, num_kv_heads=2, head_dim=hd,
                          q_dtype=qd, kv_dtype=kv, o_dtype=qd, q_len_per_req=Q,
                          layout=layout, logits_soft_cap=cap, window_left=window,
                          k_scale=1 / 64 if kv == "e4m3" else 1.0,
                          v_scale=1 / 64 if kv == "e4m3" else 1.0,
                          lengths=("fixed", [Q, 33, 200, 900, 1700]))
    say(w, "theta", theta, "scale", scale, "split", split)
    case = wl.make_case(w, device="cuda")
    check_rope(w, case, theta, scale, split)


@pytest.mark.parametrize("kv", ["f16", "bf16"])
def test_rope_at_long_positions(kv):
    """Angles of positions up to 1.3e5 tokens: the split of the frequency into
    two floats keeps the angle exact enough for the o tolerance."""
    w = wl.small_workload(seed=101, batch=2, num_qo_heads=8, num_kv_heads=1, head_dim=128,
                          q_dtype=kv, kv_dtype=kv, o_dtype=kv,
                          lengths=("fixed", [70001, 131000]))
    say(w)
    case = wl.make_case(w, device="cuda")
    check_rope(w, case, 1e4, 1.0, 64)


def test_serving_rope_full_size():
    """The serving batch with RoPE at full size, in the launch configuration
    of the bench, against the oracle on every request."""
    w = wl.WORKLOADS["serving_rope"]
    say(w.name)
    case = wl.make_case(w, device="cuda")
    o, lse, plan = run_gpu(w, case)
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    ref_o, ref_l = oracle_all(w, case)
    eo = max_abs(o, ref_o)
    say(w.name, "all", w.batch, "requests: o max-abs", eo, "items", plan.info.num_items)
    assert eo <= o_tol(w)
    check_rope_lse(w, case, range(w.batch), lse, ref_l, w.rope_theta, w.rope_scale)
