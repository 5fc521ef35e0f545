"""GPU parity at the edges of the method, through the C-ABI, against the fp64
oracle on every request: many tiny requests (a long work queue), logits in
the hundreds (a nearly one-hot softmax, and split states whose lse differ by
hundreds), a soft cap driven into saturation, window edges around the
sequence length, one request long enough to need several LDS page windows
without a split, page size 1 over a long sequence, and calibration scales on
16-bit K/V. Every test prints its case before it touches the GPU."""
import numpy as np
import pytest
import torch

from paged_kv_decode_09_amd import workloads as wl
from helpers import LSE_TOL, max_abs, o_bounds, o_tol, oracle_all, plan_for, run_gpu

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def check_all(w, case, o, lse, lse_bound=LSE_TOL, q=None):
    """o within o_bounds (the max-abs tolerance, widened to half an ulp of
    the output dtype where |o| is too large for it), lse within LSE_TOL."""
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    ref_o, ref_l = oracle_all(w, case, q=q)
    err = np.abs(o.float().cpu().double().numpy() - ref_o)
    bound = o_bounds(w, ref_o)
    el = max_abs(lse, ref_l)
    say("o max-abs", float(err.max()), "worst o err/bound", float(np.max(err / bound)),
        "lse max-abs", el)
    assert np.all(err <= bound), float(np.max(err / bound))
    assert el <= lse_bound, el


def test_many_tiny_requests():
    """4096 requests of 1-64 tokens (many of them one page, some one token):
    32768 units through the work counter, most workgroups running dozens."""
    w = wl.small_workload(seed=201, batch=4096, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                          layout="HND", q_dtype="bf16", kv_dtype="bf16", o_dtype="bf16",
                          lengths=("uniform", 1, 64))
    say(w.name, "batch", w.batch)
    case = wl.make_case(w, device="cuda", poison=True)
    o, lse, plan = run_gpu(w, case)
    say("units", plan.info.num_items)
    assert plan.info.num_items == 4096 * 8
    check_all(w, case, o, lse)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("split", [None, 2])
def test_logits_in_the_hundreds(dt, split):
    """q scaled by 30: logits of standard deviation 30 (extremes near 150), so
    each softmax is nearly one-hot and split states' lse differ by far more
    than the exponent range of a single rescale."""
    w = wl.small_workload(seed=203, batch=6, num_qo_heads=16, num_kv_heads=4, head_dim=128,
                          q_dtype=dt, kv_dtype=dt, o_dtype=dt,
                          lengths=("fixed", [1, 17, 300, 2000, 5000, 777]))
    say(w, "q x30", "split", split)
    case = wl.make_case(w, device="cuda", q_scale=30.0)
    o, lse, _ = run_gpu(w, case, fixed_split_size=split)
    check_all(w, case, o, lse)


def test_soft_cap_saturates():
    """cap 5 with logits near +-150: every capped logit sits within a hair
    of +-5, so the softmax is nearly flat over the tokens the cap clips."""
    w = wl.small_workload(seed=205, batch=4, num_qo_heads=16, num_kv_heads=8, head_dim=256,
                          q_dtype="bf16", kv_dtype="bf16", o_dtype="bf16", logits_soft_cap=5.0,
                          lengths=("fixed", [3, 100, 1000, 4000]))
    say(w, "q x30")
    case = wl.make_case(w, device="cuda", q_scale=30.0)
    o, lse, _ = run_gpu(w, case)
    check_all(w, case, o, lse)


def test_window_edges_around_the_length():
    """One window (500) and lengths around it: shorter than the window, equal
    to it, one past it (the window covers exactly the whole request), and
    two, three and seventeen past it (the window starts at token 1, 2, 16)."""
    window = 500
    lengths = [window - 5, window, window + 1, window + 2, window + 3, window + 17, 1]
    w = wl.small_workload(seed=207, batch=len(lengths), num_qo_heads=8, num_kv_heads=2,
                          head_dim=128, window_left=window, lengths=("fixed", lengths))
    say(w)
    case = wl.make_case(w, device="cuda", poison=True)
    for split in (None, 3):
        o, lse, _ = run_gpu(w, case, fixed_split_size=split)
        check_all(w, case, o, lse)


def test_one_long_request_without_split():
    """100 000 tokens in one unit per kv head (disable_split_kv): 6250 pages,
    taken through seven windows of page ids in LDS."""
    w = wl.small_workload(seed=209, batch=1, num_qo_heads=16, num_kv_heads=2, head_dim=128,
                          q_dtype="bf16", kv_dtype="bf16", o_dtype="bf16",
                          lengths=("fixed", [100000]))
    say(w)
    case = wl.make_case(w, device="cuda")
    o, lse, plan = run_gpu(w, case, disable_split_kv=True)
    assert plan.info.num_items == 2 and plan.info.num_partials == 0
    check_all(w, case, o, lse)


def test_page_size_one_long_sequence():
    """One token per page over 20 000 tokens (a new LDS page window every
    1023 tokens), in both layouts, split and unsplit."""
    for layout in ("NHD", "HND"):
        w = wl.small_workload(seed=211, batch=3, num_qo_heads=8, num_kv_heads=4, head_dim=64,
                              page_size=1, layout=layout, lengths=("fixed", [20000, 1, 4097]))
        say(w)
        case = wl.make_case(w, device="cuda", poison=True)
        for split in (None, 1000):
            o, lse, _ = run_gpu(w, case, fixed_split_size=split)
            check_all(w, case, o, lse)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_scales_on_16_bit_kv(dt):
    """q_scale, k_scale and v_scale are plain multipliers for 16-bit K/V too
    (the run gets q_scale 1.5; the workload carries k_scale 0.5, v_scale 3)."""
    import oracle
    from helpers import sub_pool
    w = wl.small_workload(seed=213, batch=4, num_qo_heads=16, num_kv_heads=4, head_dim=128,
                          q_dtype=dt, kv_dtype=dt, o_dtype=dt, k_scale=0.5, v_scale=3.0,
                          lengths=("fixed", [1, 64, 1000, 3000]))
    say(w, "q_scale 1.5")
    case = wl.make_case(w, device="cuda")
    plan = plan_for(w, case)
    o, lse = plan.run(case.q, case.pool, q_scale=1.5, k_scale=w.k_scale, v_scale=w.v_scale,
                      return_lse=True)
    torch.cuda.synchronize()
    pool, indptr, indices, last = sub_pool(case, range(w.batch))
    args = (wl.raw_numpy(case.q, w.q_dtype), wl.raw_numpy(pool, w.kv_dtype), w.layout, indptr,
            indices, last, w.page_size, w.q_dtype, w.kv_dtype, w.sm_scale)
    ref_o, ref_l = oracle.batch_decode(*args, q_scale=1.5, k_scale=w.k_scale, v_scale=w.v_scale)
    err = np.abs(o.float().cpu().double().numpy() - ref_o)
    el = max_abs(lse, ref_l)
    # o is v_scale times a convex combination of stored rows: the arithmetic
    # part of its error scales with v_scale, the output rounding with |o|
    bound = np.maximum(w.v_scale * o_tol(w), o_bounds(w, ref_o))
    say("o max-abs", float(err.max()), "worst o err/bound", float(np.max(err / bound)),
        "lse max-abs", el)
    assert np.all(err <= bound) and el <= LSE_TOL
    # the scales are applied: without q_scale the oracle is far off
    un_o, _ = oracle.batch_decode(*args, k_scale=w.k_scale, v_scale=w.v_scale)
    assert max_abs(o, un_o) > 10 * o_tol(w)
