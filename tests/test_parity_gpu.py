"""GPU parity: the HIP path through the C-ABI against the fp64 oracle.

Every test prints the case it runs before touching the GPU, so that a failing
run names its case."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_09_amd as pkd
from paged_kv_decode_09_amd import workloads as wl
from helpers import (LSE_TOL, max_abs, o_tol, oracle_for, plan_for, run_gpu)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def check(w, case, o, lse, requests=None, split_pages=None, q=None):
    ref_o, ref_l = oracle_for(w, case, requests, split_pages, q)
    idx = slice(None) if requests is None else torch.tensor(list(requests))
    eo = max_abs(o[idx], ref_o)
    el = max_abs(lse[idx], ref_l)
    assert not torch.isnan(o).any()
    assert eo <= o_tol(w), f"o max-abs {eo} > {o_tol(w)}"
    assert el <= LSE_TOL, f"lse max-abs {el} > {LSE_TOL}"
    return eo, el


def test_worked_example_matches_oracle():
    w = wl.WORKLOADS["worked_example"]
    say(w.name)
    case = wl.make_case(w, device="cuda")
    o, lse, _ = run_gpu(w, case)
    assert tuple(o.shape) == (7, 64, 128) and o.dtype == torch.float16
    check(w, case, o, lse)


SMALL = []
for hd in (64, 128, 256):
    for group in (1, 2, 4, 8, 16):
        SMALL.append(dict(head_dim=hd, num_qo_heads=2 * group, num_kv_heads=2))
GRID = []
for i, shape in enumerate(SMALL):
    layout = "NHD" if i % 2 else "HND"
    dt = ["f16", "bf16"][i % 2 if i < 8 else (i // 2) % 2]
    ps = [16, 1, 4, 64, 16, 2][i % 6]
    GRID.append(dict(shape, layout=layout, q_dtype=dt, kv_dtype=dt, o_dtype=dt,
                     page_size=ps))


@pytest.mark.parametrize("cfg", GRID, ids=lambda c: "hd{head_dim}-g{g}-{layout}-{q_dtype}-p{page_size}".format(g=c["num_qo_heads"] // c["num_kv_heads"], **c))
@pytest.mark.parametrize("split", [None, 1, 3])
def test_small_grid(cfg, split):
    w = wl.small_workload(seed=17, batch=5, lengths=("fixed", [1, 17, 100, 333, 64]),
                          **cfg)
    say(w, "split", split)
    case = wl.make_case(w, device="cuda")
    o, lse, plan = run_gpu(w, case, fixed_split_size=split)
    check(w, case, o, lse)


@pytest.mark.parametrize("cap,window", [(50.0, -1), (0.0, 0), (0.0, 37), (5.0, 100), (30.0, 4096)])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_soft_cap_and_window(cap, window, dt):
    w = wl.small_workload(seed=23, batch=6, num_qo_heads=16, num_kv_heads=8, head_dim=256,
                          lengths=("fixed", [1, 5, 31, 130, 700, 1500]), q_dtype=dt,
                          kv_dtype=dt, o_dtype=dt, logits_soft_cap=cap, window_left=window)
    say(w)
    # q scaled up so that the cap saturates a good share of the logits
    case = wl.make_case(w, device="cuda", q_scale=8.0 if cap else 1.0)
    for split in (None, 2):
        o, lse, _ = run_gpu(w, case, fixed_split_size=split)
        check(w, case, o, lse)


@pytest.mark.parametrize("qdt", ["bf16", "f16"])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_fp8_kv(qdt, layout):
    w = wl.small_workload(seed=29, batch=4, num_qo_heads=64, num_kv_heads=8, head_dim=128,
                          lengths=("fixed", [1, 40, 513, 2000]), q_dtype=qdt,
                          kv_dtype="e4m3", o_dtype=qdt, layout=layout,
                          k_scale=1.0 / 64, v_scale=1.0 / 64)
    say(w)
    case = wl.make_case(w, device="cuda")
    for split in (None, 4):
        o, lse, _ = run_gpu(w, case, fixed_split_size=split)
        check(w, case, o, lse)


def test_tuple_cache_form_equals_5d():
    w = wl.small_workload(seed=31, batch=3, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                          lengths=("fixed", [70, 5, 300]))
    say(w)
    case = wl.make_case(w, device="cuda")
    o5, l5, plan = run_gpu(w, case)
    k = case.pool[:, 0].contiguous()
    v = case.pool[:, 1].contiguous()
    o2, l2 = plan.run(case.q, (k, v), return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o5, o2) and torch.equal(l5, l2)
    # strided views of the 5-D cache are accepted as they are
    o3, l3 = plan.run(case.q, (case.pool[:, 0], case.pool[:, 1]), return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o5, o3)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_merge_states_matches_oracle(out_dtype):
    say("merge_states", out_dtype)
    g = torch.Generator().manual_seed(5)
    rows, n, hd = 37, 9, 96
    v = torch.randn(rows, n, hd, generator=g)
    s = torch.randn(rows, n, generator=g) * 3
    s[3, :] = -math.inf          # all empty
    s[4, 2] = -math.inf          # one empty state
    vo, so = pkd.merge_states(v.cuda(), s.cuda(), out_dtype)
    torch.cuda.synchronize()
    ref_v, ref_s = oracle.merge_states(v.double().numpy(), s.double().numpy())
    tol = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 1e-2}[out_dtype]
    assert np.max(np.abs(vo.float().cpu().double().numpy() - ref_v)) < tol
    fin = np.isfinite(ref_s)
    sc = so.cpu().double().numpy()
    assert np.all(np.abs(sc[fin] - ref_s[fin]) < 1e-5)
    assert np.all(np.isneginf(sc[~fin]))
    assert torch.all(vo[3] == 0)


@pytest.mark.parametrize("kv", ["f16", "bf16", "e4m3"])
def test_poisoned_slots_do_not_leak(kv):
    qd = "bf16" if kv == "e4m3" else kv
    w = wl.small_workload(seed=37, batch=6, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                          lengths=("uniform", 1, 900), pool_pages=400, pages="perm_pool",
                          q_dtype=qd, kv_dtype=kv, o_dtype=qd,
                          k_scale=1 / 64 if kv == "e4m3" else 1.0,
                          v_scale=1 / 64 if kv == "e4m3" else 1.0)
    say(w)
    clean = wl.make_case(w, device="cuda")
    dirty = wl.make_case(w, device="cuda", poison=True)
    for split in (None, 2):
        o1, l1, _ = run_gpu(w, clean, fixed_split_size=split)
        o2, l2, _ = run_gpu(w, dirty, fixed_split_size=split)
        assert not torch.isnan(o2).any() and not torch.isnan(l2).any()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
