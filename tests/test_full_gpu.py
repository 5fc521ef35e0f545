"""GPU tests at the full sizes of the named workloads, in the launch
configuration bench.py times, plus bit-exact gather probes and determinism.

Full-size parity compares o and lse with the oracle on every request of the
batch, and checks a property that pins each request's length: with q = 0
every logit is 0, so lse = ln(#attended tokens), which fixes its length,
page count and window edge to the token (a dropped or doubled token moves o
by only about 1/L, below the o tolerance on long requests)."""
import math

import numpy as np
import pytest
import torch

from paged_kv_decode_09_amd import workloads as wl
from helpers import LSE_TOL, max_abs, o_tol, oracle_all, oracle_for, plan_for, run_gpu

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def attended(w, lengths):
    L = np.asarray(lengths, dtype=np.int64)
    if w.window_left < 0:
        return L
    return np.minimum(L, w.window_left + 1)


@pytest.mark.parametrize("name", ["worked_example", "serving_batch", "long_context",
                                  "gemma2_decode", "fp8_kv"])
def test_full_size_workload(name):
    w = wl.WORKLOADS[name]
    say(name)
    case = wl.make_case(w, device="cuda")
    o, lse, plan = run_gpu(w, case)
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    L = case.pt.lengths
    ref_o, ref_l = oracle_all(w, case)
    eo, el = max_abs(o, ref_o), max_abs(lse, ref_l)
    say(name, "all", w.batch, "requests: o max-abs", eo, "lse max-abs", el,
        "split", plan.info.split_pages, "items", plan.info.num_items)
    assert eo <= o_tol(w) and el <= LSE_TOL
    # q = 0: lse = ln(n) on every request, to within half the gap to n +- 1
    q0 = torch.zeros_like(case.q)
    _, l0 = plan.run(q0, case.pool, k_scale=w.k_scale, v_scale=w.v_scale,
                     return_lse=True)
    torch.cuda.synchronize()
    n = attended(w, L)
    err = np.abs(l0.double().cpu().numpy() - np.log(n)[:, None])
    bound = np.minimum(2e-5, 0.45 / n)[:, None]
    assert np.all(err < bound), float(np.max(err / bound))


def plant_needles(w, case, positions, big):
    """q one-hot (dim 0) times `big` for every head; K[..., 0] = 0 except at
    each request's needle token, where K[..., 0] = the largest stored value."""
    pool = case.pool.clone()
    pt = case.pt
    if w.kv_dtype == "e4m3":
        pool[:, 0, ..., 0] = 0                      # code 0 = +0
        needle = 0x7E                               # 448
    else:
        pool[:, 0, ..., 0] = 0
        needle = None
    for i, j in positions.items():
        page = int(pt.indices[pt.indptr[i] + j // w.page_size])
        slot = j % w.page_size
        if w.layout == "NHD":
            sl = (page, 0, slot, slice(None), 0)
        else:
            sl = (page, 0, slice(None), slot, 0)
        pool[sl] = needle if needle is not None else 8.0
    q = torch.zeros_like(case.q)
    q[..., 0] = big
    return pool, q


def expected_rows(w, case, pool, positions):
    """The stored V rows of the needle tokens, per q head, as o dtype."""
    pt = case.pt
    G = w.num_qo_heads // w.num_kv_heads
    out = {}
    for i, j in positions.items():
        page = int(pt.indices[pt.indptr[i] + j // w.page_size])
        slot = j % w.page_size
        v = pool[page, 1, slot] if w.layout == "NHD" else pool[page, 1, :, slot]
        if w.kv_dtype == "e4m3":
            v = v.view(torch.float8_e4m3fn).float() * w.v_scale
        out[i] = v.float().repeat_interleave(G, dim=0).to(
            wl.TORCH_DTYPES[w.o_dtype])
    return out


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("kv", ["f16", "bf16", "e4m3"])
@pytest.mark.parametrize("page_size", [16, 4])
def test_needle_gather_is_bit_exact(layout, kv, page_size):
    qd = "bf16" if kv == "e4m3" else kv
    lengths = [1, 16, 17, 47, 300, 1000, 2049, 64]
    w = wl.small_workload(seed=41, batch=len(lengths), num_qo_heads=16, num_kv_heads=4,
                          head_dim=128, page_size=page_size, layout=layout,
                          lengths=("fixed", lengths), q_dtype=qd, kv_dtype=kv,
                          o_dtype=qd, k_scale=1 / 64 if kv == "e4m3" else 1.0,
                          v_scale=1 / 64 if kv == "e4m3" else 1.0)
    say(w)
    case = wl.make_case(w, device="cuda")
    rng = np.random.default_rng(3)
    probes = []
    for L in lengths:
        npages = (L + page_size - 1) // page_size
        pages = {0, npages - 1, *rng.integers(0, npages, 6).tolist()}
        cand = {0, L - 1, *rng.integers(0, L, 3).tolist()}
        for p in pages:            # first and last slot of sampled pages
            cand |= {p * page_size, min(L - 1, p * page_size + page_size - 1)}
        probes.append(sorted(cand))
    rounds = max(len(p) for p in probes)
    for split in (None, 3):
        plan = plan_for(w, case, fixed_split_size=split)
        for r in range(rounds):
            pos = {i: p[r % len(p)] for i, p in enumerate(probes)}
            pool, q = plant_needles(w, case, pos, 1000.0)
            o, _ = plan.run(q, pool, k_scale=w.k_scale, v_scale=w.v_scale,
                            return_lse=True)
            torch.cuda.synchronize()
            exp = expected_rows(w, case, pool, pos)
            for i in pos:
                assert torch.equal(o[i], exp[i]), (i, pos[i], split)


@pytest.mark.parametrize("qd", ["bf16", "f16"])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_every_e4m3_code_decodes_exactly(qd, layout):
    """V rows that hold all 254 finite E4M3 codes (the two NaN codes replaced
    by 0), picked by a needle logit, come back as their exact values times
    v_scale in the output dtype: the kernel's fp8 conversion rounds nothing."""
    w = wl.small_workload(seed=45, batch=2, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                          page_size=16, layout=layout, lengths=("fixed", [40, 300]),
                          q_dtype=qd, kv_dtype="e4m3", o_dtype=qd, k_scale=1 / 64,
                          v_scale=1 / 64)
    say(w)
    case = wl.make_case(w, device="cuda")
    codes = torch.arange(256, dtype=torch.int32)
    codes[(codes == 0x7F) | (codes == 0xFF)] = 0
    codes = codes.to(torch.uint8).cuda()
    pos = {0: 17, 1: 250}
    pool, q = plant_needles(w, case, pos, 1000.0)
    pt = case.pt
    for i, j in pos.items():
        page = int(pt.indices[pt.indptr[i] + j // w.page_size])
        slot = j % w.page_size
        row = codes[128 * i:128 * (i + 1)]
        if layout == "NHD":
            pool[page, 1, slot] = row
        else:
            pool[page, 1, :, slot] = row
    for split in (None, 2):
        plan = plan_for(w, case, fixed_split_size=split)
        o = plan.run(q, pool, k_scale=w.k_scale, v_scale=w.v_scale)
        torch.cuda.synchronize()
        exp = expected_rows(w, case, pool, pos)
        for i in pos:
            assert torch.equal(o[i], exp[i]), (i, split)


def test_window_zero_returns_last_row_bit_exactly():
    w = wl.small_workload(seed=43, batch=5, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                          lengths=("fixed", [1, 2, 16, 17, 999]), window_left=0,
                          q_dtype="bf16", kv_dtype="bf16", o_dtype="bf16")
    say(w)
    case = wl.make_case(w, device="cuda")
    o, lse, _ = run_gpu(w, case)
    pos = {i: int(L) - 1 for i, L in enumerate(case.pt.lengths)}
    exp = expected_rows(w, case, case.pool, pos)
    for i in pos:
        assert torch.equal(o[i], exp[i])


@pytest.mark.parametrize("name", ["long_context", "fp8_kv"])
def test_full_size_runs_repeat_bitwise(name):
    """Workgroups that run out of units take long units that others hold in
    reserve, so which workgroup runs a unit changes from run to run (these
    two workloads publish units for that). A unit's arithmetic, and the
    merge order of a split request, do not depend on it: every run gives
    the same bits."""
    w = wl.WORKLOADS[name]
    say(name)
    case = wl.make_case(w, device="cuda")
    first, lfirst, plan = run_gpu(w, case)
    for _ in range(8):
        o, lse, _ = run_gpu(w, case, plan=plan)
        assert torch.equal(o, first) and torch.equal(lse, lfirst)


@pytest.mark.parametrize("name", ["serving_batch", "long_context"])
def test_graph_replays_match_eager_runs(name):
    """pkd_run only enqueues one launch, so a decode step can be captured in a
    HIP graph. Two runs (two queries) are captured; every replay, with eager
    runs, output clears and synchronisations between replays, must give the
    eager bits, which also checks that the counters, reserve slots and merge
    counters the kernel resets for the next launch are left ready."""
    w = wl.WORKLOADS[name]
    say(name, "graph")
    case = wl.make_case(w, device="cuda")
    q2 = torch.flip(case.q, dims=[0]).contiguous()
    plan = plan_for(w, case)
    ws = (torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
          if plan.workspace_bytes else None)
    ref = []
    for q in (case.q, q2):
        o, lse = plan.run(q, case.pool, k_scale=w.k_scale, v_scale=w.v_scale,
                          return_lse=True, workspace=ws)
        ref.append((o.clone(), lse.clone()))
    torch.cuda.synchronize()
    outs = [(torch.empty_like(r[0]), torch.empty_like(r[1])) for r in ref]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for q, (o, lse) in zip((case.q, q2), outs):
            plan.run(q, case.pool, k_scale=w.k_scale, v_scale=w.v_scale,
                     out=o, lse=lse, workspace=ws)
    for rep in range(4):
        for o, lse in outs:
            o.zero_()
            lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for (o, lse), (ro, rl) in zip(outs, ref):
            assert torch.equal(o, ro) and torch.equal(lse, rl), rep
        eo, el = plan.run(q2, case.pool, k_scale=w.k_scale, v_scale=w.v_scale,
                          return_lse=True, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(eo, ref[1][0]) and torch.equal(el, ref[1][1]), rep


def test_fixed_split_is_deterministic_and_batch_invariant():
    w = wl.small_workload(seed=47, batch=5, num_qo_heads=64, num_kv_heads=8, head_dim=128,
                          lengths=("fixed", [5000, 70, 12000, 4096, 1]),
                          fixed_split_size=16)
    say(w)
    case = wl.make_case(w, device="cuda")
    plan = plan_for(w, case)
    first, lfirst = plan.run(case.q, case.pool, return_lse=True)
    for _ in range(10):
        o, l = plan.run(case.q, case.pool, return_lse=True)
        assert torch.equal(o, first) and torch.equal(l, lfirst)
    # each request alone, same pages, same split: bitwise the same
    import paged_kv_decode_09_amd as pkd
    pt = case.pt
    for i in range(w.batch):
        idx = torch.from_numpy(pt.indices[pt.indptr[i]:pt.indptr[i + 1]]).cuda()
        p1 = pkd.PagedDecodePlan([0, len(idx)], idx, pt.last_page_len[i:i + 1],
                                 w.num_qo_heads, w.num_kv_heads, w.head_dim,
                                 w.page_size, kv_layout=w.layout,
                                 fixed_split_size=16)
        o1, l1 = p1.run(case.q[i:i + 1].contiguous(), case.pool, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], first[i]) and torch.equal(l1[0], lfirst[i]), i


def test_empty_batch_runs_nothing():
    import paged_kv_decode_09_amd as pkd
    say("empty batch")
    plan = pkd.PagedDecodePlan([0], torch.zeros(0, dtype=torch.int32, device="cuda"),
                               [], 8, 2, 128, 16)
    q = torch.empty(0, 8, 128, dtype=torch.float16, device="cuda")
    pool = torch.zeros(1, 2, 16, 2, 128, dtype=torch.float16, device="cuda")
    o = plan.run(q, pool)
    torch.cuda.synchronize()
    assert o.shape == (0, 8, 128)


@pytest.mark.parametrize("hd,kv,pos", [(64, "f16", "NONE"), (64, "e4m3", "NONE"),
                                        (128, "bf16", "NONE"), (128, "e4m3", "NONE"),
                                        (256, "bf16", "NONE"), (64, "bf16", "ROPE_LLAMA"),
                                        (128, "bf16", "ROPE_LLAMA"), (128, "e4m3", "ROPE_LLAMA"),
                                        (256, "f16", "ROPE_LLAMA")])
def test_host_planning_matches_the_device_occupancy(hd, kv, pos):
    """pkd_plan_query (no GPU) must plan the same workgroups as
    pkd_plan_create, whose slot count comes from the HIP runtime (with RoPE
    at head_dim 128: two workgroups of the one-buffer kernel per compute
    unit, which their LDS must allow)."""
    import paged_kv_decode_09_amd as pkd
    say("occupancy", hd, kv, pos)
    qd = "bf16" if kv == "e4m3" else kv
    rng = np.random.default_rng(1)
    lens = rng.integers(100, 20000, 300)
    pt = wl.page_table_for(lens, 16, "perm_used", rng)
    kw = dict(num_qo_heads=32, num_kv_heads=8, head_dim=hd, page_size=16,
              q_data_type=qd, kv_data_type=kv, pos_encoding_mode=pos)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    info, items = pkd.plan_query(pt.indptr, pt.last_page_len, cus, **kw)
    plan = pkd.PagedDecodePlan(pt.indptr, torch.from_numpy(pt.indices).cuda(),
                               pt.last_page_len, **kw)
    assert plan.info.workgroups_per_cu == info.workgroups_per_cu
    assert plan.info.num_workgroups == info.num_workgroups
    assert plan.info.num_items == info.num_items


def test_many_runs_merge_matches_the_oracle_and_repeats():
    """A 60000-token request under a one-page fixed split has 3750 units
    per kv head: 469 runs of 8, whose final fold takes 30 batches (the
    running-maximum rescale between batches). Checked against the oracle,
    and bitwise against a second run of the same plan (the merge counters
    must be back to zero after a launch)."""
    from dataclasses import replace
    w = replace(wl.WORKLOADS["long_context"], name="many_runs", seed=11, batch=2,
                lengths=("fixed", [60000, 3001]), fixed_split_size=1)
    case = wl.make_case(w, device="cuda")
    o, lse, plan = run_gpu(w, case)
    say("many_runs units", plan.info.num_items, "partials", plan.info.num_partials)
    assert plan.info.num_items == (3750 + 188) * w.num_kv_heads
    ref_o, ref_l = oracle_for(w, case)
    eo, el = max_abs(o, ref_o), max_abs(lse, ref_l)
    say("many_runs o max-abs", eo, "lse max-abs", el)
    assert eo <= o_tol(w) and el <= LSE_TOL
    o2, lse2, _ = run_gpu(w, case, plan=plan)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
