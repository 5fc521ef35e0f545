"""GPU parity of the one-buffer decode kernel (RoPE at head_dim 128, or 256
with 16-bit K/V, under the planner's own split) where its code differs from
the two-buffer kernel's: units that span several LDS windows of page ids
(512 pages each at head_dim 128) and units long enough to be published for
stealing, so that a workgroup may find the unit it holds taken by another.
Outputs against the fp64 oracle within the derived RoPE bounds, and two runs
bit for bit (a unit's arithmetic does not depend on which workgroup runs
it). Every test prints its case before it touches the GPU."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_09_amd import workloads as wl
from helpers import plan_for, rope_lse_bounds, rope_o_bounds, sub_pool

pytestmark = pytest.mark.gpu

STEAL_MIN_BYTES = 512 << 10   # units of at least this many K/V bytes are published


def say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("hd,kv,page,lengths,per_cu", [
    # one token per page: units of about 1280 pages span three windows of page
    # ids, and hold about 640 KB of K/V, so they are published too
    (128, "bf16", 1, [260000, 290000], 2),
    # head_dim 256 (one workgroup per compute unit): units of about 770 KB
    (256, "f16", 16, [70000, 80000], 1),
])
def test_one_buffer_long_units(hd, kv, page, lengths, per_cu):
    w = wl.small_workload(seed=151, batch=len(lengths), num_qo_heads=16, num_kv_heads=1,
                          head_dim=hd, page_size=page, q_dtype=kv, kv_dtype=kv, o_dtype=kv,
                          pos_encoding_mode="ROPE_LLAMA", lengths=("fixed", lengths))
    say(w)
    case = wl.make_case(w, device="cuda")
    plan = plan_for(w, case, pos_encoding_mode="ROPE_LLAMA", rope_theta=w.rope_theta,
                    rope_scale=w.rope_scale)
    # the one-buffer kernel runs, with units as described above
    assert plan.info.workgroups_per_cu == per_cu
    unit_tokens = plan.info.attended_tokens * w.num_kv_heads / plan.info.num_items
    unit_bytes = unit_tokens * 2 * hd * 2
    say("items", plan.info.num_items, "tokens per unit", round(unit_tokens),
        "KB per unit", round(unit_bytes / 1024))
    assert unit_bytes >= STEAL_MIN_BYTES
    if hd == 128:
        assert unit_tokens / page > 512
    o1, l1 = plan.run(case.q, case.pool, return_lse=True)
    o2, l2 = plan.run(case.q, case.pool, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    reqs = list(range(w.batch))
    pool, indptr, indices, last = sub_pool(case, reqs)
    ref_o, ref_l = oracle.batch_decode_multi(
        wl.raw_numpy(case.q, w.q_dtype), wl.raw_numpy(pool, w.kv_dtype), w.layout, indptr,
        indices, last, w.page_size, 1, w.q_dtype, w.kv_dtype, w.sm_scale,
        rope=(w.rope_theta, w.rope_scale))
    assert not torch.isnan(o1).any()
    el = np.abs(l1.double().cpu().numpy() - ref_l)
    bl = rope_lse_bounds(w, case, reqs, w.rope_theta, w.rope_scale)
    eo = np.abs(o1.double().cpu().numpy() - ref_o)
    bo = rope_o_bounds(w, case, reqs, w.rope_theta, w.rope_scale, ref_o)
    say("lse worst err/bound", float(np.max(el / bl)), "o worst err/bound", float(np.max(eo / bo)))
    assert np.all(el <= bl), float(np.max(el / bl))
    assert np.all(eo <= bo), float(np.max(eo / bo))
