"""Runs of one plan on two streams (GPU). The workgroups of a run share the
plan's work counters, so a run on a second stream while the first is still
in flight must be refused (PKD_EBUSY), and accepted once it has finished.
Every test prints its case before it touches the GPU."""
import pytest
import torch

import paged_kv_decode_09_amd as pkd
from paged_kv_decode_09_amd import workloads as wl
from helpers import plan_for

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def keep_busy(stream):
    """Several milliseconds of matrix products queued on `stream`."""
    with torch.cuda.stream(stream):
        a = torch.randn(4096, 4096, device="cuda")
        for _ in range(8):
            a = (a @ a) * (1.0 / 64)
    return a


def test_run_on_a_second_stream_while_the_first_is_in_flight_is_refused():
    w = wl.small_workload(seed=71, batch=6, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                          lengths=("fixed", [3000, 17, 900, 4096, 1, 2500]))
    say(w)
    case = wl.make_case(w, device="cuda")
    plan = plan_for(w, case)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
    ref = plan.run(case.q, case.pool, workspace=ws)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    busy = keep_busy(s1)
    o1 = torch.empty_like(ref)
    plan.run(case.q, case.pool, out=o1, workspace=ws, stream=s1)   # queued behind it
    with pytest.raises(pkd.PkdError) as e:
        plan.run(case.q, case.pool, workspace=ws, stream=s2)
    assert e.value.status == pkd.PKD_EBUSY
    # the same stream again is ordered after the first run: accepted
    o1b = torch.empty_like(ref)
    plan.run(case.q, case.pool, out=o1b, workspace=ws, stream=s1)
    s1.synchronize()
    o2 = torch.empty_like(ref)
    plan.run(case.q, case.pool, out=o2, workspace=ws, stream=s2)
    s2.synchronize()
    assert torch.equal(o1, ref) and torch.equal(o1b, ref) and torch.equal(o2, ref)
    del busy


def test_temporaries_of_a_run_on_a_side_stream_stay_valid():
    """out, lse and the workspace allocated by the binding for a run on a
    side stream are not handed to new tensors before that run is done."""
    w = wl.small_workload(seed=73, batch=4, num_qo_heads=16, num_kv_heads=4, head_dim=128,
                          lengths=("fixed", [5000, 4000, 3000, 100]))
    say(w)
    case = wl.make_case(w, device="cuda")
    plan = plan_for(w, case)
    ref, rl = plan.run(case.q, case.pool, return_lse=True)
    torch.cuda.synchronize()
    s1 = torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    busy = keep_busy(s1)
    o, lse = plan.run(case.q, case.pool, return_lse=True, stream=s1)   # workspace allocated here
    # allocations on the current stream while the run waits on s1
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
    s1.synchronize()
    assert torch.equal(o, ref) and torch.equal(lse, rl)
    del busy, junk
