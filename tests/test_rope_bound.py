"""The per-row lse bound that the ROPE_LLAMA GPU tests use (helpers.
rope_lse_bounds) against a brute-force simulation of what it models: the
rotated q and keys rounded to nearest even in the operand type, then an
exact fp64 lse. The simulated errors must have about unit variance in units
of the modelled standard deviation (the model is neither far too wide nor
too narrow) and stay inside the bound."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_09_amd import workloads as wl
from helpers import rope_lse_bounds, rope_o_bounds, sub_pool


def _round(x, dt):
    return torch.from_numpy(x).to(torch.bfloat16 if dt == "bf16" else
                                  torch.float16).double().numpy()


@pytest.mark.parametrize("dt,hd,window", [("bf16", 128, -1), ("bf16", 64, 40),
                                          ("f16", 128, -1), ("bf16", 256, 100)])
def test_rope_lse_model_matches_simulated_operand_rounding(dt, hd, window):
    theta, scale = 1e4, 1.0
    lengths = [1, 33, 200, 900, 1700]
    w = wl.small_workload(seed=97, batch=5, num_qo_heads=8, num_kv_heads=2,
                          head_dim=hd, q_dtype=dt, kv_dtype=dt, o_dtype=dt,
                          window_left=window, lengths=("fixed", lengths))
    case = wl.make_case(w)
    sigma = rope_lse_bounds(w, case, range(w.batch), theta, scale, base=0.0,
                            sigmas=1.0)
    bound = rope_lse_bounds(w, case, range(w.batch), theta, scale)
    pool, indptr, indices, last = sub_pool(case, range(w.batch))
    qn = oracle.widen(wl.raw_numpy(case.q, dt), dt)
    kc = oracle.widen(wl.raw_numpy(pool, dt), dt)[:, 0]
    z = []
    for i, L in enumerate(lengths):
        K, _ = oracle.gather_request(kc, kc, "NHD", indices, indptr, i, L, 16)
        s0 = oracle.window_start(L, window)
        Kr = oracle.rope_rotate(K[s0:].transpose(1, 0, 2), np.arange(s0, L), theta, scale)
        qr = oracle.rope_rotate(qn[i][:, None, :], [L - 1], theta, scale)[:, 0]
        Kt, qt = _round(Kr, dt), _round(qr, dt)
        for hq in range(w.num_qo_heads):
            h = hq // (w.num_qo_heads // w.num_kv_heads)
            exact = np.logaddexp.reduce(w.sm_scale * (Kr[h] @ qr[hq]))
            rounded = np.logaddexp.reduce(w.sm_scale * (Kt[h] @ qt[hq]))
            assert abs(rounded - exact) <= bound[i, hq]
            z.append((rounded - exact) / sigma[i, hq])
    assert 0.5 < float(np.std(z)) < 1.5, np.std(z)


@pytest.mark.parametrize("dt,hd,window,G", [("bf16", 128, -1, 4), ("bf16", 64, 40, 2),
                                            ("f16", 128, -1, 4), ("bf16", 128, 3, 8)])
def test_rope_o_model_matches_simulated_rounding(dt, hd, window, G):
    """helpers.rope_o_bounds against a brute-force simulation of the RoPE
    instances' roundings: rotated q and keys rounded to the operand type, the
    softmax weights from them, each p rounded (against the maximum) as the
    P.V operand while the normaliser sums the unrounded p. The simulated o
    errors stay inside the bound and have about unit spread in units of the
    modelled standard deviation (short requests included: 1 and 3 tokens),
    for each error source alone and for both together."""
    theta, scale = 1e4, 1.0
    lengths = [1, 3, 33, 200, 900]
    w = wl.small_workload(seed=99, batch=5, num_qo_heads=2 * G, num_kv_heads=2,
                          head_dim=hd, q_dtype=dt, kv_dtype=dt, o_dtype=dt,
                          window_left=window, lengths=("fixed", lengths))
    case = wl.make_case(w)
    pool, indptr, indices, last = sub_pool(case, range(w.batch))
    qn = oracle.widen(wl.raw_numpy(case.q, dt), dt)
    kv = oracle.widen(wl.raw_numpy(pool, dt), dt)
    exact, sim, sim_ops, sim_p = [], [], [], []
    for i, L in enumerate(lengths):
        K, V = oracle.gather_request(kv[:, 0], kv[:, 1], "NHD", indices, indptr, i, L, 16)
        s0 = oracle.window_start(L, window)
        Kr = oracle.rope_rotate(K[s0:].transpose(1, 0, 2), np.arange(s0, L), theta, scale)
        qr = oracle.rope_rotate(qn[i][:, None, :], [L - 1], theta, scale)[:, 0]
        Kt, qt = _round(Kr, dt), _round(qr, dt)
        oe, os_, oo, op = [], [], [], []
        for hq in range(w.num_qo_heads):
            h = hq // G
            Vh = V[s0:, h]
            x = w.sm_scale * (Kr[h] @ qr[hq])
            p = np.exp(x - x.max())
            oe.append(p @ Vh / p.sum())
            op.append(_round(p, dt) @ Vh / p.sum())            # P rounding alone
            xt = w.sm_scale * (Kt[h] @ qt[hq])
            pt = np.exp(xt - xt.max())
            oo.append(pt @ Vh / pt.sum())                      # operand rounding alone
            os_.append(_round(pt, dt) @ Vh / pt.sum())
        exact.append(oe)
        sim.append(os_)
        sim_ops.append(oo)
        sim_p.append(op)
    exact = np.array(exact)                                    # [B, nq, hd]
    bound = rope_o_bounds(w, case, range(w.batch), theta, scale, exact)
    assert np.all(np.abs(np.array(sim) - exact) <= bound)
    for s_, parts in ((sim, ("operands", "p")), (sim_ops, ("operands",)), (sim_p, ("p",))):
        sigma = rope_o_bounds(w, case, range(w.batch), theta, scale, exact, sigmas=1.0,
                              base=False, parts=parts)
        err = np.array(s_) - exact
        z = err[sigma > 0] / sigma[sigma > 0]
        assert 0.7 < float(np.std(z)) < 1.3, (parts, np.std(z))


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_o_bounds_cover_output_rounding(dt):
    """helpers.o_bounds admits the rounding of exact outputs to the output
    dtype (what a perfect kernel would write), and equals the plain max-abs
    tolerance wherever that rounding stays below it."""
    from helpers import O_TOL, o_bounds
    w = wl.small_workload(q_dtype=dt, kv_dtype=dt, o_dtype=dt)
    x = np.random.default_rng(5).standard_normal(200000) * 4.0
    r = torch.from_numpy(x).to(torch.bfloat16 if dt == "bf16" else torch.float16).double().numpy()
    b = o_bounds(w, x)
    assert np.all(np.abs(r - x) <= b)
    small = np.abs(x) < (4.0 if dt == "bf16" else 4.0)
    assert np.all(b[small] == O_TOL[dt])
