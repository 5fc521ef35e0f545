"""Pins of the fp64 CPU oracle against facts fixed outside the oracle.

Each test checks the oracle against something other than itself: the values
the decode API page prints for its class example, a library routine
(torch's scaled_dot_product_attention, torch's fp8/bf16 casts), brute force on
tiny inputs, closed forms, or invariants of softmax attention. A plausible
mistake (a wrong head mapping, an off-by-one length or window edge, a
transposed layout, a wrong soft-cap order, a base-2 LSE) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import fp8 as ofp8
from paged_kv_decode_09_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def scatter_to_pages(K_list, V_list, layout, page_size, pool_pages, rng,
                     fill=np.nan, dtype=np.float64):
    """Independent writer: lay dense per-request K/V out in a paged cache.

    Written with explicit loops over tokens, unlike the oracle's gather.
    Returns (cache [pool, 2, ...], indptr, indices, last_page_len).
    """
    nkv, hd = K_list[0].shape[1], K_list[0].shape[2]
    npages = [(len(K) + page_size - 1) // page_size for K in K_list]
    used = sum(npages)
    perm = rng.permutation(pool_pages)[:used]
    if layout == "NHD":
        cache = np.full((pool_pages, 2, page_size, nkv, hd), fill, dtype=dtype)
    else:
        cache = np.full((pool_pages, 2, nkv, page_size, hd), fill, dtype=dtype)
    indptr = [0]
    last = []
    cursor = 0
    for K, V, n in zip(K_list, V_list, npages):
        for tok in range(len(K)):
            page = perm[cursor + tok // page_size]
            slot = tok % page_size
            for h in range(nkv):
                if layout == "NHD":
                    cache[page, 0, slot, h, :] = K[tok, h]
                    cache[page, 1, slot, h, :] = V[tok, h]
                else:
                    cache[page, 0, h, slot, :] = K[tok, h]
                    cache[page, 1, h, slot, :] = V[tok, h]
        cursor += n
        indptr.append(cursor)
        last.append(len(K) - page_size * (n - 1))
    return (cache, np.array(indptr, np.int32), perm.astype(np.int32),
            np.array(last, np.int32))


def sdpa_decode(q, K, V, sm_scale, lo=0):
    """torch SDPA (fp64, CPU) of one query row per head over tokens [lo, L).

    Grouped heads are expanded by SDPA itself (enable_gqa)."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(K[lo:].transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V[lo:].transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=sm_scale,
                                       enable_gqa=True)
    return o[0, :, 0, :].numpy()


def rand_case(rng, lengths, nq, nkv, hd):
    K = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    V = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    q = rng.standard_normal((len(lengths), nq, hd))
    return q, K, V


# ---------------------------------------------------------- stored formats

def test_e4m3_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    mine = ofp8.E4M3_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    # signed zero is preserved too
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(mine[ok]))


def test_e4m3_spot_values():
    t = ofp8.E4M3_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0       # largest finite
    assert t[0x01] == 2.0 ** -9                          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9                      # largest subnormal
    assert t[0x08] == 2.0 ** -6                          # smallest normal
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2                      # no inf, 2 NaNs


def test_bf16_and_f16_widening_match_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, 4096, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    ref = ref.double().numpy()
    mine = oracle.widen(bits, "bf16")
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    h = rng.standard_normal(1000).astype(np.float16)
    assert np.array_equal(oracle.widen(h, "f16"),
                          torch.from_numpy(h).double().numpy())
    codes = np.arange(256, dtype=np.uint8)
    sc = oracle.widen(codes, "e4m3", 1.0 / 64)
    ok = ~np.isnan(sc)
    assert np.array_equal(sc[ok], ofp8.E4M3_TABLE[ok] / 64)


# ------------------------------------------------- the pages' worked example

def test_worked_example_lengths_and_shape():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    lens = oracle.kv_lengths(g["kv_page_indptr"], g["kv_last_page_len"],
                             g["page_size"])
    assert lens.tolist() == g["kv_len_by_hand"]
    w = wl.WORKLOADS["worked_example"]
    case = wl.make_case(w)
    assert list(case.pool.shape) == g["cache_shape_per_layer"]
    assert case.pt.indptr.tolist() == g["kv_page_indptr"]
    assert case.pt.last_page_len.tolist() == g["kv_last_page_len"]
    assert case.pt.indices.tolist() == list(range(g["max_num_pages"]))
    assert case.pt.lengths.tolist() == g["kv_len_by_hand"]
    pool = wl.raw_numpy(case.pool, "f16")
    o, lse = oracle.batch_decode(
        wl.raw_numpy(case.q, "f16"), pool, "NHD", case.pt.indptr,
        case.pt.indices, case.pt.last_page_len, 16, "f16", "f16", w.sm_scale)
    assert list(o.shape) == g["printed_output_shape"]
    assert lse.shape == (g["batch_size"], g["num_qo_heads"])
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_generator_lengths_round_trip_through_kv_len():
    """The generator writes a page table from drawn lengths; the oracle's
    kv_len must read the same lengths back (independent writer/reader)."""
    rng = np.random.default_rng(3)
    for ps in (1, 2, 4, 16, 64):
        lens = rng.integers(1, 500, 40)
        pt = wl.page_table_for(lens, ps, "perm_used", rng)
        assert np.array_equal(
            oracle.kv_lengths(pt.indptr, pt.last_page_len, ps), lens)


@pytest.mark.parametrize("bad", [
    dict(indptr=[0, 0, 3], last=[1, 1]),     # empty request
    dict(indptr=[0, 2, 3], last=[0, 1]),     # last_page_len 0
    dict(indptr=[0, 2, 3], last=[17, 1]),    # last_page_len > page_size
])
def test_kv_len_rejects_invalid_tables(bad):
    with pytest.raises(ValueError):
        oracle.kv_lengths(bad["indptr"], bad["last"], 16)


# ------------------------------------------------------------------ gather

@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("page_size", [1, 2, 4, 16])
def test_gather_returns_written_rows_bit_exactly(layout, page_size):
    rng = np.random.default_rng(page_size + (layout == "HND") * 100)
    lengths = [1, page_size, page_size + 1, 37, 3 * page_size]
    _, K, V = rand_case(rng, lengths, 4, 2, 8)
    npages = sum((L + page_size - 1) // page_size for L in lengths)
    cache, indptr, indices, last = scatter_to_pages(
        K, V, layout, page_size, npages + 7, rng)
    lens = oracle.kv_lengths(indptr, last, page_size)
    assert lens.tolist() == lengths
    for i, L in enumerate(lengths):
        Kg, Vg = oracle.gather_request(cache[:, 0], cache[:, 1], layout,
                                       indices, indptr, i, int(lens[i]),
                                       page_size)
        assert Kg.shape == K[i].shape
        assert np.array_equal(Kg, K[i]) and np.array_equal(Vg, V[i])
        assert not np.isnan(Kg).any()   # unused slots (NaN) never gathered


# ------------------------------------------------- attention vs a library

@pytest.mark.parametrize("group", [1, 2, 4])
@pytest.mark.parametrize("page_size", [1, 2, 4, 16])
@pytest.mark.parametrize("hd", [4, 8])
def test_decode_matches_torch_sdpa(group, page_size, hd):
    rng = np.random.default_rng(group * 100 + page_size * 10 + hd)
    nkv = 2
    nq = nkv * group
    lengths = list(rng.integers(1, 41, 3))
    q, K, V = rand_case(rng, lengths, nq, nkv, hd)
    npages = sum((L + page_size - 1) // page_size for L in lengths)
    for layout in ("NHD", "HND"):
        cache, indptr, indices, last = scatter_to_pages(
            K, V, layout, page_size, npages + 3, rng)
        sm = 1.0 / math.sqrt(hd)
        o, lse = oracle.batch_decode(q, cache, layout, indptr, indices,
                                     last, page_size, "f64", "f64", sm)
        for i in range(len(lengths)):
            ref = sdpa_decode(q[i], K[i], V[i], sm)
            assert np.max(np.abs(o[i] - ref)) < 1e-12


@pytest.mark.parametrize("window", [0, 1, 5, 17, 39, 1000])
def test_window_matches_sdpa_on_the_last_tokens(window):
    rng = np.random.default_rng(window + 11)
    lengths = [40, 17, 1, 6]
    q, K, V = rand_case(rng, lengths, 4, 2, 8)
    cache, indptr, indices, last = scatter_to_pages(K, V, "NHD", 4, 40, rng)
    sm = 0.3
    o, _ = oracle.batch_decode(q, cache, "NHD", indptr, indices, last, 4,
                               "f64", "f64", sm, window_left=window)
    for i, L in enumerate(lengths):
        n_attended = min(L, window + 1)   # inclusive left window
        ref = sdpa_decode(q[i], K[i], V[i], sm, lo=L - n_attended)
        assert np.max(np.abs(o[i] - ref)) < 1e-12


# ----------------------------------------------------- closed forms/special

def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(5)
    q, K, V = rand_case(rng, [33], 8, 2, 16)
    _, _, p = oracle.attention_state(q[0], K[0], V[0], 0.25,
                                     return_weights=True)
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12


@pytest.mark.parametrize("window", [-1, 0, 3, 50, 499])
def test_zero_query_gives_log_count_and_mean(window):
    """q = 0 makes every logit 0: lse = ln(#attended), o = mean of V."""
    rng = np.random.default_rng(9)
    lengths = [500, 64, 1, 129]
    _, K, V = rand_case(rng, lengths, 4, 2, 8)
    q = np.zeros((len(lengths), 4, 8))
    cache, indptr, indices, last = scatter_to_pages(K, V, "HND", 16, 60, rng)
    o, lse = oracle.batch_decode(q, cache, "HND", indptr, indices, last, 16,
                                 "f64", "f64", 0.5, window_left=window)
    for i, L in enumerate(lengths):
        n = L if window < 0 else min(L, window + 1)
        assert np.all(np.abs(lse[i] - math.log(n)) < 1e-12)
        mean = V[i][L - n:].mean(axis=0)            # [nkv, hd]
        ref = np.repeat(mean, 2, axis=0)            # heads hq -> hq // 2
        assert np.max(np.abs(o[i] - ref)) < 1e-12


def test_constant_keys_give_closed_form_lse():
    """All keys equal k: every logit is sm*q.k, so lse = sm*q.k + ln(n)."""
    rng = np.random.default_rng(12)
    L, nkv, hd = 77, 2, 8
    k = rng.standard_normal((nkv, hd))
    K = np.broadcast_to(k, (L, nkv, hd)).copy()
    V = rng.standard_normal((L, nkv, hd))
    q = rng.standard_normal((4, hd))
    o, lse = oracle.attention_state(q, K, V, 0.7)
    for hq in range(4):
        h = hq // 2
        assert abs(lse[hq] - (0.7 * float(np.dot(q[hq], k[h])) + math.log(L))) < 1e-12
        assert np.max(np.abs(o[hq] - V[:, h].mean(axis=0))) < 1e-12


def test_window_zero_returns_last_value_exactly():
    rng = np.random.default_rng(13)
    lengths = [1, 2, 19, 64]
    q, K, V = rand_case(rng, lengths, 6, 3, 8)
    cache, indptr, indices, last = scatter_to_pages(K, V, "NHD", 16, 10, rng)
    o, lse = oracle.batch_decode(q, cache, "NHD", indptr, indices, last, 16,
                                 "f64", "f64", 1.0, window_left=0)
    for i, L in enumerate(lengths):
        assert np.array_equal(o[i], np.repeat(V[i][L - 1], 2, axis=0))


def test_soft_cap_huge_equals_uncapped():
    rng = np.random.default_rng(14)
    q, K, V = rand_case(rng, [50], 4, 2, 8)
    a = oracle.attention_state(q[0], K[0], V[0], 0.35)
    b = oracle.attention_state(q[0], K[0], V[0], 0.35, logits_soft_cap=1e9)
    assert np.max(np.abs(a[0] - b[0])) < 1e-9
    assert np.max(np.abs(a[1] - b[1])) < 1e-9


def test_soft_cap_saturates_to_plus_minus_cap():
    """Logits of magnitude >> cap saturate to +-cap: the positive-logit tokens
    share the weight equally and lse = cap + ln(#positive)."""
    rng = np.random.default_rng(15)
    L, hd, cap = 40, 4, 50.0
    sign = np.where(rng.random(L) < 0.4, 1.0, -1.0)
    K = np.zeros((L, 1, hd))
    K[:, 0, 0] = sign * (1.0 + rng.random(L))
    K[:, 0, 1:] = rng.standard_normal((L, hd - 1))
    V = rng.standard_normal((L, 1, hd))
    q = np.zeros((1, hd))
    q[0, 0] = 1e4                       # |x| >= 0.5 * 1e4 >> cap
    o, lse = oracle.attention_state(q, K, V, 0.5, logits_soft_cap=cap)
    pos = sign > 0
    assert abs(lse[0] - (cap + math.log(pos.sum()))) < 1e-9
    assert np.max(np.abs(o[0] - V[pos, 0].mean(axis=0))) < 1e-12


def test_soft_cap_bounds_every_logit():
    rng = np.random.default_rng(16)
    L, cap = 64, 3.0
    q, K, V = rand_case(rng, [L], 2, 1, 8)
    q *= 20.0
    _, lse = oracle.attention_state(q[0], K[0], V[0], 1.0,
                                    logits_soft_cap=cap)
    assert np.all(lse < cap + math.log(L)) and np.all(lse > -cap + math.log(L))


# ------------------------------------------------------------ split + merge

@pytest.mark.parametrize("split_pages", [1, 2, 3, 8, 64])
@pytest.mark.parametrize("window", [-1, 0, 37, 200])
def test_split_then_merge_equals_unsplit(split_pages, window):
    rng = np.random.default_rng(split_pages * 7 + window)
    lengths = [1, 16, 17, 250, 129]
    q, K, V = rand_case(rng, lengths, 8, 2, 8)
    cache, indptr, indices, last = scatter_to_pages(K, V, "NHD", 16, 40, rng)
    args = (q, cache, "NHD", indptr, indices, last, 16, "f64", "f64", 0.4)
    o1, l1 = oracle.batch_decode(*args, window_left=window)
    o2, l2 = oracle.batch_decode_split(*args, split_pages, window_left=window)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l1 - l2)) < 1e-12


def test_merge_states_of_disjoint_parts_matches_sdpa_on_union():
    rng = np.random.default_rng(21)
    L, nkv, hd = 90, 2, 8
    q, K, V = rand_case(rng, [L], 4, nkv, hd)
    cuts = [0, 13, 14, 60, 90]
    parts = [oracle.attention_state(q[0], K[0][a:b], V[0][a:b], 0.3)
             for a, b in zip(cuts[:-1], cuts[1:])]
    v = np.stack([p[0] for p in parts], axis=1)
    s = np.stack([p[1] for p in parts], axis=1)
    o, _ = oracle.merge_states(v, s)
    ref = sdpa_decode(q[0], K[0], V[0], 0.3)
    assert np.max(np.abs(o - ref)) < 1e-12


def test_merge_states_empty_states():
    v = np.ones((3, 2, 4))
    s = np.array([[-np.inf, -np.inf], [-np.inf, 0.5], [1.0, 1.0]])
    vo, so = oracle.merge_states(v * np.array([1.0, 2.0])[None, :, None], s)
    assert np.all(vo[0] == 0) and so[0] == -np.inf
    assert np.allclose(vo[1], 2.0) and so[1] == 0.5
    assert np.allclose(vo[2], 1.5) and abs(so[2] - (1.0 + math.log(2))) < 1e-15


def test_chunk_bounds_cover_the_attended_range():
    for L in (1, 15, 16, 17, 255, 256, 257, 4096, 5000):
        for S in (1, 2, 5, 16):
            for w in (-1, 0, 10, 300):
                ch = oracle.chunk_bounds(L, 16, S, w)
                s0 = oracle.window_start(L, w)
                assert ch[0][0] == s0 and ch[-1][1] == L
                for (a, b), (c, _) in zip(ch[:-1], ch[1:]):
                    assert b == c and b % (16 * S) == 0
                for a, b in ch:
                    assert 0 < b - a <= 16 * S


# ------------------------------------------- inputs used by the GPU parity

@pytest.mark.parametrize("name", ["worked_example", "serving_batch",
                                  "long_context", "gemma2_decode", "fp8_kv"])
def test_named_workload_page_tables(name):
    w = wl.WORKLOADS[name]
    rng = np.random.default_rng(w.seed)
    pt = wl.make_page_table(w, rng)
    assert len(pt.lengths) == w.batch
    assert np.array_equal(oracle.kv_lengths(pt.indptr, pt.last_page_len,
                                            w.page_size), pt.lengths)
    # every page used once, inside the pool
    assert len(np.unique(pt.indices)) == len(pt.indices)
    assert pt.indices.min() >= 0 and pt.indices.max() < pt.pool_pages


def test_poison_fills_only_unreadable_slots():
    w = wl.small_workload(batch=4, lengths=("uniform", 1, 60), pool_pages=30)
    case = wl.make_case(w, poison=True)
    pool = wl.raw_numpy(case.pool, "f16").astype(np.float64)
    lens = oracle.kv_lengths(case.pt.indptr, case.pt.last_page_len, 16)
    seen = 0
    for i, L in enumerate(lens):
        K, V = oracle.gather_request(pool[:, 0], pool[:, 1], "NHD",
                                     case.pt.indices, case.pt.indptr, i,
                                     int(L), 16)
        assert not np.isnan(K).any() and not np.isnan(V).any()
        seen += int(L)
    # everything not gathered is NaN
    total = pool[:, 0, :, 0, 0].size
    assert np.isnan(pool[:, 0, :, 0, 0]).sum() == total - seen


# ------------------------------------------- several query tokens per request

def sdpa_masked(q_rows, K, V, sm_scale, mask):
    """torch SDPA (fp64, CPU) of query rows [Q, nq, hd] over K/V [L, nkv, hd]
    with a boolean mask [Q, L] (True = attend), grouped heads expanded."""
    qt = torch.from_numpy(np.ascontiguousarray(q_rows.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    m = torch.from_numpy(mask)[None, None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=sm_scale,
                                       enable_gqa=True)
    return o[0].numpy().transpose(1, 0, 2)


def prefill_causal_mask(qo_len, kv_len, window_left=-1):
    """The custom-mask construction of the prefill wrapper's example on the
    decode API page (lower triangle with diagonal kv_len - qo_len), with the
    inclusive left window cut out below it."""
    m = torch.tril(torch.full((qo_len, kv_len), True),
                   diagonal=kv_len - qo_len)
    if window_left >= 0:
        m &= torch.triu(torch.full((qo_len, kv_len), True),
                        diagonal=kv_len - qo_len - window_left)
    return m.numpy()


@pytest.mark.parametrize("Q,group", [(2, 1), (3, 2), (4, 4), (8, 2), (16, 1)])
@pytest.mark.parametrize("page_size", [1, 4, 16])
def test_multi_token_matches_sdpa_with_the_prefill_causal_mask(Q, group,
                                                              page_size):
    rng = np.random.default_rng(Q * 100 + group * 10 + page_size)
    nkv, hd = 2, 8
    nq = nkv * group
    lengths = [Q, Q + 1, int(rng.integers(Q, 45)), 37]
    K = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    V = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    q = rng.standard_normal((len(lengths) * Q, nq, hd))
    npages = sum((L + page_size - 1) // page_size for L in lengths)
    for layout in ("NHD", "HND"):
        cache, indptr, indices, last = scatter_to_pages(
            K, V, layout, page_size, npages + 2, rng)
        o, lse = oracle.batch_decode_multi(q, cache, layout, indptr, indices,
                                           last, page_size, Q, "f64", "f64",
                                           0.35)
        for i, L in enumerate(lengths):
            ref = sdpa_masked(q[i * Q:(i + 1) * Q], K[i], V[i], 0.35,
                              prefill_causal_mask(Q, L))
            assert np.max(np.abs(o[i * Q:(i + 1) * Q] - ref)) < 1e-12


@pytest.mark.parametrize("window", [0, 1, 3, 10, 100])
def test_multi_token_window_matches_sdpa(window):
    rng = np.random.default_rng(window + 5)
    Q, nkv, group, hd = 4, 2, 2, 8
    lengths = [4, 5, 23, 40]
    K = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    V = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    q = rng.standard_normal((len(lengths) * Q, nkv * group, hd))
    cache, indptr, indices, last = scatter_to_pages(K, V, "NHD", 4, 40, rng)
    o, _ = oracle.batch_decode_multi(q, cache, "NHD", indptr, indices, last, 4,
                                     Q, "f64", "f64", 0.3, window_left=window,
                                     logits_soft_cap=0.0)
    for i, L in enumerate(lengths):
        ref = sdpa_masked(q[i * Q:(i + 1) * Q], K[i], V[i], 0.3,
                          prefill_causal_mask(Q, L, window))
        assert np.max(np.abs(o[i * Q:(i + 1) * Q] - ref)) < 1e-12


def test_multi_token_zero_query_counts_each_tokens_prefix():
    # q = 0: every visible logit is 0, so lse of query token j is the log of
    # the number of tokens it sees: min(L - Q + j + 1, window + 1).
    rng = np.random.default_rng(3)
    Q, nkv, hd = 3, 2, 4
    lengths = [3, 9, 30]
    K = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    V = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    cache, indptr, indices, last = scatter_to_pages(K, V, "HND", 2, 30, rng)
    for window in (-1, 0, 4):
        q = np.zeros((len(lengths) * Q, nkv, hd))
        _, lse = oracle.batch_decode_multi(q, cache, "HND", indptr, indices,
                                           last, 2, Q, "f64", "f64", 1.0,
                                           window_left=window)
        for i, L in enumerate(lengths):
            for j in range(Q):
                seen = L - Q + j + 1
                if window >= 0:
                    seen = min(seen, window + 1)
                assert np.allclose(lse[i * Q + j], math.log(seen), atol=1e-12)


def test_multi_token_last_token_is_the_single_token_decode():
    rng = np.random.default_rng(8)
    Q, nkv, hd = 4, 2, 8
    lengths = [4, 19, 33]
    K = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    V = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    q = rng.standard_normal((len(lengths) * Q, 2 * nkv, hd))
    cache, indptr, indices, last = scatter_to_pages(K, V, "NHD", 4, 20, rng)
    o, lse = oracle.batch_decode_multi(q, cache, "NHD", indptr, indices, last,
                                       4, Q, "f64", "f64", 0.2)
    o1, lse1 = oracle.batch_decode(q[Q - 1::Q], cache, "NHD", indptr, indices,
                                   last, 4, "f64", "f64", 0.2)
    assert np.array_equal(o[Q - 1::Q], o1) and np.array_equal(lse[Q - 1::Q], lse1)


def test_multi_token_rejects_short_requests():
    rng = np.random.default_rng(1)
    K = [rng.standard_normal((2, 1, 4))]
    cache, indptr, indices, last = scatter_to_pages(K, K, "NHD", 4, 2, rng)
    with pytest.raises(ValueError):
        oracle.batch_decode_multi(np.zeros((3, 1, 4)), cache, "NHD", indptr,
                                  indices, last, 4, 3, "f64", "f64", 1.0)


# ------------------------------------------------------ block-table page input

@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_block_table_gather_returns_written_rows(layout):
    """Independent writer: tokens written, one by one, into the slot
    t % P of page block_tables[i][t // P]; the oracle's CSR view of the
    table must gather them back bit-exactly."""
    rng = np.random.default_rng(12)
    P, nkv, hd, max_blocks = 4, 2, 3, 6
    lens = [1, 4, 5, 23, 24]
    pool = 40
    cache = np.full((pool, 2) + ((P, nkv, hd) if layout == "NHD" else (nkv, P, hd)),
                    np.nan)
    table = rng.permutation(pool)[:len(lens) * max_blocks].reshape(len(lens),
                                                                  max_blocks)
    dense = []
    for i, L in enumerate(lens):
        K = rng.standard_normal((L, nkv, hd))
        V = rng.standard_normal((L, nkv, hd))
        for t in range(L):
            pg, sl = table[i, t // P], t % P
            for h in range(nkv):
                if layout == "NHD":
                    cache[pg, 0, sl, h], cache[pg, 1, sl, h] = K[t, h], V[t, h]
                else:
                    cache[pg, 0, h, sl], cache[pg, 1, h, sl] = K[t, h], V[t, h]
        dense.append((K, V))
    indptr, indices, last = oracle.csr_from_block_table(lens, table, P)
    assert list(oracle.kv_lengths(indptr, last, P)) == lens
    for i, L in enumerate(lens):
        K, V = oracle.gather_request(cache[:, 0], cache[:, 1], layout, indices,
                                     indptr, i, L, P)
        assert np.array_equal(K, dense[i][0]) and np.array_equal(V, dense[i][1])


def test_block_table_rejects_short_rows():
    with pytest.raises(ValueError):
        oracle.csr_from_block_table([9], np.zeros((1, 2), np.int32), 4)
    with pytest.raises(ValueError):
        oracle.csr_from_block_table([0], np.zeros((1, 2), np.int32), 4)


# ------------------------------------------------------------ attention sinks

def test_sink_of_minus_infinity_changes_nothing():
    rng = np.random.default_rng(21)
    q, K, V = rng.standard_normal((4, 8)), rng.standard_normal((9, 2, 8)), \
        rng.standard_normal((9, 2, 8))
    a = oracle.attention_state(q, K, V, 0.4)
    b = oracle.attention_state(q, K, V, 0.4, sinks=np.full(4, -np.inf))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_sink_with_zero_query_closed_form():
    # every logit 0: o = n/(n + e^s) * mean(V), lse = ln(n + e^s)
    rng = np.random.default_rng(22)
    n = 13
    K, V = rng.standard_normal((n, 1, 4)), rng.standard_normal((n, 1, 4))
    for s in (-3.0, 0.0, 2.5, 40.0):
        o, lse = oracle.attention_state(np.zeros((2, 4)), K, V, 1.0,
                                        sinks=np.array([s, s]))
        z = n + math.exp(s)
        assert np.allclose(o[0], V[:, 0].sum(0) / z, atol=1e-12)
        assert abs(lse[0] - math.log(z)) < 1e-12


def test_sink_equals_sdpa_with_a_zero_value_key():
    """The sink acts as one more key whose logit is s and whose value row is
    zero: SDPA (fp64) over K and V extended by such a row, per q head."""
    rng = np.random.default_rng(23)
    nq, nkv, hd, n = 4, 2, 8, 11
    q = rng.standard_normal((nq, hd))
    K, V = rng.standard_normal((n, nkv, hd)), rng.standard_normal((n, nkv, hd))
    sinks = rng.standard_normal(nq) * 2
    sm = 0.3
    o, _ = oracle.attention_state(q, K, V, sm, sinks=sinks)
    for hq in range(nq):
        h = hq // (nq // nkv)
        ks = q[hq] * sinks[hq] / (sm * (q[hq] @ q[hq]))   # sm * q.ks = sink
        Ke = np.concatenate([K[:, h], ks[None]])[None, None]
        Ve = np.concatenate([V[:, h], np.zeros((1, hd))])[None, None]
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[hq][None, None, None]),
                                             torch.from_numpy(Ke), torch.from_numpy(Ve),
                                             scale=sm)[0, 0, 0].numpy()
        assert np.max(np.abs(o[hq] - ref)) < 1e-12


# ------------------------------------------------------------------- ALiBi

def test_alibi_slopes_of_eight_heads_are_the_powers_of_one_half():
    # the ALiBi paper's example: 8 heads get 1/2, 1/4, ..., 1/256
    assert np.array_equal(oracle.alibi_slopes(8), 0.5 ** np.arange(1, 9))
    # 16 heads: 2^-0.5, 2^-1, ..., 2^-8
    assert np.allclose(oracle.alibi_slopes(16), 2.0 ** (-0.5 * np.arange(1, 17)))
    # 12 heads: the 8-head slopes, then 2^-1/2^-... odd powers of 2^(-4/8)
    s12 = oracle.alibi_slopes(12)
    assert np.array_equal(s12[:8], oracle.alibi_slopes(8))
    assert np.allclose(s12[8:], 2.0 ** (-0.5 * np.array([1, 3, 5, 7])))


@pytest.mark.parametrize("Q,window", [(1, -1), (1, 6), (3, -1), (2, 4)])
def test_alibi_matches_sdpa_with_a_distance_bias(Q, window):
    """SDPA (fp64) with a float mask: slope_h * (t - position of the query
    token), -inf where the causal / window mask hides t."""
    rng = np.random.default_rng(31 + Q)
    nkv, group, hd = 2, 4, 8
    nq = nkv * group
    lengths = [Q, 14, 33]
    K = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    V = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    q = rng.standard_normal((len(lengths) * Q, nq, hd))
    cache, indptr, indices, last = scatter_to_pages(K, V, "HND", 4, 30, rng)
    o, _ = oracle.batch_decode_multi(q, cache, "HND", indptr, indices, last, 4, Q,
                                     "f64", "f64", 0.3, window_left=window,
                                     alibi=True)
    slopes = oracle.alibi_slopes(nq)
    for i, L in enumerate(lengths):
        allowed = prefill_causal_mask(Q, L, window)
        pos = np.arange(L - Q, L)[:, None]
        t = np.arange(L)[None, :]
        bias = slopes[None, :, None, None] * (t - pos)[None, None]   # [1, nq, Q, L]
        bias = np.where(allowed[None, None], bias, -np.inf)
        qt = torch.from_numpy(np.ascontiguousarray(q[i * Q:(i + 1) * Q].transpose(1, 0, 2)))[None]
        kt = torch.from_numpy(np.ascontiguousarray(K[i].transpose(1, 0, 2)))[None]
        vt = torch.from_numpy(np.ascontiguousarray(V[i].transpose(1, 0, 2)))[None]
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(bias),
                                             scale=0.3, enable_gqa=True)[0].numpy()
        assert np.max(np.abs(o[i * Q:(i + 1) * Q] - ref.transpose(1, 0, 2))) < 1e-12


# ---------------------------------------------------------------- ROPE_LLAMA

def test_rope_of_a_two_dim_head_is_a_plane_rotation():
    # head_dim 2: one pair, frequency theta^0 = 1, angle = position / scale
    x = np.array([[0.3, -1.2], [2.0, 0.5]])
    for scale in (1.0, 4.0):
        r = oracle.rope_rotate(x, [7, 130000], rope_scale=scale)
        for row, pos in zip(range(2), (7, 130000)):
            a = pos / scale
            ref = [x[row, 0] * math.cos(a) - x[row, 1] * math.sin(a),
                   x[row, 1] * math.cos(a) + x[row, 0] * math.sin(a)]
            assert np.allclose(r[row], ref, atol=1e-12)


def test_rope_dot_products_depend_on_position_differences_only():
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    base = oracle.rope_rotate(q[None], [1000])[0] @ oracle.rope_rotate(k[None], [990])[0]
    for shift in (1, 17, 50000):
        d = oracle.rope_rotate(q[None], [1000 + shift])[0] @ \
            oracle.rope_rotate(k[None], [990 + shift])[0]
        assert abs(d - base) < 1e-9
    # rotations keep norms, and position 0 is the identity
    assert np.allclose(np.linalg.norm(oracle.rope_rotate(q[None], [12345])), np.linalg.norm(q))
    assert np.array_equal(oracle.rope_rotate(q[None], [0])[0], q)


def test_rope_decode_matches_sdpa_on_rotated_inputs():
    """Decode with ROPE_LLAMA = SDPA (fp64) over keys rotated at their token
    positions by an independent rotation (complex multiplication), q rotated
    at its query position."""
    rng = np.random.default_rng(10)
    nkv, group, hd, L = 2, 2, 16, 37
    theta, scale = 500.0, 2.0
    K, V = rng.standard_normal((L, nkv, hd)), rng.standard_normal((L, nkv, hd))
    q = rng.standard_normal((1, nkv * group, hd))
    cache, indptr, indices, last = scatter_to_pages([K], [V], "NHD", 4, 12, rng)
    o, _ = oracle.batch_decode(q, cache, "NHD", indptr, indices, last, 4, "f64", "f64",
                               0.25, rope=(theta, scale))

    def rot(x, pos):   # pairs as complex numbers times e^{i angle}
        half = hd // 2
        w = np.exp(1j * pos / scale * theta ** (-2.0 * np.arange(half) / hd))
        z = (x[..., :half] + 1j * x[..., half:]) * w
        return np.concatenate([z.real, z.imag], axis=-1)
    Kr = np.stack([rot(K[t], t) for t in range(L)])
    qr = rot(q[0], L - 1)
    ref = sdpa_decode(qr, Kr, V, 0.25)
    assert np.max(np.abs(o[0] - ref)) < 1e-12


def _rot_complex(x, positions, theta, scale):
    """Independent rotation: pairs (x[i], x[i + hd/2]) as complex numbers
    times e^{i * position / scale * theta^(-2i/hd)}; x [n, ..., hd]."""
    hd = x.shape[-1]
    half = hd // 2
    ang = np.asarray(positions, np.float64)[:, None] / scale * \
        theta ** (-2.0 * np.arange(half) / hd)[None, :]
    w = np.exp(1j * ang).reshape((len(positions),) + (1,) * (x.ndim - 2) + (half,))
    z = (x[..., :half] + 1j * x[..., half:]) * w
    return np.concatenate([z.real, z.imag], axis=-1)


def _rope_sdpa_reference(q_rows, K, V, L, Q, sm, theta, scale, window):
    """SDPA (fp64) over every key of the request rotated at its absolute
    token index 0..L-1, query token j rotated at L-Q+j, with the prefill
    page's causal mask (diagonal kv_len - qo_len) and the inclusive window;
    lse from torch.logsumexp over the same masked logits."""
    Kr = _rot_complex(K, np.arange(L), theta, scale)             # [L, nkv, hd]
    qr = _rot_complex(q_rows, np.arange(L - Q, L), theta, scale)  # [Q, nq, hd]
    mask = prefill_causal_mask(Q, L, window)
    o = sdpa_masked(qr, Kr, V, sm, mask)
    nq, nkv = q_rows.shape[1], K.shape[1]
    Ke = torch.from_numpy(np.repeat(Kr, nq // nkv, axis=1).transpose(1, 0, 2).copy())
    logits = sm * torch.einsum("jhd,htd->jht", torch.from_numpy(qr), Ke)
    logits = logits.masked_fill(~torch.from_numpy(mask)[:, None, :], -math.inf)
    return o, torch.logsumexp(logits, dim=-1).numpy()


def _rope_window_case(Q, window, seed):
    rng = np.random.default_rng(seed)
    nkv, group, hd = 2, 2, 16
    lengths = [Q + window + 9, 57, Q]     # windows that start past 0, and a full one
    K = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    V = [rng.standard_normal((L, nkv, hd)) for L in lengths]
    q = rng.standard_normal((len(lengths) * Q, nkv * group, hd))
    cache, indptr, indices, last = scatter_to_pages(K, V, "NHD", 4, 40, rng)
    return lengths, K, V, q, (cache, indptr, indices, last)


@pytest.mark.parametrize("Q,window", [(1, 5), (1, 20), (3, 4), (4, 0), (2, 11)])
def test_rope_with_window_and_several_tokens_matches_sdpa_at_absolute_positions(Q, window):
    """ROPE_LLAMA under a window and with q_len_per_req > 1: keys keep their
    absolute token index as position (not an index relative to the window
    start) and query token j sits at L-Q+j."""
    theta, scale, sm = 300.0, 1.5, 0.3
    lengths, K, V, q, (cache, indptr, indices, last) = _rope_window_case(Q, window, 70 + Q)
    o, lse = oracle.batch_decode_multi(q, cache, "NHD", indptr, indices, last, 4, Q,
                                       "f64", "f64", sm, window_left=window,
                                       rope=(theta, scale))
    for i, L in enumerate(lengths):
        ro, rl = _rope_sdpa_reference(q[i * Q:(i + 1) * Q], K[i], V[i], L, Q, sm,
                                      theta, scale, window)
        assert np.max(np.abs(o[i * Q:(i + 1) * Q] - ro)) < 1e-12
        assert np.max(np.abs(lse[i * Q:(i + 1) * Q] - rl)) < 1e-12
    if Q == 1:
        # the one-token entry point gives the same
        o1, l1 = oracle.batch_decode(q, cache, "NHD", indptr, indices, last, 4, "f64",
                                     "f64", sm, window_left=window, rope=(theta, scale))
        assert np.max(np.abs(o1 - o)) < 1e-12 and np.max(np.abs(l1 - lse)) < 1e-12


def test_rope_window_pin_rejects_window_relative_key_positions(monkeypatch):
    """The pin above fails for an oracle that rotates keys at positions
    counted from the window start (a planted mistake in the oracle)."""
    import oracle.oracle as om
    real = om.rope_rotate

    def relative(x, positions, rope_theta=1e4, rope_scale=1.0):
        p = np.asarray(positions)
        if p.size > 1:                        # the keys: shift to the window start
            p = p - p[0]
        return real(x, p, rope_theta, rope_scale)

    monkeypatch.setattr(om, "rope_rotate", relative)
    theta, scale, sm, Q, window = 300.0, 1.5, 0.3, 1, 5
    lengths, K, V, q, (cache, indptr, indices, last) = _rope_window_case(Q, window, 71)
    o, _ = oracle.batch_decode_multi(q, cache, "NHD", indptr, indices, last, 4, Q,
                                     "f64", "f64", sm, window_left=window,
                                     rope=(theta, scale))
    ro, _ = _rope_sdpa_reference(q[:Q], K[0], V[0], lengths[0], Q, sm, theta, scale,
                                 window)
    assert np.max(np.abs(o[:Q] - ro)) > 1e-2
