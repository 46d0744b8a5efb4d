"""Pins of the oracle to facts the pages and the mathematics fix.

Each test would fail for a plausible mistake in oracle/quest.py: swapped
min/max or sign selection (worked example, closed form, box corners), a
wrong GQA head mapping (per-head invariant), a padded tail page (tail pins),
a wrong softmax scale or causal limit (library attention), a wrong tie rule
(all-equal and brute-force top-K), duplicate or invalid pages counted
(invariance tests)."""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import formats, quest, run_decode
from tests.conftest import load_golden
from workloads import tiny_single_head, llama2_7b_layer, batched_gqa_append, figure2_case, worked_example_case


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------- the pages' examples ----

def test_worked_example_summary_and_bound():
    g = load_golden("quest_worked_example.json")
    keys = np.array(g["keys"], float)[:, None, :]
    m, M = quest.page_summaries(keys, len(keys), S=len(keys))
    assert m[0, 0].tolist() == g["m"]
    assert M[0, 0].tolist() == g["M"]
    q = np.array([g["q"]], float)
    U = quest.head_bounds(q, m, M)
    assert U[0, 0] == g["U"]
    assert (keys[:, 0] @ q[0]).tolist() == g["dots"]
    # the alternative keys share the summary and the bound, not the max dot
    alt = np.array(g["alt_keys"], float)[:, None, :]
    m2, M2 = quest.page_summaries(alt, len(alt), S=len(alt))
    assert quest.head_bounds(q, m2, M2)[0, 0] == g["alt_U"]
    assert (alt[:, 0] @ q[0]).tolist() == g["alt_dots"]
    assert max(g["alt_dots"]) < g["alt_U"]


def test_figure2_two_steps():
    g = load_golden("quest_figure2.json")
    S = g["page_capacity"]
    A = np.array(g["keys_A"], float)
    B = np.array(g["keys_B"], float)
    keys = np.concatenate([A, B])[:, None, :]
    L = len(keys)
    m, M = quest.page_summaries(keys, L, S)
    q_t = np.array([g["q_t"]], float)
    U = quest.head_bounds(q_t, m, M)[0]
    assert U.tolist() == [g["U_A_t"], g["U_B_t"]]
    assert quest.top_k_pages(U, 1) == [0]            # page A
    q_t1 = np.array([g["q_t1"]], float)
    assert quest.head_bounds(q_t1, m, M)[0, 1] == g["U_B_t1_without_append"]
    # append (-2, 5) to B with eq. (8)
    k_new = np.array(g["appended_to_B"], float)[None, :]
    mB, MB = quest.append_to_summary(m[1], M[1], k_new, offset=L % S)
    assert mB[0].tolist() == g["m_B_after"] and MB[0].tolist() == g["M_B_after"]
    m2, M2 = m.copy(), M.copy()
    m2[1], M2[1] = mB, MB
    U1 = quest.head_bounds(q_t1, m2, M2)[0]
    assert U1.tolist() == [g["U_A_t1"], g["U_B_t1"]]
    assert quest.top_k_pages(U1, 1) == [1]           # page B
    # bulk summaries over the three-token B agree with the append
    keys3 = np.concatenate([keys, k_new[:, None, :]])
    mb, Mb = quest.page_summaries(keys3, L + 1, S)
    assert np.array_equal(mb[1], mB) and np.array_equal(Mb[1], MB)


def test_figure2_case_padded_layout():
    """The zero-padded d=16 / S=4 workload built from the same reading gives
    the printed bounds through the whole-request oracle."""
    case = figure2_case()
    r0 = run_decode(case, step=-1)[0]
    assert r0["U"][0].tolist() == [8.0, 0.0] and r0["sel"] == [[0]]
    r1 = run_decode(case, step=0)[0]
    assert r1["U"][0].tolist() == [1.0, 5.0] and r1["sel"] == [[1]]


def test_worked_example_case_padded():
    for second in (False, True):
        r = run_decode(worked_example_case(second_set=second))[0]
        assert r["U"][0, 0] == 8.0


def test_four_page_topk():
    g = load_golden("quest_four_pages.json")
    bound = np.array(g["bound"], float)
    names = g["pages"]
    assert [names[j] for j in quest.top_k_pages(bound, 2)] == g["selected_K2"]
    assert [names[j] for j in quest.top_k_pages(bound, 3)] == g["selected_K3"]
    # the bound is valid (never below the true max) even where recall fails
    assert np.all(bound >= np.array(g["true_max"]))


def test_union_and_membership_example():
    g = load_golden("pageweaver_union.json")
    sets = [g["sets"]["q0"], g["sets"]["q2"]]
    union, member = quest.union_with_membership(sets)
    assert union == g["union"]
    for row, name in enumerate(("q0", "q2")):
        masked = [p for u, p in enumerate(union) if member[row, u] == 0]
        assert masked == g["masked"][name]


# ---------------------------------------------------- closed forms, bounds --

def test_regroup_worked_example():
    """[PageWeaver] Algorithm 1 step-by-step example (g = 3): seed 0, first
    costs 2,1,2,2,2, pi = [0,2,3,1,4,5]; page visits of the two groups go
    from 5 + 5 = 10 in the original order to 4 + 3 = 7."""
    g = load_golden("pageweaver_regroup.json")
    sets = [set(x) for x in g["sets"]]
    # the printed first-round costs |S_j minus S_0| of candidates 1..5
    assert [len(sets[j] - sets[0]) for j in range(1, 6)] == g["seed0_costs"]
    pi = quest.regroup_window(sets, g["group"])
    assert pi == g["pi"]

    def visits(order):
        G = g["group"]
        return sum(len(quest.union_with_membership([sets[i] for i in order[k:k + G]])[0])
                   for k in range(0, len(order), G))
    assert visits(list(range(6))) == g["pages_original_order"]
    assert visits(pi) == g["pages_regrouped"]
    # windows within a request: one window holding all six gives the same
    assert quest.regroup([list(x) for x in g["sets"]], [11], [0, 6], 8, 3, 512) == pi


def test_regroup_uses_marginal_increase_not_overlap():
    """With sets of different sizes the notes keep the marginal increase
    |S_j minus U| (not the largest overlap): S_1 shares 2 pages with S_0 but
    adds 4, S_2 shares none and adds 1."""
    sets = [{1, 2, 3, 4}, {1, 2, 5, 6, 7, 8}, {9}]
    assert quest.regroup_window(sets, 2) == [0, 2, 1]


def test_regroup_is_a_windowed_bijection():
    rng = _rng(33)
    for _ in range(40):
        B = int(rng.integers(1, 4))
        counts = rng.integers(0, 40, size=B)
        q_indptr = np.concatenate([[0], np.cumsum(counts)])
        n_pages = rng.integers(1, 30, size=B)
        N = int(q_indptr[-1])
        sets = [list(rng.integers(-2, 35, size=5)) for _ in range(N)]
        W = int(rng.choice([8, 16, 64]))
        g = int(rng.choice([1, 2, 4, 8]))
        cap = int(rng.choice([8, 512]))
        ids = quest.regroup(sets, n_pages, q_indptr, W, g, cap)
        assert sorted(ids) == list(range(N))
        for r in range(B):
            a, b = int(q_indptr[r]), int(q_indptr[r + 1])
            assert sorted(ids[a:b]) == list(range(a, b))        # stays in its request
            for w0 in range(a, b, W):                            # and in its window
                assert sorted(ids[w0:min(b, w0 + W)]) == list(range(w0, min(b, w0 + W)))
            if n_pages[r] > cap or g == 1:
                assert ids[a:b] == list(range(a, b))             # identity
    # equal sets: every cost ties, the lowest ID wins, so the order is kept
    assert quest.regroup_window([{1, 2}] * 9, 4) == list(range(9))


def test_bound_closed_form():
    """A box's support function is q.(M+m)/2 + |q|.(M-m)/2."""
    rng = _rng(1)
    for _ in range(20):
        d, P = int(rng.integers(1, 40)), int(rng.integers(1, 9))
        a, b = rng.normal(size=(2, P, 1, d))
        m, M = np.minimum(a, b), np.maximum(a, b)
        q = rng.normal(size=(1, d))
        U = quest.head_bounds(q, m, M)[0]
        closed = (m[:, 0] + M[:, 0]) @ q[0] / 2 + (M[:, 0] - m[:, 0]) @ np.abs(q[0]) / 2
        np.testing.assert_allclose(U, closed, rtol=1e-12, atol=1e-12)


def test_bound_equals_max_over_box_corners():
    """Brute force: the bound equals the largest dot product over all 2^d
    corners of the box [m, M] (the Quest page, §3.1, support function)."""
    rng = _rng(2)
    d = 10
    for _ in range(5):
        a, b = rng.normal(size=(2, 1, 1, d))
        m, M = np.minimum(a, b), np.maximum(a, b)
        q = rng.normal(size=(1, d))
        best = -np.inf
        for corner in itertools.product((0, 1), repeat=d):
            c = np.where(np.array(corner) == 1, M[0, 0], m[0, 0])
            best = max(best, float(c @ q[0]))
        assert abs(quest.head_bounds(q, m, M)[0, 0] - best) < 1e-12


def test_bound_invariant_and_tightness():
    """eq. (4): U_p(q) >= q.k for every key of the page; a one-token page is
    tight."""
    rng = _rng(3)
    for S in (1, 3, 16):
        keys = rng.normal(size=(S * 20, 2, 32))
        L = keys.shape[0]
        m, M = quest.page_summaries(keys, L, S)
        q = rng.normal(size=(4, 32))            # g = 2
        U = quest.head_bounds(q, m, M)
        for i in range(4):
            h = i // 2
            dots = (keys[:, h, :] @ q[i]).reshape(-1, S).max(axis=1)
            assert np.all(U[i] >= dots - 1e-12)
            if S == 1:
                np.testing.assert_allclose(U[i], dots, rtol=1e-12, atol=1e-12)


def test_bound_homogeneity_and_zero_query():
    rng = _rng(4)
    keys = rng.normal(size=(64, 1, 8))
    m, M = quest.page_summaries(keys, 64, 16)
    q = rng.normal(size=(1, 8))
    U = quest.head_bounds(q, m, M)
    np.testing.assert_allclose(quest.head_bounds(2.5 * q, m, M), 2.5 * U, rtol=1e-12)
    assert np.all(quest.head_bounds(0 * q, m, M) == 0)


def test_gqa_group_score_bounds_every_head():
    """The shared per-KV-head score bounds the true max logit of every query
    head of the group (eq. (4) per head), is attained by one of them, and
    with g = 1 is the head's own bound."""
    rng = _rng(5)
    H_kv, g, S, d = 3, 4, 8, 16
    keys = rng.normal(size=(S * 12, H_kv, d)) * np.arange(1, H_kv + 1)[None, :, None]
    m, M = quest.page_summaries(keys, keys.shape[0], S)
    q = rng.normal(size=(H_kv * g, d))
    U_heads = quest.head_bounds(q, m, M)
    U = quest.kv_head_scores(U_heads, H_kv)
    for i in range(H_kv * g):
        h = i // g
        dots = (keys[:, h, :] @ q[i]).reshape(-1, S).max(axis=1)
        assert np.all(U[h] >= dots - 1e-12)
    for h in range(H_kv):
        grp = U_heads[h * g:(h + 1) * g]
        assert np.all(np.any(np.abs(grp - U[h]) == 0, axis=0))
    one = quest.kv_head_scores(U_heads[:H_kv], H_kv)
    assert np.array_equal(one, U_heads[:H_kv])


# ------------------------------------------------------------- summaries ----

@pytest.mark.parametrize("L", [1, 15, 16, 17, 33, 100])
def test_summaries_bulk_equals_replay(L):
    rng = _rng(6 + L)
    keys = rng.normal(size=(L + 5, 2, 8))
    m, M = quest.page_summaries(keys, L, 16)
    m2, M2 = quest.replay_summaries(keys, L, 16)
    assert np.array_equal(m, m2) and np.array_equal(M, M2)
    assert m.shape[0] == quest.num_pages(L, 16) == (L + 15) // 16


def test_tail_page_uses_valid_tokens_only():
    """Lengths 1, 15, 16, 17 at S = 16 (the Quest page, §1.2, tail length):
    tokens at or beyond L never enter a summary."""
    rng = _rng(7)
    keys = rng.normal(size=(32, 1, 4))
    poisoned = keys.copy()
    for L, pages, last_len in ((1, 1, 1), (15, 1, 15), (16, 1, 16), (17, 2, 1)):
        poisoned[L:] = 1e9 * np.sign(rng.normal(size=poisoned[L:].shape))
        m, M = quest.page_summaries(poisoned, L, 16)
        assert m.shape[0] == pages
        tail = keys[(pages - 1) * 16:(pages - 1) * 16 + last_len]
        assert np.array_equal(m[-1], tail.min(axis=0))
        assert np.array_equal(M[-1], tail.max(axis=0))
        poisoned[:] = keys
    m, M = quest.page_summaries(keys, 17, 16)
    assert np.array_equal(m[1], keys[16]) and np.array_equal(M[1], keys[16])


# ----------------------------------------------------------------- top-K ----

def test_topk_bruteforce_with_ties():
    rng = _rng(8)
    for _ in range(30):
        P = int(rng.integers(1, 40))
        s = rng.integers(-3, 4, size=P).astype(float)   # many exact ties
        for K in range(1, P + 3):
            sel = quest.top_k_pages(s, K)
            assert len(sel) == min(K, P) and sel == sorted(sel)
            assert len(set(sel)) == len(sel)
            out = [j for j in range(P) if j not in sel]
            for i in sel:
                for j in out:
                    assert (s[i] > s[j]) or (s[i] == s[j] and i < j)


def test_topk_all_equal_and_all_pages():
    assert quest.top_k_pages(np.zeros(10), 3) == [0, 1, 2]
    assert quest.top_k_pages(np.arange(5.0), 9) == [0, 1, 2, 3, 4]


# ------------------------------------------------- fixed local / sink pages ----

def test_local_sink_budget_worked_example():
    """[Quest] §2.2: 2048 tokens, 512 recent + 4 sinks kept, 1532 slots left,
    which pay for 95 whole pages at S = 16."""
    g = load_golden("quest_local_sink_budget.json")
    assert g["total_tokens"] - g["local_tokens"] - g["sink_tokens"] == g["remaining_tokens"]
    assert quest.quest_budget_pages(g["total_tokens"], g["local_tokens"], g["sink_tokens"],
                                    g["page_size"]) == g["quest_whole_pages"]


def test_fixed_pages_by_token_positions():
    # L = 100, S = 16: pages 0..6, the last holding tokens 96..99
    assert quest.fixed_pages(100, 16, 4, 0) == ({0}, set())
    assert quest.fixed_pages(100, 16, 16, 0) == ({0}, set())
    assert quest.fixed_pages(100, 16, 17, 0) == ({0, 1}, set())
    # the last 20 tokens are 80..99: pages 5 and 6, not only the last page
    assert quest.fixed_pages(100, 16, 0, 20) == (set(), {5, 6})
    assert quest.fixed_pages(100, 16, 0, 4) == (set(), {6})
    assert quest.fixed_pages(100, 16, 0, 5) == (set(), {5, 6})
    # windows longer than the request keep every page; none past the length
    assert quest.fixed_pages(100, 16, 1000, 1000) == (set(range(7)), set(range(7)))
    assert quest.fixed_pages(0, 16, 4, 20) == (set(), set())


def test_mixed_pages_union_bruteforce():
    """[Quest] §3.2: C = C_local | C_sink | C_quest, overlaps once; without
    fixed pages it is the plain top-K."""
    rng = _rng(21)
    for _ in range(200):
        S = int(rng.choice([1, 4, 16]))
        L = int(rng.integers(1, 300))
        P = quest.num_pages(L, S)
        s = rng.integers(-3, 4, size=P).astype(float)
        K = int(rng.integers(1, P + 3))
        sink, local = int(rng.integers(0, 40)), int(rng.integers(0, 80))
        C = quest.mixed_pages(s, K, L, S, sink, local)
        top = set(quest.top_k_pages(s, K))
        fs, fl = quest.fixed_pages(L, S, sink, local)
        assert C == sorted(set(C)) and all(0 <= j < P for j in C)
        assert top <= set(C) and fs <= set(C) and fl <= set(C)
        assert set(C) <= top | fs | fl
        assert len(C) <= min(K, P) + len(fs) + len(fl)
        # brute force over token positions for the fixed sets
        assert fs == {t // S for t in range(min(sink, L))}
        assert fl == {t // S for t in range(max(0, L - local), L)}
        assert quest.mixed_pages(s, K, L, S, 0, 0) == quest.top_k_pages(s, K)


# ------------------------------------------------------- fp8 summaries ----

def test_e4m3_directed_rounding_by_hand():
    """e4m3fn (3 fraction bits, bias 7, subnormal step 2^-9): 0.3 = 1.2 * 2^-2
    lies between 1.125 * 2^-2 and 1.25 * 2^-2."""
    assert quest.e4m3_down(0.3) == 0.28125 and quest.e4m3_up(0.3) == 0.3125
    assert quest.e4m3_down(-0.3) == -0.3125 and quest.e4m3_up(-0.3) == -0.28125
    for x in (0.0, 1.0, -1.0, 448.0, -448.0, 2.0 ** -9, 0.875 * 2.0 ** -6, 240.0):
        assert quest.e4m3_down(x) == x and quest.e4m3_up(x) == x
    assert quest.e4m3_down(1e-4) == 0.0 and quest.e4m3_up(1e-4) == 2.0 ** -9
    assert quest.e4m3_down(-1e-4) == -(2.0 ** -9) and quest.e4m3_up(-1e-4) == 0.0
    assert quest.e4m3_down(447.0) == 416.0 and quest.e4m3_up(417.0) == 448.0


def test_summary_scale_is_the_smallest_power_of_two():
    e = quest.summary_scale_exponent
    assert e(0.0) == 0 and e(448.0) == 0 and e(448.0001) == 1
    assert e(224.0) == -1 and e(224.5) == 0 and e(1.0) == -8 and e(1.75) == -8
    assert e(1.7500001) == -7 and e(65504.0) == 8


def test_fp8_summaries_are_outer_bounds():
    """[Quest] §3: min toward -inf, max toward +inf keeps eq. (4); each
    bound moves by at most one e4m3 step (1/8 of its magnitude, or the
    subnormal step 2^-9 * s near zero)."""
    rng = _rng(41)
    for _ in range(20):
        S, d = 8, 16
        keys = rng.standard_normal((40, 3, d)) * rng.choice([1e-3, 1.0, 300.0])
        keys = keys.astype(np.float16).astype(np.float64)
        m, M = quest.page_summaries(keys, 40, S)
        mh, Mh, s = quest.fp8_summaries(m, M)
        assert np.all(mh <= m) and np.all(Mh >= M)
        step = np.maximum(np.abs(np.stack([m, M])) / 8, 2.0 ** -9 * s[None, :, :, None])
        assert np.all(m - mh <= step[0]) and np.all(Mh - M <= step[1])
        assert np.all(np.maximum(np.abs(mh), np.abs(Mh)) <= 448 * s[:, :, None])
        q = rng.standard_normal((3, d))
        U = quest.head_bounds(q, m, M)
        U8 = quest.head_bounds(q, mh, Mh)
        assert np.all(U8 >= U - 1e-9)
        for h in range(3):
            for p in range(len(m)):
                toks = keys[p * S:(p + 1) * S, h]
                assert U8[h, p] >= (toks @ q[h]).max() - 1e-9


# ------------------------------------------------------------- attention ----

def _sdpa(q, k, v, scale):
    """Library attention (torch, float64, CPU) over the whole given keys."""
    qt = torch.tensor(q, dtype=torch.float64)[None, None, None, :]
    kt = torch.tensor(k, dtype=torch.float64)[None, None]
    vt = torch.tensor(v, dtype=torch.float64)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    z = (kt[0, 0] @ qt[0, 0, 0]) * scale
    return o[0, 0, 0].numpy(), float(torch.logsumexp(z, 0))


def test_all_pages_is_dense_attention():
    """The Quest page, §1.2: a budget of all pages reproduces dense paged
    attention.  Checked against torch's scaled_dot_product_attention with
    its default 1/sqrt(d) scale."""
    rng = _rng(9)
    for L, S in ((64, 4), (37, 16), (1, 16)):
        d = 16
        keys = rng.normal(size=(L, 1, d))
        values = rng.normal(size=(L, 1, d))
        q = rng.normal(size=(1, d))
        P = quest.num_pages(L, S)
        res = quest.decode_request(q, keys, values, L, S, K=P)
        o_ref, lse_ref = _sdpa(q[0], keys[:, 0], values[:, 0], 1 / math.sqrt(d))
        np.testing.assert_allclose(res["out"][0], o_ref, rtol=1e-12, atol=1e-12)
        assert abs(res["lse"][0] - lse_ref) < 1e-10


def test_causal_limit_is_inclusive():
    """Support keeps t <= c: equals dense attention over the first c+1 keys."""
    rng = _rng(10)
    L, S, d = 40, 8, 8
    keys = rng.normal(size=(L, d))
    values = rng.normal(size=(L, d))
    q = rng.normal(size=d)
    for c in (0, 7, 8, 20, 39):
        A = quest.support(range(quest.num_pages(L, S)), L, c, S)
        o, lse = quest.attend(q, keys, values, A, 1 / math.sqrt(d))
        o_ref, lse_ref = _sdpa(q, keys[:c + 1], values[:c + 1], 1 / math.sqrt(d))
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
        assert abs(lse - lse_ref) < 1e-10


def test_zero_query_gives_mean_and_single_token_gives_value():
    rng = _rng(11)
    keys = rng.normal(size=(32, 4))
    values = rng.normal(size=(32, 4))
    A = quest.support([0, 2], 32, 31, 8)
    o, _ = quest.attend(np.zeros(4), keys, values, A, 0.5)
    np.testing.assert_allclose(o, values[A].mean(axis=0), rtol=1e-12)
    A1 = quest.support([3], 25, 24, 8)             # page 3 holds only t = 24
    assert list(A1) == [24]
    o1, _ = quest.attend(rng.normal(size=4), keys, values, A1, 0.5)
    np.testing.assert_allclose(o1, values[24], rtol=1e-12)


def test_support_ignores_order_duplicates_invalid_and_empty_is_zero():
    rng = _rng(12)
    L, S, d = 50, 8, 4                              # 7 pages
    keys = rng.normal(size=(L, d))
    values = rng.normal(size=(L, d))
    q = rng.normal(size=d)
    base = quest.attend(q, keys, values, quest.support([1, 3, 6], L, L - 1, S), 0.5)
    for ids in ([6, 1, 3], [3, 3, 1, 6, 1], [1, -1, 3, 7, 6, 2**31 - 1, -7, 12]):
        o, lse = quest.attend(q, keys, values, quest.support(ids, L, L - 1, S), 0.5)
        np.testing.assert_array_equal(o, base[0])
        assert lse == base[1]
    for ids in ([], [-1, 7, 100], [5] if False else [-3]):
        o, lse = quest.attend(q, keys, values, quest.support(ids, L, L - 1, S), 0.5)
        assert np.array_equal(o, np.zeros(d)) and lse == -np.inf


def test_sparse_output_error_bound_eq7():
    """The Quest page, §1.1 eq. (6)-(7): |o - o_C| <= 2 eps V_max, with eps the
    dense probability mass outside C."""
    rng = _rng(13)
    L, S, d = 256, 16, 16
    for _ in range(10):
        keys = rng.normal(size=(L, d)) * 2
        values = rng.normal(size=(L, d))
        q = rng.normal(size=d)
        scale = 1 / math.sqrt(d)
        pages = rng.choice(L // S, size=5, replace=False)
        C = quest.support(pages, L, L - 1, S)
        o_C, _ = quest.attend(q, keys, values, C, scale)
        o, _ = quest.attend(q, keys, values, np.arange(L), scale)
        z = scale * keys @ q
        p = np.exp(z - z.max())
        p /= p.sum()
        eps = 1 - p[C].sum()
        vmax = np.linalg.norm(values, axis=1).max()
        assert np.linalg.norm(o - o_C) <= 2 * eps * vmax + 1e-12


def test_chunk_attention_per_query_matches_decode_definition():
    """A chunk query with c = L-1 and the request's own page list is exactly
    the decode result; executing as a union does not change the result."""
    case = tiny_single_head()
    keys = case.keys[0].astype(np.float64)
    values = case.values[0].astype(np.float64)
    q = case.q[0, 0].astype(np.float64)
    res = quest.decode_request(q, keys, values, 64, 4, 4)
    sets = np.array([[res["sel"][0]]])
    out, lse = quest.chunk_attention(q[None], keys, values, sets, [64], [63], 4, 1)
    np.testing.assert_array_equal(out[0], res["out"])


# ------------------------------------- chunk / GQA attention against SDPA ----
#
# [PageWeaver] eq. (1)-(2): query n, head i attends over the tokens t of KV
# head i // g whose page floor(t/S) is in its own set, with t < L_n and
# t <= c_n.  The pins below build that support as a dense boolean mask from
# per-page membership (np.repeat over the S tokens of a page, not the
# oracle's list-of-tokens route) and hand it to torch's float64
# scaled_dot_product_attention with enable_gqa=True, whose head grouping is
# the library's own (consecutive query heads share a KV head).


def _membership_mask(sets, L, c, S, T, g):
    """Dense mask [N][H_q][T]: page membership expanded over its S tokens,
    then the length and causal limits; per KV head, repeated g times over
    the query heads that read it."""
    N, H_kv = len(sets), len(sets[0])
    mask = np.zeros((N, H_kv, T), dtype=bool)
    n_pages = -(-T // S)
    t = np.arange(T)
    for n in range(N):
        for h in range(H_kv):
            on = np.zeros(n_pages, dtype=bool)
            for p in sets[n][h]:
                if 0 <= p < n_pages and p * S < L[n]:
                    on[p] = True
            mask[n, h] = np.repeat(on, S)[:T] & (t < L[n]) & (t <= c[n])
    return np.repeat(mask, g, axis=1)


def _sdpa_masked(q, keys, values, mask, scale):
    """torch SDPA (float64, CPU, enable_gqa) of q [N][H_q][d] over keys /
    values [T][H_kv][d] with mask [N][H_q][T]; rows with an empty mask come
    back as NaN and are the caller's to skip.  Also the log-sum-exp of the
    masked logits (KV heads expanded by repeat_interleave)."""
    qt = torch.tensor(q).permute(1, 0, 2)[None]            # [1][H_q][N][d]
    kt = torch.tensor(keys).permute(1, 0, 2)[None]         # [1][H_kv][T][d]
    vt = torch.tensor(values).permute(1, 0, 2)[None]
    mt = torch.tensor(mask).permute(1, 0, 2)[None]         # [1][H_q][N][T]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt,
                                                         scale=scale, enable_gqa=True)
    g = q.shape[1] // keys.shape[1]
    z = (qt @ torch.repeat_interleave(kt, g, dim=1).transpose(-1, -2)) * scale
    z = z.masked_fill(~mt, -math.inf)
    return o[0].permute(1, 0, 2).numpy(), torch.logsumexp(z, -1)[0].T.numpy()


def _chunk_case(seed, g, H_kv=2, d=8, S=4, T=40):
    """Queries with their own lengths and causal limits inside pages, sets
    with duplicates, invalid IDs and pages past the limit, one empty set."""
    rng = _rng(seed)
    keys = rng.normal(size=(T, H_kv, d)) * np.arange(1, H_kv + 1)[None, :, None]
    values = rng.normal(size=(T, H_kv, d)) + np.arange(H_kv)[None, :, None]
    L = [40, 37, 40, 33, 29, 40]
    c = [39, 30, 21, 13, 28, 5]          # limits inside pages (S = 4)
    N = len(L)
    q = rng.normal(size=(N, H_kv * g, d))
    P = -(-T // S)
    sets = []
    for n in range(N):
        row = []
        for h in range(H_kv):
            ids = list(rng.choice(P, size=5, replace=False))
            ids += [ids[0], -1, P, 2 ** 31 - 1]       # duplicate and invalid IDs
            ids.append(c[n] // S)                     # the page the limit falls in
            row.append(ids)
        sets.append(row)
    sets[4][1] = [-3, P + 1]                          # empty support for KV head 1
    return q, keys, values, sets, L, c, S


def _pin_chunk_against_sdpa(qmod, g):
    q, keys, values, sets, L, c, S = _chunk_case(40 + g, g)
    scale = 1 / math.sqrt(q.shape[2])
    out, lse = qmod.chunk_attention(q, keys, values, sets, L, c, S, g, scale=scale)
    mask = _membership_mask(sets, L, c, S, keys.shape[0], g)
    o_ref, lse_ref = _sdpa_masked(q, keys, values, mask, scale)
    empty = ~mask.any(axis=2)
    assert empty.any() and not empty.all()
    np.testing.assert_allclose(out[~empty], o_ref[~empty], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[~empty], lse_ref[~empty], rtol=1e-12, atol=1e-12)
    assert np.all(out[empty] == 0) and np.all(np.isneginf(lse[empty]))


@pytest.mark.parametrize("g", [1, 2, 4])
def test_chunk_attention_equals_masked_sdpa(g):
    """Multi-query chunk ([PageWeaver] eq. (1)-(2)) with per-query lengths,
    causal limits inside pages and query head i on KV head i // g."""
    _pin_chunk_against_sdpa(quest, g)


def _pin_decode_gqa_against_sdpa(qmod, g):
    """decode_request at g > 1 on given lists and on its own top-K lists:
    c = L - 1, query head i on KV head i // g."""
    rng = _rng(50 + g)
    H_kv, d, S, L = 3, 8, 4, 45
    keys = rng.normal(size=(L, H_kv, d)) * np.arange(1, H_kv + 1)[None, :, None]
    values = rng.normal(size=(L, H_kv, d)) + 2.0 * np.arange(H_kv)[None, :, None]
    q = rng.normal(size=(H_kv * g, d))
    scale = 1 / math.sqrt(d)
    P = quest.num_pages(L, S)
    given = [[0, 3, 3, -1, P - 1], [5, 7, P], [1, 2, 4, 6, 8, 10]]
    for ids in (given, None):
        res = qmod.decode_request(q, keys, values, L, S, 4, scale=scale, page_ids=ids)
        lists = res["sel"] if ids is None else ids
        mask = _membership_mask([lists], [L], [L - 1], S, L, g)
        o_ref, lse_ref = _sdpa_masked(q[None], keys, values, mask, scale)
        np.testing.assert_allclose(res["out"], o_ref[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["lse"], lse_ref[0], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("g", [2, 4])
def test_decode_request_gqa_equals_masked_sdpa(g):
    _pin_decode_gqa_against_sdpa(quest, g)


def _planted(old, new, where):
    """A copy of oracle.quest with one line of function `where` replaced."""
    import types
    src = open(quest.__file__).read()
    head, sep, body = src.partition(f"def {where}(")
    first, nxt, rest = body.partition("\ndef ")
    assert sep and old in first, (where, old)
    mod = types.ModuleType("quest_planted")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(head + sep + first.replace(old, new) + nxt + rest, "quest_planted", "exec"),
         mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new,where,pin", [
    ("support(sets[n][h], L[n], c[n], S)", "support(sets[n][h], L[n], L[n] - 1, S)",
     "chunk_attention", "chunk"),                                  # ignores c_n
    ("h = i // g", "h = i % keys.shape[1]", "chunk_attention", "chunk"),  # wrong head map
    ("h = i // g", "h = i % H_kv", "decode_request", "decode"),
    ("support(lists[h], L, L - 1, S)", "support(lists[h], L, L - 2, S)",
     "decode_request", "decode"),                                   # exclusive limit
])
def test_planted_attention_mistakes_fail_a_pin(old, new, where, pin):
    """Each mistake planted in a copy of the oracle fails the SDPA pins."""
    mod = _planted(old, new, where)
    fn = _pin_chunk_against_sdpa if pin == "chunk" else _pin_decode_gqa_against_sdpa
    failed = 0
    for g in (2, 4):
        try:
            fn(mod, g)
        except AssertionError:
            failed += 1
    assert failed == 2, f"planted '{new}' in {where} passed a pin"


def test_workload_cases_are_well_formed():
    c1 = tiny_single_head()
    assert c1.keys[0].shape == (64, 1, 16) and c1.K == 4
    assert sorted(c1.pages[0].tolist()) == sorted(set(c1.pages[0].tolist()))
    c2 = llama2_7b_layer(L=256, H=2)
    assert c2.keys[0].dtype == np.float16 and c2.keys[0].shape == (256, 2, 128)
    c3 = batched_gqa_append(B=2, L_min=40, L_max=70, steps=3)
    assert all(k.shape[0] == L + 3 for k, L in zip(c3.keys, c3.seq_lens))
    flat = np.concatenate(c3.pages)
    assert len(set(flat.tolist())) == len(flat) and flat.max() < c3.num_pool_pages


# ----------------------------------------------------------- NEXT-4 pins ----

@pytest.mark.parametrize("L_old,L_new", [(37, 33), (37, 32), (40, 17), (17, 16), (5, 1),
                                         (64, 63), (30, 29)])
def test_rollback_rescan_equals_summaries_of_the_kept_tokens(L_old, L_new):
    """Cutting the cache back and rescanning the tail page gives the summaries
    the kept tokens define ([Quest] §1.1 eq. (1) over t < L_new)."""
    S = 8
    keys = _rng(70 + L_old + L_new).standard_normal((L_old, 3, 5))
    m, M = quest.page_summaries(keys, L_old, S)
    m2, M2 = quest.rollback_summaries(m, M, keys, L_new, S)
    me, Me = quest.page_summaries(keys, L_new, S)
    assert np.array_equal(m2, me) and np.array_equal(M2, Me)


def test_rollback_without_rescan_keeps_a_revoked_extreme():
    """The case [Quest] §3 warns of: the revoked token held the page's extreme,
    so the old min/max would keep covering a point that no longer exists."""
    keys = np.array([[1.0, 0.0], [2.0, 1.0], [9.0, -5.0]])[:, None, :]
    m, M = quest.page_summaries(keys, 3, S=4)
    assert M[0, 0].tolist() == [9.0, 1.0] and m[0, 0].tolist() == [1.0, -5.0]
    m2, M2 = quest.rollback_summaries(m, M, keys, 2, S=4)
    assert M2[0, 0].tolist() == [2.0, 1.0] and m2[0, 0].tolist() == [1.0, 0.0]


def _spec_case(seed, L, gamma, S=4, H_q=4, H_kv=2, d=8):
    r = _rng(seed)
    keys = r.standard_normal((L, H_kv, d))
    values = r.standard_normal((L, H_kv, d))
    qb = r.standard_normal((gamma, H_q, d))
    return keys, values, qb


def test_speculative_single_position_is_a_decode_step():
    keys, values, qb = _spec_case(80, L=37, gamma=1)
    res = quest.speculative_positions(qb, keys, values, 37, 4, K=3)
    ref = quest.decode_request(qb[0], keys, values, 37, 4, 3)
    assert res[0]["sel"] == ref["sel"]
    assert np.allclose(res[0]["out"], ref["out"], rtol=0, atol=1e-12)


def test_speculative_position_closing_a_page_is_a_decode_step_on_the_cut_cache():
    """Draft positions 12..16 with S = 4: position 3 (c = 15) closes page 3, so
    the pages it scores hold exactly the tokens it sees and its result is the
    decode step of the cache cut after token 15; position 0 (c = 12) scores
    page 3 with the later drafts inside its bound and may not see them."""
    L, gamma, S, K = 17, 5, 4, 2
    keys, values, qb = _spec_case(81, L, gamma, S=S)
    res = quest.speculative_positions(qb, keys, values, L, S, K)
    assert [r["L"] for r in res] == [13, 14, 15, 16, 17]
    ref = quest.decode_request(qb[3], keys[:16], values[:16], 16, S, K)
    assert res[3]["sel"] == ref["sel"]
    assert np.allclose(res[3]["out"], ref["out"], rtol=0, atol=1e-12)
    assert res[0]["U"].shape[1] == 4
    for r in res:
        c = r["L"] - 1
        for h, lst in enumerate(r["sel"]):
            assert all(p * S <= c for p in lst)       # only pages it may see


def test_speculative_positions_do_not_share_one_set():
    """Each position ranks with its own query: with distinct queries the sets
    differ from the first position's, and every position equals attention
    over its own top-K support."""
    L, gamma, S, K = 64, 4, 4, 3
    keys, values, qb = _spec_case(82, L, gamma, S=S)
    res = quest.speculative_positions(qb, keys, values, L, S, K)
    assert any(r["sel"] != res[0]["sel"] for r in res[1:])
    m, M = quest.page_summaries(keys, L, S)
    for i, r in enumerate(res):
        c = L - gamma + i
        U = quest.kv_head_scores(quest.head_bounds(qb[i], m, M), 2)[:, :quest.num_pages(c + 1, S)]
        assert np.array_equal(U, r["U"])
        for qi in range(qb.shape[1]):
            A = quest.support(r["sel"][qi // 2], L, c, S)
            o, _ = quest.attend(qb[i][qi], keys[:, qi // 2], values[:, qi // 2], A,
                                1 / math.sqrt(qb.shape[2]))
            assert np.allclose(o, r["out"][qi], rtol=0, atol=1e-12)


def test_branch_and_bound_four_page_example():
    g = load_golden("quest_four_pages_bnb.json")
    names = g["pages"]
    page_logits = [[(float(v), j)] for j, v in enumerate(g["true_max"])]
    read, top, tau = quest.branch_and_bound(g["bound"], page_logits, g["R"])
    assert [names[p] for p in read] == g["read_order"]
    assert [names[t] for _, t in top] == g["top"]
    assert tau == g["tau_final"]


def test_branch_and_bound_keeps_reading_at_an_equal_bound():
    """A page whose bound equals tau_R may hold a token tied with it at a lower
    token index, so only a bound strictly below tau_R stops the search."""
    page_logits = [[(5.0, 0)], [(5.0, 1)]]
    read, top, _ = quest.branch_and_bound([5.0, 6.0], page_logits, 1)
    assert read == [1, 0] and top == [(5.0, 0)]


@pytest.mark.parametrize("seed,R,spread", [(90, 1, 1.0), (91, 8, 1.0), (92, 50, 1.0),
                                           (93, 8, 6.0), (94, 200, 1.0)])
def test_branch_and_bound_is_the_exact_top_r(seed, R, spread):
    """The certificate's claim: the tokens found equal the brute-force top R
    over all tokens, and the first unread page's bound is below tau_R."""
    r = _rng(seed)
    L, S, d = 203, 8, 16
    keys = r.standard_normal((L, 1, d))
    q = r.standard_normal(d)
    # a few aligned tokens make the bounds tight for the top pages
    hot = r.choice(L, size=5, replace=False)
    keys[hot, 0] += spread * q / np.linalg.norm(q) * math.sqrt(d)
    m, M = quest.page_summaries(keys, L, S)
    read, top, tau = quest.exact_top_r(q, keys[:, 0], L, S, R, m[:, 0], M[:, 0])
    assert top == quest.brute_top_r(q, keys[:, 0], L, R)
    P = quest.num_pages(L, S)
    bounds = np.maximum(q * m[:, 0], q * M[:, 0]).sum(axis=1)
    unread = [p for p in range(P) if p not in read]
    if unread:
        assert max(bounds[p] for p in unread) < tau
    assert len(set(read)) == len(read) <= P
    if spread > 1.0 and R == 8:
        assert len(read) < P                          # tight bounds stop early


def test_branch_and_bound_with_r_at_least_the_tokens_reads_everything():
    r = _rng(95)
    L, S = 21, 4
    keys = r.standard_normal((L, 1, 4))
    q = r.standard_normal(4)
    m, M = quest.page_summaries(keys, L, S)
    read, top, _ = quest.exact_top_r(q, keys[:, 0], L, S, 30, m[:, 0], M[:, 0])
    assert sorted(read) == list(range(quest.num_pages(L, S)))
    assert [t for _, t in top] == [t for _, t in quest.brute_top_r(q, keys[:, 0], L, L)]


def test_kv_quantisation_is_per_head_and_in_float32():
    """PageWeaver SS2UKVF2 (FP8 E4M3 K/V with a per-KV-head scale): code of
    x / scale[h]; a value at the head's amax lands on 448 whatever the head,
    and the quotient is the float32 one (a float64 quotient rounds a value
    just below a code midpoint down where float32 rounds it to the midpoint
    and then to the even code)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 3, 16)).astype(np.float32)
    scale = (np.abs(x).max(axis=(0, 2)) / np.float32(448.0)).astype(np.float32)
    codes = quest.quantize_kv_e4m3(x, scale)
    vals = formats.decode_e4m3fn(codes)
    for h in range(3):
        at = np.unravel_index(np.abs(x[:, h]).argmax(), x[:, h].shape)
        assert abs(vals[at[0], h, at[1]]) == 448.0
    # each element is the nearest code value to its float32 quotient
    q = (x / scale[None, :, None]).astype(np.float64)
    grid = np.unique(formats.decode_e4m3fn(np.arange(256, dtype=np.uint8)))
    grid = grid[np.isfinite(grid)]
    nearest = np.abs(q[..., None] - grid).min(axis=-1)
    assert np.allclose(np.abs(vals - q), nearest, rtol=0, atol=0)
    # float32 vs float64 quotient: for these float32 values x / s is
    # 1.18749999... (just below the midpoint of 1.125 and 1.25) in float64,
    # but exactly the midpoint 1.1875 in float32, which ties to the even code
    # 1.25 (0x3A) instead of 1.125 (0x39)
    s = np.float32(0.9505132436752319)
    xv = np.float32(1.1287344694137573)
    assert float(xv) / float(s) < 1.1875 and float(xv / s) == 1.1875
    assert quest.quantize_kv_e4m3(np.full((1, 1, 1), xv, np.float32), [s])[0, 0, 0] == 0x3A


def test_chunk_workload_codes_are_the_oracle_quantisation():
    """The fp8 chunk workload's stored codes (its input generator casts the
    float32 quotients with torch) equal the oracle's quantisation of the same
    float32 K/V with the same per-head scales, code for code."""
    from workloads import multiquery_chunk
    case = multiquery_chunk(seed=9, L=700, S=32, N=5, H_q=8, H_kv=2, kq=6, keep=4)
    for codes, src, scale in ((case.keys, case.keys_src, case.k_scale),
                              (case.values, case.values_src, case.v_scale)):
        ref = quest.quantize_kv_e4m3(src, scale)
        assert np.array_equal(formats.decode_e4m3fn(codes), formats.decode_e4m3fn(ref))
