"""Per-kernel GPU parity against the oracle: each kernel gets the oracle's own
inputs (summaries from the same keys, identical fp32 scores, the oracle's
page lists) and is compared element by element."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import quest
from tests.gpu_util import (ATTN_TOL, assert_attn_close, assert_scores_close,
                            check_selection, out_to_numpy, say, score_denominator)
from workloads import (tiny_single_head, llama2_7b_layer, batched_gqa_append, stress_long_context, corrupt_lists,
                       figure2_case, worked_example_case)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qas():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import query_aware_sparse_amd
    return query_aware_sparse_amd


def _stage(qas, case, lengths=None):
    from query_aware_sparse_amd.staging import PagedCache, prefill
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype)
    db = prefill(pc, case, lengths)
    return pc, db


def _q(case, step=-1):
    from query_aware_sparse_amd.staging import to_device
    return to_device(case.q[step + 1], case.q_dtype)


SCORE_CASES = {
    "worked-example": lambda: worked_example_case(),
    "worked-example-b": lambda: worked_example_case(second_set=True),
    "figure2": lambda: figure2_case(),
    "tiny_single_head": lambda: tiny_single_head(),
    "llama2_7b_layer-small-shuffled": lambda: llama2_7b_layer(L=3001, H=4, identity_table=False),
    "batched_gqa_append-small-gqa": lambda: batched_gqa_append(B=3, L_min=300, L_max=2000, steps=0),
    "stress_long_context-small": lambda: stress_long_context(B=2, L=4096, H_q=8, H_kv=2),
    "d64-bf16-g8": lambda: batched_gqa_append(B=2, L_min=100, L_max=700, H_q=16, H_kv=2, d=64,
                                   S=32, steps=0),
    # matrix-core scores (d=128, 16-bit, g >= 2): g=8 joins two output
    # quads; 2 KV heads divide the kernel's 4 waves (one head per wave),
    # 3 and 16 do not, so the query operands change from task to task and
    # tasks past the end are dropped
    "d128-f16-g8": lambda: stress_long_context(B=2, L=3001, H_q=16, H_kv=2),
    "d128-bf16-g2-h3": lambda: batched_gqa_append(B=3, L_min=200, L_max=1700, H_q=6, H_kv=3,
                                                  steps=0),
    "d128-bf16-g2-h16": lambda: batched_gqa_append(B=2, L_min=40, L_max=900, H_q=32, H_kv=16,
                                                   steps=0),
}


@pytest.mark.parametrize("name", list(SCORE_CASES))
def test_summaries_and_scores(qas, name):
    case = SCORE_CASES[name]()
    say(f"[scores] {name}: B={case.B} H={case.H_q}/{case.H_kv} d={case.d} S={case.S}")
    pc, db = _stage(qas, case)
    q = _q(case)
    scores = torch.full((db.total_pages * case.H_kv,), float("nan"), device="cuda")
    qas.qas_score_pages(pc.cache, db.batch, q, scores)
    torch.cuda.synchronize()
    got = scores.cpu().numpy().astype(np.float64)
    summ = pc.summary.float().cpu().numpy().astype(np.float64)
    ref = oracle.run_decode(case)
    for r in range(case.B):
        res = ref[r]
        P = len(res["U"][0])
        phys = case.pages[r][:P]
        # summaries are exact (min/max of stored values)
        assert np.array_equal(summ[phys, :, 0, :], res["m"]), f"min summary r={r}"
        assert np.array_equal(summ[phys, :, 1, :], res["M"]), f"max summary r={r}"
        base = db.indptr_host[r] * case.H_kv
        q_heads = oracle.decode(case.q[0][r], case.q_dtype)
        denom = score_denominator(q_heads, res["m"], res["M"], case.g)
        for h in range(case.H_kv):
            row = got[base + h * P: base + (h + 1) * P]
            assert_scores_close(row, res["U"][h], denom[h], f"{name} r={r} h={h}")


def _topk_rows(rng, B, H, maxP):
    lens = rng.integers(1, maxP + 1, size=B)
    return lens


def _topk_scores(kind, total, rng):
    """Seeded score rows that exercise every branch of a histogram select."""
    if kind == "ints":
        return rng.integers(-20, 20, size=total).astype(np.float32)       # heavy ties
    if kind == "normal":
        return rng.standard_normal(total).astype(np.float32)
    if kind == "zeros":                                                    # -0 == +0
        return np.where(rng.random(total) < 0.5, np.float32(0.0), np.float32(-0.0))
    if kind == "cluster":
        # most values within a few ulps of 1000, the rest spread wide: the
        # crossing bin is narrowed several times
        ulp = np.spacing(np.float32(1000))
        c = np.float32(1000) + rng.integers(0, 40, size=total).astype(np.float32) * ulp
        wide = (rng.standard_normal(total) * 5000).astype(np.float32)
        return np.where(rng.random(total) < 0.85, c, wide).astype(np.float32)
    if kind == "huge":
        # a range beyond fp32 (and -inf entries): binning by order keys; the
        # samples past the fp32 range become +-inf on purpose
        with np.errstate(over="ignore"):
            x = (rng.standard_normal(total) * 1e38).astype(np.float32)
        pick = rng.random(total)
        x[pick < 0.05] = -np.inf
        x[(pick >= 0.05) & (pick < 0.1)] = np.float32(3.4e38)
        x[(pick >= 0.1) & (pick < 0.15)] = np.float32(-3.4e38)
        return x
    if kind == "subnormal":
        # a range far below any fp32 scale: binning by order keys
        return (rng.integers(0, 3000, size=total) * np.float32(1e-45)).astype(np.float32)
    raise ValueError(kind)


TOPK_KINDS = ["ints", "normal", "zeros", "cluster", "huge", "subnormal"]
TOPK_ROWS = {"short": [1, 300, 2048, 1000, 77], "long": [4097, 16384, 9000],
             # around the 512 candidates ranked directly from LDS
             "edge": [512, 511, 513, 65, 64]}


@pytest.mark.parametrize("rows", list(TOPK_ROWS))
@pytest.mark.parametrize("K", [1, 4, 64, 256, 4096])
def test_topk_exact_on_identical_scores(qas, K, rows):
    """The oracle's top-K on the very fp32 scores the kernel reads: exact,
    up to the longest row the kernel takes (16384 pages)."""
    from query_aware_sparse_amd.staging import DeviceBatch
    rng = np.random.default_rng(100 + K + 7 * len(rows))
    H, S = 3, 16
    P = TOPK_ROWS[rows]
    B = len(P)
    lens = [p * S - int(rng.integers(0, S)) for p in P]
    pages = [np.arange(p, dtype=np.int32) for p in P]
    db = DeviceBatch(lens, pages, S)
    total = db.total_pages * H
    for kind in TOPK_KINDS:
        s = _topk_scores(kind, total, rng)
        say(f"[topk] K={K} rows={rows} kind={kind}")
        scores = torch.from_numpy(s).cuda()
        sel = torch.full((B, H, K), 12345, dtype=torch.int32, device="cuda")
        cnt = torch.zeros((B, H), dtype=torch.int32, device="cuda")
        qas.qas_topk_pages(scores, db.batch, H, S, K, sel, cnt)
        torch.cuda.synchronize()
        sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
        for r in range(B):
            base = db.indptr_host[r] * H
            for h in range(H):
                row = s[base + h * P[r]: base + (h + 1) * P[r]].astype(np.float64)
                ref = quest.top_k_pages(row, K)
                take = min(K, P[r])
                assert cnt_h[r, h] == take
                assert list(sel_h[r, h, :take]) == ref, (kind, r, h)
                assert np.all(sel_h[r, h, take:] == -1)


@pytest.mark.parametrize("L", [1, 15, 16, 17, 33, 250])
def test_append_decode_steps_and_boundaries(qas, L):
    """Prefill L tokens, then decode-append 20 single tokens (crossing page
    boundaries); summaries stay exactly the oracle's after every step."""
    from query_aware_sparse_amd.staging import DeviceBatch, to_device
    case = batched_gqa_append(B=2, L_min=L, L_max=L, H_q=4, H_kv=2, d=128, S=16, steps=20)
    pc, _ = _stage(qas, case)
    for s in range(case.steps):
        lengths = case.lengths(s)
        db = DeviceBatch(lengths, case.pages, case.S)
        k_new = np.stack([case.keys[r][lengths[r] - 1] for r in range(case.B)])
        v_new = np.stack([case.values[r][lengths[r] - 1] for r in range(case.B)])
        kn, vn = to_device(k_new, "bf16"), to_device(v_new, "bf16")
        out = torch.empty((case.B, case.H_q, case.d), dtype=torch.bfloat16, device="cuda")
        ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, pc.cache, db.batch, case.H_q, case.K)
        qas.qas_decode_layer(pc.cache, db.batch, _q(case, s), case.K, case.sm_scale, out,
                             None, ws, k_new=kn, v_new=vn)
    torch.cuda.synchronize()
    summ = pc.summary.float().cpu().numpy()
    kp = pc.k_pool.float().cpu().numpy()
    lengths = case.lengths(case.steps - 1)
    for r in range(case.B):
        keys = oracle.decode(case.keys[r][:lengths[r]], "bf16")
        m, M = quest.page_summaries(keys, int(lengths[r]), case.S)
        m2, M2 = quest.replay_summaries(keys, int(lengths[r]), case.S)
        assert np.array_equal(m, m2)
        phys = case.pages[r][:len(m)]
        assert np.array_equal(summ[phys, :, 0], m) and np.array_equal(summ[phys, :, 1], M)
        # the pool holds the appended rows at their slots
        t = int(lengths[r]) - 1
        assert np.array_equal(kp[case.pages[r][t // case.S], :, t % case.S], keys[t])


def test_recycled_page_summary_equals_fresh(qas):
    """A physical page whose summary holds stale extremes from a previous
    owner, reused by a new request, ends with the same summary as a fresh
    page (the Quest page, §3, page recycling)."""
    from query_aware_sparse_amd.staging import DeviceBatch, PagedCache, to_device
    case = llama2_7b_layer(L=40, H=2, d=128, identity_table=False)
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype)
    pc.summary.fill_(1000.0)                     # stale values of a former owner
    pc.summary[:, :, 0].fill_(-1000.0)
    before = DeviceBatch([0], case.pages, case.S)
    full = DeviceBatch([40], case.pages, case.S)
    batch = qas.make_batch(before.seq_lens, full.page_indptr, full.page_indices,
                           full.total_pages, full.max_pages)
    new_indptr = torch.tensor([0, 40], dtype=torch.int32, device="cuda")
    qas.qas_append(pc.cache, batch, new_indptr, 40, 40, to_device(case.keys[0], "f16"),
                   to_device(case.values[0], "f16"))
    torch.cuda.synchronize()
    keys = oracle.decode(case.keys[0], "f16")
    m, M = quest.page_summaries(keys, 40, case.S)
    summ = pc.summary.float().cpu().numpy()
    phys = case.pages[0][:3]
    assert np.array_equal(summ[phys, :, 0], m) and np.array_equal(summ[phys, :, 1], M)


def _sparse_decode(qas, case, pc, db, lists, step=-1):
    B, H, kk = lists.shape
    sel = torch.from_numpy(np.ascontiguousarray(lists, np.int32)).cuda()
    q = _q(case, step)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, case.H_q), float("nan"), device="cuda")
    ws = qas.make_workspace(qas.QAS_OP_SPARSE_DECODE, pc.cache, db.batch, case.H_q, kk)
    qas.qas_sparse_decode(pc.cache, db.batch, q, sel, kk, case.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    return out_to_numpy(out), lse.cpu().numpy().astype(np.float64)


SPARSE_CASES = {
    "tiny_single_head": lambda: tiny_single_head(),
    "llama2_7b_layer-small": lambda: llama2_7b_layer(L=5000, H=4, K=40),
    "batched_gqa_append-small": lambda: batched_gqa_append(B=3, L_min=900, L_max=3000, steps=0, K=37),
    "stress_long_context-small": lambda: stress_long_context(B=4, L=6000, H_q=8, H_kv=2, K=12),
    # logits on matrix cores (16-bit K/V, d=128, g = 4 or 8, S >= 16), with
    # partial last pages and tiles past a page's tokens
    "g8-f16-S32": lambda: stress_long_context(B=3, L=5001, H_q=16, H_kv=2, K=14),
    "g8-bf16-S16": lambda: batched_gqa_append(B=3, L_min=700, L_max=2600, H_q=16, H_kv=2,
                                              steps=0, K=29),
    "g4-bf16-S64": lambda: batched_gqa_append(B=2, L_min=1500, L_max=4000, H_q=8, H_kv=2, S=64,
                                              steps=0, K=9),
    "g4-f16-S256": lambda: stress_long_context(B=2, L=3001, H_q=8, H_kv=2, S=256, K=3),
}


@pytest.mark.parametrize("name", list(SPARSE_CASES))
def test_sparse_decode_on_corrupted_lists(qas, name):
    """Attention over the oracle's own top-K lists after seeded corruption:
    duplicates, invalid IDs (-1, -7, P, P+5, INT32_MAX), shuffled order and
    fully invalid rows (zero output, lse = -inf)."""
    case = SPARSE_CASES[name]()
    say(f"[sparse] {name}")
    pc, db = _stage(qas, case)
    ref = oracle.run_decode(case)
    lists = np.full((case.B, case.H_kv, case.K), -1, dtype=np.int64)
    for r in range(case.B):
        for h in range(case.H_kv):
            s = ref[r]["sel"][h]
            lists[r, h, :len(s)] = s
    P = [len(ref[r]["U"][0]) for r in range(case.B)]
    bad, cat = corrupt_lists(lists, P, seed=7, n_slots=max(1, case.K // 5))
    rng = np.random.default_rng(3)
    for r in range(case.B):
        for h in range(case.H_kv):
            bad[r, h] = bad[r, h, rng.permutation(case.K)]
    got, lse = _sparse_decode(qas, case, pc, db, bad)
    ref2 = oracle.run_decode(case, page_ids=bad)
    for r in range(case.B):
        assert_attn_close(got[r], ref2[r]["out"], case.kv_dtype, f"{name} r={r}")
        fin = np.isfinite(ref2[r]["lse"])
        assert np.array_equal(np.isfinite(lse[r]), fin)
        assert np.allclose(lse[r][fin], ref2[r]["lse"][fin], atol=1e-4, rtol=1e-5)
        for h in range(case.H_kv):
            if cat[r, h] == 4:
                assert np.all(got[r, h * case.g:(h + 1) * case.g] == 0.0)


def test_dense_fallback_all_pages(qas):
    """K = all pages reproduces dense paged attention (the Quest page, §1.2)."""
    case = llama2_7b_layer(L=2000, H=2, K=10000)
    pc, db = _stage(qas, case)
    q = _q(case)
    out = torch.empty_like(q)
    lse = torch.empty((1, case.H_q), device="cuda")
    ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, pc.cache, db.batch, case.H_q, case.K)
    sel = torch.empty((1, case.H_kv, case.K), dtype=torch.int32, device="cuda")
    qas.qas_decode_layer(pc.cache, db.batch, q, case.K, case.sm_scale, out, lse, ws,
                         sel_out=sel)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy()[0, :, :125], np.tile(np.arange(125), (2, 1)))
    keys = oracle.decode(case.keys[0], "f16")
    vals = oracle.decode(case.values[0], "f16")
    qh = oracle.decode(case.q[0][0], "f16")
    for i in range(case.H_q):
        o, l = quest.attend(qh[i], keys[:, i], vals[:, i], np.arange(2000), case.sm_scale)
        assert_attn_close(out_to_numpy(out)[0, i], o, "f16", f"head {i}")


def test_empty_and_zero_length_requests(qas):
    """A zero-length request in a ragged batch gets no pages, no selection and
    a zero output; its neighbours are unaffected."""
    from query_aware_sparse_amd.staging import DeviceBatch, PagedCache, prefill
    case = batched_gqa_append(B=3, L_min=100, L_max=400, steps=0, K=8)
    case.seq_lens[1] = 0
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype)
    db = prefill(pc, case)
    q = _q(case)
    out = torch.full_like(q, float("nan"))
    lse = torch.empty((case.B, case.H_q), device="cuda")
    sel = torch.empty((case.B, case.H_kv, case.K), dtype=torch.int32, device="cuda")
    ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, pc.cache, db.batch, case.H_q, case.K)
    qas.qas_decode_layer(pc.cache, db.batch, q, case.K, case.sm_scale, out, lse, ws,
                         sel_out=sel)
    torch.cuda.synchronize()
    got = out_to_numpy(out)
    assert np.all(got[1] == 0) and np.all(np.isneginf(lse.cpu().numpy()[1]))
    assert np.all(sel.cpu().numpy()[1] == -1)
    ref = oracle.run_decode(case, requests=[0, 2])
    for r, res in zip((0, 2), ref):
        assert_attn_close(got[r], res["out"], "bf16", f"r={r}")


def test_longest_row(qas):
    """A row of 16384 pages, the longest the decode layer takes."""
    case = tiny_single_head(L=65536, S=4, K=300)            # 16384 pages, fp32, d=16
    pc, db = _stage(qas, case)
    q = _q(case)
    out = torch.empty_like(q)
    lse = torch.empty((1, 1), device="cuda")
    sel = torch.empty((1, 1, case.K), dtype=torch.int32, device="cuda")
    ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, pc.cache, db.batch, case.H_q, case.K)
    qas.qas_decode_layer(pc.cache, db.batch, q, case.K, case.sm_scale, out, lse, ws,
                         sel_out=sel)
    torch.cuda.synchronize()
    ref = oracle.run_decode(case)[0]
    from tests.gpu_util import check_selection
    got_sel = sel.cpu().numpy()
    if not check_selection(got_sel[0, 0], ref["U"][0], case.K):
        # near tie: the oracle's attention over the GPU's own set
        ref = oracle.run_decode(case, page_ids=got_sel.astype(np.int64))[0]
    assert_attn_close(out_to_numpy(out)[0], ref["out"], "f32", "long row")
    np.testing.assert_allclose(lse.cpu().numpy()[0], ref["lse"], rtol=1e-5, atol=1e-4)
