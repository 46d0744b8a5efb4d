"""GPU parity of the e4m3 summary copy (the Quest page, §3 on the summary
dtype: the min rounded toward -inf, the max toward +inf, one power-of-two
scale per (page, KV head)).  Codes and scales written by the bulk append and
by the decode-layer append equal the oracle's outward quantisation of the
exact summaries value for value; scores taken from the copy match the
oracle's bounds over the copy and are never below the exact bounds; the
decode layer selects on them and attends over what it selected."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quest
from oracle.formats import decode_e4m3fn
from tests.gpu_util import (assert_attn_close, assert_scores_close, check_selection,
                            out_to_numpy, say, score_denominator)
from workloads import batched_gqa_append, llama2_7b_layer, tiny_single_head

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qas():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import query_aware_sparse_amd
    return query_aware_sparse_amd


def _stage8(case, lengths=None):
    from query_aware_sparse_amd.staging import PagedCache, prefill
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype,
                    fp8_summaries=True)
    db = prefill(pc, case, lengths)
    return pc, db


def _copy_values(pc):
    """The copy as values: scale * e4m3 value of each code, [pool][H][2][d]."""
    codes = pc.summary_fp8.cpu().numpy()
    scale = pc.summary_fp8_scale.cpu().numpy().astype(np.float64)
    return decode_e4m3fn(codes) * scale[:, :, None, None], scale


def _oracle_copy(case, r, L):
    keys = oracle.decode(case.keys[r][:L], case.kv_dtype)
    m, M = quest.page_summaries(keys, L, case.S)
    return (m, M) + quest.fp8_summaries(m, M)


CASES = {
    "llama2_7b_layer-small": lambda: llama2_7b_layer(L=3001, H=4, K=40),
    "batched_gqa-bf16-g4": lambda: batched_gqa_append(B=3, L_min=300, L_max=2000, steps=0),
    "tiny_single_head-f32": lambda: tiny_single_head(L=301, K=9),
    "d64-bf16-g8": lambda: batched_gqa_append(B=2, L_min=100, L_max=700, H_q=16, H_kv=2, d=64,
                                              S=32, steps=0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_copy_and_scores(qas, name):
    case = CASES[name]()
    say(f"[fp8 summary] {name}: B={case.B} H={case.H_q}/{case.H_kv} d={case.d} S={case.S}")
    pc, db = _stage8(case)
    vals, scale = _copy_values(pc)
    from query_aware_sparse_amd.staging import to_device
    q = to_device(case.q[0], case.q_dtype)
    scores = torch.full((db.total_pages * case.H_kv,), float("nan"), device="cuda")
    qas.qas_score_pages(pc.cache, db.batch, q, scores)
    torch.cuda.synchronize()
    got = scores.cpu().numpy().astype(np.float64)
    for r in range(case.B):
        L = int(case.seq_lens[r])
        m, M, mh, Mh, s = _oracle_copy(case, r, L)
        phys = case.pages[r][:len(m)]
        assert np.array_equal(scale[phys], s), f"scales r={r}"
        assert np.array_equal(vals[phys, :, 0, :], mh), f"min copy r={r}"
        assert np.array_equal(vals[phys, :, 1, :], Mh), f"max copy r={r}"
        q_heads = oracle.decode(case.q[0][r], case.q_dtype)
        U8 = quest.kv_head_scores(quest.head_bounds(q_heads, mh, Mh), case.H_kv)
        U = quest.kv_head_scores(quest.head_bounds(q_heads, m, M), case.H_kv)
        denom = score_denominator(q_heads, mh, Mh, case.g)
        P = len(m)
        base = db.indptr_host[r] * case.H_kv
        for h in range(case.H_kv):
            row = got[base + h * P: base + (h + 1) * P]
            assert_scores_close(row, U8[h], denom[h], f"{name} r={r} h={h}")
            assert np.all(row >= U[h] - 1e-5 * np.maximum(np.abs(U[h]), denom[h]))


@pytest.mark.parametrize("L", [1, 15, 16, 17, 250])
def test_fp8_copy_through_decode_appends(qas, L):
    """Decode-layer appends across page boundaries keep the copy equal to the
    outward quantisation of the exact summaries."""
    from query_aware_sparse_amd.staging import DeviceBatch, to_device
    case = batched_gqa_append(B=2, L_min=L, L_max=L, H_q=4, H_kv=2, d=128, S=16, steps=20)
    pc, _ = _stage8(case, case.lengths(-1))
    for s in range(case.steps):
        lengths = case.lengths(s)
        db = DeviceBatch(lengths, case.pages, case.S)
        kn = to_device(np.stack([case.keys[r][lengths[r] - 1] for r in range(case.B)]), "bf16")
        vn = to_device(np.stack([case.values[r][lengths[r] - 1] for r in range(case.B)]), "bf16")
        out = torch.empty((case.B, case.H_q, case.d), dtype=torch.bfloat16, device="cuda")
        ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, pc.cache, db.batch, case.H_q, case.K)
        qas.qas_decode_layer(pc.cache, db.batch, to_device(case.q[s + 1], case.q_dtype), case.K,
                             case.sm_scale, out, None, ws, k_new=kn, v_new=vn)
    torch.cuda.synchronize()
    vals, scale = _copy_values(pc)
    summ = pc.summary.float().cpu().numpy()
    lengths = case.lengths(case.steps - 1)
    for r in range(case.B):
        m, M, mh, Mh, s = _oracle_copy(case, r, int(lengths[r]))
        phys = case.pages[r][:len(m)]
        assert np.array_equal(summ[phys, :, 0], m) and np.array_equal(summ[phys, :, 1], M)
        assert np.array_equal(scale[phys], s)
        assert np.array_equal(vals[phys, :, 0], mh) and np.array_equal(vals[phys, :, 1], Mh)


def test_decode_layer_on_fp8_summaries(qas):
    from query_aware_sparse_amd.staging import to_device
    case = llama2_7b_layer(L=5000, H=4, K=40)
    pc, db = _stage8(case)
    q = to_device(case.q[0], case.q_dtype)
    ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, pc.cache, db.batch, case.H_q, case.K)
    sel = torch.full((1, case.H_kv, case.K), 777, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    lse = torch.empty((1, case.H_q), device="cuda")
    qas.qas_decode_layer(pc.cache, db.batch, q, case.K, case.sm_scale, out, lse, ws, sel_out=sel)
    torch.cuda.synchronize()
    sel_h = sel.cpu().numpy()
    m, M, mh, Mh, s = _oracle_copy(case, 0, int(case.seq_lens[0]))
    q_heads = oracle.decode(case.q[0][0], case.q_dtype)
    U8 = quest.kv_head_scores(quest.head_bounds(q_heads, mh, Mh), case.H_kv)
    for h in range(case.H_kv):
        check_selection(sel_h[0, h], U8[h], case.K)
    ref = oracle.run_decode(case, page_ids=sel_h.astype(np.int64))
    assert_attn_close(out_to_numpy(out)[0], ref[0]["out"], case.kv_dtype, "fp8-summary layer")
