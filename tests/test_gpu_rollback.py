"""GPU parity of the rollback rescan (the Quest page, §3 on the cache
lifecycle: a cut inside a page rebuilds that page's min/max from its
surviving keys).  After qas_rollback the exact records and their e4m3 copies
equal the oracle's summaries of the kept tokens value for value, and appends
of different tokens at the cut, plus a decode-layer call, then agree with the
oracle on the new sequence."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quest
from oracle.formats import decode_e4m3fn
from tests.gpu_util import assert_attn_close, out_to_numpy, say
from workloads import batched_gqa_append
from workloads.cases import cast

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qas():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import query_aware_sparse_amd
    return query_aware_sparse_amd


def _records(pc, phys):
    summ = pc.summary.float().cpu().numpy()[phys]
    codes = pc.summary_fp8.cpu().numpy()[phys]
    scale = pc.summary_fp8_scale.cpu().numpy().astype(np.float64)[phys]
    return summ, decode_e4m3fn(codes) * scale[:, :, None, None], scale


def _check_against(case, pc, r, keys_r, L):
    """Records of request r's kept pages against the oracle's summaries of
    keys_r[:L] (exact) and their outward e4m3 copy (exact)."""
    if L == 0:
        return
    m, M = quest.page_summaries(oracle.decode(keys_r[:L], case.kv_dtype), L, case.S)
    mh, Mh, s = quest.fp8_summaries(m, M)
    phys = case.pages[r][:len(m)]
    summ, vals, scale = _records(pc, phys)
    assert np.array_equal(summ[:, :, 0], m) and np.array_equal(summ[:, :, 1], M), f"r={r} L={L}"
    assert np.array_equal(scale, s), f"scales r={r}"
    assert np.array_equal(vals[:, :, 0], mh) and np.array_equal(vals[:, :, 1], Mh), f"copy r={r}"


def test_rollback_then_append_and_decode(qas):
    from query_aware_sparse_amd.staging import (DeviceBatch, PagedCache, make_batch, prefill,
                                                to_device)
    case = batched_gqa_append(B=5, L_min=60, L_max=300, H_q=8, H_kv=2, d=128, S=16, steps=40,
                              K=6)
    S = case.S
    L_old = np.array([int(L) + 20 for L in case.seq_lens], np.int32)
    # cuts: inside a page, onto a page boundary, to one token, to nothing, not at all
    L_new = np.array([(L_old[0] // S - 1) * S + 5, (L_old[1] - 5) // S * S, 1, 0, L_old[4]],
                     np.int32)
    say(f"[rollback] L_old={L_old.tolist()} L_new={L_new.tolist()}")
    pc = PagedCache(case.num_pool_pages, case.H_kv, S, case.d, case.kv_dtype, fp8_summaries=True)
    prefill(pc, case, L_old)
    stale = pc.summary.float().cpu().numpy()
    db = DeviceBatch(L_new, case.pages, S)
    qas.qas_rollback(pc.cache, db.batch)
    torch.cuda.synchronize()
    for r in range(case.B):
        _check_against(case, pc, r, case.keys[r], int(L_new[r]))
    # the inside cut really changed a record the revoked tokens had widened
    tail = case.pages[0][(int(L_new[0]) - 1) // S]
    assert not np.array_equal(stale[tail], pc.summary.float().cpu().numpy()[tail])

    # append different tokens at the cut: n_r new tokens per request
    rng = np.random.default_rng(7)
    n = np.array([9, 18, 3, 17, 0], np.int32)
    new_keys = [cast(rng.standard_normal((int(n[r]), case.H_kv, case.d)), case.kv_dtype)
                for r in range(case.B)]
    new_vals = [cast(rng.standard_normal((int(n[r]), case.H_kv, case.d)), case.kv_dtype)
                for r in range(case.B)]
    indptr = np.zeros(case.B + 1, np.int32)
    indptr[1:] = np.cumsum(n)
    full = DeviceBatch(L_new + n, case.pages, S)
    before = make_batch(db.seq_lens, full.page_indptr, full.page_indices, full.total_pages,
                        full.max_pages)
    kn = to_device(np.concatenate(new_keys), case.kv_dtype)
    vn = to_device(np.concatenate(new_vals), case.kv_dtype)
    qas.qas_append(pc.cache, before, torch.from_numpy(indptr).cuda(), int(indptr[-1]),
                   int(n.max()), kn, vn)
    torch.cuda.synchronize()
    keys2 = [np.concatenate([case.keys[r][:L_new[r]], new_keys[r]]) for r in range(case.B)]
    vals2 = [np.concatenate([case.values[r][:L_new[r]], new_vals[r]]) for r in range(case.B)]
    for r in range(case.B):
        _check_against(case, pc, r, keys2[r], int(L_new[r] + n[r]))

    # a decode-layer call on the new sequences against the oracle
    L2 = L_new + n
    q = to_device(case.q[0], case.q_dtype)
    ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, pc.cache, full.batch, case.H_q, case.K)
    sel = torch.full((case.B, case.H_kv, case.K), 777, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    qas.qas_decode_layer(pc.cache, full.batch, q, case.K, case.sm_scale, out, None, ws,
                         sel_out=sel)
    torch.cuda.synchronize()
    got = out_to_numpy(out)
    sel_h = sel.cpu().numpy()
    for r in range(case.B):
        L = int(L2[r])
        qh = oracle.decode(case.q[0][r], case.q_dtype)
        kk = oracle.decode(keys2[r], case.kv_dtype)
        vv = oracle.decode(vals2[r], case.kv_dtype)
        if L == 0:
            assert np.all(got[r] == 0)
            continue
        ids = [[int(x) for x in sel_h[r, h] if x >= 0] for h in range(case.H_kv)]
        ref = quest.decode_request(qh, kk, vv, L, S, case.K, scale=case.sm_scale, page_ids=ids)
        assert_attn_close(got[r], ref["out"], case.kv_dtype, f"r={r}")
        # the GPU's lists are the oracle's top-K outside near ties
        for h in range(case.H_kv):
            assert len(ids[h]) == min(case.K, quest.num_pages(L, S))


def test_rollback_validation_without_launch(qas):
    import ctypes
    assert qas.lib.qas_rollback(None, None, None) == 1
