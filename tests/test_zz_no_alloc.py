"""qas_decode_layer_noalloc (the decode layer on the library's static
per-GPU scratch, for callers that cannot allocate) against qas_decode_layer
with a caller workspace: the same kernels, so outputs, lse and selected
lists must be identical, and both within the oracle's tolerance.  Two calls
in a row, the second on a smaller input; an input whose scratch need exceeds
the maximum is rejected before any launch."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_attn_close, check_selection, out_to_numpy, say
from workloads import batched_gqa_append, llama2_7b_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qas():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import query_aware_sparse_amd
    return query_aware_sparse_amd


def _run_both(qas, case):
    from query_aware_sparse_amd.staging import PagedCache, prefill, to_device
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype)
    db = prefill(pc, case)
    q = to_device(case.q[0], case.q_dtype)
    L = case.seq_lens
    # the current token appended by both calls (the same key folded twice
    # leaves the summary and the pool unchanged)
    kn = to_device(np.stack([case.keys[r][L[r] - 1] for r in range(case.B)]), case.kv_dtype)
    vn = to_device(np.stack([case.values[r][L[r] - 1] for r in range(case.B)]), case.kv_dtype)
    res = []
    for noalloc in (False, True):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((case.B, case.H_q), float("nan"), device="cuda")
        sel = torch.full((case.B, case.H_kv, case.K), -9, dtype=torch.int32, device="cuda")
        if noalloc:
            qas.qas_decode_layer_noalloc(pc.cache, db.batch, q, case.K, case.sm_scale, out, lse,
                                         k_new=kn, v_new=vn, sel_out=sel)
        else:
            ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, pc.cache, db.batch, case.H_q,
                                    case.K)
            qas.qas_decode_layer(pc.cache, db.batch, q, case.K, case.sm_scale, out, lse, ws,
                                 k_new=kn, v_new=vn, sel_out=sel)
        torch.cuda.synchronize()
        res.append((out_to_numpy(out), lse.cpu().numpy(), sel.cpu().numpy()))
    return pc, db, res


def test_noalloc_equals_workspace_call_twice(qas):
    """A 16K-token Llama-shaped layer, then a smaller ragged GQA batch."""
    cases = [llama2_7b_layer(L=16384, H=32, K=128),
             batched_gqa_append(B=2, L_min=900, L_max=2000, steps=0, K=24)]
    sizes = []
    for case in cases:
        say(f"[noalloc] {case.name} B={case.B} lengths={case.seq_lens.tolist()} K={case.K}")
        pc, db, ((o1, l1, s1), (o2, l2, s2)) = _run_both(qas, case)
        sizes.append(qas.qas_workspace_bytes(qas.QAS_OP_DECODE_LAYER, pc.cache, db.batch,
                                             case.H_q, case.K))
        assert np.array_equal(s1, s2)
        assert np.array_equal(o1, o2)
        assert np.array_equal(l1, l2)
        ref = oracle.run_decode(case)
        for r, res in enumerate(ref):
            same = [check_selection(s2[r, h], res["U"][h], case.K) for h in range(case.H_kv)]
            if not all(same):
                res = oracle.run_decode(case, page_ids=s2.astype(np.int64), requests=[r])[0]
            assert_attn_close(o2[r], res["out"], case.kv_dtype, f"noalloc {case.name} r={r}")
            np.testing.assert_allclose(l2[r], res["lse"], rtol=1e-5, atol=1e-4)
    assert sizes[1] < sizes[0]


def test_noalloc_rejects_inputs_beyond_the_scratch(qas):
    """A batch whose scratch need exceeds the maximum returns
    QAS_ERR_WORKSPACE before anything is enqueued (nothing is written)."""
    from query_aware_sparse_amd.staging import DeviceBatch
    H_kv, d, S, K, B, L = 8, 128, 16, 64, 128, 65536
    k_pool = torch.zeros((1, H_kv, S, d), dtype=torch.float16, device="cuda")
    summary = torch.zeros((1, H_kv, 2, d), dtype=torch.float16, device="cuda")
    cache = qas.make_cache(k_pool, k_pool, summary)
    db = DeviceBatch([L] * B, [np.zeros(L // S, np.int32)] * B, S)
    need = qas.qas_workspace_bytes(qas.QAS_OP_DECODE_LAYER, cache, db.batch, H_kv, K)
    assert need > 16 << 20
    q = torch.zeros((B, H_kv, d), dtype=torch.float16, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(qas.QasError) as e:
        qas.qas_decode_layer_noalloc(cache, db.batch, q, K, 0.1, out, None)
    assert e.value.status == 5 and "maximum" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
