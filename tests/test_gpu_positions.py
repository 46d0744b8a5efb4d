"""GPU parity of per-position speculative selection (the Quest page, §1.2 on
speculative decoding: draft positions depend on earlier drafts, so each one
ranks pages with its own query).  qas_decode_positions against
oracle.quest.speculative_positions: every (request, position, KV head) list
equals the oracle's outside near ties of its own bounds, and the attention of
each position over the lists it chose, with its own causal limit, matches
the oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quest
from tests.gpu_util import assert_attn_close, check_selection, out_to_numpy, say
from workloads import batched_gqa_append, llama2_7b_layer
from workloads.cases import cast

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qas():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import query_aware_sparse_amd
    return query_aware_sparse_amd


def _run(qas, pc, db, qb_raw, case, gamma):
    from query_aware_sparse_amd.staging import to_device
    B = qb_raw.shape[0]
    q = to_device(qb_raw, case.q_dtype)                  # [B][gamma][H_q][d]
    n = qas.qas_positions_workspace_bytes(pc.cache, db.batch, case.H_q, gamma, case.K)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    sel = torch.full((B, gamma, case.H_kv, case.K), 777, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    lse = torch.empty((B, gamma, case.H_q), device="cuda")
    qas.qas_decode_positions(pc.cache, db.batch, q, case.K, case.sm_scale, out, lse, ws,
                             sel_out=sel)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), out_to_numpy(out), lse.cpu().numpy()


def _check(case, r, keys, values, L, qb, sel, out, lse, S, gamma, rows=None):
    res = quest.speculative_positions(qb, keys, values, L, S, case.K, scale=case.sm_scale)
    for i, pos in enumerate(res):
        c = L - gamma + i
        for h in range(case.H_kv):
            check_selection(sel[i, h], pos["U"][h], case.K)
        heads = range(case.H_q) if rows is None else rows
        for qi in heads:
            h = qi // case.g
            ids = [int(x) for x in sel[i, h] if x >= 0]
            A = quest.support(ids, L, c, S)
            o, l = quest.attend(qb[i][qi], keys[:, h], values[:, h], A, case.sm_scale)
            assert_attn_close(out[i, qi][None], o[None], case.kv_dtype, f"r={r} pos={i} head={qi}")
            if len(A) == 0:
                assert np.all(out[i, qi] == 0) and lse[i, qi] == -np.inf
            else:
                assert abs(lse[i, qi] - l) <= 1e-4 + 1e-5 * abs(l)


@pytest.mark.parametrize("gamma", [1, 4, 7])
def test_positions_match_the_oracle(qas, gamma):
    from query_aware_sparse_amd.staging import PagedCache, prefill
    case = batched_gqa_append(B=3, L_min=400, L_max=1500, H_q=8, H_kv=2, d=128, S=16, steps=8,
                              K=9)
    S = case.S
    # with the drafts appended: a request shorter than the draft block, a
    # short one and a long one
    lengths = np.array([2, 37 + gamma, int(case.seq_lens[2]) + gamma], np.int32)
    say(f"[positions] gamma={gamma} lengths={lengths.tolist()}")
    pc = PagedCache(case.num_pool_pages, case.H_kv, S, case.d, case.kv_dtype)
    db = prefill(pc, case, lengths)
    rng = np.random.default_rng(100 + gamma)
    qb_raw = cast(rng.standard_normal((case.B, gamma, case.H_q, case.d)), case.q_dtype)
    sel, out, lse = _run(qas, pc, db, qb_raw, case, gamma)
    for r in range(case.B):
        L = int(lengths[r])
        keys = oracle.decode(case.keys[r][:L], case.kv_dtype)
        values = oracle.decode(case.values[r][:L], case.kv_dtype)
        qb = oracle.decode(qb_raw[r], case.q_dtype)
        _check(case, r, keys, values, L, qb, sel[r], out[r], lse[r], S, gamma)


def test_single_position_is_the_decode_layer(qas):
    """gamma = 1 runs the same kernels as qas_decode_layer without an append:
    identical lists and bitwise identical outputs."""
    from query_aware_sparse_amd.staging import PagedCache, prefill, to_device
    case = batched_gqa_append(B=3, L_min=300, L_max=2000, H_q=8, H_kv=2, d=128, S=16, steps=0,
                              K=11)
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype)
    db = prefill(pc, case)
    sel, out, lse = _run(qas, pc, db, case.q[0][:, None], case, 1)
    q = to_device(case.q[0], case.q_dtype)
    ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, pc.cache, db.batch, case.H_q, case.K)
    sel2 = torch.full((case.B, case.H_kv, case.K), 777, dtype=torch.int32, device="cuda")
    out2 = torch.full_like(q, float("nan"))
    lse2 = torch.empty((case.B, case.H_q), device="cuda")
    qas.qas_decode_layer(pc.cache, db.batch, q, case.K, case.sm_scale, out2, lse2, ws,
                         sel_out=sel2)
    torch.cuda.synchronize()
    assert np.array_equal(sel[:, 0], sel2.cpu().numpy())
    assert np.array_equal(out[:, 0], out_to_numpy(out2))
    assert np.array_equal(lse[:, 0], lse2.cpu().numpy())


def test_positions_full_size_layer(qas):
    """The 32K-context layer (2048 pages, 32 heads) with a 4-token draft: all
    lists checked, attention on a sample of heads."""
    from query_aware_sparse_amd.staging import PagedCache, prefill
    gamma = 4
    case = llama2_7b_layer()
    L = int(case.seq_lens[0])
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype)
    db = prefill(pc, case)
    rng = np.random.default_rng(11)
    qb_raw = cast(rng.standard_normal((1, gamma, case.H_q, case.d)), case.q_dtype)
    sel, out, lse = _run(qas, pc, db, qb_raw, case, gamma)
    keys = oracle.decode(case.keys[0][:L], case.kv_dtype)
    values = oracle.decode(case.values[0][:L], case.kv_dtype)
    qb = oracle.decode(qb_raw[0], case.q_dtype)
    _check(case, 0, keys, values, L, qb, sel[0], out[0], lse[0], case.S, gamma,
           rows=[0, 7, 19, 31])


def test_positions_validation_without_launch(qas):
    lib = qas.lib
    assert lib.qas_decode_positions(None, None, None, 0, 0, 1, 1, 0.1, None, None, None, None,
                                    0, None) == 1
    assert lib.qas_positions_workspace_bytes(None, None, 8, 0, 4) == 0
