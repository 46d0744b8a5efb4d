"""GPU parity of the candidate set that joins the Quest top-K with fixed sink
and local-window pages (the Quest page, §2.2 and §3.2: C = C_local | C_sink |
C_quest): the standalone selection on identical fp32 scores must equal the
oracle exactly; the decode layer's lists must equal the oracle's outside
near ties and its attention must match the oracle on the lists it chose."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quest
from tests.gpu_util import TIE_RTOL, assert_attn_close, out_to_numpy, say
from workloads import batched_gqa_append, llama2_7b_layer, tiny_single_head

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qas():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import query_aware_sparse_amd
    return query_aware_sparse_amd


WINDOWS = [(0, 0), (4, 0), (0, 512), (4, 512), (17, 33), (100000, 0), (0, 100000), (1, 1)]


@pytest.mark.parametrize("sink,local", WINDOWS)
def test_select_pages_exact_on_identical_scores(qas, sink, local):
    from query_aware_sparse_amd.staging import DeviceBatch
    rng = np.random.default_rng(300 + sink + 7 * local)
    H, S = 3, 16
    P = [1, 300, 2048, 37, 0, 1000]
    lens = [p * S - int(rng.integers(0, S)) if p else 0 for p in P]
    pages = [np.arange(max(p, 1), dtype=np.int32) for p in P]
    db = DeviceBatch(lens, pages, S)
    total = db.total_pages * H
    B = len(P)
    for kind in ("ints", "normal"):
        s = (rng.integers(-20, 20, size=total) if kind == "ints"
             else rng.standard_normal(total)).astype(np.float32)
        scores = torch.from_numpy(s).cuda()
        for K in (1, 8, 64):
            cap = qas.qas_selection_capacity(K, S, sink, local)
            say(f"[select] sink={sink} local={local} kind={kind} K={K} cap={cap}")
            sel = torch.full((B, H, cap + 3), 12345, dtype=torch.int32, device="cuda")
            cnt = torch.full((B, H), -7, dtype=torch.int32, device="cuda")
            qas.qas_select_pages(scores, db.batch, H, S, K, sink, local, sel, cnt)
            torch.cuda.synchronize()
            sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
            for r in range(B):
                base = db.indptr_host[r] * H
                for h in range(H):
                    row = s[base + h * P[r]: base + (h + 1) * P[r]].astype(np.float64)
                    ref = quest.mixed_pages(row, K, lens[r], S, sink, local)
                    assert cnt_h[r, h] == len(ref), (kind, K, r, h)
                    assert list(sel_h[r, h, :len(ref)]) == ref, (kind, K, r, h)
                    assert np.all(sel_h[r, h, len(ref):] == -1)


def _check_mixed(got, U, K, L, S, sink, local):
    """The GPU list against the oracle's float64 scores: exact outside a near
    tie at the K-th bound; inside it, every page clearly above is kept, every
    page clearly below that is not fixed is left out, and the fixed pages are
    always there."""
    fs, fl = quest.fixed_pages(L, S, sink, local)
    fixed = fs | fl
    got = [int(x) for x in got if x >= 0]
    assert got == sorted(set(got)) and fixed <= set(got)
    n = len(U)
    ref = quest.mixed_pages(U, K, L, S, sink, local)
    if min(K, n) == n:
        assert got == ref
        return
    order = sorted(range(n), key=lambda j: (-U[j], j))
    uk, uk1 = U[order[K - 1]], U[order[K]]
    delta = TIE_RTOL * abs(uk)
    if uk - uk1 > delta:
        assert got == ref
        return
    gs = set(got)
    for j in range(n):
        if U[j] > uk + delta:
            assert j in gs
        if U[j] < uk - delta and j not in fixed:
            assert j not in gs


MIXED_CASES = {
    "llama2_7b_layer-5k": (lambda: llama2_7b_layer(L=5000, H=4, K=40), 4, 512),
    "batched_gqa-ragged": (lambda: batched_gqa_append(B=3, L_min=900, L_max=3000, steps=0, K=37),
                           16, 100),
    "long-rows-separate-topk": (lambda: tiny_single_head(L=20001, S=4, K=50), 8, 101),
}


@pytest.mark.parametrize("name", list(MIXED_CASES))
def test_decode_layer_mixed_matches_oracle(qas, name):
    from query_aware_sparse_amd.staging import PagedCache, prefill, to_device
    make, sink, local = MIXED_CASES[name]
    case = make()
    say(f"[mixed] {name}: B={case.B} H={case.H_q}/{case.H_kv} S={case.S} K={case.K} "
        f"sink={sink} local={local}")
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype)
    db = prefill(pc, case)
    q = to_device(case.q[0], case.q_dtype)
    cap = qas.qas_selection_capacity(case.K, case.S, sink, local)
    ws = qas.make_workspace(qas.QAS_OP_DECODE_LAYER, pc.cache, db.batch, case.H_q, cap)
    sel = torch.full((case.B, case.H_kv, cap), 777, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, float("nan"))
    lse = torch.empty((case.B, case.H_q), device="cuda")
    qas.qas_decode_layer_mixed(pc.cache, db.batch, q, case.K, sink, local, case.sm_scale, out,
                               lse, ws, sel_out=sel)
    torch.cuda.synchronize()
    sel_h = sel.cpu().numpy()
    ref = oracle.run_decode(case, sink_tokens=sink, local_tokens=local)
    for r in range(case.B):
        L = ref[r]["L"]
        for h in range(case.H_kv):
            _check_mixed(sel_h[r, h], ref[r]["U"][h], case.K, L, case.S, sink, local)
    # attention over the lists the GPU chose
    ref2 = oracle.run_decode(case, page_ids=sel_h.astype(np.int64))
    got = out_to_numpy(out)
    for r in range(case.B):
        assert_attn_close(got[r], ref2[r]["out"], case.kv_dtype, f"{name} r={r}")
        assert np.allclose(lse.cpu().numpy()[r], ref2[r]["lse"], atol=1e-4, rtol=1e-5)
