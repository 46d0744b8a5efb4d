"""GPU parity of the exact token top-R by branch-and-bound (the Quest page,
§3.2: read pages by descending bound, stop when the next bound is below
tau_R).  The tokens qas_exact_top_r returns are the brute-force top R of all
tokens (the certificate's claim) outside near ties at the R-th logit, their
logits match float64 dot products, the list is ordered by (logit desc,
token asc), and tight bounds stop the search before the last page."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quest
from tests.gpu_util import say
from workloads import batched_gqa_append, llama2_7b_layer, tiny_single_head

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qas():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import query_aware_sparse_amd
    return query_aware_sparse_amd


def _run(qas, pc, db, case, R, q_raw=None):
    from query_aware_sparse_amd.staging import to_device
    q = to_device(case.q[0] if q_raw is None else q_raw, case.q_dtype)
    tok = torch.full((case.B, case.H_q, R), 12345, dtype=torch.int32, device="cuda")
    lg = torch.full((case.B, case.H_q, R), 7.0, device="cuda")
    pr = torch.full((case.B, case.H_q), -3, dtype=torch.int32, device="cuda")
    n = qas.qas_exact_top_r_workspace_bytes(pc.cache, db.batch, case.H_q, R)
    ws = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")   # no zero-fill needed
    qas.qas_exact_top_r(pc.cache, db.batch, q, R, tok, lg, ws, pages_read=pr)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), lg.cpu().numpy(), pr.cpu().numpy()


def _check_row(q_head, keys_h, L, S, R, tok, lg, n_read, what):
    ref = quest.brute_top_r(q_head, keys_h, L, R + 1)
    take = min(R, L)
    got = [int(t) for t in tok[:take]]
    assert all(t == -1 for t in tok[take:]) and np.all(lg[take:] == -np.inf), what
    assert len(set(got)) == take and all(0 <= t < L for t in got), what
    z = {t: float(keys_h[t] @ q_head) for t in got}
    scale = max(1.0, abs(ref[0][0]))
    tol = 1e-5 * scale
    for t, v in zip(got, lg[:take]):
        assert abs(v - z[t]) <= tol, (what, t, v, z[t])
    # ordered by the returned logits, ties to the lower token
    for a, b in zip(range(take - 1), range(1, take)):
        assert (lg[a] > lg[b]) or (lg[a] == lg[b] and got[a] < got[b]), what
    # the set is the exact top R outside a near tie at the boundary
    ref_set = {t for _, t in ref[:take]}
    if take < L and ref[take - 1][0] - ref[take][0] > 2 * tol:
        assert set(got) == ref_set, what
    else:
        for v, t in ref[:take]:
            if v > ref[take - 1][0] + 2 * tol:
                assert t in set(got), what
    P = quest.num_pages(L, S)
    assert 1 <= n_read <= P, (what, n_read, P)


CASES = {
    "tiny-f32": (lambda: tiny_single_head(L=301, K=4), [1, 5, 40, 400]),
    "gqa-bf16": (lambda: batched_gqa_append(B=3, L_min=200, L_max=3000, H_q=8, H_kv=2, steps=0), [16]),
    "llama-f16-5k": (lambda: llama2_7b_layer(L=5000, H=4, K=40), [8, 512]),
    # R = 512: a merge batch holds 8 lists, and ~24 lists (the pilot's and
    # ~23 scan chunks') take four batches
    "llama-f16-12k": (lambda: llama2_7b_layer(L=12000, H=2, K=40), [512]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_exact_top_r_matches_brute_force(qas, name):
    from query_aware_sparse_amd.staging import PagedCache, prefill
    make, Rs = CASES[name]
    case = make()
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype)
    db = prefill(pc, case)
    for R in Rs:
        say(f"[top-R] {name} R={R}")
        tok, lg, pr = _run(qas, pc, db, case, R)
        for r in range(case.B):
            L = int(case.seq_lens[r])
            keys = oracle.decode(case.keys[r][:L], case.kv_dtype)
            qh = oracle.decode(case.q[0][r], case.q_dtype)
            for i in range(case.H_q):
                h = i // case.g
                _check_row(qh[i], keys[:, h], L, case.S, R, tok[r, i], lg[r, i], pr[r, i],
                           f"{name} R={R} r={r} head={i}")


def test_tight_bounds_stop_early(qas):
    """A few tokens aligned with the query: their pages' bounds stand far above
    every other page's, so the search stops after few pages, with the same
    result and read count as the oracle's branch-and-bound."""
    from query_aware_sparse_amd.staging import PagedCache, prefill
    case = tiny_single_head(L=400, K=4)
    qv = case.q[0][0, 0].astype(np.float64)
    hot = [17, 123, 250, 251, 399]
    for t in hot:
        case.keys[0][t, 0] = (3.0 * qv).astype(np.float32)
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype)
    db = prefill(pc, case)
    R = 5
    tok, lg, pr = _run(qas, pc, db, case, R)
    keys = oracle.decode(case.keys[0][:400], "f32")[:, 0]
    m, M = quest.page_summaries(keys[:, None], 400, case.S)
    read, top, tau = quest.exact_top_r(qv, keys, 400, case.S, R, m[:, 0], M[:, 0])
    assert sorted(int(t) for t in tok[0, 0]) == sorted(hot)
    assert [t for _, t in top] == [int(t) for t in tok[0, 0]]
    P = quest.num_pages(400, case.S)
    n = int(pr[0, 0])
    # rounds of whole pages (the first ceil(R/S), then doubling): at least the
    # page-by-page reads, at most about twice them, far below P
    assert len(read) <= n <= 2 * len(read) + -(-R // case.S) < P
    say(f"[top-R] tight bounds: {n} of {P} pages read (page by page: {len(read)})")


def test_exact_top_r_full_size_layer(qas):
    """The 32K-context layer (2048 pages, 32 heads), R = 64: every head's list
    against brute force over all 32768 tokens."""
    from query_aware_sparse_amd.staging import PagedCache, prefill
    case = llama2_7b_layer()
    L = int(case.seq_lens[0])
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype)
    db = prefill(pc, case)
    tok, lg, pr = _run(qas, pc, db, case, 64)
    keys = oracle.decode(case.keys[0][:L], case.kv_dtype)
    qh = oracle.decode(case.q[0][0], case.q_dtype)
    for i in range(case.H_q):
        _check_row(qh[i], keys[:, i], L, case.S, 64, tok[0, i], lg[0, i], pr[0, i], f"head={i}")
    say(f"[top-R] 32K layer R=64: pages read per head min {pr.min()} max {pr.max()} of 2048")


def test_exact_top_r_degenerate_rows(qas):
    """A ragged batch with an empty request, a one-token request and one whose
    last page is partly filled: the empty rows return -1 / -inf and no pages,
    the others match brute force (R above and below the row's token count)."""
    from query_aware_sparse_amd.staging import PagedCache, prefill
    case = batched_gqa_append(B=4, L_min=200, L_max=3000, H_q=8, H_kv=2, steps=0)
    case.seq_lens[1] = 0
    case.seq_lens[2] = 1
    case.seq_lens[3] = 16 * 40 + 7
    pc = PagedCache(case.num_pool_pages, case.H_kv, case.S, case.d, case.kv_dtype)
    db = prefill(pc, case)
    for R in (3, 64):
        say(f"[top-R] degenerate rows R={R}")
        tok, lg, pr = _run(qas, pc, db, case, R)
        assert np.all(tok[1] == -1) and np.all(np.isneginf(lg[1])) and np.all(pr[1] == 0)
        for r in (0, 2, 3):
            L = int(case.seq_lens[r])
            keys = oracle.decode(case.keys[r][:L], case.kv_dtype)
            qh = oracle.decode(case.q[0][r], case.q_dtype)
            for i in range(case.H_q):
                _check_row(qh[i], keys[:, i // case.g], L, case.S, R, tok[r, i], lg[r, i],
                           pr[r, i], f"R={R} r={r} head={i}")


def test_exact_top_r_validation_without_launch(qas):
    assert qas.lib.qas_exact_top_r(None, None, None, 0, 1, 1, None, None, None, None, 0,
                                   None) == 1
    assert qas.lib.qas_exact_top_r_workspace_bytes(None, None, 8, 4) == 0
