"""GPU parity of the multi-query chunk path (query unions with membership
masks, fp8 K/V, MFMA tiles) against the oracle: union preparation exactly,
attention per query within the fp8 tolerance, including ragged groups,
duplicate / invalid / empty page sets, causal limits inside pages and two
requests in one call."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quest
from tests.gpu_util import assert_attn_close, out_to_numpy, say
from workloads import multiquery_chunk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qas():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import query_aware_sparse_amd
    return query_aware_sparse_amd


def _run(qas, cb):
    out = torch.full((cb.N, cb.q.shape[1], cb.q.shape[2]), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((cb.N, cb.q.shape[1]), float("nan"), device="cuda")
    qas.qas_chunk_attention(cb.cache, cb.db.batch, cb.q_indptr, cb.q_pos, cb.q, cb.sets,
                            cb.group, 1.0 / np.sqrt(cb.q.shape[2]), out, lse)
    torch.cuda.synchronize()
    return out_to_numpy(out), lse.cpu().numpy().astype(np.float64)


def _check(case, got, lse, queries, base=0):
    ref_o, ref_l = oracle.run_chunk(case, queries)
    for k, n in enumerate(queries):
        assert_attn_close(got[base + n], ref_o[k], "e4m3", f"{case.name} query {n}")
        fin = np.isfinite(ref_l[k])
        assert np.array_equal(np.isfinite(lse[base + n]), fin)
        assert np.allclose(lse[base + n][fin], ref_l[k][fin], atol=5e-2)


def _corrupt(case, seed):
    """Seeded duplicates and invalid IDs in some sets, one fully invalid set."""
    rng = np.random.default_rng(seed)
    sets = case.sets.copy()
    N, H, kq = sets.shape
    P = -(-case.L // case.S)
    for _ in range(N):
        n, h = int(rng.integers(N)), int(rng.integers(H))
        a, b = rng.choice(kq, 2, replace=False)
        sets[n, h, a] = sets[n, h, b]                      # duplicate
        sets[n, h, int(rng.integers(kq))] = [-1, -5, P, P + 3, 2**31 - 1][int(rng.integers(5))]
    sets[3, 2, :] = -1                                     # empty support for (3, h2)
    case.sets = sets
    return case


def test_union_pages_match_oracle(qas):
    from query_aware_sparse_amd.staging import ChunkBatch
    case = _corrupt(multiquery_chunk(L=8192, N=61), 1)
    cb = ChunkBatch([case])
    G = qas.qas_chunk_groups(cb.N, 1, case.group)
    cap = case.group * case.kq
    ul = torch.full((G, case.H_kv, cap), -9, dtype=torch.int32, device="cuda")
    uc = torch.full((G, case.H_kv), -9, dtype=torch.int32, device="cuda")
    um = torch.zeros((G, case.H_kv, cap), dtype=torch.uint8, device="cuda")
    qas.qas_union_pages(cb.db.batch, cb.q_indptr, cb.sets, case.group, case.S, ul, uc, um)
    torch.cuda.synchronize()
    ul, uc, um = ul.cpu().numpy(), uc.cpu().numpy(), um.cpu().numpy()
    P = -(-case.L // case.S)
    n_groups = -(-case.N // case.group)
    for gi in range(G):
        for h in range(case.H_kv):
            if gi >= n_groups:
                assert uc[gi, h] == 0 and np.all(ul[gi, h] == -1)
                continue
            qs = range(gi * case.group, min(case.N, (gi + 1) * case.group))
            valid = [[int(p) for p in case.sets[n, h] if 0 <= p < P] for n in qs]
            union, member = quest.union_with_membership(valid)
            U = len(union)
            assert uc[gi, h] == U
            assert ul[gi, h, :U].tolist() == union and np.all(ul[gi, h, U:] == -1)
            bits = np.zeros(U, dtype=np.int64)
            for i in range(len(valid)):
                bits |= member[i].astype(np.int64) << i
            assert np.array_equal(um[gi, h, :U], bits)


def test_chunk_attention_small_all_queries(qas):
    """Every query of a small chunk (ragged last group of 5 queries)."""
    from query_aware_sparse_amd.staging import ChunkBatch
    case = _corrupt(multiquery_chunk(L=8192, N=61), 2)
    say(f"[chunk] {case.name} L={case.L} N={case.N}")
    got, lse = _run(qas, ChunkBatch([case]))
    _check(case, got, lse, list(range(case.N)))
    assert np.all(got[3, 8:12] == 0) and np.all(np.isneginf(lse[3, 8:12]))


def test_chunk_attention_page_size_32(qas):
    from query_aware_sparse_amd.staging import ChunkBatch
    case = multiquery_chunk(L=4000, S=32, N=24, kq=40, keep=28)
    got, lse = _run(qas, ChunkBatch([case]))
    _check(case, got, lse, list(range(case.N)))


def test_chunk_attention_two_requests(qas):
    """Two requests in one call share the fp8 pool and scales; groups never
    cross the request boundary."""
    from query_aware_sparse_amd.staging import ChunkBatch
    a = multiquery_chunk(seed=41, L=6000, N=21)
    b = multiquery_chunk(seed=42, L=9000, N=13, scales=(a.k_scale, a.v_scale))
    got, lse = _run(qas, ChunkBatch([a, b]))
    _check(a, got, lse, list(range(a.N)))
    _check(b, got, lse, list(range(b.N)), base=a.N)


def test_chunk_attention_full_size(qas):
    """The 64K-context, 512-query chunk (S=64, 64-page sets, 32/8 heads, fp8)
    at full size; a seeded sample of queries is compared (all heads)."""
    from query_aware_sparse_amd.staging import ChunkBatch
    case = multiquery_chunk()
    say(f"[chunk] {case.name} L={case.L} N={case.N}")
    got, lse = _run(qas, ChunkBatch([case]))
    qs = sorted(set(np.random.default_rng(9).choice(case.N, 24, replace=False).tolist()
                    + [0, 7, 8, 511]))
    _check(case, got, lse, qs)
    assert np.all(np.isfinite(got))
