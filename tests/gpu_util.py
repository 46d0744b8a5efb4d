"""Helpers of the GPU parity tests: tolerances (written here, derived in the
design notes), selection checks, and driving the library on a workload."""
import math

import numpy as np
import torch

import oracle
from oracle.formats import decode

# Attention output tolerance |o - o_ref| <= atol + rtol * |o_ref|, by K/V dtype.
ATTN_TOL = {"f32": (2e-3, 1e-2), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2),
            "e4m3": (2e-2, 2e-2)}
SCORE_RTOL = 1e-5       # page bounds, fp32 accumulation
TIE_RTOL = 1e-4         # sets must match where the K-th / (K+1)-th gap exceeds this


def say(*a):
    print(*a, flush=True)


def score_denominator(q_heads, m, M, g):
    """max over the group's query heads of sum_d |u_d|, u_d = max(q_d m_d,
    q_d M_d): the scale of the fp32 rounding error of a bound, so near-zero
    bounds get an absolute floor.  [H_kv][P]"""
    P, H_kv, _ = m.shape
    out = np.zeros((H_kv, P))
    for h in range(H_kv):
        for i in range(h * g, (h + 1) * g):
            u = np.maximum(q_heads[i][None, :] * m[:, h, :], q_heads[i][None, :] * M[:, h, :])
            out[h] = np.maximum(out[h], np.abs(u).sum(axis=1))
    return out


def assert_scores_close(got, ref, denom, what=""):
    tol = SCORE_RTOL * np.maximum(np.abs(ref), denom)
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} scores beyond 1e-5 rel, worst "
                           f"{(err / np.maximum(tol, 1e-30)).max():.3g}x tolerance")


def check_selection(sel_row, U, K):
    """Check a selected list against the oracle's float64 scores U of one row.
    Returns True if it must equal (and equals) the oracle's set, False if the
    K-th / (K+1)-th gap is within the near-tie band and the list is only
    checked for validity."""
    n = len(U)
    take = min(K, n)
    got = [int(x) for x in sel_row if x >= 0]
    assert len(got) == take and len(set(got)) == take, (len(got), take)
    assert got == sorted(got) and all(0 <= x < n for x in got)
    assert all(x == -1 for x in sel_row[take:])
    ref = oracle.quest.top_k_pages(U, K)
    if take == n:
        assert got == ref
        return True
    order = sorted(range(n), key=lambda j: (-U[j], j))
    uk, uk1 = U[order[take - 1]], U[order[take]]
    delta = TIE_RTOL * abs(uk)
    if uk - uk1 > delta:
        assert got == ref, "selected set differs from the oracle's outside any near tie"
        return True
    gs = set(got)
    for j in range(n):
        if U[j] > uk + delta:
            assert j in gs, f"page {j} clearly above the K-th bound was not selected"
        if U[j] < uk - delta:
            assert j not in gs, f"page {j} clearly below the K-th bound was selected"
    return got == ref


def assert_attn_close(got, ref, dtype, what=""):
    atol, rtol = ATTN_TOL[dtype]
    err = np.abs(got - ref) - (atol + rtol * np.abs(ref))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err.max() <= 0, (f"{what}: {int((err > 0).sum())} outputs beyond tolerance, "
                            f"worst excess {err.max():.3g}")


def out_to_numpy(t):
    return t.float().cpu().numpy().astype(np.float64)
