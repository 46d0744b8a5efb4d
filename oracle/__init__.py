"""Oracle: a plain, slow, float64 CPU implementation of Quest-style
query-aware sparse attention over a paged KV cache.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only the tests under tests/, the
smoke() check of __graft_entry__ and the cpu_baseline leg of bench.py may
import or call it.  The product (query_aware_sparse_amd) never does, and it
shares no code with it: the oracle has its own number-format decoders
(oracle.formats) and its own arithmetic (oracle.quest).  The only code both
sides use is the seeded input generator package ``workloads``, which holds
none of the method's arithmetic.

Every function of oracle.quest cites the passage it follows and is pinned by
tests/test_oracle_pins.py to facts the pages and mathematics fix (the pages'
worked examples, closed forms, brute force, invariants, library special
cases).  Absolute attention values at workload scale beyond those properties
are "parity unpinned": there is no other implementation to compare with.

The helpers below only decode a workload's raw arrays (storage dtype ->
float64, times the per-head fp8 scale where there is one) and run
oracle.quest per request.
"""
import numpy as np

from . import formats, quest
from .formats import decode


def _decoded_kv(case, r, upto=None):
    keys = decode(case.keys[r][:upto], case.kv_dtype)
    values = decode(case.values[r][:upto], case.kv_dtype)
    if case.k_scale is not None:
        keys = keys * np.asarray(case.k_scale, np.float64)[None, :, None]
        values = values * np.asarray(case.v_scale, np.float64)[None, :, None]
    return keys, values


def decoded_kv(case, r):
    """float64 keys and values of request r (all T_r tokens), for reuse over
    several calls of run_decode."""
    return _decoded_kv(case, r)


def run_decode(case, step=-1, page_ids=None, requests=None, decoded=None, sink_tokens=0,
               local_tokens=0):
    """Oracle of one decode call of a DecodeCase: the call before the first
    append (step=-1) or the call after step ``step``'s append.  ``page_ids``
    ([B][H_kv][*]) replaces the top-K lists; ``sink_tokens`` / ``local_tokens``
    add the fixed sink and local pages to them.  ``decoded`` optionally maps a
    request to decoded_kv(case, r).  Returns one result dict per request (see
    quest.decode_request)."""
    lengths = case.lengths(step)
    q_all = decode(case.q[step + 1], case.q_dtype)
    out = []
    for r in (range(case.B) if requests is None else requests):
        L = int(lengths[r])
        if decoded is not None and r in decoded:
            keys, values = decoded[r]
            keys, values = keys[:L], values[:L]
        else:
            keys, values = _decoded_kv(case, r, L)
        res = quest.decode_request(q_all[r], keys, values, L, case.S, case.K,
                                   scale=case.sm_scale,
                                   page_ids=None if page_ids is None else page_ids[r],
                                   sink_tokens=sink_tokens, local_tokens=local_tokens)
        res["L"] = L
        out.append(res)
    return out


def run_chunk(case, queries=None):
    """Oracle of the multi-query chunk call of a ChunkCase, for all queries
    or the listed ones.  Returns (out [n][H_q][d], lse [n][H_q])."""
    keys = decode(case.keys, case.kv_dtype)
    values = decode(case.values, case.kv_dtype)
    if case.k_scale is not None:
        keys = keys * np.asarray(case.k_scale, np.float64)[None, :, None]
        values = values * np.asarray(case.v_scale, np.float64)[None, :, None]
    idx = np.arange(case.N) if queries is None else np.asarray(queries)
    q = decode(case.q[idx], case.q_dtype)
    return quest.chunk_attention(q, keys, values, case.sets[idx],
                                 case.q_len[idx], case.q_pos[idx], case.S,
                                 case.g, scale=case.sm_scale)


__all__ = ["formats", "quest", "decode", "decoded_kv", "run_decode", "run_chunk"]
