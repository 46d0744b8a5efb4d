"""Workload definitions (see the package docstring for the RNG recipe).

A DecodeCase is a batch of requests with a paged KV cache:
  * ``keys[r]`` / ``values[r]``: token-ordered raw arrays [T_r][H_kv][d] in
    the storage dtype (np.float32 for 'f32', np.float16 for 'f16', uint16
    bit patterns for 'bf16', uint8 codes for 'e4m3'), T_r = L_r + steps.
  * ``seq_lens[r]`` = L_r tokens are in the cache at the first decode call
    (the current token included); decode step s then appends token L_r + s
    and decodes at length L_r + s + 1.
  * ``q[0]`` is the query of the first decode call, ``q[s + 1]`` that of
    step s: shape [1 + steps][B][H_q][d].
  * ``pages[r]`` lists the physical page of every logical page the request
    will ever use; a call at length L uses the first ceil(L/S) of them.

A ChunkCase is one request with many query positions, each with its own
page set per KV head (the multi-query chunk of the PageWeaver notes).
"""
import concurrent.futures
import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

# stream ids, so that every tensor of a case has an independent RNG stream
_KEYS, _VALUES, _QUERY, _TABLE, _OUTLIER, _SETS, _LENS, _CORRUPT = range(1, 9)
STEP_STREAM = 100

INVALID_IDS = (-1, -7, None, None, 2**31 - 1)  # None -> P and P + 5 (per row)


def _rng(*keys):
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in keys]))


def cast(x, dtype):
    """Cast float32/float64 samples to a storage dtype with round-to-nearest-
    even; returns the raw storage array (see module docstring)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        t = torch.from_numpy(x).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if dtype == "e4m3":
        x = np.clip(x, -448.0, 448.0)
        t = torch.from_numpy(x).to(torch.float8_e4m3fn)
        return t.view(torch.uint8).numpy().copy()
    raise ValueError(dtype)


def ceil_div(a, b):
    return -(-int(a) // int(b))


@dataclass
class DecodeCase:
    name: str
    B: int
    H_q: int
    H_kv: int
    d: int
    S: int
    K: int
    kv_dtype: str
    q_dtype: str
    seq_lens: np.ndarray
    keys: List[np.ndarray]
    values: List[np.ndarray]
    q: np.ndarray
    pages: List[np.ndarray]
    num_pool_pages: int
    steps: int = 0
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    notes: str = ""

    @property
    def g(self):
        return self.H_q // self.H_kv

    @property
    def sm_scale(self):
        return 1.0 / math.sqrt(self.d)

    def lengths(self, step=-1):
        """Per-request lengths of the decode call before step 0 (step=-1) or
        after step ``step``'s append."""
        return (self.seq_lens + (step + 1)).astype(np.int32)

    def page_table(self, lengths):
        """CSR page table (indptr [B+1], indices) covering ceil(L_r/S) pages."""
        counts = [ceil_div(L, self.S) for L in lengths]
        indptr = np.zeros(self.B + 1, dtype=np.int32)
        indptr[1:] = np.cumsum(counts)
        indices = np.concatenate(
            [self.pages[r][:counts[r]] for r in range(self.B)]).astype(np.int32)
        return indptr, indices


@dataclass
class ChunkCase:
    name: str
    H_q: int
    H_kv: int
    d: int
    S: int
    L: int
    N: int
    kq: int
    group: int
    kv_dtype: str
    q_dtype: str
    keys: np.ndarray          # raw [L][H_kv][d]
    values: np.ndarray
    k_scale: Optional[np.ndarray]
    v_scale: Optional[np.ndarray]
    q: np.ndarray             # raw [N][H_q][d]
    q_pos: np.ndarray         # c_i, int32 [N]
    q_len: np.ndarray         # L_i, int32 [N]
    sets: np.ndarray          # int32 [N][H_kv][kq] logical page IDs
    pages: np.ndarray         # physical page of each logical page
    num_pool_pages: int
    notes: str = ""
    # fp8 cases: the float32 K/V drawn before quantisation ([L][H_kv][d]),
    # the input of a writer that quantises itself
    keys_src: Optional[np.ndarray] = None
    values_src: Optional[np.ndarray] = None

    @property
    def g(self):
        return self.H_q // self.H_kv

    @property
    def sm_scale(self):
        return 1.0 / math.sqrt(self.d)


# ----------------------------------------------------------------- helpers --

def _normal(seed, stream, idx, shape):
    return _rng(seed, stream, idx).standard_normal(shape, dtype=np.float32)


_CHUNK = 2048  # tokens per independent RNG stream of a token-ordered tensor


def _tokens(seed, stream, idx, T, H, d, dtype, dist="normal", nu=3.0,
            col_scale=None, head_scale=None):
    """Token-ordered [T][H][d] tensor in storage dtype `dtype`.  Token chunk c
    (tokens c*2048 ...) draws from SeedSequence([seed, stream, idx, c]), so
    chunks are generated in parallel threads and the result does not depend
    on the thread count.  col_scale ([H][d]) multiplies the samples before
    the cast; head_scale ([H]) divides them (fp8 quantisation scale)."""
    out_dt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16,
              "e4m3": np.uint8}[dtype]
    out = np.empty((T, H, d), dtype=out_dt)

    def work(c):
        t0, t1 = c * _CHUNK, min(T, (c + 1) * _CHUNK)
        g = _rng(seed, stream, idx, c)
        if dist == "normal":
            x = g.standard_normal((t1 - t0, H, d), dtype=np.float32)
        else:
            x = np.clip(g.standard_t(nu, size=(t1 - t0, H, d)), -65504.0, 65504.0)
        if col_scale is not None:
            x = x * col_scale[None]
        if head_scale is not None:
            x = x / head_scale[None, :, None]
        out[t0:t1] = cast(x, dtype)

    n = ceil_div(T, _CHUNK)
    with concurrent.futures.ThreadPoolExecutor(min(16, max(1, n))) as ex:
        list(ex.map(work, range(n)))
    return out


def _pool_permutation(seed, total, extra):
    """Physical pages for `total` logical pages drawn from a shuffled pool of
    total + extra pages (the extra ones stay unallocated)."""
    perm = _rng(seed, _TABLE).permutation(total + extra).astype(np.int32)
    return perm[:total], total + extra


def _split_pages(flat, counts):
    out, pos = [], 0
    for c in counts:
        out.append(flat[pos:pos + c])
        pos += c
    return out


# --------------------------------------------------------------- workloads --

def tiny_single_head(seed=1, L=64, S=4, d=16, K=4):
    """Tiny single instance: 1 request, 1 KV head, 1 query head, d=16, S=4,
    L=64 (16 pages), K=4, fp32 N(0,1); physical pages are a seeded
    permutation inside a slightly larger pool."""
    keys = _normal(seed, _KEYS, 0, (L, 1, d))
    values = _normal(seed, _VALUES, 0, (L, 1, d))
    q = _normal(seed, _QUERY, 0, (1, 1, 1, d))
    P = ceil_div(L, S)
    phys, pool = _pool_permutation(seed, P, 4)
    return DecodeCase("tiny-single-head-d16", 1, 1, 1, d, S, K, "f32", "f32",
                      np.array([L], np.int32), [keys], [values], q, [phys],
                      pool)


def llama2_7b_layer(seed=2, L=32768, H=32, d=128, S=16, K=256, outliers=4,
            outlier_scale=8.0, identity_table=True):
    """Llama-2-7B-shaped decode layer: B=1, 32 query heads = 32 KV heads,
    d=128, S=16, L=32768 (2048 pages), K=256; fp16 K/V N(0,1) with 4 seeded
    channels per KV head scaled x8 in both K and V; fp16 query N(0,1).
    Smaller L / H give the same recipe at test sizes."""
    orng = _rng(seed, _OUTLIER)
    col = np.ones((H, d), np.float32)
    for h in range(H):
        col[h, orng.choice(d, size=min(outliers, d), replace=False)] = outlier_scale
    keys = _tokens(seed, _KEYS, 0, L, H, d, "f16", col_scale=col)
    values = _tokens(seed, _VALUES, 0, L, H, d, "f16", col_scale=col)
    q = _normal(seed, _QUERY, 0, (1, 1, H, d))
    P = ceil_div(L, S)
    if identity_table:
        phys, pool = np.arange(P, dtype=np.int32), P
    else:
        phys, pool = _pool_permutation(seed, P, 8)
    return DecodeCase("llama2-7b-layer-32k", 1, H, H, d, S, K, "f16",
                      "f16", np.array([L], np.int32), [keys],
                      [values], cast(q, "f16"), [phys], pool,
                      notes="4 outlier channels per KV head x8 in K and V")


def batched_gqa_append(seed=3, B=8, L_min=8192, L_max=65536, H_q=32, H_kv=8, d=128,
            S=16, K=128, steps=16):
    """Batched GQA decode with append: B requests, L_r ~ U{L_min..L_max},
    32 query / 8 KV heads, d=128, S=16, K=128, bf16 K/V/q N(0,1).  Each of
    `steps` decode steps appends one token per request; physical pages come
    from one seeded shuffled pool (the next page is used at a boundary)."""
    lens = _rng(seed, _LENS).integers(L_min, L_max, size=B,
                                      endpoint=True).astype(np.int32)
    keys, values = [], []
    for r in range(B):
        T = int(lens[r]) + steps
        keys.append(_tokens(seed, _KEYS, r, T, H_kv, d, "bf16"))
        values.append(_tokens(seed, _VALUES, r, T, H_kv, d, "bf16"))
    q = cast(_normal(seed, _QUERY, 0, (1 + steps, B, H_q, d)), "bf16")
    counts = [ceil_div(int(L) + steps, S) for L in lens]
    flat, pool = _pool_permutation(seed, sum(counts), 16)
    return DecodeCase("batched-gqa-append", B, H_q, H_kv, d, S, K,
                      "bf16", "bf16", lens, keys, values, q,
                      _split_pages(flat, counts), pool, steps=steps)


def stress_long_context(seed=5, B=16, L=131072, H_q=32, H_kv=8, d=128, S=32, K=None,
            nu=3.0):
    """Stress: B requests at L tokens, 32 query / 8 KV heads, d=128, S=32,
    K = 1% of the pages rounded to nearest (41 for 4096 pages); keys are
    i.i.d. Student-t(nu=3) per element, V and q N(0,1), all fp16.  The
    corrupted page lists are made by corrupt_lists() from a real top-K."""
    P = ceil_div(L, S)
    if K is None:
        K = max(1, int(round(0.01 * P)))
    keys, values = [], []
    for r in range(B):
        keys.append(_tokens(seed, _KEYS, r, L, H_kv, d, "f16", dist="t", nu=nu))
        values.append(_tokens(seed, _VALUES, r, L, H_kv, d, "f16"))
    q = cast(_normal(seed, _QUERY, 0, (1, B, H_q, d)), "f16")
    flat, pool = _pool_permutation(seed, B * P, 32)
    return DecodeCase("stress-16x128k", B, H_q, H_kv, d, S, K, "f16", "f16",
                      np.full(B, L, np.int32), keys, values, q,
                      _split_pages(flat, [P] * B), pool,
                      notes="Student-t(3) keys; lists corrupted after top-K")


def corrupt_lists(lists, num_pages, seed=5, n_slots=8):
    """Seeded corruption of selected page lists [B][H_kv][K] (a copy is
    returned).  Rows are split by exact counts: 5% fully invalid, 5% with
    n_slots duplicates and n_slots invalid IDs, 10% with duplicates only,
    10% with invalid IDs only, the rest untouched.  A duplicate copies the
    ID of another, untouched slot of the same row; invalid IDs cycle through
    -1, -7, P, P+5 and INT32_MAX (P = pages of the request).  Returns
    (corrupted lists, per-row category array)."""
    lists = np.array(lists, dtype=np.int64, copy=True)
    B, H, K = lists.shape
    rows = B * H
    rng = _rng(seed, _CORRUPT)
    order = rng.permutation(rows)
    n_empty = int(round(0.05 * rows))
    n_both = int(round(0.05 * rows))
    n_dup = int(round(0.10 * rows))
    n_inv = int(round(0.10 * rows))
    cat = np.zeros(rows, dtype=np.int32)  # 0 untouched
    pos = 0
    for c, n in ((4, n_empty), (3, n_both), (1, n_dup), (2, n_inv)):
        cat[order[pos:pos + n]] = c
        pos += n

    def invalid(P, i):
        v = INVALID_IDS[i % len(INVALID_IDS)]
        if v is None:
            v = P if i % len(INVALID_IDS) == 2 else P + 5
        return v

    for row in range(rows):
        r, h = divmod(row, H)
        P = int(num_pages[r])
        c = cat[row]
        if c == 4:
            for i in range(K):
                lists[r, h, i] = invalid(P, i + int(rng.integers(5)))
            continue
        if c == 0:
            continue
        need = (n_slots if c in (1, 3) else 0) + (n_slots if c in (2, 3) else 0)
        need = min(need, K - 1)
        slots = rng.permutation(K)[:need]
        keep = np.setdiff1d(np.arange(K), slots)
        n_d = min(n_slots, need) if c in (1, 3) else 0
        for s in slots[:n_d]:
            lists[r, h, s] = lists[r, h, keep[int(rng.integers(len(keep)))]]
        for j, s in enumerate(slots[n_d:]):
            lists[r, h, s] = invalid(P, j + int(rng.integers(5)))
    return lists.astype(np.int32), cat.reshape(B, H)


def multiquery_chunk(seed=4, L=65536, S=64, N=512, H_q=32, H_kv=8, d=128, kq=64,
            keep=45, group=8, scales=None):
    """Multi-query sparse chunk: one request of L tokens, S=64, N query
    positions c_i = L - N + i (L_i = L), each with its own kq-page set per KV
    head that always holds the query's own page floor(c_i/S).  S_0 = own page
    + kq-1 seeded pages <= own page; S_i = own page + `keep` seeded members
    of S_{i-1} (own page excluded) + fresh pages <= own page not in S_{i-1},
    filled to kq, so neighbours share ~70% of their pages.  K/V N(0,1)
    quantised to fp8 e4m3 with a per-KV-head scale amax/448; q bf16 N(0,1).
    Entries of each set are stored in seeded random order.  `scales`
    ((k_scale, v_scale)) quantises with given per-head scales instead (so
    several requests can share one fp8 cache)."""
    keys = _tokens(seed, _KEYS, 0, L, H_kv, d, "f32")
    values = _tokens(seed, _VALUES, 0, L, H_kv, d, "f32")
    if scales is None:
        k_scale = (np.abs(keys).max(axis=(0, 2)) / np.float32(448.0)).astype(np.float32)
        v_scale = (np.abs(values).max(axis=(0, 2)) / np.float32(448.0)).astype(np.float32)
    else:
        k_scale, v_scale = (np.asarray(x, np.float32) for x in scales)
    k_codes = cast(keys / k_scale[None, :, None], "e4m3")
    v_codes = cast(values / v_scale[None, :, None], "e4m3")
    q = cast(_normal(seed, _QUERY, 0, (N, H_q, d)), "bf16")
    q_pos = (L - N + np.arange(N)).astype(np.int32)
    q_len = np.full(N, L, np.int32)
    srng = _rng(seed, _SETS)
    sets = np.zeros((N, H_kv, kq), dtype=np.int32)
    for h in range(H_kv):
        prev = None
        for i in range(N):
            own = int(q_pos[i]) // S
            if prev is None:
                others = srng.choice(own, size=kq - 1, replace=False) if own >= kq - 1 \
                    else np.arange(own)
                cur = [own] + [int(x) for x in others]
            else:
                pool_prev = [p for p in prev if p != own]
                kept = srng.choice(pool_prev, size=min(keep, len(pool_prev)),
                                   replace=False)
                cur = [own] + [int(x) for x in kept]
                have = set(prev) | set(cur)
                fresh = [p for p in range(own + 1) if p not in have]
                need = kq - len(cur)
                if need > 0:
                    add = srng.choice(fresh, size=min(need, len(fresh)),
                                      replace=False)
                    cur += [int(x) for x in add]
            cur = list(srng.permutation(cur))
            sets[i, h, :len(cur)] = cur
            sets[i, h, len(cur):] = -1
            prev = [int(p) for p in cur]
    P = ceil_div(L, S)
    phys, pool = _pool_permutation(seed, P, 8)
    return ChunkCase("multiquery-chunk-64k", H_q, H_kv, d, S, L, N, kq,
                     group, "e4m3", "bf16", k_codes, v_codes, k_scale,
                     v_scale, q, q_pos, q_len, sets, phys, pool,
                     keys_src=keys, values_src=values)


def layer_queries(case, n_layers, seed=2):
    """Queries for n_layers copies of a single-call DecodeCase (one per layer
    of a model): layer 0 keeps case.q[0], layer i > 0 draws N(0,1) from its
    own stream.  Returns raw [n_layers][B][H_q][d] in case.q_dtype."""
    out = [case.q[0]]
    for i in range(1, n_layers):
        out.append(cast(_normal(seed, _QUERY, 1000 + i, (case.B, case.H_q, case.d)),
                        case.q_dtype))
    return np.stack(out)


# ------------------------------------------------------ pages' fixed cases --

def worked_example_case(second_set=False, d=16, S=4):
    """The Quest page's 2-D worked example (§1.1, eq. (5)), zero-padded to d
    dimensions: one page holding keys (1,4), (3,-2), (-1,1) and query
    (2,-1); with ``second_set`` the keys are (3,4), (-1,-2) instead.  Values
    are seeded N(0,1) (the example gives none).  fp32, K = 1."""
    if second_set:
        pts = [(3.0, 4.0), (-1.0, -2.0)]
    else:
        pts = [(1.0, 4.0), (3.0, -2.0), (-1.0, 1.0)]
    L = len(pts)
    keys = np.zeros((L, 1, d), np.float32)
    for t, (a, b) in enumerate(pts):
        keys[t, 0, 0], keys[t, 0, 1] = a, b
    values = _normal(11 + int(second_set), _VALUES, 0, (L, 1, d))
    q = np.zeros((1, 1, 1, d), np.float32)
    q[0, 0, 0, 0], q[0, 0, 0, 1] = 2.0, -1.0
    return DecodeCase("worked-example" + ("-b" if second_set else ""), 1, 1, 1,
                      d, S, 1, "f32", "f32", np.array([L], np.int32), [keys],
                      [values], q, [np.array([0], np.int32)], 1)


def figure2_case(d=16, S=4):
    """The Quest page's Fig. 2 two-step example, zero-padded to d dimensions.
    The figure prints only summaries and bounds; the keys are a reading that
    reproduces every printed number: page A = (3,1), (0,-2), (1,0) [plus
    (2,0), which keeps A's summary, to fill a 4-token page], page B = (1,2),
    (0,4).  The first decode uses q_t = (2,-1); step 0 appends (-2,5) to B
    and decodes with q_{t+1} = (0,1).  K = 1; values seeded N(0,1)."""
    A = [(3.0, 1.0), (0.0, -2.0), (1.0, 0.0), (2.0, 0.0)][:S]
    B_ = [(1.0, 2.0), (0.0, 4.0), (-2.0, 5.0)]
    pts = A + B_
    T = len(pts)
    keys = np.zeros((T, 1, d), np.float32)
    for t, (a, b) in enumerate(pts):
        keys[t, 0, 0], keys[t, 0, 1] = a, b
    values = _normal(13, _VALUES, 0, (T, 1, d))
    q = np.zeros((2, 1, 1, d), np.float32)
    q[0, 0, 0, :2] = (2.0, -1.0)
    q[1, 0, 0, :2] = (0.0, 1.0)
    return DecodeCase("figure2", 1, 1, 1, d, S, 1, "f32", "f32",
                      np.array([T - 1], np.int32), [keys], [values], q,
                      [np.array([1, 0], np.int32)], 2, steps=1)
