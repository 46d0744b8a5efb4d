"""Plain float64 CPU oracle of Quest-style query-aware sparse attention.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Slow and literal on
purpose: every function follows one passage of the pages and is written so a
reader can check it against that passage by eye.  Nothing here is blocked,
fused or reordered beyond what the definitions state.

Sources (cited by page title and section / equation):
  [Quest]      PaperTrace knowledge page "3.1.1 · Quest" (min/max page bounds).
  [PageWeaver] Reading notes on "PageWeaver: KV-Guided Query Unions for
               Sparse Attention" (support semantics, query unions).

Notation follows the Quest page: S = tokens per page, P = pages of a
request, K = pages selected, m/M = per-dimension key min/max of a page,
U_p(q) = page bound.  Query head i reads KV head i // g, where g = H_q/H_kv
(the grouping of consecutive query heads onto one KV head).

Readings taken where the pages leave a step open (each one also listed in
the design notes of the repository):
  * GQA: the per-KV-head score is the max over the group's query heads of
    their bounds ([Quest] §2.1, the group-max aggregate), which keeps eq. (4)
    true for every head of the group.
  * The score is the unscaled bound; no 1/sqrt(d) ([Quest] §1.1 notes the
    ranking is unchanged by that scale).
  * Top-K ties go to the lower page index; if K >= P all P pages are taken;
    the selected list is returned in ascending page order.
  * Only pages j < ceil(L/S) exist; a partially filled tail page is
    summarised over its valid tokens only ([Quest] §1.2, tail length).
  * Softmax scale 1/sqrt(d) ([PageWeaver] eq. (1)-(2)).
  * Decode: the current token is already appended, so c = L - 1.
"""
import math

import numpy as np

from .formats import decode_e4m3fn, encode_e4m3fn_rne


# ---------------------------------------------------------------- pages ----

def num_pages(L, S):
    """Pages holding at least one valid token: ceil(L / S)."""
    return -(-int(L) // int(S))


def page_summaries(keys, L, S):
    """[Quest] §1.1 eq. (1): for every page p and dimension j,
    m_{p,j} = min_r k_j^(r) and M_{p,j} = max_r k_j^(r), taken over the page's
    valid tokens t < L only ([Quest] §1.2, the tail page's valid length).

    keys: float64 [>= L][H_kv][d] in token order.  Returns (m, M), each
    [P][H_kv][d] with P = ceil(L / S)."""
    P = num_pages(L, S)
    H, d = keys.shape[1], keys.shape[2]
    m = np.empty((P, H, d))
    M = np.empty((P, H, d))
    for p in range(P):
        block = keys[p * S: min((p + 1) * S, L)]
        m[p] = block.min(axis=0)
        M[p] = block.max(axis=0)
    return m, M


def append_to_summary(m_p, M_p, k, offset):
    """[Quest] §1.2 eq. (8) and §3 eq. (14): write one key into its page.
    A page receiving its first token (offset 0) starts from max = -inf and
    min = +inf, so afterwards m = M = k.  Returns the new (m_p, M_p)."""
    if offset == 0:
        m_p = np.full_like(k, np.inf)
        M_p = np.full_like(k, -np.inf)
    return np.minimum(m_p, k), np.maximum(M_p, k)


def replay_summaries(keys, L, S):
    """The same summaries built incrementally, one token at a time, with
    eq. (8); used to pin page_summaries (bulk build == incremental append)."""
    P = num_pages(L, S)
    H, d = keys.shape[1], keys.shape[2]
    m = np.zeros((P, H, d))
    M = np.zeros((P, H, d))
    for t in range(L):
        p, off = divmod(t, S)
        m[p], M[p] = append_to_summary(m[p], M[p], keys[t], off)
    return m, M


# --------------------------------------------------------------- scores ----

def head_bounds(q, m, M):
    """[Quest] §1.1 eq. (2)-(3): for query head i (reading KV head i // g) and
    page p, u_{p,j}(q) = max(q_j m_{p,j}, q_j M_{p,j}) and U_p(q) = sum_j u_{p,j}.

    q: [H_q][d]; m, M: [P][H_kv][d].  Returns U: [H_q][P]."""
    H_q, d = q.shape
    P, H_kv, _ = m.shape
    g = H_q // H_kv
    U = np.empty((H_q, P))
    for i in range(H_q):
        h = i // g
        u = np.maximum(q[i][None, :] * m[:, h, :], q[i][None, :] * M[:, h, :])
        U[i] = u.sum(axis=1)
    return U


def kv_head_scores(U_heads, H_kv):
    """[Quest] §2.1 (GQA): one shared page ranking per KV head, using the
    group maximum U_{g,p} = max_{i in group} U_{i,p}.  U_heads: [H_q][P] ->
    [H_kv][P]."""
    H_q, P = U_heads.shape
    g = H_q // H_kv
    out = np.empty((H_kv, P))
    for h in range(H_kv):
        out[h] = U_heads[h * g:(h + 1) * g].max(axis=0)
    return out


# ------------------------------------------------- fp8 page summaries -----
#
# [Quest] §3 (summary dtype): an FP8 summary saves scan bytes but must stay
# an outer interval: the min is quantised toward -inf and the max toward
# +inf, so the bound of eq. (2)-(3) over the stored box is still >= every
# dot product in the page (eq. (4) kept), at the cost of more false
# positives.  Reading taken here: OCP e4m3fn codes with one power-of-two
# scale per (page, KV head), the smallest 2^k with max |m|, |M| <= 448 * 2^k,
# so that scaling is exact and the rounding direction is decided once, on
# the code.

def _e4m3_finite_values():
    codes = np.arange(256, dtype=np.uint8)
    vals = decode_e4m3fn(codes)
    return np.unique(vals[np.isfinite(vals)])          # sorted, -0 == +0


E4M3_MAX = 448.0


def e4m3_down(x):
    """Largest finite e4m3 value <= x (x >= -448), from the value table."""
    vals = _e4m3_finite_values()
    return float(vals[np.searchsorted(vals, x, side="right") - 1])


def e4m3_up(x):
    """Smallest finite e4m3 value >= x (x <= 448), from the value table."""
    vals = _e4m3_finite_values()
    return float(vals[np.searchsorted(vals, x, side="left")])


def summary_scale_exponent(amax):
    """Smallest integer k with amax <= 448 * 2^k (k = 0 for amax = 0)."""
    if amax == 0:
        return 0
    k = 0
    while E4M3_MAX * 2.0 ** k < amax:
        k += 1
    while E4M3_MAX * 2.0 ** (k - 1) >= amax:
        k -= 1
    return k


def fp8_summaries(m, M):
    """Outward-quantised copy of summaries m, M ([P][H][d]): per (page, head)
    the scale s = 2^k of summary_scale_exponent(max |m|, |M|), then
    m_hat = s * e4m3_down(m / s) <= m and M_hat = s * e4m3_up(M / s) >= M.
    Returns (m_hat, M_hat, s [P][H])."""
    P, H, d = m.shape
    m_hat = np.zeros_like(m, dtype=np.float64)
    M_hat = np.zeros_like(M, dtype=np.float64)
    scale = np.ones((P, H))
    for p in range(P):
        for h in range(H):
            amax = max(np.abs(m[p, h]).max(), np.abs(M[p, h]).max())
            s = 2.0 ** summary_scale_exponent(amax)
            scale[p, h] = s
            for j in range(d):
                m_hat[p, h, j] = s * e4m3_down(m[p, h, j] / s)
                M_hat[p, h, j] = s * e4m3_up(M[p, h, j] / s)
    return m_hat, M_hat, scale


def quantize_kv_e4m3(x, scale):
    """FP8 E4M3 K or V of the multi-query path ([PageWeaver] SS2UKVF2: FP8
    E4M3 K/V, BF16 queries): each element of KV head h is stored as the
    code of x / scale[h], rounded to nearest (ties to even) after clamping
    to +-448, and read back as scale[h] * code.  x is [T][H][d] float32; the
    quotient is formed in float32 (the precision of the stored inputs and
    scales, so the code - an integer - is decided in the writer's
    precision).  Returns uint8 codes [T][H][d]."""
    x = np.asarray(x, np.float32)
    s = np.asarray(scale, np.float32)[None, :, None]
    return encode_e4m3fn_rne((x / s).astype(np.float64))


# ---------------------------------------------------------------- top-K ----

def top_k_pages(scores, K):
    """[Quest] §1 / Fig. 1: the K pages with the largest bound.  Order is by
    (score descending, page index ascending); min(K, P) pages are taken and
    returned in ascending page order."""
    scores = np.asarray(scores)
    P = scores.shape[0]
    order = sorted(range(P), key=lambda j: (-scores[j], j))
    return sorted(order[:min(int(K), P)])


# ------------------------------------------- fixed local / sink pages ----

def fixed_pages(L, S, sink_tokens, local_tokens):
    """[Quest] §2.2 and §3.2 (local window and sink kept besides Quest): the
    sink pages are those holding the first ``sink_tokens`` tokens, the local
    pages those holding the last ``local_tokens`` tokens, t in
    [L - local_tokens, L).  Only pages holding a valid token count.  Returns
    (sink set, local set)."""
    P = num_pages(L, S)
    sink = set()
    if sink_tokens > 0:
        sink = set(range(min(P, -(-int(sink_tokens) // S))))
    local = set()
    if local_tokens > 0:
        first = max(0, L - int(local_tokens)) // S
        local = set(range(first, P))
    return sink, local


def mixed_pages(scores, K, L, S, sink_tokens, local_tokens):
    """[Quest] §3.2: C = C_local | C_sink | C_quest, where C_quest is the
    usual top-K over all the request's pages; the three may overlap and a
    page counts once.  Returned in ascending page order."""
    sink, local = fixed_pages(L, S, sink_tokens, local_tokens)
    return sorted(set(top_k_pages(scores, K)) | sink | local)


def quest_budget_pages(total_tokens, local_tokens, sink_tokens, S):
    """[Quest] §2.2 worked budget: after the local window and the sinks, the
    remaining token slots pay for whole Quest pages."""
    return (int(total_tokens) - int(local_tokens) - int(sink_tokens)) // int(S)


# ------------------------------------------------------------ attention ----

def support(page_ids, L, c, S):
    """[PageWeaver] eq. (1)-(2) (support of query i): the tokens t with
    floor(t/S) in the page set, 0 <= t < L and t <= c.  Page IDs outside
    [0, ceil(L/S)) are ignored and a page listed twice counts once."""
    P = num_pages(L, S)
    ids = np.asarray(page_ids, dtype=np.int64).ravel()
    pages = np.unique(ids[(ids >= 0) & (ids < P)])      # valid, each once
    t = (pages[:, None] * S + np.arange(S)[None, :]).ravel()
    return t[(t < L) & (t <= c)]


def attend(q, keys, values, tokens, scale):
    """[PageWeaver] eq. (1)-(2): z_t = scale * q . k_t over the support, then
    o = sum_t e^{z_t} v_t / sum_t e^{z_t}.  An empty support gives o = 0.
    Also returns lse = log sum_t e^{z_t} (-inf for an empty support), the
    quantity a log-sum-exp merge of partial results combines.

    q: [d]; keys, values: [T][d] (one KV head); tokens: indices into them."""
    d = values.shape[1]
    if len(tokens) == 0:
        return np.zeros(d), -np.inf
    k = keys[tokens]
    v = values[tokens]
    z = scale * (k @ q)
    zmax = z.max()
    w = np.exp(z - zmax)
    o = (w @ v) / w.sum()
    return o, zmax + math.log(w.sum())


def decode_request(q, keys, values, L, S, K, scale=None, page_ids=None, sink_tokens=0,
                   local_tokens=0):
    """One decode step of one request, all heads: summaries (eq. (1)), head
    bounds (eq. (2)-(3)), KV-head scores (group max), top-K (joined with the
    fixed sink and local pages when those are asked for, [Quest] §3.2), then
    exact attention over each query head's support with c = L - 1.

    q: [H_q][d]; keys, values: [>= L][H_kv][d] float64.  If ``page_ids``
    ([H_kv][*]) is given it replaces the top-K lists (attention over given
    page sets).  Returns a dict of every intermediate."""
    H_q, d = q.shape
    H_kv = keys.shape[1]
    g = H_q // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    m, M = page_summaries(keys, L, S)
    U_heads = head_bounds(q, m, M)
    U = kv_head_scores(U_heads, H_kv)
    if sink_tokens or local_tokens:
        sel = [mixed_pages(U[h], K, L, S, sink_tokens, local_tokens) for h in range(H_kv)]
    else:
        sel = [top_k_pages(U[h], K) for h in range(H_kv)]
    lists = sel if page_ids is None else page_ids
    out = np.zeros((H_q, d))
    lse = np.zeros(H_q)
    for i in range(H_q):
        h = i // g
        A = support(lists[h], L, L - 1, S)
        out[i], lse[i] = attend(q[i], keys[:, h, :], values[:, h, :], A, scale)
    return {"m": m, "M": M, "U_heads": U_heads, "U": U, "sel": sel,
            "out": out, "lse": lse}


# ------------------------------------------ cache lifecycle (rollback) ----

def rollback_summaries(m, M, keys, L_new, S):
    """[Quest] §3 (cache lifecycle, rollback): when the cache is cut back to
    L_new tokens, pages wholly past the cut are dropped; if the cut falls
    inside a page, the revoked tokens cannot be taken out of its min/max (one
    of them may hold an extreme, and the summary would keep covering a point
    that no longer exists), so that page is rescanned over its surviving
    keys.  Pages before it are full and keep their summaries.

    m, M: [>= ceil(L_new/S)][H_kv][d] summaries before the cut; keys:
    [>= L_new][H_kv][d].  Returns (m, M) of the ceil(L_new/S) kept pages."""
    P = num_pages(L_new, S)
    m2 = np.array(m[:P], dtype=np.float64)
    M2 = np.array(M[:P], dtype=np.float64)
    if L_new % S:
        p = P - 1
        block = keys[p * S:L_new]
        m2[p] = block.min(axis=0)
        M2[p] = block.max(axis=0)
    return m2, M2


# -------------------------------------- per-position speculative selection ---

def speculative_positions(q_block, keys, values, L, S, K, scale=None):
    """[Quest] §1.2 (speculative decoding): a draft of gamma tokens occupies
    positions L - gamma .. L - 1 of the cache (already appended); the query
    of draft position i may see only tokens t <= c_i = L - gamma + i, and it
    depends on the earlier draft tokens, so it ranks pages with its own
    bound instead of reusing another position's set.  Reading taken: every
    position scores the pages that hold a token it may see, pages
    [0, ceil((c_i + 1)/S)), on the summaries of the cache as it stands (all L
    tokens: a bound for every token the position sees), and attends over its
    own top-K support with causal limit c_i.

    q_block: [gamma][H_q][d]; keys, values: [>= L][H_kv][d].  Returns one
    dict per position with its length L_i = c_i + 1, scores U [H_kv][P_i],
    lists sel, out [H_q][d] and lse [H_q]."""
    gamma, H_q, d = q_block.shape
    H_kv = keys.shape[1]
    g = H_q // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    m, M = page_summaries(keys, L, S)
    res = []
    for i in range(gamma):
        c = L - gamma + i
        P_i = num_pages(c + 1, S)
        U = kv_head_scores(head_bounds(q_block[i], m[:P_i], M[:P_i]), H_kv)
        sel = [top_k_pages(U[h], K) for h in range(H_kv)]
        out = np.zeros((H_q, d))
        lse = np.zeros(H_q)
        for qi in range(H_q):
            h = qi // g
            A = support(sel[h], L, c, S)
            out[qi], lse[qi] = attend(q_block[i][qi], keys[:, h, :], values[:, h, :], A, scale)
        res.append({"L": c + 1, "U": U, "sel": sel, "out": out, "lse": lse})
    return res


# ------------------------------------ branch-and-bound exact top-R (§3.2) ---

def branch_and_bound(bounds, page_logits, R):
    """[Quest] §3.2 (stopping rules beyond a fixed top-K): read pages in
    descending bound order (ties to the lower page index), keep tau_R, the
    R-th largest true logit among the tokens read so far, and stop when the
    next unread page's bound is below tau_R: no token of the remaining pages
    can enter the top R.  With fewer than R tokens read the search goes on.

    bounds: [P]; page_logits: list of P arrays, the true logits of each
    page's tokens, paired with token ids as (logit, token) tuples.  Returns
    (pages read in order, top R (logit, token) pairs ordered by logit
    descending then token ascending, tau_R at the stop)."""
    P = len(bounds)
    order = sorted(range(P), key=lambda j: (-bounds[j], j))
    seen = []
    read = []
    for p in order:
        if len(seen) >= R:
            tau = sorted(seen, key=lambda x: (-x[0], x[1]))[R - 1][0]
            if bounds[p] < tau:
                break
        read.append(p)
        seen.extend(page_logits[p])
    top = sorted(seen, key=lambda x: (-x[0], x[1]))[:R]
    tau = top[-1][0] if len(top) >= R else -np.inf
    return read, top, tau


def exact_top_r(q_head, keys_h, L, S, R, m_h, M_h):
    """Exact token top-R of one query head by branch-and-bound over its page
    bounds ([Quest] §1.1 eq. (2)-(3) for this head alone, §3.2): true logits
    are the unscaled dot products q . k_t (the bound's units; a positive
    softmax scale does not reorder them) over tokens t < L.

    q_head: [d]; keys_h: [>= L][d]; m_h, M_h: [P][d] this KV head's
    summaries.  Returns (pages read, top-R (logit, token) pairs, tau_R)."""
    P = num_pages(L, S)
    bounds = np.maximum(q_head[None, :] * m_h[:P], q_head[None, :] * M_h[:P]).sum(axis=1)
    page_logits = []
    for p in range(P):
        toks = range(p * S, min((p + 1) * S, L))
        page_logits.append([(float(keys_h[t] @ q_head), t) for t in toks])
    return branch_and_bound(bounds, page_logits, R)


def brute_top_r(q_head, keys_h, L, R):
    """The R largest logits q . k_t over all tokens t < L, ordered by logit
    descending then token ascending (what the certificate must reproduce)."""
    z = [(float(keys_h[t] @ q_head), t) for t in range(L)]
    return sorted(z, key=lambda x: (-x[0], x[1]))[:R]


# ----------------------------------------------------------- query union ---

def union_with_membership(page_sets):
    """[PageWeaver] query union: U_G = union of the group's page sets, and for
    every row r of the group and union page p a membership bit
    1[p in S_r].  Returns (sorted union list, membership [rows][len(U_G)])."""
    union = sorted({int(p) for s in page_sets for p in s})
    member = np.zeros((len(page_sets), len(union)), dtype=np.uint8)
    for r, s in enumerate(page_sets):
        s = {int(p) for p in s}
        for u, p in enumerate(union):
            member[r, u] = 1 if p in s else 0
    return union, member


# ------------------------------------------------------------- regroup ---

def regroup_window(page_sets, g):
    """[PageWeaver] Algorithm 1 (windowed page-affinity grouping) on one
    window, as the notes walk through it: the lowest unassigned query seeds a
    group with U = its set; the next member is the unassigned query j with the
    smallest (|S_j minus U|, j), after which U grows by S_j and the costs are
    taken again; a group closes at g members or when the window is used up.
    ``page_sets`` are the window's sets in query order; returns the window's
    local indices in execution order (a permutation)."""
    left = list(range(len(page_sets)))
    order = []
    while left:
        seed = min(left)
        left.remove(seed)
        group = [seed]
        U = set(page_sets[seed])
        while len(group) < g and left:
            j = min(left, key=lambda j: (len(set(page_sets[j]) - U), j))
            left.remove(j)
            group.append(j)
            U |= set(page_sets[j])
        order += group
    return order


def regroup(sets, n_pages, q_indptr, window, g, capacity):
    """[PageWeaver] windowed regroup of one KV head's queries: windows of
    ``window`` consecutive queries that stay inside their request; a query's
    set is its deduplicated valid page IDs (0 <= p < n_pages[r]); a request
    with more than ``capacity`` pages keeps the identity order.  Returns ids
    [N]: ids[n] is the original query executed in slot n (a bijection inside
    every request)."""
    ids = []
    for r in range(len(q_indptr) - 1):
        a, b = int(q_indptr[r]), int(q_indptr[r + 1])
        if n_pages[r] > capacity:
            ids += list(range(a, b))
            continue
        for w0 in range(a, b, window):
            w1 = min(b, w0 + window)
            win = [{int(p) for p in sets[n] if 0 <= p < n_pages[r]} for n in range(w0, w1)]
            ids += [w0 + i for i in regroup_window(win, g)]
    return ids


def chunk_attention(q, keys, values, sets, L, c, S, g, scale=None):
    """Multi-query chunk ([PageWeaver] eq. (1)-(2)): every query position n has
    its own page set per KV head, its own length L[n] and causal limit c[n].
    Executing queries as unions with membership masks does not change the
    result, so the definition is applied per query and head.

    q: [N][H_q][d]; keys, values: [T][H_kv][d]; sets: [N][H_kv][*].
    Returns (out [N][H_q][d], lse [N][H_q])."""
    N, H_q, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((N, H_q, d))
    lse = np.zeros((N, H_q))
    for n in range(N):
        for i in range(H_q):
            h = i // g
            A = support(sets[n][h], L[n], c[n], S)
            out[n, i], lse[n, i] = attend(q[n, i], keys[:, h, :],
                                          values[:, h, :], A, scale)
    return out, lse
