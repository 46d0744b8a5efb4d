/*
 * qas.h - C ABI of libqas.so: query-aware sparse attention over a paged KV
 * cache (Quest-style page selection), hand-written HIP for gfx950.
 *
 * Sources are cited by page title and section / equation:
 *   [Quest]      PaperTrace knowledge page "3.1.1 · Quest".
 *   [PageWeaver] Reading notes on "PageWeaver: KV-Guided Query Unions for
 *                Sparse Attention".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership.  Every buffer is owned by the caller.  Pointers documented as
 *   "device" must point to device memory of the current HIP device; the
 *   library keeps no pointer after a call returns and allocates no memory
 *   (scratch space is passed in as a workspace).  The library has no global
 *   state apart from a thread-local error string and the static per-GPU
 *   scratch array of qas_decode_layer_noalloc, and may be called from
 *   several threads.
 * Execution.  Work is enqueued asynchronously on `stream` (a hipStream_t
 *   passed as void*; NULL is the null stream).  No call synchronises.
 * Errors.  Argument problems are reported with a non-zero qas_status
 *   before anything is enqueued; the detail is available from
 *   qas_last_error() on the same thread.  A failed launch returns
 *   QAS_ERR_HIP.  No C++ exception crosses the ABI.
 * Not errors.  Page IDs in selected lists that are negative, beyond the
 *   request's pages, or repeated are semantics, not errors ([PageWeaver]
 *   eq. (1)-(2): invalid IDs are ignored, duplicates count once, an empty
 *   support gives a zero output).
 * Caller contract.  Physical page numbers in page tables must lie in
 *   [0, num_pool_pages); lengths must be covered by the page tables.
 *   Violations are undefined behaviour (they are not checked on the device).
 *
 * Layouts (row-major, innermost last)
 * -----------------------------------
 *   K / V pool  [num_pool_pages][H_kv][S][d]          kv_dtype (an FP8 V pool:
 *                                                     see qas_chunk_attention)
 *   summary     [num_pool_pages][H_kv][2][d]          kv_dtype, [..][0] = min m,
 *                                                     [..][1] = max M ([Quest] eq. (1))
 *   q, out      [B][H_q][d]                           q_dtype (out has q's dtype)
 *   lse         [B][H_q]                              float, natural log of the
 *                                                     softmax denominator
 *   scores      request r, KV head h, logical page j at
 *               page_indptr[r]*H_kv + h*P_r + j, P_r = page_indptr[r+1]-page_indptr[r]
 *   selected    [B][H_kv][stride] int32 logical page IDs
 * Query head i reads KV head i / (H_q / H_kv).
 */
#ifndef QAS_H
#define QAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qas_status {
  QAS_OK = 0,
  QAS_ERR_NULL = 1,        /* a required pointer is NULL                      */
  QAS_ERR_SHAPE = 2,       /* a size is out of range or sizes disagree        */
  QAS_ERR_DTYPE = 3,       /* dtype not accepted for this operand             */
  QAS_ERR_UNSUPPORTED = 4, /* valid request the library does not implement (e.g. head_dim) */
  QAS_ERR_WORKSPACE = 5,   /* workspace NULL, not 16-byte aligned, too small  */
  QAS_ERR_HIP = 6          /* a HIP runtime call or launch failed             */
} qas_status;

typedef enum qas_dtype {
  QAS_F32 = 0,
  QAS_F16 = 1,            /* IEEE binary16                                   */
  QAS_BF16 = 2,           /* bfloat16                                        */
  QAS_FP8_E4M3 = 3        /* OCP FP8 E4M3 (finite variant), with per-KV-head scale */
} qas_dtype;

/* Paged KV cache of one layer. */
typedef struct qas_cache {
  int32_t page_size;      /* S, tokens per page: a power of two in [1, 256]   */
  int32_t head_dim;       /* d: 16, 64 or 128                                 */
  int32_t num_kv_heads;   /* H_kv >= 1                                        */
  int32_t num_pool_pages; /* physical pages in the pool                      */
  int32_t kv_dtype;       /* qas_dtype of K, V and the summaries             */
  int32_t reserved;
  void* k_pool;           /* device [num_pool_pages][H_kv][S][d]              */
  void* v_pool;           /* device [num_pool_pages][H_kv][S][d]              */
  void* summary;          /* device [num_pool_pages][H_kv][2][d]              */
  const float* k_scale;   /* device [H_kv] dequantisation scales (fp8 only, else NULL) */
  const float* v_scale;   /* device [H_kv]                                    */
  /* Optional e4m3 copy of the summaries ([Quest] §3, summary dtype; NULL
   * for none): codes [num_pool_pages][H_kv][2][d] and one scale per
   * (page, KV head) [num_pool_pages][H_kv] float, the smallest power of two
   * 2^k with max |m|, |M| <= 448 * 2^k; min codes round toward -inf and max
   * codes toward +inf, so the copy is an outer interval of the exact record.
   * When given, qas_append and the decode-layer append keep it current next
   * to the exact summary, and page scores (qas_score_pages, the decode
   * layer) are taken from it: half the scan bytes, a bound that is still
   * >= every dot product of the page, and a looser one (more false
   * positives) than the exact summary's. */
  void* summary_fp8;
  float* summary_fp8_scale;
} qas_cache;

/* A batch of B requests (ragged, [Quest] §2.1 continuous batching). */
typedef struct qas_batch {
  int32_t batch;              /* B >= 1                                       */
  int32_t total_pages;        /* page_indptr[B] (host copy, for sizing)       */
  int32_t max_pages;          /* max_r P_r (host copy, for launch sizing)     */
  int32_t reserved;
  const int32_t* seq_lens;    /* device [B]: valid tokens L_r of each request */
  const int32_t* page_indptr; /* device [B+1]: CSR offsets into page_indices  */
  const int32_t* page_indices;/* device [total_pages]: physical page of logical
                                 page j of request r at page_indptr[r] + j    */
} qas_batch;

/*
 * qas_append - write new tokens' K/V rows into the pool and maintain the
 * per-page key min/max summaries ([Quest] §1.2 eq. (8), §3 eq. (14)).
 *
 * batch->seq_lens are the lengths BEFORE the append; request r receives
 * n_r = new_indptr[r+1] - new_indptr[r] tokens at positions
 * seq_lens[r] .. seq_lens[r] + n_r - 1, whose pages must already be in the
 * page table.  A page whose offset-0 token is among the new ones starts
 * from max = -inf / min = +inf (so a recycled physical page never keeps
 * stale extremes); otherwise the existing summary is extended.  Covers both
 * the prefill bulk build (n_r = L_r on empty requests) and single-token
 * decode appends (n_r = 1).  seq_lens is not modified.
 *
 *   new_indptr  device [B+1]
 *   total_new   = new_indptr[B] (host)
 *   max_new     >= max_r n_r (host, for launch sizing)
 *   k_new/v_new device [total_new][H_kv][d], kv_dtype
 */
qas_status qas_append(const qas_cache* cache, const qas_batch* batch,
                      const int32_t* new_indptr, int32_t total_new,
                      int32_t max_new, const void* k_new, const void* v_new,
                      void* stream);

/*
 * qas_append_fp8 - write new tokens' K/V rows into the FP8 E4M3 cache that
 * qas_chunk_attention reads ([PageWeaver] SS2UKVF2: FP8 E4M3 K/V with a
 * per-KV-head scale, BF16 queries).  Each element x of KV head h is stored
 * as the e4m3 code of x / scale[h] (quotient in fp32, clamped to +-448,
 * rounded to the nearest code, ties to even; k_scale for K, v_scale for V),
 * so the chunk call reads scale[h] * code.  Codes are placed in the MFMA
 * operand order of qas_chunk_attention's pools: a (page, KV head) tile the
 * new tokens open is written whole, with zero codes in its rows past the
 * new tokens; a tile they extend keeps its earlier rows.  No summary is kept
 * (the chunk path reads none).
 *
 * batch->seq_lens are the lengths BEFORE the append, and new_indptr /
 * total_new / max_new are as in qas_append.
 *   cache         kv_dtype QAS_FP8_E4M3, head_dim 128, page_size 32 or 64,
 *                 k_pool / v_pool / k_scale / v_scale given
 *   k_new, v_new  device [total_new][H_kv][128] in new_dtype (QAS_F32,
 *                 QAS_F16 or QAS_BF16)
 * Errors: QAS_ERR_DTYPE for a cache that is not FP8, QAS_ERR_UNSUPPORTED
 * for other input dtypes, head sizes or page sizes.
 */
qas_status qas_append_fp8(const qas_cache* cache, const qas_batch* batch,
                          const int32_t* new_indptr, int32_t total_new,
                          int32_t max_new, const void* k_new, const void* v_new,
                          int32_t new_dtype, void* stream);

/*
 * qas_rollback - restore the summaries after the cache is cut back
 * ([Quest] §3, cache lifecycle: rollback).  batch->seq_lens are the lengths
 * AFTER the cut.  Pages wholly past a request's new length are the caller's
 * to drop from its page table (their records are no longer read).  If the
 * new length ends inside a page, the revoked tokens cannot be taken out of
 * that page's min/max, so its record is rebuilt from the surviving keys in
 * the pool (tokens [p*S, L) of tail page p = (L-1)/S), starting from
 * -inf/+inf, and the e4m3 copy, if the cache has one, is re-quantised.  The
 * pool's K/V rows are not touched; later appends at the cut overwrite the
 * revoked rows.  Requests with L = 0, L a multiple of S, or a tail page
 * outside their page-table row are left alone.  One launch, asynchronous on
 * `stream`; argument errors return before anything is enqueued.
 */
qas_status qas_rollback(const qas_cache* cache, const qas_batch* batch, void* stream);

/*
 * qas_score_pages - page bounds of the current queries ([Quest] §1.1
 * eq. (2)-(3)): U_{h,j} = max over the query heads i of KV head h of
 * sum_d max(q_{i,d} m_{j,d}, q_{i,d} M_{j,d}), unscaled, fp32 accumulate
 * ([Quest] §2.1 group-max aggregate for GQA).  Pages j < ceil(L_r/S) are
 * scored; allocated pages beyond them get -inf.
 *
 *   q        device [B][H_q][d], q_dtype == kv_dtype (f32/f16/bf16)
 *   scores   device float, layout above (total_pages * H_kv floats)
 */
qas_status qas_score_pages(const qas_cache* cache, const qas_batch* batch,
                           const void* q, int32_t q_dtype, int32_t num_q_heads,
                           float* scores, void* stream);

/*
 * qas_topk_pages - per (request, KV head) the min(k, ceil(L_r/S)) pages with
 * the largest score, ordered by (score descending, page index ascending);
 * written in ascending page order and padded with -1 ([Quest] §1, Fig. 1
 * Top-K stage).  -0.0 and +0.0 are equal scores.  NaN scores are not
 * supported.
 *
 *   scores     device float, layout of qas_score_pages
 *   sel        device [B][H_kv][k] int32
 *   sel_count  device [B][H_kv] int32, may be NULL
 *   Rows longer than 16384 pages return QAS_ERR_UNSUPPORTED.
 */
qas_status qas_topk_pages(const float* scores, const qas_batch* batch,
                          int32_t num_kv_heads, int32_t page_size, int32_t k,
                          int32_t* sel, int32_t* sel_count, void* stream);

/*
 * qas_selection_capacity - entries a selected list can hold when the top-k
 * is joined with fixed pages: k + ceil(sink_tokens / S) + (local_tokens > 0 ?
 * ceil(local_tokens / S) + 1 : 0).  Returns 0 for invalid arguments.
 */
int32_t qas_selection_capacity(int32_t k, int32_t page_size, int32_t sink_tokens,
                               int32_t local_tokens);

/*
 * qas_select_pages - the candidate set C = C_local | C_sink | C_quest of
 * [Quest] §3.2 (local window and sinks kept besides the Quest pages, §2.2):
 * C_quest is the top-k of qas_topk_pages over all of the row's pages, C_sink
 * the pages holding tokens [0, sink_tokens), C_local the pages holding tokens
 * [L_r - local_tokens, L_r); a page in several sets counts once.  Written in
 * ascending page order, padded with -1 to sel_stride; sel_count (may be
 * NULL) receives |C| per row.  sink_tokens = local_tokens = 0 is
 * qas_topk_pages.
 *   sel        device [B][H_kv][sel_stride] int32,
 *              sel_stride >= qas_selection_capacity(k, S, sink, local)
 */
qas_status qas_select_pages(const float* scores, const qas_batch* batch,
                            int32_t num_kv_heads, int32_t page_size, int32_t k,
                            int32_t sink_tokens, int32_t local_tokens,
                            int32_t* sel, int32_t sel_stride, int32_t* sel_count,
                            void* stream);

/*
 * qas_sparse_decode - exact softmax attention of each query head over its
 * support ([PageWeaver] eq. (1)-(2); [Quest] §2.1 paged sparse load):
 * A = { t : floor(t/S) in the KV head's selected list, t < L_r } (decode,
 * c = L_r - 1), z_t = sm_scale * q . k_t, out = sum softmax(z)_t v_t.
 * Selected lists may hold duplicates, invalid IDs and any order; an empty
 * support gives out = 0 and lse = -inf.  K/V are read in place through the
 * page table (no gather copy); split-page partial softmax states are merged
 * with log-sum-exp.
 *
 *   sel        device [B][H_kv][sel_stride] int32, first sel_len used per row
 *   out        device [B][H_q][d], q_dtype
 *   lse        device [B][H_q] float, may be NULL
 *   workspace  device, >= qas_workspace_bytes(QAS_OP_SPARSE_DECODE, ...)
 */
qas_status qas_sparse_decode(const qas_cache* cache, const qas_batch* batch,
                             const void* q, int32_t q_dtype,
                             int32_t num_q_heads, const int32_t* sel,
                             int32_t sel_stride, int32_t sel_len,
                             float sm_scale, void* out, float* lse,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * qas_decode_layer - one decode-layer call of the whole path: optional
 * append of the current token, page scores, top-k, sparse attention.
 * If k_new/v_new (device [B][H_kv][d], kv_dtype) are given, the token at
 * position seq_lens[r] - 1 of each request is appended first (seq_lens
 * already count it).  sel_out (device [B][H_kv][k] int32) may be NULL;
 * otherwise it receives the selected lists.  Other arguments as in the
 * calls above.
 */
qas_status qas_decode_layer(const qas_cache* cache, const qas_batch* batch,
                            const void* q, int32_t q_dtype,
                            int32_t num_q_heads, int32_t k, float sm_scale,
                            const void* k_new, const void* v_new,
                            int32_t* sel_out, void* out, float* lse,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * qas_decode_layer_mixed - qas_decode_layer whose lists are the candidate
 * set of qas_select_pages (top-k joined with the sink pages of the first
 * sink_tokens tokens and the local pages of the last local_tokens tokens,
 * [Quest] §2.2, §3.2).  sel_out, if given, is [B][H_kv][cap] with cap =
 * qas_selection_capacity(k, S, sink_tokens, local_tokens); the workspace
 * must hold qas_workspace_bytes(QAS_OP_DECODE_LAYER, ..., cap).  With
 * sink_tokens = local_tokens = 0 this is qas_decode_layer.
 */
qas_status qas_decode_layer_mixed(const qas_cache* cache, const qas_batch* batch,
                                  const void* q, int32_t q_dtype,
                                  int32_t num_q_heads, int32_t k,
                                  int32_t sink_tokens, int32_t local_tokens,
                                  float sm_scale, const void* k_new,
                                  const void* v_new, int32_t* sel_out, void* out,
                                  float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * qas_decode_layer_noalloc - qas_decode_layer for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same call, kernels and results, with
 * its scratch space (page scores, split partials, counters) taken from a
 * library-owned static device array of QAS_NOALLOC_SCRATCH_BYTES per GPU
 * instead of a caller workspace.  Calls whose qas_workspace_bytes(
 * QAS_OP_DECODE_LAYER, cache, batch, num_q_heads, k) exceeds that maximum
 * return QAS_ERR_WORKSPACE before anything is enqueued.  The call allocates
 * nothing (no hipMalloc / hipFree); on its first use on a device it looks up
 * that device's copy of the array.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (several streams or threads)
 * race and must be serialised by the caller.  Other arguments and errors as
 * in qas_decode_layer.
 */
#define QAS_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
qas_status qas_decode_layer_noalloc(const qas_cache* cache, const qas_batch* batch,
                                    const void* q, int32_t q_dtype,
                                    int32_t num_q_heads, int32_t k, float sm_scale,
                                    const void* k_new, const void* v_new,
                                    int32_t* sel_out, void* out, float* lse,
                                    void* stream);

/*
 * Multi-query chunk ([PageWeaver] eq. (1)-(2) per query; query unions and
 * membership masks, annotations SS2BST9I / AWLR3K97 / 5ALRMYYY).
 *
 * Query n belongs to request r with q_indptr[r] <= n < q_indptr[r+1]; it has
 * its own page set per KV head, sets[n][h][0..kq), and causal limit
 * q_pos[n] = c_n, and attends over
 *   A = { t : floor(t/S) in its set, t < seq_lens[r], t <= c_n }
 * (invalid IDs ignored, duplicates once, empty support -> 0, lse -inf).
 * Queries are executed in groups of `group` consecutive queries of one
 * request; a group's query heads of one KV head form one 32-row tile
 * (group * (H_q / H_kv) <= 32, group <= 8, group * kq <= 1024) that walks
 * the union of the group's page sets with per-query membership masks.
 * Groups are numbered request by request; qas_chunk_groups() bounds their
 * number for sizing.
 */
int32_t qas_chunk_groups(int32_t num_queries, int32_t batch, int32_t group);

/*
 * qas_regroup_queries - windowed page-affinity regroup ([PageWeaver]
 * Algorithm 1, annotations 69BMX58K / TT5ABQLD / AWLR3K97): for every KV
 * head h, each request's queries are cut into windows of `window`
 * consecutive queries; inside a window, the lowest unassigned query seeds a
 * group with union U = its set, and the next member is the unassigned query
 * j with the smallest (|S_j minus U|, j), U growing after every pick, until
 * the group has `group` members.  S_j is query j's deduplicated set of valid
 * page IDs (0 <= p < ceil(L_r / S)).  Writes ids[h][slot] = the original
 * query executed in slot `slot`, a bijection inside every request (groups of
 * `group` consecutive slots are the union kernel's groups).  Requests of more
 * than 1024 pages keep the identity order; group = 1 is the identity.
 *   sets   device [N][H_kv][kq] int32
 *   ids    device [H_kv][N] int32
 *   window in [1, 128] and a multiple of group; group in [1, 8].
 */
qas_status qas_regroup_queries(const qas_batch* batch, const int32_t* q_indptr,
                               int32_t num_queries, const int32_t* sets,
                               int32_t num_kv_heads, int32_t kq, int32_t page_size,
                               int32_t window, int32_t group, int32_t* ids,
                               void* stream);

/*
 * qas_union_pages - union preparation alone: for every group g and KV head
 * h, the ascending union of the group's valid page IDs, its size, and one
 * membership byte per union page (bit i: the query in slot i of the group
 * holds the page).  ids (device [H_kv][N], may be NULL = identity) is an
 * execution order from qas_regroup_queries: group g of head h is then the
 * queries ids[h][slots of g].
 *   union_pages  device [groups][H_kv][group * kq] int32, -1 padded
 *   union_count  device [groups][H_kv] int32
 *   membership   device [groups][H_kv][group * kq] uint8
 * groups = qas_chunk_groups(num_queries, B, group); missing groups get 0.
 */
qas_status qas_union_pages(const qas_batch* batch, const int32_t* q_indptr,
                           int32_t num_queries, const int32_t* sets,
                           int32_t num_kv_heads, int32_t kq, int32_t group,
                           int32_t page_size, const int32_t* ids,
                           int32_t* union_pages, int32_t* union_count,
                           uint8_t* membership, void* stream);

/*
 * qas_chunk_attention - attention of every query of the chunk over its own
 * support, executed over group unions with MFMA tiles.  The cache must be
 * FP8 E4M3 with k_scale/v_scale (k = k_scale[h] * code).  Its pools are
 * laid out for the MFMA operands: each (page, KV head) tile of S * 128 bytes
 * is a sequence of blocks of 64 lanes x 16 bytes (lane l: row = l % 32,
 * hf = l / 32).  K: blocks (tau < S/32, ks < 2, c < 2) in that order, lane
 * l holding token 32*tau + row, dims 64*ks + 32*hf + 16*c + [0, 16).  V:
 * blocks (dt < 4, c < S/32), lane l holding dim 32*dt + row at k slots
 * (S/2)*hf + 16*c + [0, 16), where token t (w = t % 32, tau = t / 32) is k
 * slot (S/2)*((w/4) % 2) + 16*tau + 4*(w/8) + w % 4.  q is bf16
 * [N][H_q][128]; out is bf16 [N][H_q][128], lse float [N][H_q] (may be
 * NULL).  Page size 32 or 64.  QK^T runs with the query row quantised to
 * e4m3 (per-row scale) and PV with probabilities scaled by 256 and
 * quantised to e4m3; running max/sum and accumulation are fp32.  No summary
 * is read and no workspace is needed.  ids (may be NULL) is an execution
 * order as in qas_union_pages; every query still reads its own Q row, set
 * and causal limit and writes its own output row, so the result does not
 * depend on the order beyond rounding.
 */
qas_status qas_chunk_attention(const qas_cache* cache, const qas_batch* batch,
                               const int32_t* q_indptr, int32_t num_queries,
                               const int32_t* q_pos, const void* q, int32_t q_dtype,
                               int32_t num_q_heads, const int32_t* sets, int32_t kq,
                               int32_t group, const int32_t* ids, float sm_scale,
                               void* out, float* lse, void* stream);

/*
 * qas_decode_positions - the decode layer for a speculative verification
 * block ([Quest] §1.2, speculative decoding): each request carries gamma
 * draft tokens, already appended (seq_lens count them), whose queries
 * depend on the earlier drafts, so each draft position selects its own
 * pages instead of sharing one set.  Position i of request r has causal
 * limit c = seq_lens[r] - gamma + i: its query is scored over the pages
 * holding a token t <= c (on the summaries as they stand, a bound for every
 * token it sees), the top-k pages per (position, KV head) are selected
 * (ties to the lower page index), and attention runs over its support with
 * that causal limit.  A position with c < 0 has an empty support: out = 0,
 * lse = -inf.  Requests of more than 4096 pages (the in-kernel top-k)
 * return QAS_ERR_UNSUPPORTED.
 *
 *   q        device [B][gamma][H_q][d], kv_dtype
 *   sel_out  device [B][gamma][H_kv][k] int32 or NULL (lists, -1 padded)
 *   out      device [B][gamma][H_q][d], kv_dtype
 *   lse      device [B][gamma][H_q] float, may be NULL
 *   workspace >= qas_positions_workspace_bytes(cache, batch, H_q, gamma, k),
 *            16-byte aligned
 */
qas_status qas_decode_positions(const qas_cache* cache, const qas_batch* batch,
                                const void* q, int32_t q_dtype, int32_t num_q_heads,
                                int32_t gamma, int32_t k, float sm_scale,
                                int32_t* sel_out, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * qas_exact_top_r - exact token top-R per (request, query head) with a
 * branch-and-bound certificate ([Quest] §3.2, stopping rules beyond a fixed
 * top-K): pages are read in descending order of this head's bound (eq.
 * (2)-(3) with its own query; ties to the lower page index), and the search
 * stops when the next page's bound is below tau_R, the R-th largest logit
 * read so far; no token of an unread page can then enter the top R.  The
 * bound is raised by 2^-15 * sum_j |q_j| max(|m_j|, |M_j|) so that fp32
 * rounding of bounds and logits cannot end the search early.  Logits are the
 * unscaled dot products q . k_t (fp32) over tokens t < seq_lens[r]; the
 * number of pages read is data dependent (up to all of them).  Four
 * launches: the bounds of every page; per row a pilot that reads pages in
 * bound order, in rounds of whole pages within 64 pages, and finishes the
 * row if the stop rule fires (it hands over early when its bounds are loose
 * against the logits it has read); otherwise every unread page whose bound
 * is not below the pilot's tau_R (which can only rise) is read by many
 * workgroups at once, and a merge keeps the best R.  The result does not
 * depend on that schedule; pages_read counts the pages actually read.
 *
 *   q           device [B][H_q][d], kv_dtype (fp32, fp16 or bf16 caches)
 *   R           1 .. 512; requests of up to 4096 pages (else QAS_ERR_UNSUPPORTED)
 *   top_tokens  device [B][H_q][R] int32: token positions ordered by logit
 *               descending, then position ascending; -1 past the tokens held
 *   top_logits  device [B][H_q][R] float: their logits, -inf past the end
 *   pages_read  device [B][H_q] int32 or NULL: pages read (pilot and scan)
 */
qas_status qas_exact_top_r(const qas_cache* cache, const qas_batch* batch, const void* q,
                           int32_t q_dtype, int32_t num_q_heads, int32_t R,
                           int32_t* top_tokens, float* top_logits, int32_t* pages_read,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace of qas_exact_top_r (16-byte aligned); 0 for invalid arguments. */
size_t qas_exact_top_r_workspace_bytes(const qas_cache* cache, const qas_batch* batch,
                                       int32_t num_q_heads, int32_t R);

/* Workspace of qas_decode_positions; 0 for invalid arguments. */
size_t qas_positions_workspace_bytes(const qas_cache* cache, const qas_batch* batch,
                                     int32_t num_q_heads, int32_t gamma, int32_t k);

enum { QAS_OP_SPARSE_DECODE = 1, QAS_OP_DECODE_LAYER = 2 };

/*
 * qas_workspace_bytes - workspace size an operation needs for these
 * arguments (k = sel_len for QAS_OP_SPARSE_DECODE, the budget for
 * QAS_OP_DECODE_LAYER).  Returns 0 for invalid arguments.  A workspace must
 * be 16-byte aligned (the decode layer reads its page scores as 16-byte
 * words); allocations of hipMalloc and torch are.
 */
size_t qas_workspace_bytes(int32_t op, const qas_cache* cache,
                           const qas_batch* batch, int32_t num_q_heads,
                           int32_t k);

/* Static description of a status code. */
const char* qas_status_string(int32_t status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* qas_last_error(void);

/* Library version string. */
const char* qas_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QAS_H */
