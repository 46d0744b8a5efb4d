// Host side of the libqas C ABI: argument validation, workspace carving and
// launch geometry.  Every check runs before anything is enqueued, so an
// error status means the stream was left untouched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "qas.h"
#include <stdint.h>
#include "qas_internal.h"

namespace {

thread_local char g_err[512] = "";

qas_status fail(qas_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

qas_status ok() {
  g_err[0] = '\0';
  return QAS_OK;
}

qas_status hip_fail(hipError_t e, const char* what) {
  return fail(QAS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

qas_status check_cache(const qas_cache* c, bool need_pools, bool need_summary) {
  if (!c) return fail(QAS_ERR_NULL, "cache is NULL");
  if (!pow2_in(c->page_size, 1, 256))
    return fail(QAS_ERR_SHAPE, "page_size %d is not a power of two in [1, 256]", c->page_size);
  if (c->num_kv_heads < 1) return fail(QAS_ERR_SHAPE, "num_kv_heads %d < 1", c->num_kv_heads);
  if (c->num_pool_pages < 1) return fail(QAS_ERR_SHAPE, "num_pool_pages %d < 1", c->num_pool_pages);
  if (c->head_dim != 16 && c->head_dim != 64 && c->head_dim != 128)
    return fail(QAS_ERR_UNSUPPORTED, "head_dim %d not in {16, 64, 128}", c->head_dim);
  if (c->kv_dtype != QAS_F32 && c->kv_dtype != QAS_F16 && c->kv_dtype != QAS_BF16)
    return fail(QAS_ERR_DTYPE, "kv_dtype %d not supported by the decode path (f32/f16/bf16)",
                c->kv_dtype);
  if (need_pools && (!c->k_pool || !c->v_pool)) return fail(QAS_ERR_NULL, "k_pool/v_pool is NULL");
  if (need_summary && !c->summary) return fail(QAS_ERR_NULL, "summary is NULL");
  if ((c->summary_fp8 == nullptr) != (c->summary_fp8_scale == nullptr))
    return fail(QAS_ERR_NULL, "summary_fp8 and summary_fp8_scale must both be given or NULL");
  if (c->summary_fp8 && !qas::score8_supported(c->head_dim, c->num_kv_heads))
    return fail(QAS_ERR_UNSUPPORTED, "fp8 summaries: %d KV heads of d=%d exceed 512 lanes",
                c->num_kv_heads, c->head_dim);
  if (c->summary_fp8 && !c->summary)
    return fail(QAS_ERR_NULL, "an fp8 summary copy needs the exact summary");
  return QAS_OK;
}

qas_status check_batch(const qas_batch* b) {
  if (!b) return fail(QAS_ERR_NULL, "batch is NULL");
  if (b->batch < 1) return fail(QAS_ERR_SHAPE, "batch %d < 1", b->batch);
  if (b->total_pages < 0 || b->max_pages < 0)
    return fail(QAS_ERR_SHAPE, "negative total_pages / max_pages");
  if (b->max_pages > b->total_pages)
    return fail(QAS_ERR_SHAPE, "max_pages %d > total_pages %d", b->max_pages, b->total_pages);
  if (!b->seq_lens || !b->page_indptr || (!b->page_indices && b->total_pages > 0))
    return fail(QAS_ERR_NULL, "seq_lens / page_indptr / page_indices is NULL");
  return QAS_OK;
}

qas_status check_heads(const qas_cache* c, int num_q_heads, int* g) {
  if (num_q_heads < 1 || num_q_heads % c->num_kv_heads != 0)
    return fail(QAS_ERR_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, c->num_kv_heads);
  *g = num_q_heads / c->num_kv_heads;
  if (*g != 1 && *g != 2 && *g != 4 && *g != 8)
    return fail(QAS_ERR_UNSUPPORTED, "group size %d not in {1, 2, 4, 8}", *g);
  return QAS_OK;
}

// Workspace layout:
//   sparse decode: [split partials][tickets]
//   decode layer:  [scores][physical pages][split partials][tickets], plus [sel][sel_phys]
//                  for rows too long for the in-kernel top-K
struct DecodePlan {
  int n_split;
  size_t partial_bytes;
  size_t ticket_bytes;
};

DecodePlan plan_decode(const qas_cache* c, const qas_batch* b, int num_q_heads, int sel_len) {
  DecodePlan p;
  p.n_split = qas::decode_num_splits(b->batch * c->num_kv_heads, sel_len);
  p.partial_bytes = align256((size_t)b->batch * num_q_heads * p.n_split *
                             (c->head_dim + 2) * sizeof(float));
  p.ticket_bytes = align256((size_t)b->batch * c->num_kv_heads * sizeof(unsigned int));
  return p;
}

// Scores of the decode layer: [B][H_kv][max_pages] when the attention kernel
// selects in-kernel (fixed row stride), else the packed qas_score_pages layout.
bool layer_fused_topk(const qas_batch* b);
// Row stride of the fixed-stride layout: max_pages rounded up to 4 entries,
// so that with a 16-byte aligned workspace every row starts 16-byte aligned
// and the attention kernel reads its row as 16-byte words.
int layer_score_stride(const qas_batch* b) { return (b->max_pages + 3) & ~3; }
size_t layer_scores_bytes(const qas_cache* c, const qas_batch* b) {
  const size_t n = layer_fused_topk(b) ? (size_t)b->batch * layer_score_stride(b)
                                       : (size_t)b->total_pages;
  return align256(n * c->num_kv_heads * sizeof(float));
}

// Physical page of each scored page, [B][stride] int32, beside the scores:
// the attention kernel reads it as 16-byte words instead of the caller's
// page table (whose rows need not be aligned).
size_t layer_phys_bytes(const qas_batch* b) {
  return layer_fused_topk(b) ? align256((size_t)b->batch * layer_score_stride(b) * sizeof(int32_t))
                             : 0;
}

bool layer_fused_topk(const qas_batch* b) {
  return b->max_pages <= qas::decode_fused_topk_max_pages();
}

size_t layer_sel_bytes(const qas_cache* c, const qas_batch* b, int k) {
  if (layer_fused_topk(b)) return 0;
  return align256((size_t)b->batch * c->num_kv_heads * k * sizeof(int32_t));
}

qas::ScoreArgs score_args(const qas_cache* c, const qas_batch* b, const void* q, int num_q_heads,
                          int g, float* scores) {
  qas::ScoreArgs a;
  a.summary = c->summary;
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.k_pool = c->k_pool;
  a.v_pool = c->v_pool;
  a.q = q;
  a.seq_lens = b->seq_lens;
  a.page_indptr = b->page_indptr;
  a.page_indices = b->page_indices;
  a.scores = scores;
  a.B = b->batch;
  a.H_kv = c->num_kv_heads;
  a.H_q = num_q_heads;
  a.d = c->head_dim;
  a.S = c->page_size;
  a.max_pages = b->max_pages;
  a.kv_dtype = c->kv_dtype;
  a.g = g;
  a.summary_fp8 = c->summary_fp8;
  a.summary_fp8_scale = c->summary_fp8_scale;
  a.pages_per_iter = c->summary_fp8
                         ? qas::score8_pages_per_iter(c->head_dim, c->num_kv_heads)
                         : qas::score_pages_per_iter(c->kv_dtype, c->head_dim, c->num_kv_heads);
  a.tickets = nullptr;
  a.row_stride = 0;
  a.phys_out = nullptr;
  a.gamma = 1;
  return a;
}

qas::DecodeArgs decode_args(const qas_cache* c, const qas_batch* b, const void* q,
                            int num_q_heads, int g, const int32_t* sel, int sel_stride,
                            int sel_len, float sm_scale, void* out, float* lse, float* partials,
                            int n_split, int dedupe) {
  qas::DecodeArgs a;
  a.k_pool = c->k_pool;
  a.v_pool = c->v_pool;
  a.q = q;
  a.seq_lens = b->seq_lens;
  a.page_indptr = b->page_indptr;
  a.page_indices = b->page_indices;
  a.sel = sel;
  a.sel_phys = nullptr;
  a.out = out;
  a.lse = lse;
  a.partials = partials;
  a.B = b->batch;
  a.H_kv = c->num_kv_heads;
  a.H_q = num_q_heads;
  a.d = c->head_dim;
  a.S = c->page_size;
  a.kv_dtype = c->kv_dtype;
  a.g = g;
  a.sel_stride = sel_stride;
  a.sel_len = sel_len;
  a.n_split = n_split;
  a.dedupe = dedupe;
  a.sm_scale = sm_scale;
  a.tickets = nullptr;
  a.scores = nullptr;
  a.score_stride = 0;
  a.phys_rows = nullptr;
  a.gamma = 1;
  a.sel_out = nullptr;
  a.max_pages = b->max_pages;
  a.clear_tickets = 0;
  a.k = sel_len;
  a.sink_tokens = 0;
  a.local_tokens = 0;
  return a;
}

qas::AppendArgs append_args(const qas_cache* c, const qas_batch* b, const int32_t* new_indptr,
                            int max_new, const void* k_new, const void* v_new) {
  qas::AppendArgs a;
  a.k_pool = c->k_pool;
  a.v_pool = c->v_pool;
  a.summary = c->summary;
  a.k_new = k_new;
  a.v_new = v_new;
  a.seq_lens = b->seq_lens;
  a.new_indptr = new_indptr;
  a.page_indptr = b->page_indptr;
  a.page_indices = b->page_indices;
  a.B = b->batch;
  a.H_kv = c->num_kv_heads;
  a.d = c->head_dim;
  a.S = c->page_size;
  a.kv_dtype = c->kv_dtype;
  a.max_new = max_new;
  a.summary_fp8 = c->summary_fp8;
  a.summary_fp8_scale = c->summary_fp8_scale;
  a.rescan = 0;
  return a;
}

}  // namespace

extern "C" {

const char* qas_version(void) { return "qas 0.1.0 (gfx950)"; }

const char* qas_last_error(void) { return g_err; }

const char* qas_status_string(int32_t s) {
  switch (s) {
    case QAS_OK: return "ok";
    case QAS_ERR_NULL: return "null pointer";
    case QAS_ERR_SHAPE: return "bad shape";
    case QAS_ERR_DTYPE: return "unsupported dtype";
    case QAS_ERR_UNSUPPORTED: return "unsupported configuration";
    case QAS_ERR_WORKSPACE: return "workspace too small";
    case QAS_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

size_t qas_workspace_bytes(int32_t op, const qas_cache* cache, const qas_batch* batch,
                           int32_t num_q_heads, int32_t k) {
  if (!cache || !batch || batch->batch < 1 || cache->num_kv_heads < 1 || num_q_heads < 1 ||
      k < 1)
    return 0;
  const DecodePlan p = plan_decode(cache, batch, num_q_heads, k);
  if (op == QAS_OP_SPARSE_DECODE) return p.partial_bytes + p.ticket_bytes;
  if (op == QAS_OP_DECODE_LAYER)
    return layer_scores_bytes(cache, batch) + layer_phys_bytes(batch) + p.partial_bytes +
           p.ticket_bytes + 2 * layer_sel_bytes(cache, batch, k);
  return 0;
}

qas_status qas_append(const qas_cache* cache, const qas_batch* batch, const int32_t* new_indptr,
                      int32_t total_new, int32_t max_new, const void* k_new, const void* v_new,
                      void* stream) {
  qas_status st = check_cache(cache, true, true);
  if (st) return st;
  if ((st = check_batch(batch))) return st;
  if (!new_indptr) return fail(QAS_ERR_NULL, "new_indptr is NULL");
  if (total_new < 0 || max_new < 0 || max_new > total_new)
    return fail(QAS_ERR_SHAPE, "total_new %d / max_new %d inconsistent", total_new, max_new);
  if (total_new == 0) return ok();
  if (!k_new || !v_new) return fail(QAS_ERR_NULL, "k_new / v_new is NULL");
  if (!qas::append_supported(cache->kv_dtype, cache->head_dim))
    return fail(QAS_ERR_UNSUPPORTED, "append: dtype %d / head_dim %d", cache->kv_dtype,
                cache->head_dim);
  qas::AppendArgs a = append_args(cache, batch, new_indptr, max_new, k_new, v_new);
  hipError_t e = qas::launch_append(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

qas_status qas_append_fp8(const qas_cache* cache, const qas_batch* batch,
                          const int32_t* new_indptr, int32_t total_new, int32_t max_new,
                          const void* k_new, const void* v_new, int32_t new_dtype,
                          void* stream) {
  if (!cache) return fail(QAS_ERR_NULL, "cache is NULL");
  if (cache->kv_dtype != QAS_FP8_E4M3)
    return fail(QAS_ERR_DTYPE, "kv_dtype %d: the fp8 writer needs an FP8 E4M3 cache",
                cache->kv_dtype);
  if (cache->num_kv_heads < 1) return fail(QAS_ERR_SHAPE, "num_kv_heads %d < 1", cache->num_kv_heads);
  if (cache->num_pool_pages < 1)
    return fail(QAS_ERR_SHAPE, "num_pool_pages %d < 1", cache->num_pool_pages);
  if (!qas::append_fp8_supported(new_dtype, cache->head_dim, cache->page_size))
    return fail(QAS_ERR_UNSUPPORTED,
                "fp8 writer: inputs f32/f16/bf16, d = 128, page size 32 or 64 "
                "(dtype %d, d %d, S %d)", new_dtype, cache->head_dim, cache->page_size);
  if (!cache->k_pool || !cache->v_pool || !cache->k_scale || !cache->v_scale)
    return fail(QAS_ERR_NULL, "k_pool / v_pool / k_scale / v_scale is NULL");
  qas_status st = check_batch(batch);
  if (st) return st;
  if (!new_indptr) return fail(QAS_ERR_NULL, "new_indptr is NULL");
  if (total_new < 0 || max_new < 0 || max_new > total_new)
    return fail(QAS_ERR_SHAPE, "total_new %d / max_new %d inconsistent", total_new, max_new);
  if (total_new == 0) return ok();
  if (!k_new || !v_new) return fail(QAS_ERR_NULL, "k_new / v_new is NULL");
  qas::Fp8AppendArgs a;
  a.k_pool = cache->k_pool;
  a.v_pool = cache->v_pool;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_dtype = new_dtype;
  a.seq_lens = batch->seq_lens;
  a.new_indptr = new_indptr;
  a.page_indptr = batch->page_indptr;
  a.page_indices = batch->page_indices;
  a.B = batch->batch;
  a.H_kv = cache->num_kv_heads;
  a.S = cache->page_size;
  a.max_new = max_new;
  hipError_t e = qas::launch_append_fp8(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fp8 append launch");
  return ok();
}

qas_status qas_rollback(const qas_cache* cache, const qas_batch* batch, void* stream) {
  qas_status st = check_cache(cache, true, true);
  if (st) return st;
  if ((st = check_batch(batch))) return st;
  if (!qas::append_supported(cache->kv_dtype, cache->head_dim))
    return fail(QAS_ERR_UNSUPPORTED, "rollback: dtype %d / head_dim %d", cache->kv_dtype,
                cache->head_dim);
  if (batch->batch == 0) return ok();
  qas::AppendArgs a = append_args(cache, batch, nullptr, 0, nullptr, nullptr);
  a.rescan = 1;
  hipError_t e = qas::launch_append(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rollback launch");
  return ok();
}

qas_status qas_score_pages(const qas_cache* cache, const qas_batch* batch, const void* q,
                           int32_t q_dtype, int32_t num_q_heads, float* scores, void* stream) {
  qas_status st = check_cache(cache, false, true);
  if (st) return st;
  if ((st = check_batch(batch))) return st;
  int g;
  if ((st = check_heads(cache, num_q_heads, &g))) return st;
  if (!q || !scores) return fail(QAS_ERR_NULL, "q / scores is NULL");
  if (q_dtype != cache->kv_dtype)
    return fail(QAS_ERR_DTYPE, "q_dtype %d must equal kv_dtype %d", q_dtype, cache->kv_dtype);
  if (!qas::score_supported(cache->kv_dtype, cache->head_dim, g, cache->num_kv_heads))
    return fail(QAS_ERR_UNSUPPORTED, "score: %d KV heads of d=%d", cache->num_kv_heads,
                cache->head_dim);
  if (batch->max_pages == 0) return ok();
  qas::ScoreArgs a = score_args(cache, batch, q, num_q_heads, g, scores);
  hipError_t e = qas::launch_score(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "score launch");
  return ok();
}

int32_t qas_selection_capacity(int32_t k, int32_t page_size, int32_t sink_tokens,
                               int32_t local_tokens) {
  if (k < 1 || page_size < 1 || sink_tokens < 0 || local_tokens < 0) return 0;
  const int64_t cap = (int64_t)k + (sink_tokens + (int64_t)page_size - 1) / page_size +
                      (local_tokens > 0 ? (local_tokens + (int64_t)page_size - 1) / page_size + 1
                                        : 0);
  return cap > INT32_MAX ? 0 : (int32_t)cap;
}

qas_status qas_select_pages(const float* scores, const qas_batch* batch, int32_t num_kv_heads,
                            int32_t page_size, int32_t k, int32_t sink_tokens,
                            int32_t local_tokens, int32_t* sel, int32_t sel_stride,
                            int32_t* sel_count, void* stream) {
  qas_status st = check_batch(batch);
  if (st) return st;
  if (!scores || !sel) return fail(QAS_ERR_NULL, "scores / sel is NULL");
  if (num_kv_heads < 1) return fail(QAS_ERR_SHAPE, "num_kv_heads %d < 1", num_kv_heads);
  if (!pow2_in(page_size, 1, 256)) return fail(QAS_ERR_SHAPE, "page_size %d", page_size);
  if (k < 1) return fail(QAS_ERR_SHAPE, "k %d < 1", k);
  if (sink_tokens < 0 || local_tokens < 0)
    return fail(QAS_ERR_SHAPE, "sink_tokens %d / local_tokens %d < 0", sink_tokens, local_tokens);
  const int32_t cap = qas_selection_capacity(k, page_size, sink_tokens, local_tokens);
  if (cap < 1 || sel_stride < cap)
    return fail(QAS_ERR_SHAPE, "sel_stride %d < qas_selection_capacity %d", sel_stride, cap);
  if (batch->max_pages > qas::kTopkMaxPages)
    return fail(QAS_ERR_UNSUPPORTED, "rows of %d pages exceed %d", batch->max_pages,
                qas::kTopkMaxPages);
  qas::TopkArgs a;
  a.scores = scores;
  a.seq_lens = batch->seq_lens;
  a.page_indptr = batch->page_indptr;
  a.page_indices = batch->page_indices;
  a.sel = sel;
  a.sel_phys = nullptr;
  a.sel_count = sel_count;
  a.B = batch->batch;
  a.H_kv = num_kv_heads;
  a.S = page_size;
  a.k = k;
  a.max_pages = batch->max_pages;
  a.sink_tokens = sink_tokens;
  a.local_tokens = local_tokens;
  a.sel_stride = sel_stride;
  hipError_t e = qas::launch_topk(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return ok();
}

qas_status qas_topk_pages(const float* scores, const qas_batch* batch, int32_t num_kv_heads,
                          int32_t page_size, int32_t k, int32_t* sel, int32_t* sel_count,
                          void* stream) {
  return qas_select_pages(scores, batch, num_kv_heads, page_size, k, 0, 0, sel, k, sel_count,
                          stream);
}

qas_status qas_sparse_decode(const qas_cache* cache, const qas_batch* batch, const void* q,
                             int32_t q_dtype, int32_t num_q_heads, const int32_t* sel,
                             int32_t sel_stride, int32_t sel_len, float sm_scale, void* out,
                             float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  qas_status st = check_cache(cache, true, false);
  if (st) return st;
  if ((st = check_batch(batch))) return st;
  int g;
  if ((st = check_heads(cache, num_q_heads, &g))) return st;
  if (!q || !out || !sel) return fail(QAS_ERR_NULL, "q / out / sel is NULL");
  if (q_dtype != cache->kv_dtype)
    return fail(QAS_ERR_DTYPE, "q_dtype %d must equal kv_dtype %d", q_dtype, cache->kv_dtype);
  if (sel_len < 1 || sel_stride < sel_len)
    return fail(QAS_ERR_SHAPE, "sel_len %d / sel_stride %d", sel_len, sel_stride);
  if (sel_len > qas::decode_max_dedupe_row())
    return fail(QAS_ERR_UNSUPPORTED, "sel_len %d > %d", sel_len, qas::decode_max_dedupe_row());
  DecodePlan p = plan_decode(cache, batch, num_q_heads, sel_len);
  const size_t need = p.partial_bytes + p.ticket_bytes;
  if (!workspace || workspace_bytes < need)
    return fail(QAS_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(QAS_ERR_WORKSPACE, "workspace %p is not 16-byte aligned", workspace);
  qas::DecodeArgs a = decode_args(cache, batch, q, num_q_heads, g, sel, sel_stride, sel_len,
                                  sm_scale, out, lse, (float*)workspace, p.n_split, 1);
  a.tickets = (unsigned int*)((char*)workspace + p.partial_bytes);
  a.clear_tickets = 1;
  hipError_t e = qas::launch_decode(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

qas_status qas_decode_layer_mixed(const qas_cache* cache, const qas_batch* batch,
                                  const void* q, int32_t q_dtype, int32_t num_q_heads, int32_t k,
                                  int32_t sink_tokens, int32_t local_tokens, float sm_scale,
                                  const void* k_new, const void* v_new, int32_t* sel_out,
                                  void* out, float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  qas_status st = check_cache(cache, true, true);
  if (st) return st;
  if ((st = check_batch(batch))) return st;
  int g;
  if ((st = check_heads(cache, num_q_heads, &g))) return st;
  if (!q || !out) return fail(QAS_ERR_NULL, "q / out is NULL");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(QAS_ERR_NULL, "k_new and v_new must both be given or both be NULL");
  if (q_dtype != cache->kv_dtype)
    return fail(QAS_ERR_DTYPE, "q_dtype %d must equal kv_dtype %d", q_dtype, cache->kv_dtype);
  if (k < 1) return fail(QAS_ERR_SHAPE, "k %d < 1", k);
  if (sink_tokens < 0 || local_tokens < 0)
    return fail(QAS_ERR_SHAPE, "sink_tokens %d / local_tokens %d < 0", sink_tokens, local_tokens);
  const int32_t cap = qas_selection_capacity(k, cache->page_size, sink_tokens, local_tokens);
  if (cap < 1) return fail(QAS_ERR_SHAPE, "selection capacity overflows");
  if (batch->max_pages > qas::kTopkMaxPages)
    return fail(QAS_ERR_UNSUPPORTED, "rows of %d pages exceed %d", batch->max_pages,
                qas::kTopkMaxPages);
  const size_t need = qas_workspace_bytes(QAS_OP_DECODE_LAYER, cache, batch, num_q_heads, cap);
  if (!workspace || workspace_bytes < need)
    return fail(QAS_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(QAS_ERR_WORKSPACE, "workspace %p is not 16-byte aligned", workspace);
  if (!qas::score_supported(cache->kv_dtype, cache->head_dim, g, cache->num_kv_heads))
    return fail(QAS_ERR_UNSUPPORTED, "score: %d KV heads of d=%d", cache->num_kv_heads,
                cache->head_dim);
  hipStream_t s = (hipStream_t)stream;
  const DecodePlan p = plan_decode(cache, batch, num_q_heads, cap);
  char* ws = (char*)workspace;
  float* scores = (float*)ws;
  ws += layer_scores_bytes(cache, batch);
  int32_t* phys_rows = (int32_t*)ws;
  ws += layer_phys_bytes(batch);
  float* partials = (float*)ws;
  ws += p.partial_bytes;
  unsigned int* tickets = (unsigned int*)ws;
  ws += p.ticket_bytes;

  // 1. page bounds (with the current token's append folded in); clears the
  //    attention kernel's tickets
  hipError_t e;
  qas::ScoreArgs sa = score_args(cache, batch, q, num_q_heads, g, scores);
  sa.k_new = k_new;
  sa.v_new = v_new;
  sa.tickets = tickets;
  sa.row_stride = layer_fused_topk(batch) ? layer_score_stride(batch) : 0;
  sa.phys_out = layer_fused_topk(batch) ? phys_rows : nullptr;
  if ((e = qas::launch_score(sa, s)) != hipSuccess) return hip_fail(e, "score launch");
  // lists hold the top-k joined with the fixed pages: cap entries per row
  qas::DecodeArgs da = decode_args(cache, batch, q, num_q_heads, g, nullptr, cap, cap, sm_scale,
                                   out, lse, partials, p.n_split, 0);
  da.tickets = tickets;
  da.k = k;
  da.sink_tokens = sink_tokens;
  da.local_tokens = local_tokens;
  if (layer_fused_topk(batch)) {
    // 2. top-k per (request, KV head) inside the attention kernel
    da.scores = scores;
    da.score_stride = layer_score_stride(batch);
    da.phys_rows = phys_rows;
    da.sel_out = sel_out;
  } else {
    // 2. top-k per (request, KV head) in a kernel of its own (long rows)
    int32_t* sel = sel_out ? sel_out : (int32_t*)ws;
    ws += layer_sel_bytes(cache, batch, cap);
    int32_t* sel_phys = (int32_t*)ws;
    qas::TopkArgs ta;
    ta.scores = scores;
    ta.seq_lens = batch->seq_lens;
    ta.page_indptr = batch->page_indptr;
    ta.page_indices = batch->page_indices;
    ta.sel = sel;
    ta.sel_phys = sel_phys;
    ta.sel_count = nullptr;
    ta.B = batch->batch;
    ta.H_kv = cache->num_kv_heads;
    ta.S = cache->page_size;
    ta.k = k;
    ta.max_pages = batch->max_pages;
    ta.sink_tokens = sink_tokens;
    ta.local_tokens = local_tokens;
    ta.sel_stride = cap;
    if ((e = qas::launch_topk(ta, s)) != hipSuccess) return hip_fail(e, "top-k launch");
    da.sel = sel;
    da.sel_phys = sel_phys;
  }
  // 3. sparse attention with the split merge
  if ((e = qas::launch_decode(da, s)) != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

qas_status qas_decode_layer(const qas_cache* cache, const qas_batch* batch, const void* q,
                            int32_t q_dtype, int32_t num_q_heads, int32_t k, float sm_scale,
                            const void* k_new, const void* v_new, int32_t* sel_out, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return qas_decode_layer_mixed(cache, batch, q, q_dtype, num_q_heads, k, 0, 0, sm_scale, k_new,
                                v_new, sel_out, out, lse, workspace, workspace_bytes, stream);
}

// Workspace of qas_exact_top_r, carved in this order (each part 256-aligned).
struct ToprPlan {
  size_t state, pages, pilot, chunks, counts;
  int page_stride, scan_chunks;
  size_t total() const { return state + pages + pilot + chunks + counts; }
};
ToprPlan plan_topr(const qas_cache* c, const qas_batch* b, int num_q_heads, int R) {
  ToprPlan p;
  const size_t rows = (size_t)b->batch * num_q_heads;
  p.page_stride = b->max_pages > 0 ? b->max_pages : 1;
  const int per_chunk = qas::topr_threads() / c->page_size;   // pages a scan workgroup reads
  p.scan_chunks = (p.page_stride + per_chunk - 1) / per_chunk;
  p.state = align256(rows * 4 * sizeof(int));
  p.pages = align256(rows * p.page_stride * sizeof(uint64_t));
  p.pilot = align256(rows * R * sizeof(uint64_t));
  p.chunks = align256(rows * p.scan_chunks * R * sizeof(uint64_t));
  p.counts = align256(rows * p.scan_chunks * sizeof(int));
  return p;
}

size_t qas_exact_top_r_workspace_bytes(const qas_cache* cache, const qas_batch* batch,
                                       int32_t num_q_heads, int32_t R) {
  if (!cache || !batch || batch->batch < 1 || num_q_heads < 1 || R < 1 ||
      !pow2_in(cache->page_size, 1, 256))
    return 0;
  return plan_topr(cache, batch, num_q_heads, R).total();
}

qas_status qas_exact_top_r(const qas_cache* cache, const qas_batch* batch, const void* q,
                           int32_t q_dtype, int32_t num_q_heads, int32_t R, int32_t* top_tokens,
                           float* top_logits, int32_t* pages_read, void* workspace,
                           size_t workspace_bytes, void* stream) {
  qas_status st = check_cache(cache, true, true);
  if (st) return st;
  if ((st = check_batch(batch))) return st;
  int g;
  if ((st = check_heads(cache, num_q_heads, &g))) return st;
  if (!q || !top_tokens || !top_logits) return fail(QAS_ERR_NULL, "q / top_tokens / top_logits is NULL");
  if (q_dtype != cache->kv_dtype)
    return fail(QAS_ERR_DTYPE, "q_dtype %d must equal kv_dtype %d", q_dtype, cache->kv_dtype);
  if (R < 1) return fail(QAS_ERR_SHAPE, "R %d < 1", R);
  if (R > qas::topr_max_r())
    return fail(QAS_ERR_UNSUPPORTED, "R %d > %d", R, qas::topr_max_r());
  if (batch->max_pages > qas::topr_max_pages())
    return fail(QAS_ERR_UNSUPPORTED, "rows of %d pages exceed %d", batch->max_pages,
                qas::topr_max_pages());
  if (cache->kv_dtype == QAS_FP8_E4M3)
    return fail(QAS_ERR_UNSUPPORTED, "exact top-R reads fp32/fp16/bf16 keys");
  const ToprPlan tp = plan_topr(cache, batch, num_q_heads, R);
  if (!workspace || workspace_bytes < tp.total())
    return fail(QAS_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, tp.total());
  if (reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(QAS_ERR_WORKSPACE, "workspace %p is not 16-byte aligned", workspace);
  qas::ToprArgs a;
  char* ws = (char*)workspace;
  a.ws_state = (int*)ws;
  ws += tp.state;
  a.ws_pages = (uint64_t*)ws;
  ws += tp.pages;
  a.ws_pilot = (uint64_t*)ws;
  ws += tp.pilot;
  a.ws_chunks = (uint64_t*)ws;
  ws += tp.chunks;
  a.ws_counts = (int*)ws;
  a.page_stride = tp.page_stride;
  a.scan_chunks = tp.scan_chunks;
  a.pilot_pages = 64;
  a.k_pool = cache->k_pool;
  a.summary = cache->summary;
  a.q = q;
  a.seq_lens = batch->seq_lens;
  a.page_indptr = batch->page_indptr;
  a.page_indices = batch->page_indices;
  a.top_tokens = top_tokens;
  a.top_logits = top_logits;
  a.pages_read = pages_read;
  a.B = batch->batch;
  a.H_kv = cache->num_kv_heads;
  a.H_q = num_q_heads;
  a.d = cache->head_dim;
  a.S = cache->page_size;
  a.kv_dtype = cache->kv_dtype;
  a.R = R;
  hipError_t e = qas::launch_topr(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "top-R launch");
  return ok();
}

size_t qas_positions_workspace_bytes(const qas_cache* cache, const qas_batch* batch,
                                     int32_t num_q_heads, int32_t gamma, int32_t k) {
  if (!batch || gamma < 1 || batch->batch < 1 || batch->batch > INT32_MAX / gamma) return 0;
  qas_batch rows = *batch;             // one row per (request, draft position)
  rows.batch = batch->batch * gamma;
  return qas_workspace_bytes(QAS_OP_DECODE_LAYER, cache, &rows, num_q_heads, k);
}

qas_status qas_decode_positions(const qas_cache* cache, const qas_batch* batch, const void* q,
                                int32_t q_dtype, int32_t num_q_heads, int32_t gamma, int32_t k,
                                float sm_scale, int32_t* sel_out, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  qas_status st = check_cache(cache, true, true);
  if (st) return st;
  if ((st = check_batch(batch))) return st;
  int g;
  if ((st = check_heads(cache, num_q_heads, &g))) return st;
  if (!q || !out) return fail(QAS_ERR_NULL, "q / out is NULL");
  if (q_dtype != cache->kv_dtype)
    return fail(QAS_ERR_DTYPE, "q_dtype %d must equal kv_dtype %d", q_dtype, cache->kv_dtype);
  if (k < 1) return fail(QAS_ERR_SHAPE, "k %d < 1", k);
  if (gamma < 1 || batch->batch > INT32_MAX / gamma)
    return fail(QAS_ERR_SHAPE, "gamma %d out of range", gamma);
  if (!layer_fused_topk(batch))
    return fail(QAS_ERR_UNSUPPORTED, "rows of %d pages exceed the in-kernel top-k (%d)",
                batch->max_pages, qas::decode_fused_topk_max_pages());
  qas_batch rows = *batch;             // one row per (request, draft position)
  rows.batch = batch->batch * gamma;
  const size_t need = qas_workspace_bytes(QAS_OP_DECODE_LAYER, cache, &rows, num_q_heads, k);
  if (!workspace || workspace_bytes < need)
    return fail(QAS_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(QAS_ERR_WORKSPACE, "workspace %p is not 16-byte aligned", workspace);
  if (!qas::score_supported(cache->kv_dtype, cache->head_dim, g, cache->num_kv_heads))
    return fail(QAS_ERR_UNSUPPORTED, "score: %d KV heads of d=%d", cache->num_kv_heads,
                cache->head_dim);
  hipStream_t s = (hipStream_t)stream;
  const DecodePlan p = plan_decode(cache, &rows, num_q_heads, k);
  char* ws = (char*)workspace;
  float* scores = (float*)ws;
  ws += layer_scores_bytes(cache, &rows);
  int32_t* phys_rows = (int32_t*)ws;
  ws += layer_phys_bytes(&rows);
  float* partials = (float*)ws;
  ws += p.partial_bytes;
  unsigned int* tickets = (unsigned int*)ws;

  // 1. page bounds of every position's query over the pages it may see
  hipError_t e;
  qas::ScoreArgs sa = score_args(cache, &rows, q, num_q_heads, g, scores);
  sa.tickets = tickets;
  sa.row_stride = layer_score_stride(&rows);
  sa.phys_out = phys_rows;
  sa.gamma = gamma;
  if ((e = qas::launch_score(sa, s)) != hipSuccess) return hip_fail(e, "score launch");
  // 2. + 3. top-k per (position, KV head) and attention inside one kernel
  qas::DecodeArgs da = decode_args(cache, &rows, q, num_q_heads, g, nullptr, k, k, sm_scale, out,
                                   lse, partials, p.n_split, 0);
  da.tickets = tickets;
  da.k = k;
  da.sink_tokens = 0;
  da.local_tokens = 0;
  da.scores = scores;
  da.score_stride = layer_score_stride(&rows);
  da.phys_rows = phys_rows;
  da.sel_out = sel_out;
  da.gamma = gamma;
  if ((e = qas::launch_decode(da, s)) != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

int32_t qas_chunk_groups(int32_t num_queries, int32_t batch, int32_t group) {
  if (num_queries < 0 || batch < 1 || group < 1) return 0;
  return (num_queries + group - 1) / group + batch;
}

static qas_status check_chunk(const qas_batch* batch, const int32_t* q_indptr, int32_t num_queries,
                              const int32_t* sets, int32_t num_kv_heads, int32_t kq,
                              int32_t group, int32_t page_size) {
  qas_status st = check_batch(batch);
  if (st) return st;
  if (!q_indptr || !sets) return fail(QAS_ERR_NULL, "q_indptr / sets is NULL");
  if (num_queries < 1) return fail(QAS_ERR_SHAPE, "num_queries %d < 1", num_queries);
  if (num_kv_heads < 1 || kq < 1 || group < 1 || group > 8 || group * kq > 1024)
    return fail(QAS_ERR_SHAPE, "num_kv_heads %d / kq %d / group %d out of range", num_kv_heads,
                kq, group);
  if (page_size != 32 && page_size != 64)
    return fail(QAS_ERR_UNSUPPORTED, "chunk attention: page_size %d not in {32, 64}", page_size);
  if (batch->max_pages > qas::union_max_pages())
    return fail(QAS_ERR_UNSUPPORTED, "rows of %d pages exceed %d", batch->max_pages,
                qas::union_max_pages());
  return QAS_OK;
}

static qas::UnionArgs union_args(const qas_batch* batch, const int32_t* q_indptr,
                                 int32_t num_queries, const int32_t* sets, int32_t H_kv, int32_t kq,
                                 int32_t group, int32_t S) {
  qas::UnionArgs a;
  std::memset(&a, 0, sizeof(a));
  a.seq_lens = batch->seq_lens;
  a.page_indptr = batch->page_indptr;
  a.page_indices = batch->page_indices;
  a.q_indptr = q_indptr;
  a.sets = sets;
  a.B = batch->batch;
  a.H_kv = H_kv;
  a.kq = kq;
  a.group = group;
  a.S = S;
  a.max_groups = qas_chunk_groups(num_queries, batch->batch, group);
  a.N = num_queries;
  a.ids = nullptr;
  return a;
}

qas_status qas_regroup_queries(const qas_batch* batch, const int32_t* q_indptr,
                               int32_t num_queries, const int32_t* sets, int32_t num_kv_heads,
                               int32_t kq, int32_t page_size, int32_t window, int32_t group,
                               int32_t* ids, void* stream) {
  qas_status st = check_batch(batch);
  if (st) return st;
  if (!q_indptr || !sets || !ids) return fail(QAS_ERR_NULL, "q_indptr / sets / ids is NULL");
  if (num_queries < 1) return fail(QAS_ERR_SHAPE, "num_queries %d < 1", num_queries);
  if (num_kv_heads < 1 || kq < 1 || page_size < 1)
    return fail(QAS_ERR_SHAPE, "num_kv_heads %d / kq %d / page_size %d", num_kv_heads, kq,
                page_size);
  if (group < 1 || group > 8 || window < 1 || window > qas::regroup_max_window() ||
      window % group != 0)
    return fail(QAS_ERR_SHAPE, "window %d must be a multiple of group %d (1..8), at most %d",
                window, group, qas::regroup_max_window());
  qas::RegroupArgs a;
  a.seq_lens = batch->seq_lens;
  a.page_indptr = batch->page_indptr;
  a.q_indptr = q_indptr;
  a.sets = sets;
  a.ids = ids;
  a.B = batch->batch;
  a.N = num_queries;
  a.H_kv = num_kv_heads;
  a.kq = kq;
  a.S = page_size;
  a.window = window;
  a.group = group;
  a.max_windows = (num_queries + window - 1) / window + batch->batch;
  hipError_t e = qas::launch_regroup(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "regroup launch");
  return ok();
}

qas_status qas_union_pages(const qas_batch* batch, const int32_t* q_indptr, int32_t num_queries,
                           const int32_t* sets, int32_t num_kv_heads, int32_t kq, int32_t group,
                           int32_t page_size, const int32_t* ids, int32_t* union_pages,
                           int32_t* union_count, uint8_t* membership, void* stream) {
  qas_status st = check_chunk(batch, q_indptr, num_queries, sets, num_kv_heads, kq, group,
                              page_size);
  if (st) return st;
  if (!union_pages || !union_count || !membership)
    return fail(QAS_ERR_NULL, "union outputs are NULL");
  qas::UnionArgs a = union_args(batch, q_indptr, num_queries, sets, num_kv_heads, kq, group,
                                page_size);
  a.union_out = union_pages;
  a.count_out = union_count;
  a.member_out = membership;
  a.ids = ids;
  hipError_t e = qas::launch_union_prep(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "union prep launch");
  return ok();
}

qas_status qas_chunk_attention(const qas_cache* cache, const qas_batch* batch,
                               const int32_t* q_indptr, int32_t num_queries, const int32_t* q_pos,
                               const void* q, int32_t q_dtype, int32_t num_q_heads,
                               const int32_t* sets, int32_t kq, int32_t group,
                               const int32_t* ids, float sm_scale, void* out, float* lse,
                               void* stream) {
  if (!cache) return fail(QAS_ERR_NULL, "cache is NULL");
  qas_status st = check_chunk(batch, q_indptr, num_queries, sets, cache->num_kv_heads, kq, group,
                              cache->page_size);
  if (st) return st;
  if (!cache->k_pool || !cache->v_pool || !cache->k_scale || !cache->v_scale)
    return fail(QAS_ERR_NULL, "k_pool / v_pool / k_scale / v_scale is NULL");
  if (!q || !out || !q_pos) return fail(QAS_ERR_NULL, "q / out / q_pos is NULL");
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads != 0)
    return fail(QAS_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                cache->num_kv_heads);
  const int g = num_q_heads / cache->num_kv_heads;
  if (!qas::union_supported(cache->kv_dtype, q_dtype, cache->head_dim, cache->page_size, g, group,
                            kq))
    return fail(QAS_ERR_UNSUPPORTED,
                "chunk attention needs fp8 K/V, bf16 q, d=128, S in {32,64}, group*g <= 32 "
                "(kv %d, q %d, d %d, S %d, g %d, group %d)",
                cache->kv_dtype, q_dtype, cache->head_dim, cache->page_size, g, group);
  qas::UnionArgs a = union_args(batch, q_indptr, num_queries, sets, cache->num_kv_heads, kq, group,
                                cache->page_size);
  a.k_pool = cache->k_pool;
  a.v_pool = cache->v_pool;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.q_pos = q_pos;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.H_q = num_q_heads;
  a.g = g;
  a.sm_scale = sm_scale;
  a.ids = ids;
  hipError_t e = qas::launch_union_attn(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "union attention launch");
  return ok();
}

}  // extern "C"

// ------------------------------------------------- decode layer, no alloc ----
// Scratch of qas_decode_layer_noalloc: a static device array, one copy per
// GPU the library runs on, held until the process ends.  In host code its
// name stands for a host-side shadow, not a device address: kernels receive
// the device address looked up per device below.  Zero-initialised at load;
// the decode-layer call leaves the counters it uses at zero.
static __device__ __align__(256) unsigned char scratch[QAS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];   // device address of `scratch`, per device

// The device address of `scratch` on the current device, looked up once per
// device with that device current.
qas_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QAS_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(QAS_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return QAS_OK;
}

}  // namespace

extern "C" qas_status qas_decode_layer_noalloc(const qas_cache* cache, const qas_batch* batch,
                                               const void* q, int32_t q_dtype,
                                               int32_t num_q_heads, int32_t k, float sm_scale,
                                               const void* k_new, const void* v_new,
                                               int32_t* sel_out, void* out, float* lse,
                                               void* stream) {
  const size_t need = qas_workspace_bytes(QAS_OP_DECODE_LAYER, cache, batch, num_q_heads, k);
  if (need > QAS_NOALLOC_SCRATCH_BYTES)
    return fail(QAS_ERR_WORKSPACE, "decode layer needs %zu bytes of scratch, above the %zu-byte "
                "maximum of qas_decode_layer_noalloc", need, (size_t)QAS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const qas_status st = scratch_address(&ws);
  if (st) return st;
  // argument checks (and the launch) are the workspace entry point's
  return qas_decode_layer(cache, batch, q, q_dtype, num_q_heads, k, sm_scale, k_new, v_new,
                          sel_out, out, lse, ws, QAS_NOALLOC_SCRATCH_BYTES, stream);
}
