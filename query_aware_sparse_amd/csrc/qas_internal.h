// Internal launch interface between the host ABI (qas_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qas {

struct ScoreArgs {
  void* summary;             // [pool][H_kv][2][d]
  const void* q;             // [B][H_q][d]
  const int32_t* seq_lens;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  float* scores;             // row_stride 0: [pbeg*H_kv + h*P_r + j], else [(r*H_kv + h)*row_stride + j]
  int row_stride;
  int32_t* phys_out;         // optional (row_stride > 0): [r*row_stride + j] physical page of page j
  int gamma;                 // rows per request: row r is draft position r % gamma of request
                             // r / gamma, of length seq_lens - (gamma - 1 - r % gamma)
  // optional decode append of the token at seq_lens[r] - 1 (k_new != NULL)
  const void* k_new;         // [B][H_kv][d]
  const void* v_new;
  void* k_pool;
  void* v_pool;
  int B, H_kv, H_q, d, S, max_pages;
  int kv_dtype, g;
  int pages_per_iter;        // pages one workgroup covers per lane step
  unsigned int* tickets;     // optional [B][H_kv] counters zeroed for the attention kernel
  // optional e4m3 summary copy: scores are taken from it (the append keeps
  // both the exact record and the copy current)
  void* summary_fp8;         // [pool][H_kv][2][d] codes
  float* summary_fp8_scale;  // [pool][H_kv]
};
hipError_t launch_score(const ScoreArgs& a, hipStream_t s);
bool score_supported(int kv_dtype, int d, int g, int H_kv);
int score_pages_per_iter(int kv_dtype, int d, int H_kv);
int score8_pages_per_iter(int d, int H_kv);
bool score8_supported(int d, int H_kv);   // scores from the e4m3 summary copy

struct TopkArgs {
  const float* scores;
  const int32_t* seq_lens;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  int32_t* sel;
  int32_t* sel_phys;         // optional physical pages of `sel`
  int32_t* sel_count;        // pages written per row (top-K and fixed pages)
  int B, H_kv, S, k;
  int max_pages;             // longest row (sizes the per-thread register run)
  int sink_tokens, local_tokens;   // fixed pages joined with the top-K (0: none)
  int sel_stride;            // row stride of sel / sel_phys (>= the row's count)
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
constexpr int kTopkMaxPages = 16384;  // 512 threads x 32 scores held in registers

struct AppendArgs {
  void* k_pool;
  void* v_pool;
  void* summary;
  const void* k_new;
  const void* v_new;
  const int32_t* seq_lens;
  const int32_t* new_indptr;   // NULL: one token per request at seq_lens[r]-1
  const int32_t* page_indptr;
  const int32_t* page_indices;
  void* summary_fp8;         // optional e4m3 copy [pool][H_kv][2][d]
  float* summary_fp8_scale;  //   and its scale [pool][H_kv]
  int B, H_kv, d, S, kv_dtype;
  int max_new;
  int rescan;                // 1: rebuild each request's tail record from the pool's
                             //    keys (seq_lens = lengths after a rollback); no K/V written
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
bool append_supported(int kv_dtype, int d);

struct Fp8AppendArgs {
  void* k_pool;              // e4m3 tiles in the union kernel's operand order
  void* v_pool;
  const float* k_scale;      // [H_kv]
  const float* v_scale;
  const void* k_new;         // [total_new][H_kv][128] in new_dtype
  const void* v_new;
  int new_dtype;
  const int32_t* seq_lens;   // lengths before the new tokens
  const int32_t* new_indptr; // [B+1]
  const int32_t* page_indptr;
  const int32_t* page_indices;
  int B, H_kv, S, max_new;
};
hipError_t launch_append_fp8(const Fp8AppendArgs& a, hipStream_t s);
bool append_fp8_supported(int new_dtype, int d, int S);

struct ToprArgs {
  const void* k_pool;
  const void* summary;
  const void* q;             // [B][H_q][d]
  const int32_t* seq_lens;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  int32_t* top_tokens;       // [B][H_q][R]
  float* top_logits;         // [B][H_q][R]
  int32_t* pages_read;       // optional [B][H_q]
  int B, H_kv, H_q, d, S, kv_dtype, R;
  // workspace, per row (request, query head)
  int* ws_state;             // [rows][4]: finished, pilot pages, pages left to scan, pilot kept
  uint64_t* ws_pages;        // [rows][page_stride] page sort keys
  uint64_t* ws_pilot;        // [rows][R] the pilot's best keys
  uint64_t* ws_chunks;       // [rows][scan_chunks][R] each chunk's best keys
  int* ws_counts;            // [rows][scan_chunks]
  int page_stride, scan_chunks, pilot_pages;
};
hipError_t launch_topr(const ToprArgs& a, hipStream_t s);
int topr_max_pages();
int topr_max_r();
int topr_threads();

struct DecodeArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;
  const int32_t* seq_lens;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* sel;
  const int32_t* sel_phys;   // physical pages of sel (canonical lists), or NULL
  void* out;
  float* lse;
  float* partials;           // [B][H_q][n_split][2 + d]
  unsigned int* tickets;     // [B][H_kv] split arrival counters, zero on entry
  // in-kernel top-K (scores != NULL): select sel_len pages per (request, KV
  // head) from scores laid out [B][H_kv][score_stride]; sel / sel_phys unused
  const float* scores;
  int score_stride;          // row stride of scores (>= max_pages, a multiple of 4)
  const int32_t* phys_rows;  // [B][score_stride] physical page of each scored page
  int gamma;                 // rows per request (draft positions), as in ScoreArgs
  int32_t* sel_out;          // optional [B][H_kv][sel_len] copy of the selection
  int max_pages;
  int k;                     // in-kernel top-K: pages Quest selects per row
  int sink_tokens, local_tokens;   // in-kernel top-K: fixed pages joined with it
  int B, H_kv, H_q, d, S, kv_dtype, g;
  int sel_stride, sel_len, n_split;
  int dedupe;                // 0: lists known unique and valid-or-negative
  int clear_tickets;         // zero the tickets in a kernel of their own first
  float sm_scale;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
bool decode_supported(int kv_dtype, int d, int g);
int decode_num_splits(int rows, int sel_len);
int decode_max_dedupe_row();
int decode_fused_topk_max_pages();   // longest row the in-kernel top-K takes

struct UnionArgs {
  const void* k_pool;        // fp8 [pool][H_kv][S][d]
  const void* v_pool;
  const float* k_scale;      // [H_kv]
  const float* v_scale;
  const int32_t* seq_lens;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* q_indptr;   // [B+1] queries of each request
  const int32_t* q_pos;      // [N] causal limit c_i
  const void* q;             // bf16 [N][H_q][d]
  const int32_t* sets;       // [N][H_kv][kq]
  void* out;                 // bf16 [N][H_q][d]
  float* lse;                // [N][H_q] or NULL
  int32_t* union_out;        // union prep only: [groups][H_kv][group * kq]
  int32_t* count_out;        //                  [groups][H_kv]
  unsigned char* member_out; //                  [groups][H_kv][group * kq]
  const int32_t* ids;        // [H_kv][N] execution order per KV head, NULL = identity
  int N;
  int B, H_kv, H_q, g, S, kq, group, max_groups;
  float sm_scale;
};
hipError_t launch_union_attn(const UnionArgs& a, hipStream_t s);
hipError_t launch_union_prep(const UnionArgs& a, hipStream_t s);
bool union_supported(int kv_dtype, int q_dtype, int d, int S, int g, int group, int kq);
int union_max_pages();

struct RegroupArgs {
  const int32_t* seq_lens;
  const int32_t* page_indptr;
  const int32_t* q_indptr;   // [B+1]
  const int32_t* sets;       // [N][H_kv][kq]
  int32_t* ids;              // [H_kv][N] out: original query of each slot
  int B, N, H_kv, kq, S, window, group, max_windows;
};
hipError_t launch_regroup(const RegroupArgs& a, hipStream_t s);
int regroup_max_pages();      // bitmap capacity; longer requests keep their order
int regroup_max_window();

}  // namespace qas
