// Internal launch interface between the host ABI (qas_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qas {

struct ScoreArgs {
  const void* summary;       // [pool][H_kv][2][d]
  const void* q;             // [B][H_q][d]
  const int32_t* seq_lens;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  float* scores;
  int B, H_kv, H_q, d, S, max_pages;
  int kv_dtype, g;
  int recs_per_block;        // (page, KV head) records per workgroup
};
hipError_t launch_score(const ScoreArgs& a, hipStream_t s);
bool score_supported(int kv_dtype, int d, int g);
int score_recs_per_block(int kv_dtype, int d, long total_recs);

struct TopkArgs {
  const float* scores;
  const int32_t* seq_lens;
  const int32_t* page_indptr;
  int32_t* sel;
  int32_t* sel_count;
  int B, H_kv, S, k;
  int max_pages;             // longest row (sizes the LDS key array)
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
constexpr int kTopkMaxPages = 15360;  // 60 KiB of LDS keys

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
  int B, H_kv, d, S, kv_dtype;
  int max_new;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
bool append_supported(int kv_dtype, int d);

struct DecodeArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;
  const int32_t* seq_lens;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* sel;
  void* out;
  float* lse;
  float* partials;           // [B][H_q][n_split][2 + d]
  int B, H_kv, H_q, d, S, kv_dtype, g;
  int sel_stride, sel_len, n_split;
  int dedupe;                // 0: lists known unique and valid-or-negative
  float sm_scale;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
bool decode_supported(int kv_dtype, int d, int g);
int decode_num_splits(int rows, int sel_len);

}  // namespace qas
