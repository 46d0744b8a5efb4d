// Kernel templates of the sparse paged decode attention over each query's
// support ("PageWeaver" notes, eq. (1)-(2): pages in the selected list,
// t < L, invalid IDs ignored, duplicates once, empty support -> 0), reading
// the selected pages in place through the page table ("3.1.1 · Quest",
// §2.1), with split-page partial softmax states merged by log-sum-exp (the
// QuantSpec post's flash-decoding chunk merge; §2.1 of the Quest page on one
// global max and sum per row).
//
// Grid (split, KV head, request).  A workgroup first finds the distinct
// valid physical pages of its slice of the selected list and stages them in
// LDS.  The list either comes from the caller (any content: duplicates and
// invalid IDs are dropped) or is selected in the workgroup itself from the
// page scores (the top-K stage of the decode layer, topk_block.h: every
// split of a row repeats the same selection over the row's scores and keeps
// its own slice, which saves a kernel boundary and a round trip of the list
// through memory).  The workgroup then streams the pages' K/V and merges the
// split states (attend_block.h).
//
// Included by one translation unit per K/V dtype (decode_f32.hip, ...).
#pragma once

#include "qas_device.h"
#include "qas_internal.h"
#include "attend_block.h"
#include "topk_block.h"

namespace qas {

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / kWave;
// token groups in flight per wave (bounded by registers)
// K/V rows each wave loads per batch: as many as the registers hold at two
// waves per SIMD (f16 products read packed halves; bf16/f32 unpack to fp32)
template <int DT, int G> constexpr int dec_unroll() {
  return DT == kBF16 && G == 8 ? 1 : (DT == kF16 ? 16 : 8) / (G <= 2 ? 1 : G <= 4 ? 2 : 4);
}
constexpr int kDecMaxList = 1024;      // selected entries per split
constexpr int kDecMaxRow = 4096;       // entries of a row when deduplicating
constexpr int kDecFusedTopkPT = 8;    // in-kernel top-K: scores per thread at most

namespace decode_detail {


__device__ __forceinline__ int block_excl_count(bool flag, int* scratch, int* total) {
  const uint64_t mask = __ballot(flag);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
  if (lane == 0) scratch[wave] = __popcll(mask);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    const int c = scratch[w];
    before += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + in_wave;
}

// TPT = 0: the caller's lists; TPT > 0: select the top-K pages in the
// workgroup from the page scores, TPT scores per thread at most.  MF: the
// logits on matrix cores (attend_split_mfma; 16-bit K/V, d = 128, 4 or 8
// query heads per KV head, S >= 16).
template <int DT, int D, int G, int TPT, bool MF>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeArgs a) {
  constexpr int EPL = epl<DT>();
  constexpr int RL = D / EPL;                 // lanes per token row
  constexpr int BYTES = DType<DT>::bytes;
  extern __shared__ int s_row[];              // staged row prefix (dedupe only)
  __shared__ int s_phys[kDecMaxList];
  __shared__ int s_ntok[kDecMaxList];
  __shared__ unsigned char s_keep[kDecMaxList];
  __shared__ int s_cnt[kDecWaves];

  const int split = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int H = a.H_kv, S = a.S;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  // in-kernel top-K: the row's scores and physical pages sit at a fixed
  // stride (a multiple of 4 entries in a 16-byte aligned workspace), so their
  // 16-byte loads go out first, before the request's bounds are known
  TopkRow<(TPT > 0 ? TPT : 4), kDecThreads> t;
  const int cap = min(a.max_pages, kDecThreads * TPT);  // the host keeps rows within this
  if constexpr (TPT > 0)
    t.issue_x4(a.scores + ((size_t)r * H + h) * a.score_stride,
               a.phys_rows + (size_t)r * a.score_stride, cap);
  // this lane's 16-byte slice of each query head of the group (or its query
  // operand for the matrix cores), loaded now so that it lands during the
  // selection instead of before the K/V stream
  uint4 qraw[MF ? 4 : G];
  if constexpr (MF) {
    load_q_operand<G>(reinterpret_cast<const char*>(a.q) + ((size_t)r * a.H_q + h * G) * D * BYTES,
                      qraw);
  } else {
#pragma unroll
    for (int gg = 0; gg < G; ++gg)
      qraw[gg] = load16(reinterpret_cast<const char*>(a.q) +
                        (((size_t)r * a.H_q + h * G + gg) * D + (lane % RL) * EPL) * BYTES);
  }
  // row r: a request, or draft position r % gamma of request r / gamma whose
  // causal limit is its own position (length seq_lens - (gamma - 1 - i))
  const int req = r / a.gamma;
  const int L = a.seq_lens[req] - (a.gamma - 1 - r % a.gamma);
  const int pbeg = a.page_indptr[req];
  const int P_r = a.page_indptr[req + 1] - pbeg;
  const int n_pages = L > 0 ? min((L + S - 1) / S, P_r) : 0;
  const int per = (a.sel_len + a.n_split - 1) / a.n_split;
  const int e0 = min(a.sel_len, split * per);
  const int e1 = min(a.sel_len, e0 + per);

  int npg = 0;
  if constexpr (TPT > 0) {
    // ---- 1. top-K of the row's scores; keep selected positions [e0, e1) ---
    __shared__ TopkShared tsh;
    const int n_tk = min(n_pages, cap);
    const int take = min(a.k, n_tk);
    t.finish_x4(cap, n_tk);
    t.set_fixed(L, S, a.sink_tokens, a.local_tokens);
    t.select(take, tsh);
    int count;
    int pos = t.first_position(tsh, &count);
    int32_t* so = a.sel_out ? a.sel_out + ((size_t)r * H + h) * a.sel_len : nullptr;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      if (t.selected(k)) {
        if (pos >= e0 && pos < e1) {
          const int j = t.j0 + k;
          s_phys[pos - e0] = t.pv[k];
          s_ntok[pos - e0] = min(S, L - j * S);
          if (so) so[pos] = j;
        }
        ++pos;
      }
    }
    if (so)
      for (int e = max(e0, count) + tid; e < e1; e += kDecThreads) so[e] = -1;
    npg = max(0, min(e1, count) - e0);
  } else {
    // ---- 1. distinct valid pages of entries [e0, e1), in entry order --------
    const int32_t* row = a.sel + ((size_t)r * H + h) * a.sel_stride;
    if (a.dedupe) {
      for (int j = tid; j < e1; j += kDecThreads) s_row[j] = row[j];
      __syncthreads();
      // wave w decides entries e0 + w, e0 + w + 4, ...: an entry is kept if its
      // ID is a page of the request and no earlier entry of the row holds it
      for (int e = e0 + wave; e < e1; e += kDecWaves) {
        const int id = s_row[e];
        bool seen = false;
        for (int j = lane; j < e; j += kWave) seen |= s_row[j] == id;
        const bool dup = __ballot(seen) != 0;
        if (lane == 0) s_keep[e - e0] = (id >= 0 && id < n_pages && !dup) ? 1 : 0;
      }
      __syncthreads();
    }
    const int32_t* prow = a.sel_phys ? a.sel_phys + ((size_t)r * H + h) * a.sel_stride : nullptr;
    for (int eb = e0; eb < e1; eb += kDecThreads) {
      const int e = eb + tid;
      int id = -1, phys = 0;
      bool keep = false;
      if (e < e1) {
        id = a.dedupe ? s_row[e] : row[e];
        if (prow) phys = prow[e];
        keep = a.dedupe ? s_keep[e - e0] != 0 : (id >= 0 && id < n_pages);
      }
      int total;
      const int pos = npg + block_excl_count(keep, s_cnt, &total);
      if (keep) {
        s_phys[pos] = prow ? phys : a.page_indices[pbeg + id];
        s_ntok[pos] = min(S, L - id * S);
      }
      npg += total;
    }
  }
  __syncthreads();

  // ---- 2. stream K/V of the pages, merge the states ----------------------
  AttendOut o;
  o.out = a.out;
  o.lse = a.lse;
  o.partials = a.partials;
  o.ticket = a.tickets + (size_t)r * H + h;
  o.rowq0 = (size_t)r * a.H_q + h * G;
  o.n_split = a.n_split;
  o.split = split;
  if constexpr (MF)
    attend_split_mfma<DT, G, kDecWaves>(
        s_phys, s_ntok, npg, S, reinterpret_cast<const char*>(a.k_pool),
        reinterpret_cast<const char*>(a.v_pool), (size_t)H * S * D * BYTES,
        (uint32_t)(h * S * D * BYTES), qraw, a.sm_scale, o);
  else
    attend_split<DT, D, G, dec_unroll<DT, G>(), kDecWaves>(
        s_phys, s_ntok, npg, S, reinterpret_cast<const char*>(a.k_pool),
        reinterpret_cast<const char*>(a.v_pool), (size_t)H * S * D * BYTES,
        (uint32_t)(h * S * D * BYTES), qraw, a.sm_scale, o);
}

// The matrix-core stream where it applies (16-bit K/V, d = 128, g = 4 or 8,
// pages of at least 16 tokens), else the VALU stream.
template <int DT, int D, int G, int TPT>
void launch_kernel(const DecodeArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  if constexpr (DT != kF32 && D == 128 && (G == 4 || G == 8)) {
    if (a.S >= 16) {
      hipLaunchKernelGGL((decode_kernel<DT, D, G, TPT, true>), grid, dim3(kDecThreads), lds, s, a);
      return;
    }
  }
  hipLaunchKernelGGL((decode_kernel<DT, D, G, TPT, false>), grid, dim3(kDecThreads), lds, s, a);
}

template <int DT, int D, int G>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.H_kv, a.B);
  if (a.scores) {
    if (a.max_pages <= kDecThreads * 4)
      launch_kernel<DT, D, G, 4>(a, grid, 0, s);
    else if (a.max_pages <= kDecThreads * kDecFusedTopkPT)
      launch_kernel<DT, D, G, kDecFusedTopkPT>(a, grid, 0, s);
    else
      return hipErrorInvalidValue;
  } else {
    const size_t lds = a.dedupe ? (size_t)a.sel_len * sizeof(int) : 0;
    launch_kernel<DT, D, G, 0>(a, grid, lds, s);
  }
  return hipGetLastError();
}

template <int DT, int D>
hipError_t by_g(const DecodeArgs& a, hipStream_t s) {
  switch (a.g) {
    case 1: return launch_t<DT, D, 1>(a, s);
    case 2: return launch_t<DT, D, 2>(a, s);
    case 4: return launch_t<DT, D, 4>(a, s);
    case 8: return launch_t<DT, D, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t by_d(const DecodeArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return by_g<DT, 16>(a, s);
    case 64: return by_g<DT, 64>(a, s);
    case 128: return by_g<DT, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace decode_detail

template <int DT>
hipError_t launch_decode_dtype(const DecodeArgs& a, hipStream_t s) {
  return decode_detail::by_d<DT>(a, s);
}

}  // namespace qas
