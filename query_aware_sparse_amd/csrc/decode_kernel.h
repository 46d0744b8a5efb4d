// Kernel templates of the sparse paged decode attention over each query's
// support ("PageWeaver"
// notes, eq. (1)-(2): pages in the selected list, t < L, invalid IDs
// ignored, duplicates once, empty support -> 0), reading the selected pages
// in place through the page table ("3.1.1 · Quest", §2.1), with split-page
// partial softmax states merged by log-sum-exp (the QuantSpec post's
// flash-decoding chunk merge; §2.1 of the Quest page on one global max and
// sum per row).
//
// Grid (split, KV head, request).  A workgroup first finds the distinct
// valid physical pages of its slice of the selected list and stages them in
// LDS.  The list either comes from the caller (any content: duplicates and
// invalid IDs are dropped) or is selected in the workgroup itself from the
// page scores (the top-K stage of the decode layer, topk_block.h: every
// split of a row repeats the same selection over the row's scores and keeps
// its own slice, which saves a kernel boundary and a round trip of the list
// through memory).  Its four waves then stream "token groups" (TPI token
// rows of one page = one 16-byte load per lane for K and one for V), all of
// a wave's groups in flight at once where registers allow.  Each lane keeps
// a private online-softmax state (max, sum, accumulator of its 16-byte dim
// chunk) per query head of the group over the token rows it sees; lanes of
// one token row share the logit after a DPP reduction.  States are merged
// across lanes, then waves.  With several splits per row, each split stores
// its state with device-coherent stores and takes a ticket from the row's
// counter; the split that arrives last merges all states by log-sum-exp and
// writes the output.  Coherent (sc1) stores and loads keep this free of the
// L2 writeback and invalidate that a device-scope fence costs on this
// multi-XCD part.
//
// Included by one translation unit per K/V dtype (decode_f32.hip, ...).
#pragma once

#include "qas_device.h"
#include "qas_internal.h"
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
constexpr float kLog2e = 1.4426950408889634f;

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

// Merge online-softmax state (m2, l2, acc2) into (m, l, acc); -inf max means
// an empty state.
template <int N>
__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float m2,
                                            float l2, const float* acc2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  const float a1 = fast_exp2(m - mm), a2 = fast_exp2(m2 - mm);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = acc[e] * a1 + acc2[e] * a2;
  m = mm;
}

// Device-coherent float store / load (agent scope, relaxed): visible across
// XCDs without cache maintenance.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// TPT = 0: the caller's lists; TPT > 0: select the top-K pages in the
// workgroup from the page scores, TPT scores per thread at most.
template <int DT, int D, int G, int TPT>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeArgs a) {
  constexpr int EPL = epl<DT>();
  constexpr int RL = D / EPL;                 // lanes per token row
  constexpr int TPI = kWave / RL;             // token rows per wave load
  constexpr int BYTES = DType<DT>::bytes;
  extern __shared__ int s_row[];              // staged row prefix (dedupe only)
  __shared__ int s_phys[kDecMaxList];
  __shared__ int s_ntok[kDecMaxList];
  __shared__ unsigned char s_keep[kDecMaxList];
  __shared__ int s_cnt[kDecWaves];
  __shared__ float red_m[kDecWaves][G];
  __shared__ float red_l[kDecWaves][G];
  __shared__ float red_acc[kDecWaves][G][D];
  __shared__ int s_last;

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
  // this lane's 16-byte slice of each query head of the group, loaded now so
  // that it lands during the selection instead of before the K/V stream
  uint4 qraw[G];
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
    qraw[gg] = load16(reinterpret_cast<const char*>(a.q) +
                      (((size_t)r * a.H_q + h * G + gg) * D + (lane % RL) * EPL) * BYTES);
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

  // ---- 2. stream K/V of the pages, online softmax per lane -----------------
  const int c = lane % RL;
  const int trow = lane / RL;
  const int NI = S > TPI ? S / TPI : 1;       // token groups per page (a power of two)
  const int lni = __ffs(NI) - 1;
  const int units = npg * NI;
  // byte offsets: page stride and head offset are uniform, so a load's
  // address is one 64-bit multiply-add of its physical page
  const size_t pstride = (size_t)H * S * D * BYTES;
  const uint32_t hoff = (uint32_t)(h * S * D * BYTES) + c * 16;
  const float qscale = a.sm_scale * kLog2e;   // logits in log2 units
  float qf[G][EPL];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    unpack16<DT>(qraw[gg], qf[gg]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[gg][e] *= qscale;
  }
  float m_run[G], l_run[G], acc[G][EPL];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    m_run[gg] = -INFINITY;
    l_run[gg] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[gg][e] = 0.f;
  }
  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);

  constexpr int UNR = dec_unroll<DT, G>();
  for (int u0 = wave; u0 < units; u0 += kDecWaves * UNR) {
    uint4 kr[UNR], vr[UNR];
    bool ok[UNR];
    // Every load is unconditional: a unit past the end is clamped to the last
    // unit and a token row past the page's tokens to the page's last row, so
    // each address stays inside an allocated page, and `ok` drops the value.
    // (A load under a branch makes the compiler wait for every earlier load
    // before it.)  All K loads go first, so the logits start while V is still
    // in flight.
    size_t offs[UNR];
#pragma unroll
    for (int b = 0; b < UNR; ++b) {
      const int u = min(u0 + b * kDecWaves, units - 1);
      const int pi = u >> lni, gi = u & (NI - 1);
      const int tip = gi * TPI + trow;
      ok[b] = (u0 + b * kDecWaves < units) & (tip < s_ntok[pi]);
      offs[b] = (size_t)(uint32_t)s_phys[pi] * pstride +
                (hoff + (uint32_t)(min(tip, S - 1) * D * BYTES));
    }
#pragma unroll
    for (int b = 0; b < UNR; ++b) kr[b] = load16(kbase + offs[b]);
#pragma unroll
    for (int b = 0; b < UNR; ++b) vr[b] = load16(vbase + offs[b]);
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      float z[UNR];
      float zmax = m_run[gg];
#pragma unroll
      for (int b = 0; b < UNR; ++b) {
        float kf[EPL];
        unpack16<DT>(kr[b], kf);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot += qf[gg][e] * kf[e];
        dot = group_sum<RL>(dot);
        z[b] = ok[b] ? dot : -INFINITY;
        zmax = fmaxf(zmax, z[b]);
      }
      // No branch on the batch's content: a branch here lets the compiler
      // sink the V loads below the logits, a second round trip per batch.
      // With no valid logit yet the stand-in maximum 0 gives alpha = 0 and
      // p = 0 on a zero state; rows not loaded read as zero words.
      const float zm = zmax == -INFINITY ? 0.f : zmax;
      const float alpha = fast_exp2(m_run[gg] - zm);
      float l = l_run[gg] * alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[gg][e] *= alpha;
#pragma unroll
      for (int b = 0; b < UNR; ++b) {
        const float p = ok[b] ? fast_exp2(z[b] - zm) : 0.f;
        const uint4 w = ok[b] ? vr[b] : make_uint4(0, 0, 0, 0);
        float vf[EPL];
        unpack16<DT>(w, vf);
        l += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[gg][e] += p * vf[e];
      }
      l_run[gg] = l;
      m_run[gg] = zmax;
    }
  }

  // ---- 3. merge lanes of one dim chunk, then the waves ---------------------
#pragma unroll
  for (int off = RL; off < kWave; off <<= 1) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const float m2 = shfl_xor_f(m_run[gg], off);
      const float l2 = shfl_xor_f(l_run[gg], off);
      float acc2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc2[e] = shfl_xor_f(acc[gg][e], off);
      merge_state<EPL>(m_run[gg], l_run[gg], acc[gg], m2, l2, acc2);
    }
  }
  if (lane < RL) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      if (lane == 0) {
        red_m[wave][gg] = m_run[gg];
        red_l[wave][gg] = l_run[gg];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_acc[wave][gg][c * EPL + e] = acc[gg][e];
    }
  }
  __syncthreads();
  const bool single = a.n_split == 1;
  for (int t = tid; t < G * D; t += kDecThreads) {
    const int gg = t / D, dim = t - (t / D) * D;
    float m = -INFINITY, l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float one[1] = {red_acc[w][gg][dim]};
      merge_state<1>(m, l, &o, red_m[w][gg], red_l[w][gg], one);
    }
    const size_t rowq = (size_t)r * a.H_q + h * G + gg;
    if (single) {
      store_rn<DT>(a.out, rowq * D + dim, m == -INFINITY ? 0.f : o / l);
      if (dim == 0 && a.lse)
        a.lse[rowq] = m == -INFINITY ? -INFINITY : (m + log2f(l)) * 0.6931471805599453f;
      continue;
    }
    float* part = a.partials + (rowq * a.n_split + split) * (D + 2);
    if (dim == 0) {
      store_coherent(part, m);
      store_coherent(part + 1, l);
    }
    store_coherent(part + 2 + dim, o);
  }
  if (single) return;

  // ---- 4. the last split of the row merges all split states ---------------
  __builtin_amdgcn_s_waitcnt(0);             // this thread's states are stored
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.tickets + (size_t)r * H + h, 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(a.n_split - 1);
  }
  __syncthreads();
  if (!s_last) return;
  constexpr int MB = 16;
  for (int t = tid; t < G * D; t += kDecThreads) {
    const int gg = t / D, dim = t - (t / D) * D;
    const size_t rowq = (size_t)r * a.H_q + h * G + gg;
    const float* part = a.partials + rowq * a.n_split * (D + 2);
    float M = -INFINITY, lsum = 0.f, o = 0.f;
    for (int sb = 0; sb < a.n_split; sb += MB) {
      float ms[MB], ls[MB], os[MB];
#pragma unroll
      for (int k = 0; k < MB; ++k) {
        const int sp = sb + k;
        const bool in = sp < a.n_split;
        ms[k] = in ? load_coherent(part + sp * (D + 2)) : -INFINITY;
        ls[k] = in ? load_coherent(part + sp * (D + 2) + 1) : 0.f;
        os[k] = in ? load_coherent(part + sp * (D + 2) + 2 + dim) : 0.f;
      }
#pragma unroll
      for (int k = 0; k < MB; ++k) merge_state<1>(M, lsum, &o, ms[k], ls[k], &os[k]);
    }
    store_rn<DT>(a.out, rowq * D + dim, M == -INFINITY ? 0.f : o / lsum);
    if (dim == 0 && a.lse)
      a.lse[rowq] = M == -INFINITY ? -INFINITY : (M + log2f(lsum)) * 0.6931471805599453f;
  }
  // leave the counter at zero for the next call
  if (tid == 0)
    __hip_atomic_store(a.tickets + (size_t)r * H + h, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT, int D, int G>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.H_kv, a.B);
  if (a.scores) {
    if (a.max_pages <= kDecThreads * 4)
      hipLaunchKernelGGL((decode_kernel<DT, D, G, 4>), grid, dim3(kDecThreads), 0, s, a);
    else if (a.max_pages <= kDecThreads * kDecFusedTopkPT)
      hipLaunchKernelGGL((decode_kernel<DT, D, G, kDecFusedTopkPT>), grid, dim3(kDecThreads), 0, s, a);
    else
      return hipErrorInvalidValue;
  } else {
    const size_t lds = a.dedupe ? (size_t)a.sel_len * sizeof(int) : 0;
    hipLaunchKernelGGL((decode_kernel<DT, D, G, 0>), grid, dim3(kDecThreads), lds, s, a);
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
