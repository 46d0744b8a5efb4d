// Sparse paged decode attention over each query's support ("PageWeaver"
// notes, eq. (1)-(2): pages in the selected list, t < L, invalid IDs
// ignored, duplicates once, empty support -> 0), reading the selected pages
// in place through the page table ("3.1.1 · Quest", §2.1), with split-page
// partial softmax states merged by log-sum-exp (the QuantSpec post's
// flash-decoding chunk merge; §2.1 of the Quest page on one global max and
// sum per row).
//
// Grid (split, KV head, request).  A workgroup first turns its slice of the
// selected list into distinct valid physical pages in LDS (lists from the
// top-K stage are already canonical and carry their physical pages, so only
// padding is dropped), then its four waves stream "token groups" (TPI token
// rows of one page = one 16-byte load per lane for K and one for V), all of
// a wave's groups in flight at once where registers allow.  Each lane keeps
// a private online-softmax state (max, sum, accumulator of its 16-byte dim
// chunk) per query head of the group over the token rows it sees; lanes of
// one token row share the logit after a DPP reduction.  States are merged
// across lanes, then waves; the split's state goes to the workspace, and a
// small second kernel merges the splits of every (request, query head) by
// log-sum-exp.  (Merging in the last-arriving split instead needs an
// agent-scope fence per workgroup, which on this multi-XCD part writes back
// and invalidates the XCD's L2 each time; the kernel boundary does that once.)
#include "qas_device.h"
#include "qas_internal.h"

namespace qas {

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
// token groups in flight per wave (bounded by registers)
template <int G> constexpr int dec_unroll() { return G <= 2 ? 16 : 8; }
constexpr int kDecMaxList = 1024;      // selected entries per split
constexpr int kDecMaxRow = 4096;       // entries of a row when deduplicating
constexpr float kLog2e = 1.4426950408889634f;

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

template <int DT, int D, int G>
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

  const int split = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int H = a.H_kv, S = a.S;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int L = a.seq_lens[r];
  const int pbeg = a.page_indptr[r];
  const int P_r = a.page_indptr[r + 1] - pbeg;
  const int n_pages = L > 0 ? min((L + S - 1) / S, P_r) : 0;
  const int per = (a.sel_len + a.n_split - 1) / a.n_split;
  const int e0 = min(a.sel_len, split * per);
  const int e1 = min(a.sel_len, e0 + per);
  const int32_t* row = a.sel + ((size_t)r * H + h) * a.sel_stride;

  // ---- 1. distinct valid pages of entries [e0, e1), in entry order --------
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
  int npg = 0;
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
  __syncthreads();

  // ---- 2. stream K/V of the pages, online softmax per lane -----------------
  const int c = lane % RL;
  const int trow = lane / RL;
  const int NI = S > TPI ? S / TPI : 1;       // token groups per page
  const int units = npg * NI;
  const float qscale = a.sm_scale * kLog2e;   // logits in log2 units
  float qf[G][EPL];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const size_t qo = ((size_t)r * a.H_q + h * G + gg) * D + c * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[gg][e] = load_scalar<DT>(a.q, qo + e) * qscale;
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

  constexpr int UNR = dec_unroll<G>();
  for (int u0 = wave; u0 < units; u0 += kDecWaves * UNR) {
    uint4 kr[UNR], vr[UNR];
    bool ok[UNR];
#pragma unroll
    for (int b = 0; b < UNR; ++b) {
      const int u = u0 + b * kDecWaves;
      kr[b] = make_uint4(0, 0, 0, 0);
      vr[b] = make_uint4(0, 0, 0, 0);
      ok[b] = false;
      if (u < units) {
        const int pi = u / NI, gi = u - (u / NI) * NI;
        const int tip = gi * TPI + trow;
        ok[b] = tip < s_ntok[pi];
        if (ok[b]) {
          const size_t off = ((((size_t)s_phys[pi] * H + h) * S + tip) * D) * BYTES + c * 16;
          kr[b] = load16(kbase + off);
          vr[b] = load16(vbase + off);
        }
      }
    }
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
      if (zmax == -INFINITY) continue;
      const float alpha = fast_exp2(m_run[gg] - zmax);
      float l = l_run[gg] * alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[gg][e] *= alpha;
#pragma unroll
      for (int b = 0; b < UNR; ++b) {
        if (!ok[b]) continue;
        const float p = fast_exp2(z[b] - zmax);
        float vf[EPL];
        unpack16<DT>(vr[b], vf);
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
  for (int t = tid; t < G * D; t += kDecThreads) {
    const int gg = t / D, dim = t - (t / D) * D;
    float m = -INFINITY, l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float one[1] = {red_acc[w][gg][dim]};
      merge_state<1>(m, l, &o, red_m[w][gg], red_l[w][gg], one);
    }
    float* part = a.partials +
                  (((size_t)r * a.H_q + h * G + gg) * a.n_split + split) * (D + 2);
    if (dim == 0) {
      part[0] = m;
      part[1] = l;
    }
    part[2 + dim] = o;
  }

}

// Log-sum-exp merge of the split states of one (request, query head): one
// workgroup per row, one thread per output dim; the split states are loaded
// MB at a time (independent loads in flight) and merged online.
template <int DT, int D>
__global__ __launch_bounds__(D) void merge_kernel(DecodeArgs a) {
  constexpr int MB = 16;
  const int rowq = blockIdx.x;                 // r * H_q + i
  const int dim = threadIdx.x;
  const float* part = a.partials + (size_t)rowq * a.n_split * (D + 2);
  float M = -INFINITY, lsum = 0.f, o = 0.f;
  for (int sb = 0; sb < a.n_split; sb += MB) {
    float ms[MB], ls[MB], os[MB];
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const int sp = sb + k;
      const bool in = sp < a.n_split;
      ms[k] = in ? part[sp * (D + 2)] : -INFINITY;
      ls[k] = in ? part[sp * (D + 2) + 1] : 0.f;
      os[k] = in ? part[sp * (D + 2) + 2 + dim] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < MB; ++k) merge_state<1>(M, lsum, &o, ms[k], ls[k], &os[k]);
  }
  o = M == -INFINITY ? 0.f : o / lsum;
  store_rn<DT>(a.out, (size_t)rowq * D + dim, o);
  if (dim == 0 && a.lse)
    a.lse[rowq] = M == -INFINITY ? -INFINITY : (M + log2f(lsum)) * 0.6931471805599453f;
}

template <int DT, int D, int G>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.H_kv, a.B);
  const size_t lds = a.dedupe ? (size_t)a.sel_len * sizeof(int) : 0;
  hipLaunchKernelGGL((decode_kernel<DT, D, G>), grid, dim3(kDecThreads), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((merge_kernel<DT, D>), dim3(a.B * a.H_q), dim3(D), 0, s, a);
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

}  // namespace

bool decode_supported(int kv_dtype, int d, int g) {
  return (kv_dtype == kF32 || kv_dtype == kF16 || kv_dtype == kBF16) &&
         (d == 16 || d == 64 || d == 128) && (g == 1 || g == 2 || g == 4 || g == 8);
}

int decode_num_splits(int rows, int sel_len) {
  if (sel_len < 1) sel_len = 1;
  int n = (512 + rows - 1) / rows;
  const int cap = (sel_len + 3) / 4;
  if (n > cap) n = cap;
  const int need = (sel_len + kDecMaxList - 1) / kDecMaxList;
  if (n < need) n = need;
  if (n < 1) n = 1;
  return n;
}

int decode_max_dedupe_row() { return kDecMaxRow; }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  switch (a.kv_dtype) {
    case kF32: return by_d<kF32>(a, s);
    case kF16: return by_d<kF16>(a, s);
    case kBF16: return by_d<kBF16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qas
