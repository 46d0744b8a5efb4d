// Top-K page selection per (request, KV head): the Quest page's second stage
// ("3.1.1 · Quest", §1 and Fig. 1), ordered by (score descending, page index
// ascending) so ties go to the lower page index.
//
// One workgroup per row; the row's scores (and page table, when physical
// pages are emitted) are staged in LDS with all loads in flight at once.
// Selection narrows a closed score interval [lo, hi] that holds the K-th
// largest score:
//   * histogram the candidates into NB bins by (s - lo) / (hi - lo) * NB, a
//     map that is monotone in s in fp32 (a correctly rounded quotient by a
//     fixed positive range, an exact power-of-two scale), so every score in
//     a higher bin is larger; lo falls in bin 0 and hi in the top bin;
//   * walk the bins from the top to the one holding the K-th score; scores
//     in higher bins are taken and that bin's scores are the candidates
//     (if still too many, [lo, hi] shrinks to their exact min/max and the
//     step repeats; each repeat drops at least one distinct value);
//   * rank the candidates exactly by (score desc, index asc).  The last
//     candidate taken is the threshold (T_s, T_j): page j is selected iff
//     s_j > T_s, or s_j == T_s and j <= T_j.
// An index-ordered compaction (per-thread contiguous runs plus a workgroup
// scan) writes the selected pages in ascending order, with their physical
// pages.  -0.0 and +0.0 compare equal, as scores.
//
// Workgroup barriers and LDS round trips dominate the cost at these sizes,
// so every step uses at most one barrier where possible and scans run on
// DPP inside a wave.
#include <float.h>

#include "qas_device.h"
#include "qas_internal.h"

namespace qas {

namespace {

constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkBins = 1024;
constexpr int kTkCand = 512;         // candidates ranked exactly
constexpr int kTkBatch = 8;          // loads per thread in flight
constexpr size_t kTkLdsBudget = 65536;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_shift(int v) {
  // lanes without a source (or outside ROW_MASK) read 0
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes: row_shr 1/2/4/8 scan each row of
// 16 lanes, row_bcast 15/31 carry row totals into the following rows.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_shift<0x111, 0xF>(v);   // row_shr:1
  v += dpp_shift<0x112, 0xF>(v);   // row_shr:2
  v += dpp_shift<0x114, 0xF>(v);   // row_shr:4
  v += dpp_shift<0x118, 0xF>(v);   // row_shr:8
  v += dpp_shift<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_shift<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// Exclusive prefix sum over the workgroup in thread order; one barrier.
// `scratch` (kTkWaves ints) must not be reused before another barrier.
__device__ __forceinline__ int block_excl_scan(int v, int* scratch, int* total) {
  const int incl = wave_incl_scan(v);
  if (lane_id() == kWave - 1) scratch[wave_id()] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const int c = scratch[w];
    before += w < wave_id() ? c : 0;
    all += c;
  }
  *total = all;
  return before + incl - v;
}

__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dpp_f<0xB1>(v));
  v = fminf(v, dpp_f<0x4E>(v));
  v = fminf(v, dpp_f<0x141>(v));
  v = fminf(v, dpp_f<0x140>(v));
  v = fminf(v, __shfl_xor(v, 16, kWave));
  return fminf(v, __shfl_xor(v, 32, kWave));
}

// (min, max) over the workgroup; one barrier.  `scratch`: 2 * kTkWaves floats.
__device__ __forceinline__ void block_minmax(float& lo, float& hi, float* scratch) {
  lo = wave_min(lo);
  hi = group_max<kWave>(hi);
  if (lane_id() == 0) {
    scratch[2 * wave_id()] = lo;
    scratch[2 * wave_id() + 1] = hi;
  }
  __syncthreads();
  lo = scratch[0];
  hi = scratch[1];
#pragma unroll
  for (int w = 1; w < kTkWaves; ++w) {
    lo = fminf(lo, scratch[2 * w]);
    hi = fmaxf(hi, scratch[2 * w + 1]);
  }
}

__device__ __forceinline__ int score_bin(float s, float lo, float range) {
  const float t = (s - lo) / range * (float)kTkBins;
  return t >= (float)(kTkBins - 1) ? kTkBins - 1 : (int)t;
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ float s_score[];          // [max_pages] (+ page table)
  __shared__ int hist[kTkBins];
  __shared__ int s_cidx[kTkCand];
  __shared__ float s_cval[kTkCand];
  __shared__ int s_scan[3][kTkWaves];
  __shared__ float s_mm[2][2 * kTkWaves];
  __shared__ int s_b, s_above, s_cnt, s_tj;
  __shared__ float s_ts;

  const bool with_phys = a.sel_phys != nullptr;
  int* s_pt = reinterpret_cast<int*>(s_score + a.max_pages);
  const int row = blockIdx.x;
  const int H = a.H_kv;
  const int r = row / H, h = row - (row / H) * H;
  const int tid = threadIdx.x;
  const int pbeg = a.page_indptr[r];
  const int P_r = a.page_indptr[r + 1] - pbeg;
  const int L = a.seq_lens[r];
  // never more scores than the LDS array sized by max_pages holds
  const int n = L > 0 ? min(min((L + a.S - 1) / a.S, P_r), a.max_pages) : 0;
  const int K = a.k;
  const int take = min(K, n);
  int32_t* out = a.sel + (size_t)row * K;
  int32_t* out_phys = with_phys ? a.sel_phys + (size_t)row * K : nullptr;
  const int32_t* pt = a.page_indices + pbeg;
  if (a.sel_count && tid == 0) a.sel_count[row] = take;
  // each thread owns the contiguous run [j0, j1) of the row
  const int per = (n + kTkThreads - 1) / kTkThreads;
  const int j0 = min(n, tid * per), j1 = min(n, j0 + per);

  // ---- stage the row (and clear the histogram meanwhile) -------------------
  for (int b = tid; b < kTkBins; b += kTkThreads) hist[b] = 0;
  const float* srow = a.scores + (size_t)pbeg * H + (size_t)h * P_r;
  float lo = FLT_MAX, hi = -FLT_MAX;
  for (int base = 0; base < n; base += kTkThreads * kTkBatch) {
    float sv[kTkBatch];
    int pv[kTkBatch];
#pragma unroll
    for (int b = 0; b < kTkBatch; ++b) {
      const int j = base + b * kTkThreads + tid;
      sv[b] = j < n ? srow[j] : 0.f;
      pv[b] = (j < n && with_phys) ? pt[j] : 0;
    }
#pragma unroll
    for (int b = 0; b < kTkBatch; ++b) {
      const int j = base + b * kTkThreads + tid;
      if (j < n) {
        const float v = sv[b] == 0.f ? 0.f : sv[b];   // -0 -> +0
        s_score[j] = v;
        if (with_phys) s_pt[j] = pv[b];
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
      }
    }
  }
  block_minmax(lo, hi, s_mm[0]);               // also publishes s_score

  float Ts = -FLT_MAX;
  int Tj = n;                                  // take == n: everything
  if (take < n) {
    int kk = take;                             // still to take among candidates
    int ncand = n;
    // candidates: lo <= s <= hi, and (after a binning step) bin == cbin
    float crange = 0.f;
    int cbin = -1;
    int round = 0;
    while (ncand > kTkCand && lo < hi && hi - lo >= FLT_MIN) {
      const float range = hi - lo;
      if (round > 0) {
        for (int b = tid; b < kTkBins; b += kTkThreads) hist[b] = 0;
        __syncthreads();
      }
      for (int j = j0; j < j1; ++j) {
        const float s = s_score[j];
        if (s >= lo && s <= hi) atomicAdd(&hist[score_bin(s, lo, range)], 1);
      }
      __syncthreads();
      if (wave_id() == 0) {
        // lane l owns bins NB-1-16l ... NB-16-16l: lane order walks downward
        constexpr int PER = kTkBins / kWave;
        const int lane = lane_id();
        int local = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) local += hist[kTkBins - 1 - (lane * PER + k)];
        const int incl = wave_incl_scan(local);
        const int excl = incl - local;
        if (excl < kk && incl >= kk) {
          int run = excl;
          for (int k = 0; k < PER; ++k) {
            const int b = kTkBins - 1 - (lane * PER + k);
            const int c = hist[b];
            if (run + c >= kk) {
              s_b = b;
              s_above = run;
              s_cnt = c;
              break;
            }
            run += c;
          }
        }
      }
      __syncthreads();
      cbin = s_b;
      crange = range;
      kk -= s_above;
      ncand = s_cnt;
      ++round;
      if (ncand <= kTkCand) break;
      // too many left: shrink [lo, hi] to the crossing bin's exact extremes
      float nlo = FLT_MAX, nhi = -FLT_MAX;
      for (int j = j0; j < j1; ++j) {
        const float s = s_score[j];
        if (s >= lo && s <= hi && score_bin(s, lo, range) == cbin) {
          nlo = fminf(nlo, s);
          nhi = fmaxf(nhi, s);
        }
      }
      block_minmax(nlo, nhi, s_mm[round & 1]);
      lo = nlo;
      hi = nhi;
      cbin = -1;
    }

    if (lo == hi) {
      // every candidate ties: the kk-th lowest index holding the value
      int mine = 0;
      for (int j = j0; j < j1; ++j) mine += s_score[j] == lo ? 1 : 0;
      int total;
      int seen = block_excl_scan(mine, s_scan[0], &total);
      for (int j = j0; j < j1; ++j) {
        if (s_score[j] == lo) {
          if (++seen == kk) s_tj = j;
        }
      }
      __syncthreads();
      Ts = lo;
      Tj = s_tj;
    } else if (ncand > kTkCand) {
      // only for score ranges below FLT_MIN: rank in place against the row
      for (int j = tid; j < n; j += kTkThreads) {
        const float sj = s_score[j];
        if (!(sj >= lo && sj <= hi)) continue;
        int rank = 0;
        for (int t = 0; t < n; ++t) {
          const float st = s_score[t];
          rank += (st >= lo && st <= hi && (st > sj || (st == sj && t < j))) ? 1 : 0;
        }
        if (rank == kk - 1) {
          s_ts = sj;
          s_tj = j;
        }
      }
      __syncthreads();
      Ts = s_ts;
      Tj = s_tj;
    } else {
      // gather the candidates in index order, then rank each exactly
      int mine = 0;
      for (int j = j0; j < j1; ++j) {
        const float s = s_score[j];
        mine += (s >= lo && s <= hi && (cbin < 0 || score_bin(s, lo, crange) == cbin)) ? 1 : 0;
      }
      int total;
      int at = block_excl_scan(mine, s_scan[0], &total);
      for (int j = j0; j < j1; ++j) {
        const float s = s_score[j];
        if (s >= lo && s <= hi && (cbin < 0 || score_bin(s, lo, crange) == cbin)) {
          s_cidx[at] = j;
          s_cval[at] = s;
          ++at;
        }
      }
      __syncthreads();
      for (int i = tid; i < total; i += kTkThreads) {
        const float si = s_cval[i];
        int rank = 0;
        for (int t = 0; t < total; ++t) {
          const float st = s_cval[t];
          rank += (st > si || (st == si && t < i)) ? 1 : 0;
        }
        if (rank == kk - 1) {
          s_ts = si;
          s_tj = s_cidx[i];
        }
      }
      __syncthreads();
      Ts = s_ts;
      Tj = s_tj;
    }
  }

  // ---- index-ordered compaction ---------------------------------------------
  int mine = 0;
  for (int j = j0; j < j1; ++j) {
    const float s = s_score[j];
    mine += (s > Ts || (s == Ts && j <= Tj)) ? 1 : 0;
  }
  int total;
  int pos = block_excl_scan(mine, s_scan[1], &total);
  for (int j = j0; j < j1; ++j) {
    const float s = s_score[j];
    if (s > Ts || (s == Ts && j <= Tj)) {
      out[pos] = j;
      if (out_phys) out_phys[pos] = s_pt[j];
      ++pos;
    }
  }
  for (int j = take + tid; j < K; j += kTkThreads) {
    out[j] = -1;
    if (out_phys) out_phys[j] = -1;
  }
}

size_t topk_dyn_lds(int max_pages, bool with_phys) {
  return (size_t)max_pages * sizeof(float) * (with_phys ? 2 : 1);
}

constexpr size_t kTkStaticLds =
    (kTkBins + 2 * kTkCand + 3 * kTkWaves + 4 * kTkWaves + 8) * sizeof(int);

}  // namespace

bool topk_phys_fits(int max_pages) {
  return topk_dyn_lds(max_pages, true) + kTkStaticLds <= kTkLdsBudget;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  const bool with_phys = a.sel_phys != nullptr;
  const size_t lds = topk_dyn_lds(a.max_pages > 0 ? a.max_pages : 1, with_phys);
  if (lds + kTkStaticLds > kTkLdsBudget) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_kernel, dim3(a.B * a.H_kv), dim3(kTkThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace qas
