// Workgroup-level top-K page selection for one (request, KV head) row: the
// Quest page's second stage ("3.1.1 · Quest", §1 and Fig. 1), ordered by
// (score descending, page index ascending) so ties go to the lower index.
// Used by the standalone top-K kernel and inside the attention kernel of the
// decode layer.
//
// A workgroup of NT threads (kTkThreads in the standalone kernel, the
// attention kernel's workgroup inside it) holds the row in registers: thread t
// keeps the run of scores j in [t*PT, t*PT + PT) and their physical pages.
// Per-element steps are branch-free (invalid elements get the bin past the
// last one and count in no bin: their LDS atomics are masked off, as
// thousands of them on one spare bin serialised on its address in rows much
// shorter than the workgroup's capacity), block-uniform values live in
// scalar registers, and
// reductions within a wave use DPP, so one select costs a few thousand
// cycles (a wave64 vector instruction occupies its SIMD for four cycles, so
// the instruction count is the cost).  Selection narrows a closed score
// interval [lo, hi] that holds the K-th largest score:
//   * histogram the candidates into kTkBins bins through a monotone map
//     (lo in bin 0, hi in the top bin);
//   * every wave walks the bins from the top to the one holding the K-th
//     score (a scan over the lanes' 16-bin sums finds the lane, a row scan
//     over that lane's bins the bin); scores in higher bins are taken and
//     that bin's scores are the candidates (if still too many, [lo, hi]
//     shrinks to their exact min/max and the step repeats; the bin misses
//     lo or hi, so each repeat drops at least one distinct value); a row
//     of no more than kTkDirect scores skips the histogram, and one of up
//     to kTkCand takes at most kTkSmallRounds rounds;
//   * rank the candidates exactly by (score desc, index asc).  The last one
//     taken is the threshold (T_s, T_j): page j is selected iff s_j > T_s,
//     or s_j == T_s and j <= T_j.
// An index-ordered compaction (one workgroup scan over the runs) gives every
// selected page its position in the ascending output list.  Pages fixed in
// advance (the sink pages j < fs_end and the local-window pages j >=
// fl_begin, the Quest page's §3.2 candidate set C_local | C_sink | C_quest)
// join the top-K in that list; a page in several sets appears once.  -0.0 and +0.0
// are equal scores; NaN ranks below every number.
#pragma once

#include <float.h>

#include "qas_device.h"

namespace qas {

constexpr int kTkThreads = 512;      // workgroup of the standalone top-K kernel
constexpr int kTkMaxWaves = 8;       // largest workgroup a row select runs in
constexpr int kTkBins = 1024;
constexpr int kTkCand = 512;         // candidates ranked from LDS
// Ranking n candidates costs each thread ~n / 2 broadcast reads, so rows
// whose candidates number more than kTkDirect take histogram rounds first
// (at most kTkSmallRounds of them while they number no more than kTkCand).
constexpr int kTkDirect = 64;
constexpr int kTkSmallRounds = 2;
constexpr float kTkMinRange = 1e-30f;

struct TopkShared {
  __align__(16) int hist[kTkBins + 4];
  // candidates as 64-bit keys: order key of the score above the complement
  // of the page index, so a larger key ranks higher (ties to the lower index)
  __align__(16) uint64_t ckey[kTkCand];
  int scan[2][kTkMaxWaves];
  float mm[2 * kTkMaxWaves];
  int nslot, tj;
  float ts;
};

namespace tk {

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

// Exclusive prefix sum over the workgroup (NW waves) in thread order; one
// barrier.  `scratch` (NW ints) must not be rewritten before another barrier.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* scratch, int* total) {
  const int incl = wave_incl_scan(v);
  if (lane_id() == kWave - 1) scratch[wave_id()] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
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

// min and max over the wave, returned in every lane: DPP within rows of 16
// lanes, then row_bcast:15 / row_bcast:31 carry the row results upwards
// (rows outside the row mask keep their value), so lane 63 holds the
// wave's result; no LDS traffic.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_keep_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                    ROW_MASK, 0xF, false));
}
__device__ __forceinline__ void wave_minmax(float& lo, float& hi) {
  lo = fminf(lo, dpp_f<0xB1>(lo));
  hi = fmaxf(hi, dpp_f<0xB1>(hi));
  lo = fminf(lo, dpp_f<0x4E>(lo));
  hi = fmaxf(hi, dpp_f<0x4E>(hi));
  lo = fminf(lo, dpp_f<0x141>(lo));
  hi = fmaxf(hi, dpp_f<0x141>(hi));
  lo = fminf(lo, dpp_f<0x140>(lo));
  hi = fmaxf(hi, dpp_f<0x140>(hi));
  lo = fminf(lo, dpp_keep_f<0x142, 0xA>(lo));
  hi = fmaxf(hi, dpp_keep_f<0x142, 0xA>(hi));
  lo = fminf(lo, dpp_keep_f<0x143, 0xC>(lo));
  hi = fmaxf(hi, dpp_keep_f<0x143, 0xC>(hi));
  lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lo), kWave - 1));
  hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hi), kWave - 1));
}

// (min, max) over the workgroup (NW waves); one barrier.
template <int NW>
__device__ __forceinline__ void block_minmax(float& lo, float& hi, float* scratch) {
  wave_minmax(lo, hi);
  if (lane_id() == 0) {
    scratch[2 * wave_id()] = lo;
    scratch[2 * wave_id() + 1] = hi;
  }
  __syncthreads();
  lo = scratch[0];
  hi = scratch[1];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lo = fminf(lo, scratch[2 * w]);
    hi = fmaxf(hi, scratch[2 * w + 1]);
  }
}

__device__ __forceinline__ float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
__device__ __forceinline__ int uniform_i(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Monotone map of a score in [lo, hi] to one of kTkBins bins, with lo in bin
// 0 and hi in a higher bin whenever lo < hi.  Normal ranges bin the float
// value linearly; ranges too narrow (or too wide) for a finite fp32 scale
// bin the order-preserving integer key, shifted so that the key range
// spans fewer than kTkBins bins.  lo and hi must be block-uniform.
struct Binner {
  float lo, inv;
  uint32_t klo;
  int kshift;
  bool by_key;
  __device__ __forceinline__ void init(float l, float h) {
    const float range = h - l;
    by_key = uniform_i(!(range >= kTkMinRange && range <= FLT_MAX) ? 1 : 0) != 0;
    lo = l;
    inv = uniform_f(by_key ? 0.f : (float)kTkBins / range);
    klo = order_key(l);
    const uint32_t span = order_key(h) - klo;
    // smallest shift with (span >> shift) < kTkBins (= 2^10)
    const int bits = span ? 32 - __clz((int)span) : 0;
    kshift = uniform_i(bits > 10 ? bits - 10 : 0);
  }
  // the two maps; callers branch once on the uniform by_key
  __device__ __forceinline__ int by_value(float s) const {
    const float t = fminf(fmaxf((s - lo) * inv, 0.f), (float)(kTkBins - 1));
    return (int)t;
  }
  __device__ __forceinline__ int by_order_key(float s) const {
    return (int)((order_key(s) - klo) >> kshift);
  }
};

}  // namespace tk

// One row held by the workgroup: PT scores per thread.
template <int PT, int NT = kTkThreads>
struct TopkRow {
  static constexpr int NW = NT / kWave;
  static_assert(NT % kWave == 0 && NW <= kTkMaxWaves, "workgroup of whole waves");
  float v[PT];
  int pv[PT];
  int j0, n;
  float Ts;
  int Tj;
  int fs_end = 0;                 // pages j < fs_end are kept (sinks)
  int fl_begin = 0x7fffffff;      // pages j >= fl_begin are kept (local window)

  // Fixed pages of a row of L tokens (n valid pages of S tokens): those
  // holding the first sink_tokens tokens and the last local_tokens tokens.
  __device__ __forceinline__ void set_fixed(int L, int S, int sink_tokens, int local_tokens) {
    fs_end = sink_tokens > 0 ? min(n, (sink_tokens + S - 1) / S) : 0;
    fl_begin = local_tokens > 0 ? max(0, L - local_tokens) / S : 0x7fffffff;
  }

  // Scores srow[j] for j < cap (the row's allocated extent; entries at or
  // beyond the row length are loaded but never used).
  __device__ __forceinline__ void load_scores(const float* srow, int cap) {
    j0 = threadIdx.x * PT;
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      const int j = j0 + k;
      v[k] = j < cap ? srow[j] : 0.f;
    }
  }

  // Row length n_ and, if pt != NULL, the physical pages pt[0, n_).
  __device__ __forceinline__ void load_pages(const int32_t* pt, int n_) {
    n = n_;
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      const int j = j0 + k;
      pv[k] = (j < n && pt) ? pt[j] : 0;
    }
  }

  // Scores and physical pages of a row as 16-byte words, in two steps so
  // that the loads can be issued at kernel entry, before the row's length is
  // known: issue_x4 loads quads [j0, j0 + PT) of srow and prow (both 16-byte
  // aligned, holding at least cap rounded up to 4 entries; a quad past cap
  // reads the row's first quad), finish_x4 keeps scores below cap and pages
  // below n_.
  float4 xs[PT / 4];
  int4 xp[PT / 4];
  __device__ __forceinline__ void issue_x4(const float* srow, const int32_t* prow, int cap) {
    static_assert(PT % 4 == 0, "quads per thread");
    j0 = threadIdx.x * PT;
#pragma unroll
    for (int q = 0; q < PT / 4; ++q) {
      const int o = j0 + 4 * q < cap ? j0 + 4 * q : 0;
      xs[q] = *reinterpret_cast<const float4*>(srow + o);
      xp[q] = *reinterpret_cast<const int4*>(prow + o);
    }
  }
  __device__ __forceinline__ void finish_x4(int cap, int n_) {
    n = n_;
#pragma unroll
    for (int q = 0; q < PT / 4; ++q) {
      const int j = j0 + 4 * q;
      v[4 * q] = j < cap ? xs[q].x : 0.f;
      v[4 * q + 1] = j + 1 < cap ? xs[q].y : 0.f;
      v[4 * q + 2] = j + 2 < cap ? xs[q].z : 0.f;
      v[4 * q + 3] = j + 3 < cap ? xs[q].w : 0.f;
      pv[4 * q] = j < n ? xp[q].x : 0;
      pv[4 * q + 1] = j + 1 < n ? xp[q].y : 0;
      pv[4 * q + 2] = j + 2 < n ? xp[q].z : 0;
      pv[4 * q + 3] = j + 3 < n ? xp[q].w : 0;
    }
  }

  __device__ __forceinline__ void load(const float* srow, const int32_t* pt, int n_) {
    load_scores(srow, n_);
    load_pages(pt, n_);
  }

  __device__ __forceinline__ bool valid(int k) const { return j0 + k < n; }

  __device__ __forceinline__ bool selected(int k) const {
    const int j = j0 + k;
    return valid(k) & ((v[k] > Ts) | ((v[k] == Ts) & (j <= Tj)) | (j < fs_end) | (j >= fl_begin));
  }

  // Find (Ts, Tj) for the top `take` (<= n) entries; every thread of the
  // workgroup must call this.
  __device__ void select(int take, TopkShared& sh) {
    using namespace tk;
    const int tid = threadIdx.x;
    float lo = FLT_MAX, hi = -FLT_MAX;
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      // -0 ranks as +0 and NaN below every number
      float x = v[k];
      x = x == 0.f ? 0.f : x;
      x = x != x ? -INFINITY : x;
      v[k] = x;
      const bool ok = valid(k);
      lo = fminf(lo, ok ? x : FLT_MAX);
      hi = fmaxf(hi, ok ? x : -FLT_MAX);
    }
    Ts = -INFINITY;
    Tj = n;                                    // take == n: everything
    if (take >= n) return;

    for (int b = tid; b < kTkBins + 4; b += NT) sh.hist[b] = 0;
    if (tid == 0) sh.nslot = 0;
    block_minmax<NW>(lo, hi, sh.mm);
    lo = uniform_f(lo);
    hi = uniform_f(hi);
    int kk = take;                             // still to take among candidates
    int ncand = n;
    Binner bin;
    int cbin = -1;                             // bin of the candidates (last round)
    int bk[PT];                                // element bins of the last round
    int round = 0;
    // more rounds pay while the candidates are many (the rank is quadratic)
    auto narrow = [&](int nc, int r) {
      return nc > kTkCand || (nc > kTkDirect && r < kTkSmallRounds);
    };
    while (narrow(ncand, round) && lo < hi) {
      bin.init(lo, hi);
      if (round > 0) {
        for (int b = tid; b < kTkBins + 4; b += NT) sh.hist[b] = 0;
        __syncthreads();
      }
      // skipped elements get bin kTkBins and are not counted; out-of-range
      // values may map anywhere, the select discards them
      if (bin.by_key) {
#pragma unroll
        for (int k = 0; k < PT; ++k) {
          // the empty asm keeps the key computation on this (rare) path
          float x = v[k];
          asm volatile("" : "+v"(x));
          const int b = bin.by_order_key(x);
          bk[k] = (valid(k) & (v[k] >= lo) & (v[k] <= hi)) ? b : kTkBins;
        }
      } else {
#pragma unroll
        for (int k = 0; k < PT; ++k) {
          const int b = bin.by_value(v[k]);
          bk[k] = (valid(k) & (v[k] >= lo) & (v[k] <= hi)) ? b : kTkBins;
        }
      }
#pragma unroll
      for (int k = 0; k < PT; ++k)
        if (bk[k] < kTkBins) atomicAdd(&sh.hist[bk[k]], 1);
      __syncthreads();
      {
        // every wave walks the histogram itself, so no barrier publishes the
        // result; lane l owns bins NB-1-16l ... NB-16-16l (lane order walks
        // downward)
        constexpr int PER = kTkBins / kWave;
        static_assert(PER == 16, "one row of 16 lanes re-reads a lane's bins");
        const int lane = lane_id();
        int local = 0;
        const int4* hv = reinterpret_cast<const int4*>(sh.hist + kTkBins - PER * (lane + 1));
#pragma unroll
        for (int q4 = 0; q4 < PER / 4; ++q4) {
          const int4 x = hv[q4];
          local += (x.x + x.y) + (x.z + x.w);
        }
        const int incl = wave_incl_scan(local);
        const int excl = incl - local;
        // the lane whose 16 bins hold the kk-th largest element
        const uint64_t here = __ballot(excl < kk && incl >= kk);
        const int src = uniform_i(__ffsll((unsigned long long)here) - 1);
        const int above_src = __builtin_amdgcn_readlane(excl, src);
        // lanes 16m + i (every row alike) take bin i of that lane in walk
        // order (descending bins); a row scan finds the crossing bin
        const int i = lane & (PER - 1);
        const int bi = kTkBins - 1 - (src * PER + i);
        const int ci = sh.hist[bi];
        int run = ci;
        run += dpp_shift<0x111, 0xF>(run);   // row_shr:1
        run += dpp_shift<0x112, 0xF>(run);   // row_shr:2
        run += dpp_shift<0x114, 0xF>(run);   // row_shr:4
        run += dpp_shift<0x118, 0xF>(run);   // row_shr:8
        const int before = above_src + run - ci;
        const uint64_t hit = __ballot((before < kk) & (before + ci >= kk)) & 0xFFFFull;
        const int at = uniform_i(__ffsll((unsigned long long)hit) - 1);
        cbin = __builtin_amdgcn_readlane(bi, at);
        kk -= __builtin_amdgcn_readlane(before, at);
        ncand = __builtin_amdgcn_readlane(ci, at);
      }
      ++round;
      if (!narrow(ncand, round)) break;
      // too many left: shrink [lo, hi] to the crossing bin's exact extremes
      // (it misses lo or hi, so every round drops at least one value)
      float nlo = FLT_MAX, nhi = -FLT_MAX;
#pragma unroll
      for (int k = 0; k < PT; ++k) {
        const bool in = bk[k] == cbin;
        nlo = fminf(nlo, in ? v[k] : FLT_MAX);
        nhi = fmaxf(nhi, in ? v[k] : -FLT_MAX);
      }
      block_minmax<NW>(nlo, nhi, sh.mm);
      lo = uniform_f(nlo);
      hi = uniform_f(nhi);
      cbin = -1;
    }
    // candidates: the crossing bin of the last round, else all of [lo, hi]
    auto is_cand = [&](int k) {
      return cbin >= 0 ? bk[k] == cbin : (valid(k) & (v[k] >= lo) & (v[k] <= hi));
    };

    if (lo == hi) {
      // every candidate ties: the kk-th lowest index holding the value
      int mine = 0;
#pragma unroll
      for (int k = 0; k < PT; ++k) mine += (valid(k) & (v[k] == lo)) ? 1 : 0;
      int total;
      int seen = block_excl_scan<NW>(mine, sh.scan[0], &total);
#pragma unroll
      for (int k = 0; k < PT; ++k) {
        const bool eq = valid(k) & (v[k] == lo);
        seen += eq ? 1 : 0;
        if (eq && seen == kk) sh.tj = j0 + k;
      }
      __syncthreads();
      Ts = lo;
      Tj = uniform_i(sh.tj);
    } else {
      // at most kTkCand (= ncand) candidates: gather their keys in any order
      // (one LDS atomic per wave) and rank each exactly by (score desc, index
      // asc); the keys are distinct, so the ranks are 0 .. ncand - 1
      const int total = ncand;
      const int padded = (total + 7) & ~7;    // <= kTkCand; zero keys rank below all
      for (int i = total + tid; i < padded; i += NT) sh.ckey[i] = 0ull;
      int mine = 0;
#pragma unroll
      for (int k = 0; k < PT; ++k) mine += is_cand(k) ? 1 : 0;
      const int incl = wave_incl_scan(mine);
      const int wave_total = __builtin_amdgcn_readlane(incl, kWave - 1);
      if (wave_total > 0) {                    // uniform; most waves hold none
        int base = 0;
        if (lane_id() == kWave - 1) base = atomicAdd(&sh.nslot, incl);
        int at = __builtin_amdgcn_readlane(base, kWave - 1) + incl - mine;
        if (mine > 0) {
#pragma unroll
          for (int k = 0; k < PT; ++k) {
            if (is_cand(k)) {
              sh.ckey[at] = ((uint64_t)order_key(v[k]) << 32) | (uint32_t)~(uint32_t)(j0 + k);
              ++at;
            }
          }
        }
      }
      __syncthreads();
      // CPT candidates per thread (2 in a 256-thread workgroup, 1 in a
      // 512-thread one) share every 16-byte broadcast read of the key list
      // (a real key's order half is at least order_key(-inf) > 0, so the
      // zero padding counts for none)
      constexpr int CPT = (kTkCand + NT - 1) / NT;
      for (int i0 = tid; i0 < total; i0 += CPT * NT) {
        uint64_t kc[CPT];
        int rk[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const int i = i0 + c * NT;
          kc[c] = i < total ? sh.ckey[i] : ~0ull;
          rk[c] = 0;
        }
        for (int t = 0; t < padded; t += 8) {
          const ulonglong2* kp = reinterpret_cast<const ulonglong2*>(sh.ckey + t);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const ulonglong2 x = kp[u];
#pragma unroll
            for (int c = 0; c < CPT; ++c) rk[c] += (x.x > kc[c] ? 1 : 0) + (x.y > kc[c] ? 1 : 0);
          }
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          if (i0 + c * NT < total && rk[c] == kk - 1) {
            const uint32_t ok = (uint32_t)(kc[c] >> 32);
            sh.ts = __uint_as_float((ok & 0x80000000u) ? (ok ^ 0x80000000u) : ~ok);
            sh.tj = (int)~(uint32_t)kc[c];
          }
        }
      }
      __syncthreads();
      Ts = uniform_f(sh.ts);
      Tj = uniform_i(sh.tj);
    }
  }

  // Output position of this thread's first selected page (selected pages
  // are numbered in ascending page order) and, in *count, the number of
  // selected pages; every thread must call this.
  __device__ __forceinline__ int first_position(TopkShared& sh, int* count) const {
    int mine = 0;
#pragma unroll
    for (int k = 0; k < PT; ++k) mine += selected(k) ? 1 : 0;
    return tk::block_excl_scan<NW>(mine, sh.scan[1], count);
  }
};

}  // namespace qas
