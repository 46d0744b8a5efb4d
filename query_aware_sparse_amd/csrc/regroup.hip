// Windowed page-affinity regroup of a chunk's queries (the PageWeaver notes,
// Algorithm 1 and its GPU mapping, annotations 69BMX58K / TT5ABQLD /
// AWLR3K97): per KV head and per window of W consecutive queries of one
// request, the lowest unassigned query seeds a group whose union U starts as
// its page set; the next member is the unassigned query with the smallest
// (|S_j minus U|, j), after which U grows and the costs are taken again; a
// group closes at `group` members.  The output is only the execution order
// (original query ID of every slot); the union kernel reads Q, causal limits
// and sets through it and writes outputs to the original rows.
//
// One workgroup per (window, KV head), four lanes per query: lane 4q + k
// holds words [8k, 8k + 8) of query q's page bitmap (1024 pages) and the same
// words of the group's union U.  A pick is one round: each lane's popcount of
// its words of S_j and not U, a quad sum, a wave argmin of (cost, query) by
// DPP, one LDS exchange of the per-wave minima (one barrier), then every lane
// ORs the winner's words into U straight from the LDS bitmaps (broadcast
// reads).  A group's seed is the same round with every cost taken as 0, so
// the lowest unassigned query wins.  The pages' bitmaps hold 512 pages
// (their 64K context at page size 128); here 1024, so a 64K context at page
// size 64 is still regrouped.  Requests with more pages keep the identity
// order, as the pages do.
#include "qas_device.h"
#include "qas_internal.h"

namespace qas {

namespace {

constexpr int kRgWords = 32;                    // 1024 pages
constexpr int kRgLanesPerQuery = 4;
constexpr int kRgWordsPerLane = kRgWords / kRgLanesPerQuery;
constexpr int kRgMaxWindow = 128;

struct WindowInfo {
  int r, q0, nq;   // request, first query, queries in the window (0: none)
};

// Window wi of the launch: requests contribute ceil(n_r / W) windows each.
__device__ WindowInfo find_window(const int32_t* q_indptr, int B, int W, int wi) {
  WindowInfo w{0, 0, 0};
  int base = 0;
  for (int r = 0; r < B; ++r) {
    const int a = q_indptr[r], n = q_indptr[r + 1] - a;
    const int nw = (n + W - 1) / W;
    if (wi < base + nw) {
      const int local = wi - base;
      w.r = r;
      w.q0 = a + local * W;
      w.nq = min(W, n - local * W);
      return w;
    }
    base += nw;
  }
  return w;
}

// min over the wave of a 32-bit key: DPP within each row of 16 lanes, then
// row_bcast:15 / row_bcast:31 carry the row minima upwards (rows outside the
// row mask keep their value), so lane 63 ends with the wave's minimum
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// Page bitmaps of the window's queries in LDS (rows of RS words, zeroed
// here): every thread issues BL set-entry loads before its LDS atomics, so
// the loads of a batch are in flight together.  Ends with a barrier.
template <int NT, int RS>
__device__ __forceinline__ void build_bitmaps(const RegroupArgs& a, const WindowInfo& win, int h,
                                              int n_pages, uint32_t* bm, int rows) {
  constexpr int BL = 8;
  const int tid = threadIdx.x;
  for (int i = tid; i < rows * RS; i += NT) bm[i] = 0u;
  __syncthreads();
  const int entries = win.nq * a.kq;                 // >= 1
  for (int e0 = 0; e0 < entries; e0 += NT * BL) {
    int pg[BL];
#pragma unroll
    for (int b = 0; b < BL; ++b) {
      const int e = min(e0 + b * NT + tid, entries - 1);
      const int i = e / a.kq;
      pg[b] = a.sets[((size_t)(win.q0 + i) * a.H_kv + h) * a.kq + (e - i * a.kq)];
    }
#pragma unroll
    for (int b = 0; b < BL; ++b) {
      const int e = e0 + b * NT + tid;
      const int p = pg[b];
      if (e < entries && p >= 0 && p < n_pages) atomicOr(&bm[(e / a.kq) * RS + (p >> 5)], 1u << (p & 31));
    }
  }
  __syncthreads();
}

// WQ = queries per window slot range (64 or 128): 4 * WQ threads
template <int WQ>
__global__ __launch_bounds__(kRgLanesPerQuery * WQ) void regroup_kernel(RegroupArgs a) {
  constexpr int NT = kRgLanesPerQuery * WQ;
  constexpr int NW = NT / kWave;
  __shared__ __align__(16) uint32_t bm[WQ][kRgWords];
  __shared__ uint32_t wmin[2][NW];
  const int wi = blockIdx.x, h = blockIdx.y;
  const WindowInfo win = find_window(a.q_indptr, a.B, a.window, wi);
  if (win.nq == 0) return;                    // uniform: no such window
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int32_t* out = a.ids + (size_t)h * a.N + win.q0;
  const int L = a.seq_lens[win.r];
  const int P_r = a.page_indptr[win.r + 1] - a.page_indptr[win.r];
  const int n_pages = L > 0 ? min((L + a.S - 1) / a.S, P_r) : 0;
  if (n_pages > kRgWords * 32 || a.group <= 1) {   // identity order
    for (int i = tid; i < win.nq; i += NT) out[i] = win.q0 + i;
    return;
  }

  // ---- page bitmaps of the window's queries --------------------------------
  build_bitmaps<NT, kRgWords>(a, win, h, n_pages, &bm[0][0], WQ);
  const int q = tid / kRgLanesPerQuery;       // this lane's query
  const int k = tid % kRgLanesPerQuery;       // and its word range
  uint32_t b[kRgWordsPerLane], U[kRgWordsPerLane];
#pragma unroll
  for (int w = 0; w < kRgWordsPerLane; ++w) b[w] = bm[q][k * kRgWordsPerLane + w];
  bool alive = q < win.nq;

  int in_group = 0;
  for (int pos = 0; pos < win.nq; ++pos) {
    const bool seed = in_group == 0;
    uint32_t cost = 0;
    if (!seed) {
      uint32_t c[4] = {0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < kRgWordsPerLane; ++w) c[w & 3] += __popc(b[w] & ~U[w]);
      cost = c[0] + c[1] + c[2] + c[3];
      // quad sum: the four lanes of the query
      cost += (uint32_t)__builtin_amdgcn_mov_dpp((int)cost, 0xB1, 0xF, 0xF, true);
      cost += (uint32_t)__builtin_amdgcn_mov_dpp((int)cost, 0x4E, 0xF, 0xF, true);
    }
    const uint32_t key = alive ? (cost << 8) | (uint32_t)q : 0xffffffffu;
    const uint32_t wk = wave_min_u32(key);
    if (lane == 0) wmin[pos & 1][wave] = wk;
    __syncthreads();
    uint32_t best = wmin[pos & 1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) best = min(best, wmin[pos & 1][w]);
    const int winq = (int)(best & 0xffu);
    if (tid == 0) out[pos] = win.q0 + winq;
    if (q == winq) alive = false;
#pragma unroll
    for (int w = 0; w < kRgWordsPerLane; ++w) {
      const uint32_t x = bm[winq][k * kRgWordsPerLane + w];
      U[w] = seed ? x : (U[w] | x);
    }
    in_group = in_group + 1 == a.group ? 0 : in_group + 1;
  }
}

}  // namespace

int regroup_max_pages() { return kRgWords * 32; }
int regroup_max_window() { return kRgMaxWindow; }

hipError_t launch_regroup(const RegroupArgs& a, hipStream_t s) {
  dim3 grid(a.max_windows, a.H_kv);
  if (a.window <= 64)
    hipLaunchKernelGGL(regroup_kernel<64>, grid, dim3(kRgLanesPerQuery * 64), 0, s, a);
  else
    hipLaunchKernelGGL(regroup_kernel<128>, grid, dim3(kRgLanesPerQuery * 128), 0, s, a);
  return hipGetLastError();
}

}  // namespace qas
