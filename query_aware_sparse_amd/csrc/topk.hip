// Top-K page selection per (request, KV head): the Quest page's second stage
// ("3.1.1 · Quest", §1 and Fig. 1), with ties going to the lower page index.
//
// One workgroup per row.  Scores become order-preserving uint32 keys in LDS;
// a most-significant-digit-first radix select (four 8-bit passes, LDS
// histograms) finds the K-th largest key T and how many keys equal to T must
// be taken.  An index-ordered compaction (wave ballot + mbcnt prefix counts)
// then emits the selected pages in ascending order, which also resolves ties
// to the lower index without any sort.
#include "qas_device.h"
#include "qas_internal.h"

namespace qas {

namespace {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Exclusive count of set flags before this thread in the workgroup, in
// thread order; *total receives the workgroup's count.  Uses `scratch`
// (kTopkWaves ints); contains two barriers.
__device__ __forceinline__ int block_excl_count(bool flag, int* scratch, int* total) {
  const uint64_t mask = __ballot(flag);
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
  if (lane == 0) scratch[wave] = __popcll(mask);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int c = scratch[w];
    before += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + in_wave;
}

// Inclusive prefix sum over the workgroup in thread order.
__device__ __forceinline__ int block_incl_scan(int v, int* scratch) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == kWave - 1) scratch[wave] = v;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) before += w < wave ? scratch[w] : 0;
  __syncthreads();
  return v + before;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ uint32_t keys[];
  __shared__ int hist[256];
  __shared__ int scan_scratch[kTopkWaves];
  __shared__ int cnt_scratch[kTopkWaves];
  __shared__ uint32_t s_prefix;
  __shared__ int s_kk;

  const int row = blockIdx.x;
  const int H = a.H_kv;
  const int r = row / H, h = row - (row / H) * H;
  const int pbeg = a.page_indptr[r];
  const int P_r = a.page_indptr[r + 1] - pbeg;
  const int L = a.seq_lens[r];
  // never more keys than the LDS array sized by max_pages holds
  const int n = min(min((L + a.S - 1) / a.S, P_r), a.max_pages);
  const int K = a.k;
  const int take = min(K, n);
  const int tid = threadIdx.x;
  int32_t* out = a.sel + (size_t)row * K;
  if (a.sel_count && tid == 0) a.sel_count[row] = take;

  if (take == n) {  // every existing page is selected
    for (int j = tid; j < K; j += kTopkThreads) out[j] = j < n ? j : -1;
    return;
  }

  const float* srow = a.scores + (size_t)pbeg * H + (size_t)h * P_r;
  for (int j = tid; j < n; j += kTopkThreads) keys[j] = order_key(srow[j]);

  uint32_t prefix = 0, pmask = 0;
  int kk = take;  // keys still to take among those matching `prefix`
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < n; j += kTopkThreads) {
      const uint32_t key = keys[j];
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    // thread t owns digit 255 - t: scanning in thread order walks digits
    // from the largest down
    const int cnt = hist[255 - tid];
    const int incl = block_incl_scan(cnt, scan_scratch);
    const int excl = incl - cnt;
    if (excl < kk && incl >= kk) {
      s_prefix = prefix | ((uint32_t)(255 - tid) << shift);
      s_kk = kk - excl;
    }
    __syncthreads();
    prefix = s_prefix;
    kk = s_kk;
    pmask |= 255u << shift;
  }
  const uint32_t T = prefix;  // the K-th largest key; take kk keys equal to T

  int eq_carry = 0, sel_carry = 0;
  for (int base = 0; base < n; base += kTopkThreads) {
    const int j = base + tid;
    const uint32_t key = j < n ? keys[j] : 0u;
    const bool gt = j < n && key > T;
    const bool eq = j < n && key == T;
    int eq_total, sel_total;
    const int eq_rank = eq_carry + block_excl_count(eq, cnt_scratch, &eq_total);
    const bool s = gt || (eq && eq_rank < kk);
    const int pos = sel_carry + block_excl_count(s, cnt_scratch, &sel_total);
    if (s) out[pos] = j;
    eq_carry += eq_total;
    sel_carry += sel_total;
  }
  for (int j = take + tid; j < K; j += kTopkThreads) out[j] = -1;
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  // the LDS key array is sized for the longest row of the batch
  const size_t lds = (size_t)(a.max_pages > 0 ? a.max_pages : 1) * sizeof(uint32_t);
  dim3 grid(a.B * a.H_kv);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(kTopkThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace qas
