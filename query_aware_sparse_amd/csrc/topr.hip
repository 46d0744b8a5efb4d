// Exact token top-R by branch-and-bound over the page bounds ("3.1.1 ·
// Quest", §3.2 on stopping rules beyond a fixed top-K): pages are read in
// descending bound order (ties to the lower page index), the R-th largest
// true logit read so far is tau_R, and the search stops when the next page's
// bound is below tau_R, since no token of the remaining pages can then enter
// the top R.  The reads are data dependent: tight bounds stop early, loose
// ones open nearly every page.  Rounds read whole pages (first enough for R
// tokens, then twice as many each round), so the pages opened are at most
// about twice the pages the page-by-page rule would read.
//
// One workgroup of 512 threads per (request, query head).  Bounds are this
// head's own ([Quest] §1.1 eq. (2)-(3) with its query, not the group max),
// each raised by 2^-15 * sum_j |q_j| max(|m_j|, |M_j|): that covers the fp32
// rounding of the bound and of a logit (sums of at most 128 products), so a
// page whose raised bound is below tau_R holds no token whose computed logit
// could reach tau_R.  Pages are sorted by 64-bit keys (bound descending,
// index ascending) with a bitonic sort in LDS; then each round reads 512
// tokens (one per thread, logit = q . k in fp32, unscaled: the bound's
// units), keeps the tokens that beat the current R-th, and merges them into
// the sorted list of the best R by rank (keys (logit descending, token
// ascending) are unique, so ties between logits go to the lower token).
#include "qas_device.h"
#include "qas_internal.h"

namespace qas {

namespace {

constexpr int kTrThreads = 512;
constexpr int kTrWaves = kTrThreads / kWave;
constexpr int kTrMaxPages = 4096;
constexpr int kTrMaxR = 512;
constexpr int kTrBuf = kTrMaxR + kTrThreads;     // kept + new candidates of a round

// 64-bit key, ascending = value descending then index ascending
__device__ __forceinline__ uint64_t desc_key(float v, uint32_t idx) {
  return ((uint64_t)(~order_key(v)) << 32) | idx;
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t k = ~(uint32_t)(key >> 32);          // order_key of the value
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// exclusive count of `flag` over the workgroup in thread order; two barriers
__device__ __forceinline__ int tr_excl_count(bool flag, int* scratch, int* total) {
  const uint64_t mask = __ballot(flag);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
  if (lane == 0) scratch[wave] = __popcll(mask);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTrWaves; ++w) {
    const int c = scratch[w];
    before += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + in_wave;
}

// ascending bitonic sort of n (a power of two) keys in LDS
__device__ void bitonic_sort(uint64_t* s, int n) {
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kTrThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = s[i], y = s[ixj];
          if ((x > y) == ((i & k) == 0)) {
            s[i] = y;
            s[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
}

template <int DT, int D>
__global__ __launch_bounds__(kTrThreads) void topr_kernel(ToprArgs a) {
  constexpr int EPL = epl<DT>();
  constexpr int BYTES = DType<DT>::bytes;
  __shared__ uint64_t s_pages[kTrMaxPages];
  __shared__ uint64_t s_buf[2][kTrBuf];
  __shared__ float s_q[D];
  __shared__ int s_cnt[kTrWaves];

  const int qh = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int H = a.H_kv, S = a.S, h = qh / (a.H_q / a.H_kv);
  const int L = a.seq_lens[r];
  const int pbeg = a.page_indptr[r];
  const int P_r = a.page_indptr[r + 1] - pbeg;
  // the host keeps rows within kTrMaxPages; the clamp keeps LDS in bounds regardless
  const int P = L > 0 ? min(min((L + S - 1) / S, P_r), kTrMaxPages) : 0;
  const size_t orow = (size_t)r * a.H_q + qh;
  for (int d = tid; d < D; d += kTrThreads) s_q[d] = load_scalar<DT>(a.q, orow * D + d);
  __syncthreads();

  // 1. this head's bounds, raised by the rounding margin, as sort keys
  int Pp = 1;
  while (Pp < P) Pp <<= 1;
  const char* summ = reinterpret_cast<const char*>(a.summary);
  for (int p = tid; p < Pp; p += kTrThreads) {
    uint64_t key = ~0ull;
    if (p < P) {
      const size_t rec = ((size_t)a.page_indices[pbeg + p] * H + h) * 2 * D;
      float u = 0.f, mag = 0.f;
#pragma unroll 4
      for (int c = 0; c < D / EPL; ++c) {
        float m[EPL], M[EPL];
        unpack16<DT>(load16(summ + (rec + c * EPL) * BYTES), m);
        unpack16<DT>(load16(summ + (rec + D + c * EPL) * BYTES), M);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float qd = s_q[c * EPL + e];
          u += fmaxf(qd * m[e], qd * M[e]);
          mag += fabsf(qd) * fmaxf(fabsf(m[e]), fabsf(M[e]));
        }
      }
      key = desc_key(u + ldexpf(mag, -15), (uint32_t)p);
    }
    s_pages[p] = key;
  }
  __syncthreads();
  bitonic_sort(s_pages, Pp);

  // 2. rounds of kTrThreads tokens in bound order until the next bound is below tau_R
  const int R = a.R;
  // pages per round: first enough for R tokens, then doubling up to one
  // token per thread, so that tight bounds stop after few pages and loose
  // ones read 512 tokens a round (S <= 256)
  const int cp = kTrThreads / S;
  int np_round = max(1, min(cp, (R + S - 1) / S));
  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  int kept = 0, cur = 0, next = 0;
  while (next < P) {
    if (kept >= R && key_value(s_pages[next]) < key_value(s_buf[cur][R - 1])) break;
    const int np = min(np_round, P - next);
    np_round = min(cp, 2 * np_round);
    bool cand = false;
    uint64_t ck = 0;
    if (tid < np * S) {
      const int j = (int)(uint32_t)s_pages[next + tid / S];
      const int off = tid % S;
      const int t = j * S + off;
      if (t < L) {
        const size_t row = (((size_t)a.page_indices[pbeg + j] * H + h) * S + off) * D;
        float z = 0.f;
#pragma unroll 4
        for (int c = 0; c < D / EPL; ++c) {
          float k[EPL];
          unpack16<DT>(load16(kpool + (row + c * EPL) * BYTES), k);
#pragma unroll
          for (int e = 0; e < EPL; ++e) z += s_q[c * EPL + e] * k[e];
        }
        ck = desc_key(z, (uint32_t)t);
        cand = kept < R || ck < s_buf[cur][R - 1];
      }
    }
    int total;
    const int pos = tr_excl_count(cand, s_cnt, &total);
    if (cand) s_buf[cur][kept + pos] = ck;
    __syncthreads();
    if (total > 0) {
      // rank of every entry among old (sorted) + new (unsorted), unique keys
      const int n = kept + total;
      for (int i = tid; i < n; i += kTrThreads) {
        const uint64_t x = s_buf[cur][i];
        int rank = 0;
        if (i < kept) {
          rank = i;
        } else {
          int lo = 0, hi = kept;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_buf[cur][mid] < x) lo = mid + 1; else hi = mid;
          }
          rank = lo;
        }
        for (int q = kept; q < n; ++q) rank += s_buf[cur][q] < x ? 1 : 0;
        if (rank < R) s_buf[cur ^ 1][rank] = x;
      }
      kept = min(n, R);
      cur ^= 1;
      __syncthreads();
    }
    next += np;
  }

  // 3. the best R by (logit descending, token ascending), padded
  for (int i = tid; i < R; i += kTrThreads) {
    const bool ok = i < kept;
    a.top_tokens[orow * R + i] = ok ? (int)(uint32_t)s_buf[cur][i] : -1;
    a.top_logits[orow * R + i] = ok ? key_value(s_buf[cur][i]) : -INFINITY;
  }
  if (tid == 0 && a.pages_read) a.pages_read[orow] = next;
}

template <int DT, int D>
hipError_t launch_t(const ToprArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((topr_kernel<DT, D>), dim3(a.H_q, a.B), dim3(kTrThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t by_d(const ToprArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_t<DT, 16>(a, s);
    case 64: return launch_t<DT, 64>(a, s);
    case 128: return launch_t<DT, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int topr_max_pages() { return kTrMaxPages; }
int topr_max_r() { return kTrMaxR; }

hipError_t launch_topr(const ToprArgs& a, hipStream_t s) {
  switch (a.kv_dtype) {
    case kF32: return by_d<kF32>(a, s);
    case kF16: return by_d<kF16>(a, s);
    case kBF16: return by_d<kBF16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qas
