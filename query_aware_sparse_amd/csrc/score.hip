// Page-score kernel: the Quest page bound ("3.1.1 · Quest", §1.1 eq. (2)-(3))
// with the group-max aggregate for grouped-query heads (§2.1).
//
// The summaries of one request are streamed as (page, KV head) records of
// 2*d elements ([min | max]).  A record is read by RL = d*bytes/16 lanes,
// each lane holding 16 bytes of min and the matching 16 bytes of max, so a
// wave reads whole 512-byte records with 16-byte loads.  Each thread keeps
// U records in flight.  Queries live in LDS as fp32.
#include "qas_device.h"
#include "qas_internal.h"

namespace qas {

namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreUnroll = 4;

template <int DT, int D, int G>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
  constexpr int EPL = epl<DT>();
  constexpr int RL = D / EPL;                 // lanes per record half
  constexpr int RPB = kScoreThreads / RL;     // records per block iteration
  constexpr int BYTES = DType<DT>::bytes;
  extern __shared__ float q_lds[];            // [H_q][D] fp32

  const int r = blockIdx.y;
  const int H = a.H_kv;
  const int pbeg = a.page_indptr[r];
  const int P_r = a.page_indptr[r + 1] - pbeg;
  const int total = P_r * H;
  const int rec0 = blockIdx.x * a.recs_per_block;
  if (rec0 >= total) return;
  const int rec1 = min(rec0 + a.recs_per_block, total);
  const int L = a.seq_lens[r];
  const int n_used = min((L + a.S - 1) / a.S, P_r);

  const int tid = threadIdx.x;
  const int HQ = a.H_q;
  for (int i = tid; i < HQ * D; i += kScoreThreads)
    q_lds[i] = load_scalar<DT>(a.q, (size_t)r * HQ * D + i);
  __syncthreads();

  const int slot = tid / RL;
  const int c = tid % RL;
  const int* pt = a.page_indices + pbeg;
  float* srow = a.scores + (size_t)pbeg * H;
  const char* sum_base = reinterpret_cast<const char*>(a.summary);

  for (int base = rec0; base < rec1; base += RPB * kScoreUnroll) {
    uint4 mn[kScoreUnroll], mx[kScoreUnroll];
    int rec[kScoreUnroll];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      rec[u] = base + u * RPB + slot;
      mn[u] = make_uint4(0, 0, 0, 0);
      mx[u] = make_uint4(0, 0, 0, 0);
      if (rec[u] < rec1) {
        const int j = rec[u] / H, h = rec[u] - (rec[u] / H) * H;
        if (j < n_used) {
          const size_t pp = (size_t)pt[j];
          const char* p = sum_base + ((pp * H + h) * 2 * D) * BYTES + c * 16;
          mn[u] = load16(p);
          mx[u] = load16(p + D * BYTES);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const bool live = rec[u] < rec1;
      const int j = rec[u] / H, h = rec[u] - (rec[u] / H) * H;
      float m[EPL], M[EPL];
      unpack16<DT>(mn[u], m);
      unpack16<DT>(mx[u], M);
      float best = -INFINITY;
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const float* qv = q_lds + ((live ? h : 0) * G + gg) * D + c * EPL;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float qe = qv[e];
          s += qe >= 0.f ? qe * M[e] : qe * m[e];   // eq. (2)
        }
        s = group_sum<RL>(s);                       // eq. (3)
        best = fmaxf(best, s);                      // group max
      }
      if (live && c == 0) srow[(size_t)h * P_r + j] = j < n_used ? best : -INFINITY;
    }
  }
}

template <int DT, int D, int G>
hipError_t launch_t(const ScoreArgs& a, hipStream_t s) {
  const int rpb = a.recs_per_block;
  dim3 grid((a.max_pages * a.H_kv + rpb - 1) / rpb, a.B);
  size_t lds = (size_t)a.H_q * D * sizeof(float);
  hipLaunchKernelGGL((score_kernel<DT, D, G>), grid, dim3(kScoreThreads), lds, s, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t by_g(const ScoreArgs& a, hipStream_t s) {
  switch (a.g) {
    case 1: return launch_t<DT, D, 1>(a, s);
    case 2: return launch_t<DT, D, 2>(a, s);
    case 4: return launch_t<DT, D, 4>(a, s);
    case 8: return launch_t<DT, D, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t by_d(const ScoreArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return by_g<DT, 16>(a, s);
    case 64: return by_g<DT, 64>(a, s);
    case 128: return by_g<DT, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool score_supported(int kv_dtype, int d, int g) {
  return (kv_dtype == kF32 || kv_dtype == kF16 || kv_dtype == kBF16) &&
         (d == 16 || d == 64 || d == 128) && (g == 1 || g == 2 || g == 4 || g == 8);
}

int score_recs_per_block(int kv_dtype, int d, long total_recs) {
  const int e = kv_dtype == kF32 ? 4 : 8;
  const int rpb = kScoreThreads / (d / e) * kScoreUnroll;
  long want = (total_recs + 1023) / 1024;
  long n = (want + rpb - 1) / rpb;
  if (n < 1) n = 1;
  return (int)(n * rpb);
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t s) {
  switch (a.kv_dtype) {
    case kF32: return by_d<kF32>(a, s);
    case kF16: return by_d<kF16>(a, s);
    case kBF16: return by_d<kBF16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qas
