// Summary append: write new tokens' K/V rows into the paged pool and keep the
// per-page key min/max summaries current ("3.1.1 · Quest", §1.2 eq. (8) and
// §3 eq. (14)); a page whose first token is written starts from
// max = -inf / min = +inf, so a recycled physical page never keeps stale
// extremes (§3, page recycling).
//
// With an fp8 summary copy (the Quest page, §3 on the summary dtype), each
// written record is also stored as e4m3 codes with one power-of-two scale per
// (page, KV head): the smallest 2^k with max |m|, |M| <= 448 * 2^k, the min
// rounded toward -inf and the max toward +inf, so the copy stays an outer
// interval of the exact record.
//
// One workgroup per (page touched, KV head, request).  Lanes own 16-byte
// chunks of a token row (RL lanes per row, TS rows in flight), copy K and V
// into the pool, reduce min/max over their tokens, then the workgroup
// reduces over token slots in LDS and writes the page's record.  The same
// kernel serves prefill (many tokens per request) and decode (one token).
//
// Rescan mode (rollback, the Quest page's §3 on the cache lifecycle): after
// the cache is cut back, a cut inside a page cannot be undone on the min/max
// (a revoked token may hold an extreme), so the tail page's record is rebuilt
// from the surviving keys in the pool, starting from -inf/+inf, and its e4m3
// copy re-quantised; nothing is written to the pool.
#include "qas_device.h"
#include "qas_internal.h"

namespace qas {

namespace {

constexpr int kAppendThreads = 256;

template <int DT, int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  constexpr int EPL = epl<DT>();
  constexpr int RL = D / EPL;                 // lanes per token row
  constexpr int TS = kAppendThreads / RL;     // token slots
  constexpr int BYTES = DType<DT>::bytes;
  __shared__ float red_min[TS][D];
  __shared__ float red_max[TS][D];
  __shared__ float red_amax[D];

  const int u = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int H = a.H_kv, S = a.S;
  int L0, n, src0;
  if (a.rescan) {            // tokens [p*S, L) of the tail page p, from the pool
    const int L = a.seq_lens[r];
    const int P_r = a.page_indptr[r + 1] - a.page_indptr[r];
    if (u != 0 || L <= 0 || L % S == 0 || (L - 1) / S >= P_r) return;
    L0 = (L - 1) / S * S;
    n = L - L0;
    src0 = 0;
  } else if (a.new_indptr) {
    L0 = a.seq_lens[r];
    src0 = a.new_indptr[r];
    n = a.new_indptr[r + 1] - src0;
  } else {  // decode: the current token sits at position seq_lens[r] - 1
    L0 = a.seq_lens[r] - 1;
    src0 = r;
    n = 1;
  }
  if (n <= 0 || L0 < 0) return;
  const int p = L0 / S + u;                   // logical page touched
  if (p > (L0 + n - 1) / S) return;
  const int t0 = max(L0, p * S);
  const int t1 = min(L0 + n, (p + 1) * S);
  const size_t phys = (size_t)a.page_indices[a.page_indptr[r] + p];

  const int tid = threadIdx.x;
  const int slot = tid / RL, c = tid % RL;
  float mn[EPL], mx[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    mn[e] = INFINITY;
    mx[e] = -INFINITY;
  }
  const char* ksrc = reinterpret_cast<const char*>(a.k_new);
  const char* vsrc = reinterpret_cast<const char*>(a.v_new);
  char* kdst = reinterpret_cast<char*>(a.k_pool);
  char* vdst = reinterpret_cast<char*>(a.v_pool);
  for (int t = t0 + slot; t < t1; t += TS) {
    const size_t dst = (((phys * H + h) * S + (t - p * S)) * D) * BYTES + c * 16;
    uint4 kr;
    if (a.rescan) {
      kr = load16(kdst + dst);
    } else {
      const size_t src = (((size_t)(src0 + t - L0) * H + h) * D) * BYTES + c * 16;
      kr = load16(ksrc + src);
      const uint4 vr = load16(vsrc + src);
      *reinterpret_cast<uint4*>(kdst + dst) = kr;
      *reinterpret_cast<uint4*>(vdst + dst) = vr;
    }
    float kf[EPL];
    unpack16<DT>(kr, kf);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {              // eq. (8)
      mn[e] = fminf(mn[e], kf[e]);
      mx[e] = fmaxf(mx[e], kf[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    red_min[slot][c * EPL + e] = mn[e];
    red_max[slot][c * EPL + e] = mx[e];
  }
  __syncthreads();
  typedef typename Store<DT>::T ST;
  ST* sum = reinterpret_cast<ST*>(a.summary) + (phys * H + h) * 2 * D;
  const bool fresh = t0 == p * S;   // the page's offset-0 token is new
  for (int dim = tid; dim < D; dim += kAppendThreads) {
    float m = INFINITY, M = -INFINITY;
    const int slots = min(TS, t1 - t0);
    for (int s = 0; s < slots; ++s) {
      m = fminf(m, red_min[s][dim]);
      M = fmaxf(M, red_max[s][dim]);
    }
    if (!fresh) {
      m = fminf(m, load_scalar<DT>(sum, dim));
      M = fmaxf(M, load_scalar<DT>(sum, D + dim));
    }
    sum[dim] = Store<DT>::from(m);
    sum[D + dim] = Store<DT>::from(M);
    red_amax[dim] = fmaxf(fabsf(m), fabsf(M));
    red_min[0][dim] = m;            // this thread's own column: no other reader
    red_max[0][dim] = M;
  }
  if (a.summary_fp8 == nullptr) return;
  __syncthreads();
  float amax = 0.f;
  for (int j = 0; j < D; ++j) amax = fmaxf(amax, red_amax[j]);
  const int k = summary_scale_exponent(amax);
  unsigned char* codes = reinterpret_cast<unsigned char*>(a.summary_fp8) + (phys * H + h) * 2 * D;
  for (int dim = tid; dim < D; dim += kAppendThreads) {
    codes[dim] = (unsigned char)e4m3_down(ldexpf(red_min[0][dim], -k));
    codes[D + dim] = (unsigned char)e4m3_up(ldexpf(red_max[0][dim], -k));
  }
  if (tid == 0) a.summary_fp8_scale[phys * H + h] = ldexpf(1.f, k);
}

template <int DT, int D>
hipError_t launch_t(const AppendArgs& a, hipStream_t s) {
  const int pages = a.new_indptr && !a.rescan ? (a.max_new + a.S - 1) / a.S + 1 : 1;
  dim3 grid(pages, a.H_kv, a.B);
  hipLaunchKernelGGL((append_kernel<DT, D>), grid, dim3(kAppendThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t by_d(const AppendArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_t<DT, 16>(a, s);
    case 64: return launch_t<DT, 64>(a, s);
    case 128: return launch_t<DT, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool append_supported(int kv_dtype, int d) {
  return (kv_dtype == kF32 || kv_dtype == kF16 || kv_dtype == kBF16) &&
         (d == 16 || d == 64 || d == 128);
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  switch (a.kv_dtype) {
    case kF32: return by_d<kF32>(a, s);
    case kF16: return by_d<kF16>(a, s);
    case kBF16: return by_d<kBF16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qas
