// Page-score kernel: the Quest page bound ("3.1.1 · Quest", §1.1 eq. (2)-(3))
// with the group-max aggregate for grouped-query heads (§2.1), optionally
// preceded by the decode append of the current token (§1.2 eq. (8)).
//
// Lane layout: a page's record for one KV head is 2*d elements ([min | max])
// read by RL = d*bytes/16 lanes, each holding 16 bytes of min and the
// matching 16 bytes of max.  A workgroup has H_kv * RL * PPI lanes, so every
// lane keeps one KV head and one 16-byte dim chunk for the whole kernel
// (its query slice lives in registers) and walks PPI-strided pages of the
// workgroup's page range, U pages in flight.  Dependent global loads are
// three levels deep: request bounds and queries, then the page table, then
// the summaries.
//
// Fused append: the lanes that own the request's tail page first copy the
// current token's K/V row into the pool and fold the key into the page's
// min/max (starting from +-inf when the token opens the page), then score
// the updated record.  No other workgroup reads that record, and the
// attention stage runs in a later kernel, so no synchronisation is needed.
// The first workgroup of each request also zeroes the attention kernel's
// split counters of that request.
#include "qas_device.h"
#include "qas_internal.h"

namespace qas {

namespace {

constexpr int kScoreUnroll = 4;       // pages in flight per lane

// elementwise min / max of two 16-byte chunks of stored values (exact)
template <int DT, bool IS_MAX>
__device__ __forceinline__ uint4 minmax16(const uint4& a, const uint4& b) {
  constexpr int EPL = epl<DT>();
  float fa[EPL], fb[EPL];
  unpack16<DT>(a, fa);
  unpack16<DT>(b, fb);
  typedef typename Store<DT>::T ST;
  ST out[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    out[e] = Store<DT>::from(IS_MAX ? fmaxf(fa[e], fb[e]) : fminf(fa[e], fb[e]));
  return *reinterpret_cast<const uint4*>(out);
}

template <int DT, int D, int G>
__global__ __launch_bounds__(1024) void score_kernel(ScoreArgs a) {
  constexpr int EPL = epl<DT>();
  constexpr int RL = D / EPL;                 // lanes per record half
  constexpr int BYTES = DType<DT>::bytes;

  const int r = blockIdx.y;
  const int H = a.H_kv;
  const int tid = threadIdx.x;
  const int lanes_pp = H * RL;                // lanes per page
  const int ps = tid / lanes_pp;              // page slot
  const int h = (tid / RL) % H;
  const int c = tid % RL;
  const int PPI = a.pages_per_iter;
  const int j0 = blockIdx.x * PPI * kScoreUnroll;

  // level 1: request bounds, query slices, the appended token
  const int req = r / a.gamma;                // request of the row (draft positions)
  const int pbeg = a.page_indptr[req];
  const int P_r = a.page_indptr[req + 1] - pbeg;
  const int L = a.seq_lens[req] - (a.gamma - 1 - r % a.gamma);
  float qf[G][EPL];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const uint4 qr = load16(reinterpret_cast<const char*>(a.q) +
                            (((size_t)r * a.H_q + h * G + gg) * D) * BYTES + c * 16);
    unpack16<DT>(qr, qf[gg]);
  }
  uint4 knew = make_uint4(0, 0, 0, 0), vnew = make_uint4(0, 0, 0, 0);
  const bool appending = a.k_new != nullptr && L > 0;
  if (appending) {
    const size_t o = (((size_t)r * H + h) * D) * BYTES + c * 16;
    knew = load16(reinterpret_cast<const char*>(a.k_new) + o);
    vnew = load16(reinterpret_cast<const char*>(a.v_new) + o);
  }
  if (a.tickets && blockIdx.x == 0)
    for (int i = tid; i < H; i += blockDim.x) a.tickets[(size_t)r * H + i] = 0u;
  if (j0 >= P_r) return;
  const int n_used = L > 0 ? min((L + a.S - 1) / a.S, P_r) : 0;
  const int tail = n_used - 1;

  // level 2: page table.  Indices past the used pages are clamped to a page
  // of the request (j0 < P_r, so there is one) and their results dropped:
  // every load is unconditional, so each level's loads are all in flight at
  // once (a load under a branch makes the compiler wait for all earlier
  // loads before issuing it).
  const int jlast = max(n_used, 1) - 1;
  int j[kScoreUnroll];
  int pp[kScoreUnroll];
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    j[u] = j0 + ps + u * PPI;
    pp[u] = a.page_indices[pbeg + min(j[u], jlast)];
  }
  // level 3: summaries (a page the append opens is overwritten below)
  const char* sum_base = reinterpret_cast<const char*>(a.summary);
  uint4 mn[kScoreUnroll], mx[kScoreUnroll];
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    const char* p = sum_base + (((size_t)pp[u] * H + h) * 2 * D) * BYTES + c * 16;
    mn[u] = load16(p);
    mx[u] = load16(p + D * BYTES);
  }
  if (appending) {
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      if (j[u] != tail) continue;
      const int off = (L - 1) % a.S;
      if (off == 0) {          // the token opens the page: -inf/+inf start
        mn[u] = knew;
        mx[u] = knew;
      } else {
        mn[u] = minmax16<DT, false>(mn[u], knew);
        mx[u] = minmax16<DT, true>(mx[u], knew);
      }
      char* p = reinterpret_cast<char*>(a.summary) + (((size_t)pp[u] * H + h) * 2 * D) * BYTES +
                c * 16;
      *reinterpret_cast<uint4*>(p) = mn[u];
      *reinterpret_cast<uint4*>(p + D * BYTES) = mx[u];
      const size_t row = ((((size_t)pp[u] * H + h) * a.S + off) * D) * BYTES + c * 16;
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.k_pool) + row) = knew;
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.v_pool) + row) = vnew;
    }
  }

  float* srow = a.row_stride ? a.scores + ((size_t)r * H + h) * a.row_stride
                             : a.scores + (size_t)pbeg * H + (size_t)h * P_r;
  const int lim = a.row_stride ? min(P_r, a.row_stride) : P_r;   // stay inside the row
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    float m[EPL], M[EPL];
    unpack16<DT>(mn[u], m);
    unpack16<DT>(mx[u], M);
    float best = -INFINITY;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float qe = qf[gg][e];
        s += qe >= 0.f ? qe * M[e] : qe * m[e];   // eq. (2)
      }
      s = group_sum<RL>(s);                       // eq. (3)
      best = fmaxf(best, s);                      // group max
    }
    if (c == 0 && j[u] < lim) srow[j[u]] = j[u] < n_used ? best : -INFINITY;
    if (a.phys_out && h == 0 && c == 0 && j[u] < lim)
      a.phys_out[(size_t)r * a.row_stride + j[u]] = pp[u];
  }
}

// four e4m3 codes of a word -> their values (exact)
__device__ __forceinline__ void unpack_e4m3x4(uint32_t w, float* out) {
  out[0] = __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
  out[1] = __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
  out[2] = __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
  out[3] = __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
}

// Page scores from the e4m3 summary copy (the Quest page, §3 on the summary
// dtype; outward-rounded, so the bound stays above every dot product of the
// page).  A record half is d one-byte codes: RL8 = d/16 lanes, each holding
// 16 codes of min and 16 of max and the matching 16 dims of each query head;
// U = s * sum_d max(q_d m_d, q_d M_d) over the codes' values, s the record's
// power-of-two scale (exact).  The fused append updates the tail page's
// exact record, then re-quantises the copy from it (same rule as the append
// kernel) and scores the new copy.
template <int DT, int D, int G>
__global__ __launch_bounds__(512) void score8_kernel(ScoreArgs a) {
  constexpr int RL8 = D / 16;                 // lanes per record half
  constexpr int BYTES = DType<DT>::bytes;

  const int r = blockIdx.y;
  const int H = a.H_kv;
  const int tid = threadIdx.x;
  const int lanes_pp = H * RL8;
  const int ps = tid / lanes_pp;
  const int h = (tid / RL8) % H;
  const int c = tid % RL8;
  const int PPI = a.pages_per_iter;
  const int j0 = blockIdx.x * PPI * kScoreUnroll;
  const int d0 = c * 16;                      // this lane's 16 dims

  // level 1: request bounds, query slices, the appended token
  const int req = r / a.gamma;                // request of the row (draft positions)
  const int pbeg = a.page_indptr[req];
  const int P_r = a.page_indptr[req + 1] - pbeg;
  const int L = a.seq_lens[req] - (a.gamma - 1 - r % a.gamma);
  constexpr int EPL = epl<DT>();
  float qf[G][16];
#pragma unroll
  for (int gg = 0; gg < G; ++gg)
#pragma unroll
    for (int v = 0; v < 16 / EPL; ++v)
      unpack16<DT>(load16(reinterpret_cast<const char*>(a.q) +
                          (((size_t)r * a.H_q + h * G + gg) * D + d0 + v * EPL) * BYTES),
                   qf[gg] + v * EPL);
  // the appended token's 16 dims of K and V, as 16-byte words
  constexpr int NV = 16 / EPL;
  const bool appending = a.k_new != nullptr && L > 0;
  uint4 kw[NV], vw[NV];
  if (appending) {
    const size_t o = (((size_t)r * H + h) * D + d0) * BYTES;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      kw[v] = load16(reinterpret_cast<const char*>(a.k_new) + o + v * 16);
      vw[v] = load16(reinterpret_cast<const char*>(a.v_new) + o + v * 16);
    }
  }
  if (a.tickets && blockIdx.x == 0)
    for (int i = tid; i < H; i += blockDim.x) a.tickets[(size_t)r * H + i] = 0u;
  if (j0 >= P_r) return;
  const int n_used = L > 0 ? min((L + a.S - 1) / a.S, P_r) : 0;
  const int tail = n_used - 1;

  // level 2: page table, clamped as in score_kernel so that every load is
  // unconditional and each level is in flight at once
  const int jlast = max(n_used, 1) - 1;
  int j[kScoreUnroll];
  int pp[kScoreUnroll];
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    j[u] = j0 + ps + u * PPI;
    pp[u] = a.page_indices[pbeg + min(j[u], jlast)];
  }
  // which of this lane's pages is the tail the token goes to (-1: none)
  int ut = -1, pt = 0;
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u)
    if (j[u] == tail) {
      ut = u;
      pt = pp[u];
    }
  const bool owns_tail = appending && ut >= 0;
  const int off = appending ? (L - 1) % a.S : 0;

  // level 3: summary codes and scales; then, on the lanes of the tail page
  // only and issued last, its exact record
  const unsigned char* codes = reinterpret_cast<const unsigned char*>(a.summary_fp8);
  uint4 mn[kScoreUnroll], mx[kScoreUnroll];
  float sc[kScoreUnroll];
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    const size_t rec = (size_t)pp[u] * H + h;
    mn[u] = load16(codes + rec * 2 * D + d0);
    mx[u] = load16(codes + rec * 2 * D + D + d0);
    sc[u] = a.summary_fp8_scale[rec];
  }
  const size_t rec_t = (size_t)pt * H + h;
  char* sum_t = reinterpret_cast<char*>(a.summary) + (rec_t * 2 * D + d0) * BYTES;
  uint4 smn[NV], smx[NV];
  if (owns_tail && off != 0) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      smn[v] = load16(sum_t + v * 16);
      smx[v] = load16(sum_t + D * BYTES + v * 16);
    }
  }
  if (owns_tail) {
    // exact record: min/max with the token (the token alone when it opens
    // the page: the -inf/+inf start), then the token's K/V rows
    const size_t row = ((((size_t)pt * H + h) * a.S + off) * D + d0) * BYTES;
    float m[16], M[16], amax = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      smn[v] = off == 0 ? kw[v] : minmax16<DT, false>(smn[v], kw[v]);
      smx[v] = off == 0 ? kw[v] : minmax16<DT, true>(smx[v], kw[v]);
      *reinterpret_cast<uint4*>(sum_t + v * 16) = smn[v];
      *reinterpret_cast<uint4*>(sum_t + D * BYTES + v * 16) = smx[v];
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.k_pool) + row + v * 16) = kw[v];
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.v_pool) + row + v * 16) = vw[v];
      unpack16<DT>(smn[v], m + v * EPL);
      unpack16<DT>(smx[v], M + v * EPL);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fmaxf(fabsf(m[e]), fabsf(M[e])));
    // re-quantise the copy (same rule as the append kernel), then score it
    amax = group_max<RL8>(amax);
    const int k = summary_scale_exponent(amax);
    uint32_t wm[4] = {0, 0, 0, 0}, wM[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      wm[e / 4] |= e4m3_down(ldexpf(m[e], -k)) << (8 * (e % 4));
      wM[e / 4] |= e4m3_up(ldexpf(M[e], -k)) << (8 * (e % 4));
    }
    const uint4 cm = make_uint4(wm[0], wm[1], wm[2], wm[3]);
    const uint4 cM = make_uint4(wM[0], wM[1], wM[2], wM[3]);
    const float sk = ldexpf(1.f, k);
    unsigned char* cw = reinterpret_cast<unsigned char*>(a.summary_fp8);
    *reinterpret_cast<uint4*>(cw + rec_t * 2 * D + d0) = cm;
    *reinterpret_cast<uint4*>(cw + rec_t * 2 * D + D + d0) = cM;
    if (c == 0) a.summary_fp8_scale[rec_t] = sk;
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u)
      if (u == ut) {
        mn[u] = cm;
        mx[u] = cM;
        sc[u] = sk;
      }
  }

  float* srow = a.row_stride ? a.scores + ((size_t)r * H + h) * a.row_stride
                             : a.scores + (size_t)pbeg * H + (size_t)h * P_r;
  const int lim = a.row_stride ? min(P_r, a.row_stride) : P_r;   // stay inside the row
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    const uint32_t wm[4] = {mn[u].x, mn[u].y, mn[u].z, mn[u].w};
    const uint32_t wM[4] = {mx[u].x, mx[u].y, mx[u].z, mx[u].w};
    float m[16], M[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      unpack_e4m3x4(wm[i], m + 4 * i);
      unpack_e4m3x4(wM[i], M + 4 * i);
    }
    float best = -INFINITY;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float qe = qf[gg][e];
        s += qe >= 0.f ? qe * M[e] : qe * m[e];   // eq. (2) on the codes' values
      }
      s = group_sum<RL8>(s) * sc[u];              // eq. (3), times the exact scale
      best = fmaxf(best, s);
    }
    if (c == 0 && j[u] < lim) srow[j[u]] = j[u] < n_used ? best : -INFINITY;
    if (a.phys_out && h == 0 && c == 0 && j[u] < lim)
      a.phys_out[(size_t)r * a.row_stride + j[u]] = pp[u];
  }
}

template <int DT, int D, int G>
hipError_t launch_t(const ScoreArgs& a, hipStream_t s) {
  if (a.summary_fp8) {
    const int lanes_pp = a.H_kv * (D / 16);
    const int threads = lanes_pp * a.pages_per_iter;
    const int ppb = a.pages_per_iter * kScoreUnroll;
    dim3 grid((a.max_pages + ppb - 1) / ppb, a.B);
    hipLaunchKernelGGL((score8_kernel<DT, D, G>), grid, dim3(threads), 0, s, a);
    return hipGetLastError();
  }
  constexpr int RL = D / epl<DT>();
  const int lanes_pp = a.H_kv * RL;
  const int threads = lanes_pp * a.pages_per_iter;
  const int ppb = a.pages_per_iter * kScoreUnroll;
  dim3 grid((a.max_pages + ppb - 1) / ppb, a.B);
  hipLaunchKernelGGL((score_kernel<DT, D, G>), grid, dim3(threads), 0, s, a);
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

bool score_supported(int kv_dtype, int d, int g, int H_kv) {
  if (!(kv_dtype == kF32 || kv_dtype == kF16 || kv_dtype == kBF16)) return false;
  if (!(d == 16 || d == 64 || d == 128)) return false;
  if (!(g == 1 || g == 2 || g == 4 || g == 8)) return false;
  const int rl = d * (kv_dtype == kF32 ? 4 : 2) / 16;
  return H_kv * rl <= 1024;
}

int score8_pages_per_iter(int d, int H_kv) {
  const int lanes_pp = H_kv * (d / 16);
  int ppi = 512 / lanes_pp;
  return ppi < 1 ? 1 : ppi;
}

bool score8_supported(int d, int H_kv) { return H_kv * (d / 16) <= 512; }

int score_pages_per_iter(int kv_dtype, int d, int H_kv) {
  const int rl = d * (kv_dtype == kF32 ? 4 : 2) / 16;
  const int lanes_pp = H_kv * rl;
  int ppi = 512 / lanes_pp;
  return ppi < 1 ? 1 : ppi;
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
