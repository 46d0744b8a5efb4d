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
//
// Grouped-query heads (g >= 2) with d = 128 and 16-bit records take
// score_mfma_kernel instead: the same bound as a small GEMM on matrix cores.
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

// ---- grouped-query heads on matrix cores ----------------------------------
// With G query heads per KV head the bound is a small GEMM.  Writing
// max(q m, q M) = min(q, 0) m + max(q, 0) M (exact: one of the two products
// is a product with zero), U_i = sum_k A[i][k] B[k][j] with A the sign-split
// query rows [min(q_i, 0) | max(q_i, 0)] (16 x 256, rows i >= G zero) and B
// the stored records [min | max] of 16 pages (256 x 16): eight
// v_mfma_f32_16x16x32 steps per 16 pages, the products exact and summed in
// fp32, as the VALU kernel does.  The group max is then a max over the G
// output rows of each page column.
//
// Operand lanes (16x16x32 layout: A lane l holds row l % 16, k = 8 (l / 16)
// + [0, 8) of the step; B lane l holds those k of column l % 16): k step s
// covers bytes [64 s + 16 (l / 16), +16) of a page's record, so lane l takes
// record element 32 s + 8 (l / 16) + e - a min for s < 4, the max of dim
// 32 (s - 4) + 8 (l / 16) + e for s >= 4 - and the query row's matching
// dims.  Loaded that way, every 16 consecutive lanes would touch 16 records;
// instead each load instruction reads two whole records (lane l: record
// 2 s + l / 32, bytes 16 (l % 32) + [0, 16)), and the wave turns them into
// the operand layout through a private LDS tile (records 33 16-byte units
// apart, so both the writes and the operand reads are free of bank
// conflicts).  A task is 16 consecutive pages of one KV head; a workgroup
// of 4 waves owns ng * 16 pages of one row, every KV head of them, and each
// wave keeps T = 2 tasks' records (8 KiB each) in flight.  Small workgroups
// with two tasks per wave measured faster than 8 waves or 4 tasks per wave
// (more workgroups resident per CU, shorter tails).  Tasks go round-robin
// over the waves with the head varying fastest, so the waves read
// neighbouring heads of the same pages (one page's heads are contiguous)
// and, when H_kv divides the wave count, every task of a wave has one head
// whose query operands are loaded once.
constexpr int kMfmaWaves = 4;
constexpr int kMfmaTasks = 2;          // tasks in flight per wave
constexpr int kMfmaD = 128;
constexpr int kMfmaUnits = 33;         // LDS record stride in 16-byte units

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <int DT>
__device__ __forceinline__ float4_t mfma_16x16x32(const uint4& a, const uint4& b,
                                                  const float4_t& c) {
  if constexpr (DT == kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Sign split of eight 16-bit floats: neg keeps the elements whose sign bit
// is set (min(x, 0), up to the sign of zero), pos the others (max(x, 0)).
__device__ __forceinline__ void sign_split(const uint4& x, uint4& neg, uint4& pos) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t n[4], p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = ((w[i] >> 15) & 0x00010001u) * 0xFFFFu;
    n[i] = w[i] & m;
    p[i] = w[i] & ~m;
  }
  neg = make_uint4(n[0], n[1], n[2], n[3]);
  pos = make_uint4(p[0], p[1], p[2], p[3]);
}

// This lane's query row (lane % 16; row 0 when it is not one of the G rows,
// zeroed by split_a) of KV head h: dims 32 s + 8 (lane / 16) + [0, 8) in
// raw[s], s < 4.
template <int G>
__device__ __forceinline__ void load_q_rows(const ScoreArgs& a, int r, int h, int col, int quad,
                                            uint4* raw) {
  const int i = col < G ? col : 0;
  const char* q = reinterpret_cast<const char*>(a.q) +
                  (((size_t)r * a.H_q + h * G + i) * kMfmaD) * 2 + quad * 16;
#pragma unroll
  for (int s = 0; s < 4; ++s) raw[s] = load16(q + s * 64);
}

// A operands of the 8 k steps from load_q_rows' registers, split by sign.
template <int G>
__device__ __forceinline__ void split_a(const uint4* raw, int col, uint4* A) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    sign_split(col < G ? raw[s] : make_uint4(0, 0, 0, 0), A[s], A[s + 4]);
}

template <int DT, int G, bool ONE_HEAD>
__global__ __launch_bounds__(kMfmaWaves * kWave) void score_mfma_kernel(ScoreArgs a, int ng) {
  constexpr int D = kMfmaD;
  constexpr int T = kMfmaTasks;
  constexpr int BYTES = 2;
  static_assert(DType<DT>::bytes == BYTES, "16-bit records");
  __shared__ uint4 tile[kMfmaWaves][16 * kMfmaUnits];

  const int r = blockIdx.y;
  const int H = a.H_kv;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int col = lane & 15, quad = lane >> 4;
  const int half = lane >> 5, unit = lane & 31;   // load layout: record 2 s + half
  const int ntasks = H * ng;
  const int j0 = blockIdx.x * 16 * ng;

  const int req = r / a.gamma;                // request of the row (draft positions)
  const int pbeg = a.page_indptr[req];
  const int P_r = a.page_indptr[req + 1] - pbeg;
  const int L = a.seq_lens[req] - (a.gamma - 1 - r % a.gamma);
  if (a.tickets && blockIdx.x == 0)
    for (int i = threadIdx.x; i < H; i += blockDim.x) a.tickets[(size_t)r * H + i] = 0u;
  if (j0 >= P_r) return;
  const int n_used = L > 0 ? min((L + a.S - 1) / a.S, P_r) : 0;
  const int tail = n_used - 1;
  const int jlast = max(n_used, 1) - 1;
  const bool appending = a.k_new != nullptr && L > 0;
  const int off = appending ? (L - 1) % a.S : 0;
  const int lim = a.row_stride ? min(P_r, a.row_stride) : P_r;   // stay inside the row
  const char* sum_base = reinterpret_cast<const char*>(a.summary);
  uint4* my = tile[w];

  uint4 A1[8];
  if constexpr (ONE_HEAD) {
    uint4 q1[4];
    load_q_rows<G>(a, r, w % H, col, quad, q1);
    split_a<G>(q1, col, A1);
  }

  for (int t0 = w; t0 < ntasks; t0 += kMfmaWaves * T) {
    // page table, then records: every load unconditional (tasks past the
    // end repeat the last one, pages past the used ones are clamped to a
    // page of the request, and their results are dropped)
    int hh[T], jj[T], pp[T];
    uint4 qr[T][4];                           // query rows when the head varies
#pragma unroll
    for (int u = 0; u < T; ++u) {
      const int t = min(t0 + u * kMfmaWaves, ntasks - 1);
      hh[u] = t % H;
      jj[u] = j0 + 16 * (t / H) + col;
      if constexpr (!ONE_HEAD) load_q_rows<G>(a, r, hh[u], col, quad, qr[u]);
      pp[u] = a.page_indices[pbeg + min(jj[u], jlast)];
    }
    // every task's page-table and query loads are issued before the first
    // wait (the records' addresses need the page indices of other lanes)
    __builtin_amdgcn_sched_barrier(0);
    uint4 raw[T][8];
#pragma unroll
    for (int u = 0; u < T; ++u)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int pj = __shfl(pp[u], 2 * s + half, kWave);   // lane j < 16 holds page j
        raw[u][s] = load16(sum_base + (((size_t)pj * H + hh[u]) * 2 * D) * BYTES + unit * 16);
      }
#pragma unroll
    for (int u = 0; u < T; ++u) {
      // transpose through the wave's LDS tile into the operand layout
      uint4 b[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) my[(2 * s + half) * kMfmaUnits + unit] = raw[u][s];
#pragma unroll
      for (int s = 0; s < 8; ++s) b[s] = my[col * kMfmaUnits + 4 * s + quad];
      const bool valid = t0 + u * kMfmaWaves < ntasks;
      // fused append on the tail page's four lanes: K/V row, then min/max
      // (the token alone when it opens the page: the -inf/+inf start)
      if (appending && valid && jj[u] == tail) {
        const int h = hh[u];
        const size_t o = (((size_t)r * H + h) * D) * BYTES + quad * 16;
        const char* kn = reinterpret_cast<const char*>(a.k_new) + o;
        const char* vn = reinterpret_cast<const char*>(a.v_new) + o;
        char* sum = reinterpret_cast<char*>(a.summary) +
                    (((size_t)pp[u] * H + h) * 2 * D) * BYTES + quad * 16;
        const size_t row = ((((size_t)pp[u] * H + h) * a.S + off) * D) * BYTES + quad * 16;
        char* kr = reinterpret_cast<char*>(a.k_pool) + row;
        char* vr = reinterpret_cast<char*>(a.v_pool) + row;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 kw = load16(kn + s * 64), vw = load16(vn + s * 64);
          b[s] = off == 0 ? kw : minmax16<DT, false>(b[s], kw);
          b[s + 4] = off == 0 ? kw : minmax16<DT, true>(b[s + 4], kw);
          *reinterpret_cast<uint4*>(sum + s * 64) = b[s];
          *reinterpret_cast<uint4*>(sum + D * BYTES + s * 64) = b[s + 4];
          *reinterpret_cast<uint4*>(kr + s * 64) = kw;
          *reinterpret_cast<uint4*>(vr + s * 64) = vw;
        }
      }
      uint4 At[8];
      if constexpr (!ONE_HEAD) split_a<G>(qr[u], col, At);
      const uint4* A = ONE_HEAD ? A1 : At;
      float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s) acc = mfma_16x16x32<DT>(A[s], b[s], acc);
      // lane l holds rows 4 (l / 16) + [0, 4) of page column l % 16
      float best = acc[0];
#pragma unroll
      for (int i = 1; i < (G < 4 ? G : 4); ++i) best = fmaxf(best, acc[i]);
      if constexpr (G == 8) best = fmaxf(best, __shfl_xor(best, 16, kWave));
      const int j = jj[u];
      if (quad == 0 && valid && j < lim) {
        float* srow = a.row_stride ? a.scores + ((size_t)r * H + hh[u]) * a.row_stride
                                   : a.scores + (size_t)pbeg * H + (size_t)hh[u] * P_r;
        srow[j] = j < n_used ? best : -INFINITY;
        if (a.phys_out && hh[u] == 0) a.phys_out[(size_t)r * a.row_stride + j] = pp[u];
      }
    }
  }
}

template <int DT, int D, int G>
hipError_t launch_t(const ScoreArgs& a, hipStream_t s) {
  if constexpr (D == kMfmaD && G >= 2 && DT != kF32) {
    if (!a.summary_fp8) {
      const int per = kMfmaWaves * kMfmaTasks;          // tasks of one pass of the waves
      const int ng = a.H_kv >= per ? 1 : per / a.H_kv;  // 16-page groups per workgroup
      dim3 grid((a.max_pages + 16 * ng - 1) / (16 * ng), a.B);
      if (kMfmaWaves % a.H_kv == 0)
        hipLaunchKernelGGL((score_mfma_kernel<DT, G, true>), grid, dim3(kMfmaWaves * kWave), 0, s,
                           a, ng);
      else
        hipLaunchKernelGGL((score_mfma_kernel<DT, G, false>), grid, dim3(kMfmaWaves * kWave), 0,
                           s, a, ng);
      return hipGetLastError();
    }
  }
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
