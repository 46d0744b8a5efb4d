// Exact token top-R by branch-and-bound over the page bounds ("3.1.1 ·
// Quest", §3.2 on stopping rules beyond a fixed top-K): pages are read in
// descending bound order (ties to the lower page index), the R-th largest
// true logit read so far is tau_R, and the search stops when the next page's
// bound is below tau_R, since no token of the remaining pages can then enter
// the top R.  The reads are data dependent: tight bounds stop early, loose
// ones open nearly every page.  Rounds read whole pages (first enough for R
// tokens, then twice as many each round), so a search that stops in the
// pilot opens at most about twice the pages the page-by-page rule would
// read; one that does not reads the remaining candidate pages in parallel.
//
// Four launches: page bounds for every (request, query head); the pilot,
// one 512-thread workgroup per (request, query head); the scan of the pages
// the pilot leaves, one workgroup per 512 tokens; the merge of the lists.
// Bounds are the head's own ([Quest] §1.1 eq. (2)-(3) with its query, not
// the group max), each raised by 2^-15 * sum_j |q_j| max(|m_j|, |M_j|):
// that covers the fp32 rounding of the bound and of a logit (sums of at
// most 128 products, in any order), so a page whose raised bound is below
// tau_R holds no token whose computed logit could reach tau_R.  Pages and
// tokens are ordered by 64-bit keys: (bound descending, page ascending) and
// (logit q . k in fp32, unscaled: the bound's units, descending; token
// ascending).  Keys are unique, so ties between logits go to the lower
// token.
#include "qas_device.h"
#include "qas_internal.h"
#include "topk_block.h"

namespace qas {

namespace {

constexpr int kTrThreads = 512;
constexpr int kTrWaves = kTrThreads / kWave;
constexpr int kTrMaxPages = 4096;
constexpr int kTrMaxR = 512;
constexpr int kTrBuf = kTrMaxR + kTrThreads;     // kept + new candidates of a round
constexpr int kTrMaxPilot = 64;                  // most pages of the pilot
constexpr int kTrBail = 4;                       // pilot rounds worth of pages before the scan

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

// Keys of s[lo, hi) below x, for an LDS array s that is 16-byte aligned;
// every lane reads the same words.  Two keys per 16-byte read and eight
// reads in flight, so the count does not wait one LDS round trip per key.
__device__ __forceinline__ int count_below(const uint64_t* s, int lo, int hi, uint64_t x) {
  int c = 0;
  if ((lo & 1) && lo < hi) {
    c += s[lo] < x ? 1 : 0;
    ++lo;
  }
  const ulonglong2* p = reinterpret_cast<const ulonglong2*>(s + lo);
  const int pairs = (hi - lo) >> 1;
  int i = 0;
  for (; i + 8 <= pairs; i += 8) {
    ulonglong2 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = p[i + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) c += (w[u].x < x ? 1 : 0) + (w[u].y < x ? 1 : 0);
  }
  for (; i < pairs; ++i) {
    const ulonglong2 w = p[i];
    c += (w.x < x ? 1 : 0) + (w.y < x ? 1 : 0);
  }
  if (lo < hi && ((hi - lo) & 1)) c += s[hi - 1] < x ? 1 : 0;
  return c;
}

// Rank merge of the sorted best `kept` keys of buf[cur] with `total` unsorted
// keys appended after them (keys unique); the best min(kept + total, R) go
// to buf[cur ^ 1] in order.  Every thread calls it; ends with a barrier.
__device__ void rank_merge(uint64_t (*buf)[kTrBuf], int& cur, int& kept, int total, int R) {
  const int n = kept + total;
  for (int i = threadIdx.x; i < n; i += kTrThreads) {
    const uint64_t x = buf[cur][i];
    int rank = 0;
    if (i < kept) {
      rank = i;
    } else {
      int lo = 0, hi = kept;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (buf[cur][mid] < x) lo = mid + 1; else hi = mid;
      }
      rank = lo;
    }
    rank += count_below(buf[cur], kept, n, x);
    if (rank < R) buf[cur ^ 1][rank] = x;
  }
  kept = min(n, R);
  cur ^= 1;
  __syncthreads();
}

// Logits q . k (fp32, unscaled: the bound's units) of the nt = np * S
// tokens of np pages, token u being row u % S of physical page pp[u / S],
// into z[u] (LDS).  RL = D / EPL lanes share a row, each loading 16 bytes
// of it with the matching slice qf of the query, and a DPP sum joins them:
// one wave load covers 64 / RL whole rows.  Rows of the tail page past the
// sequence are read too (they lie inside the page) and left to the caller
// to drop.  Ends without a barrier.
template <int DT, int D>
__device__ __forceinline__ void page_logits(const ToprArgs& a, const float* qf, int h,
                                            const int* pp, int np, float* z) {
  constexpr int EPL = epl<DT>();
  constexpr int RL = D / EPL;
  constexpr int TPP = kTrThreads / RL;                 // rows per pass of the workgroup
  constexpr int UNR = 8;                               // passes in flight
  constexpr int BYTES = DType<DT>::bytes;
  const int ls = __ffs(a.S) - 1;                       // S is a power of two
  const int nt = np << ls, g = threadIdx.x / RL, c = threadIdx.x % RL;
  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  for (int b = 0; b < nt; b += TPP * UNR) {
    uint4 raw[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = min(b + u * TPP + g, nt - 1);
      const size_t row = (((size_t)pp[t >> ls] * a.H_kv + h) << ls) + (t & (a.S - 1));
      raw[u] = load16(kpool + (row * D + c * EPL) * BYTES);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float k[EPL];
      unpack16<DT>(raw[u], k);
      float v = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) v += qf[e] * k[e];
      v = group_sum<RL>(v);
      const int t = b + u * TPP + g;
      if (c == 0 && t < nt) z[t] = v;
    }
  }
}

// This lane's slice of the row's query head for page_logits; returns P (pages of the row)
template <int DT, int D>
__device__ __forceinline__ int row_setup(const ToprArgs& a, float* qf, int r, int qh, int& L,
                                         int& pbeg) {
  constexpr int EPL = epl<DT>();
  constexpr int RL = D / EPL;
  L = a.seq_lens[r];
  pbeg = a.page_indptr[r];
  const int P_r = a.page_indptr[r + 1] - pbeg;
  const size_t orow = (size_t)r * a.H_q + qh;
  unpack16<DT>(load16(reinterpret_cast<const char*>(a.q) +
                      (orow * D + (threadIdx.x % RL) * EPL) * DType<DT>::bytes), qf);
  // the host keeps rows within kTrMaxPages and the batch's max_pages (the
  // workspace row stride); the clamp keeps LDS and the workspace in bounds regardless
  return L > 0 ? min(min((L + a.S - 1) / a.S, P_r), min(kTrMaxPages, a.page_stride)) : 0;
}

__device__ __forceinline__ void write_result(const ToprArgs& a, size_t orow, const uint64_t* best,
                                             int kept, int pages) {
  for (int i = threadIdx.x; i < a.R; i += kTrThreads) {
    const bool ok = i < kept;
    a.top_tokens[orow * a.R + i] = ok ? (int)(uint32_t)best[i] : -1;
    a.top_logits[orow * a.R + i] = ok ? key_value(best[i]) : -INFINITY;
  }
  if (threadIdx.x == 0 && a.pages_read) a.pages_read[orow] = pages;
}

// 0. bounds: this head's page bounds ([Quest] eq. (2)-(3) with its own
//    query), raised by the rounding margin, as sort keys in the workspace.
//    RL lanes share a record (16-byte chunks of min and of max), so the
//    summary reads coalesce; kTbPages pages per workgroup.
constexpr int kTbThreads = 256;
constexpr int kTbPages = 64;
template <int DT, int D>
__global__ __launch_bounds__(kTbThreads) void topr_bounds_kernel(ToprArgs a) {
  constexpr int EPL = epl<DT>();
  constexpr int RL = D / EPL;                 // lanes per record half
  constexpr int PPS = kTbThreads / RL;        // pages per step of the workgroup
  constexpr int BYTES = DType<DT>::bytes;
  const int qh = blockIdx.y, r = blockIdx.z, tid = threadIdx.x;
  const int H = a.H_kv, S = a.S, h = qh / (a.H_q / a.H_kv);
  const int L = a.seq_lens[r];
  const int pbeg = a.page_indptr[r];
  const int P_r = a.page_indptr[r + 1] - pbeg;
  const int P = L > 0 ? min(min((L + S - 1) / S, P_r), min(kTrMaxPages, a.page_stride)) : 0;
  const int p_end = min(P, (blockIdx.x + 1) * kTbPages);
  const size_t orow = (size_t)r * a.H_q + qh;
  const int c = tid % RL;
  float qf[EPL];
  unpack16<DT>(load16(reinterpret_cast<const char*>(a.q) + (orow * D + c * EPL) * BYTES), qf);
  const char* summ = reinterpret_cast<const char*>(a.summary);
  uint64_t* wk = a.ws_pages + orow * a.page_stride;
  for (int p = blockIdx.x * kTbPages + tid / RL; p < p_end; p += PPS) {
    const size_t rec = ((size_t)a.page_indices[pbeg + p] * H + h) * 2 * D + c * EPL;
    float m[EPL], M[EPL];
    unpack16<DT>(load16(summ + rec * BYTES), m);
    unpack16<DT>(load16(summ + (rec + D) * BYTES), M);
    float u = 0.f, mag = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      u += fmaxf(qf[e] * m[e], qf[e] * M[e]);
      mag += fabsf(qf[e]) * fmaxf(fabsf(m[e]), fabsf(M[e]));
    }
    u = group_sum<RL>(u);
    mag = group_sum<RL>(mag);
    if (c == 0) wk[p] = desc_key(u + ldexpf(mag, -15), (uint32_t)p);
  }
}

// 1. plan: the branch-and-bound pilot.  The pages of largest bound that
//    whole rounds can read within a.pilot_pages (ties to the lower index:
//    the page keys' order) are picked by the workgroup top-K select and
//    ranked; the pilot reads them in that order, and gives up early when
//    too many unread pages still reach tau_R.  A row whose stop rule fires,
//    or whose largest unread bound is below tau_R, or that has no page left,
//    is finished here; otherwise the pilot's best R go to the workspace with
//    the list of the unread pages whose bound is not below the pilot's
//    tau_R (every unread page while fewer than R tokens are known), left to
//    the scan.
template <int DT, int D, int PT>
__global__ __launch_bounds__(kTrThreads) void topr_plan_kernel(ToprArgs a) {
  // PT bounds per thread: rows of up to kTrThreads * PT pages
  __shared__ TopkShared tsh;
  __shared__ __align__(16) uint64_t s_sel[kTrMaxPilot];
  __shared__ int s_phys[kTrMaxPilot];
  __shared__ int s_selp[kTrMaxPilot];
  __shared__ __align__(16) uint64_t s_buf[2][kTrBuf];
  __shared__ float s_z[kTrThreads];
  __shared__ int s_cnt[kTrWaves];

  const int qh = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int S = a.S, h = qh / (a.H_q / a.H_kv);
  const size_t orow = (size_t)r * a.H_q + qh;
  int L, pbeg;
  float qf[epl<DT>()];
  const int P = row_setup<DT, D>(a, qf, r, qh, L, pbeg);
  const uint64_t* wk = a.ws_pages + orow * a.page_stride;

  // rounds read whole pages: first enough for R tokens, then twice as many
  // each round up to one token per thread; the pilot is the rounds that fit
  // in a.pilot_pages pages
  const int R = a.R;
  const int cp = kTrThreads / S;
  const int s0 = max(1, min(cp, (R + S - 1) / S));
  int cap = 0;
  for (int np = s0; cap + np <= a.pilot_pages; np = min(cp, 2 * np)) cap += np;
  const int npil = min(P, cap > 0 ? cap : a.pilot_pages);

  // the pilot pages: the npil largest bounds, ordered by (bound desc, index asc)
  // (each thread's page-table entries are loaded with its bounds, so the
  // pilot pages' physical pages need no further round trip)
  TopkRow<PT, kTrThreads> t;
  t.j0 = tid * PT;
  t.n = P;
  if (P > 0) {
#pragma unroll
    for (int k = 0; k < PT; ++k) t.pv[k] = a.page_indices[pbeg + min(t.j0 + k, P - 1)];
  }
#pragma unroll
  for (int k = 0; k < PT; ++k) t.v[k] = t.j0 + k < P ? key_value(wk[t.j0 + k]) : 0.f;
  t.select(npil, tsh);
  int count;
  int pos = t.first_position(tsh, &count);
  float out_max = -INFINITY;                          // largest bound outside the pilot
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    if (t.selected(k)) {
      s_sel[pos] = desc_key(t.v[k], (uint32_t)(t.j0 + k));
      s_selp[pos++] = t.pv[k];
    } else if (t.valid(k)) {
      out_max = fmaxf(out_max, t.v[k]);
    }
  }
  float lo_dummy = FLT_MAX;
  tk::block_minmax<kTrWaves>(lo_dummy, out_max, tsh.mm);   // barrier: s_sel complete
  {
    // rank the pilot pages
    uint64_t x = 0;
    int rank = 0, phys = 0;
    if (tid < npil) {
      x = s_sel[tid];
      phys = s_selp[tid];
      rank = count_below(s_sel, 0, npil, x);
    }
    __syncthreads();
    if (tid < npil) {
      s_sel[rank] = x;
      s_phys[rank] = phys;
    }
    __syncthreads();
  }

  // pilot rounds over the pilot pages in order.  After a round, a pilot
  // whose bounds are loose against the logits it has read (even the largest
  // one is below the bound of its last page) and that still has more than
  // kTrBail rounds' worth of unread pages with bounds not below tau_R would
  // not end soon: it hands them to the scan (the result is the same; only
  // the schedule changes).
  int np_round = s0;
  int kept = 0, cur = 0, next = 0;
  bool stopped = false;
  // unread: a page outside the pilot, or a pilot page ranked at or after `next`
  auto unread = [&](int k, int nxt) {
    return t.valid(k) &&
           (!t.selected(k) ||
            (nxt < npil && !(desc_key(t.v[k], (uint32_t)(t.j0 + k)) < s_sel[nxt])));
  };
  while (next < npil) {
    if (kept >= R && key_value(s_sel[next]) < key_value(s_buf[cur][R - 1])) {
      stopped = true;
      break;
    }
    const int np = min(np_round, npil - next);
    np_round = min(cp, 2 * np_round);
    page_logits<DT, D>(a, qf, h, s_phys + next, np, s_z);
    __syncthreads();
    bool cand = false;
    uint64_t ck = 0;
    if (tid < np * S) {
      const int j = (int)(uint32_t)s_sel[next + tid / S];
      const int tt = j * S + tid % S;
      if (tt < L) {
        ck = desc_key(s_z[tid], (uint32_t)tt);
        cand = kept < R || ck < s_buf[cur][R - 1];
      }
    }
    int total;
    const int p2 = tr_excl_count(cand, s_cnt, &total);
    if (cand) s_buf[cur][kept + p2] = ck;
    __syncthreads();
    if (total > 0) rank_merge(s_buf, cur, kept, total, R);
    next += np;
    // (not before two rounds: tau_R from the first alone leaves the scan
    // most tokens as candidates)
    if (kept >= R && next >= 3 * s0 && next < npil &&
        key_value(s_buf[cur][0]) < key_value(s_sel[npil - 1])) {
      const float tr = key_value(s_buf[cur][R - 1]);
      int above = 0;
#pragma unroll
      for (int k = 0; k < PT; ++k) above += (unread(k, next) && !(t.v[k] < tr)) ? 1 : 0;
      int n_above;
      (void)tk::block_excl_scan<kTrWaves>(above, tsh.scan[1], &n_above);
      if (n_above > kTrBail * np_round) break;
    }
  }
  const float tau = kept >= R ? key_value(s_buf[cur][R - 1]) : -INFINITY;
  // largest bound not read: the next pilot page's or the best outside the pilot
  const float rest_max = fmaxf(out_max, next < npil ? key_value(s_sel[next]) : -INFINITY);
  int* st = a.ws_state + orow * 4;
  if (stopped || (next == npil && npil == P) || (kept >= R && rest_max < tau)) {
    write_result(a, orow, s_buf[cur], kept, next);
    if (tid == 0) st[0] = 1;
    return;
  }
  // the unread pages the pilot cannot exclude, in page order
  int mine = 0;
#pragma unroll
  for (int k = 0; k < PT; ++k) mine += (unread(k, next) && (kept < R || !(t.v[k] < tau))) ? 1 : 0;
  int n_scan;
  int at = tk::block_excl_scan<kTrWaves>(mine, tsh.scan[0], &n_scan);
  uint64_t* wp = a.ws_pages + orow * a.page_stride;
  __syncthreads();                                    // every wk read above is done
#pragma unroll
  for (int k = 0; k < PT; ++k)
    if (unread(k, next) && (kept < R || !(t.v[k] < tau)))
      wp[at++] = desc_key(t.v[k], (uint32_t)(t.j0 + k));
  uint64_t* wb = a.ws_pilot + orow * R;
  for (int i = tid; i < kept; i += kTrThreads) wb[i] = s_buf[cur][i];
  if (tid == 0) {
    st[0] = 0;
    st[1] = next;          // pages read by the pilot
    st[2] = n_scan;        // pages left to the scan
    st[3] = kept;
  }
}

// 2. scan: one workgroup per (chunk of kTrThreads tokens of the pages left,
//    query head, request) computes their exact logits and keeps the best R
//    of those beating the pilot's R-th (all of them if the pilot holds fewer
//    than R), in order.
template <int DT, int D>
__global__ __launch_bounds__(kTrThreads) void topr_scan_kernel(ToprArgs a) {
  __shared__ __align__(16) uint64_t s_cand[kTrThreads];
  __shared__ float s_z[kTrThreads];
  __shared__ int s_pp[kTrThreads], s_j[kTrThreads];
  __shared__ int s_cnt[kTrWaves];
  const int c = blockIdx.x, qh = blockIdx.y, r = blockIdx.z, tid = threadIdx.x;
  const size_t orow = (size_t)r * a.H_q + qh;
  const int* st = a.ws_state + orow * 4;
  const int nchunks = a.scan_chunks;
  uint64_t* out = a.ws_chunks + (orow * nchunks + c) * a.R;
  int* cnt = a.ws_counts + orow * nchunks + c;
  if (st[0] != 0) return;                              // finished by the pilot
  const int S = a.S, cp = kTrThreads / S;
  const int p0 = c * cp, p1 = min(st[2], p0 + cp);
  if (p0 >= p1) {
    if (tid == 0) *cnt = 0;
    return;
  }
  const int R = a.R;
  const int pilot_kept = st[3];
  const uint64_t bar = pilot_kept >= R ? a.ws_pilot[orow * R + R - 1] : ~0ull;
  int L, pbeg;
  float qf[epl<DT>()];
  (void)row_setup<DT, D>(a, qf, r, qh, L, pbeg);
  const int h = qh / (a.H_q / a.H_kv);
  const uint64_t* wp = a.ws_pages + orow * a.page_stride;
  const int np = p1 - p0;
  if (tid < np) {
    const int j = (int)(uint32_t)wp[p0 + tid];
    s_j[tid] = j;
    s_pp[tid] = a.page_indices[pbeg + j];
  }
  __syncthreads();
  page_logits<DT, D>(a, qf, h, s_pp, np, s_z);
  __syncthreads();
  bool cand = false;
  uint64_t ck = 0;
  if (tid < np * S) {
    const int t = s_j[tid / S] * S + tid % S;
    if (t < L) {
      ck = desc_key(s_z[tid], (uint32_t)t);
      cand = ck < bar;
    }
  }
  int total;
  const int pos = tr_excl_count(cand, s_cnt, &total);
  if (cand) s_cand[pos] = ck;
  __syncthreads();
  // the best min(total, R) of the candidates, ranked (keys unique)
  if (tid < total) {
    const uint64_t x = s_cand[tid];
    const int rank = count_below(s_cand, 0, total, x);
    if (rank < R) out[rank] = x;
  }
  if (tid == 0) *cnt = min(total, R);
}

// 3. merge: the pilot's list and the chunks' lists, each sorted, merged
//    pairwise in a tree in LDS.  A list sits in a slot of W keys (R rounded
//    up to a power of two), padded with ~0, which is above every key.  Two
//    slots merge into the best W of their union: a key moves to its index
//    plus the number of keys of the other list below it (keys are unique,
//    so the best W land on distinct places, and the padding fills the rest).
//    The search for that number runs on all of a thread's keys in step, one
//    LDS read each per step.  Lists beyond one batch of slots are merged a
//    batch at a time, the running result in the first slot.
// One level of the merge tree: slots 2s and 2s + 1 of `in` (W = 2^lw keys
// each, n slots) into slot s of `out`, KK keys per thread: keys e = e0 +
// threadIdx.x + k * kTrThreads, k < KK (calls with e0 = 0, KK * kTrThreads, ...
// cover the n * W keys in use; they read only `in` and write only `out`).
template <int KK>
__device__ __forceinline__ void merge_level(const uint64_t* in, uint64_t* out, int n, int lw,
                                            int e0 = 0) {
  const int W = 1 << lw, eb = e0 + threadIdx.x;
  uint64_t x[KK];
  int base[KK], pos[KK];
  bool pair[KK];
#pragma unroll
  for (int k = 0; k < KK; ++k) {
    const int e = eb + k * kTrThreads;
    const int slot = e >> lw;
    const bool live = e < n * W;
    pair[k] = live && (slot ^ 1) < n;
    x[k] = in[live ? e : 0];
    base[k] = pair[k] ? (slot ^ 1) << lw : 0;
    pos[k] = 0;
  }
  for (int step = W >> 1; step > 0; step >>= 1) {
    uint64_t y[KK];
#pragma unroll
    for (int k = 0; k < KK; ++k) y[k] = in[base[k] + pos[k] + step - 1];
#pragma unroll
    for (int k = 0; k < KK; ++k) pos[k] += y[k] < x[k] ? step : 0;
  }
  uint64_t y[KK];
#pragma unroll
  for (int k = 0; k < KK; ++k) y[k] = in[base[k] + pos[k]];
#pragma unroll
  for (int k = 0; k < KK; ++k) {
    pos[k] += y[k] < x[k] ? 1 : 0;
    const int e = eb + k * kTrThreads;
    const int slot = e >> lw, i = e & (W - 1);
    const int at = pair[k] ? i + pos[k] : i;           // an unpaired last slot passes through
    if (e < n * W && at < W) out[((slot >> 1) << lw) + at] = x[k];
  }
}

constexpr int kTrMaxChunks = kTrMaxPages / 2;   // page size <= 256: at least 2 pages a chunk
constexpr int kTrMergeKeys = kTrMaxPages;       // keys in a batch of slots
template <int DT, int D>
__global__ __launch_bounds__(kTrThreads) void topr_merge_kernel(ToprArgs a) {
  constexpr int KPT = kTrMergeKeys / kTrThreads;      // keys per thread
  constexpr int CPT = kTrMaxChunks / kTrThreads;      // chunk counts per thread
  __shared__ __align__(16) uint64_t s_m[2][kTrMergeKeys];
  __shared__ int s_off[kTrMaxChunks + 1];
  __shared__ int s_scan[kTrWaves];
  const int qh = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const size_t orow = (size_t)r * a.H_q + qh;
  const int R = a.R, S = a.S, cp = kTrThreads / S;
  const int lw = 32 - __clz(R - 1);                    // W = 2^lw >= R
  const int W = 1 << lw;
  const int NS = kTrMergeKeys / W;                     // slots of a batch
  // The global loads of the first two batches go out at entry, before the
  // row state is known: the state, the chunk counts and the keys of both
  // batches (batch 1: slot s holds list s, the pilot's and then chunk s - 1's;
  // batch 2: slot s >= 1 holds list NS + s - 1, slot 0 the running result),
  // none of whose addresses depends on the counts.  Addresses outside the
  // rows read the pilot list's first entry; validity is applied once state
  // and counts have landed.
  const int* st = a.ws_state + orow * 4;
  const int st0 = st[0], st1 = st[1], st2 = st[2], pilot = st[3];
  const int* cnts = a.ws_counts + orow * a.scan_chunks;
  int cn[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int i = tid * CPT + k;
    cn[k] = cnts[i < a.scan_chunks ? i : 0];
  }
  const uint64_t* pil = a.ws_pilot + orow * R;
  uint64_t v[KPT], v2[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int e = tid + k * kTrThreads;
    const int slot = e >> lw, i = e & (W - 1);
    const uint64_t* src = pil;
    const uint64_t* src2 = pil;
    if (i < R) {
      if (slot == 0) src = pil + i;
      else if (slot - 1 < a.scan_chunks)
        src = a.ws_chunks + (orow * a.scan_chunks + slot - 1) * R + i;
      const int c2 = NS + slot - 2;                    // chunk of list NS + slot - 1
      if (slot >= 1 && c2 < a.scan_chunks) src2 = a.ws_chunks + (orow * a.scan_chunks + c2) * R + i;
    }
    v[k] = *src;
    v2[k] = *src2;
  }
  // a row the plan finished has nothing to merge (no lists, no result)
  const bool live_row = st0 == 0;
  const int nch = live_row ? (st2 + cp - 1) / cp : 0;  // chunks the scan used
  // list offsets: CPT consecutive counts per thread, one block scan
  int mine = 0;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    cn[k] = tid * CPT + k < nch ? cn[k] : 0;
    mine += cn[k];
  }
  int total;
  int run = tk::block_excl_scan<kTrWaves>(mine, s_scan, &total);
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int i = tid * CPT + k;
    if (i < nch) s_off[i] = run;
    run += cn[k];
  }
  if (tid == 0) s_off[nch] = total;
  __syncthreads();

  const int nl = 1 + nch;                              // the pilot's list, then the chunks'
  int cur = 0, done = 0, first = 0;
  while (done < nl) {
    const int fresh = min(NS - first, nl - done);      // lists loaded in this batch
    int n = first + fresh;                             // slots in use
    if (done == NS) {
#pragma unroll
      for (int k = 0; k < KPT; ++k) v[k] = v2[k];
    } else if (done > 0) {
      // batches after the second: slot s >= 1 holds list done + s - 1;
      // every load issued before any LDS store
#pragma unroll
      for (int k = 0; k < KPT; ++k) {
        const int e = tid + k * kTrThreads;
        const int slot = e >> lw, i = e & (W - 1);
        const int list = done + slot - first;
        const bool act = slot >= first && slot < n && i < R;
        v[k] = *(act ? a.ws_chunks + (orow * a.scan_chunks + list - 1) * R + i : pil);
      }
    }
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int e = tid + k * kTrThreads;
      const int slot = e >> lw, i = e & (W - 1);
      if (slot >= first && slot < n) {
        const int list = done + slot - first;
        const int cnt = list == 0 ? pilot : s_off[list] - s_off[list - 1];
        s_m[cur][e] = i < cnt ? v[k] : ~0ull;
      }
    }
    __syncthreads();
    while (n > 1) {
      // keys per thread at this level: n * W halves with every level
      const int live = (n * W + kTrThreads - 1) / kTrThreads;
      if (live > 4) merge_level<KPT>(s_m[cur], s_m[cur ^ 1], n, lw);
      else if (live > 2) merge_level<4>(s_m[cur], s_m[cur ^ 1], n, lw);
      else if (live > 1) merge_level<2>(s_m[cur], s_m[cur ^ 1], n, lw);
      else merge_level<1>(s_m[cur], s_m[cur ^ 1], n, lw);
      __syncthreads();
      cur ^= 1;
      n = (n + 1) >> 1;
    }
    done += fresh;
    first = 1;
  }
  if (live_row) write_result(a, orow, s_m[cur], min(R, pilot + total), st1 + st2);
}

template <int DT, int D>
hipError_t launch_t(const ToprArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((topr_bounds_kernel<DT, D>),
                     dim3((a.page_stride + kTbPages - 1) / kTbPages, a.H_q, a.B), dim3(kTbThreads),
                     0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.page_stride <= kTrThreads * 4)
    hipLaunchKernelGGL((topr_plan_kernel<DT, D, 4>), dim3(a.H_q, a.B), dim3(kTrThreads), 0, s, a);
  else
    hipLaunchKernelGGL((topr_plan_kernel<DT, D, kTrMaxPages / kTrThreads>), dim3(a.H_q, a.B),
                       dim3(kTrThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((topr_scan_kernel<DT, D>), dim3(a.scan_chunks, a.H_q, a.B), dim3(kTrThreads),
                     0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((topr_merge_kernel<DT, D>), dim3(a.H_q, a.B), dim3(kTrThreads), 0, s, a);
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
int topr_threads() { return kTrThreads; }
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
