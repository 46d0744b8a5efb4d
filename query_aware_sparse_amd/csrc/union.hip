// Multi-query chunk attention over query unions (the PageWeaver notes:
// support semantics of eq. (1)-(2), annotation 2BIFS6UT; query union and
// membership masks, SS2BST9I; union preparation, AWLR3K97; per-group tiles
// that keep each query's own softmax, 5ALRMYYY; FP8 QK / FP8 PV with fp32
// running statistics, SS2UKVF2).
//
// A group is `group` consecutive queries of one request; with g query heads
// per KV head its rows form one 32-row MFMA tile (rows = query * g + head).
// One workgroup per (pair of consecutive groups, KV head), 8 waves, mapped
// so that all groups of one KV head land on the same XCD (their page unions
// overlap, so neighbours hit in that XCD's L2):
//   1. union preparation, one half of the workgroup per group: each query's
//      valid page IDs set bits in a per-query bitmap in LDS; OR-ing them
//      gives the union, emitted in ascending page order with an 8-bit
//      membership mask per page and its physical page;
//   2. four waves per group (two of the first four and two of the last
//      four, so that neither group's waves are all the younger ones on
//      their SIMDs) stream its union pages, the older two taking 7 of
//      every 24 pages each and the younger two 5, so that the group's
//      waves and both groups end together (a fixed share keeps the result
//      bitwise repeatable).  S^T = K Q^T with
//      the fp8 K tile as A straight from HBM/L2 and Q quantised per row to
//      e4m3 as B (v_mfma 32x32x64 f8f6f4); each lane then owns one row's
//      logits, so the mask (membership, t <= c_i, t < L) and the online
//      softmax are lane-local; P is scaled by 256 and quantised to e4m3 and
//      feeds O^T += V^T P^T from registers.  The fp8 pools store each
//      (page, head) tile in operand order: blocks of 64 lanes x 16 bytes,
//      each block holding one 16-byte piece of every lane's A (K) or B (V^T,
//      tokens in the order of the MFMA's k slots) operand, so a wave load
//      reads 1 KiB of consecutive bytes: no LDS staging or byte gathers;
//   3. each group's four wave states are merged in LDS and written at the
//      queries' own output rows.
#include "qas_device.h"
#include "qas_internal.h"

namespace qas {

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kUThreads = 256;
constexpr int kUWaves = kUThreads / kWave;
constexpr int kURows = 32;                  // MFMA tile rows
constexpr int kUMaxGroup = 8;               // queries per group (membership byte)
constexpr int kUMaxWords = 512;             // bitmap words: pages < 16384
constexpr int kUMaxUnion = 1024;            // union pages per group
constexpr int kUD = 128;                    // head dim
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kULazy = 0.75f;             // running-max slack, log2 units

struct UnionShared {
  uint32_t bm[kUMaxGroup][kUMaxWords];
  int ulist[kUMaxUnion];
  int uphys[kUMaxUnion];
  unsigned char umask[kUMaxUnion];
  int cpos[kUMaxGroup];
  int qid[kUMaxGroup];       // original query of each execution slot
  int wave_tot[kUWaves];
  int count;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Exclusive prefix sum over kUThreads threads (order of the local index
// tid), one workgroup barrier after the per-wave totals are published;
// *total gets the sum.
__device__ __forceinline__ int block_excl(int v, int tid, int* scratch, int* total) {
  const int lane = lane_id(), wave = tid / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kUWaves; ++w) {
    before += w < wave ? scratch[w] : 0;
    all += scratch[w];
  }
  *total = all;
  return before + incl - v;
}

struct GroupInfo {
  int r, q0, nq;   // request, first query, queries in the group (0: none)
};

// Group gi of the launch: requests contribute ceil(n_r / group) groups each,
// in request order.
__device__ GroupInfo find_group(const int32_t* q_indptr, int B, int group, int gi) {
  GroupInfo gr{0, 0, 0};
  int base = 0;
  for (int r = 0; r < B; ++r) {
    const int a = q_indptr[r], n = q_indptr[r + 1] - a;
    const int ng = (n + group - 1) / group;
    if (gi < base + ng) {
      const int local = gi - base;
      gr.r = r;
      gr.q0 = a + local * group;
      gr.nq = min(group, n - local * group);
      return gr;
    }
    base += ng;
  }
  return gr;
}

// Groups gi and gi + 1 of the launch (as find_group), from one pass over the
// request bounds.
__device__ void find_group_pair(const int32_t* q_indptr, int B, int group, int gi,
                                GroupInfo* gr) {
  gr[0] = GroupInfo{0, 0, 0};
  gr[1] = GroupInfo{0, 0, 0};
  int base = 0;
  for (int r = 0; r < B; ++r) {
    const int a = q_indptr[r], n = q_indptr[r + 1] - a;
    const int ng = (n + group - 1) / group;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int local = gi + k - base;
      if (local >= 0 && local < ng) {
        gr[k].r = r;
        gr[k].q0 = a + local * group;
        gr[k].nq = min(group, n - local * group);
      }
    }
    base += ng;
    if (gi + 1 < base) break;
  }
}

constexpr int kUEpt = kUMaxUnion / kUThreads;   // set entries per thread

// A group's set entries and causal limits loaded ahead of the union build
// (ok: they belong to the group being built).
struct PreSets {
  int v[kUEpt];   // entry tid + k * kUThreads of the group's concatenated sets
  int cpos;       // threads < kUMaxGroup: causal limit of that query
  bool ok;
};

// Union of the group's page sets in ascending order with membership bits
// and physical pages (the PageWeaver notes, SS2BST9I / AWLR3K97), built by
// kUThreads threads (local index tid) while every thread of the workgroup
// takes the same barriers.  Returns the union size; the lists are in `sh`.
// A group with no queries gets an empty union.
__device__ int build_union(UnionShared& sh, const UnionArgs& a, const GroupInfo& gr, int h,
                           int n_pages, int pbeg, const PreSets& pre, int tid) {
  const int words = (n_pages + 31) / 32;
  for (int i = tid; i < kUMaxGroup * words; i += kUThreads) sh.bm[i / words][i % words] = 0;
  // the original query of every slot (an execution order from the regroup,
  // else the identity)
  int my_qid = 0;
  if (tid < kUMaxGroup) {
    const int slot = gr.q0 + (tid < gr.nq ? tid : 0);
    my_qid = a.ids ? a.ids[(size_t)h * a.N + slot] : slot;
    sh.qid[tid] = my_qid;
  }
  __syncthreads();
  // entries <= kUMaxUnion: every set entry's load is issued before any is
  // used, and the slots' causal limits (the union preparation alone has
  // none) are loaded beside them
  constexpr int EPT = kUEpt;
  const int entries = gr.nq * a.kq;
  int ids[EPT];
  if (pre.ok) {
#pragma unroll
    for (int k = 0; k < EPT; ++k) ids[k] = pre.v[k];
  } else {
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = max(0, min(tid + k * kUThreads, entries - 1));
      const int i = e / a.kq;
      ids[k] = a.sets[((size_t)sh.qid[i] * a.H_kv + h) * a.kq + (e - i * a.kq)];
    }
  }
  if (tid < kUMaxGroup)
    sh.cpos[tid] = (a.q_pos && tid < gr.nq) ? (pre.ok ? pre.cpos : a.q_pos[my_qid]) : -1;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + k * kUThreads;
    const int id = ids[k];
    if (e < entries && id >= 0 && id < n_pages) atomicOr(&sh.bm[e / a.kq][id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  // each thread owns bpt consecutive bits of the bitmaps (pages), 4 to 64
  // so that the union is spread over as many threads as it has 4-page
  // slices: a slice of one word (bpt <= 32) or two whole words (bpt = 64);
  // its per-query words are read once into registers, masked to the slice
  constexpr int WPT = kUMaxWords / kUThreads;   // words of the widest slice
  static_assert(WPT == 2, "slices are one word or two");
  const int bpt = words <= 32 ? 4 : words <= 64 ? 8 : words <= 128 ? 16 : words <= 256 ? 32 : 64;
  const int b0 = tid * bpt;
  const int w0 = b0 >> 5;
  const uint32_t smask = bpt >= 32 ? ~0u : ((1u << bpt) - 1u) << (b0 & 31);
  uint32_t qw[WPT][kUMaxGroup];
  int mine = 0;
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int w = w0 + k;
    const bool in = (k == 0 || bpt == 64) && w < words;
#pragma unroll
    for (int i = 0; i < kUMaxGroup; ++i)
      qw[k][i] = (in && i < gr.nq) ? sh.bm[i][in ? w : 0] & smask : 0u;
    uint32_t u = 0;
#pragma unroll
    for (int i = 0; i < kUMaxGroup; ++i) u |= qw[k][i];
    mine += __popc(u);
  }
  int total;
  int pos = block_excl(mine, tid, sh.wave_tot, &total);
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int w = w0 + k;
    uint32_t u = 0;
#pragma unroll
    for (int i = 0; i < kUMaxGroup; ++i) u |= qw[k][i];
    while (u) {
      const int b = __builtin_ctz(u);
      u &= u - 1;
      unsigned char m = 0;
#pragma unroll
      for (int i = 0; i < kUMaxGroup; ++i) m |= ((qw[k][i] >> b) & 1u) << i;
      sh.ulist[pos] = w * 32 + b;
      sh.umask[pos] = m;
      ++pos;
    }
  }
  __syncthreads();
  // physical pages of the union: independent loads, all in flight together
  // (total <= kUMaxUnion; an index past the union rereads its last page)
  if (total > 0) {
    int ph[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) ph[k] = a.page_indices[pbeg + sh.ulist[min(tid + k * kUThreads, total - 1)]];
#pragma unroll
    for (int k = 0; k < EPT; ++k)
      if (tid + k * kUThreads < total) sh.uphys[tid + k * kUThreads] = ph[k];
  }
  if (tid == 0) sh.count = total;
  __syncthreads();
  return total;
}

__device__ __forceinline__ float lane_rowmax(float v) { return fmaxf(v, __shfl_xor(v, 32, kWave)); }

constexpr int kUPair = 2;                          // groups per workgroup
constexpr int kUPairThreads = kUPair * kUThreads;  // 8 waves, two per SIMD
// pages of a group: per kUCycle, kUOld to each older and kUYoung to each
// younger wave (7:5, measured against 4:3, 5:4, 3:2 and an even split)
constexpr int kUOld = 7, kUYoung = 5, kUCycle = 2 * (kUOld + kUYoung);

// Wave w of the workgroup computes group (w ^ (w >> 2)) & 1 of its pair as
// that group's wave w >> 1: each group gets two of the first four waves and
// two of the last four, one per SIMD when the waves are dealt out to the
// SIMDs in turn, so that the issue priority of older waves favours neither
// group.
__device__ __forceinline__ int pair_unit(int wave) { return (wave ^ (wave >> 2)) & 1; }

template <int G, int NT>
__global__ __launch_bounds__(kUPairThreads, 2) void union_attn_kernel(UnionArgs a) {
  constexpr int S = 32 * NT;                  // page size
  __shared__ UnionShared shu[kUPair];
  __shared__ __align__(16) float red_buf[kUPair][2][32][kUD + 2];   // wave merge per group

  const int H = a.H_kv;
  const int h = blockIdx.x % H;
  const int pair = blockIdx.x / H;
  // the wave index as a uniform value, so that everything derived from it
  // (the groups, their bounds) stays in scalar registers and scalar loads
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // each half of the workgroup builds the union of one group of the pair ...
  const int bh = wave / kUWaves, btid = threadIdx.x % kUThreads;
  // ... and each wave computes one group's pages
  const int unit = pair_unit(wave), lw = wave >> 1;
  UnionShared& sh = shu[unit];
  // ---- per-lane row: row = query * G + head (S^T / O^T column = lane % 32)
  const int row = lane % 32, hf = lane / 32;
  const int qi = row / G, hq = row % G;

  GroupInfo grp[kUPair];
  find_group_pair(a.q_indptr, a.B, a.group, kUPair * pair, grp);
  if (grp[0].nq == 0) return;                 // uniform: no group in the pair
  const GroupInfo grb = bh ? grp[1] : grp[0], grc = unit ? grp[1] : grp[0];
  const bool row_ok = qi < grc.nq;
  // Everything the union build and the query rows need is loaded together
  // as soon as the groups are known: in identity order the built group's
  // set entries and causal limits (with an execution order they follow
  // the order's entries inside the build), the computed group's query rows,
  // and the request bounds.  Slots are clamped to N - 1, so a group with
  // fewer queries (or none) stays in bounds.
  PreSets pre;
  pre.ok = a.ids == nullptr;
  uint4 qraw[8];
  // computed group: Q row slice, dims 64*ks + 32*hf + [0, 32) for ks = 0, 1,
  // quantised per row (a row past the group is zeroed)
  auto load_q = [&](int qid) {
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     (((size_t)qid * a.H_q + h * G + hq) * kUD) * 2;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int c = 0; c < 4; ++c) qraw[4 * ks + c] = load16(qp + (64 * ks + 32 * hf + 8 * c) * 2);
  };
  // the query rows first: with an execution order their address waits for
  // the order's entry, and that wait must not cover the set loads
  const int cslot = min(grc.q0 + (row_ok ? qi : 0), a.N - 1);
  load_q(a.ids ? a.ids[(size_t)h * a.N + cslot] : cslot);
  if (pre.ok) {
    const int gkq = a.group * a.kq;
#pragma unroll
    for (int k = 0; k < kUEpt; ++k) {
      const int e = min(btid + k * kUThreads, gkq - 1);
      const int i = e / a.kq;
      const int qid = min(grb.q0 + i, a.N - 1);
      pre.v[k] = a.sets[((size_t)qid * H + h) * a.kq + (e - i * a.kq)];
    }
    pre.cpos = a.q_pos[min(grb.q0 + (btid < kUMaxGroup ? btid : 0), a.N - 1)];
  }
  // built group: its request's pages (none for a group with no queries)
  const int Lb = grb.nq > 0 ? a.seq_lens[grb.r] : 0;
  const int pbeg = a.page_indptr[grb.r];
  const int P_r = a.page_indptr[grb.r + 1] - pbeg;
  const int n_pages = Lb > 0 ? min(min((Lb + S - 1) / S, P_r), kUMaxWords * 32) : 0;
  const int L = a.seq_lens[grc.r];

  build_union(shu[bh], a, grb, h, n_pages, pbeg, pre, btid);
  const int U = sh.count;
  const int cq = row_ok ? sh.cpos[qi] : -1;
  float qf[64];
#pragma unroll
  for (int i = 0; i < 8; ++i) unpack16<kBF16>(qraw[i], qf + 8 * i);
  if (!row_ok)
#pragma unroll
    for (int e = 0; e < 64; ++e) qf[e] = 0.f;
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 64; ++e) amax = fmaxf(amax, fabsf(qf[e]));
  amax = lane_rowmax(amax);
  const float qs = amax > 0.f ? amax / 448.f : 1.f;
  // q / qs as q times one reciprocal (within an ulp of the quotient, far
  // below the e4m3 step), clamped to +-448 (the conversion does not
  // saturate), four codes per word from two packed conversions
  const float rqs = 1.f / qs;
  v8i_t qop[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint32_t w[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      float x[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        x[k] = __builtin_amdgcn_fmed3f(qf[ks * 32 + 4 * b + k] * rqs, -448.f, 448.f);
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], __float_as_int(x[2]), false);
      w[b] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
    }
    qop[ks] = *reinterpret_cast<v8i_t*>(w);
  }
  // logit scale (log2 units) of this row, floored at a tiny positive value
  // so that a masked logit (-inf) times it stays -inf
  const float zscale = fmaxf(qs * a.k_scale[h] * a.sm_scale * kLog2e, 1e-30f);

  float m_run = -INFINITY, l_run = 0.f;
  v16f_t acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

  const char* kbase = reinterpret_cast<const char*>(a.k_pool);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool);

  // K operand of union page u: token 32*tau + lane%32, dims 64*ks + 32*hf + [0, 32).
  // The tile is stored in operand order, blocks (tau, ks, c) of 64 lanes x
  // 16 bytes, so each load reads 1 KiB of consecutive bytes.
  auto load_k = [&](int u, v8i_t (&kk)[NT][2]) {
    const size_t tile = ((size_t)sh.uphys[u] * H + h) * S * kUD;   // bytes (fp8)
#pragma unroll
    for (int tau = 0; tau < NT; ++tau)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const char* p = kbase + tile + (size_t)(2 * tau + ks) * 2048 + lane * 16;
        const uint4 x0 = load16(p), x1 = load16(p + 1024);
        const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        kk[tau][ks] = *reinterpret_cast<const v8i_t*>(w);
      }
  };
  // V^T operand of union page u: lane (dim 32 dt + row, hf) holds k slots
  // (S/2) hf + [0, S/2) of that dim row, in the order the PV MFMA takes the
  // tokens; the tile is stored as blocks (dt, c) of 64 lanes x 16 bytes
  auto load_v = [&](int u, v8i_t (&vv)[4]) {
    const size_t tile = ((size_t)sh.uphys[u] * H + h) * S * kUD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const char* vr = vbase + tile + (size_t)(dt * NT) * 1024 + lane * 16;
      uint32_t vw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      const uint4 y0 = load16(vr);
      vw[0] = y0.x;
      vw[1] = y0.y;
      vw[2] = y0.z;
      vw[3] = y0.w;
      if constexpr (NT == 2) {
        const uint4 y1 = load16(vr + 1024);
        vw[4] = y1.x;
        vw[5] = y1.y;
        vw[6] = y1.z;
        vw[7] = y1.w;
      }
      vv[dt] = *reinterpret_cast<const v8i_t*>(vw);
    }
  };
  // The operands of a wave's next page are loaded into the registers of the
  // current one as soon as its MFMAs have read them (K after QK, V after PV),
  // so the loads fly during the softmax and the MFMAs; the last page's
  // loads repeat it and are not used.
  v8i_t kop[NT][2], vop[4];
  // A operand whose row 0 is all ones (e4m3 1.0 = 0x38) and the rest zero:
  // lanes 0 and 32 hold row 0's two k halves
  v8i_t ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (lane & 31) == 0 ? 0x38383838 : 0;
  // Union pages per group wave, fixed so that the result does not depend
  // on timing: of every kUCycle consecutive pages the group's two older
  // waves (lw 0, 1: among the first four of the workgroup, favoured by
  // their SIMDs' issue arbitration) take kUOld each and the two younger
  // ones kUYoung each, interleaved, so that all four end together.
  auto page_of = [&](int k) {
    const int per = lw < 2 ? kUOld : kUYoung;
    const int c = k / per, j = k - c * per;
    return c * kUCycle + (lw < 2 ? 2 * j + lw : 2 * kUOld + 2 * j + (lw - 2));
  };
  int kk = 0;
  int u = page_of(0);
  int un = page_of(1);
  if (u < U) {
    load_k(u, kop);
    load_v(u, vop);
  }
  while (u < U) {
    const int id = sh.ulist[u];
    const unsigned char mk = sh.umask[u];
    const int ul = min(un, U - 1);          // next operands (the last page repeats itself)
    // S^T = K Q^T: lane holds row `row`, tokens 32 tau + 8 (e/4) + 4 hf + e%4
    v16f_t st[NT];
#pragma unroll
    for (int tau = 0; tau < NT; ++tau) {
#pragma unroll
      for (int e = 0; e < 16; ++e) st[tau][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        st[tau] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop[tau][ks], qop[ks], st[tau],
                                                                  0, 0, 0, 0, 0, 0);
    }
    load_k(ul, kop);
    // mask + online softmax, lane-local per row.  Pages that every row of
    // the wave sees whole (all but those at a causal limit or the sequence
    // end) skip the per-token mask; element k = 16 tau + e of a lane is
    // token 32 tau + 8 (e/4) + 4 hf + e%4 of the page.
    const bool member = row_ok && ((mk >> qi) & 1);
    const int pend = id * S + S - 1;
    if (__ballot(member && !(pend <= cq && pend < L)) != 0) {
#pragma unroll
      for (int tau = 0; tau < NT; ++tau)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = id * S + 32 * tau + 8 * (e / 4) + 4 * hf + (e % 4);
          st[tau][e] = (t <= cq && t < L) ? st[tau][e] : -INFINITY;
        }
    }
    float zr = -INFINITY;                       // unscaled row max
#pragma unroll
    for (int tau = 0; tau < NT; ++tau)
#pragma unroll
      for (int e = 0; e < 16; ++e) zr = fmaxf(zr, st[tau][e]);
    zr = member ? zr : -INFINITY;
    const float zmax = lane_rowmax(zr == -INFINITY ? -INFINITY : zr * zscale);
    // The running max moves only when a row's max passes it by more than
    // kULazy (log2 units): p = 2^8 exp2(z - m) then stays below
    // 2^(8 + kULazy) < 448, inside e4m3, and most pages skip the rescale.
    const bool grow = zmax > m_run + kULazy;    // same for both lanes of a row
    const float m_use = grow ? zmax : m_run;
    const bool live = m_use != -INFINITY;
    // P^T operand: 32 e4m3 bytes.  No branch on the row: a row that is not
    // a member of the page, or has no logit yet, takes an offset of -inf, so
    // all its p are exp2(-inf) = 0 (the logits are finite or -inf).
    uint32_t pw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const float off = member && live ? 8.f - m_use : -INFINITY;
#pragma unroll
    for (int tau = 0; tau < NT; ++tau)
#pragma unroll
      for (int e = 0; e < 16; e += 4) {
        const int k = 16 * tau + e;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(st[tau][e + i], zscale, off));
        // the first conversion keeps the high half of its third operand,
        // which the second one overwrites: a logit no longer needed will do
        const int lo =
            __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(st[tau][e]), false);
        pw[k / 4] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
      }
    const v8i_t pop = *reinterpret_cast<const v8i_t*>(pw);
    // the row sum over the quantised values (the ones the PV product uses),
    // on the matrix cores: a product with an all-ones row 0 sums each P^T
    // column, i.e. each row's p over the page, into output row 0 (register 0
    // of lanes 0-31, lane = row); lanes 32-63 take their row's from there
    const v16f_t rs = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pop, v16f_t{}, 0, 0,
                                                                      0, 0, 0, 0);
    const float rs_up = __shfl_xor(rs[0], 32, kWave);
    const float lsum = hf ? rs_up : rs[0];
    const float alpha = grow ? fast_exp2(m_run - m_use) : 1.f;   // 0 on a row's first page
    if (live) {
      l_run = l_run * alpha + lsum * (1.f / 256.f);
      m_run = m_use;
    }
    if (__ballot(grow) != 0) {                  // a row's max moved: rescale
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[dt][e] *= alpha;
    }
    // O^T += V^T P^T: lane (dim 32 dt + lane%32, hf) holds the same k slots
    // (tokens 32 tau + 8 (e/4) + 4 hf + e%4) as its P bytes
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      acc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[dt], pop, acc[dt], 0, 0, 0, 0,
                                                                0, 0);
    load_v(ul, vop);
    u = un;
    ++kk;
    un = page_of(kk + 1);
  }

  // ---- merge each group's waves: 2,3 -> 0,1 then 1 -> 0 ---------------------
  float* red = &red_buf[unit][0][0][0];      // [2][32 rows][130]
  constexpr int RS = kUD + 2;
  __syncthreads();
#pragma unroll
  for (int step = 0; step < 2; ++step) {
    const int lo_w = step == 0 ? 2 : 1;       // waves >= lo_w publish
    if (lw >= lo_w && lw < 2 * lo_w) {
      float* dst = red + (size_t)(lw - lo_w) * kURows * RS + row * RS;
      if (hf == 0) {
        dst[0] = m_run;
        dst[1] = l_run;
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[2 + 32 * dt + 8 * (e / 4) + 4 * hf + (e % 4)] = acc[dt][e];
    }
    __syncthreads();
    if (lw < lo_w) {
      const float* src = red + (size_t)lw * kURows * RS + row * RS;
      const float m2 = src[0], l2 = src[1];
      const float mm = fmaxf(m_run, m2);
      if (mm != -INFINITY) {
        const float a1 = fast_exp2(m_run - mm), a2 = fast_exp2(m2 - mm);
        l_run = l_run * a1 + l2 * a2;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            acc[dt][e] = acc[dt][e] * a1 + src[2 + 32 * dt + 8 * (e / 4) + 4 * hf + (e % 4)] * a2;
        m_run = mm;
      }
    }
    __syncthreads();
  }

  // ---- outputs at the queries' own rows ----------------------------------------
  if (lw == 0 && row_ok) {
    const size_t orow = (size_t)sh.qid[qi] * a.H_q + h * G + hq;
    const float oscale = l_run > 0.f ? a.v_scale[h] / (256.f * l_run) : 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        store_rn<kBF16>(a.out, orow * kUD + 32 * dt + 8 * (e / 4) + 4 * hf + (e % 4),
                        acc[dt][e] * oscale);
    if (hf == 0 && a.lse)
      a.lse[orow] = l_run > 0.f ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
  }
}

// Standalone union preparation: lists, counts and membership per (group, head).
__global__ __launch_bounds__(kUThreads) void union_prep_kernel(UnionArgs a) {
  __shared__ UnionShared sh;
  const int H = a.H_kv;
  const int h = blockIdx.x % H;
  const int gi = blockIdx.x / H;
  const GroupInfo gr = find_group(a.q_indptr, a.B, a.group, gi);
  const int cap = a.group * a.kq;
  int32_t* ul = a.union_out + ((size_t)gi * H + h) * cap;
  unsigned char* um = a.member_out + ((size_t)gi * H + h) * cap;
  int U = 0;
  if (gr.nq > 0) {
    const int L = a.seq_lens[gr.r];
    const int pbeg = a.page_indptr[gr.r];
    const int P_r = a.page_indptr[gr.r + 1] - pbeg;
    const int n_pages = L > 0 ? min(min((L + a.S - 1) / a.S, P_r), kUMaxWords * 32) : 0;
    PreSets none;
    none.ok = false;
    U = build_union(sh, a, gr, h, n_pages, pbeg, none, threadIdx.x);
  }
  for (int i = threadIdx.x; i < cap; i += kUThreads) {
    ul[i] = i < U ? sh.ulist[i] : -1;
    um[i] = i < U ? sh.umask[i] : 0;
  }
  if (threadIdx.x == 0) a.count_out[(size_t)gi * H + h] = U;
}

}  // namespace

bool union_supported(int kv_dtype, int q_dtype, int d, int S, int g, int group, int kq) {
  return kv_dtype == kE4M3 && q_dtype == kBF16 && d == kUD && (S == 32 || S == 64) &&
         (g == 1 || g == 2 || g == 4 || g == 8) && group >= 1 && group * g <= kURows &&
         group <= kUMaxGroup && group * kq <= kUMaxUnion && kq >= 1;
}

int union_max_pages() { return kUMaxWords * 32; }

hipError_t launch_union_attn(const UnionArgs& a, hipStream_t s) {
  dim3 grid((a.max_groups + kUPair - 1) / kUPair * a.H_kv);
#define QAS_UNION_CASE(GG, NT)                                                            \
  if (a.g == GG && a.S == 32 * NT) {                                                      \
    hipLaunchKernelGGL((union_attn_kernel<GG, NT>), grid, dim3(kUPairThreads), 0, s, a); \
    return hipGetLastError();                                                             \
  }
  QAS_UNION_CASE(1, 1) QAS_UNION_CASE(1, 2) QAS_UNION_CASE(2, 1) QAS_UNION_CASE(2, 2)
  QAS_UNION_CASE(4, 1) QAS_UNION_CASE(4, 2) QAS_UNION_CASE(8, 1) QAS_UNION_CASE(8, 2)
#undef QAS_UNION_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_union_prep(const UnionArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(union_prep_kernel, dim3(a.max_groups * a.H_kv), dim3(kUThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace qas
