// Workgroup-level sparse attention over a list of pages staged in LDS, with
// the split merge: the streaming and merging half of the decode attention
// kernel (decode_kernel.h), kept apart from the list building.
//
// Semantics ("PageWeaver" notes, eq. (1)-(2); "3.1.1 · Quest", §2.1): for
// each query head of the KV head's group, exact softmax attention over the
// token rows of the staged pages (a page contributes its first ntok rows);
// the partial softmax states of the splits of a row are merged by
// log-sum-exp (the QuantSpec post's flash-decoding chunk merge), and an
// empty support gives out = 0 and lse = -inf.  Groups of 4 or 8 query heads
// with 16-bit K/V take attend_split_mfma (at the end of this file), which
// runs both products on matrix cores; both streams end in
// attend_merge_waves.
//
// Execution.  The workgroup's waves stream "token groups" (TPI token rows of
// one page = one 16-byte load per lane for K and one for V), UNR groups per
// wave in flight.  Each lane keeps a private online-softmax state (max, sum,
// accumulator of its 16-byte dim chunk) per query head of the group over the
// token rows it sees; lanes of one token row share the logit after a DPP
// reduction.  States are merged across lanes, then waves (LDS).  With
// several splits per row, each split stores its state and takes a ticket
// from the row's counter; the split that arrives last merges all states by
// log-sum-exp and writes the output.
//
// Memory ordering of the split merge (gfx950).  A split's states are
// written with agent-scope relaxed atomic stores, which compile to global
// stores with the sc1 (device-coherence) bit: they are written through the
// XCD's L2 to the device's coherence point instead of staying dirty in it.
// Each thread then waits for its stores with s_waitcnt vmcnt(0); the memory
// model's own agent-scope sequences rely on that wait meaning the store is
// performed at the coherence point (a device-scope store followed by that
// wait is what orders it before a later operation).  The workgroup meets at
// a barrier, and only then does one thread take the ticket with an
// agent-scope atomic add, performed at the same point.  The split that
// draws the last ticket value therefore follows every other split's ticket,
// each taken after that split's states were performed, and it reads the
// states with agent-scope loads (sc1: served from the coherence point, not
// from a line its own XCD's L2 may hold).  The release/acquire pairing of
// the HIP memory model would add an L2 writeback (buffer_wbl2) before each
// ticket and an L2 invalidate (buffer_inv) after the last one; measured on
// this part they cost about 2 us per decode-layer call here (and far more
// where many workgroups hand off), and with every shared word written and
// read device-coherently there is nothing dirty for them to write back or
// stale for them to drop.
#pragma once

#include "qas_device.h"

namespace qas {

constexpr float kLog2e = 1.4426950408889634f;

namespace attend_detail {

// Merge online-softmax state (m2, l2, acc2) into (m, l, acc); -inf max means
// an empty state.
template <int N>
__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float m2,
                                            float l2, const float* acc2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  const float a1 = fast_exp2(m - mm), a2 = fast_exp2(m2 - mm);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = acc[e] * a1 + acc2[e] * a2;
  m = mm;
}

// Device-coherent word stores / loads (agent scope, relaxed; sc1 on this
// part): see the ordering note above.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace attend_detail

// Where the split's result goes.
struct AttendOut {
  void* out;                 // [rows][H_q][D] (row = request or draft row)
  float* lse;                // [rows][H_q] or NULL
  float* partials;           // [rows][H_q][n_split][2 + D]
  unsigned int* ticket;      // this (row, KV head)'s split counter (n_split > 1)
  size_t rowq0;              // index of the group's first query head: row * H_q + h * G
  int n_split, split;
};

// Merge of the lanes' online-softmax states (m_run, l_run, acc[G][epl]: lane
// lane % (D / epl) holds dims [epl * that, +epl) of each query head's
// accumulator) over the workgroup's waves, then over the row's splits, and
// the output.  Every thread of the workgroup must call this.
// The waves' states, published in LDS (red_m / red_l [NW][G], red_acc
// [NW][G][D]), merged over the workgroup's waves and then over the row's
// splits, and the output.  Every thread of the workgroup must call this.
template <int DT, int D, int G, int NW>
__device__ __forceinline__ void attend_merge_waves(const float (*red_m)[G],
                                                   const float (*red_l)[G],
                                                   const float (*red_acc)[G][D],
                                                   const AttendOut& o) {
  using namespace attend_detail;
  constexpr int NT = NW * kWave;
  __shared__ int s_last;
  const int tid = threadIdx.x;
  __syncthreads();
  const bool single = o.n_split == 1;
  for (int t = tid; t < G * D; t += NT) {
    const int gg = t / D, dim = t - (t / D) * D;
    float m = -INFINITY, l = 0.f, ov = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float one[1] = {red_acc[w][gg][dim]};
      merge_state<1>(m, l, &ov, red_m[w][gg], red_l[w][gg], one);
    }
    const size_t rowq = o.rowq0 + gg;
    if (single) {
      store_rn<DT>(o.out, rowq * D + dim, m == -INFINITY ? 0.f : ov / l);
      if (dim == 0 && o.lse)
        o.lse[rowq] = m == -INFINITY ? -INFINITY : (m + log2f(l)) * 0.6931471805599453f;
      continue;
    }
    float* part = o.partials + (rowq * o.n_split + o.split) * (D + 2);
    if (dim == 0) {
      store_coherent(part, m);
      store_coherent(part + 1, l);
    }
    store_coherent(part + 2 + dim, ov);
  }
  if (single) return;

  // ---- the last split of the row merges all split states -----------------
  __builtin_amdgcn_s_waitcnt(0);             // this thread's states are stored
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(o.ticket, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(o.n_split - 1);
  }
  __syncthreads();
  if (!s_last) return;
  constexpr int MB = 16;
  for (int t = tid; t < G * D; t += NT) {
    const int gg = t / D, dim = t - (t / D) * D;
    const size_t rowq = o.rowq0 + gg;
    const float* part = o.partials + rowq * o.n_split * (D + 2);
    float M = -INFINITY, lsum = 0.f, ov = 0.f;
    for (int sb = 0; sb < o.n_split; sb += MB) {
      float ms[MB], ls[MB], os[MB];
#pragma unroll
      for (int k = 0; k < MB; ++k) {
        const int sp = sb + k;
        const bool in = sp < o.n_split;
        ms[k] = in ? load_coherent(part + sp * (D + 2)) : -INFINITY;
        ls[k] = in ? load_coherent(part + sp * (D + 2) + 1) : 0.f;
        os[k] = in ? load_coherent(part + sp * (D + 2) + 2 + dim) : 0.f;
      }
#pragma unroll
      for (int k = 0; k < MB; ++k) merge_state<1>(M, lsum, &ov, ms[k], ls[k], &os[k]);
    }
    store_rn<DT>(o.out, rowq * D + dim, M == -INFINITY ? 0.f : ov / lsum);
    if (dim == 0 && o.lse)
      o.lse[rowq] = M == -INFINITY ? -INFINITY : (M + log2f(lsum)) * 0.6931471805599453f;
  }
  // leave the counter at zero for the next call
  if (tid == 0) __hip_atomic_store(o.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT, int D, int G, int NW>
__device__ __forceinline__ void attend_finish(float* m_run, float* l_run,
                                              float (*acc)[epl<DT>()], const AttendOut& o) {
  using namespace attend_detail;
  constexpr int EPL = epl<DT>();
  constexpr int RL = D / EPL;                 // lanes per token row
  __shared__ float red_m[NW][G];
  __shared__ float red_l[NW][G];
  __shared__ float red_acc[NW][G][D];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int c = lane % RL;

  // ---- merge lanes of one dim chunk, then the waves ------------------------
#pragma unroll
  for (int off = RL; off < kWave; off <<= 1) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const float m2 = shfl_xor_f(m_run[gg], off);
      const float l2 = shfl_xor_f(l_run[gg], off);
      float acc2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc2[e] = shfl_xor_f(acc[gg][e], off);
      merge_state<EPL>(m_run[gg], l_run[gg], acc[gg], m2, l2, acc2);
    }
  }
  if (lane < RL) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      if (lane == 0) {
        red_m[wave][gg] = m_run[gg];
        red_l[wave][gg] = l_run[gg];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_acc[wave][gg][c * EPL + e] = acc[gg][e];
    }
  }
  attend_merge_waves<DT, D, G, NW>(red_m, red_l, red_acc, o);
}

// The workgroup (NW waves) attends over npg pages staged in s_phys / s_ntok
// (physical page, token rows to read).  qraw holds this
// lane's 16-byte chunk (lane % (D / epl)) of each query head of the group.
// Every thread of the workgroup must call this; LDS of the staged lists may
// be reused only after it returns.
template <int DT, int D, int G, int UNR, int NW>
__device__ __forceinline__ void attend_split(const int* s_phys, const int* s_ntok, int npg,
                                             int S, const char* kbase, const char* vbase,
                                             size_t pstride, uint32_t hoff_head,
                                             const uint4* qraw, float sm_scale,
                                             const AttendOut& o) {
  using namespace attend_detail;
  constexpr int EPL = epl<DT>();
  constexpr int RL = D / EPL;                 // lanes per token row
  constexpr int TPI = kWave / RL;             // token rows per wave load
  constexpr int BYTES = DType<DT>::bytes;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int c = lane % RL;
  const int trow = lane / RL;
  const int NI = S > TPI ? S / TPI : 1;       // token groups per page (a power of two)
  const int lni = __ffs(NI) - 1;
  const int units = npg * NI;
  // byte offsets: page stride and head offset are uniform, so a load's
  // address is one 64-bit multiply-add of its physical page
  const uint32_t hoff = hoff_head + c * 16;
  const float qscale = sm_scale * kLog2e;     // logits in log2 units
  float qf[G][EPL];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    unpack16<DT>(qraw[gg], qf[gg]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[gg][e] *= qscale;
  }
  float m_run[G], l_run[G], acc[G][EPL];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    m_run[gg] = -INFINITY;
    l_run[gg] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[gg][e] = 0.f;
  }

  for (int u0 = wave; u0 < units; u0 += NW * UNR) {
    uint4 kr[UNR], vr[UNR];
    bool ok[UNR];
    // Every load is unconditional: a unit past the end is clamped to the last
    // unit and a token row past the page's tokens to the page's last row, so
    // each address stays inside an allocated page, and `ok` drops the value.
    // (A load under a branch makes the compiler wait for every earlier load
    // before it.)  All K loads go first, so the logits start while V is still
    // in flight.
    size_t offs[UNR];
#pragma unroll
    for (int b = 0; b < UNR; ++b) {
      const int u = min(u0 + b * NW, units - 1);
      const int pi = u >> lni, gi = u & (NI - 1);
      const int tip = gi * TPI + trow;
      ok[b] = (u0 + b * NW < units) & (tip < s_ntok[pi]);
      offs[b] = (size_t)(uint32_t)s_phys[pi] * pstride +
                (hoff + (uint32_t)(min(tip, S - 1) * D * BYTES));
    }
#pragma unroll
    for (int b = 0; b < UNR; ++b) kr[b] = load16(kbase + offs[b]);
#pragma unroll
    for (int b = 0; b < UNR; ++b) vr[b] = load16(vbase + offs[b]);
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      float z[UNR];
      float zmax = m_run[gg];
#pragma unroll
      for (int b = 0; b < UNR; ++b) {
        float kf[EPL];
        unpack16<DT>(kr[b], kf);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot += qf[gg][e] * kf[e];
        dot = group_sum<RL>(dot);
        z[b] = ok[b] ? dot : -INFINITY;
        zmax = fmaxf(zmax, z[b]);
      }
      // No branch on the batch's content: a branch here lets the compiler
      // sink the V loads below the logits, a second round trip per batch.
      // With no valid logit yet the stand-in maximum 0 gives alpha = 0 and
      // p = 0 on a zero state; rows not loaded read as zero words.
      const float zm = zmax == -INFINITY ? 0.f : zmax;
      const float alpha = fast_exp2(m_run[gg] - zm);
      float l = l_run[gg] * alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[gg][e] *= alpha;
#pragma unroll
      for (int b = 0; b < UNR; ++b) {
        const float p = ok[b] ? fast_exp2(z[b] - zm) : 0.f;
        const uint4 w = ok[b] ? vr[b] : make_uint4(0, 0, 0, 0);
        float vf[EPL];
        unpack16<DT>(w, vf);
        l += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[gg][e] += p * vf[e];
      }
      l_run[gg] = l;
      m_run[gg] = zmax;
    }
  }

  attend_finish<DT, D, G, NW>(m_run, l_run, acc, o);
}

// ---- grouped-query heads on matrix cores ----------------------------------
// With G = 4 or 8 query heads per KV head (16-bit K/V, d = 128, S a multiple
// of 16) both products of a wave's batch of two 16-token tiles run on
// v_mfma_f32_16x16x32 (A lane l: row l % 16, k = 8 (l / 16) + [0, 8) of
// the step; B lane l: those k of column l % 16; D lane l: rows
// 4 (l / 16) + [0, 4) of column l % 16):
//
// * logits, per tile: D[i][t] = q_i . k_t over d = 128 in four steps (query
//   rows i >= G zero).  K step s of lane l reads bytes [64 s + 16 (l / 16),
//   +16) of tile row l % 16, so each load covers 64 contiguous bytes of all
//   16 rows of the 4 KiB tile; a tile never crosses a page, so no address is
//   clamped, and rows past the page's tokens are dropped.  Products exact,
//   sums in fp32, then scaled by sm_scale log2(e) in fp32.
// * softmax: lane l holds the logits of heads 4 (l / 16) + r of token l % 16,
//   so a head's batch max and probability sum are reductions over one
//   16-lane row, and a head's running max and sum are the same in all lanes
//   of its row.  The sum adds p = exp2(z - m) in fp32.  The PV operand is p
//   split into two values of the K/V dtype, p_hi = rn(p) and
//   p_lo = rn(p - p_hi), each multiplied with V on the matrix cores: p alone
//   rounded to bf16 (relative 2^-9) would put outputs with cancelling terms
//   outside 2e-3; the pair leaves an error near 2^-18 p (or 2^-25 for f16
//   subnormal remainders), as good as fp32 for this purpose.
// * values: O[i][d] += sum_t P[i][t] V[t][d] over the batch's 32 tokens, one
//   step per 16 dims and per half of p (sixteen).  P goes to LDS
//   token-major ([token][p_hi of the heads | p_lo of the heads], 4G bytes
//   a token) and V row by row (whole 16-byte chunks, rows past the
//   tokens zeroed), and both operands come back with the transposing LDS
//   read ds_read_b64_tr_b16: within each 16 lanes, lane i receives element
//   i % 4 of the 8-byte words addressed by lanes 4 k + i / 4, k = 0..3 (lane
//   layout checked on the device).  So lane l of group g = l / 16 addressing
//   row 8 g + 4 h + (l % 16) / 4, columns 4 ((l % 16) % 4) + [0, 4) of a
//   16-column block, for h = 0 and 1, gets the 8 k-values of column l % 16
//   that the operand layout asks for.  V rows sit 288 bytes apart, with rows
//   8..15 of each 16 swapped in halves, so that the 8 rows one half-wave
//   reads fall in 8 different 32-byte bank groups.
// The accumulators are then in the MFMA output layout (lane l: heads
// 4 (l / 16) + r, dim 16 n + l % 16 of block n); attend_finish_mfma
// publishes them for attend_merge_waves.

// Query operand of the group for attend_split_mfma: lane l takes head row
// l % 16 of the group (zero for rows >= G), dims 32 s + 8 (l / 16) + [0, 8)
// in qa[s].  qrow: the group's first query head, 128 16-bit values per head.
template <int G>
__device__ __forceinline__ void load_q_operand(const char* qrow, uint4* qa) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = lane & 15, quad = lane >> 4;
  const char* q = qrow + (size_t)(i < G ? i : 0) * 256 + quad * 16;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qa[s] = load16(q + 64 * s);
    if (i >= G) qa[s] = make_uint4(0, 0, 0, 0);
  }
}

typedef __bf16 attend_bf16x8_t __attribute__((ext_vector_type(8)));
typedef short attend_s4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) attend_s4_t attend_lds_s4_t;

template <int DT>
__device__ __forceinline__ float4_t attend_mfma(const uint4& a, const uint4& b,
                                                const float4_t& c) {
  if constexpr (DT == kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(attend_bf16x8_t, a),
                                                   __builtin_bit_cast(attend_bf16x8_t, b), c, 0,
                                                   0, 0);
}

// two transposing 8-byte LDS reads -> one 16-byte operand register
__device__ __forceinline__ uint4 lds_read_tr2(const unsigned char* p0, const unsigned char* p1) {
  const attend_s4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((attend_lds_s4_t*)p0);
  const attend_s4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((attend_lds_s4_t*)p1);
  const uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
  return make_uint4(x.x, x.y, y.x, y.y);
}

// p (finite, >= 0) as two values of the 16-bit K/V dtype, each rounded to
// nearest even: returns the bits of hi = rn(p), *lo the bits of rn(p - hi)
// (p - hi is exact in fp32)
template <int DT>
__device__ __forceinline__ uint32_t round16(float p, uint32_t* lo) {
  if constexpr (DT == kF16) {
    const _Float16 h = (_Float16)p;
    *lo = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(p - (float)h));
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
  } else {
    const uint32_t u = __float_as_uint(p);
    const uint32_t h = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
    const uint32_t r = __float_as_uint(p - __uint_as_float(h));   // either sign
    const uint32_t rl = (r & 0x7fffffffu) == 0 ? r : r + 0x7fffu + ((r >> 16) & 1u);
    *lo = rl >> 16;
    return h >> 16;
  }
}

// Publishes attend_split_mfma's wave states (lane l: heads 4 (l / 16) + r,
// dims 16 n + l % 16) for attend_merge_waves.
template <int DT, int G, int NW>
__device__ __forceinline__ void attend_finish_mfma(const float* m_run, const float* l_run,
                                                   const float4_t* acc, const AttendOut& o) {
  constexpr int D = 128;
  __shared__ float red_m[NW][G];
  __shared__ float red_l[NW][G];
  __shared__ float red_acc[NW][G][D];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int col = lane & 15, quad = lane >> 4;
  if (quad < G / 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gg = 4 * quad + r;
      if (col == 0) {
        red_m[wave][gg] = m_run[r];
        red_l[wave][gg] = l_run[r];
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) red_acc[wave][gg][16 * n + col] = acc[n][r];
    }
  }
  attend_merge_waves<DT, D, G, NW>(red_m, red_l, red_acc, o);
}

constexpr int kMfVRow = 288;               // LDS bytes between V rows
constexpr int kMfLds = 32 * kMfVRow + 32 * 32 + 16;   // V rows, P rows, zero word

// As attend_split, for DT f16/bf16, d = 128, G in {4, 8} and S a multiple of
// 16.  qa: load_q_operand's registers.
template <int DT, int G, int NW>
__device__ __forceinline__ void attend_split_mfma(const int* s_phys, const int* s_ntok, int npg,
                                                  int S, const char* kbase, const char* vbase,
                                                  size_t pstride, uint32_t hoff_head,
                                                  const uint4* qa, float sm_scale,
                                                  const AttendOut& o) {
  constexpr int D = 128;
  constexpr int ROW = D * 2;                  // bytes of a token row
  constexpr int UT = 2;                       // tiles per batch: one 32-token PV step
  constexpr int PS = 4 * G;                   // LDS bytes of a token's P row (hi | lo)
  static_assert(DType<DT>::bytes == 2 && (G == 4 || G == 8), "16-bit K/V, 4 or 8 heads");
  __shared__ __align__(16) unsigned char mf_lds[NW][kMfLds];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int col = lane & 15, quad = lane >> 4;   // MFMA column / row quad; V: chunk, row
  unsigned char* vl = mf_lds[wave];
  unsigned char* pl = vl + 32 * kMfVRow;
  unsigned char* zl = pl + 32 * 32;
  if (lane < 4) reinterpret_cast<uint32_t*>(zl)[lane] = 0u;
  // transposing-read addresses: row 8 g + 4 h + k, word m of a 16-column block
  const int tk = col >> 2, tm = col & 3;
  int vrow[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 8 * quad + 4 * h + tk;
    vrow[h] = (t ^ (((t >> 3) & 1) << 2)) * kMfVRow + 8 * tm;
  }
  const unsigned char* pa0 = tm < G / 4 ? pl + (8 * quad + tk) * PS + 8 * tm : zl;
  const unsigned char* pa1 = tm < G / 4 ? pl + (8 * quad + 4 + tk) * PS + 8 * tm : zl;
  const int lo = tm < G / 4 ? 2 * G : 0;      // offset of the p_lo half

  const int TPP = S >> 4;                     // tiles per page (a power of two)
  const int ltp = __ffs(TPP) - 1;
  const int units = npg * TPP;
  const float qscale = sm_scale * kLog2e;     // logits in log2 units
  float m_run[4], l_run[4];                   // heads 4 quad + r
  float4_t acc[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
#pragma unroll
  for (int n = 0; n < 8; ++n) acc[n] = {0.f, 0.f, 0.f, 0.f};

  for (int u0 = wave * UT; u0 < units; u0 += NW * UT) {
    // two consecutive tiles; every load unconditional (a tile past the end
    // repeats the last one and its rows are dropped); K first, so the
    // logits start while V is in flight
    size_t tb[UT];
    int nrow[UT];
#pragma unroll
    for (int b = 0; b < UT; ++b) {
      const int u = min(u0 + b, units - 1);
      const int pi = u >> ltp, ti = u & (TPP - 1);
      nrow[b] = u0 + b < units ? s_ntok[pi] - 16 * ti : 0;   // rows kept: t < nrow
      tb[b] = (size_t)(uint32_t)s_phys[pi] * pstride + (hoff_head + (uint32_t)(16 * ti * ROW));
    }
    uint4 kr[UT][4], vr[UT][4];
#pragma unroll
    for (int b = 0; b < UT; ++b)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kr[b][s] = load16(kbase + tb[b] + (col * ROW + 64 * s + 16 * quad));
#pragma unroll
    for (int b = 0; b < UT; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vr[b][j] = load16(vbase + tb[b] + ((4 * j + quad) * ROW + 16 * col));
    float4_t lg[UT];
#pragma unroll
    for (int b = 0; b < UT; ++b) {
      lg[b] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) lg[b] = attend_mfma<DT>(qa[s], kr[b][s], lg[b]);
    }
    // softmax over the batch, per head row (lanes of one quad)
    float z[UT][4], zm[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float zmax = -INFINITY;
#pragma unroll
      for (int b = 0; b < UT; ++b) {
        z[b][r] = col < nrow[b] ? lg[b][r] * qscale : -INFINITY;
        zmax = fmaxf(zmax, z[b][r]);
      }
      zmax = fmaxf(group_max<16>(zmax), m_run[r]);
      // as in attend_split: with no valid logit yet the stand-in maximum 0
      // gives alpha = 0 and p = 0 on a zero state
      zm[r] = zmax == -INFINITY ? 0.f : zmax;
      const float alpha = fast_exp2(m_run[r] - zm[r]);
      m_run[r] = zmax;
      l_run[r] *= alpha;
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[n][r] *= alpha;
    }
    float psum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < UT; ++b) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(z[b][r] - zm[r]);
        wh[r] = round16<DT>(p, &wl[r]);
        psum[r] += p;
      }
      if (quad < G / 4) {
        unsigned char* pr = pl + (16 * b + col) * PS + 8 * quad;
        *reinterpret_cast<uint2*>(pr) = make_uint2(wh[0] | (wh[1] << 16), wh[2] | (wh[3] << 16));
        *reinterpret_cast<uint2*>(pr + 2 * G) =
            make_uint2(wl[0] | (wl[1] << 16), wl[2] | (wl[3] << 16));
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) l_run[r] += group_sum<16>(psum[r]);
    // V rows to LDS (rows past the tokens as zeros: their p is zero, and
    // 0 * inf or nan would not be)
#pragma unroll
    for (int b = 0; b < UT; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * b + 4 * j + quad;
        const uint4 x = 4 * j + quad < nrow[b] ? vr[b][j] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(vl + (t ^ (((t >> 3) & 1) << 2)) * kMfVRow + 16 * col) = x;
      }
    // this wave's LDS writes are done before its transposing reads
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const uint4 phi = lds_read_tr2(pa0, pa1);
    const uint4 plo = lds_read_tr2(pa0 + lo, pa1 + lo);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint4 vop = lds_read_tr2(vl + vrow[0] + 32 * n, vl + vrow[1] + 32 * n);
      acc[n] = attend_mfma<DT>(phi, vop, acc[n]);
      acc[n] = attend_mfma<DT>(plo, vop, acc[n]);
    }
    // the reads are done before the next batch's writes
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  attend_finish_mfma<DT, G, NW>(m_run, l_run, acc, o);
}

}  // namespace qas
