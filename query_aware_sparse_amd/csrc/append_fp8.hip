// FP8 E4M3 K/V writer of the multi-query chunk path ("PageWeaver" notes,
// SS2UKVF2: FP8 E4M3 K/V with one scale per KV head, BF16 queries): every
// element of a new token's K or V row of KV head h is stored as the e4m3
// code of x / scale[h] (the quotient in fp32, clamped to +-448, rounded to
// the nearest code with ties to even), and read back by the chunk kernel as
// scale[h] * code.
//
// Codes go straight into the layout the union attention kernel reads
// (union.hip): each (page, KV head) tile of S * 128 bytes is a sequence of
// blocks of 64 lanes x 16 bytes holding MFMA operands (lane l: row = l % 32,
// hf = l / 32).  K block (tau, ks, c), tau < S/32, ks < 2, c < 2, gives lane
// l token 32 tau + row, dims 64 ks + 32 hf + 16 c + [0, 16).  V block
// (dt, c), dt < 4, c < S/32, gives lane l dim 32 dt + row at k slots
// (S/2) hf + 16 c + [0, 16), token t (w = t % 32, tau = t / 32) sitting at k
// slot (S/2)((w/4) % 2) + 16 tau + 4 (w/8) + w % 4.  A page is therefore
// written as a whole: one workgroup per (page touched, KV head, request)
// builds the tile in LDS - zeros for a page the new tokens open (rows past
// the sequence must hold finite codes: the PV product multiplies them by a
// zero probability), else the tile as it stands in the pool - places the new
// tokens' codes, and writes the tile back as 16-byte words.
#include "qas_device.h"
#include "qas_internal.h"

namespace qas {

namespace {

constexpr int kFp8Threads = 256;
constexpr int kFp8D = 128;
constexpr int kFp8MaxS = 64;

// byte of (token t, dim d) inside a K tile
__device__ __forceinline__ int k_tile_byte(int t, int d) {
  const int tau = t >> 5, row = t & 31;
  const int ks = d >> 6, hf = (d >> 5) & 1, c = (d >> 4) & 1, e = d & 15;
  return (((tau * 2 + ks) * 2 + c) * 64 + row + 32 * hf) * 16 + e;
}

// byte of (token t, dim d) inside a V tile of page size S
__device__ __forceinline__ int v_tile_byte(int t, int d, int S) {
  const int w = t & 31, tau = t >> 5;
  const int slot = (S / 2) * ((w >> 2) & 1) + 16 * tau + 4 * (w >> 3) + (w & 3);
  const int hf = slot / (S / 2), rem = slot - hf * (S / 2);
  const int c = rem >> 4, e = rem & 15;
  const int dt = d >> 5, row = d & 31;
  return ((dt * (S / 32) + c) * 64 + row + 32 * hf) * 16 + e;
}

// e4m3 codes of x / s for 16 consecutive elements, four per word
__device__ __forceinline__ uint4 quantize16(const float* x, float s) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = fminf(fmaxf(__fdiv_rn(x[4 * i + k], s), -448.f), 448.f);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    w[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// 16 input elements (a row chunk of the caller's K or V) as floats
template <int DT>
__device__ __forceinline__ void load_row16(const char* p, float* x) {
  constexpr int EPL = epl<DT>();
#pragma unroll
  for (int v = 0; v < 16 / EPL; ++v) unpack16<DT>(load16(p + 16 * v), x + v * EPL);
}

template <int DT>
__global__ __launch_bounds__(kFp8Threads) void append_fp8_kernel(Fp8AppendArgs a) {
  constexpr int BYTES = DType<DT>::bytes;
  __shared__ __align__(16) unsigned char ktile[kFp8MaxS * kFp8D];
  __shared__ __align__(16) unsigned char vtile[kFp8MaxS * kFp8D];
  const int u = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int H = a.H_kv, S = a.S;
  const int L0 = a.seq_lens[r];
  const int src0 = a.new_indptr[r];
  const int n = a.new_indptr[r + 1] - src0;
  if (n <= 0 || L0 < 0) return;
  const int p = L0 / S + u;                   // logical page touched
  if (p > (L0 + n - 1) / S) return;
  const int t0 = max(L0, p * S);
  const int t1 = min(L0 + n, (p + 1) * S);
  const size_t phys = (size_t)a.page_indices[a.page_indptr[r] + p];
  const int tile = S * kFp8D;
  uint4* kdst = reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.k_pool) + (phys * H + h) * tile);
  uint4* vdst = reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.v_pool) + (phys * H + h) * tile);
  const int tid = threadIdx.x;
  const bool fresh = t0 == p * S;             // the page's first token is new
  for (int i = tid; i < tile / 16; i += kFp8Threads) {
    const uint4 kz = fresh ? make_uint4(0, 0, 0, 0) : kdst[i];
    const uint4 vz = fresh ? make_uint4(0, 0, 0, 0) : vdst[i];
    reinterpret_cast<uint4*>(ktile)[i] = kz;
    reinterpret_cast<uint4*>(vtile)[i] = vz;
  }
  __syncthreads();
  const float ks = a.k_scale[h], vs = a.v_scale[h];
  const char* ksrc = reinterpret_cast<const char*>(a.k_new);
  const char* vsrc = reinterpret_cast<const char*>(a.v_new);
  const int items = (t1 - t0) * (kFp8D / 16);
  for (int it = tid; it < items; it += kFp8Threads) {
    const int t = t0 + it / (kFp8D / 16);     // token of the sequence
    const int d0 = (it % (kFp8D / 16)) * 16;  // first of its 16 dims
    const size_t src = (((size_t)(src0 + t - L0) * H + h) * kFp8D + d0) * BYTES;
    float x[16];
    load_row16<DT>(ksrc + src, x);
    const uint4 kc = quantize16(x, ks);
    load_row16<DT>(vsrc + src, x);
    const uint4 vc = quantize16(x, vs);
    const int tp = t - p * S;                 // token row of the page
    *reinterpret_cast<uint4*>(ktile + k_tile_byte(tp, d0)) = kc;
    const uint32_t vw[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
    for (int e = 0; e < 16; ++e)
      vtile[v_tile_byte(tp, d0 + e, S)] = (unsigned char)(vw[e >> 2] >> (8 * (e & 3)));
  }
  __syncthreads();
  for (int i = tid; i < tile / 16; i += kFp8Threads) {
    kdst[i] = reinterpret_cast<const uint4*>(ktile)[i];
    vdst[i] = reinterpret_cast<const uint4*>(vtile)[i];
  }
}

template <int DT>
hipError_t launch_t(const Fp8AppendArgs& a, hipStream_t s) {
  dim3 grid((a.max_new + a.S - 1) / a.S + 1, a.H_kv, a.B);
  hipLaunchKernelGGL((append_fp8_kernel<DT>), grid, dim3(kFp8Threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool append_fp8_supported(int new_dtype, int d, int S) {
  return (new_dtype == kF32 || new_dtype == kF16 || new_dtype == kBF16) && d == kFp8D &&
         (S == 32 || S == 64);
}

hipError_t launch_append_fp8(const Fp8AppendArgs& a, hipStream_t s) {
  switch (a.new_dtype) {
    case kF32: return launch_t<kF32>(a, s);
    case kF16: return launch_t<kF16>(a, s);
    case kBF16: return launch_t<kBF16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qas
