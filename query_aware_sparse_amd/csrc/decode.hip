// Host side of the sparse paged decode attention: split planning, limits,
// ticket clearing and the dispatch to the per-dtype kernel translation units
// (the kernels and their design are in decode_kernel.h).
#include "decode_kernel.h"

namespace qas {

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_f16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);

namespace {

__global__ void clear_tickets_kernel(unsigned int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

bool decode_supported(int kv_dtype, int d, int g) {
  return (kv_dtype == kF32 || kv_dtype == kF16 || kv_dtype == kBF16) &&
         (d == 16 || d == 64 || d == 128) && (g == 1 || g == 2 || g == 4 || g == 8);
}

int decode_num_splits(int rows, int sel_len) {
  if (sel_len < 1) sel_len = 1;
  int n = (256 + rows - 1) / rows;            // one workgroup per CU
  const int cap = (sel_len + 3) / 4;
  if (n > cap) n = cap;
  const int need = (sel_len + kDecMaxList - 1) / kDecMaxList;
  if (n < need) n = need;
  if (n < 1) n = 1;
  return n;
}

int decode_max_dedupe_row() { return kDecMaxRow; }

int decode_fused_topk_max_pages() { return kDecThreads * kDecFusedTopkPT; }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.clear_tickets && a.n_split > 1) {
    const int n = a.B * a.H_kv;
    hipLaunchKernelGGL(clear_tickets_kernel, dim3((n + 255) / 256), dim3(256), 0, s, a.tickets, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (a.kv_dtype) {
    case kF32: return launch_decode_f32(a, s);
    case kF16: return launch_decode_f16(a, s);
    case kBF16: return launch_decode_bf16(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qas
