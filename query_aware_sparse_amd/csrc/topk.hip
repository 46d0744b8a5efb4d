// Standalone top-K page selection per (request, KV head): the Quest page's
// second stage ("3.1.1 · Quest", §1 and Fig. 1), ordered by (score
// descending, page index ascending), joined with the fixed sink and
// local-window pages when asked (§3.2), written in ascending page order and
// padded with -1.  One 512-thread workgroup per row runs the
// register-resident histogram select of topk_block.h.
#include "qas_device.h"
#include "qas_internal.h"
#include "topk_block.h"

namespace qas {

namespace {

template <int PT>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkArgs a) {
  __shared__ TopkShared sh;
  const int row = blockIdx.x;
  const int H = a.H_kv;
  const int r = row / H, h = row - (row / H) * H;
  const int tid = threadIdx.x;
  const int pbeg = a.page_indptr[r];
  const int P_r = a.page_indptr[r + 1] - pbeg;
  const int L = a.seq_lens[r];
  // never more scores than the registers hold
  const int n = L > 0 ? min(min((L + a.S - 1) / a.S, P_r), kTkThreads * PT) : 0;
  const int take = min(a.k, n);
  int32_t* out = a.sel + (size_t)row * a.sel_stride;
  int32_t* out_phys = a.sel_phys ? a.sel_phys + (size_t)row * a.sel_stride : nullptr;

  TopkRow<PT> t;
  t.load(a.scores + (size_t)pbeg * H + (size_t)h * P_r,
         out_phys ? a.page_indices + pbeg : nullptr, n);
  t.set_fixed(L, a.S, a.sink_tokens, a.local_tokens);
  t.select(take, sh);
  int count;
  int pos = t.first_position(sh, &count);
  if (a.sel_count && tid == 0) a.sel_count[row] = count;
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    if (t.selected(k)) {
      out[pos] = t.j0 + k;
      if (out_phys) out_phys[pos] = t.pv[k];
      ++pos;
    }
  }
  for (int j = count + tid; j < a.sel_stride; j += kTkThreads) {
    out[j] = -1;
    if (out_phys) out_phys[j] = -1;
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  const int m = a.max_pages > 0 ? a.max_pages : 1;
  dim3 grid(a.B * a.H_kv);
  dim3 block(kTkThreads);
  if (m <= kTkThreads * 4) {
    hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, a);
  } else if (m <= kTkThreads * 8) {
    hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, a);
  } else if (m <= kTkThreads * 16) {
    hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, a);
  } else if (m <= kTkThreads * 32) {
    hipLaunchKernelGGL(topk_kernel<32>, grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qas
