// Measurement kernels behind the rates the decode path is compared with
// (built into libqas_micro.so, separate from libqas.so, and driven by
// `bench.py --micro`): the read rate of the access pattern the attention
// kernel uses (whole tiles of a few KiB at scattered tile-aligned offsets,
// 16-byte loads, 16 tile rows of 1 KiB in flight per wave), the same bytes
// read in order, the cost of an empty kernel inside a HIP graph, and the
// latency of a chain of dependent global loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kMbThreads = 512;
constexpr int kMbWaves = kMbThreads / 64;
constexpr int kMbUnroll = 16;          // 1 KiB wave loads in flight per wave

// Each workgroup reads tiles ids[wg * per .. wg * per + per) of tile_bytes each
// (tile id -> byte offset id * tile_bytes), as 1 KiB wave loads, the waves
// taking interleaved 1 KiB rows of the workgroup's tiles; the words are
// summed and one value per workgroup is stored so nothing is dropped.
__global__ __launch_bounds__(kMbThreads) void read_tiles_kernel(const char* base,
                                                                const uint32_t* ids, int per,
                                                                int tile_bytes, uint32_t* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x / 64;
  const int rows_per_tile = tile_bytes / 1024;
  const int rows = per * rows_per_tile;
  const uint32_t* my = ids + (size_t)blockIdx.x * per;
  uint32_t acc = 0;
  for (int r0 = wave; r0 < rows; r0 += kMbWaves * kMbUnroll) {
    uint4 v[kMbUnroll];
#pragma unroll
    for (int b = 0; b < kMbUnroll; ++b) {
      const int r = min(r0 + b * kMbWaves, rows - 1);
      const int t = r / rows_per_tile, row = r - t * rows_per_tile;
      const size_t off = (size_t)my[t] * tile_bytes + (size_t)row * 1024 + lane * 16;
      v[b] = *reinterpret_cast<const uint4*>(base + off);
    }
#pragma unroll
    for (int b = 0; b < kMbUnroll; ++b) acc += v[b].x ^ v[b].y ^ v[b].z ^ v[b].w;
  }
  acc += __shfl_xor(acc, 1);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ void empty_kernel() {}

// One lane follows next[] for `steps` dependent loads from index 0.
__global__ void chase_kernel(const uint32_t* next, int steps, uint32_t* out) {
  uint32_t i = 0;
  for (int s = 0; s < steps; ++s) i = next[i];
  out[0] = i;
}

}  // namespace

extern "C" {

// Read n_wg * per tiles listed in ids (device uint32 [n_wg * per]) from buf.
int qas_micro_read_tiles(const void* buf, const uint32_t* ids, int n_wg, int per,
                         int tile_bytes, uint32_t* sink, void* stream) {
  if (!buf || !ids || !sink || n_wg < 1 || per < 1 || tile_bytes < 1024 || tile_bytes % 1024)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_tiles_kernel, dim3(n_wg), dim3(kMbThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const char*>(buf), ids, per, tile_bytes, sink);
  return (int)hipGetLastError();
}

int qas_micro_empty(void* stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

int qas_micro_chase(const uint32_t* next, int steps, uint32_t* out, void* stream) {
  if (!next || !out || steps < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(chase_kernel, dim3(1), dim3(1), 0, (hipStream_t)stream, next, steps, out);
  return (int)hipGetLastError();
}

}  // extern "C"
