// Sparse paged decode attention kernels for f32 K/V (decode_kernel.h).
#include "decode_kernel.h"

namespace qas {

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) {
  return launch_decode_dtype<kF32>(a, s);
}

}  // namespace qas
