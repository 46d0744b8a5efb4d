// Sparse paged decode attention kernels for f16 K/V (decode_kernel.h).
#include "decode_kernel.h"

namespace qas {

hipError_t launch_decode_f16(const DecodeArgs& a, hipStream_t s) {
  return launch_decode_dtype<kF16>(a, s);
}

}  // namespace qas
