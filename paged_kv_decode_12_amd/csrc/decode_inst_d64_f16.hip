// decode_inst_d64_f16.hip -- the decode and merge kernels for head_dim 64,
// IEEE fp16 inputs (one translation unit per head_dim and element type, so the
// instantiations compile in parallel).
#include "decode_kernel.h"

namespace pkvd {

KernelPair kernels_d64_f16(int path, int rows_per_tile, bool pow2) {
  return dev::select_kernels<64, false>(path, rows_per_tile, pow2);
}

}  // namespace pkvd
