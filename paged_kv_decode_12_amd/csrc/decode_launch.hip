// decode_launch.hip -- launch of the persistent decode kernel (and of the
// merge kernel when the plan uses it) for one pkvd_decode call.
#include "decode_kernel.h"

namespace pkvd {

namespace {

bool page_pow2(int ps) { return ps >= kBlockKeys && (ps & (ps - 1)) == 0; }

KernelPair kernels(int path, int rows_per_tile, int head_dim, bool bf16, bool pow2) {
  if (head_dim == 128) return bf16 ? kernels_d128_bf16(path, rows_per_tile, pow2)
                                   : kernels_d128_f16(path, rows_per_tile, pow2);
  if (head_dim == 64) return bf16 ? kernels_d64_bf16(path, rows_per_tile, pow2)
                                  : kernels_d64_f16(path, rows_per_tile, pow2);
  return KernelPair{nullptr, nullptr};
}

}  // namespace

int decode_group_waves(int path, int rows_per_tile, int head_dim) {
  using namespace dev;
  int wpe = 0;
  if (path == kPathMfma)
    wpe = rows_per_tile != 16 ? 0 : (head_dim == 64 ? mfma_wpe<64>() : mfma_wpe<128>());
  else if (rows_per_tile == 4)
    wpe = valu_wpe<4>();
  else if (rows_per_tile == 8)
    wpe = valu_wpe<8>();
  return kSimdsPerCu * wpe;
}

size_t decode_lds_bytes(int B, int threads, int sinks, bool packed) {
  return sizeof(int) * (size_t)dev::lds_layout(B, threads, sinks, packed).total;
}

hipError_t launch_decode(const DecodeArgs& a, int path, int rows_per_tile, bool bf16,
                         hipStream_t stream) {
  const KernelPair k = kernels(path, rows_per_tile, a.D, bf16, page_pow2(a.ps));
  if (!k.decode || !k.merge) return hipErrorInvalidValue;
  const int waves = decode_group_waves(path, rows_per_tile, a.D);
  if (!waves || (int64_t)a.groups * waves < a.num_waves) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k.decode, dim3(a.groups), dim3(64 * waves),
                     decode_lds_bytes(a.B, 64 * waves, a.sinks ? a.Hq : 0, a.qo != nullptr),
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.merge_kernel) return e;
  // one wave per (unit, row of its tile)
  const int pairs = a.B * a.Hkv * a.row_tiles * rows_per_tile;
  hipLaunchKernelGGL(k.merge, dim3((pairs + dev::kMergeWaves - 1) / dev::kMergeWaves),
                     dim3(64 * dev::kMergeWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkvd
