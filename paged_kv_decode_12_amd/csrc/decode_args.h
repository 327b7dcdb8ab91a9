// decode_args.h -- launch arguments shared by the host planner (api.cpp) and
// the device kernels (decode_kernel.hip).  Internal; not part of the C ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace pkvd {

constexpr int kBlockKeys = 16;   // keys per block: the unit a wave loads and scores
constexpr int kMaxSinkHeads = 4096;   // sink logits the decode kernel stages in LDS
constexpr int kSimdsPerCu = 4;   // a decode workgroup holds WPE waves on each SIMD of a CU
constexpr int kMaxBatch = 8192;        // requests per call (the schedule keeps a prefix in LDS)
// Size of the static workspace of pkvd_decode_static (static_scratch.hip).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;

enum Path : int { kPathValu = 0, kPathMfma = 1 };
enum OutType : int { kOutBf16 = 0, kOutF16 = 1, kOutF32 = 2 };

struct DecodeArgs {
  // inputs (element strides)
  const uint16_t* q;
  int64_t q_sr, q_sh;              // q[r * q_sr + h * q_sh + d]
  const uint16_t* k;
  int64_t k_sp, k_sh;              // k[page * k_sp + kvh * k_sh + slot * D + d]
  const uint16_t* v;
  int64_t v_sp, v_sh;
  const int32_t* bt;
  int64_t bt_sr;                   // bt[b * bt_sr + c]
  const int32_t* seq_lens;
  const int32_t* qo;               // nullptr: Lq rows per request; else (B + 1) cumulative
                                   // offsets of packed query rows (request b owns rows
                                   // qo[b] .. qo[b + 1] - 1, at most Lq of them)
  const float* sinks;              // nullptr: no sinks
  // outputs
  void* out;                       // contiguous (rows, Hq, D), element type out_type
  float* lse;                      // nullptr: not requested
  // workspace: a wave whose slice cuts a unit leaves a normalised partial
  // state in slot 2 * wave + side (decode_common.h, unit_pieces); the wave
  // whose blocks complete the unit merges them (or the merge kernel does)
  float* ws_o;                     // [slots][rows_per_tile * D], engine order
  float* ws_lse;                   // [slots][rows_per_tile], base 2
  // int32 state that every call leaves at zero
  int32_t* counters;               // [B * Hkv * row_tiles] blocks of each unit delivered
  int32_t* ws_pref;                // [B + 1] block prefix of the requests (merge kernel mode)
  int32_t* ws_vpref;               // [B + 1] the same in the virtual block space
  // shapes
  int32_t B, Hq, Hkv, g, Lq, ps, P, C, D;
  int32_t rows;                    // query rows of q / out (B * Lq when qo is null)
  int32_t window_left;
  int32_t causal;                  // 1: bottom-right causal rows, 0: every row sees keys < n
  float scale_log2;                // scale * log2(e): scores are kept in base 2
  float out_scale;                 // factor on the output
  int32_t out_type;                // OutType
  int32_t row_tiles;               // row tiles per (request, kv head) at Lq rows
  int32_t rows_per_tile;           // query rows of one tile (the engine's kRows)
  int32_t num_waves;               // waves of the persistent grid
  int32_t groups;                  // workgroups launched (groups * waves per group >= num_waves)
  int32_t min_wave_blocks;         // a wave gets at least this many blocks (fewer waves run)
  int32_t merge_kernel;            // 1: cut units are merged by a second kernel, not in place
  int32_t seg_cost;                // virtual blocks ahead of each unit in the sliced space
  int32_t unit_mode;               // 1: slice bounds snap to unit starts (every unit whole)
  int32_t slot_w[4];               // slice weight of the waves at position 0, 1, 2, >= 3 on their SIMD
  // The full grid (NW = num_waves, which a block space of T >= full_T real
  // blocks always gets): the parts of its slicing that do not depend on the
  // lengths, set by the host (schedule.h: grid_slices)
  int32_t full_T;
  int32_t full_per, full_uniform;
  int64_t full_sp, full_s;
#ifdef PKVD_TRACE
  uint64_t* trace;                 // instrumented builds only: [waves][16] timestamps
#endif
};

using KernelFn = void (*)(DecodeArgs);
struct KernelPair {
  KernelFn decode, merge;   // nullptr where none is built
};
// The kernels of one head_dim and element type (decode_inst_*.hip): path,
// tile height and whether page_size is a power of two >= 16.
KernelPair kernels_d128_bf16(int path, int rows_per_tile, bool pow2);
KernelPair kernels_d128_f16(int path, int rows_per_tile, bool pow2);
KernelPair kernels_d64_bf16(int path, int rows_per_tile, bool pow2);
KernelPair kernels_d64_f16(int path, int rows_per_tile, bool pow2);

// The current device's address of the static workspace and its size
// (static_scratch.hip).  Allocates nothing.
hipError_t static_scratch(void** ptr, size_t* bytes);

// Launcher (decode_launch.hip).  Returns the hipError_t of the launch.
hipError_t launch_decode(const DecodeArgs& a, int path, int rows_per_tile, bool bf16,
                         hipStream_t stream);
// Waves per workgroup of the decode kernel for a path (0 on error): all the
// waves one CU holds at the kernel's register budget, so one workgroup fills
// a CU and every wave of a CU starts together.
int decode_group_waves(int path, int rows_per_tile, int head_dim);
// Dynamic LDS bytes of a launch for B requests, `threads` per workgroup,
// `sinks` sink logits staged in LDS and (packed) query offsets staged or not.
size_t decode_lds_bytes(int B, int threads, int sinks, bool packed);

}  // namespace pkvd
