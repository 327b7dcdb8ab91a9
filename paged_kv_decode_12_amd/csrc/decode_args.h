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

enum Path : int { kPathValu = 0, kPathMfma = 1 };

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
  const float* sinks;              // nullptr: no sinks
  // outputs
  uint16_t* out;                   // contiguous (B * Lq, Hq, D)
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
  int32_t window_left;
  float scale_log2;                // scale * log2(e): scores are kept in base 2
  int32_t row_tiles;               // row tiles per (request, kv head)
  int32_t num_waves;               // waves of the persistent grid
  int32_t groups;                  // workgroups launched (groups * waves per group >= num_waves)
  int32_t min_wave_blocks;         // a wave gets at least this many blocks (fewer waves run)
  int32_t merge_kernel;            // 1: cut units are merged by a second kernel, not in place
  int32_t seg_cost;                // virtual blocks ahead of each unit in the sliced space
  int32_t slot_w[4];               // slice weight of the waves at position 0, 1, 2, >= 3 on their SIMD
#ifdef PKVD_TRACE
  uint64_t* trace;                 // instrumented builds only: [waves][16] timestamps
#endif
};

// Launcher (decode_kernel.hip).  Returns the hipError_t of the launch.
hipError_t launch_decode(const DecodeArgs& a, int path, int rows_per_tile, bool bf16,
                         hipStream_t stream);
// Waves per workgroup of the decode kernel for a path (0 on error): all the
// waves one CU holds at the kernel's register budget, so one workgroup fills
// a CU and every wave of a CU starts together.
int decode_group_waves(int path, int rows_per_tile, int head_dim);
// Dynamic LDS bytes of a launch for B requests, `threads` per workgroup and
// `sinks` sink logits staged in LDS.
size_t decode_lds_bytes(int B, int threads, int sinks);
// Workgroups of the decode kernel that fit on one CU at once (0 on error).
int decode_blocks_per_cu(int path, int rows_per_tile, int head_dim, bool bf16, bool page_pow2,
                         size_t lds_bytes);

}  // namespace pkvd
