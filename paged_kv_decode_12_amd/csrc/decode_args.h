// decode_args.h -- launch arguments shared by the host planner (api.cpp) and
// the device kernels (decode_kernels.hip).  Internal; not part of the C ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace pkvd {

constexpr int kBlockKeys = 16;   // keys per block: the unit a wave loads and scores
constexpr int kWaves = 4;        // waves per workgroup of the decode kernels
constexpr int kThreads = 64 * kWaves;
constexpr int kWavePages = 512;        // block-table columns one wave stages in LDS at a time
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
  float* ws_o;                     // partial states [2 * num_waves][rows_per_tile * D], order set by the engine
  float* ws_lse;                   // [2 * num_waves][rows_per_tile]
  int32_t* counters;               // [B * Hkv * row_tiles] arrival tickets, zero between calls
  // shapes
  int32_t B, Hq, Hkv, g, Lq, ps, P, C, D;
  int32_t window_left;
  float scale_log2;                // scale * log2(e): scores are kept in base 2
  int32_t row_tiles;               // row tiles per (request, kv head)
  int32_t num_waves;               // waves of the persistent grid (4 per workgroup)
  int32_t min_wave_blocks;         // a wave gets at least this many blocks (fewer waves run)
#ifdef PKVD_TRACE
  uint64_t* trace;                 // instrumented builds only: [waves][16] timestamps
#endif
};

// Launchers (decode_valu.hip).  Return the hipError_t of the launch.
hipError_t launch_decode(const DecodeArgs& a, int path, int rows_per_tile, bool bf16,
                         hipStream_t stream);
// Dynamic LDS bytes of a launch for B requests.
size_t decode_lds_bytes(int B, int path, int head_dim);
// Workgroups of the decode kernel that fit on one CU at once (0 on error).
int decode_blocks_per_cu(int path, int rows_per_tile, int head_dim, bool bf16, bool page_pow2,
                         size_t lds_bytes);

}  // namespace pkvd
