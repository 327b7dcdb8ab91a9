// prefill_args.h -- launch arguments of the context-attention (prefill)
// kernel, shared by the host (api.cpp) and the kernel (prefill_kernel.hip).
// Internal; not part of the C ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace pkvd {

enum PrefillMask : int { kPrefillCausal = 0, kPrefillDense = 1, kPrefillVariable = 2 };

struct PrefillArgs {
  // inputs (element strides; head_dim is innermost and dense)
  const uint16_t* q;
  int64_t q_sr, q_sh;          // q[row * q_sr + head * q_sh + d], row = token of the call
  const uint16_t* k;
  int64_t k_sr, k_sh;          // k[row * k_sr + kv_head * k_sh + d]
  const uint16_t* v;
  int64_t v_sr, v_sh;
  const int32_t* qo;           // nullptr: fixed rows; else (B + 1) packed query offsets
  const int32_t* kvo;          // with qo: (B + 1) packed key/value offsets
  const int32_t* starts;       // variable window: (B, Sq) inclusive first key per query
  const int32_t* ends;         //                  (B, Sq) inclusive last key per query
  // output: contiguous (rows_q, Hq, D) of out_type (0 bf16, 1 fp16, 2 fp32)
  void* out;
  int32_t out_type;
  // shapes
  int32_t B, Hq, Hkv, g, D;
  int32_t Sq, Sk;              // fixed lengths (packed: Sq = the largest query count)
  int32_t rows_q, rows_kv;     // rows of q / out and of k, v
  int32_t mask;                // PrefillMask
  int32_t window_left;         // -1: none
  float scale_log2;            // sm_scale * log2(e)
  float out_scale;             // factor on the output
  int32_t m_tiles;             // query tiles per (request, head)
  int32_t items;               // B * Hq * m_tiles
};

// Query rows per workgroup for a head_dim (the tile the grid counts).
int prefill_block_rows(int head_dim);
// Launch (prefill_kernel.hip).  Returns the hipError_t of the launch.
hipError_t launch_prefill(const PrefillArgs& a, bool bf16, hipStream_t stream);

}  // namespace pkvd
