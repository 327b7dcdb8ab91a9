// prefill_args.h -- launch arguments of the context-attention (prefill)
// kernel, shared by the host (prefill_api.cpp) and the kernel
// (prefill_kernel.hip).  Internal; not part of the C ABI.
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
  // grid: a workgroup takes hpw query heads of one kv head (a head group)
  // times tt query tokens; items run over (token tile, request, kv head,
  // head group), token tiles from the last to the first
  int32_t hpw;                 // query heads per workgroup (divides g)
  int32_t tt;                  // query tokens per workgroup
  int32_t groups;              // B * Hkv * (g / hpw)
  int32_t m_tiles;             // token tiles: ceil(Sq / tt)
  int32_t items;               // m_tiles * groups
  int32_t safe_grid;           // workgroups of the rescaling kernel (<= items)
};

// Query heads and tokens per workgroup for a head_dim and GQA group size g:
// *hpw = the largest power of two dividing both g and the workgroup's number
// of 16-row tiles, *tt = its rows / *hpw (a multiple of 16).  Returns false
// for an unsupported head_dim.
bool prefill_geometry(int head_dim, int g, int* hpw, int* tt);
// Launch (prefill_kernel.hip).  Returns the hipError_t of the launch.
hipError_t launch_prefill(const PrefillArgs& a, bool bf16, hipStream_t stream);

}  // namespace pkvd
