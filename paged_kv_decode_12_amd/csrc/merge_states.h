// merge_states.h -- arguments and launcher of the cascade merge kernel
// (merge_states.hip).  Shared by the kernel and the C ABI (api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkvd {

struct MergeArgs {
  const void* v;        // (S, items, D) partial outputs, contiguous, bf16/fp16/fp32
  const float* s;       // (S, items) base-2 LSEs
  const float* sinks;   // (H,) sink logits or nullptr
  void* v_out;          // (items, D), v's dtype
  float* s_out;         // (items,) or nullptr
  int64_t S;            // states per (row, head)
  int64_t items;        // rows * H
  int32_t H;
  int32_t D;
};

// dtype: 0 bf16, 1 fp16, 2 fp32.  Returns the launch's hipError_t.
hipError_t launch_merge_states(const MergeArgs& a, int dtype, hipStream_t stream);

}  // namespace pkvd
