// merge_states.hip -- the cascade merge of partial attention states.
//
// S states of the same (row, head), each computed over its own disjoint set
// of keys, are combined into the state over their union.  A state is a
// normalised output v_s[D] and its base-2 log-sum-exp s_s, the form the
// decode writes (flashinfer.cudnn.cudnn_batch_decode_with_kv_cache, Note /
// LSE convention: the base-2 LSE is what the cascade-merge kernels consume).
// State s weighs 2^s_s; an optional sink logit (Parameters / sinks) adds
// e^sink to the denominator only:
//   v = sum_s 2^s_s v_s / (sum_s 2^s_s + e^sink),   s = log2 sum_s 2^s_s.
// Every exponent is taken relative to the largest one.  An empty state
// (s_s = -inf) weighs 0; rows whose states are all empty give v = 0,
// s = -inf.
//
// One wave per (row, head): the lanes reduce the S LSEs (64 at a time) to
// their maximum, then each lane accumulates up to four of its dims over the
// states in order, eight states' loads in flight.  HBM-bound: S (D elt + 4)
// bytes read and D elt + 4 written per (row, head).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "merge_states.h"

namespace pkvd {
namespace {

constexpr int kMsWaves = 4;   // waves per workgroup
constexpr float kLog2eMs = 1.4426950408889634f;

__device__ __forceinline__ float ms_wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

template <int DT>
struct Elem;
template <>
struct Elem<0> {   // bf16
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    const uint32_t b = static_cast<const uint16_t*>(p)[i];
    return __uint_as_float(b << 16);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float x) {
    // round to nearest even; NaN stays NaN
    const uint32_t u = __float_as_uint(x);
    const uint32_t r = (u & 0x7fffffffu) > 0x7f800000u ? (u | 0x00400000u)
                                                       : u + 0x7fffu + ((u >> 16) & 1u);
    static_cast<uint16_t*>(p)[i] = (uint16_t)(r >> 16);
  }
};
template <>
struct Elem<1> {   // fp16
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return (float)static_cast<const _Float16*>(p)[i];
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float x) {
    static_cast<_Float16*>(p)[i] = (_Float16)x;
  }
};
template <>
struct Elem<2> {   // fp32
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float x) {
    static_cast<float*>(p)[i] = x;
  }
};

template <int DT>
__global__ __launch_bounds__(64 * kMsWaves) void merge_states_kernel(const MergeArgs a) {
  constexpr int kDl = 4;       // dims per lane per pass (256 dims per pass)
  constexpr int kDepth = 8;    // states whose loads are in flight together
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * kMsWaves + (threadIdx.x >> 6);   // row * H + head
  if (item >= a.items) return;
  const int head = (int)(item % a.H);
  const int64_t S = a.S;
  // the largest exponent: the states' LSEs and the sink (in base 2)
  float M = -INFINITY;
  for (int64_t c = lane; c < S; c += 64) M = fmaxf(M, a.s[c * a.items + item]);
  M = ms_wave_max(M);
  const bool has_sink = a.sinks != nullptr;
  const float sink2 = has_sink ? a.sinks[head] * kLog2eMs : -INFINITY;
  if (M == -INFINITY) {   // no key in any state
    for (int d = lane; d < a.D; d += 64) Elem<DT>::store(a.v_out, item * a.D + d, 0.f);
    if (a.s_out && lane == 0) a.s_out[item] = -INFINITY;
    return;
  }
  const float top = fmaxf(M, sink2);
  for (int d0 = 0; d0 < a.D; d0 += 64 * kDl) {
    // lane holds dims d0 + lane + 64 e (coalesced across the wave)
    float acc[kDl], W = 0.f;
#pragma unroll
    for (int e = 0; e < kDl; ++e) acc[e] = 0.f;
    for (int64_t s0 = 0; s0 < S; s0 += kDepth) {
      float l[kDepth], x[kDepth][kDl];
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const bool live = s0 + u < S;
        const int64_t st = live ? s0 + u : s0;   // padding entries re-read a live state
        l[u] = live ? a.s[st * a.items + item] : -INFINITY;
#pragma unroll
        for (int e = 0; e < kDl; ++e) {
          const int d = d0 + lane + 64 * e;
          x[u][e] = d < a.D ? Elem<DT>::load(a.v, (st * a.items + item) * a.D + d) : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const float w = l[u] == -INFINITY ? 0.f : exp2f(l[u] - top);
        W += w;
#pragma unroll
        for (int e = 0; e < kDl; ++e)   // select: an empty state's v is never used
          acc[e] = w == 0.f ? acc[e] : fmaf(w, x[u][e], acc[e]);
      }
    }
    const float Z = W + (has_sink ? exp2f(sink2 - top) : 0.f);
#pragma unroll
    for (int e = 0; e < kDl; ++e) {
      const int d = d0 + lane + 64 * e;
      if (d < a.D) Elem<DT>::store(a.v_out, item * a.D + d, acc[e] / Z);
    }
    if (d0 == 0 && lane == 0 && a.s_out) a.s_out[item] = top + log2f(W);
  }
}

}  // namespace

hipError_t launch_merge_states(const MergeArgs& a, int dtype, hipStream_t stream) {
  if (a.items <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.items + kMsWaves - 1) / kMsWaves));
  const dim3 block(64 * kMsWaves);
  switch (dtype) {
    case 0: hipLaunchKernelGGL(merge_states_kernel<0>, grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL(merge_states_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(merge_states_kernel<2>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkvd
