// decode_common.h -- device helpers shared by the VALU and MFMA decode kernels:
// element formats, wavefront primitives, the key range of a request, the
// per-workgroup page list, and the split epilogue that merges partial
// attention states with the base-2 LSE rule.
//
// Reference semantics: flashinfer.cudnn.cudnn_batch_decode_with_kv_cache
// (Parameters: q_len_per_req, window_left, sinks; Note: LSE convention).
#pragma once

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "decode_args.h"
#include "schedule.h"

namespace pkvd {
namespace dev {

constexpr float kTau = 8.0f;          // lazy-rescale threshold, base-2 units
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes: 8 bf16/fp16 values

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// read of K/V page data, used once per call
#ifndef PKVD_NT_LOADS
#define PKVD_NT_LOADS 1
#endif
__device__ __forceinline__ u32x4 load16_stream(const uint16_t* p) {
#if PKVD_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

// Device-coherent scalar accesses for data exchanged between workgroups of one
// launch (split partials).  Agent-scope relaxed atomics compile to plain
// loads/stores that bypass the per-XCD L2 (sc1), so no L2 write-back or
// invalidate is needed around the exchange.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_coherent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Instrumented builds (-DPKVD_TRACE) stamp the 100 MHz real-time counter at
// numbered points of each wave; normal builds compile these away.
#ifdef PKVD_TRACE
#define PKVD_STAMP(a, gw, k)                                                      \
  do {                                                                            \
    if ((a).trace && __lane_id() == 0)                                            \
      (a).trace[(int64_t)(gw) * 16 + (k)] = __builtin_amdgcn_s_memrealtime();     \
  } while (0)
#define PKVD_COUNT(a, gw, k, v)                                                   \
  do {                                                                            \
    if ((a).trace && __lane_id() == 0) (a).trace[(int64_t)(gw) * 16 + (k)] = (v); \
  } while (0)
#else
#define PKVD_STAMP(a, gw, k) ((void)0)
#define PKVD_COUNT(a, gw, k, v) ((void)0)
#endif

// ---------------------------------------------------------------------------
// element formats (storage: 16-bit patterns in uint16/uint32 words)
// ---------------------------------------------------------------------------
template <bool BF16>
struct Fmt;

template <>
struct Fmt<true> {
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  }
  static __device__ __forceinline__ float lo(uint32_t u) { return __uint_as_float(u << 16); }
  static __device__ __forceinline__ float hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
  static __device__ __forceinline__ uint16_t encode(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);   // round to nearest even
  }
  // (a, b) rounded to nearest even and packed, a in the low half
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
  }
};

template <>
struct Fmt<false> {
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
  }
  static __device__ __forceinline__ float lo(uint32_t u) {
    return (float)__builtin_bit_cast(f16x2_t, u).x;
  }
  static __device__ __forceinline__ float hi(uint32_t u) {
    return (float)__builtin_bit_cast(f16x2_t, u).y;
  }
  static __device__ __forceinline__ uint16_t encode(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
  }
};

// Low halves of w0 and w1 packed (w0's in the low half), and the high halves.
__device__ __forceinline__ uint32_t pair_lo(uint32_t w0, uint32_t w1) {
  return __builtin_amdgcn_perm(w1, w0, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t w0, uint32_t w1) {
  return __builtin_amdgcn_perm(w1, w0, 0x07060302u);
}

// ---------------------------------------------------------------------------
// wavefront primitives
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7-i within each 8
constexpr int kDppRor8 = 0x128;         // lane i <- lane (i+8) mod 16 within each 16

// Sum over an aligned lane octet; every lane of the octet gets the total.
__device__ __forceinline__ float octet_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x;
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float shfl_xor(float x, int m) {
  const int lane = __lane_id();
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// The values of x held by a lane pair: lanes l and l ^ 16 (SWAP = 16) or
// l and l ^ 32 (SWAP = 32).  Both lanes of a pair receive the same (lo, hi):
// lo from the lane with the bit clear, hi from the lane with it set.
struct Pair {
  float lo, hi;
};
template <int SWAP>
__device__ __forceinline__ Pair lane_pair(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  if constexpr (SWAP == 16) {
    auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return {__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
  } else {
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return {__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Weight of a state with running max m merged under a common max M >= m.
__device__ __forceinline__ float rescale(float m, float M) {
  return m == -INFINITY ? 0.f : fast_exp2(m - M);
}

// From global memory (kernels that stage nothing).
__device__ __forceinline__ ReqRows req_rows(const DecodeArgs& a, int b) {
  if (!a.qo) return {b * a.Lq, a.Lq};
  return rows_of(a, clamp_row(a, a.qo[b]), clamp_row(a, a.qo[b + 1]), b);
}
// Final value of one output element: out = out_scale * O / (L + e^{sink})
// (Parameters / sinks, bmm2_scale) and, for d == 0, lse = M + log2 L (keys
// only).  An empty row (L = 0) gives out = 0 and lse = -inf.  M and L are in
// base-2 units (Note / LSE convention).
// `sink` is the row's sink logit (sinks[h], unscaled) when has_sink.
__device__ __forceinline__ float final_value(bool has_sink, float sink, float M, float L,
                                             float O, float out_scale) {
  if (!(L > 0.f)) return 0.f;
  float Z = L;
  if (has_sink) Z += fast_exp2(sink * kLog2e - M);
  return O * (out_scale / Z);
}

// Stores N consecutive output elements (N even) at element offset `off` of
// out in the call's output type (bf16 / fp16 rounded to nearest even, or
// fp32).  The type is uniform over the launch.
template <int N>
__device__ __forceinline__ void store_out(const DecodeArgs& a, int64_t off, const float (&x)[N]) {
  if (a.out_type == kOutF32) {
    float* p = static_cast<float*>(a.out) + off;
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int u = 0; u < N / 4; ++u)
        reinterpret_cast<float4*>(p)[u] = make_float4(x[4 * u], x[4 * u + 1], x[4 * u + 2], x[4 * u + 3]);
    } else {
#pragma unroll
      for (int u = 0; u < N / 2; ++u) reinterpret_cast<float2*>(p)[u] = make_float2(x[2 * u], x[2 * u + 1]);
    }
    return;
  }
  uint32_t w[N / 2];
  if (a.out_type == kOutBf16) {
#pragma unroll
    for (int u = 0; u < N / 2; ++u) w[u] = Fmt<true>::pack2(x[2 * u], x[2 * u + 1]);
  } else {
#pragma unroll
    for (int u = 0; u < N / 2; ++u) w[u] = Fmt<false>::pack2(x[2 * u], x[2 * u + 1]);
  }
  uint16_t* p = static_cast<uint16_t*>(a.out) + off;
  if constexpr (N == 8) {
    *reinterpret_cast<u32x4*>(p) = u32x4{w[0], w[1], w[2], w[3]};
  } else if constexpr (N == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int u = 0; u < N / 2; ++u) reinterpret_cast<uint32_t*>(p)[u] = w[u];
  }
}

// The slices divide a virtual block space in which every unit with blocks
// is preceded by seg_cost virtual blocks that are never streamed: a wave
// whose slice starts a unit (a segment switch: epilogue, new Q rows, a
// refilled load ring) gets that many fewer real blocks.  Unit u of request b
// starts at real block pref[b] + u nblk(b) and virtual block
// vpref[b] + u (nblk(b) + seg_cost); its real blocks sit at virtual offsets
// seg_cost .. seg_cost + nblk(b) - 1.  With seg_cost = 0 both spaces agree.
// Request b holds Hkv * tiles(b) units, tiles(b) = its row tiles.
struct Prefix {
  int T;    // real blocks
  int TV;   // virtual blocks
};

// The staged per-request facts, read back from LDS with a wave-uniform b.
struct ReqInfo {
  ReqRows rows;
  UnitRange u;
  int units;   // Hkv * row tiles
};
__device__ __forceinline__ ReqInfo req_info(const DecodeArgs& a, const int* s_nlen,
                                            const int* s_qo, int b) {
  ReqInfo r;
  const int c0 = a.qo ? __builtin_amdgcn_readfirstlane(s_qo[b]) : 0;
  const int c1 = a.qo ? __builtin_amdgcn_readfirstlane(s_qo[b + 1]) : 0;
  r.rows = rows_of(a, c0, c1, b);
  r.u = unit_range_n(a, __builtin_amdgcn_readfirstlane(s_nlen[b]), r.rows.lq);
  r.units = a.qo ? a.Hkv * tiles_of(a, r.rows.lq) : a.Hkv * a.row_tiles;
  return r;
}

// Zeroes the output rows (and sets the LSE of) a request that has query rows
// but no visible key: out = 0, lse = -inf.
__device__ __forceinline__ void write_empty_request(const DecodeArgs& a, ReqRows rr) {
  for (int r = rr.row0; r < rr.row0 + rr.lq; ++r)
    for (int h = 0; h < a.Hq; ++h) {
      const int64_t rowhead = (int64_t)r * a.Hq + h;
      if (a.out_type == kOutF32) {
        for (int d = 0; d < a.D; ++d) static_cast<float*>(a.out)[rowhead * a.D + d] = 0.f;
      } else {
        for (int d = 0; d < a.D; ++d) static_cast<uint16_t*>(a.out)[rowhead * a.D + d] = 0;
      }
      if (a.lse) a.lse[rowhead] = -INFINITY;
    }
}

// Builds pref[0..B], vpref[0..B], the raw lengths nlen[0..B-1], the blocks
// per unit nb[0..B-1], (packed rows)
// the clamped query offsets qo[0..B] and (when staged) the sink logits in
// LDS (one workgroup, ends with a barrier).  Requests with query rows but no
// visible key get out = 0, lse = -inf here, written by workgroup b % gridDim.x.
template <int NT>
__device__ __forceinline__ Prefix build_prefix(const DecodeArgs& a, int* s_pref, int* s_vpref,
                                               int* s_nlen, int* s_nb, int* s_qo, int* s_scan,
                                               int* s_vscan, float* s_sink) {
  const int B = a.B;
  const int CH = (B + NT - 1) / NT;
  const int t = threadIdx.x;
  const int lo = min(B, t * CH), hi = min(B, lo + CH);
  int sum = 0, vsum = 0;
  int c_next = (a.qo && lo < hi) ? clamp_row(a, a.qo[lo]) : 0;
  for (int b = lo; b < hi; ++b) {
    const int nraw = a.seq_lens[b];
    s_nlen[b] = nraw;
    int c0 = 0, c1 = 0;
    if (a.qo) {
      c0 = c_next;
      c1 = clamp_row(a, a.qo[b + 1]);
      c_next = c1;
      s_qo[b] = c0;
      if (b + 1 == B) s_qo[B] = c1;
    }
    int nb, units;
    const ReqRows rr = req_blocks(a, b, nraw, c0, c1, nb, units);
    s_nb[b] = nb;
    sum += nb * units;
    vsum += unit_vspan(a, nb) * units;
    if (nb == 0 && rr.lq > 0 && b % (int)gridDim.x == (int)blockIdx.x) write_empty_request(a, rr);
  }
  if (a.sinks)
    for (int h = t; h < a.Hq; h += NT) s_sink[h] = a.sinks[h];
  // inclusive scans: within each wave by lane shuffles, then across the
  // NT / 64 wave totals (two barriers in all)
  const int lane = t & 63, wv = t >> 6;
  int x = sum, vx = vsum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o), vy = __shfl_up(vx, o);
    if (lane >= o) {
      x += y;
      vx += vy;
    }
  }
  if (lane == 63) {
    s_scan[wv] = x;
    s_vscan[wv] = vx;
  }
  __syncthreads();
  int base = 0, vbase = 0;
  for (int w = 0; w < wv; ++w) {
    base += s_scan[w];
    vbase += s_vscan[w];
  }
  int excl = base + x - sum, vexcl = vbase + vx - vsum;
  for (int b = lo; b < hi; ++b) {
    s_pref[b] = excl;
    s_vpref[b] = vexcl;
    int nb, units;   // this thread's own LDS writes: no barrier needed
    req_blocks(a, b, s_nlen[b], a.qo ? s_qo[b] : 0, a.qo ? s_qo[b + 1] : 0, nb, units);
    excl += nb * units;
    vexcl += unit_vspan(a, nb) * units;
  }
  if (t == NT - 1) {
    s_pref[B] = base + x;
    s_vpref[B] = vbase + vx;
  }
  __syncthreads();
  Prefix p;
  p.T = s_pref[B];
  p.TV = s_vpref[B];
  return p;
}

// Largest b with pref[b] <= pos (the request holding linear block pos), for
// a nondecreasing pref with pref[0] <= pos.  A 64-way search: each lane
// reads one sample of the range and a ballot picks the last sample <= pos,
// so B <= 64 takes one LDS read (a binary search takes log2 B dependent
// reads).  Called by all lanes of a wave with a wave-uniform pos.
__device__ __forceinline__ int find_request(const int* s_pref, int B, int pos) {
  const int lane = __lane_id();
  int base = 0, span = B;   // the answer lies in [base, base + span)
  while (span > 64) {
    const int stride = (span + 63) >> 6;
    const int idx = base + lane * stride;
    const bool ok = idx < base + span && s_pref[idx] <= pos;
    const uint64_t m = __builtin_amdgcn_ballot_w64(ok);   // lane 0 is always set
    const int k = 63 - __builtin_clzll(m);
    const int nb = base + k * stride;
    span = min(stride, base + span - nb);
    base = nb;
  }
  const bool ok = lane < span && s_pref[base + lane] <= pos;
  const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
  return base + (63 - __builtin_clzll(m));
}

// find_request for two positions at once (one LDS read per lane when B <= 64).
__device__ __forceinline__ void find_request2(const int* s_pref, int B, int p0, int p1, int& b0,
                                              int& b1) {
  if (B > 64) {
    b0 = find_request(s_pref, B, p0);
    b1 = find_request(s_pref, B, p1);
    return;
  }
  const int lane = __lane_id();
  const int x = lane < B ? s_pref[lane] : 0;
  const uint64_t m0 = __builtin_amdgcn_ballot_w64(lane < B && x <= p0);
  const uint64_t m1 = __builtin_amdgcn_ballot_w64(lane < B && x <= p1);
  b0 = 63 - __builtin_clzll(m0);
  b1 = 63 - __builtin_clzll(m1);
}

// A unit's slice of one wave's range.
struct Segment {
  int b, kvh, tile;
  UnitRange u;
  int row0, lq, R;           // the request's query rows, and R = g * lq live rows
  int blk_begin, blk_end;    // absolute 16-key blocks [blk_begin, blk_end)
  int ustart, uend;          // the unit's linear block range (the block space fits int32)
  int vstart;                // the unit's first virtual block
  int whole;                 // the range holds the entire unit (int: stays in registers)
  int side;                  // 0: first segment of the wave, 1: a later one
};

// The segment from real block pos of request b (real and virtual prefixes
// pref_b, vpref_b), unit uidx of the request, within the wave's range
// [wave_lo, wave_hi).
__device__ __forceinline__ Segment segment_at(const DecodeArgs& a, const int* s_nlen,
                                              const int* s_qo, int b, int pref_b, int vpref_b,
                                              int uidx, int pos, int wave_lo, int wave_hi) {
  Segment g;
  g.b = b;
  const ReqInfo ri = req_info(a, s_nlen, s_qo, b);
  g.u = ri.u;
  g.row0 = ri.rows.row0;
  g.lq = ri.rows.lq;
  g.R = a.g * g.lq;
  const int nb = g.u.nblk > 0 ? g.u.nblk : 1;   // pos lies in a unit with blocks
  const int per_req = ri.units > 0 ? ri.units : 1;
  int tiles = a.qo ? tiles_of(a, g.lq) : a.row_tiles;
  tiles = tiles > 0 ? tiles : 1;
  uidx = uidx < 0 ? 0 : (uidx >= per_req ? per_req - 1 : uidx);
  g.kvh = tiles == 1 ? uidx : uidx / tiles;
  g.tile = uidx - g.kvh * tiles;
  g.ustart = pref_b + uidx * nb;
  g.uend = g.ustart + nb;
  g.vstart = vpref_b + uidx * unit_vspan(a, nb);
  const int seg_end = wave_hi < g.uend ? wave_hi : g.uend;
  g.blk_begin = g.u.first_blk + (pos - g.ustart);
  g.blk_end = g.blk_begin + (seg_end - pos);
  g.whole = pos == g.ustart && seg_end == g.uend;
  g.side = pos == wave_lo ? 0 : 1;
  return g;
}

// The segment that starts at real block pos.
__device__ __forceinline__ Segment locate(const DecodeArgs& a, const int* s_pref,
                                          const int* s_vpref, const int* s_nlen, const int* s_nb,
                                          const int* s_qo, int pos, int wave_lo, int wave_hi) {
  const int b = find_request(s_pref, a.B, pos);
  const int pref_b = __builtin_amdgcn_readfirstlane(s_pref[b]);
  const int vpref_b = __builtin_amdgcn_readfirstlane(s_vpref[b]);
  int nb = __builtin_amdgcn_readfirstlane(s_nb[b]);
  nb = nb > 0 ? nb : 1;
  return segment_at(a, s_nlen, s_qo, b, pref_b, vpref_b, (pos - pref_b) / nb, pos, wave_lo,
                    wave_hi);
}

// ---------------------------------------------------------------------------
// page ids of a chunk
// ---------------------------------------------------------------------------
// Page ids of a chunk's block-table columns col0 .. col0 + 127, one column per
// lane in each of two registers, as loaded.  They are clamped into the pool
// [0, plast] where a page is taken from the window, not when the window is
// fetched: a clamp at the fetch would make the wave wait for the block-table
// load there (and so for every load issued before it), a full memory round
// trip at each chunk set-up.
struct PageWindow {
  int p0, p1;   // columns col0 + lane, col0 + 64 + lane (unclamped)
  int col0;
  int plast;    // last page of the pool
};

__device__ __forceinline__ int clamp_page(const PageWindow& w, int p) {
  return (unsigned)p <= (unsigned)w.plast ? p : w.plast;
}
// Page of column col0 + c for a wave-uniform c.
__device__ __forceinline__ int page_uniform(const PageWindow& w, int c) {
  return clamp_page(w, __builtin_amdgcn_readlane(c < 64 ? w.p0 : w.p1, c & 63));
}
// Page of column col0 + c for a per-lane c.
__device__ __forceinline__ int page_lane(const PageWindow& w, int c) {
  const int a0 = __builtin_amdgcn_ds_bpermute((c & 63) << 2, w.p0);
  const int a1 = __builtin_amdgcn_ds_bpermute((c & 63) << 2, w.p1);
  return clamp_page(w, c < 64 ? a0 : a1);
}

}  // namespace dev
}  // namespace pkvd
