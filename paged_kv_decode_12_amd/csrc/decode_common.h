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

// ---------------------------------------------------------------------------
// key range of one request
// ---------------------------------------------------------------------------
// Keys some row of request b may see: [lo(row 0), n - 1], where row 0 has the
// lowest diagonal n - Lq (Parameters / q_len_per_req) and the window keeps
// window_left keys before the diagonal (Parameters / window_left).  The range
// is cut into 16-key blocks aligned to the absolute key index; the waves'
// slices are runs of these blocks.
struct UnitRange {
  int n;          // sequence length, clamped to the block table's capacity
  int key_lo;     // first key some row sees
  int first_blk;  // block holding key_lo
  int nblk;       // blocks covering [key_lo, n)
};

__device__ __forceinline__ UnitRange unit_range_n(const DecodeArgs& a, int n_raw) {
  UnitRange u;
  const int cap = a.C * a.ps;
  const int n = n_raw < 0 ? 0 : (n_raw > cap ? cap : n_raw);
  u.n = n;
  const int lo = (a.window_left < 0) ? 0 : n - a.Lq - a.window_left;
  u.key_lo = lo < 0 ? 0 : lo;
  if (u.key_lo >= n) {
    u.first_blk = 0;
    u.nblk = 0;
  } else {
    u.first_blk = u.key_lo / kBlockKeys;
    u.nblk = (n - 1) / kBlockKeys - u.first_blk + 1;
  }
  return u;
}

__device__ __forceinline__ UnitRange unit_range(const DecodeArgs& a, int b) {
  return unit_range_n(a, a.seq_lens[b]);
}

// Final value of one output element: out = O / (L + e^{sink}) and, for d == 0,
// lse = M + log2 L (keys only).  An empty row (L = 0) gives out = 0 and
// lse = -inf.  M and L are in base-2 units (Parameters / sinks; Note / LSE
// convention).
// `sink` is the row's sink logit (sinks[h], unscaled) when has_sink.
template <bool BF16>
__device__ __forceinline__ float final_value(bool has_sink, float sink, float M, float L,
                                             float O) {
  if (!(L > 0.f)) return 0.f;
  float Z = L;
  if (has_sink) Z += fast_exp2(sink * kLog2e - M);
  return O / Z;
}

// floor(n / d) for 0 <= n < 2^62, 0 < d < 2^62, and a quotient below 2^31.
// The fp64 quotient has a relative error of about 2^-52 (the rounding of n
// and of the division), so it is within one of the true quotient; integer
// corrections make it exact.  About a tenth of the instructions of a generic
// 64-bit integer division, which matters in the prologue every wave runs.
__device__ __forceinline__ int64_t qdiv(int64_t n, int64_t d) {
  int64_t q = (int)((double)n / (double)d);
  int64_t r = n - q * d;
  if (r < 0) { --q; r += d; }
  if (r < 0) { --q; r += d; }
  if (r >= d) { ++q; r -= d; }
  if (r >= d) ++q;
  return q;
}

// ---------------------------------------------------------------------------
// balanced persistent schedule
// ---------------------------------------------------------------------------
// The work is the linear block space [0, T) of all units (request b, kv head,
// row tile) in that order: request b owns blocks [pref[b], pref[b + 1]) and
// each of its Hkv * row_tiles units holds nblk(b) consecutive blocks.  The
// NW waves split it into consecutive slices, wave w's in proportion to its
// weight.  Waves are numbered group by group, PER = ceil(NW / groups) per
// group, and a group's wave i runs on SIMD i % 4 as the (i / 4)-th wave
// there; W[s] is the weight of the waves at position s = min(i / 4, 3) on
// their SIMD.  (Of two waves sharing a SIMD the first issues ahead of the
// second and streams faster, so it may be given more blocks.)  Equal weights
// give [w T / NW, (w + 1) T / NW): every wave streams the same number of
// blocks (to within one) whatever the mix of sequence lengths.  The slice
// sizes never depend on the lengths, only on T.
struct Slices {
  int T, NW;
  int uniform;   // all weights in use equal: closed forms
  int PER;       // waves per group
  int W[4];
  int64_t SP;    // total weight of one group's PER waves
  int64_t S;     // total weight of the NW waves
  int n_min;     // blocks of the shortest slice (a lower bound)
};
// Total weight of the first m waves of a group (0 <= m <= PER).
__device__ __forceinline__ int64_t group_weight(const Slices& s, int m) {
  int64_t acc = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int lo = r * kSimdsPerCu;
    int n = m - lo;
    n = n < 0 ? 0 : (r < 3 && n > kSimdsPerCu ? kSimdsPerCu : n);
    acc += (int64_t)n * s.W[r];
  }
  return acc;
}
// Total weight of waves [0, w).
__device__ __forceinline__ int64_t weight_before(const Slices& s, int w) {
  const int full = w / s.PER;
  return (int64_t)full * s.SP + group_weight(s, w - full * s.PER);
}
__device__ __forceinline__ Slices make_slices(const DecodeArgs& a, int T, int NW) {
  Slices s;
  s.T = T;
  s.NW = NW;
  const int groups = a.groups > 0 ? a.groups : 1;
  s.PER = (NW + groups - 1) / groups;
  int wmin = 1 << 30;
  s.uniform = 1;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s.W[r] = a.slot_w[r];
    if (r * kSimdsPerCu < s.PER) {
      if (s.W[r] != s.W[0]) s.uniform = 0;
      if (s.W[r] < wmin) wmin = s.W[r];
    }
  }
  s.SP = group_weight(s, s.PER);
  s.S = weight_before(s, NW);
  s.n_min = s.uniform ? T / NW : (int)qdiv((int64_t)T * wmin, s.S);
  return s;
}
// First block of wave w's slice (w <= NW).
__device__ __forceinline__ int slice_begin(const Slices& s, int w) {
  if (s.uniform) return (int)qdiv((int64_t)s.T * w, s.NW);
  return (int)qdiv((int64_t)s.T * weight_before(s, w), s.S);
}
// The wave whose slice holds block x (0 <= x < T): the largest w with
// slice_begin(w) <= x, i.e. with weight_before(w) <= ((x + 1) S - 1) / T.
// That weight is inverted in closed form: whole groups first, then the
// group's waves slot by slot (weights are positive).
__device__ __forceinline__ int slice_of(const Slices& s, int64_t x) {
  if (s.uniform) return (int)qdiv((x + 1) * s.NW - 1, s.T);
  const int64_t target = qdiv((x + 1) * s.S - 1, s.T);
  const int64_t full = qdiv(target, s.SP);
  int64_t rem = target - full * s.SP;
  int m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int lo = r * kSimdsPerCu;
    int cap = s.PER - lo;
    cap = cap < 0 ? 0 : (r < 3 && cap > kSimdsPerCu ? kSimdsPerCu : cap);
    int64_t n = rem / s.W[r];
    n = n > cap ? cap : n;
    if (m == lo) {   // earlier slots full: this slot's waves follow
      m += (int)n;
      rem -= n * s.W[r];
    }
  }
  const int64_t w = full * s.PER + m;
  return (int)(w < s.NW - 1 ? w : s.NW - 1);
}

// Where the partial states of a cut unit are.  Wave w writes the partial
// state of each unit its slice cuts into slot 2 w + side: side 0 for the
// slice's first segment, 1 for its last (a slice cuts at most those two).
// Slices are taken in the virtual block space: the unit starts at virtual
// block vs and its real blocks sit at [vs + seg_cost, vs + seg_cost + nblk).
// The candidates are the waves w0 .. w1 whose slices hold those blocks; wave
// w's piece is its first segment exactly when its slice starts at or after
// vs (a slice that starts among the unit's virtual blocks starts at the
// unit's first real block).  Every candidate with a non-empty slice holds
// real blocks of the unit and wrote a partial state; a unit with a single
// non-empty candidate was whole in that slice and written directly.
struct UnitPieces {
  int w0;      // first wave holding a block of the unit
  int n;       // candidates: waves w0 .. w0 + n - 1
};
__device__ __forceinline__ UnitPieces unit_pieces(const Slices& s, int64_t vs, int seg_cost,
                                                  int nblk) {
  UnitPieces p;
  p.w0 = slice_of(s, vs + seg_cost);
  p.n = slice_of(s, vs + seg_cost + nblk - 1) - p.w0 + 1;
  return p;
}
// Slot of candidate c, and whether it holds a partial state of this call.
__device__ __forceinline__ int candidate_slot(const UnitPieces& p, const Slices& s, int64_t vs,
                                              int c, bool& written) {
  const int w = p.w0 + c;
  const int b0 = slice_begin(s, w);
  written = b0 < slice_begin(s, w + 1);
  return 2 * w + (b0 >= vs ? 0 : 1);
}

// Waves that take part: at most one per min_wave_blocks blocks, and >= 1.
__device__ __forceinline__ int wave_count(const DecodeArgs& a, int T) {
  int nw = T / a.min_wave_blocks;
  return nw < 1 ? 1 : (nw > a.num_waves ? a.num_waves : nw);
}

// Dynamic LDS of a workgroup of NT threads, in 32-bit words: the scan scratch (NT),
// the prefix (B + 1) and the raw lengths (B).  Host (launch size) and kernel
// (carve-up) both take the offsets from here.
struct LdsLayout {
  int scan, vscan, pref, vpref, nlen, sink, total;
};
// NS: sink logits staged in LDS (Hq when they are, else 0).
__host__ __device__ inline LdsLayout lds_layout(int B, int NT, int NS) {
  LdsLayout l;
  l.scan = 0;
  l.vscan = l.scan + NT;
  l.pref = l.vscan + NT;
  l.vpref = l.pref + B + 1;
  l.nlen = l.vpref + B + 1;
  l.sink = l.nlen + B;
  l.total = l.sink + NS;
  return l;
}

// The slices divide a virtual block space in which every unit with blocks
// is preceded by seg_cost virtual blocks that are never streamed: a wave
// whose slice starts a unit (a segment switch: epilogue, new Q rows, a
// refilled load ring) gets that many fewer real blocks.  Unit u of request b
// starts at real block pref[b] + u nblk(b) and virtual block
// vpref[b] + u (nblk(b) + seg_cost); its real blocks sit at virtual offsets
// seg_cost .. seg_cost + nblk(b) - 1.  With seg_cost = 0 both spaces agree.
struct Prefix {
  int T;    // real blocks
  int TV;   // virtual blocks
};

// Builds pref[0..B], vpref[0..B], the raw lengths nlen[0..B-1] and (when
// staged) the sink logits in LDS (one workgroup, ends with a barrier).  Requests with no visible key get
// out = 0, lse = -inf here, written by workgroup b % gridDim.x.
template <bool BF16, int NT>
__device__ __forceinline__ Prefix build_prefix(const DecodeArgs& a, int* s_pref, int* s_vpref,
                                               int* s_nlen, int* s_scan, int* s_vscan,
                                               float* s_sink) {
  const int B = a.B;
  const int per_req = a.Hkv * a.row_tiles;
  const int c = a.seg_cost;
  const int CH = (B + NT - 1) / NT;
  const int t = threadIdx.x;
  const int lo = min(B, t * CH), hi = min(B, lo + CH);
  int sum = 0, vsum = 0;
  for (int b = lo; b < hi; ++b) {
    const int nraw = a.seq_lens[b];
    s_nlen[b] = nraw;
    const int nb = unit_range_n(a, nraw).nblk;
    sum += nb * per_req;
    vsum += (nb > 0 ? nb + c : 0) * per_req;
    if (nb == 0 && b % (int)gridDim.x == (int)blockIdx.x) {
      for (int r = b * a.Lq; r < (b + 1) * a.Lq; ++r)
        for (int h = 0; h < a.Hq; ++h) {
          const int rowhead = r * a.Hq + h;
          for (int d = 0; d < a.D; ++d) a.out[(int64_t)rowhead * a.D + d] = 0;
          if (a.lse) a.lse[rowhead] = -INFINITY;
        }
    }
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
    const int nb = unit_range_n(a, s_nlen[b]).nblk;
    excl += nb * per_req;
    vexcl += (nb > 0 ? nb + c : 0) * per_req;
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

// A unit's slice of one wave's range.
struct Segment {
  int b, kvh, tile;
  UnitRange u;
  int blk_begin, blk_end;    // absolute 16-key blocks [blk_begin, blk_end)
  int ustart, uend;          // the unit's linear block range (the block space fits int32)
  int vstart;                // the unit's first virtual block
  int whole;                 // the range holds the entire unit (int: stays in registers)
  int side;                  // 0: first segment of the wave, 1: a later one
};

__device__ __forceinline__ Segment locate(const DecodeArgs& a, const int* s_pref,
                                          const int* s_vpref, const int* s_nlen, int pos,
                                          int wave_lo, int wave_hi) {
  Segment g;
  g.b = find_request(s_pref, a.B, pos);
  g.u = unit_range_n(a, __builtin_amdgcn_readfirstlane(s_nlen[g.b]));
  const int pref_b = __builtin_amdgcn_readfirstlane(s_pref[g.b]);
  const int vpref_b = __builtin_amdgcn_readfirstlane(s_vpref[g.b]);
  const int nb = g.u.nblk > 0 ? g.u.nblk : 1;   // pos lies in a unit with blocks
  const int off = pos - pref_b;
  const int per_req = a.Hkv * a.row_tiles;
  int uidx = off / nb;
  uidx = uidx < 0 ? 0 : (uidx >= per_req ? per_req - 1 : uidx);
  g.kvh = uidx / a.row_tiles;
  g.tile = uidx - g.kvh * a.row_tiles;
  g.ustart = pref_b + uidx * nb;
  g.uend = g.ustart + nb;
  g.vstart = vpref_b + uidx * (nb + a.seg_cost);
  const int seg_end = wave_hi < g.uend ? wave_hi : g.uend;
  g.blk_begin = g.u.first_blk + (pos - g.ustart);
  g.blk_end = g.blk_begin + (seg_end - pos);
  g.whole = pos == g.ustart && seg_end == g.uend;
  g.side = pos == wave_lo ? 0 : 1;
  return g;
}

// The real block at virtual block v (0 <= v <= TV): the unit's first real
// block for its virtual blocks, T at the end.
__device__ __forceinline__ int real_of(const DecodeArgs& a, const int* s_pref, const int* s_vpref,
                                       const int* s_nlen, const Prefix& p, int v) {
  if (v >= p.TV) return p.T;
  const int b = find_request(s_vpref, a.B, v);   // a request with blocks
  const int nb = unit_range_n(a, __builtin_amdgcn_readfirstlane(s_nlen[b])).nblk;
  const int vu = nb + a.seg_cost;
  const int off = v - __builtin_amdgcn_readfirstlane(s_vpref[b]);
  const int ul = off / vu;
  const int o = off - ul * vu - a.seg_cost;
  return __builtin_amdgcn_readfirstlane(s_pref[b]) + ul * nb + (o > 0 ? o : 0);
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
