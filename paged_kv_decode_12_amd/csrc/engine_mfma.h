// engine_mfma.h -- MFMA engine of the persistent decode kernel: 16 rows per
// tile (GQA group x query tokens filling a dense 16-row MFMA tile).
//
// Per 16-key block (matrix shapes as M x K times K x N):
//  * S^T[keys x rows] = K[keys x D] . Q^T[D x rows] with
//    v_mfma_f32_16x16x32_{bf16,f16}: lane l (j = l % 16, q = l / 16) feeds
//    key j's dims c*32 + 8q .. +8 as the A operand straight from a 16-byte
//    load of the page tile, and row j's same dims of Q as the B operand.  The
//    result gives lane l the scores of row j for keys 4q + i, i = 0..3.
//  * masks (window, causal, length) by select; the row max rises lazily
//    (only when a score exceeds it by more than kTau, base 2); when it does,
//    the exact block max of the row is taken across its four lanes.
//  * P x V with v_mfma_f32_16x16x16_{bf16,f16}: the four probabilities of
//    lane l are exactly the A operand of row j, keys 4q + e (packed to
//    bf16/fp16); the B operand of output tile t holds V[4q + e][j * DJ + t],
//    built with byte permutes from the lane's four 16-byte (D = 128) or
//    8-byte (D = 64) loads of rows 4q + e, dims j * DJ .. j * DJ + DJ - 1.
//    Output tile t therefore covers dims {j * DJ + t}, so lane l ends with
//    rows 4q + i, dims j * DJ .. j * DJ + DJ - 1 of O, all in registers.
#pragma once

#include "decode_common.h"

namespace pkvd {
namespace dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2 load8_stream(const uint16_t* p) {
#if PKVD_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
#else
  return *reinterpret_cast<const u32x2*>(p);
#endif
}

// K rows are read 64 bytes per key per instruction (16 keys per MFMA operand),
// so each 128-byte line is touched by two instructions in a row
#ifndef PKVD_MFMA_K_NT
#define PKVD_MFMA_K_NT 1
#endif
__device__ __forceinline__ u32x4 load16_k(const uint16_t* p) {
#if PKVD_MFMA_K_NT
  return load16_stream(p);
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

template <bool BF16>
struct Mfma;

template <>
struct Mfma<true> {
  static __device__ __forceinline__ f32x4_t qk(const u32x4& a, const u32x4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(const u32x2& a, const u32x2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                     __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<false> {
  static __device__ __forceinline__ f32x4_t qk(const u32x4& a, const u32x4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(const u32x2& a, const u32x2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
};

template <int D>
struct VRow;
template <>
struct VRow<128> {
  using T = u32x4;   // 8 dims
  static __device__ __forceinline__ T load(const uint16_t* p) { return load16_stream(p); }
  static __device__ __forceinline__ uint32_t word(const T& v, int u) { return v[u]; }
};
template <>
struct VRow<64> {
  using T = u32x2;   // 4 dims
  static __device__ __forceinline__ T load(const uint16_t* p) { return load8_stream(p); }
  static __device__ __forceinline__ uint32_t word(const T& v, int u) { return v[u]; }
};

template <int D, bool BF16>
struct MfmaEngine {
  static constexpr int kRows = 16;
  static constexpr int kKeysPerGroup = kBlockKeys;
  static constexpr int kGroupsPerBlock = 1;
  static constexpr int NC = D / 32;          // 32-dim chunks of q . k
  static constexpr int DJ = D / 16;          // output dims per lane (= P x V tiles)
  static constexpr int kItems = 4;           // rows 4q + i
  static constexpr int kItemDims = DJ;
  static constexpr int kItemLanes = 16;

  struct Lane {
    int j, q, lane;
  };
  struct Q {
    u32x4 c[NC];   // row j, dims c*32 + 8q .. +8
  };
  struct Buf {
    u32x4 k[NC];                      // key j, dims c*32 + 8q .. +8
    typename VRow<D>::T v[4];         // key 4q + e, dims j*DJ .. +DJ
  };
  struct State {
    f32x4_t acc[DJ];   // acc[t][i]: row 4q + i, dim j*DJ + t
    float m, l;        // row j: running max (uniform over its 4 lanes), lane's partial sum
    int lo, hi;        // row j's visible keys
  };

  static __device__ __forceinline__ Lane lane_of(int lane) { return {lane & 15, lane >> 4, lane}; }

  static __device__ __forceinline__ void fetch_q(const DecodeArgs& a, const Segment& sg,
                                                 const Lane& ln, Q& q) {
    const int rr = sg.tile * kRows + ln.j;
    const bool live = rr < sg.R;
    const int i = live ? rr / a.g : 0;
    const int hl = live ? rr - i * a.g : 0;
    const uint16_t* qp = a.q + (int64_t)(sg.row0 + i) * a.q_sr +
                         (int64_t)(sg.kvh * a.g + hl) * a.q_sh + ln.q * 8;
#pragma unroll
    // padding lanes (rows past R) load row 0 of the unit, which is live,
    // rather than selecting zeros: a select on the loaded value would make
    // the wave wait for the load here.  Padding rows are never stored.
    for (int c = 0; c < NC; ++c) q.c[c] = load16(qp + c * 32);
  }

  // Row i of the request sees [max(0, p_i - window_left), p_i] (causal) or
  // [max(0, p_i - window_left), n - 1] (dense), p_i = n - lq + i.
  static __device__ __forceinline__ void reset(const DecodeArgs& a, const Segment& sg,
                                               const Lane& ln, State& st, int& max_lo,
                                               int& min_hi) {
    // the tile's live rows: tokens (tile*16) / g .. min(R - 1, tile*16 + 15) / g
    const int r0 = sg.tile * kRows, r1 = min(sg.R, r0 + kRows) - 1;
    const int i0 = r0 / a.g, i1 = r1 / a.g;
    const int diag0 = sg.u.n - sg.lq + i0, diag1 = sg.u.n - sg.lq + i1;
    min_hi = min(sg.u.n - 1, a.causal ? diag0 : sg.u.n - 1);
    max_lo = max(sg.u.key_lo, a.window_left < 0 ? 0 : max(diag1 - a.window_left, 0));
    const int rr = r0 + ln.j;
    const bool live = rr < sg.R;
    const int diag = sg.u.n - sg.lq + (live ? rr / a.g : 0);
    st.lo = live ? max(a.window_left < 0 ? 0 : diag - a.window_left, 0) : 1;
    st.hi = live ? (a.causal ? diag : sg.u.n - 1) : 0;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int t = 0; t < DJ; ++t) st.acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  template <bool PAGE_POW2>
  static __device__ __forceinline__ void load(Buf& x, const DecodeArgs& a, int kvh, int gi, int kb,
                                              int ke, const PageWindow& pw, int ps_shift,
                                              const Lane& ln) {
    const int j0 = gi * kBlockKeys;
    // keys outside [kb, ke) read the clamped key (masked later); the block
    // holds a key of [kb, ke), so clamped keys stay at rows 0..15 of it
    const int jk = min(max(j0 + ln.j, kb), ke - 1);
    int jv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) jv[e] = min(max(j0 + 4 * ln.q + e, kb), ke - 1);
    if (PAGE_POW2) {
      const int page = page_uniform(pw, (j0 >> ps_shift) - pw.col0);
      const int slot0 = j0 & (a.ps - 1);
      const uint16_t* kbase = a.k + (int64_t)page * a.k_sp + (int64_t)kvh * a.k_sh + slot0 * D;
      const uint16_t* vbase = a.v + (int64_t)page * a.v_sp + (int64_t)kvh * a.v_sh + slot0 * D;
      const uint32_t koff = (uint32_t)(jk - j0) * D + ln.q * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c) x.k[c] = load16_k(kbase + koff + c * 32);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x.v[e] = VRow<D>::load(vbase + (uint32_t)(jv[e] - j0) * D + ln.j * DJ);
    } else {
      {
        const int col = jk / a.ps;
        const int page = page_lane(pw, col - pw.col0);
        const uint16_t* kr = a.k + (int64_t)page * a.k_sp + (int64_t)kvh * a.k_sh +
                             (int64_t)(jk - col * a.ps) * D + ln.q * 8;
#pragma unroll
        for (int c = 0; c < NC; ++c) x.k[c] = load16_k(kr + c * 32);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = jv[e] / a.ps;
        const int page = page_lane(pw, col - pw.col0);
        x.v[e] = VRow<D>::load(a.v + (int64_t)page * a.v_sp + (int64_t)kvh * a.v_sh +
                               (int64_t)(jv[e] - col * a.ps) * D + ln.j * DJ);
      }
    }
  }

  static __device__ __forceinline__ void score(State& st, const Buf& x, const Q& q,
                                               float scale_log2, bool full, int j0,
                                               const Lane& ln) {
    using Mf = Mfma<BF16>;
    using F = Fmt<BF16>;
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) s = Mf::qk(x.k[c], q.c[c], s);
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = s[i] * scale_log2;
      if (!full) {
        const int key = j0 + 4 * ln.q + i;
        sv[i] = (key >= st.lo && key <= st.hi) ? sv[i] : -INFINITY;
      }
    }
    const float lmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    if (wave_any(lmax > st.m + kTau)) {
      // the block max of row j over its four lanes (l, l^16, l^32, l^48)
      const Pair p16 = lane_pair<16>(lmax);
      const float m16 = fmaxf(p16.lo, p16.hi);
      const Pair p32 = lane_pair<32>(m16);
      const float mn = fmaxf(st.m, fmaxf(p32.lo, p32.hi));
      const float alpha = rescale(st.m, mn);
      st.m = mn;
      st.l *= alpha;
      // accumulator rows are 4q + i: take each row's factor from lane 4q + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute((4 * ln.q + i) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
        for (int t = 0; t < DJ; ++t) st.acc[t][i] *= ai;
      }
    }
    // a row with no visible key yet has m = -inf and every score = -inf: p = 0
    const float ms = st.m == -INFINITY ? 0.f : st.m;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - ms);
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
    const u32x2 pa = {F::pack2(p[0], p[1]), F::pack2(p[2], p[3])};
#pragma unroll
    for (int t = 0; t < DJ; ++t) {
      const int u = t >> 1;
      u32x2 vb;
      if (t & 1) {
        vb[0] = pair_hi(VRow<D>::word(x.v[0], u), VRow<D>::word(x.v[1], u));
        vb[1] = pair_hi(VRow<D>::word(x.v[2], u), VRow<D>::word(x.v[3], u));
      } else {
        vb[0] = pair_lo(VRow<D>::word(x.v[0], u), VRow<D>::word(x.v[1], u));
        vb[1] = pair_lo(VRow<D>::word(x.v[2], u), VRow<D>::word(x.v[3], u));
      }
      st.acc[t] = Mf::pv(pa, vb, st.acc[t]);
    }
  }

  // Completes row j's sum over its four lanes.
  static __device__ __forceinline__ void finish(State& st, const Lane&) {
    const Pair p16 = lane_pair<16>(st.l);
    const float l16 = p16.lo + p16.hi;
    const Pair p32 = lane_pair<32>(l16);
    st.l = p32.lo + p32.hi;
  }

  // Output item k of the lane: row 4q + k, dims j*DJ .. +DJ.  Every lane must
  // call it (cross-lane reads of the row's M and L).
  static __device__ __forceinline__ bool item(const State& st, const Lane& ln, int k, int& r,
                                              int& d0, float& M, float& L, float (&O)[8]) {
    r = 4 * ln.q + k;
    d0 = ln.j * DJ;
    M = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(r << 2, __builtin_bit_cast(int, st.m)));
    L = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(r << 2, __builtin_bit_cast(int, st.l)));
#pragma unroll
    for (int e = 0; e < 8; ++e) O[e] = e < DJ ? st.acc[e < DJ ? e : 0][k] : 0.f;
    return true;
  }
  static __device__ __forceinline__ void item_pos(const Lane& ln, int k, int& r, int& d0) {
    r = 4 * ln.q + k;
    d0 = ln.j * DJ;
  }
  // Index within a slot's partial block: [row][e][j]
  static __device__ __forceinline__ int pidx(const Lane& ln, int r, int e) {
    return (r * DJ + e) * 16 + ln.j;
  }
  // The same index for element (row r, dim d): d = j * DJ + e
  static __device__ __forceinline__ int ppos(int r, int d) { return (r * DJ + d % DJ) * 16 + d / DJ; }
};

}  // namespace dev
}  // namespace pkvd
