// engine_valu.h -- VALU dot-product engine of the persistent decode kernel
// (rows per tile <= 8): q . k and P x V with v_dot2 on bf16/fp16 pairs.
//
// Lane layout (LPK = D / 8 lanes per key, KPS = 64 / LPK keys per step):
// lane (kq, part) holds the 16-byte piece `part` (dims part*8 .. part*8+7) of
// key kq of each step, so one wave-wide 16-byte load reads KPS whole
// contiguous key rows of the [page_size, D] page tile; Q sits in registers
// with the same dim split.  Two steps form a group (4 KB of K and V per
// wave).  q . k ends in a DPP all-reduce over the LPK lanes of the key.
// Every key lane group is an independent online-softmax stream whose max
// rises lazily (only when a score exceeds it by more than kTau, base 2), so
// the rescale branch is rare.  P x V: the lane's two keys of a group give a
// pair of probabilities, packed to bf16/fp16 and multiplied into
// byte-permuted (V[k][d], V[k + KPS][d]) pairs with v_dot2; sums l stay in
// fp32.  At a segment's end the KPS streams merge by DPP and lane-pair swaps.
#pragma once

#include "decode_common.h"

namespace pkvd {
namespace dev {

template <int D>
struct Geo {
  static constexpr int LPK = D / 8;           // lanes per key (one 16-byte piece each)
  static constexpr int KPS = 64 / LPK;        // keys per step
  static constexpr int KPG = 2 * KPS;         // keys per group (two steps)
  static constexpr int GPB = kBlockKeys / KPG;  // groups per 16-key block
};

struct KeyRegs {
  u32x4 k[2];   // [step]: the lane's 16-byte piece of its key of that step
  u32x4 v[2];
};

// Loads group gi (keys gi * KPG ..) of a chunk whose keys are [kb, ke) and
// whose block-table columns sit in pw.
template <int D, bool PAGE_POW2>
__device__ __forceinline__ void load_group(KeyRegs& x, const DecodeArgs& a, int kvh, int gi,
                                           int kb, int ke, const PageWindow& pw, int ps_shift,
                                           int kq, int part) {
  using G = Geo<D>;
  const int j0 = gi * G::KPG;
  if (PAGE_POW2) {
    // page_size is a power of two >= 16: the group's 16-key block lies in one
    // page, so the tile base is wave-uniform (scalar) and each lane adds a
    // 32-bit offset.  A key outside [kb, ke) reads the clamped key instead
    // (masked later); the block always holds a key of [kb, ke), so the clamped
    // key is in the same page at a row 0..15 past the block start, even when
    // this group itself lies wholly before kb or after ke - 1.
    const int jb = j0 & ~(kBlockKeys - 1);
    const int page = page_uniform(pw, (jb >> ps_shift) - pw.col0);
    const int slot0 = jb & (a.ps - 1);
    const uint16_t* kbase = a.k + (int64_t)page * a.k_sp + (int64_t)kvh * a.k_sh + slot0 * D;
    const uint16_t* vbase = a.v + (int64_t)page * a.v_sp + (int64_t)kvh * a.v_sh + slot0 * D;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t jr = (uint32_t)(min(max(j0 + t * G::KPS + kq, kb), ke - 1) - jb);
      const uint32_t off = jr * D + part * 8;
      x.k[t] = load16_stream(kbase + off);
      x.v[t] = load16_stream(vbase + off);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int jc = min(max(j0 + t * G::KPS + kq, kb), ke - 1);
      const int col = jc / a.ps;
      const int page = page_lane(pw, col - pw.col0);
      const int slot = jc - col * a.ps;
      const int64_t off = (int64_t)slot * D + part * 8;
      x.k[t] = load16_stream(a.k + (int64_t)page * a.k_sp + (int64_t)kvh * a.k_sh + off);
      x.v[t] = load16_stream(a.v + (int64_t)page * a.v_sp + (int64_t)kvh * a.v_sh + off);
    }
  }
}

template <int RT>
struct Stream {
  float m[RT], l[RT];
  float o[RT][8];   // this lane's 8 dims: part * 8 + e
};

// Sum over the LPK lanes of a key (aligned lane groups of 8 or 16).
template <int LPK>
__device__ __forceinline__ float key_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  if constexpr (LPK == 16) x += dpp<kDppRor8>(x);
  return x;
}

// Scores one group: key kq in step 0 and key kq + KPS in step 1.  The two
// probabilities of a row are packed as a 16-bit pair and multiplied into V
// with v_dot2 against (V[kq][d], V[kq + KPS][d]) pairs built by byte
// permutes; the running sums l stay in fp32.
template <int D, int RT, bool BF16>
__device__ __forceinline__ void score_group(Stream<RT>& st, const KeyRegs& x,
                                            const u32x4 (&qr)[RT], float scale_log2, bool full,
                                            int j0, int kq, const int (&lo_r)[RT],
                                            const int (&hi_r)[RT]) {
  using F = Fmt<BF16>;
  using G = Geo<D>;
  float s[2][RT];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float acc = F::dot2(qr[r].x, x.k[t].x, 0.f);
      acc = F::dot2(qr[r].y, x.k[t].y, acc);
      acc = F::dot2(qr[r].z, x.k[t].z, acc);
      acc = F::dot2(qr[r].w, x.k[t].w, acc);
      s[t][r] = key_sum<G::LPK>(acc) * scale_log2;
    }
  }
  if (!full) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = j0 + t * G::KPS + kq;
#pragma unroll
      for (int r = 0; r < RT; ++r) s[t][r] = (j >= lo_r[r] && j <= hi_r[r]) ? s[t][r] : -INFINITY;
    }
  }
  bool need = false;
#pragma unroll
  for (int r = 0; r < RT; ++r) need |= fmaxf(s[0][r], s[1][r]) > st.m[r] + kTau;
  if (wave_any(need)) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const float mn = fmaxf(st.m[r], fmaxf(s[0][r], s[1][r]));
      const float alpha = rescale(st.m[r], mn);
      st.m[r] = mn;
      st.l[r] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.o[r][e] *= alpha;
    }
  }
  uint32_t pp[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    // a row with no visible key yet has m = -inf and every s = -inf: p = 0
    const float ms = st.m[r] == -INFINITY ? 0.f : st.m[r];
    const float p0 = fast_exp2(s[0][r] - ms), p1 = fast_exp2(s[1][r] - ms);
    st.l[r] += p0 + p1;
    pp[r] = F::pack2(p0, p1);
  }
  const uint32_t w0[4] = {x.v[0].x, x.v[0].y, x.v[0].z, x.v[0].w};
  const uint32_t w1[4] = {x.v[1].x, x.v[1].y, x.v[1].z, x.v[1].w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t vlo = pair_lo(w0[u], w1[u]), vhi = pair_hi(w0[u], w1[u]);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      st.o[r][2 * u] = F::dot2(pp[r], vlo, st.o[r][2 * u]);
      st.o[r][2 * u + 1] = F::dot2(pp[r], vhi, st.o[r][2 * u + 1]);
    }
  }
}

// Merges the KPS key streams of the wave into every lane (lanes of different
// streams differ in bits log2(LPK) .. 5): bit 3 within each 16-lane row by
// DPP (when LPK = 8), bits 4 and 5 by lane-pair swaps.
template <int D, int RT>
__device__ __forceinline__ void merge_streams(Stream<RT>& st) {
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    if constexpr (Geo<D>::LPK == 8) {
      const float mo = dpp<kDppRor8>(st.m[r]);
      const float M = fmaxf(st.m[r], mo);
      const float a0 = rescale(st.m[r], M), a1 = rescale(mo, M);
      st.l[r] = st.l[r] * a0 + dpp<kDppRor8>(st.l[r]) * a1;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.o[r][e] = st.o[r][e] * a0 + dpp<kDppRor8>(st.o[r][e]) * a1;
      st.m[r] = M;
    }
    {
      const Pair m = lane_pair<16>(st.m[r]);
      const float M = fmaxf(m.lo, m.hi);
      const float a0 = rescale(m.lo, M), a1 = rescale(m.hi, M);
      const Pair l = lane_pair<16>(st.l[r]);
      st.l[r] = l.lo * a0 + l.hi * a1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const Pair o = lane_pair<16>(st.o[r][e]);
        st.o[r][e] = o.lo * a0 + o.hi * a1;
      }
      st.m[r] = M;
    }
    {
      const Pair m = lane_pair<32>(st.m[r]);
      const float M = fmaxf(m.lo, m.hi);
      const float a0 = rescale(m.lo, M), a1 = rescale(m.hi, M);
      const Pair l = lane_pair<32>(st.l[r]);
      st.l[r] = l.lo * a0 + l.hi * a1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const Pair o = lane_pair<32>(st.o[r][e]);
        st.o[r][e] = o.lo * a0 + o.hi * a1;
      }
      st.m[r] = M;
    }
  }
}


template <int D, int RT, bool BF16>
struct ValuEngine {
  using G = Geo<D>;
  static constexpr int kRows = RT;
  static constexpr int kKeysPerGroup = G::KPG;
  static constexpr int kGroupsPerBlock = G::GPB;
  static constexpr int kItems = (RT + G::KPS - 1) / G::KPS;   // output rows per lane
  static constexpr int kItemDims = 8;                         // dims per output item
  static constexpr int kItemLanes = G::LPK;                   // lanes sharing a row's item

  struct Lane {
    int kq, part;
  };
  struct Q {
    u32x4 r[RT];
  };
  using Buf = KeyRegs;
  struct State {
    Stream<RT> s;
    int lo[RT], hi[RT];   // visible key range per row
  };

  static __device__ __forceinline__ Lane lane_of(int lane) { return {lane / G::LPK, lane % G::LPK}; }

  // Q rows of a tile (rr = tile * RT + r -> token rr / g, head rr % g): the
  // lane's 16-byte piece of each row
  static __device__ __forceinline__ void fetch_q(const DecodeArgs& a, const Segment& sg,
                                                 const Lane& ln, Q& q) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int rr = sg.tile * RT + r;
      const bool live = rr < sg.R;
      const int i = live ? rr / a.g : 0;
      const int hl = live ? rr - i * a.g : 0;
      const uint16_t* qp = a.q + (int64_t)(sg.row0 + i) * a.q_sr +
                           (int64_t)(sg.kvh * a.g + hl) * a.q_sh + ln.part * 8;
      // a padding row (past R) loads row 0 of the unit, which is live,
      // rather than selecting zeros: a select on the loaded value would make
      // the wave wait for the load here.  Padding rows are never stored.
      q.r[r] = load16(qp);
    }
  }

  // Reset for a new segment; returns the key range every row sees fully
  // ([max_lo, min_hi]: groups inside it need no mask).  Row i of the request
  // sees [max(0, p_i - window_left), p_i] (causal) or [max(0, p_i -
  // window_left), n - 1] (dense), p_i = n - lq + i.
  static __device__ __forceinline__ void reset(const DecodeArgs& a, const Segment& sg,
                                               const Lane&, State& st, int& max_lo, int& min_hi) {
    max_lo = sg.u.key_lo;
    min_hi = sg.u.n - 1;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int rr = sg.tile * RT + r;
      const bool live = rr < sg.R;
      const int diag = sg.u.n - sg.lq + (live ? rr / a.g : 0);
      const int rlo = max(a.window_left < 0 ? 0 : diag - a.window_left, 0);
      const int rhi = a.causal ? diag : sg.u.n - 1;
      st.lo[r] = live ? rlo : 1;     // dead rows see nothing
      st.hi[r] = live ? rhi : 0;
      if (live) {
        max_lo = max(max_lo, rlo);
        min_hi = min(min_hi, rhi);
      }
      st.s.m[r] = -INFINITY;
      st.s.l[r] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.s.o[r][e] = 0.f;
    }
  }

  template <bool PAGE_POW2>
  static __device__ __forceinline__ void load(Buf& x, const DecodeArgs& a, int kvh, int gi, int kb,
                                              int ke, const PageWindow& pw, int ps_shift,
                                              const Lane& ln) {
    load_group<D, PAGE_POW2>(x, a, kvh, gi, kb, ke, pw, ps_shift, ln.kq, ln.part);
  }

  static __device__ __forceinline__ void score(State& st, const Buf& x, const Q& q,
                                               float scale_log2, bool full, int j0,
                                               const Lane& ln) {
    score_group<D, RT, BF16>(st.s, x, q.r, scale_log2, full, j0, ln.kq, st.lo, st.hi);
  }

  static __device__ __forceinline__ void finish(State& st, const Lane&) { merge_streams<D, RT>(st.s); }

  // Output item k of the lane: row r, dims d0 .. d0 + 7, with its (M, L, O).
  static __device__ __forceinline__ bool item(const State& st, const Lane& ln, int k, int& r,
                                              int& d0, float& M, float& L, float (&O)[8]) {
    r = ln.kq + k * G::KPS;
    d0 = ln.part * 8;
    M = -INFINITY;
    L = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) O[e] = 0.f;
#pragma unroll
    for (int rr = 0; rr < RT; ++rr)
      if (rr == r) {
        M = st.s.m[rr];
        L = st.s.l[rr];
#pragma unroll
        for (int e = 0; e < 8; ++e) O[e] = st.s.o[rr][e];
      }
    return r < RT;
  }
  // Row and dims of item k without the state (for merges).
  static __device__ __forceinline__ void item_pos(const Lane& ln, int k, int& r, int& d0) {
    r = ln.kq + k * G::KPS;
    d0 = ln.part * 8;
  }
  // Index within a slot's partial block: [row][e][lane-in-item]
  static __device__ __forceinline__ int pidx(const Lane& ln, int r, int e) {
    return (r * 8 + e) * G::LPK + ln.part;
  }
  // The same index for element (row r, dim d): d = part * 8 + e
  static __device__ __forceinline__ int ppos(int r, int d) { return (r * 8 + (d & 7)) * G::LPK + (d >> 3); }
};

}  // namespace dev
}  // namespace pkvd
