// decode_kernel.h -- the persistent paged-KV decode kernel and the merge
// kernel (templates; instantiated per head_dim and element type by the
// decode_inst_*.hip files, launched from decode_launch.hip).
//
// Operation: flashinfer.cudnn.cudnn_batch_decode_with_kv_cache (Parameters,
// Note / LSE convention).  A unit of work is (request b, kv head, row tile);
// the rows of a tile are the Hq/Hkv query heads sharing the kv head times the
// q_len_per_req query tokens, so every K/V byte a wave loads serves all of
// them (grouped-query packing).
//
// Schedule (persistent, balanced): one grid of exactly the resident number
// of waves.  Every workgroup rebuilds, from seq_lens_kv, the prefix of the
// linear block space of all units, so planning never reads lengths on the
// host; wave w then streams its own slice of that space (decode_common.h:
// equal slices, or weighted by the wave's position on its SIMD), crossing
// unit boundaries as needed, so a wave's share of the work is set by its
// weight alone, whatever the mix of lengths.  The slice is one continuous
// stream of chunks: the last round of a chunk already issues the first loads
// of the next one (next segment included), and the next segment's Q rows are
// loaded before the current segment's epilogue.  A unit inside one slice is written
// directly; a unit cut between slices leaves a normalised partial state (o,
// base-2 LSE) per piece in the slot of the wave that streamed it.  Either
// the wave whose blocks complete the unit (an
// atomic count of delivered blocks, taken once its slice is streamed) merges
// the pieces in block order with the base-2 LSE rule (Note / LSE
// convention: base-2 LSE states are what the cascade merge consumes), or a
// second kernel merges all cut units.  The split of the work depends on the
// shapes and lengths only, so the result is the same in every call.
//
// The per-wave arithmetic comes from an engine: VALU dot products for tiles
// of up to 8 rows (engine_valu.h), MFMA for 16-row tiles (engine_mfma.h).
// For the VALU engine (LPK = D / 8 lanes per key, KPS = 64 / LPK keys per
// step):
//  * lane (kq, part) holds the 16-byte piece `part` (dims part*8 .. part*8+7)
//    of key kq of each step, so one wave-wide 16-byte load reads KPS whole
//    contiguous key rows of the [page_size, D] page tile; Q sits in
//    registers with the same dim split;
//  * two steps form a group (4 KB of K and V per wave); groups are loaded PF
//    ahead of the scoring through a register ring with no branch around the
//    loads (keys outside the segment are redirected to a key inside it and
//    masked), so they stay in flight across the scoring;
//  * q . k: v_dot2 on bf16/fp16 pairs, then a DPP all-reduce over the LPK
//    lanes of the key;
//  * every key lane group is an independent online-softmax stream (running
//    max m, sum l, accumulator for its 8 dims); m rises lazily, only when a
//    score exceeds it by more than kTau (base 2), so probabilities stay
//    <= 2^kTau and the rescale branch is rare;
//  * P x V: the lane's two keys of a group (steps 0 and 1) give a pair of
//    probabilities, packed to bf16/fp16 and multiplied into byte-permuted
//    (V[k][d], V[k + KPS][d]) pairs with v_dot2; sums l stay in fp32;
//  * the page ids of the next 128 block-table columns sit in two registers
//    (one column per lane), read with readlane / ds_bpermute;
//  * at a segment's end the KPS streams merge by DPP and lane-pair swaps.
#pragma once

#include "engine_mfma.h"
#include "engine_valu.h"

namespace pkvd {
namespace dev {

// Writes one output item (N = 8 or 4 consecutive dims from d0) and, from the
// row's lead lane, its LSE.
template <int D, int N>
__device__ __forceinline__ void store_item(const DecodeArgs& a, const float* s_sink,
                                           int64_t rowhead, int qhead, int d0, bool lead, float M,
                                           float L, const float (&O)[8]) {
  // the decode kernel keeps the sink logits in LDS: a global load here would
  // make the wave wait for every K/V load still in flight
  const bool has_sink = a.sinks != nullptr;
  float sink = 0.f;
  if (has_sink) sink = s_sink[qhead];
  float x[N];
#pragma unroll
  for (int e = 0; e < N; ++e) x[e] = final_value(has_sink, sink, M, L, O[e], a.out_scale);
  store_out<N>(a, (int64_t)rowhead * D + d0, x);
  if (a.lse && lead) a.lse[rowhead] = L > 0.f ? M + log2f(L) : -INFINITY;
}

// Writes one item of a slice's partial state for a cut unit: the normalised
// output o = O / L (in the engine's lane-contiguous order, with
// device-coherent stores so that a merging wave on another CU reads them
// after its ticket) and, from the row's lead lane, its base-2 LSE.
template <class Eng, int D>
__device__ __forceinline__ void store_partial(const DecodeArgs& a, int slot,
                                              const typename Eng::Lane& ln, int r, int d0,
                                              float M, float L, const float (&O)[8]) {
  constexpr int RT = Eng::kRows;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* po = a.ws_o + (int64_t)slot * RT * D;
#pragma unroll
  for (int e = 0; e < Eng::kItemDims; ++e) store_coherent(po + Eng::pidx(ln, r, e), O[e] * inv);
  if (d0 == 0) store_coherent(a.ws_lse + (int64_t)slot * RT + r, L > 0.f ? M + log2f(L) : -INFINITY);
}

// Merge of the partial states of one cut unit (virtual start vs, nblk
// blocks per unit) for all output items of the lane, in steps, so that a
// wave completing two units has the first loads of both in flight at once:
// begin() works out the first batch of candidates and issues its loads,
// finish() consumes them, takes the remaining pieces and writes the final
// values.  Candidates are taken 64 at a time (lane c works out whether
// candidate c wrote a partial state); the written ones are read kDepth at a
// time in block order (every item's loads in flight), raising the running
// maximum once per group.  Only rows below R = g * lq hold partial states
// (the rest of a 16-row MFMA tile is padding).
template <class Eng, int D>
struct UnitMerge {
  static constexpr int RT = Eng::kRows, N = Eng::kItemDims, NI = Eng::kItems;
  // (deeper batches for 32-float items, 4 or 8 pieces, measured no faster)
  static constexpr int kDepth = NI * N <= 8 ? 8 : (NI * N <= 16 ? 4 : 2);
  // Groups of more than two pieces take no loads and no products for their
  // empty places (those of a unit's last group), and the set-up of equal
  // slices below; each would otherwise cost its instructions at the end of
  // the kernel.  Groups of two (the 16-row tiles' 32-float items) keep the
  // general forms: with either change the MFMA kernels measured slower.
  static constexpr bool kSkip = kDepth > 2;
  int unit, vs, nblk, tile, kvh, R;
  ReqRows rows;
  UnitPieces up;
  int rr[NI], dd[NI];
  float Mx[NI], W[NI], acc[NI][8];
  // the candidate batch being read: candidates c0 .. c0 + 63, the lane's
  // slot, the written ones not yet loaded (m), the batch's first written slot
  int c0, slot, sl0;
  uint64_t m;
  float lv[kDepth][NI], ov[kDepth][NI][N];
  bool on[kDepth];

  // Equal slices of at least one block (eq), for the merges with groups of
  // more than two: the slice of a block from a hardware reciprocal of the
  // sliced space's size, corrected exactly by the remainder (quot_est), and
  // every candidate after the first holds blocks of the unit (its slice
  // starts inside the unit: its first segment), so only the first
  // candidate's slot (slot_first) needs its slice's start.  The same results
  // as unit_pieces and candidate_slot with far fewer dependent instructions:
  // per-wave stamps put the general forms at ~1.3 us of a merging wave's
  // tail.
  bool eq;
  int slot_first;
  float inv_t, inv_nw;   // 1 / T and 1 / NW (hardware reciprocals)
  // floor(n / d) for 0 <= n < 2^30, 0 < d < 2^30 with a quotient below
  // 2^15, from inv = 1 / d within two ulps: the estimate is within 0.01
  // of n / d, so its truncation is the quotient or a neighbour, which the
  // remainder corrects (n + d < 2^31: no overflow).
  static __device__ __forceinline__ int quot_est(int n, int d, float inv) {
    int q = (int)((float)n * inv);
    const int r = n - q * d;
    return r < 0 ? q - 1 : (r >= d ? q + 1 : q);
  }
  // n / d for n >= 0 and d > 0: a shift when d is a power of two
  static __device__ __forceinline__ int quot_pow2(int n, int d) {
    return (d & (d - 1)) == 0 ? n >> __builtin_ctz(d) : n / d;
  }
  __device__ __forceinline__ int slice_at(const Slices& sl_, int64_t x) const {
    const int64_t n = (x + 1) * sl_.NW - 1;
    if (eq && n < 0x40000000LL) return quot_est((int)n, sl_.T, inv_t);
    return slice_of(sl_, x);
  }
  // slice_begin of equal slices: qT w + floor(rT w / NW)
  __device__ __forceinline__ int slice_start(const Slices& sl_, int w) const {
    return sl_.qT * w + quot_est(sl_.rT * w, sl_.NW, inv_nw);
  }
  // Candidates of the batch at c0 and its mask; skips batches with no
  // written piece.  False when none remain.
  __device__ __forceinline__ bool open_batch(const Slices& sl_, int lane) {
    for (; c0 < up.n; c0 += 64) {
      const int c = c0 + lane;
      bool valid = false;
      slot = 0;
      if constexpr (kSkip) {
        if (eq) {
          valid = c < up.n;
          slot = c == 0 ? slot_first : 2 * (up.w0 + c);
        } else if (c < up.n) {
          slot = candidate_slot(up, sl_, vs, c, valid);
        }
      } else {
        if (c < up.n) slot = candidate_slot(up, sl_, vs, c, valid);
      }
      m = __builtin_amdgcn_ballot_w64(valid);
      if (m) {
        // off entries of a group of two read the batch's first written
        // piece (finite values) with weight 0
        sl0 = __builtin_amdgcn_readlane(slot, (int)__builtin_ctzll(m));
        return true;
      }
    }
    return false;
  }
  // loads of the batch's next kDepth written pieces
  __device__ __forceinline__ void issue(const DecodeArgs& a, const typename Eng::Lane& ln) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      on[u] = m != 0;
      if constexpr (kSkip)
        if (!on[u]) continue;   // uniform
      const int q = on[u] ? (int)__builtin_ctzll(m) : 0;
      m = on[u] ? m & (m - 1) : m;
      const int sl = on[u] ? __builtin_amdgcn_readlane(slot, q) : sl0;
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        // padding rows read row 0's values (loaded by other lanes anyway)
        const int r = rr[it] < RT && tile * RT + rr[it] < R ? rr[it] : 0;
        lv[u][it] = load_coherent(a.ws_lse + (int64_t)sl * RT + r);
#pragma unroll
        for (int e = 0; e < N; ++e)
          ov[u][it][e] = load_coherent(a.ws_o + (int64_t)sl * RT * D + Eng::pidx(ln, r, e));
      }
    }
  }
  __device__ __forceinline__ void consume() {
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      float Mn = Mx[it];
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        if constexpr (kSkip) {
          if (on[u]) Mn = fmaxf(Mn, lv[u][it]);
        } else {
          Mn = fmaxf(Mn, on[u] ? lv[u][it] : -INFINITY);
        }
      }
      const float sc = rescale(Mx[it], Mn);
      W[it] *= sc;
#pragma unroll
      for (int e = 0; e < N; ++e) acc[it][e] *= sc;
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        if constexpr (kSkip)
          if (!on[u]) continue;   // uniform
        const float wt = on[u] ? rescale(lv[u][it], Mn) : 0.f;
        W[it] += wt;
#pragma unroll
        for (int e = 0; e < N; ++e) acc[it][e] = fmaf(wt, ov[u][it][e], acc[it][e]);
      }
      Mx[it] = Mn;
    }
  }
  bool first;   // a first batch was issued (some piece was written)
  // Set-up and the first batch's loads.
  __device__ __forceinline__ void begin(const DecodeArgs& a, const Slices& sl_, int unit_, int vs_,
                                        int nblk_, ReqRows rows_, const typename Eng::Lane& ln,
                                        int lane) {
    unit = unit_;
    vs = vs_;
    nblk = nblk_;
    rows = rows_;
    const int per_req = a.Hkv * a.row_tiles;
    if constexpr (kSkip) {
      const int b = quot_pow2(unit, per_req), uidx = unit - b * per_req;
      kvh = quot_pow2(uidx, a.row_tiles);
      tile = uidx - kvh * a.row_tiles;
    } else {
      const int b = unit / per_req, uidx = unit - b * per_req;
      kvh = uidx / a.row_tiles;
      tile = uidx - kvh * a.row_tiles;
    }
    R = a.g * rows.lq;
    if constexpr (kSkip) {
      // (NW <= 32768 keeps rT w below 2^30 and every quotient below 2^15)
      eq = sl_.uniform && sl_.qT > 0 && sl_.NW <= 32768 && sl_.T < 0x40000000;
      inv_t = __builtin_amdgcn_rcpf((float)sl_.T);
      inv_nw = __builtin_amdgcn_rcpf((float)sl_.NW);
      up.w0 = slice_at(sl_, (int64_t)vs + a.seg_cost);
      up.n = slice_at(sl_, (int64_t)vs + a.seg_cost + nblk - 1) - up.w0 + 1;
      slot_first = 2 * up.w0 + (eq && slice_start(sl_, up.w0) >= vs ? 0 : 1);
    } else {
      up = unit_pieces(sl_, vs, a.seg_cost, nblk);
    }
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      Eng::item_pos(ln, it, rr[it], dd[it]);
      Mx[it] = -INFINITY;
      W[it] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[it][e] = 0.f;
    }
    c0 = 0;
    first = open_batch(sl_, lane);
    if (first) issue(a, ln);
  }
  __device__ __forceinline__ void finish(const DecodeArgs& a, const float* s_sink, const Slices& sl_,
                                         const typename Eng::Lane& ln, int lane) {
    if (first) {
      consume();
      for (;;) {
        while (m) {   // uniform: the batch's further written pieces, in order
          issue(a, ln);
          consume();
        }
        c0 += 64;
        if (!open_batch(sl_, lane)) break;
      }
    }
    // acc / W is the merged normalised output; final_value divides by W + sink
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int r = rr[it], row = tile * RT + r;
      if (!(r < RT && row < R)) continue;
      const int ti = kSkip ? quot_pow2(row, a.g) : row / a.g, qhead = kvh * a.g + (row - ti * a.g);
      store_item<D, N>(a, s_sink, ((int64_t)rows.row0 + ti) * a.Hq + qhead, qhead, dd[it],
                       dd[it] == 0, Mx[it], W[it], acc[it]);
    }
  }
};

template <class Eng, int D, bool PAGE_POW2, int PF, int WPE>
__global__ __launch_bounds__(64 * kSimdsPerCu * WPE) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void decode_kernel(const DecodeArgs a) {
  // one workgroup per CU: WPE waves on each of its SIMDs
  constexpr int kWaves = kSimdsPerCu * WPE, kThreads = 64 * kWaves;
  constexpr int RT = Eng::kRows;
  constexpr int NBUF = PF + 1;
  constexpr int kWindow = 128;                        // block-table columns per chunk
  constexpr int GPB = Eng::kGroupsPerBlock, KPG = Eng::kKeysPerGroup;
  extern __shared__ int lds[];
  const LdsLayout L = lds_layout(a.B, kThreads, a.sinks ? a.Hq : 0, a.qo != nullptr);
  int* s_scan = lds + L.scan;
  int* s_vscan = lds + L.vscan;
  int* s_pref = lds + L.pref;
  int* s_vpref = lds + L.vpref;
  int* s_nlen = lds + L.nlen;
  int* s_nb = lds + L.nb;
  int* s_qo = lds + L.qo;
  float* s_sink = reinterpret_cast<float*>(lds + L.sink);

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const typename Eng::Lane ln = Eng::lane_of(lane);

#ifdef PKVD_TRACE
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
#endif
  Prefix pf = build_prefix<kThreads>(a, s_pref, s_vpref, s_nlen, s_nb, s_qo, s_scan, s_vscan,
                                     s_sink);
  pf.T = uniform(pf.T);
  pf.TV = uniform(pf.TV);
  const int T = pf.T;
#ifdef PKVD_TRACE
  const uint64_t t_prefix = __builtin_amdgcn_s_memrealtime();
#endif
  if (a.merge_kernel && blockIdx.x == 0)   // the prefixes, for the merge kernel
    for (int i = threadIdx.x; i <= a.B; i += kThreads) {
      a.ws_pref[i] = s_pref[i];
      a.ws_vpref[i] = s_vpref[i];
    }
  // slices of the virtual block space, mapped back to real blocks
  int NW;
  const Slices sl_ = grid_slices(a, pf.TV, T, NW);
  // Each workgroup takes a run of consecutive slices (its CU then streams
  // neighbouring kv heads of the same requests): PER = ceil(NW / groups)
  // waves of each group are active, so a short grid still spreads over all
  // groups.
  const int active = sl_.PER;
  const int gw = wave < active ? (int)blockIdx.x * active + wave : NW;
#ifdef PKVD_TRACE
  const uint64_t t_slices = __builtin_amdgcn_s_memrealtime();
#endif
  if (T == 0 || gw >= NW) return;   // no slice
  // The slice's virtual bounds, their requests (one search for both) and
  // real blocks; the request and unit found for the first bound also give
  // the first segment (a virtual block maps into its own request).
  const int v_lo = slice_begin(sl_, gw), v_hi = slice_begin(sl_, gw + 1);
  int b_lo, b_hi;
  find_request2(s_vpref, a.B, v_lo, v_hi, b_lo, b_hi);
  const int pref_lo = __builtin_amdgcn_readfirstlane(s_pref[b_lo]);
  const int vpref_lo = __builtin_amdgcn_readfirstlane(s_vpref[b_lo]);
  const int nb_lo = __builtin_amdgcn_readfirstlane(s_nb[b_lo]);
  const int pref_hi = __builtin_amdgcn_readfirstlane(s_pref[b_hi]);
  const int vpref_hi = __builtin_amdgcn_readfirstlane(s_vpref[b_hi]);
  const int nb_hi = __builtin_amdgcn_readfirstlane(s_nb[b_hi]);
  int ul_lo, ul_hi;
  const int lo = v_lo < pf.TV ? pref_lo + real_off(a, nb_lo, v_lo - vpref_lo, ul_lo) : T;
  const int hi = v_hi < pf.TV ? pref_hi + real_off(a, nb_hi, v_hi - vpref_hi, ul_hi) : T;
  if (lo >= hi) return;
  PKVD_COUNT(a, gw, 0, t_start);
  PKVD_COUNT(a, gw, 1, t_prefix);
  PKVD_COUNT(a, gw, 12, t_slices);
  PKVD_STAMP(a, gw, 13);
  const int ps_shift = PAGE_POW2 ? __builtin_ctz(a.ps) : 0;
  // blocks per chunk: (blocks * 16 - 1) / ps + 2 <= kWindow columns
  const int chunk_blocks = max(1, ((kWindow - 2) * a.ps + 1) / kBlockKeys);

  // The slice is one stream of chunks: blocks [cb, ce) of a segment (a
  // unit's part of the slice), at most chunk_blocks long so its page ids fit
  // the 128-column window.  Each chunk is padded to a whole
  // number of rounds of NBUF groups (the padding groups are loaded again from
  // the chunk and not scored), so group g of every chunk lives in
  // buf[g % NBUF] and the last round of a chunk issues the first loads of the
  // next one.
  struct Chunk {
    Segment sg;
    int cb, ce, kb, ke;   // blocks and keys
    int ng, ngp;          // groups, and groups padded to rounds
    int first, last, valid;   // ints, not bools: copies of the struct stay in registers
  };
  auto make_chunk = [&](const Segment& sg, int cb) {
    Chunk c;
    c.sg = sg;
    c.cb = cb;
    c.ce = min(sg.blk_end, cb + chunk_blocks);
    c.kb = max(sg.u.key_lo, cb * kBlockKeys);
    c.ke = min(sg.u.n, c.ce * kBlockKeys);
    c.ng = (c.ce - c.cb) * GPB;
    c.ngp = (c.ng + NBUF - 1) / NBUF * NBUF;
    c.first = cb == sg.blk_begin;
    c.last = c.ce == sg.blk_end;
    c.valid = 1;
    return c;
  };
  auto chunk_end = [&](const Chunk& c) -> int {   // linear block after the chunk
    return c.sg.ustart + (c.ce - c.sg.u.first_blk);
  };
  // The chunk after c: the same segment's next one, or the next segment's
  // first (invalid at the end of the slice).
  auto next_chunk = [&](const Chunk& c) {
    const int pos = chunk_end(c);
    Chunk n = c;
    n.valid = 0;
    if (!c.last) {
      n = make_chunk(c.sg, c.ce);
    } else if (pos < hi) {
      // the segment ended with its unit: the next unit of the same request
      // (no search) or the first of a later request
      const Segment& g = c.sg;
      int tiles = a.qo ? tiles_of(a, g.lq) : a.row_tiles;
      tiles = tiles > 0 ? tiles : 1;
      const int uidx = g.kvh * tiles + g.tile;
      if (uidx + 1 < a.Hkv * tiles && g.u.nblk > 0) {
        const Segment sg = segment_at(a, s_nlen, s_qo, g.b, g.ustart - uidx * g.u.nblk,
                                      g.vstart - uidx * unit_vspan(a, g.u.nblk), uidx + 1, pos,
                                      lo, hi);
        n = make_chunk(sg, sg.blk_begin);
      } else {
        const Segment sg = locate(a, s_pref, s_vpref, s_nlen, s_nb, s_qo, pos, lo, hi);
        n = make_chunk(sg, sg.blk_begin);
      }
    }
    return n;
  };
  // page ids of a chunk's columns (issued early; clamped into the pool where used)
  auto fetch_pages = [&](const Chunk& c) {
    PageWindow w;
    w.col0 = PAGE_POW2 ? c.kb >> ps_shift : c.kb / a.ps;
    const int ncol = (PAGE_POW2 ? (c.ke - 1) >> ps_shift : (c.ke - 1) / a.ps) - w.col0 + 1;
    const int32_t* row = a.bt + (int64_t)c.sg.b * a.bt_sr + w.col0;
    const int p0 = row[min(lane, ncol - 1)];
    const int p1 = row[min(64 + lane, ncol - 1)];
    w.p0 = p0;
    w.p1 = p1;
    w.plast = a.P - 1;
    return w;
  };

#ifdef PKVD_TRACE
  int n_seg = 0, n_chunk = 0, n_blk = 0;
#endif
  {
    // pieces of units the slice cuts: at most its first and last segments;
    // their tickets are taken once the slice is streamed
    int pend_unit[2] = {-1, -1}, pend_n[2] = {0, 0}, pend_vs[2] = {0, 0}, pend_nb[2] = {0, 0};
    Chunk cur;
    {
      const Segment sg = segment_at(a, s_nlen, s_qo, b_lo, pref_lo, vpref_lo, ul_lo, lo, lo, hi);
      cur = make_chunk(sg, sg.blk_begin);
    }
    PKVD_STAMP(a, gw, 14);
    PageWindow pw = fetch_pages(cur);
    PKVD_STAMP(a, gw, 15);
    // the next chunk and its page ids before the first K/V loads: a slice
    // may start with a few blocks of a unit, and then its first chunk ends
    // soon after those loads return
    Chunk nxt = next_chunk(cur);
    PageWindow pwn = nxt.valid ? fetch_pages(nxt) : pw;
    PKVD_STAMP(a, gw, 3);
    // Q rows of the segment being scored (qr) and of the next one (qn).  The
    // next segment's rows are loaded as soon as it is known, at the start of
    // the current segment's last chunk, so they have long arrived when the
    // segment switches; loading them at the switch made the first score of
    // the new segment wait for that load, and so for every K/V load issued
    // before it (one memory latency per switch).
    typename Eng::Q qr, qn;
    typename Eng::State st;
    int max_lo = 0, min_hi = 0;
    typename Eng::Buf buf[NBUF];
    // loads of group g of chunk c (clamped to its last group)
    auto load_group = [&](typename Eng::Buf& x, const Chunk& c, const PageWindow& w, int g) {
      Eng::template load<PAGE_POW2>(x, a, c.sg.kvh, c.cb * GPB + min(g, c.ng - 1), c.kb, c.ke, w,
                                    ps_shift, ln);
    };
#pragma unroll
    for (int s = 0; s < PF; ++s) load_group(buf[s], cur, pw, s);
    PKVD_STAMP(a, gw, 4);
    Eng::fetch_q(a, cur.sg, ln, qr);
    if (cur.last && nxt.valid) Eng::fetch_q(a, nxt.sg, ln, qn);
    Eng::reset(a, cur.sg, ln, st, max_lo, min_hi);
    PKVD_STAMP(a, gw, 2);

    for (;;) {
#ifdef PKVD_TRACE
      n_chunk++;
      n_blk += cur.ce - cur.cb;
#endif
      {
        const int g0 = cur.cb * GPB;
        const int rounds = cur.ngp / NBUF;
        auto score = [&](int s, int i) {
          if (i < cur.ng) {   // padding groups are not scored
            const int j0 = (g0 + i) * KPG;
            const bool full = j0 >= max_lo && j0 + KPG - 1 <= min_hi;
            Eng::score(st, buf[s], qr, a.scale_log2, full, j0, ln);
          }
        };
        // each sub-step issues the loads of the group PF ahead, then scores its own
        for (int rd = 0; rd + 1 < rounds; ++rd) {
#pragma unroll
          for (int s = 0; s < NBUF; ++s) {
            load_group(buf[(s + PF) % NBUF], cur, pw, rd * NBUF + s + PF);
            score(s, rd * NBUF + s);
          }
        }
        // last round: sub-steps s >= NBUF - PF load groups s + PF - NBUF of the
        // next chunk (at the end of the slice: this chunk's last group again)
        const Chunk& lc = nxt.valid ? nxt : cur;
        const PageWindow lw = nxt.valid ? pwn : pw;
        const int i0 = (rounds - 1) * NBUF;
#pragma unroll
        for (int s = 0; s < NBUF; ++s) {
          if (s + PF < NBUF) load_group(buf[(s + PF) % NBUF], cur, pw, i0 + s + PF);
          else load_group(buf[(s + PF) % NBUF], lc, lw, nxt.valid ? s + PF - NBUF : cur.ng - 1);
          score(s, i0 + s);
        }
      }
      if (cur.last) {
        // the segment is done: the next one's Q rows (loaded a chunk ago)
        if (nxt.valid) qr = qn;
        // the whole unit's output, or this piece's partial
        const Segment& sg = cur.sg;
        const int unit = (sg.b * a.Hkv + sg.kvh) * a.row_tiles + sg.tile;
        Eng::finish(st, ln);
        const int slot = 2 * gw + sg.side;
#pragma unroll
        for (int it = 0; it < Eng::kItems; ++it) {
          int r, d0;
          float M, Lsum, O[8];
          const bool ok = Eng::item(st, ln, it, r, d0, M, Lsum, O);
          const int row = sg.tile * RT + r;
          if (!(ok && row < sg.R)) continue;   // padding rows are neither stored nor kept
          if (sg.whole) {
            const int ti = row / a.g, qhead = sg.kvh * a.g + (row - ti * a.g);
            store_item<D, Eng::kItemDims>(a, s_sink, ((int64_t)sg.row0 + ti) * a.Hq + qhead,
                                          qhead, d0, d0 == 0, M, Lsum, O);
          } else {
            store_partial<Eng, D>(a, slot, ln, r, d0, M, Lsum, O);
          }
        }
        if (!sg.whole) {
          const int k = sg.side;
          pend_unit[k] = unit;
          pend_n[k] = sg.blk_end - sg.blk_begin;
          pend_vs[k] = sg.vstart;
          pend_nb[k] = sg.uend - sg.ustart;
        }
#ifdef PKVD_TRACE
        if (n_seg++ == 0) PKVD_STAMP(a, gw, 5);
#endif
      }
      if (!nxt.valid) break;
      cur = nxt;
      pw = pwn;
      if (cur.first) Eng::reset(a, cur.sg, ln, st, max_lo, min_hi);
      nxt = next_chunk(cur);
      if (nxt.valid) pwn = fetch_pages(nxt);
      if (cur.last && nxt.valid) Eng::fetch_q(a, nxt.sg, ln, qn);
    }
    PKVD_STAMP(a, gw, 6);

    if (!a.merge_kernel && (pend_unit[0] >= 0 || pend_unit[1] >= 0)) {
      // Tickets of the cut units: blocks delivered, once this slice's
      // partial states are stored.  The wave whose ticket completes a unit
      // merges it.  Ordering (agent scope): every partial-state store is an
      // agent-scope atomic store, which on this hardware writes through to
      // device-coherent memory; the wave waits until all of its stores have
      // completed (vmcnt 0, with compiler barriers on both sides so that no
      // memory access moves across the wait) before lane 0 adds to the
      // counter.  That is the part of a release fence these stores need; the
      // fence itself would also write back this XCD's whole L2 (non-atomic
      // data the merge never reads), which measured 19 us per call on the
      // 64-request Llama-3-8B batch (128 vs 110 us).  The completing wave
      // executes an agent-scope acquire fence before its first partial-state
      // load (measured free), and reads with agent-scope atomic loads.
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      int prev[2] = {0, 0};
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (pend_unit[k] >= 0 && lane == 0)
          prev[k] = __hip_atomic_fetch_add(&a.counters[pend_unit[k]], pend_n[k], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      // the units this wave completes; both merges' first loads go out
      // together
      bool done[2];
#pragma unroll
      for (int k = 0; k < 2; ++k)
        done[k] = pend_unit[k] >= 0 && uniform(prev[k]) + pend_n[k] == pend_nb[k];
      if (done[0] || done[1]) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        UnitMerge<Eng, D> mg[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if (!done[k]) continue;
          if (lane == 0) store_coherent(&a.counters[pend_unit[k]], 0);   // ready for the next call
          const int per_req = a.Hkv * a.row_tiles;
          const int b = UnitMerge<Eng, D>::kSkip ? UnitMerge<Eng, D>::quot_pow2(pend_unit[k], per_req)
                                                 : pend_unit[k] / per_req;
          const ReqRows rows = req_info(a, s_nlen, s_qo, b).rows;
          mg[k].begin(a, sl_, pend_unit[k], pend_vs[k], pend_nb[k], rows, ln, lane);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k)
          if (done[k]) mg[k].finish(a, s_sink, sl_, ln, lane);
      }
    }
  }
  PKVD_STAMP(a, gw, 7);
#ifdef PKVD_TRACE
  PKVD_COUNT(a, gw, 8, n_seg);
  PKVD_COUNT(a, gw, 9, n_chunk);
  PKVD_COUNT(a, gw, 10, n_blk);
  {
    uint32_t hwid = __builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11));   // HW_ID
    uint32_t xcc = __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (3 << 11));    // XCC_ID
    PKVD_COUNT(a, gw, 11, ((uint64_t)xcc << 32) | hwid);
  }
#endif
}

// Merge kernel (for plans whose cut units leave large partial states): one
// wave per (unit, row of its tile), launched after the decode kernel.  Lane c
// takes candidate c (64 at a time, written or not); the batch maximum of the
// written pieces' LSEs and their weights 2^(lse - max) come from wave
// reductions, and every lane accumulates its D / 64 output dims over those
// pieces in block order, eight pieces' loads in flight.  Each lane owns its
// dims, so every sum has a fixed order for a given set of pieces.  Writes out
// (sink in the denominator) and the base-2 LSE.  A unit with fewer than two
// written partials was whole in one slice and is left as the decode kernel
// wrote it.
constexpr int kMergeWaves = 4;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <class Eng, int D>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(const DecodeArgs a) {
  constexpr int RT = Eng::kRows, NDL = D / 64;   // dims per lane
  const int lane = threadIdx.x & 63;
  const int pair = (int)blockIdx.x * kMergeWaves + (int)(threadIdx.x >> 6);
  const int per_req = a.Hkv * a.row_tiles;
  const int unit = pair / RT, r = pair - unit * RT;
  const int b = unit / per_req, uidx = unit - b * per_req;
  if (b >= a.B) return;
  const int kvh = uidx / a.row_tiles, tile = uidx - kvh * a.row_tiles;
  const int row = tile * RT + r;
  // every per-request value in one round of loads (all indices are in range)
  const int nraw = a.seq_lens[b];
  const int q0 = a.qo ? a.qo[b] : 0, q1 = a.qo ? a.qo[b + 1] : 0;
  const int T = a.ws_pref[a.B], TV = a.ws_vpref[a.B];
  const int pref_b = a.ws_pref[b], vpref_b = a.ws_vpref[b];
  const ReqRows rows = a.qo ? rows_of(a, clamp_row(a, q0), clamp_row(a, q1), b)
                            : ReqRows{b * a.Lq, a.Lq};
  if (row >= a.g * rows.lq) return;   // a padding row, or a tile the request does not have
  const UnitRange u = unit_range_n(a, nraw, rows.lq);
  if (u.nblk == 0) return;
  // the unit's place among its request's units (kv head major, then tiles)
  const int ub = a.qo ? kvh * tiles_of(a, rows.lq) + tile : uidx;
  int NW;
  const Slices sl_ = grid_slices(a, TV, T, NW);
  const int64_t us = pref_b + (int64_t)ub * u.nblk, ue = us + u.nblk;
  const int64_t vs = vpref_b + (int64_t)ub * unit_vspan(a, u.nblk);
  if (ue > T) return;
  const UnitPieces up = unit_pieces(sl_, vs, a.seg_cost, u.nblk);
  if (up.n == 1) return;   // inside one slice: written whole by the decode kernel
  float M = -INFINITY, W = 0.f, acc[NDL];
#pragma unroll
  for (int e = 0; e < NDL; ++e) acc[e] = 0.f;
  int pos[NDL];
#pragma unroll
  for (int e = 0; e < NDL; ++e) pos[e] = Eng::ppos(r, lane * NDL + e);
  int written = 0;   // candidates that wrote a partial state
  constexpr int kDepth = 8;
  for (int c0 = 0; c0 < up.n; c0 += 64) {
    const int c = c0 + lane;
    int slot = 0;
    bool valid = false;
    if (c < up.n) slot = candidate_slot(up, sl_, vs, c, valid);
    uint64_t m = __builtin_amdgcn_ballot_w64(valid);
    if (m == 0) continue;
    written += __builtin_popcountll(m);
    // The batch's LSEs and the outputs of its first kDepth written pieces
    // in one round of loads (the outputs' addresses need only the slots);
    // off entries of a group read the batch's first written piece (finite
    // values) with weight 0.
    const float l = valid ? a.ws_lse[(int64_t)slot * RT + r] : -INFINITY;
    const int sl0 = __builtin_amdgcn_readlane(slot, (int)__builtin_ctzll(m));
    int qs[kDepth];
    float oq[kDepth][NDL];
#pragma unroll
    for (int e = 0; e < kDepth; ++e) {
      const bool on = m != 0;
      qs[e] = on ? (int)__builtin_ctzll(m) : -1;
      m = on ? m & (m - 1) : m;
      const int sl = on ? __builtin_amdgcn_readlane(slot, qs[e]) : sl0;
      const float* po = a.ws_o + (int64_t)sl * RT * D;
#pragma unroll
      for (int x = 0; x < NDL; ++x) oq[e][x] = po[pos[x]];
    }
    const float Mn = fmaxf(M, wave_max(l));
    const float wt = valid ? rescale(l, Mn) : 0.f;
    const float sc = rescale(M, Mn);
    W = W * sc + wave_sum(wt);
#pragma unroll
    for (int e = 0; e < NDL; ++e) acc[e] *= sc;
    M = Mn;
    auto weight_of = [&](int q) {   // piece q's weight (0 for an off entry, q = -1)
      const float w = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), q < 0 ? 0 : q));
      return q < 0 ? 0.f : w;
    };
#pragma unroll
    for (int e = 0; e < kDepth; ++e) {
      const float w_q = weight_of(qs[e]);
#pragma unroll
      for (int x = 0; x < NDL; ++x) acc[x] = fmaf(w_q, oq[e][x], acc[x]);
    }
    while (m) {   // uniform: the batch's further written pieces, in order
      float wq[kDepth];
#pragma unroll
      for (int e = 0; e < kDepth; ++e) {
        const bool on = m != 0;
        const int q = on ? (int)__builtin_ctzll(m) : -1;
        m = on ? m & (m - 1) : m;
        wq[e] = weight_of(q);
        const int sl = on ? __builtin_amdgcn_readlane(slot, q) : sl0;
        const float* po = a.ws_o + (int64_t)sl * RT * D;
#pragma unroll
        for (int x = 0; x < NDL; ++x) oq[e][x] = po[pos[x]];
      }
#pragma unroll
      for (int e = 0; e < kDepth; ++e)
#pragma unroll
        for (int x = 0; x < NDL; ++x) acc[x] = fmaf(wq[e], oq[e][x], acc[x]);
    }
  }
  if (written < 2) return;   // whole in one slice: written by the decode kernel
  const int ti = row / a.g, qhead = kvh * a.g + (row - ti * a.g);
  const int64_t rowhead = ((int64_t)rows.row0 + ti) * a.Hq + qhead;
  const bool has_sink = a.sinks != nullptr;
  const float sink = has_sink ? a.sinks[qhead] : 0.f;
  // acc / W is the merged normalised output; final_value divides by W + sink
  float x[NDL];
#pragma unroll
  for (int e = 0; e < NDL; ++e) x[e] = final_value(has_sink, sink, M, W, acc[e], a.out_scale);
  if constexpr (NDL == 2) {
    store_out<2>(a, rowhead * D + 2 * lane, x);
  } else {
    const int64_t off = rowhead * D + lane;
    if (a.out_type == kOutF32) static_cast<float*>(a.out)[off] = x[0];
    else if (a.out_type == kOutBf16) static_cast<uint16_t*>(a.out)[off] = Fmt<true>::encode(x[0]);
    else static_cast<uint16_t*>(a.out)[off] = Fmt<false>::encode(x[0]);
  }
  if (a.lse && lane == 0) a.lse[rowhead] = W > 0.f ? M + log2f(W) : -INFINITY;
}

// blocks in flight ahead of the scoring, and waves per SIMD the register
// budget is fitted to, per engine
#ifndef PKVD_PF4
#define PKVD_PF4 3
#endif
#ifndef PKVD_WPE4
#define PKVD_WPE4 1
#endif
#ifndef PKVD_PF8
#define PKVD_PF8 1
#endif
#ifndef PKVD_WPE8
#define PKVD_WPE8 2
#endif
#ifndef PKVD_PF16
#define PKVD_PF16 2
#endif
#ifndef PKVD_WPE16
#define PKVD_WPE16 1
#endif
#ifndef PKVD_PF16_D64
#define PKVD_PF16_D64 2
#endif
#ifndef PKVD_WPE16_D64
#define PKVD_WPE16_D64 2
#endif

template <int RT>
constexpr int valu_pf() { return RT == 4 ? PKVD_PF4 : PKVD_PF8; }
template <int RT>
constexpr int valu_wpe() { return RT == 4 ? PKVD_WPE4 : PKVD_WPE8; }
template <int D>
constexpr int mfma_pf() { return D == 64 ? PKVD_PF16_D64 : PKVD_PF16; }
// a D = 64 block takes half the registers: one more wave per SIMD fits
template <int D>
constexpr int mfma_wpe() { return D == 64 ? PKVD_WPE16_D64 : PKVD_WPE16; }

// The decode and merge kernels of one (head_dim, element type) for a path
// and tile height (nullptr where none is built).
template <int D, bool BF16>
KernelPair select_kernels(int path, int rows_per_tile, bool pow2) {
  KernelPair k{nullptr, nullptr};
  if (path == kPathMfma) {
    if (rows_per_tile != 16) return k;
    k.decode = pow2 ? &decode_kernel<MfmaEngine<D, BF16>, D, true, mfma_pf<D>(), mfma_wpe<D>()>
                    : &decode_kernel<MfmaEngine<D, BF16>, D, false, mfma_pf<D>(), mfma_wpe<D>()>;
    k.merge = &merge_kernel<MfmaEngine<D, BF16>, D>;
  } else if (rows_per_tile == 4) {
    k.decode = pow2 ? &decode_kernel<ValuEngine<D, 4, BF16>, D, true, valu_pf<4>(), valu_wpe<4>()>
                    : &decode_kernel<ValuEngine<D, 4, BF16>, D, false, valu_pf<4>(), valu_wpe<4>()>;
    k.merge = &merge_kernel<ValuEngine<D, 4, BF16>, D>;
  } else if (rows_per_tile == 8) {
    k.decode = pow2 ? &decode_kernel<ValuEngine<D, 8, BF16>, D, true, valu_pf<8>(), valu_wpe<8>()>
                    : &decode_kernel<ValuEngine<D, 8, BF16>, D, false, valu_pf<8>(), valu_wpe<8>()>;
    k.merge = &merge_kernel<ValuEngine<D, 8, BF16>, D>;
  }
  return k;
}

}  // namespace dev
}  // namespace pkvd
