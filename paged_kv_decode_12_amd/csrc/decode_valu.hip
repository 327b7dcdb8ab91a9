// decode_valu.hip -- paged-KV decode, VALU dot-product path (rows per tile <= 8).
//
// Operation: flashinfer.cudnn.cudnn_batch_decode_with_kv_cache (Parameters,
// Note / LSE convention).  A unit of work is (request b, kv head, row tile);
// the rows of a tile are the Hq/Hkv query heads sharing the kv head times the
// q_len_per_req query tokens, so every K/V byte a wave loads serves all of
// them (grouped-query packing).
//
// Schedule (persistent, balanced): one grid of exactly the resident number of
// waves.  Each workgroup rebuilds, from seq_lens_kv, the prefix of the linear
// block space of all units; wave w then streams its own contiguous slice
// [w T / NW, (w + 1) T / NW) of that space, crossing unit boundaries as
// needed.  Every wave does the same amount of work whatever the mix of
// lengths.  A unit wholly inside one wave is written directly; a unit cut by
// wave boundaries leaves a partial state per piece, and the last piece to
// arrive (atomic ticket) merges them with the base-2 LSE rule (Note / LSE
// convention: base-2 LSE states are what the cascade merge consumes).  The
// ranges come from device data only, so planning never reads the lengths on
// the host.
//
// Inside a wave (LPK = D / 8 lanes per key, KPS = 64 / LPK keys per step):
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
//    (one column per lane), read with readlane / ds_bpermute; the next
//    chunk's page ids and Q rows are fetched before the current segment's
//    epilogue, and tickets are read only after the whole range is streamed;
//  * at a segment's end the KPS streams merge by DPP and lane-pair swaps.
#include "decode_common.h"

namespace pkvd {
namespace {

using namespace dev;

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

// Page ids of a chunk's block-table columns col0 .. col0 + 127, one column per
// lane in each of two registers.
struct PageWindow {
  int p0, p1;   // columns col0 + lane, col0 + 64 + lane
  int col0;
};

// Page of column col0 + c for a wave-uniform c.
__device__ __forceinline__ int page_uniform(const PageWindow& w, int c) {
  return __builtin_amdgcn_readlane(c < 64 ? w.p0 : w.p1, c & 63);
}
// Page of column col0 + c for a per-lane c.
__device__ __forceinline__ int page_lane(const PageWindow& w, int c) {
  const int a0 = __builtin_amdgcn_ds_bpermute((c & 63) << 2, w.p0);
  const int a1 = __builtin_amdgcn_ds_bpermute((c & 63) << 2, w.p1);
  return c < 64 ? a0 : a1;
}

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

// Writes one row's 8 output values (dims part*8 ..) and, from part 0, its LSE.
template <int D, bool BF16>
__device__ __forceinline__ void store_row(const DecodeArgs& a, int rowhead, int qhead, int part,
                                          float M, float L, const float (&O)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    w[u] = Fmt<BF16>::pack2(final_value<BF16>(a, qhead, M, L, O[2 * u]),
                            final_value<BF16>(a, qhead, M, L, O[2 * u + 1]));
  *reinterpret_cast<u32x4*>(a.out + (int64_t)rowhead * D + part * 8) =
      u32x4{w[0], w[1], w[2], w[3]};
  if (a.lse && part == 0) a.lse[rowhead] = L > 0.f ? M + log2f(L) : -INFINITY;
}

// Partial state layout of one slot: [row][e][part] (LPK consecutive floats per
// store instruction and key group), then the row LSEs in ws_lse.
template <int D, int RT>
__device__ __forceinline__ int64_t partial_index(int slot, int r, int e, int part) {
  return ((int64_t)slot * RT * 8 + r * 8 + e) * Geo<D>::LPK + part;
}

// Merges the partial states of one unit's pieces (waves w_first .. w_last) for
// row r (the calling lane's share: dims part*8 ..) and writes the final row.
// Four pieces' loads are in flight at a time; the running max is updated per
// group of four.
template <int D, int RT, bool BF16>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, int64_t T, int NW,
                                             int64_t ustart, int w_first, int w_last, int r,
                                             int part, int rowhead, int qhead) {
  float Mx = -INFINITY, W = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int w = w_first; w <= w_last; w += 4) {
    float l4[4], v4[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ww = min(w + u, w_last);
      const int sl = 2 * ww + (wave_begin(T, NW, ww) >= ustart ? 0 : 1);
      const float lv = load_coherent(a.ws_lse + (int64_t)sl * RT + r);
      l4[u] = w + u <= w_last ? lv : -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v4[u][e] = load_coherent(a.ws_o + partial_index<D, RT>(sl, r, e, part));
    }
    const float Mn = fmaxf(Mx, fmaxf(fmaxf(l4[0], l4[1]), fmaxf(l4[2], l4[3])));
    const float sc = rescale(Mx, Mn);
    W *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wt = rescale(l4[u], Mn);
      W += wt;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wt, v4[u][e], acc[e]);
    }
    Mx = Mn;
  }
  // acc / W is the merged normalised output; final_value divides by W + sink
  store_row<D, BF16>(a, rowhead, qhead, part, Mx, W, acc);
}

template <int D, int RT, bool BF16, bool PAGE_POW2, int PF, int WPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void decode_valu(const DecodeArgs a) {
  using G = Geo<D>;
  constexpr int NBUF = PF + 1;
  constexpr int kWindow = 128;                        // block-table columns per chunk
  constexpr int RPG = (RT + G::KPS - 1) / G::KPS;     // output rows per key group
  extern __shared__ int lds[];
  int* s_scan = lds;                                  // kThreads
  int* s_pref = lds + kThreads;                       // B + 1
  int* s_nlen = s_pref + a.B + 1;                     // B

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int kq = lane / G::LPK, part = lane % G::LPK;

  const int gw0 = (int)blockIdx.x * kWaves + wave;
  PKVD_STAMP(a, gw0, 0);
  const int64_t T = build_prefix<BF16>(a, s_pref, s_nlen, s_scan);
  PKVD_STAMP(a, gw0, 1);
  if (T == 0) return;
  // waves that take part: at most one per min_wave_blocks blocks (and <= T)
  int64_t nw = T / a.min_wave_blocks;
  nw = nw < 1 ? 1 : (nw > a.num_waves ? a.num_waves : nw);
  const int NW = (int)nw;
  const int gw = (int)blockIdx.x * kWaves + wave;
  if (gw >= NW) return;
  const int64_t lo = wave_begin(T, NW, gw), hi = wave_begin(T, NW, gw + 1);
  const int R = a.g * a.Lq;
  const int ps_shift = PAGE_POW2 ? __builtin_ctz(a.ps) : 0;
  // blocks per chunk: (blocks * 16 - 1) / ps + 2 <= kWindow columns
  const int chunk_blocks = max(1, ((kWindow - 2) * a.ps + 1) / kBlockKeys);

  // A chunk: blocks [cb, ce) of segment sg (a unit's slice of this wave's range).
  struct Chunk {
    Segment sg;
    int cb, ce, kb, ke;
    bool first, last;   // first / last chunk of its segment
  };
  auto make_chunk = [&](const Segment& sg, int cb) {
    Chunk c;
    c.sg = sg;
    c.cb = cb;
    c.ce = min(sg.blk_end, cb + chunk_blocks);
    c.kb = max(sg.u.key_lo, cb * kBlockKeys);
    c.ke = min(sg.u.n, c.ce * kBlockKeys);
    c.first = cb == sg.blk_begin;
    c.last = c.ce == sg.blk_end;
    return c;
  };
  // page ids of a chunk's columns, clamped into the pool (issued early)
  auto fetch_pages = [&](const Chunk& c) {
    PageWindow w;
    w.col0 = c.kb / a.ps;
    const int ncol = (c.ke - 1) / a.ps - w.col0 + 1;
    const int32_t* row = a.bt + (int64_t)c.sg.b * a.bt_sr + w.col0;
    const int p0 = row[min(lane, ncol - 1)];
    const int p1 = row[min(64 + lane, ncol - 1)];
    w.p0 = (unsigned)p0 < (unsigned)a.P ? p0 : a.P - 1;
    w.p1 = (unsigned)p1 < (unsigned)a.P ? p1 : a.P - 1;
    return w;
  };
  // Q rows of a segment's tile (rr = tile * RT + r -> token rr / g, head rr % g):
  // the lane's 16-byte piece of each row
  auto fetch_q = [&](const Segment& sg, u32x4 (&q)[RT]) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int rr = sg.tile * RT + r;
      const bool live = rr < R;
      const int i = live ? rr / a.g : 0;
      const int hl = live ? rr - i * a.g : 0;
      const uint16_t* qp = a.q + (int64_t)(sg.b * a.Lq + i) * a.q_sr +
                           (int64_t)(sg.kvh * a.g + hl) * a.q_sh + part * 8;
      q[r] = live ? load16(qp) : u32x4{0, 0, 0, 0};
    }
  };

  // pieces of units shared with other waves: at most the first and the last
  // segment of the range; their tickets are read after the range is done
  int pend_prev[2] = {-1, -1}, pend_unit[2] = {0, 0};
  int64_t pend_ustart[2] = {0, 0}, pend_uend[2] = {0, 0};
  int pend_tile[2] = {0, 0}, pend_b[2] = {0, 0}, pend_kvh[2] = {0, 0};

  const Segment sg0 = locate(a, s_pref, s_nlen, lo, lo, hi);
  Chunk ch = make_chunk(sg0, sg0.blk_begin);
  PageWindow pw = fetch_pages(ch);
  u32x4 qr[RT];
  fetch_q(ch.sg, qr);

  Stream<RT> st;
  int lo_r[RT], hi_r[RT];
  int max_lo = 0, min_hi = 0;
#ifdef PKVD_TRACE
  int n_seg = 0, n_chunk = 0, n_blk = 0;
#endif
  PKVD_STAMP(a, gw, 2);
  for (;;) {
    const Segment& sg = ch.sg;
    if (ch.first) {
      max_lo = sg.u.key_lo;
      min_hi = sg.u.n - 1;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int rr = sg.tile * RT + r;
        const bool live = rr < R;
        const int diag = sg.u.n - a.Lq + (live ? rr / a.g : 0);
        const int rlo = max(a.window_left < 0 ? 0 : diag - a.window_left, 0);
        lo_r[r] = live ? rlo : 1;     // dead rows see nothing
        hi_r[r] = live ? diag : 0;
        if (live) {
          max_lo = max(max_lo, rlo);
          min_hi = min(min_hi, diag);
        }
        st.m[r] = -INFINITY;
        st.l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.o[r][e] = 0.f;
      }
    }

    // stream the chunk's key groups with loads PF groups ahead
#ifdef PKVD_TRACE
    if (n_chunk == 0) PKVD_STAMP(a, gw, 3);
    n_chunk++;
    n_blk += ch.ce - ch.cb;
#endif
    {
      const int g0 = ch.cb * G::GPB, ng = (ch.ce - ch.cb) * G::GPB;
      const int kb = ch.kb, ke = ch.ke, kvh = sg.kvh;
      KeyRegs buf[NBUF];
      auto grp_of = [&](int i) { return g0 + min(i, ng - 1); };
      auto score = [&](const KeyRegs& x, int i) {
        const int j0 = (g0 + i) * G::KPG;
        const bool full = j0 >= max_lo && j0 + G::KPG - 1 <= min_hi;
        score_group<D, RT, BF16>(st, x, qr, a.scale_log2, full, j0, kq, lo_r, hi_r);
      };
#pragma unroll
      for (int s = 0; s < PF; ++s)
        load_group<D, PAGE_POW2>(buf[s], a, kvh, grp_of(s), kb, ke, pw, ps_shift, kq, part);
      // full rounds: each sub-step issues the loads of the group PF ahead (the
      // last group again near the end: a cache hit), then scores its own group
      const int rounds = ng / NBUF;
      for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
        for (int s = 0; s < NBUF; ++s) {
          const int i = rd * NBUF + s;
          load_group<D, PAGE_POW2>(buf[(s + PF) % NBUF], a, kvh, grp_of(i + PF), kb, ke, pw,
                                   ps_shift, kq, part);
          score(buf[s], i);
        }
      }
      // tail: the remaining ng % NBUF <= PF groups are already in flight
      const int i0 = rounds * NBUF;
#pragma unroll
      for (int s = 0; s < PF; ++s)
        if (i0 + s < ng) score(buf[s], i0 + s);
    }

#ifdef PKVD_TRACE
    if (n_chunk == 1) PKVD_STAMP(a, gw, 4);
#endif
    if (!ch.last) {            // next chunk of the same segment
      ch = make_chunk(sg, ch.ce);
      pw = fetch_pages(ch);
      continue;
    }

    // the segment is done: finish it
    merge_streams<D, RT>(st);
    if (sg.whole) {
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        const int r = kq + i * G::KPS;           // rows of this key group
        float M = -INFINITY, L = 0.f, O[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) O[e] = 0.f;
#pragma unroll
        for (int rr = 0; rr < RT; ++rr)
          if (rr == r) {
            M = st.m[rr];
            L = st.l[rr];
#pragma unroll
            for (int e = 0; e < 8; ++e) O[e] = st.o[rr][e];
          }
        const int row = sg.tile * RT + r;
        if (r < RT && row < R) {
          const int ti = row / a.g, qhead = sg.kvh * a.g + (row - ti * a.g);
          store_row<D, BF16>(a, (sg.b * a.Lq + ti) * a.Hq + qhead, qhead, part, M, L, O);
        }
      }
    } else {
      // a piece of a unit shared with other waves: leave the partial state,
      // then take a ticket (its value is read once the range is done)
      const int slot = 2 * gw + sg.side;
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        const int r = kq + i * G::KPS;
        float M = -INFINITY, L = 0.f, O[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) O[e] = 0.f;
#pragma unroll
        for (int rr = 0; rr < RT; ++rr)
          if (rr == r) {
            M = st.m[rr];
            L = st.l[rr];
#pragma unroll
            for (int e = 0; e < 8; ++e) O[e] = st.o[rr][e];
          }
        if (r < RT) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            store_coherent(a.ws_o + partial_index<D, RT>(slot, r, e, part), L > 0.f ? O[e] / L : 0.f);
          if (part == 0)
            store_coherent(a.ws_lse + (int64_t)slot * RT + r, L > 0.f ? M + log2f(L) : -INFINITY);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);   // partial stores complete before the ticket
      const int unit = (sg.b * a.Hkv + sg.kvh) * a.row_tiles + sg.tile;
      int prev = 0;
      if (lane == 0) prev = atomicAdd(&a.counters[unit], 1);
      auto remember = [&](int k) {
        pend_prev[k] = prev;
        pend_unit[k] = unit;
        pend_ustart[k] = sg.ustart;
        pend_uend[k] = sg.uend;
        pend_tile[k] = sg.tile;
        pend_b[k] = sg.b;
        pend_kvh[k] = sg.kvh;
      };
      if (sg.side == 0) remember(0);
      else remember(1);
    }
#ifdef PKVD_TRACE
    if (n_seg++ == 0) PKVD_STAMP(a, gw, 5);
#endif
    const int64_t next = sg.ustart + (sg.blk_end - sg.u.first_blk);
    if (next >= hi) break;
    const Segment ns = locate(a, s_pref, s_nlen, next, lo, hi);
    ch = make_chunk(ns, ns.blk_begin);
    pw = fetch_pages(ch);
    fetch_q(ns, qr);
  }

  PKVD_STAMP(a, gw, 6);
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
  // merge the units whose last piece this wave delivered
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    const int unit = pend_unit[side];
    const bool had = uniform(pend_prev[side] >= 0 ? 1 : 0) != 0;
    if (!had) continue;
    const int w_first = wave_of(pend_ustart[side], T, NW);
    const int w_last = wave_of(pend_uend[side] - 1, T, NW);
    const int prev = uniform(pend_prev[side]);
    if (prev != w_last - w_first) continue;
    if (lane == 0) a.counters[unit] = 0;   // ready for the next call
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int r = kq + i * G::KPS;
      const int row = pend_tile[side] * RT + r;
      if (!(r < RT && row < R)) continue;
      const int ti = row / a.g, qhead = pend_kvh[side] * a.g + (row - ti * a.g);
      merge_pieces<D, RT, BF16>(a, T, NW, pend_ustart[side], w_first, w_last, r, part,
                                (pend_b[side] * a.Lq + ti) * a.Hq + qhead, qhead);
    }
  }
  PKVD_STAMP(a, gw, 7);
}

// blocks in flight ahead of the scoring
#ifndef PKVD_PF4
#define PKVD_PF4 1
#endif
#ifndef PKVD_PF8
#define PKVD_PF8 1
#endif

using KernelFn = void (*)(DecodeArgs);

// waves per SIMD the register budget is fitted to
#ifndef PKVD_WPE4
#define PKVD_WPE4 4
#endif
#ifndef PKVD_WPE8
#define PKVD_WPE8 2
#endif

template <int D, int RT, bool BF16, bool POW2>
KernelFn kernel_of() {
  constexpr int pf = RT == 4 ? PKVD_PF4 : PKVD_PF8;
  constexpr int wpe = RT == 4 ? PKVD_WPE4 : PKVD_WPE8;
  return &decode_valu<D, RT, BF16, POW2, pf, wpe>;
}

KernelFn select(int rows_per_tile, int head_dim, bool bf16, bool pow2) {
#define PKVD_SEL(D, RT, BF, P2)                                                          \
  if (head_dim == D && rows_per_tile == RT && bf16 == BF && pow2 == P2) \
    return kernel_of<D, RT, BF, P2>();
#define PKVD_SEL_P2(D, RT, BF) PKVD_SEL(D, RT, BF, true) PKVD_SEL(D, RT, BF, false)
#define PKVD_SEL_BF(D, RT) PKVD_SEL_P2(D, RT, true) PKVD_SEL_P2(D, RT, false)
  PKVD_SEL_BF(128, 4)
  PKVD_SEL_BF(128, 8)
  PKVD_SEL_BF(64, 4)
  PKVD_SEL_BF(64, 8)
#undef PKVD_SEL_BF
#undef PKVD_SEL_P2
#undef PKVD_SEL
  return nullptr;
}

bool page_pow2(int ps) { return ps >= kBlockKeys && (ps & (ps - 1)) == 0; }

}  // namespace

// scan scratch, prefix, lengths
size_t decode_lds_bytes(int B) { return sizeof(int) * ((size_t)kThreads + 2 * (size_t)B + 1); }

int decode_blocks_per_cu(int path, int rows_per_tile, int head_dim, bool bf16, bool pow2,
                         size_t lds_bytes) {
  if (path != kPathValu) return 0;
  KernelFn k = select(rows_per_tile, head_dim, bf16, pow2);
  if (!k) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k), kThreads,
                                                   lds_bytes) != hipSuccess)
    return 0;
  return n;
}

hipError_t launch_decode(const DecodeArgs& a, int path, int rows_per_tile, bool bf16,
                         hipStream_t stream) {
  if (path != kPathValu) return hipErrorInvalidValue;
  KernelFn k = select(rows_per_tile, a.D, bf16, page_pow2(a.ps));
  if (!k) return hipErrorInvalidValue;
  const dim3 grid((a.num_waves + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(k, grid, dim3(kThreads), decode_lds_bytes(a.B), stream, a);
  return hipGetLastError();
}

}  // namespace pkvd
