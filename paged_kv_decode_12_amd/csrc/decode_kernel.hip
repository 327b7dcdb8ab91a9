// decode_kernel.hip -- the persistent paged-KV decode kernel and its launch.
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
//    (one column per lane), read with readlane / ds_bpermute; the next
//    chunk's page ids and Q rows are fetched before the current segment's
//    epilogue, and tickets are read only after the whole range is streamed;
//  * at a segment's end the KPS streams merge by DPP and lane-pair swaps.
#include "engine_mfma.h"
#include "engine_valu.h"

namespace pkvd {
namespace {

using namespace dev;

// Writes one output item (N = 8 or 4 consecutive dims from d0) and, from the
// row's lead lane, its LSE.
template <int D, int N, bool BF16>
__device__ __forceinline__ void store_item(const DecodeArgs& a, int rowhead, int qhead, int d0,
                                           bool lead, float M, float L, const float (&O)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int u = 0; u < N / 2; ++u)
    w[u] = Fmt<BF16>::pack2(final_value<BF16>(a, qhead, M, L, O[2 * u]),
                            final_value<BF16>(a, qhead, M, L, O[2 * u + 1]));
  if constexpr (N == 8)
    *reinterpret_cast<u32x4*>(a.out + (int64_t)rowhead * D + d0) = u32x4{w[0], w[1], w[2], w[3]};
  else
    *reinterpret_cast<uint2*>(a.out + (int64_t)rowhead * D + d0) = make_uint2(w[0], w[1]);
  if (a.lse && lead) a.lse[rowhead] = L > 0.f ? M + log2f(L) : -INFINITY;
}

// Merges the partial states of one unit's pieces (waves w_first .. w_last) for
// one output item (row r, dims d0 ..) and writes the final values.  Four
// pieces' loads are in flight at a time; the running max is updated per group
// of four.
template <class Eng, int D, bool BF16>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, int64_t T, int NW,
                                             int64_t ustart, int w_first, int w_last,
                                             const typename Eng::Lane& ln, int r, int d0,
                                             int rowhead, int qhead) {
  constexpr int RT = Eng::kRows, N = Eng::kItemDims;
  float Mx = -INFINITY, W = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int w = w_first; w <= w_last; w += 4) {
    float l4[4], v4[4][N];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ww = min(w + u, w_last);
      const int sl = 2 * ww + (wave_begin(T, NW, ww) >= ustart ? 0 : 1);
      const float lv = load_coherent(a.ws_lse + (int64_t)sl * RT + r);
      l4[u] = w + u <= w_last ? lv : -INFINITY;
#pragma unroll
      for (int e = 0; e < N; ++e)
        v4[u][e] = load_coherent(a.ws_o + (int64_t)sl * RT * D + Eng::pidx(ln, r, e));
    }
    const float Mn = fmaxf(Mx, fmaxf(fmaxf(l4[0], l4[1]), fmaxf(l4[2], l4[3])));
    const float sc = rescale(Mx, Mn);
    W *= sc;
#pragma unroll
    for (int e = 0; e < N; ++e) acc[e] *= sc;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wt = rescale(l4[u], Mn);
      W += wt;
#pragma unroll
      for (int e = 0; e < N; ++e) acc[e] = fmaf(wt, v4[u][e], acc[e]);
    }
    Mx = Mn;
  }
  // acc / W is the merged normalised output; final_value divides by W + sink
  store_item<D, N, BF16>(a, rowhead, qhead, d0, d0 == 0, Mx, W, acc);
}

// Issue priority from a wave's progress through its own range: 3 in the first
// quarter down to 0 in the last.  Waves sharing a SIMD are otherwise served
// oldest first, so the youngest fall behind and finish last; dropping the
// priority of the waves that are ahead lets the others catch up, and every
// wave's equal share then ends at about the same time.
#ifndef PKVD_PRIO
#define PKVD_PRIO 0
#endif
__device__ __forceinline__ void progress_priority(int done, int q1, int q2, int q3) {
#if PKVD_PRIO
  if (done >= q3) __builtin_amdgcn_s_setprio(0);
  else if (done >= q2) __builtin_amdgcn_s_setprio(1);
  else if (done >= q1) __builtin_amdgcn_s_setprio(2);
  else __builtin_amdgcn_s_setprio(3);
#endif
}

template <class Eng, int D, bool BF16, bool PAGE_POW2, int PF, int WPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void decode_kernel(const DecodeArgs a) {
  constexpr int RT = Eng::kRows;
  constexpr int NBUF = PF + 1;
  constexpr int kWindow = 128;                        // block-table columns per chunk
  extern __shared__ int lds[];
  constexpr int kEngWords = Eng::kLdsBytesPerWave / 4;
  const LdsLayout L = lds_layout(kEngWords, a.B);
  int* s_scan = lds + L.scan;
  int* s_pref = lds + L.pref;
  int* s_nlen = lds + L.nlen;

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const typename Eng::Lane ln = Eng::lane_of(lane, lds + L.eng + wave * kEngWords);

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
  // progress in key groups, for the issue priority
  const int total_groups = (int)(hi - lo) * Eng::kGroupsPerBlock;
  const int q1 = total_groups / 4, q2 = total_groups / 2, q3 = 3 * total_groups / 4;
  int groups_done = 0;
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
  // pieces of units shared with other waves: at most the first and the last
  // segment of the range; their tickets are read after the range is done
  int pend_prev[2] = {-1, -1}, pend_unit[2] = {0, 0};
  int64_t pend_ustart[2] = {0, 0}, pend_uend[2] = {0, 0};
  int pend_tile[2] = {0, 0}, pend_b[2] = {0, 0}, pend_kvh[2] = {0, 0};

  const Segment sg0 = locate(a, s_pref, s_nlen, lo, lo, hi);
  Chunk ch = make_chunk(sg0, sg0.blk_begin);
  PageWindow pw = fetch_pages(ch);
  typename Eng::Q qr;

  typename Eng::State st;
  int max_lo = 0, min_hi = 0;
#ifdef PKVD_TRACE
  int n_seg = 0, n_chunk = 0, n_blk = 0;
#endif
  PKVD_STAMP(a, gw, 2);
  for (;;) {
    const Segment& sg = ch.sg;
    if (ch.first) Eng::reset(a, sg, R, ln, st, max_lo, min_hi);

    // stream the chunk's key groups with loads PF groups ahead
#ifdef PKVD_TRACE
    if (n_chunk == 0) PKVD_STAMP(a, gw, 3);
    n_chunk++;
    n_blk += ch.ce - ch.cb;
#endif
    {
      constexpr int GPB = Eng::kGroupsPerBlock, KPG = Eng::kKeysPerGroup;
      const int g0 = ch.cb * GPB, ng = (ch.ce - ch.cb) * GPB;
      const int kb = ch.kb, ke = ch.ke, kvh = sg.kvh;
      typename Eng::Buf buf[NBUF];
      auto grp_of = [&](int i) { return g0 + min(i, ng - 1); };
      auto score = [&](const typename Eng::Buf& x, int i) {
        const int j0 = (g0 + i) * KPG;
        const bool full = j0 >= max_lo && j0 + KPG - 1 <= min_hi;
        Eng::score(st, x, qr, a.scale_log2, full, j0, ln);
      };
#pragma unroll
      for (int s = 0; s < PF; ++s)
        Eng::template load<PAGE_POW2>(buf[s], a, kvh, grp_of(s), kb, ke, pw, ps_shift, ln);
      // the segment's Q rows, after the first loads so their wait overlaps them
      if (ch.first) Eng::fetch_q(a, sg, R, ln, qr);
      // full rounds: each sub-step issues the loads of the group PF ahead (the
      // last group again near the end: a cache hit), then scores its own group
      const int rounds = ng / NBUF;
      for (int rd = 0; rd < rounds; ++rd) {
        progress_priority(groups_done + rd * NBUF, q1, q2, q3);
#pragma unroll
        for (int s = 0; s < NBUF; ++s) {
          const int i = rd * NBUF + s;
          Eng::template load<PAGE_POW2>(buf[(s + PF) % NBUF], a, kvh, grp_of(i + PF), kb, ke,
                                        pw, ps_shift, ln);
          score(buf[s], i);
        }
      }
      // tail: the remaining ng % NBUF <= PF groups are already in flight
      const int i0 = rounds * NBUF;
#pragma unroll
      for (int s = 0; s < PF; ++s)
        if (i0 + s < ng) score(buf[s], i0 + s);
      groups_done += ng;
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
    Eng::finish(st, ln);
    if (sg.whole) {
#pragma unroll
      for (int k = 0; k < Eng::kItems; ++k) {
        int r, d0;
        float M, L, O[8];
        const bool ok = Eng::item(st, ln, k, r, d0, M, L, O);
        const int row = sg.tile * RT + r;
        if (ok && row < R) {
          const int ti = row / a.g, qhead = sg.kvh * a.g + (row - ti * a.g);
          store_item<D, Eng::kItemDims, BF16>(a, (sg.b * a.Lq + ti) * a.Hq + qhead, qhead, d0,
                                              d0 == 0, M, L, O);
        }
      }
    } else {
      // a piece of a unit shared with other waves: leave the partial state,
      // then take a ticket (its value is read once the range is done)
      const int slot = 2 * gw + sg.side;
#pragma unroll
      for (int k = 0; k < Eng::kItems; ++k) {
        int r, d0;
        float M, L, O[8];
        const bool ok = Eng::item(st, ln, k, r, d0, M, L, O);
        if (ok) {
          float* po = a.ws_o + (int64_t)slot * RT * D;
#pragma unroll
          for (int e = 0; e < Eng::kItemDims; ++e)
            store_coherent(po + Eng::pidx(ln, r, e), L > 0.f ? O[e] / L : 0.f);
          if (d0 == 0)
            store_coherent(a.ws_lse + (int64_t)slot * RT + r, L > 0.f ? M + log2f(L) : -INFINITY);
        }
      }
      // the ticket is taken once the whole range is streamed, when these
      // stores have long completed (no wait for them here)
      const int unit = (sg.b * a.Hkv + sg.kvh) * a.row_tiles + sg.tile;
      auto remember = [&](int k) {
        pend_prev[k] = 0;
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
  // tickets of the pieces this wave left: partial stores complete first
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int side = 0; side < 2; ++side)
    if (pend_prev[side] >= 0 && lane == 0) pend_prev[side] = atomicAdd(&a.counters[pend_unit[side]], 1);
  // merge the units whose last piece this wave delivered (at the top issue
  // priority: the kernel's end waits on these)
#if PKVD_PRIO
  __builtin_amdgcn_s_setprio(3);
#endif
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
    for (int k = 0; k < Eng::kItems; ++k) {
      int r, d0;
      Eng::item_pos(ln, k, r, d0);
      const int row = pend_tile[side] * RT + r;
      if (!(r < RT && row < R)) continue;
      const int ti = row / a.g, qhead = pend_kvh[side] * a.g + (row - ti * a.g);
      merge_pieces<Eng, D, BF16>(a, T, NW, pend_ustart[side], w_first, w_last, ln, r, d0,
                                 (pend_b[side] * a.Lq + ti) * a.Hq + qhead, qhead);
    }
  }
  PKVD_STAMP(a, gw, 7);
}

// blocks in flight ahead of the scoring, and waves per SIMD the register
// budget is fitted to, per engine
#ifndef PKVD_PF4
#define PKVD_PF4 2
#endif
#ifndef PKVD_WPE4
#define PKVD_WPE4 3
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
#define PKVD_WPE16 2
#endif
#ifndef PKVD_PF16_D64
#define PKVD_PF16_D64 2
#endif
#ifndef PKVD_WPE16_D64
#define PKVD_WPE16_D64 3
#endif

using KernelFn = void (*)(DecodeArgs);

template <int D, int RT, bool BF16, bool POW2>
KernelFn valu_kernel() {
  constexpr int pf = RT == 4 ? PKVD_PF4 : PKVD_PF8;
  constexpr int wpe = RT == 4 ? PKVD_WPE4 : PKVD_WPE8;
  return &decode_kernel<ValuEngine<D, RT, BF16>, D, BF16, POW2, pf, wpe>;
}
#ifndef PKVD_MFMA_QLDS
#define PKVD_MFMA_QLDS 0
#endif
template <int D, bool BF16, bool POW2>
KernelFn mfma_kernel() {
  // a D = 64 block takes half the registers: one more wave per SIMD fits
  constexpr int pf = D == 64 ? PKVD_PF16_D64 : PKVD_PF16;
  constexpr int wpe = D == 64 ? PKVD_WPE16_D64 : PKVD_WPE16;
  return &decode_kernel<MfmaEngine<D, BF16, PKVD_MFMA_QLDS>, D, BF16, POW2, pf, wpe>;
}

KernelFn select(int path, int rows_per_tile, int head_dim, bool bf16, bool pow2) {
#define PKVD_SEL(D, BF, P2)                                                          \
  if (head_dim == D && bf16 == BF && pow2 == P2) {                                  \
    if (path == kPathMfma) return rows_per_tile == 16 ? mfma_kernel<D, BF, P2>() : nullptr; \
    if (rows_per_tile == 4) return valu_kernel<D, 4, BF, P2>();                     \
    if (rows_per_tile == 8) return valu_kernel<D, 8, BF, P2>();                     \
    return nullptr;                                                                 \
  }
  PKVD_SEL(128, true, true)
  PKVD_SEL(128, true, false)
  PKVD_SEL(128, false, true)
  PKVD_SEL(128, false, false)
  PKVD_SEL(64, true, true)
  PKVD_SEL(64, true, false)
  PKVD_SEL(64, false, true)
  PKVD_SEL(64, false, false)
#undef PKVD_SEL
  return nullptr;
}

bool page_pow2(int ps) { return ps >= kBlockKeys && (ps & (ps - 1)) == 0; }

}  // namespace

size_t decode_lds_bytes(int B, int path, int head_dim) {
  int eng = 0;
  if (path == kPathMfma)
    eng = head_dim == 128 ? MfmaEngine<128, true, PKVD_MFMA_QLDS>::kLdsBytesPerWave
                          : MfmaEngine<64, true, PKVD_MFMA_QLDS>::kLdsBytesPerWave;
  return sizeof(int) * (size_t)lds_layout(eng / 4, B).total;
}

int decode_blocks_per_cu(int path, int rows_per_tile, int head_dim, bool bf16, bool pow2,
                         size_t lds_bytes) {
  KernelFn k = select(path, rows_per_tile, head_dim, bf16, pow2);
  if (!k) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k), kThreads,
                                                   lds_bytes) != hipSuccess)
    return 0;
  return n;
}

hipError_t launch_decode(const DecodeArgs& a, int path, int rows_per_tile, bool bf16,
                         hipStream_t stream) {
  KernelFn k = select(path, rows_per_tile, a.D, bf16, page_pow2(a.ps));
  if (!k) return hipErrorInvalidValue;
  const dim3 grid((a.num_waves + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(k, grid, dim3(kThreads), decode_lds_bytes(a.B, path, a.D), stream, a);
  return hipGetLastError();
}

}  // namespace pkvd
