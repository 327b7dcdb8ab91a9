// prefill_kernel.hip -- context attention (prefill) on MFMA, the operation of
// flashinfer.attention.prims_ts.batch_prefill (summary and Parameters): fixed
// [B, S, H, D] or packed rows, head_dim 128 or 256, bottom-right causal,
// dense or per-query variable windows, a left window, sm_scale,
// output_scale and the output type.
//
// Work split.  A workgroup takes `hpw` query heads that share one kv head
// (grouped-query packing) times `tt` query tokens: 256 rows at head_dim 128
// (eight waves, two per SIMD, 32 rows each), 128 at 256 (eight waves, 16
// rows each).  Every key/value byte it stages in LDS therefore serves all of
// those rows, and each wave reads the staged tile once for its one or two
// 16-row MFMA tiles.  Items run over (token tile, request, kv head, head group)
// with the token tiles from the last to the first (the longest causal rows
// start first); when the number of (request, kv head, head group) triples is
// a multiple of eight, the items of one triple share an XCD (hardware
// dispatch is round-robin over XCDs), so their K/V stays in that XCD's L2.
//
// Two kernels.  The FAST kernel scores every row against a fixed reference
// (the score of the row's last visible key), so its loop holds no running
// maxima; a workgroup whose probabilities leave the range of their format
// marks its item and stores nothing else.  The SAFE kernel, launched next on
// the same stream, recomputes the marked items with a lazily raised running
// maximum (raised only when a score exceeds it by more than kTau) and
// rescaled accumulators.
//
// Staging.  K and V tiles of BN keys go through a four-stage LDS ring,
// filled with direct global-to-LDS 16-byte loads (no registers) two tiles
// ahead of their use (the fourth stage keeps a tile's V for the products
// the FAST loop defers past the next tile's barrier).  A key row of D elements is stored as 16-byte chunks
// whose 32-byte slot index is XORed with the key index mod 8, so the reads
// below touch spread banks.
//
// Per 32 keys and 16-row tile (matrix shapes as M x K times K x N):
//  * S^T[keys x rows] = K . Q^T with v_mfma_f32_16x16x32_{bf16,f16}: lane l
//    (j = l % 16, q = l / 16) feeds key j's dims 32c + 8q .. +8 (A) and row
//    j's same dims of Q (B, in registers); the two 16-key halves give lane l
//    the scores of row j for keys 4q + i and 16 + 4q + i, i = 0..3;
//  * masks by select (only in chunks some row sees in part); probabilities
//    2^(score - reference) in base 2; row sums by an MFMA against ones;
//    in the FAST loop a chunk's products P . V run beside the next chunk's
//    softmax (software pipelining within the wave);
//  * O += P . V with the same 16x16x32 instruction: the lane's eight
//    probabilities are the A operand of row j for the key order
//    (4q .. 4q + 3, 16 + 4q .. 16 + 4q + 3), and the B operand for output
//    dims 16u .. 16u + 15 is V at those keys, column j, which the gfx950
//    transposing LDS read (ds_read_b64_tr_b16) returns directly from the
//    row-major V tile: lane j of each 16-lane group points at 4 dims of one
//    key row and receives one dim of 4 key rows.
// Output tile u leaves lane l with rows 4q + i, dim 16u + j of O.
#include <float.h>

#include <type_traits>

#include "engine_mfma.h"
#include "prefill_args.h"

#define PKVD_LDS __attribute__((address_space(3)))

namespace pkvd {
namespace {

using namespace dev;

constexpr int kStages = 4;   // K/V tiles in the LDS ring

// Workgroup shape per head_dim: eight waves, two per SIMD (256 registers per
// lane each), so that one wave's MFMA work covers the other's softmax and
// LDS reads; 32 rows per wave at D = 128, 16 at D = 256 (whose operands are
// twice as wide).  (Three waves per SIMD at D = 128, 16 rows each, measured
// slower: each staged K byte then serves half as many rows.)
template <int D>
struct PrefillTile;
template <>
struct PrefillTile<128> {
  static constexpr int PW = 8;    // waves per workgroup
  static constexpr int TW = 2;    // 16-row tiles per wave
  static constexpr int BN = 64;   // keys per LDS tile
};
template <>
struct PrefillTile<256> {
  static constexpr int PW = 8;
  static constexpr int TW = 1;
  static constexpr int BN = 32;
};

typedef short s16x4_tr __attribute__((ext_vector_type(4)));

// Chunk position of 16-byte chunk c of key row k (an involution in c).
__device__ __forceinline__ int swz(int k, int c) { return (((c >> 1) ^ (k & 7)) << 1) | (c & 1); }

// Four 16-bit values, transposed across each 16-lane group (see above).
__device__ __forceinline__ u32x2 read_tr(const uint16_t* p) {
  const s16x4_tr x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4_tr PKVD_LDS*)((PKVD_LDS uint16_t*)p));
  return __builtin_bit_cast(u32x2, x);
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_maxi(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// Direct 16-byte global-to-LDS load: each lane's 16 bytes from `g` land at
// LDS byte address lds_base + OFF + 16 * lane (lds_base wave-uniform, in an
// SGPR; the sum goes to M0).
// Written out rather than through the builtin because the compiler, which
// cannot always tell which LDS variable such a load fills, would wait for
// all of them (vmcnt 0) before reading any stage of the ring; the kernel
// waits for each stage itself (wait_vmcnt, then a barrier).  The load has
// no register result, so no destination register can be reused while it is
// in flight; its address registers and M0 are read at issue, and M0 is
// restored before the block ends.
template <uint32_t OFF>
__device__ __forceinline__ void dma16(const uint16_t* g, uint32_t lds_base) {
  uint32_t saved;   // M0 is the compiler's register: restored before the block ends
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_add_u32 m0, %2, %3\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_base), "n"(OFF)
      : "memory", "scc");
}
// f(std::integral_constant<int, i>) for i = 0 .. N - 1.
template <int N, class Fn, int I = 0>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, Fn, I + 1>(static_cast<Fn&&>(f));
  }
}

// LDS byte address of an LDS variable (wave-uniform).
__device__ __forceinline__ uint32_t lds_address(const uint16_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(PKVD_LDS const uint16_t*)p);
}

// s_waitcnt with vmcnt = N and no wait on the other counters (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0xF70 | N);
}

// Workgroup barrier that waits only for this wave's LDS accesses (lgkmcnt 0)
// and not for its outstanding global-to-LDS loads: __syncthreads() would wait
// for every load in flight (vmcnt 0), including the tile issued for two steps
// ahead.  The loads a step needs are waited for by wait_vmcnt before it.
// Compiler-only fences keep memory accesses on their side of the barrier.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int D>
struct PrefillGeom {
  static constexpr int TW = PrefillTile<D>::TW, BN = PrefillTile<D>::BN;
  static constexpr int TILE = BN * D;   // elements of one K or V tile
};

// A workgroup item: its request b, kv head, head group hg and token tile mt,
// the request's rows (packed offsets clamped into the tensors) and the
// item's first query token.
struct PrefillItem {
  int b, kvh, hg, mt;
  int q0, sq, k0, sk;
  int t_begin;
  // false when the item holds no query token of its request (nothing to do)
  __device__ __forceinline__ bool init(const PrefillArgs& a, int item) {
    if (item >= a.items) return false;
    // Token tiles from the last to the first (the costliest first under a
    // causal mask).  Within a tile level the head groups rotate by 8 per
    // level: workgroups reach the XCDs in turn (item mod 8, which the shift
    // keeps, so an XCD keeps reading the same kv heads) and within an XCD
    // its shader engines in turn; without the shift a shader engine would
    // take the same requests at every level, and requests of unequal
    // lengths would load some engines far more than others.
    const int lvl = item / a.groups;
    mt = a.m_tiles - 1 - lvl;
    const int grp = (int)(((int64_t)(item - lvl * a.groups) + 8 * (int64_t)lvl) % a.groups);
    const int nbk = a.B * a.Hkv;
    hg = grp / nbk;
    const int bk = grp - hg * nbk;
    b = bk / a.Hkv;
    kvh = bk - b * a.Hkv;
    if (a.qo) {
      const int c0 = min(max(a.qo[b], 0), a.rows_q), c1 = min(max(a.qo[b + 1], 0), a.rows_q);
      const int d0 = min(max(a.kvo[b], 0), a.rows_kv), d1 = min(max(a.kvo[b + 1], 0), a.rows_kv);
      q0 = c0;
      sq = min(max(c1 - c0, 0), a.Sq);
      k0 = d0;
      sk = max(d1 - d0, 0);
    } else {
      q0 = b * a.Sq;
      sq = a.Sq;
      k0 = b * a.Sk;
      sk = a.Sk;
    }
    t_begin = mt * a.tt;
    return t_begin < sq;
  }
  // Element offset of the item's first output row (token t_begin, the
  // group's first query head), dim 0: a live row of the item.
  __device__ __forceinline__ int64_t first_out(const PrefillArgs& a) const {
    return ((int64_t)(q0 + t_begin) * a.Hq + kvh * a.g + hg * a.hpw) * a.D;
  }
};

// Marker an overflowed FAST pass leaves in its item's first output element
// (and nothing else): a signalling NaN of the output format.  Arithmetic
// never yields a signalling NaN (the output conversions and products quiet
// any NaN), so a marker is never a result; a stale one in a row that a
// later FAST pass overwrites is gone with it.
constexpr uint32_t kMarkF32 = 0x7FA5A5A5u;
constexpr uint16_t kMarkBf16 = 0x7F85u, kMarkF16 = 0x7D05u;

__device__ __forceinline__ void mark_overflow(const PrefillArgs& a, int64_t off) {
  if (a.out_type == kOutF32) static_cast<uint32_t*>(a.out)[off] = kMarkF32;
  else static_cast<uint16_t*>(a.out)[off] = a.out_type == kOutBf16 ? kMarkBf16 : kMarkF16;
}

__device__ __forceinline__ bool marked(const PrefillArgs& a, int64_t off) {
  if (a.out_type == kOutF32) return static_cast<const uint32_t*>(a.out)[off] == kMarkF32;
  return static_cast<const uint16_t*>(a.out)[off] ==
         (a.out_type == kOutBf16 ? kMarkBf16 : kMarkF16);
}

// The workgroup's whole computation of one item, in the FAST mode (SAFE =
// false: returns true when the pass overflowed; it then stores only the
// item's marker) or the SAFE mode (SAFE = true: the rescaling passes, one
// tile and half of the output dims at a time).  st0 .. st3: the LDS ring's
// stages (a K tile, then a V tile); s_range, s_flag: LDS scratch of the
// workgroup.
template <int D, bool BF16, bool SAFE>
__device__ __forceinline__ bool prefill_body(const PrefillArgs& a, const PrefillItem& it,
                                             uint16_t* st0, uint16_t* st1, uint16_t* st2,
                                             uint16_t* st3,
                                             int* s_range, int* s_flag) {
  using Mf = Mfma<BF16>;
  using F = Fmt<BF16>;
  constexpr int TW = PrefillTile<D>::TW, BN = PrefillTile<D>::BN;
  constexpr int RW = 16 * TW;             // rows per wave
  constexpr int NC = D / 32;              // 32-dim chunks of q . k
  constexpr int NU = D / 16;              // 16-dim output tiles
  constexpr int CPR = D / 8;              // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;           // key rows per wave-wide 16-byte load
  constexpr int TILE = BN * D;            // elements of one K or V tile
  constexpr int kPW = PrefillTile<D>::PW;
  constexpr int LPT = TILE / 8 / 64 / kPW;   // wave-wide loads per wave, tile and tensor
  static_assert(LPT >= 1 && TILE / 8 == LPT * 64 * kPW, "tile loads must divide over the waves");
  static_assert(2 * LPT < 16, "outstanding loads must fit the vmcnt field");
  static_assert(kStages == 4, "four ring stages");

  const int b = it.b, kvh = it.kvh, hg = it.hg;
  const int q0 = it.q0, sq = it.sq, k0 = it.k0, sk = it.sk;
  const int t_begin = it.t_begin;   // first query token of the workgroup

  // keys query token i sees: [lo, hi] (empty when hi < lo)
  auto bounds = [&](int i, int& lo, int& hi) {
    if (a.mask == kPrefillVariable) {
      lo = a.starts[(int64_t)b * a.Sq + i];
      hi = a.ends[(int64_t)b * a.Sq + i];
    } else {
      const int p = sk - sq + i;   // bottom-right diagonal
      hi = a.mask == kPrefillCausal ? p : sk - 1;
      lo = a.window_left < 0 ? 0 : p - a.window_left;
    }
    lo = max(lo, 0);
    hi = min(hi, sk - 1);
  };

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int tid = threadIdx.x;
  const int lj = lane & 15, lq = lane >> 4;

  // the workgroup's key range: the union over its tokens (all its heads
  // share them)
  if (tid == 0) {
    s_range[0] = INT32_MAX;
    s_range[1] = INT32_MIN;
    *s_flag = 0;
  }
  __syncthreads();
  if (tid < a.tt && t_begin + tid < sq) {
    int lo, hi;
    bounds(t_begin + tid, lo, hi);
    if (lo <= hi) {
      atomicMin(&s_range[0], lo);
      atomicMax(&s_range[1], hi);
    }
  }
  __syncthreads();
  const int klo = uniform(s_range[0]), khi = uniform(s_range[1]);
  const int kbase = klo <= khi ? (klo / 16) * 16 : 0;
  const int ntiles = klo <= khi ? (khi - kbase) / BN + 1 : 0;

  // LDS byte addresses of this wave's first load in each stage of the ring
  // (the direct loads' M0 adds a constant per load)
  const uint32_t lds_st[kStages] = {(uint32_t)uniform(lds_address(st0) + wave * 1024),
                                    (uint32_t)uniform(lds_address(st1) + wave * 1024),
                                    (uint32_t)uniform(lds_address(st2) + wave * 1024),
                                    (uint32_t)uniform(lds_address(st3) + wave * 1024)};
  // Direct loads of a tile: wave-wide load u of the wave fills key rows
  // (u * kPW + wave) * RPI .. + RPI - 1 of the tile (1 KB of LDS,
  // lane-major); lane l loads chunk swz(row, l % CPR) of its row.  The
  // lane's element offsets (row, kv head, chunk) are fixed per call; a tile
  // adds its first key's row.
  // (the host keeps a tile's span of rows and the heads within int32)
  const uint16_t* kbase_p = a.k + (int64_t)k0 * a.k_sr + (int64_t)kvh * a.k_sh;
  const uint16_t* vbase_p = a.v + (int64_t)k0 * a.v_sr + (int64_t)kvh * a.v_sh;
  int koff[LPT], voff[LPT], lrow[LPT];
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int r = (u * kPW + wave) * RPI + lane / CPR;
    const int c = swz(r, lane % CPR);
    lrow[u] = r;
    koff[u] = r * (int)a.k_sr + c * 8;
    voff[u] = r * (int)a.v_sr + c * 8;
  }
  // keys past the request's last are read as its last key (masked below)
  auto issue = [&](int i, uint32_t st) {
    const int kb = kbase + i * BN;
    if (kb + BN <= sk) {   // uniform: a whole tile of keys
      const uint16_t* kt = kbase_p + (int64_t)kb * a.k_sr;
      const uint16_t* vt = vbase_p + (int64_t)kb * a.v_sr;
      static_for<LPT>([&](auto U) {
        constexpr int u = decltype(U)::value;
        dma16<u * kPW * 1024u>(kt + koff[u], st);
        dma16<u * kPW * 1024u + 2u * TILE>(vt + voff[u], st);
      });
    } else {
      static_for<LPT>([&](auto U) {
        constexpr int u = decltype(U)::value;
        // row min(kb + r, sk - 1) of the request: koff holds r's part
        const int64_t d = (int64_t)(min(kb + lrow[u], sk - 1) - lrow[u]);
        dma16<u * kPW * 1024u>(kbase_p + d * a.k_sr + koff[u], st);
        dma16<u * kPW * 1024u + 2u * TILE>(vbase_p + d * a.v_sr + voff[u], st);
      });
    }
  };

  // FAST (one item per workgroup, the ring not yet used): the first two
  // tiles' loads go out before Q and the reference scores are read, so that
  // those latencies overlap (the Q wait below then covers them too)
  if constexpr (!SAFE) {
    if (ntiles > 0) issue(0, lds_st[0]);
    if (ntiles > 1) issue(1, lds_st[1]);
  }

  // scores are taken in base 2 with a positive factor: a negative sm_scale
  // is moved onto Q's sign bits (exact)
  const float sc = fabsf(a.scale_log2);
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;

  // this wave's tiles: tile t holds 16 tokens of one query head
  int lo_t[TW], hi_t[TW], h_t[TW], tok0_t[TW];
  u32x4 qf[TW][NC];
  // over the wave's tiles: keys no live row sees, and keys every live row sees
  int wlo = INT32_MAX, whi = INT32_MIN, wmaxlo = INT32_MIN, wminhi = INT32_MAX;
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int rho = wave * RW + 16 * t;   // the tile's first row of the workgroup
    const int hh = rho / a.tt;
    h_t[t] = kvh * a.g + hg * a.hpw + hh;
    tok0_t[t] = t_begin + (rho - hh * a.tt);
    const int tok = tok0_t[t] + lj;
    const bool live = tok < sq;
    int lo = 1, hi = 0;   // padding rows see nothing
    if (live) bounds(tok, lo, hi);
    lo_t[t] = lo;
    hi_t[t] = hi;
    const bool seen = live && lo <= hi;
    wlo = min(wlo, seen ? lo : INT32_MAX);
    whi = max(whi, seen ? hi : INT32_MIN);
    wmaxlo = max(wmaxlo, live ? lo : INT32_MIN);
    wminhi = min(wminhi, live ? hi : INT32_MAX);
  }
  // Q rows of tile t as the B operand of the scores (padding rows load the
  // workgroup's first token, which is live: never stored)
  auto load_q = [&](int t, u32x4 (&dst)[NC]) {
    const int tok = tok0_t[t] + lj;
    const int qtok = tok < sq ? tok : t_begin;
    const uint16_t* qp = a.q + (int64_t)(q0 + qtok) * a.q_sr + (int64_t)h_t[t] * a.q_sh + lq * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) dst[c] = load16(qp + c * 32) ^ qsign;
  };
#pragma unroll
  for (int t = 0; t < TW; ++t) load_q(t, qf[t]);
  // Reference of the FAST pass, per row: the score (base 2, times sc) of
  // the row's last visible key, plus 8 for fp16 probabilities (so that
  // keys may score up to 8 + 16 above it before P overflows, and what P
  // flushes to zero is below 2^-16 of the row's largest probability); -inf
  // for a row that sees no key.  The row's four lanes each take 8 dims of
  // every 32 and add across the lanes.
  float m_ref[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int tok = tok0_t[t] + lj;
    const bool seen = tok < sq && lo_t[t] <= hi_t[t];
    float dot = 0.f;
    if (seen) {   // (a request may have no keys at all)
      const uint16_t* kp = kbase_p + (int64_t)hi_t[t] * a.k_sr + lq * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 kk = load16(kp + c * 32);
#pragma unroll
        for (int w = 0; w < 4; ++w) dot = F::dot2(qf[t][c][w], kk[w], dot);
      }
    }
    const Pair p16 = lane_pair<16>(dot);
    const Pair p32 = lane_pair<32>(p16.lo + p16.hi);
    m_ref[t] = seen ? sc * (p32.lo + p32.hi) + (BF16 ? 0.f : 8.f) : -INFINITY;
  }
  // (wave-uniform: scalar registers and scalar branches below)
  wlo = uniform(wave_min(wlo));
  whi = uniform(wave_maxi(whi));
  wmaxlo = uniform(wave_maxi(wmaxlo));
  wminhi = uniform(wave_min(wminhi));

  // Q rows (and, in the FAST mode, the first two tiles) have landed before
  // the loop: it waits only for the tile loads it issues itself
  wait_vmcnt<0>();

  // B operand of ones: P . 1 gives the row sums of the probabilities as
  // rounded for P . V
  const u32x4 ones = BF16 ? u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}
                          : u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};

  // One pass over the keys for tiles T0 .. T0 + NT - 1.  FAST: every row
  // keeps the reference m_ref (its score of its last visible key, see
  // above) for the whole pass, so the accumulators are only ever touched by
  // MFMAs and no chunk takes row maxima; probabilities of keys scoring
  // above the reference may exceed 1 by as much as P's format holds.  A row
  // whose probabilities went beyond that marks the pass as overflowed: the
  // workgroup stores only its item's marker, and the SAFE kernel runs the
  // item again with a lazily raised maximum (by more than kTau at a time)
  // and rescaled accumulators.  Returns true when a FAST pass overflowed.
  auto attend = [&](auto safe_tag, auto t0_tag, auto nt_tag, auto u0_tag, auto nu_tag) -> bool {
    static_assert(decltype(safe_tag)::value == SAFE, "one mode per body");
    constexpr int T0 = decltype(t0_tag)::value, NT = decltype(nt_tag)::value;
    // output dims 16 U0 .. 16 (U0 + NUP) - 1
    constexpr int U0 = decltype(u0_tag)::value, NUP = decltype(nu_tag)::value;
    // online softmax state per tile: row j's max (uniform over its four
    // lanes); acc[t][u][i]: row 4q + i, dim 16 (U0 + u) + j; lsum[t][i]: row 4q + i's
    // sum of probabilities (the same in every column)
    float m_t[NT];
    f32x4_t acc[NT][NUP], lsum[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      m_t[t] = SAFE ? -INFINITY : m_ref[T0 + t];
      lsum[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NUP; ++u) acc[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // this pass's Q operands: the FAST pass uses those loaded for all
    // tiles; a SAFE pass loads its own again, so that only one tile's stay
    // in registers through the rescaling passes
    u32x4 qv[NT][NC];
    if constexpr (SAFE) {
#pragma unroll
      for (int t = 0; t < NT; ++t) load_q(T0 + t, qv[t]);
      wait_vmcnt<0>();
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) qv[t][c] = qf[T0 + t][c];
    }

    // A chunk is 32 keys from j0 (tile rows kc * 32 ..) of a stage's K and V
    // tiles; masked (uniform): some row sees only part of them.  The steps:
    // scores, the mask (by select), probabilities 2^(sc x - m) packed as the
    // A operand of P . V (a row that has seen no key has m = -inf and only
    // -inf scores: p = 0), and the products P . 1 (row sums) and P . V.
    //
    // FAST: chunks software-pipelined within the wave.  Chunk c's scores
    // are taken first; then chunk c - 1's products P . V (pending) run in
    // the same stretch as chunk c's probabilities, so that each wave has
    // MFMA and VALU work in flight together.  No branch touches the
    // accumulators (a join between arms that do and do not update them
    // makes the compiler copy them): every chunk of the workgroup's tiles is
    // taken, those this wave does not see fully masked, and the first
    // chunk's pending products are zero probabilities against that chunk's
    // own (loaded) V.  A pending chunk's V tile may be read after the
    // barrier that opens the next tile: four ring stages keep it from being
    // refilled until then.
    u32x4 pend_pa[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) pend_pa[t] = u32x4{0u, 0u, 0u, 0u};
    const uint16_t* pend_sV = st0 + TILE;
    int pend_kc = 0;
    auto chunk_scores = [&](const uint16_t* sK, int kc, float (&x)[NT][8]) {
      u32x4 ka[2][NC];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = kc * 32 + 16 * h + lj;
#pragma unroll
        for (int c = 0; c < NC; ++c)
          ka[h][c] = *reinterpret_cast<const u32x4*>(sK + r * D + swz(r, 4 * c + lq) * 8);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          s0 = Mf::qk(ka[0][c], qv[t][c], s0);
          s1 = Mf::qk(ka[1][c], qv[t][c], s1);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[t][i] = s0[i];
          x[t][4 + i] = s1[i];
        }
      }
    };
    auto chunk_mask = [&](int j0, float (&x)[NT][8]) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = j0 + (e < 4 ? 4 * lq + e : 16 + 4 * lq + e - 4);
          x[t][e] = (key >= lo_t[T0 + t] && key <= hi_t[T0 + t]) ? x[t][e] : -INFINITY;
        }
    };
    auto chunk_probs = [&](const float (&x)[NT][8], u32x4 (&pa)[NT]) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float nm = -fmaxf(m_t[t], -FLT_MAX);
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(x[t][e], sc, nm));
        pa[t] = u32x4{F::pack2(p[0], p[1]), F::pack2(p[2], p[3]), F::pack2(p[4], p[5]),
                      F::pack2(p[6], p[7])};
      }
    };
    // SAFE: the running maximum of each row, raised only when a score
    // exceeds it by more than kTau (base 2), the accumulators rescaled then
    auto safe_rescale = [&](const float (&x)[NT][8]) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float lmax = sc * fmaxf(fmaxf(fmaxf(x[t][0], x[t][1]), fmaxf(x[t][2], x[t][3])),
                                      fmaxf(fmaxf(x[t][4], x[t][5]), fmaxf(x[t][6], x[t][7])));
        if (wave_any(lmax > m_t[t] + kTau)) {
          // the chunk max of row j over its four lanes (l, l ^ 16, l ^ 32, l ^ 48)
          const Pair p16 = lane_pair<16>(lmax);
          const Pair p32 = lane_pair<32>(fmaxf(p16.lo, p16.hi));
          const float mn = fmaxf(m_t[t], fmaxf(p32.lo, p32.hi));
          const float alpha = rescale(m_t[t], mn);
          m_t[t] = mn;
          // accumulator rows are 4q + i: each row's factor from lane 4q + i
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float ai = __builtin_bit_cast(
                float,
                __builtin_amdgcn_ds_bpermute((4 * lq + i) << 2, __builtin_bit_cast(int, alpha)));
            lsum[t][i] *= ai;
#pragma unroll
            for (int u = 0; u < NUP; ++u) acc[t][u][i] *= ai;
          }
        }
      }
    };
    auto chunk_products = [&](const uint16_t* sV, int kc, const u32x4 (&pa)[NT]) {   // sV: a V tile
      // V operand of output tile u: keys (4q .. 4q + 3, 16 + 4q .. + 3), column j
      auto vread = [&](int u) {
        u32x4 vb;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = kc * 32 + 16 * h + 4 * lq + (lj >> 2);
          const int cc = 2 * u + ((lj & 3) >> 1);
          const u32x2 y = read_tr(sV + r * D + swz(r, cc) * 8 + (lj & 1) * 4);
          vb[2 * h] = y[0];
          vb[2 * h + 1] = y[1];
        }
        return vb;
      };
      constexpr int VPRE = 1;   // V operands read one product ahead
      u32x4 vb[VPRE];
#pragma unroll
      for (int u = 0; u < VPRE; ++u) vb[u] = vread(U0 + u);
#pragma unroll
      for (int t = 0; t < NT; ++t) lsum[t] = Mf::qk(pa[t], ones, lsum[t]);
#pragma unroll
      for (int u = 0; u < NUP; ++u) {
        const u32x4 v = vb[u % VPRE];
        if (u + VPRE < NUP) vb[u % VPRE] = vread(U0 + u + VPRE);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t][u] = Mf::qk(pa[t], v, acc[t][u]);
      }
    };

    lds_barrier();   // every wave is past its reads of an earlier pass's ring
    if constexpr (SAFE) {
      if (ntiles > 0) issue(0, lds_st[0]);
      if (ntiles > 1) issue(1, lds_st[1]);
    }
    if (ntiles > 1) wait_vmcnt<2 * LPT>();
    else wait_vmcnt<0>();
    lds_barrier();
    // step `it` reads stage it % 4 and fills stage (it + 2) % 4
    auto step = [&](int it, const uint16_t* stage, uint32_t next) {
      if (it + 2 < ntiles) issue(it + 2, next);
      const uint16_t* sK = stage;
      const uint16_t* sV = stage + TILE;
      const int kb = kbase + it * BN;
#pragma unroll
      for (int kc = 0; kc < BN / 32; ++kc) {
        const int j0 = kb + kc * 32;
        // masked unless every live row sees all of them
        const bool masked = !(j0 >= wmaxlo && j0 + 31 <= wminhi);
        if constexpr (SAFE) {
          if (j0 > whi || j0 + 31 < wlo) continue;   // no row of this wave sees these keys
          float x[NT][8];
          chunk_scores(sK, kc, x);
          if (masked) chunk_mask(j0, x);   // uniform
          safe_rescale(x);
          u32x4 pa[NT];
          chunk_probs(x, pa);
          chunk_products(sV, kc, pa);
        } else {
          float x[NT][8];
          chunk_scores(sK, kc, x);
          if (masked) chunk_mask(j0, x);   // uniform
          // the previous chunk's products beside this chunk's softmax
          u32x4 pa[NT];
          chunk_products(pend_sV, pend_kc, pend_pa);
          chunk_probs(x, pa);
          // computed here, beside the products (not sunk to their use)
#pragma unroll
          for (int t = 0; t < NT; ++t) asm volatile("" ::"v"(pa[t]));
#pragma unroll
          for (int t = 0; t < NT; ++t) pend_pa[t] = pa[t];
          pend_sV = sV;
          pend_kc = kc;
        }
      }
      if (it + 1 < ntiles) {
        // the next tile's loads have landed (the one after may still be in flight)
        if (it + 2 < ntiles) wait_vmcnt<2 * LPT>();
        else wait_vmcnt<0>();
        lds_barrier();
      }
    };
    for (int it = 0; it < ntiles; it += 4) {
      step(it, st0, lds_st[2]);
      if (it + 1 < ntiles) step(it + 1, st1, lds_st[3]);
      if (it + 2 < ntiles) step(it + 2, st2, lds_st[0]);
      if (it + 3 < ntiles) step(it + 3, st3, lds_st[1]);
    }
    if constexpr (!SAFE)
      if (ntiles > 0) chunk_products(pend_sV, pend_kc, pend_pa);   // the last chunk's products

    if constexpr (!SAFE) {
      // A probability beyond the range of P's format (or of the fp32 sums)
      // leaves an infinite or NaN row sum; below it the result is exact to
      // the formats' precision.  The workgroup's vote: any such row -> all
      // waves run the SAFE passes (every wave is past its last read of the
      // ring here).
      // Padding rows (tokens past the request's last) are not counted: they
      // are never stored, and in unmasked chunks their scores meet m = -inf.
      bool over = false;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          over |= tok0_t[T0 + t] + 4 * lq + i < sq && !(lsum[t][i] < INFINITY);
      if (wave_any(over)) *s_flag = 1;
      lds_barrier();
      if (*s_flag) {
        if (threadIdx.x == 0) mark_overflow(a, it.first_out(a));
        return true;
      }
    }

    // epilogue: out = O / l * output_scale for rows 4q + i, dims 16u + j
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * lq + i;
        const float L = lsum[t][i];
        const int tok = tok0_t[T0 + t] + r;
        if (tok >= sq) continue;
        const float f = L > 0.f ? a.out_scale / L : 0.f;
        const int64_t off = ((int64_t)(q0 + tok) * a.Hq + h_t[T0 + t]) * D + 16 * U0 + lj;
        if (a.out_type == kOutF32) {
          float* o = static_cast<float*>(a.out) + off;
#pragma unroll
          for (int u = 0; u < NUP; ++u) o[16 * u] = acc[t][u][i] * f;
        } else {
          uint16_t* o = static_cast<uint16_t*>(a.out) + off;
          if (a.out_type == kOutBf16) {
#pragma unroll
            for (int u = 0; u < NUP; ++u) o[16 * u] = Fmt<true>::encode(acc[t][u][i] * f);
          } else {
#pragma unroll
            for (int u = 0; u < NUP; ++u) o[16 * u] = Fmt<false>::encode(acc[t][u][i] * f);
          }
        }
      }
    }
    return false;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using IH = std::integral_constant<int, NU / 2>;
  if constexpr (!SAFE) {
    return attend(std::false_type{}, I0{}, std::integral_constant<int, TW>{}, I0{},
                  std::integral_constant<int, NU>{});
  } else {
    static_for<TW>([&](auto T) {
      attend(std::true_type{}, T, I1{}, I0{}, IH{});
      attend(std::true_type{}, T, I1{}, IH{}, IH{});
    });
    return false;
  }
}

// FAST pass: one workgroup per item.
template <int D, bool BF16>
__global__ __launch_bounds__(64 * PrefillTile<D>::PW, 1) void prefill_kernel(const PrefillArgs a) {
  constexpr int TILE = PrefillGeom<D>::TILE;
  __shared__ __attribute__((aligned(16))) uint16_t st0[2 * TILE], st1[2 * TILE], st2[2 * TILE],
      st3[2 * TILE];
  __shared__ int s_range[2];
  __shared__ int s_flag;   // the pass overflowed (see attend)
  PrefillItem it;
  if (!it.init(a, (int)blockIdx.x)) return;   // uniform over the workgroup
  prefill_body<D, BF16, false>(a, it, st0, st1, st2, st3, s_range, &s_flag);
}

// SAFE passes, launched after the FAST kernel on the same stream with at
// most one workgroup per CU: workgroup w takes the items w, w + G, w + 2G ..
// (G = its grid), finds with one load per thread which of them hold the
// marker of an overflowed FAST pass, and recomputes those one by one.  A
// kernel of its own, so that the rescaling passes' register demand does not
// shape the register allocation of the FAST loop.
template <int D, bool BF16>
__global__ __launch_bounds__(64 * PrefillTile<D>::PW, 1) void prefill_safe_kernel(const PrefillArgs a) {
  constexpr int TILE = PrefillGeom<D>::TILE;
  constexpr int NT = 64 * PrefillTile<D>::PW;   // items checked per pass
  __shared__ __attribute__((aligned(16))) uint16_t st0[2 * TILE], st1[2 * TILE], st2[2 * TILE],
      st3[2 * TILE];
  __shared__ int s_range[2];
  __shared__ int s_flag;
  __shared__ int s_list[NT];
  __shared__ int s_n;
  const int G = (int)gridDim.x, w = (int)blockIdx.x;
  const int ncand = (a.items - w + G - 1) / G;   // this workgroup's items
  for (int base = 0; base < ncand; base += NT) {
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    const int j = base + (int)threadIdx.x;
    PrefillItem it;
    if (j < ncand && it.init(a, w + j * G) && marked(a, it.first_out(a)))
      s_list[atomicAdd(&s_n, 1)] = w + j * G;
    __syncthreads();
    const int n = uniform(s_n);
    for (int k = 0; k < n; ++k) {
      PrefillItem m;
      m.init(a, uniform(s_list[k]));   // true: it was listed
      prefill_body<D, BF16, true>(a, m, st0, st1, st2, st3, s_range, &s_flag);
    }
    __syncthreads();   // s_n and s_list are reused by the next pass
  }
}

}  // namespace

bool prefill_geometry(int head_dim, int g, int* hpw, int* tt) {
  int rows;
  if (head_dim == 128) rows = PrefillTile<128>::PW * 16 * PrefillTile<128>::TW;
  else if (head_dim == 256) rows = PrefillTile<256>::PW * 16 * PrefillTile<256>::TW;
  else return false;
  int p = 1;
  // (tiles per workgroup) / p whole 16-row tiles per head: a tile never
  // holds two heads
  while ((rows / 16) % (p * 2) == 0 && g % (p * 2) == 0) p *= 2;
  *hpw = p;
  *tt = rows / p;
  return true;
}

namespace {
template <int D, bool BF16>
hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t stream) {
  const dim3 grid(a.items), block(64 * PrefillTile<D>::PW);
  hipLaunchKernelGGL((prefill_kernel<D, BF16>), grid, block, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_safe_kernel<D, BF16>), dim3(a.safe_grid), block, 0, stream, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, hipStream_t stream) {
  if (a.items <= 0) return hipSuccess;
  if (a.D == 128) return bf16 ? launch_prefill_d<128, true>(a, stream) : launch_prefill_d<128, false>(a, stream);
  if (a.D == 256) return bf16 ? launch_prefill_d<256, true>(a, stream) : launch_prefill_d<256, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkvd
