// prefill_kernel.hip -- context attention (prefill) on MFMA, the operation of
// flashinfer.attention.prims_ts.batch_prefill (summary and Parameters): fixed
// [B, S, H, D] or packed rows, head_dim 128 or 256, bottom-right causal,
// dense or per-query variable windows, a left window, sm_scale,
// output_scale and the output type.
//
// Work split.  A workgroup (four waves, one per SIMD) takes `hpw` query heads
// that share one kv head (grouped-query packing) times `tt` query tokens:
// 256 rows at head_dim 128 (64 per wave), 128 at 256 (32 per wave).  Every
// key/value byte it stages in LDS therefore serves all of those rows, and
// each wave reads the staged tile once for its 4 (or 2) 16-row MFMA tiles.
// Items run over (token tile, request, kv head, head group) with the token
// tiles from the last to the first (the longest causal rows start first);
// when the number of (request, kv head) pairs is a multiple of eight, the
// items of one pair share an XCD (hardware dispatch is round-robin over
// XCDs), so their K/V stays in that XCD's L2.
//
// Staging.  K and V tiles of BN keys go through a three-stage LDS ring,
// filled with direct global-to-LDS 16-byte loads (no registers) two tiles
// ahead of their use.  A key row of D elements is stored as 16-byte chunks
// whose 32-byte slot index is XORed with the key index mod 8, so the reads
// below touch spread banks.
//
// Per 32 keys and 16-row tile (matrix shapes as M x K times K x N):
//  * S^T[keys x rows] = K . Q^T with v_mfma_f32_16x16x32_{bf16,f16}: lane l
//    (j = l % 16, q = l / 16) feeds key j's dims 32c + 8q .. +8 (A) and row
//    j's same dims of Q (B, in registers); the two 16-key halves give lane l
//    the scores of row j for keys 4q + i and 16 + 4q + i, i = 0..3;
//  * masks by select; online softmax in base 2 with a lazily raised
//    maximum (only when a score exceeds it by more than kTau), row maxima
//    across the row's four lanes with lane-pair swaps;
//  * O += P . V with the same 16x16x32 instruction: the lane's eight
//    probabilities are the A operand of row j for the key order
//    (4q .. 4q + 3, 16 + 4q .. 16 + 4q + 3), and the B operand for output
//    dims 16u .. 16u + 15 is V at those keys, column j, which the gfx950
//    transposing LDS read (ds_read_b64_tr_b16) returns directly from the
//    row-major V tile: lane j of each 16-lane group points at 4 dims of one
//    key row and receives one dim of 4 key rows.
// Output tile u leaves lane l with rows 4q + i, dim 16u + j of O.
#include <type_traits>

#include "engine_mfma.h"
#include "prefill_args.h"

#define PKVD_LDS __attribute__((address_space(3)))

namespace pkvd {
namespace {

using namespace dev;

constexpr int kPW = 4;       // waves per workgroup (one per SIMD)
constexpr int kStages = 3;   // K/V tiles in the LDS ring

template <int D>
struct PrefillTile;
template <>
struct PrefillTile<128> {
  static constexpr int TW = 4;    // 16-row tiles per wave
  static constexpr int BN = 64;   // keys per LDS tile
};
template <>
struct PrefillTile<256> {
  static constexpr int TW = 2;
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
// LDS byte address lds_base + 16 * lane (lds_base wave-uniform, in M0).
// Written out rather than through the builtin because the compiler, which
// cannot always tell which LDS variable such a load fills, would wait for
// all of them (vmcnt 0) before reading any stage of the ring; the kernel
// waits for each stage itself (wait_vmcnt, then a barrier).  The load has
// no register result, so no destination register can be reused while it is
// in flight; its address registers are read at issue.
__device__ __forceinline__ void dma16(const uint16_t* g, const uint16_t* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(PKVD_LDS const uint16_t*)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(m0)
               : "memory", "m0");
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

template <int D, bool BF16>
__global__ __launch_bounds__(64 * kPW, 1) void prefill_kernel(const PrefillArgs a) {
  using Mf = Mfma<BF16>;
  using F = Fmt<BF16>;
  constexpr int TW = PrefillTile<D>::TW, BN = PrefillTile<D>::BN;
  constexpr int RW = 16 * TW;             // rows per wave
  constexpr int NC = D / 32;              // 32-dim chunks of q . k
  constexpr int NU = D / 16;              // 16-dim output tiles
  constexpr int CPR = D / 8;              // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;           // key rows per wave-wide 16-byte load
  constexpr int TILE = BN * D;            // elements of one K or V tile
  constexpr int LPT = TILE / 8 / 64 / kPW;   // wave-wide loads per wave, tile and tensor
  static_assert(LPT >= 1 && TILE / 8 == LPT * 64 * kPW, "tile loads must divide over the waves");
  static_assert(2 * LPT < 16, "outstanding loads must fit the vmcnt field");
  // the ring's stages: a K tile, then a V tile
  __shared__ __attribute__((aligned(16))) uint16_t st0[2 * TILE], st1[2 * TILE], st2[2 * TILE];
  __shared__ int s_range[2];
  __shared__ int s_flag;   // a FAST pass overflowed (see attend)
  static_assert(kStages == 3, "three ring stages");

  const int item = (int)blockIdx.x;
  if (item >= a.items) return;
  const int mt = a.m_tiles - 1 - item / a.groups;
  const int grp = item - (item / a.groups) * a.groups;
  const int nbk = a.B * a.Hkv;
  const int hg = grp / nbk, bk = grp - hg * nbk;
  const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;

  // the request's rows (packed offsets clamped into the tensors)
  int q0, sq, k0, sk;
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
  const int t_begin = mt * a.tt;   // first query token of the workgroup
  if (t_begin >= sq) return;       // uniform over the workgroup

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
    s_flag = 0;
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

  // direct loads of tile i into stage s: wave-wide load u of the wave fills
  // key rows (u * kPW + wave) * RPI .. + RPI - 1 (1 KB of LDS, lane-major);
  // keys past the request's last are read as its last key (masked below)
  auto issue = [&](int i, uint16_t* sK, uint16_t* sV) {
    const int kb = kbase + i * BN;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int inst = u * kPW + wave;
      const int r = inst * RPI + lane / CPR;
      const int c = swz(r, lane % CPR);
      const int key = min(kb + r, sk - 1);
      const uint16_t* gk = a.k + (int64_t)(k0 + key) * a.k_sr + (int64_t)kvh * a.k_sh + c * 8;
      const uint16_t* gv = a.v + (int64_t)(k0 + key) * a.v_sr + (int64_t)kvh * a.v_sh + c * 8;
      dma16(gk, sK + inst * 512);
      dma16(gv, sV + inst * 512);
    }
  };
  // this wave's tiles: tile t holds 16 tokens of one query head
  int lo_t[TW], hi_t[TW], h_t[TW], tok0_t[TW];
  int tminlo[TW], tmaxhi[TW], tmaxlo[TW], tminhi[TW];
  u32x4 qf[TW][NC];
  int wlo = INT32_MAX, whi = INT32_MIN;
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
    // blocks no live row sees are skipped; a block is unmasked only when
    // every live row sees all of it
    // (wave-uniform: held in scalar registers, so the per-tile tests below
    // are scalar branches)
    tminlo[t] = uniform(wave_min(seen ? lo : INT32_MAX));
    tmaxhi[t] = uniform(wave_maxi(seen ? hi : INT32_MIN));
    tmaxlo[t] = uniform(wave_maxi(live ? lo : INT32_MIN));
    tminhi[t] = uniform(wave_min(live ? hi : INT32_MAX));
    wlo = min(wlo, tminlo[t]);
    whi = max(whi, tmaxhi[t]);
    // padding rows load the workgroup's first token (live): never stored
    const int qtok = live ? tok : t_begin;
    const uint16_t* qp = a.q + (int64_t)(q0 + qtok) * a.q_sr + (int64_t)h_t[t] * a.q_sh + lq * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[t][c] = load16(qp + c * 32);
  }

  // Q rows are in registers (issued above) before any tile load is
  // outstanding: the loop below waits only for its own tile loads
  wait_vmcnt<0>();

  // One pass over the keys for tiles T0 .. T0 + NT - 1.  FAST: a row's maximum is set from the first
  // chunk it sees and not raised after, so the accumulators are only ever
  // touched by MFMAs (they stay in accumulation registers); probabilities
  // may then reach 2^kFast, which bf16 (and the fp32 sums) hold for
  // kFast = 64 and fp16 for 15.  A score beyond that marks the pass as
  // overflowed and the workgroup runs it again in the SAFE mode: a lazily
  // raised maximum (by more than kTau at a time) with the accumulators
  // rescaled.  Returns true when a FAST pass overflowed (nothing written).
  auto attend = [&](auto safe_tag, auto t0_tag, auto nt_tag) -> bool {
    constexpr bool SAFE = decltype(safe_tag)::value;
    constexpr int T0 = decltype(t0_tag)::value, NT = decltype(nt_tag)::value;   // tiles T0 ..
    constexpr float kFast = BF16 ? 64.f : 15.f;
    // online softmax state per tile: row j's max (uniform over its four
    // lanes) and this lane's partial sum; acc[t][u][i]: row 4q + i, dim 16u + j
    float m_t[NT], l_t[NT];
    f32x4_t acc[NT][NU];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      m_t[t] = -INFINITY;
      l_t[t] = 0.f;
#pragma unroll
      for (int u = 0; u < NU; ++u) acc[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    bool over = false;

    lds_barrier();   // every wave is past its reads of an earlier pass's ring
    if (ntiles > 0) issue(0, st0, st0 + TILE);
    if (ntiles > 1) issue(1, st1, st1 + TILE);
    if (ntiles > 1) wait_vmcnt<2 * LPT>();
    else wait_vmcnt<0>();
    lds_barrier();
    // step `it` reads stage it % 3 and fills stage (it + 2) % 3
    auto step = [&](int it, const uint16_t* sK, const uint16_t* sV, uint16_t* nK, uint16_t* nV) {
      if (it + 2 < ntiles) issue(it + 2, nK, nV);
      const int kb = kbase + it * BN;
#pragma unroll 1
      for (int kc = 0; kc < BN / 32; ++kc) {
        const int j0 = kb + kc * 32;
        if (j0 > whi || j0 + 31 < wlo) continue;   // no row of this wave sees these keys
        // phase 1: scores and probabilities of every tile (K operands shared)
        u32x4 ka[2][NC];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = kc * 32 + 16 * h + lj;
#pragma unroll
          for (int c = 0; c < NC; ++c)
            ka[h][c] = *reinterpret_cast<const u32x4*>(sK + r * D + swz(r, 4 * c + lq) * 8);
        }
        u32x4 pa[NT];
        bool on[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          on[t] = !(j0 > tmaxhi[T0 + t] || j0 + 31 < tminlo[T0 + t]);   // the tile sees some keys
          pa[t] = u32x4{0u, 0u, 0u, 0u};
          if (!on[t]) continue;
          f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            s0 = Mf::qk(ka[0][c], qf[T0 + t][c], s0);
            s1 = Mf::qk(ka[1][c], qf[T0 + t][c], s1);
          }
          float x[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[i] = s0[i] * a.scale_log2;
            x[4 + i] = s1[i] * a.scale_log2;
          }
          if (!(j0 >= tmaxlo[T0 + t] && j0 + 31 <= tminhi[T0 + t])) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int key = j0 + (e < 4 ? 4 * lq + e : 16 + 4 * lq + e - 4);
              x[e] = (key >= lo_t[T0 + t] && key <= hi_t[T0 + t]) ? x[e] : -INFINITY;
            }
          }
          const float lmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                   fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
          if constexpr (SAFE) {
            if (wave_any(lmax > m_t[t] + kTau)) {
              // the chunk max of row j over its four lanes (l, l ^ 16, l ^ 32, l ^ 48)
              const Pair p16 = lane_pair<16>(lmax);
              const Pair p32 = lane_pair<32>(fmaxf(p16.lo, p16.hi));
              const float mn = fmaxf(m_t[t], fmaxf(p32.lo, p32.hi));
              const float alpha = rescale(m_t[t], mn);
              m_t[t] = mn;
              l_t[t] *= alpha;
              // accumulator rows are 4q + i: each row's factor from lane 4q + i
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float ai = __builtin_bit_cast(
                    float,
                    __builtin_amdgcn_ds_bpermute((4 * lq + i) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
                for (int u = 0; u < NU; ++u) acc[t][u][i] *= ai;
              }
            }
          } else {
            over |= m_t[t] != -INFINITY && lmax > m_t[t] + kFast;
            if (wave_any(m_t[t] == -INFINITY && lmax != -INFINITY)) {
              // rows seeing their first keys take the chunk max (their
              // accumulators and sums are still zero)
              const Pair p16 = lane_pair<16>(lmax);
              const Pair p32 = lane_pair<32>(fmaxf(p16.lo, p16.hi));
              if (m_t[t] == -INFINITY) m_t[t] = fmaxf(p32.lo, p32.hi);
            }
          }
          // a row that has seen no key yet has m = -inf and only -inf scores: p = 0
          const float ms = m_t[t] == -INFINITY ? 0.f : m_t[t];
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = fast_exp2(x[e] - ms);
          l_t[t] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
          pa[t] = u32x4{F::pack2(p[0], p[1]), F::pack2(p[2], p[3]), F::pack2(p[4], p[5]),
                        F::pack2(p[6], p[7])};
        }
        // phase 2: O += P . V, one 16-dim output tile at a time (V operands
        // shared by the tiles)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          u32x4 vb;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int r = kc * 32 + 16 * h + 4 * lq + (lj >> 2);
            const int cc = 2 * u + ((lj & 3) >> 1);
            const u32x2 y = read_tr(sV + r * D + swz(r, cc) * 8 + (lj & 1) * 4);
            vb[2 * h] = y[0];
            vb[2 * h + 1] = y[1];
          }
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (on[t]) acc[t][u] = Mf::qk(pa[t], vb, acc[t][u]);
        }
      }
      if (it + 1 < ntiles) {
        // the next tile's loads have landed (the one after may still be in flight)
        if (it + 2 < ntiles) wait_vmcnt<2 * LPT>();
        else wait_vmcnt<0>();
        lds_barrier();
      }
    };
    for (int it = 0; it < ntiles; it += 3) {
      step(it, st0, st0 + TILE, st2, st2 + TILE);
      if (it + 1 < ntiles) step(it + 1, st1, st1 + TILE, st0, st0 + TILE);
      if (it + 2 < ntiles) step(it + 2, st2, st2 + TILE, st1, st1 + TILE);
    }

    if constexpr (!SAFE) {
      // the workgroup's vote: any wave overflowed -> all run the SAFE pass
      // (every wave is past its last read of the ring here)
      if (wave_any(over)) s_flag = 1;
      lds_barrier();
      if (s_flag) return true;
    }

    // epilogue: row sums over the four lanes of each row, then
    // out = O / l * output_scale for rows 4q + i, dims 16u + j
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const Pair p16 = lane_pair<16>(l_t[t]);
      const Pair p32 = lane_pair<32>(p16.lo + p16.hi);
      const float lsum = p32.lo + p32.hi;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * lq + i;
        const float L = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(r << 2, __builtin_bit_cast(int, lsum)));
        const int tok = tok0_t[T0 + t] + r;
        if (tok >= sq) continue;
        const float f = L > 0.f ? a.out_scale / L : 0.f;
        const int64_t off = ((int64_t)(q0 + tok) * a.Hq + h_t[T0 + t]) * D + lj;
        if (a.out_type == kOutF32) {
          float* o = static_cast<float*>(a.out) + off;
#pragma unroll
          for (int u = 0; u < NU; ++u) o[16 * u] = acc[t][u][i] * f;
        } else {
          uint16_t* o = static_cast<uint16_t*>(a.out) + off;
          if (a.out_type == kOutBf16) {
#pragma unroll
            for (int u = 0; u < NU; ++u) o[16 * u] = Fmt<true>::encode(acc[t][u][i] * f);
          } else {
#pragma unroll
            for (int u = 0; u < NU; ++u) o[16 * u] = Fmt<false>::encode(acc[t][u][i] * f);
          }
        }
      }
    }
    return false;
  };
  // FAST over all tiles; after an overflow, SAFE over half of the tiles at
  // a time (half the accumulators: the rescaling path keeps them in
  // ordinary registers)
  using I0 = std::integral_constant<int, 0>;
  if (attend(std::false_type{}, I0{}, std::integral_constant<int, TW>{})) {
    constexpr int H = TW / 2;
    attend(std::true_type{}, I0{}, std::integral_constant<int, H>{});
    attend(std::true_type{}, std::integral_constant<int, H>{}, std::integral_constant<int, TW - H>{});
  }
}

}  // namespace

bool prefill_geometry(int head_dim, int g, int* hpw, int* tt) {
  int rows;
  if (head_dim == 128) rows = kPW * 16 * PrefillTile<128>::TW;
  else if (head_dim == 256) rows = kPW * 16 * PrefillTile<256>::TW;
  else return false;
  int p = 1;
  while (p * 2 <= rows / 16 && g % (p * 2) == 0) p *= 2;
  *hpw = p;
  *tt = rows / p;
  return true;
}

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, hipStream_t stream) {
  if (a.items <= 0) return hipSuccess;
  const dim3 grid(a.items), block(64 * kPW);
  if (a.D == 128) {
    if (bf16) hipLaunchKernelGGL((prefill_kernel<128, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((prefill_kernel<128, false>), grid, block, 0, stream, a);
  } else if (a.D == 256) {
    if (bf16) hipLaunchKernelGGL((prefill_kernel<256, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((prefill_kernel<256, false>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkvd
