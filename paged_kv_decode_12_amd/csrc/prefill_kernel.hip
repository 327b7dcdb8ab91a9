// prefill_kernel.hip -- context attention (prefill) on MFMA, the operation of
// flashinfer.attention.prims_ts.batch_prefill (summary and Parameters): fixed
// [B, S, H, D] or packed rows, head_dim 128 or 256, bottom-right causal,
// dense or per-query variable windows, a left window, sm_scale,
// output_scale and the output type.
//
// One workgroup computes BM query rows of one (request, query head): four
// waves of 16 * TW rows each.  The request's keys are walked in tiles of BN
// keys; each tile of K and V is read from HBM once per workgroup (plain
// loads: the other query tiles and the query heads of the same kv head read
// it again, from L2 when the grid keeps them on one XCD), written to LDS and
// double-buffered, so the next tile's loads are in flight while the current
// one is used.  Per 16-key block a wave computes S^T = K . Q^T with
// v_mfma_f32_16x16x32_{bf16,f16} (K from LDS as the A operand, Q in registers
// as the B operand), masks by select, keeps an online softmax with a lazy
// base-2 maximum, and multiplies P . V with v_mfma_f32_16x16x16: the
// accumulator of S^T is already the A-operand layout of P, and each lane's
// V operand comes from 16-byte LDS reads of four key rows (output tile t of
// the lane's 16 covers dims j * DJ + t, so a lane ends with DJ consecutive
// dims of four rows).  The grid runs the latest (longest causal) query
// tiles first, and maps workgroups so that the XCD of a workgroup holds the
// query heads that share its kv head.
#include "engine_mfma.h"
#include "prefill_args.h"

namespace pkvd {
namespace {

using namespace dev;

constexpr int kPW = 4;   // waves per workgroup (one per SIMD)

template <int D>
struct PrefillTile;
template <>
struct PrefillTile<128> {
  static constexpr int TW = 2;    // 16-row tiles per wave
  static constexpr int BN = 64;   // keys per LDS tile
};
template <>
struct PrefillTile<256> {
  static constexpr int TW = 1;
  static constexpr int BN = 32;
};

// LDS of one workgroup: K and V tiles, two stages each, rows padded by 16
// bytes so that the 16 key rows one K read touches fall in different banks.
template <int D>
constexpr size_t prefill_lds_bytes() {
  return 2 * 2 * (size_t)PrefillTile<D>::BN * (D + 8) * sizeof(uint16_t);
}

template <int N>
__device__ __forceinline__ void store_row(const PrefillArgs& a, int64_t off, const float (&x)[N]) {
  if (a.out_type == kOutF32) {
    float* p = static_cast<float*>(a.out) + off;
#pragma unroll
    for (int u = 0; u < N / 4; ++u)
      reinterpret_cast<float4*>(p)[u] = make_float4(x[4 * u], x[4 * u + 1], x[4 * u + 2], x[4 * u + 3]);
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
#pragma unroll
  for (int u = 0; u < N / 8; ++u)
    reinterpret_cast<u32x4*>(p)[u] = u32x4{w[4 * u], w[4 * u + 1], w[4 * u + 2], w[4 * u + 3]};
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

template <int D, bool BF16>
__global__ __launch_bounds__(64 * kPW) void prefill_kernel(const PrefillArgs a) {
  using Mf = Mfma<BF16>;
  using F = Fmt<BF16>;
  constexpr int TW = PrefillTile<D>::TW, BN = PrefillTile<D>::BN;
  constexpr int NC = D / 32;              // 32-dim chunks of q . k
  constexpr int DJ = D / 16;              // output dims per lane (PV tiles)
  constexpr int VW = DJ / 8;              // 16-byte V reads per key row
  constexpr int BM = kPW * 16 * TW;       // query rows per workgroup
  constexpr int LD = D + 8;               // LDS row pitch (elements)
  constexpr int CH = BN * D / 8;          // 16-byte chunks per tile per tensor
  constexpr int CPT = CH / (64 * kPW);    // chunks per thread per tensor
  static_assert(CH % (64 * kPW) == 0, "tile chunks must divide over the workgroup");
  __shared__ __attribute__((aligned(16))) uint16_t lds_tiles[prefill_lds_bytes<D>() / 2];
  uint16_t* sK = lds_tiles;                  // [2][BN * LD]
  uint16_t* sV = lds_tiles + 2 * BN * LD;    // [2][BN * LD]
  __shared__ int s_range[2];

  // workgroups of one XCD (blockIdx % 8) take consecutive items; items run
  // from the last query tile (the most keys when causal) to the first
  const int nx = (a.items + 7) / 8;
  const int item = (int)(blockIdx.x % 8) * nx + (int)(blockIdx.x / 8);
  if (item >= a.items) return;
  const int per_tile = a.B * a.Hq;
  const int mt = a.m_tiles - 1 - item / per_tile;
  const int rest = item - (item / per_tile) * per_tile;
  const int b = rest / a.Hq, h = rest - (rest / a.Hq) * a.Hq;
  const int kvh = h / a.g;

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
  const int r_begin = mt * BM;
  if (r_begin >= sq) return;   // uniform over the workgroup

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
  const int wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const int lj = lane & 15, lq = lane >> 4;

  // the workgroup's key range: the union over its rows
  if (tid == 0) {
    s_range[0] = INT32_MAX;
    s_range[1] = INT32_MIN;
  }
  __syncthreads();
  if (tid < BM && r_begin + tid < sq) {
    int lo, hi;
    bounds(r_begin + tid, lo, hi);
    if (lo <= hi) {
      atomicMin(&s_range[0], lo);
      atomicMax(&s_range[1], hi);
    }
  }
  __syncthreads();
  const int klo = s_range[0], khi = s_range[1];

  // this wave's rows: tile t, row j = token r_begin + wave * 16 TW + 16 t + j
  const int w_row0 = r_begin + wave * 16 * TW;
  int lo_t[TW], hi_t[TW];
  int wlo = INT32_MAX, whi = INT32_MIN, wmaxlo = INT32_MIN, wminhi = INT32_MAX;
  u32x4 qf[TW][NC];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int tok = w_row0 + 16 * t + lj;
    const bool live = tok < sq;
    int lo = 1, hi = 0;   // padding rows see nothing
    if (live) bounds(tok, lo, hi);
    lo_t[t] = lo;
    hi_t[t] = hi;
    if (live) {
      // a block is unmasked only when every live row sees all of it (a live
      // row that sees nothing makes every block masked)
      wmaxlo = max(wmaxlo, lo);
      wminhi = min(wminhi, hi);
      if (lo <= hi) {   // blocks no live row sees are skipped
        wlo = min(wlo, lo);
        whi = max(whi, hi);
      }
    }
    // padding rows load the tile's first row (live): never stored
    const int qtok = live ? tok : r_begin;
    const uint16_t* qp = a.q + (int64_t)(q0 + qtok) * a.q_sr + (int64_t)h * a.q_sh + lq * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[t][c] = load16(qp + c * 32);
  }
  wlo = wave_min(wlo);
  whi = wave_maxi(whi);
  wmaxlo = wave_maxi(wmaxlo);
  wminhi = wave_min(wminhi);

  // online softmax state per tile: row j's max (uniform over its 4 lanes)
  // and this lane's partial sum; accumulators acc[t][u][i]: row 4 lq + i,
  // dim lj * DJ + u
  float m_t[TW], l_t[TW];
  f32x4_t acc[TW][DJ];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    m_t[t] = -INFINITY;
    l_t[t] = 0.f;
#pragma unroll
    for (int u = 0; u < DJ; ++u) acc[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int kbase = klo <= khi ? (klo / 16) * 16 : 0;
  const int ntiles = klo <= khi ? (khi - kbase) / BN + 1 : 0;
  u32x4 pk[CPT], pv[CPT];
  // tile loads: chunk c of the tile is key row c / (D / 8), dims (c % (D / 8)) * 8;
  // keys past the request's last are read as its last key (masked below)
  auto gload = [&](int kb) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + u * 64 * kPW;
      const int row = c / (D / 8), col = (c - row * (D / 8)) * 8;
      const int key = min(kb + row, sk - 1);
      pk[u] = load16(a.k + (int64_t)(k0 + key) * a.k_sr + (int64_t)kvh * a.k_sh + col);
      pv[u] = load16(a.v + (int64_t)(k0 + key) * a.v_sr + (int64_t)kvh * a.v_sh + col);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + u * 64 * kPW;
      const int row = c / (D / 8), col = (c - row * (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(sK + buf * BN * LD + row * LD + col) = pk[u];
      *reinterpret_cast<u32x4*>(sV + buf * BN * LD + row * LD + col) = pv[u];
    }
  };

  if (ntiles > 0) {
    gload(kbase);
    lstore(0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int kb = kbase + it * BN;
    if (it + 1 < ntiles) gload(kb + BN);   // in flight during this tile's work
    const uint16_t* tK = sK + cur * BN * LD;
    const uint16_t* tV = sV + cur * BN * LD;
#pragma unroll
    for (int kk = 0; kk < BN / 16; ++kk) {
      const int j0 = kb + kk * 16;
      if (j0 + 15 < wlo || j0 > whi) continue;   // no row of this wave sees the block
      const bool full = j0 >= wmaxlo && j0 + 15 <= wminhi;
      u32x4 kf[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kf[c] = *reinterpret_cast<const u32x4*>(tK + (kk * 16 + lj) * LD + c * 32 + lq * 8);
      u32x4 vf[4][VW];   // key rows 4 lq + e, dims lj * DJ ..
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int x = 0; x < VW; ++x)
          vf[e][x] = *reinterpret_cast<const u32x4*>(tV + (kk * 16 + 4 * lq + e) * LD + lj * DJ + 8 * x);
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) s = Mf::qk(kf[c], qf[t][c], s);
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[i] = s[i] * a.scale_log2;
          if (!full) {
            const int key = j0 + 4 * lq + i;
            sv[i] = (key >= lo_t[t] && key <= hi_t[t]) ? sv[i] : -INFINITY;
          }
        }
        const float lmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        if (wave_any(lmax > m_t[t] + kTau)) {
          // the block max of row lj over its four lanes (l, l^16, l^32, l^48)
          const Pair p16 = lane_pair<16>(lmax);
          const float m16 = fmaxf(p16.lo, p16.hi);
          const Pair p32 = lane_pair<32>(m16);
          const float mn = fmaxf(m_t[t], fmaxf(p32.lo, p32.hi));
          const float alpha = rescale(m_t[t], mn);
          m_t[t] = mn;
          l_t[t] *= alpha;
          // accumulator rows are 4 lq + i: each row's factor from lane 4 lq + i
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float ai = __builtin_bit_cast(
                float, __builtin_amdgcn_ds_bpermute((4 * lq + i) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
            for (int u = 0; u < DJ; ++u) acc[t][u][i] *= ai;
          }
        }
        // a row that has seen no key yet has m = -inf and only -inf scores: p = 0
        const float ms = m_t[t] == -INFINITY ? 0.f : m_t[t];
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - ms);
        l_t[t] += (p[0] + p[1]) + (p[2] + p[3]);
        const u32x2 pa = {F::pack2(p[0], p[1]), F::pack2(p[2], p[3])};
#pragma unroll
        for (int u = 0; u < DJ; ++u) {
          const int x = u >> 3, w = (u & 7) >> 1;
          u32x2 vb;
          if (u & 1) {
            vb[0] = pair_hi(vf[0][x][w], vf[1][x][w]);
            vb[1] = pair_hi(vf[2][x][w], vf[3][x][w]);
          } else {
            vb[0] = pair_lo(vf[0][x][w], vf[1][x][w]);
            vb[1] = pair_lo(vf[2][x][w], vf[3][x][w]);
          }
          acc[t][u] = Mf::pv(pa, vb, acc[t][u]);
        }
      }
    }
    if (it + 1 < ntiles) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: row sums over the four lanes of each row, then out = O / l *
  // output_scale for rows 4 lq + i, dims lj * DJ .. + DJ
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const Pair p16 = lane_pair<16>(l_t[t]);
    const float l16 = p16.lo + p16.hi;
    const Pair p32 = lane_pair<32>(l16);
    const float lsum = p32.lo + p32.hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lq + i;
      const float L = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute(r << 2, __builtin_bit_cast(int, lsum)));
      const int tok = w_row0 + 16 * t + r;
      if (tok >= sq) continue;
      const float f = L > 0.f ? a.out_scale / L : 0.f;
      float x[DJ];
#pragma unroll
      for (int u = 0; u < DJ; ++u) x[u] = acc[t][u][i] * f;
      store_row<DJ>(a, ((int64_t)(q0 + tok) * a.Hq + h) * D + lj * DJ, x);
    }
  }
}

}  // namespace

int prefill_block_rows(int head_dim) {
  if (head_dim == 128) return kPW * 16 * PrefillTile<128>::TW;
  if (head_dim == 256) return kPW * 16 * PrefillTile<256>::TW;
  return 0;
}

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, hipStream_t stream) {
  if (a.items <= 0) return hipSuccess;
  const dim3 grid(8 * ((a.items + 7) / 8)), block(64 * kPW);
  if (a.D == 128) {
    if (bf16)
      hipLaunchKernelGGL((prefill_kernel<128, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<128, false>), grid, block, 0, stream, a);
  } else if (a.D == 256) {
    if (bf16)
      hipLaunchKernelGGL((prefill_kernel<256, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<256, false>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkvd
