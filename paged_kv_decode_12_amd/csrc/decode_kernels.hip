// decode_kernels.hip -- batched paged-KV decode attention kernels for gfx950.
//
// Operation: flashinfer.cudnn.cudnn_batch_decode_with_kv_cache (Parameters,
// Note / LSE convention).  One workgroup handles one (request b, kv head,
// row tile, KV split).  The rows of a tile are the Hq/Hkv query heads that
// share the kv head times the q_len_per_req query tokens, so every K/V byte a
// workgroup loads serves all of them (grouped-query packing).
//
// VALU path (rows per tile <= 8):
//   * 4 waves per workgroup; wave w scores the 16-key blocks w, w+4, ... of the
//     workgroup's key range.
//   * Inside a wave, 8 lanes own one key of an 8-key step: lane (kk, part) holds
//     16-byte pieces {c * 128 + part * 16} of key kk's row, so a wave-wide load
//     instruction reads 8 contiguous 128-byte segments of the [page_size, D]
//     tile.  Q is held in registers with the same dim split.
//   * q . k: v_dot2 on bf16/fp16 pairs, then a DPP all-reduce over the 8 lanes.
//   * Each lane group is an independent online-softmax stream (running max m,
//     sum l, output accumulator O for its dims).  The running max is updated
//     lazily: only when a score exceeds m by more than kTau (base 2), so a
//     probability never exceeds 2^kTau and the rescale branch is rare.
//   * At the end the 8 streams of a wave and the 4 waves are merged with the
//     base-2 LSE rule, which is also how split partials are merged.
// Split-KV: with S > 1 splits, every split writes (o_s = O / l, lse_s) in fp32
// and merge_splits combines them (Note / LSE convention: base-2 LSE states are
// what the cascade merge consumes), adding the sink logit once.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "decode_args.h"

namespace pkvd {
namespace {

constexpr float kTau = 8.0f;          // lazy-rescale threshold, base-2 units
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// element formats
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
};

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
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7-i within 8

// Sum over the 8 lanes of an aligned lane octet; every lane gets the total.
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

// Weight of a state with max m when merged under the common max M (M >= m).
__device__ __forceinline__ float rescale(float m, float M) {
  return m == -INFINITY ? 0.f : exp2f(m - M);
}

// ---------------------------------------------------------------------------
// key range of one request
// ---------------------------------------------------------------------------
// Keys any row of request b may see: [lo(row 0), n - 1], cut into 16-key
// blocks aligned to absolute key index.  Splits partition these blocks.
struct UnitRange {
  int n;          // clamped sequence length
  int key_lo;     // first key some row sees
  int first_blk;  // block of key_lo
  int nblk;       // blocks in [key_lo, n)
};

__device__ __forceinline__ UnitRange unit_range(const DecodeArgs& a, int b) {
  UnitRange u;
  int n = a.seq_lens[b];
  const int cap = a.C * a.ps;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  u.n = n;
  int lo = (a.window_left < 0) ? 0 : n - a.Lq - a.window_left;
  u.key_lo = lo < 0 ? 0 : lo;
  if (n <= 0 || u.key_lo >= n) {
    u.first_blk = 0;
    u.nblk = 0;
  } else {
    u.first_blk = u.key_lo / kBlockKeys;
    u.nblk = (n - 1) / kBlockKeys - u.first_blk + 1;
  }
  return u;
}

__device__ __forceinline__ int valid_splits(const DecodeArgs& a, const UnitRange& u) {
  return (u.nblk + a.split_blocks - 1) / a.split_blocks;
}

// ---------------------------------------------------------------------------
// VALU decode kernel
// ---------------------------------------------------------------------------
template <int D>
struct KeyRegs {
  static constexpr int NP = D / 64;  // 16-byte pieces per lane per key row
  uint4 k[2][NP];                    // [step][piece]
  uint4 v[2][NP];
};

template <int D, bool PAGE_POW2>
__device__ __forceinline__ void load_block(KeyRegs<D>& x, const DecodeArgs& a, int b, int kvh,
                                           int blk, int kb, int ke, int ps_shift, int kk,
                                           int part) {
  constexpr int NP = D / 64;
  const int j0 = blk * kBlockKeys;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = j0 + t * 8 + kk;
    int page, slot;
    if (PAGE_POW2) {
      // page_size is a power of two >= 16: the whole block sits in one page
      page = a.bt[(int64_t)b * a.bt_sr + (j0 >> ps_shift)];
      slot = j & (a.ps - 1);
    } else {
      const int jc = j < ke ? j : ke - 1;   // keep the table index in range
      const int col = jc / a.ps;
      page = a.bt[(int64_t)b * a.bt_sr + col];
      slot = jc - col * a.ps;
    }
    page = (unsigned)page < (unsigned)a.P ? page : a.P - 1;
    const bool valid = j >= kb && j < ke;
    const uint16_t* kr = a.k + (int64_t)page * a.k_sp + (int64_t)kvh * a.k_sh + slot * D + part * 8;
    const uint16_t* vr = a.v + (int64_t)page * a.v_sp + (int64_t)kvh * a.v_sh + slot * D + part * 8;
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      if (valid) {
        x.k[t][c] = *reinterpret_cast<const uint4*>(kr + c * 64);
        x.v[t][c] = *reinterpret_cast<const uint4*>(vr + c * 64);
      } else {
        x.k[t][c] = make_uint4(0, 0, 0, 0);
        x.v[t][c] = make_uint4(0, 0, 0, 0);
      }
    }
  }
}

template <int D, int RT, bool BF16>
struct Stream {
  static constexpr int NP = D / 64;
  float m[RT], msub[RT], l[RT];
  float o[RT][NP * 8];   // this lane's dims: c * 64 + part * 8 + e
};

template <int D, int RT, bool BF16>
__device__ __forceinline__ void score_block(Stream<D, RT, BF16>& st, const KeyRegs<D>& x,
                                            const uint4 (&qr)[RT][D / 64], float scale_log2,
                                            bool full, int j0, int kk, const int (&lo_r)[RT],
                                            const int (&hi_r)[RT]) {
  using F = Fmt<BF16>;
  constexpr int NP = D / 64;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = j0 + t * 8 + kk;
    float s[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < NP; ++c) {
        acc = F::dot2(qr[r][c].x, x.k[t][c].x, acc);
        acc = F::dot2(qr[r][c].y, x.k[t][c].y, acc);
        acc = F::dot2(qr[r][c].z, x.k[t][c].z, acc);
        acc = F::dot2(qr[r][c].w, x.k[t][c].w, acc);
      }
      s[r] = octet_sum(acc) * scale_log2;
    }
    if (!full) {
#pragma unroll
      for (int r = 0; r < RT; ++r) s[r] = (j >= lo_r[r] && j <= hi_r[r]) ? s[r] : -INFINITY;
    }
    bool need = false;
#pragma unroll
    for (int r = 0; r < RT; ++r) need |= s[r] > st.m[r] + kTau;
    if (wave_any(need)) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const float mn = fmaxf(st.m[r], s[r]);
        const float alpha = rescale(st.m[r], mn);
        st.m[r] = mn;
        st.msub[r] = mn == -INFINITY ? 0.f : mn;
        st.l[r] *= alpha;
#pragma unroll
        for (int e = 0; e < NP * 8; ++e) st.o[r][e] *= alpha;
      }
    }
    float p[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      p[r] = exp2f(s[r] - st.msub[r]);
      st.l[r] += p[r];
    }
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      const uint32_t w[4] = {x.v[t][c].x, x.v[t][c].y, x.v[t][c].z, x.v[t][c].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float v0 = F::lo(w[u]), v1 = F::hi(w[u]);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          st.o[r][c * 8 + 2 * u] = fmaf(p[r], v0, st.o[r][c * 8 + 2 * u]);
          st.o[r][c * 8 + 2 * u + 1] = fmaf(p[r], v1, st.o[r][c * 8 + 2 * u + 1]);
        }
      }
    }
  }
}

template <int D, int RT, bool BF16, bool PAGE_POW2>
__global__ __launch_bounds__(kThreads) void decode_valu(const DecodeArgs a) {
  constexpr int NP = D / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kk = lane >> 3, part = lane & 7;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y / a.row_tiles;
  const int tile = blockIdx.y - kvh * a.row_tiles;
  const int b = blockIdx.z;

  const UnitRange u = unit_range(a, b);
  if (a.num_splits > 1 && split >= valid_splits(a, u)) return;
  const int blk_begin = u.first_blk + split * a.split_blocks;
  int blk_end = u.first_blk + u.nblk;
  if (a.num_splits > 1 && blk_begin + a.split_blocks < blk_end) blk_end = blk_begin + a.split_blocks;
  const int kb = max(u.key_lo, blk_begin * kBlockKeys);
  const int ke = min(u.n, blk_end * kBlockKeys);

  // rows of this tile: rr = tile * RT + r  ->  token i = rr / g, head hl = rr % g
  const int R = a.g * a.Lq;
  int lo_r[RT], hi_r[RT];
  int max_lo = kb, min_hi = ke - 1;
  uint4 qr[RT][NP];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int rr = tile * RT + r;
    const bool live = rr < R;
    const int i = live ? rr / a.g : 0;
    const int hl = live ? rr - i * a.g : 0;
    const int diag = u.n - a.Lq + i;
    int lo = a.window_left < 0 ? 0 : diag - a.window_left;
    lo = max(lo, kb);
    const int hi = min(diag, ke - 1);
    lo_r[r] = live ? lo : 1;     // dead rows see nothing
    hi_r[r] = live ? hi : 0;
    if (live) {
      max_lo = max(max_lo, lo);
      min_hi = min(min_hi, hi);
    }
    const uint16_t* qp = a.q + (int64_t)(b * a.Lq + i) * a.q_sr + (int64_t)(kvh * a.g + hl) * a.q_sh +
                         part * 8;
#pragma unroll
    for (int c = 0; c < NP; ++c)
      qr[r][c] = live ? *reinterpret_cast<const uint4*>(qp + c * 64) : make_uint4(0, 0, 0, 0);
  }

  Stream<D, RT, BF16> st;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    st.m[r] = -INFINITY;
    st.msub[r] = 0.f;
    st.l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < NP * 8; ++e) st.o[r][e] = 0.f;
  }

  const int ps_shift = PAGE_POW2 ? __builtin_ctz(a.ps) : 0;
  // software pipeline: the next block's loads are in flight while this one is scored
  KeyRegs<D> buf[2];
  int blk = blk_begin + wave;
  if (blk < blk_end) load_block<D, PAGE_POW2>(buf[0], a, b, kvh, blk, kb, ke, ps_shift, kk, part);
  for (; blk < blk_end; blk += 2 * kWaves) {
    const int blk1 = blk + kWaves;
    if (blk1 < blk_end) load_block<D, PAGE_POW2>(buf[1], a, b, kvh, blk1, kb, ke, ps_shift, kk, part);
    {
      const int j0 = blk * kBlockKeys;
      const bool full = j0 >= max_lo && j0 + kBlockKeys - 1 <= min_hi;
      score_block<D, RT, BF16>(st, buf[0], qr, a.scale_log2, full, j0, kk, lo_r, hi_r);
    }
    if (blk1 >= blk_end) break;
    const int blk2 = blk1 + kWaves;
    if (blk2 < blk_end) load_block<D, PAGE_POW2>(buf[0], a, b, kvh, blk2, kb, ke, ps_shift, kk, part);
    {
      const int j0 = blk1 * kBlockKeys;
      const bool full = j0 >= max_lo && j0 + kBlockKeys - 1 <= min_hi;
      score_block<D, RT, BF16>(st, buf[1], qr, a.scale_log2, full, j0, kk, lo_r, hi_r);
    }
  }

  // merge the 8 lane-group streams of the wave (lanes differ in bits 3..5)
#pragma unroll
  for (int x = 8; x < 64; x <<= 1) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const float mo = shfl_xor(st.m[r], x);
      const float lo = shfl_xor(st.l[r], x);
      const float M = fmaxf(st.m[r], mo);
      const float a0 = rescale(st.m[r], M), a1 = rescale(mo, M);
      st.l[r] = st.l[r] * a0 + lo * a1;
#pragma unroll
      for (int e = 0; e < NP * 8; ++e) st.o[r][e] = st.o[r][e] * a0 + shfl_xor(st.o[r][e], x) * a1;
      st.m[r] = M;
    }
  }

  // merge the waves through LDS
  __shared__ float s_o[kWaves][RT][D];
  __shared__ float s_m[kWaves][RT], s_l[kWaves][RT];
  if (kk == 0) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int c = 0; c < NP; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_o[wave][r][c * 64 + part * 8 + e] = st.o[r][c * 8 + e];
      if (part == 0) {
        s_m[wave][r] = st.m[r];
        s_l[wave][r] = st.l[r];
      }
    }
  }
  __syncthreads();

  const int NR = a.B * a.Lq * a.Hq;
  for (int idx = threadIdx.x; idx < RT * D; idx += kThreads) {
    const int r = idx / D, d = idx - r * D;
    const int rr = tile * RT + r;
    if (rr >= R) continue;
    const int i = rr / a.g, hl = rr - i * a.g;
    const int rowhead = (b * a.Lq + i) * a.Hq + kvh * a.g + hl;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][r]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = rescale(s_m[w][r], M);
      L += wt * s_l[w][r];
      O += wt * s_o[w][r][d];
    }
    if (a.num_splits == 1) {
      float res = 0.f;
      if (L > 0.f) {
        float Z = L;
        if (a.sinks) Z += exp2f(a.sinks[kvh * a.g + hl] * kLog2e - M);
        res = O / Z;
      }
      a.out[(int64_t)rowhead * D + d] = Fmt<BF16>::encode(res);
      if (a.lse && d == 0) a.lse[rowhead] = L > 0.f ? M + log2f(L) : -INFINITY;
    } else {
      const int64_t slot = (int64_t)split * NR + rowhead;
      a.ws_o[slot * D + d] = L > 0.f ? O / L : 0.f;
      if (d == 0) a.ws_lse[slot] = L > 0.f ? M + log2f(L) : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// split merge: one wave per (query row, query head)
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void merge_splits(const DecodeArgs a) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int NR = a.B * a.Lq * a.Hq;
  const int rowhead = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (rowhead >= NR) return;
  const int qrow = rowhead / a.Hq, qhead = rowhead - qrow * a.Hq;
  const int b = qrow / a.Lq;
  const UnitRange u = unit_range(a, b);
  const int S = valid_splits(a, u);
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, a.ws_lse[(int64_t)s * NR + rowhead]);
  float W = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s = 0; s < S; ++s) {
    const int64_t slot = (int64_t)s * NR + rowhead;
    const float w = rescale(a.ws_lse[slot], M);
    W += w;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(w, a.ws_o[slot * D + e * 64 + lane], acc[e]);
  }
  float Z = W;
  if (W > 0.f && a.sinks) Z += exp2f(a.sinks[qhead] * kLog2e - M);
#pragma unroll
  for (int e = 0; e < E; ++e)
    a.out[(int64_t)rowhead * D + e * 64 + lane] = Fmt<BF16>::encode(W > 0.f ? acc[e] / Z : 0.f);
  if (a.lse && lane == 0) a.lse[rowhead] = W > 0.f ? M + log2f(W) : -INFINITY;
}

template <int D, int RT, bool BF16>
hipError_t launch_valu(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  const bool pow2 = a.ps >= kBlockKeys && (a.ps & (a.ps - 1)) == 0;
  if (pow2)
    hipLaunchKernelGGL((decode_valu<D, RT, BF16, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_valu<D, RT, BF16, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_d(const DecodeArgs& a, int rt, dim3 grid, hipStream_t stream) {
  switch (rt) {
    case 4: return launch_valu<D, 4, BF16>(a, grid, stream);
    case 8: return launch_valu<D, 8, BF16>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int path, int rows_per_tile, int head_dim, bool bf16,
                         hipStream_t stream) {
  const dim3 grid(a.num_splits, a.Hkv * a.row_tiles, a.B);
  if (path != kPathValu) return hipErrorInvalidValue;
  if (head_dim == 128)
    return bf16 ? launch_d<128, true>(a, rows_per_tile, grid, stream)
                : launch_d<128, false>(a, rows_per_tile, grid, stream);
  if (head_dim == 64)
    return bf16 ? launch_d<64, true>(a, rows_per_tile, grid, stream)
                : launch_d<64, false>(a, rows_per_tile, grid, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  const int NR = a.B * a.Lq * a.Hq;
  const dim3 grid((NR + kWaves - 1) / kWaves);
  if (head_dim == 128) {
    if (bf16) hipLaunchKernelGGL((merge_splits<128, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((merge_splits<128, false>), grid, dim3(kThreads), 0, stream, a);
  } else if (head_dim == 64) {
    if (bf16) hipLaunchKernelGGL((merge_splits<64, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((merge_splits<64, false>), grid, dim3(kThreads), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkvd
