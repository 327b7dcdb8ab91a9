// schedule.h -- the integer arithmetic of the persistent decode schedule:
// the query rows and key range of a request, the slices of the block space
// the waves stream, where the pieces of a cut unit are, and the LDS layout.
// Pure functions of the launch arguments, compiled for the device (the
// decode and merge kernels) and for the host (the planner's replay of a
// schedule, pkvd_schedule_stats), so both run the same code.
//
// Reference semantics: flashinfer.cudnn.cudnn_batch_decode_with_kv_cache
// (Parameters: q_len_per_req, window_left) and
// flashinfer.attention.prims_ts.batch_decode_with_paged_kv_cache (summary and
// Parameters: qo_indptr, max_seq_len_q, mask_type).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "decode_args.h"

namespace pkvd {
namespace dev {

// ---------------------------------------------------------------------------
// query rows and key range of one request
// ---------------------------------------------------------------------------
// The query rows of request b: rows row0 .. row0 + lq - 1 of q / out.  With
// fixed rows (Parameters / q_len_per_req) every request has Lq of them; with
// packed rows (batch_decode_with_paged_kv_cache: summary, Parameters /
// qo_indptr, max_seq_len_q) request b owns rows qo[b] .. qo[b + 1] - 1, at
// most Lq of them (the capacity the plan's row tiles are sized for).  Packed
// offsets are clamped into [0, rows] and the count into [0, Lq], so offsets
// out of contract never reach memory outside q / out.
struct ReqRows {
  int row0, lq;
};
__host__ __device__ __forceinline__ int clamp_row(const DecodeArgs& a, int r) {
  return r < 0 ? 0 : (r > a.rows ? a.rows : r);
}
__host__ __device__ __forceinline__ ReqRows rows_of(const DecodeArgs& a, int c0, int c1, int b) {
  if (!a.qo) return {b * a.Lq, a.Lq};
  const int n = c1 - c0;
  return {c0, n < 0 ? 0 : (n > a.Lq ? a.Lq : n)};
}
// Row tiles of a request with lq query tokens.
__host__ __device__ __forceinline__ int tiles_of(const DecodeArgs& a, int lq) {
  return (a.g * lq + a.rows_per_tile - 1) / a.rows_per_tile;
}

// Keys some row of request b may see: [lo(row 0), n - 1], where row 0 has the
// lowest diagonal n - lq (Parameters / q_len_per_req) and the window keeps
// window_left keys before a row's diagonal position (Parameters /
// window_left); with the causal mask row i stops at its diagonal, with the
// dense one (mask_type) at n - 1, so the union ends at n - 1 either way.  A
// request without query rows has no keys to stream.  The range is cut into
// 16-key blocks aligned to the absolute key index; the waves' slices are runs
// of these blocks.
struct UnitRange {
  int n;          // sequence length, clamped to the block table's capacity
  int key_lo;     // first key some row sees
  int first_blk;  // block holding key_lo
  int nblk;       // blocks covering [key_lo, n)
};

__host__ __device__ __forceinline__ UnitRange unit_range_n(const DecodeArgs& a, int n_raw, int lq) {
  UnitRange u;
  const int cap = a.C * a.ps;
  const int n = n_raw < 0 ? 0 : (n_raw > cap ? cap : n_raw);
  u.n = n;
  const int lo = (a.window_left < 0) ? 0 : n - lq - a.window_left;
  u.key_lo = lo < 0 ? 0 : lo;
  if (u.key_lo >= n || lq <= 0) {
    u.first_blk = 0;
    u.nblk = 0;
  } else {
    u.first_blk = u.key_lo / kBlockKeys;
    u.nblk = (n - 1) / kBlockKeys - u.first_blk + 1;
  }
  return u;
}

// floor(n / d) for 0 <= n < 2^62, 0 < d < 2^62, and a quotient below 2^31.
// The fp64 quotient has a relative error of about 2^-52 (the rounding of n
// and of the division), so it is within one of the true quotient; integer
// corrections make it exact.  About a tenth of the instructions of a generic
// 64-bit integer division, which matters in the prologue every wave runs.
__host__ __device__ __forceinline__ int64_t qdiv(int64_t n, int64_t d) {
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
  int qT, rT;    // T = qT NW + rT (equal weights)
};
// Total weight of the first m waves of a group (0 <= m <= PER).
__host__ __device__ __forceinline__ int64_t group_weight(const Slices& s, int m) {
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
__host__ __device__ __forceinline__ int64_t weight_before(const Slices& s, int w) {
  const int full = w / s.PER;
  return (int64_t)full * s.SP + group_weight(s, w - full * s.PER);
}
__host__ __device__ __forceinline__ Slices make_slices(const DecodeArgs& a, int T, int NW) {
  Slices s;
  s.T = T;
  s.NW = NW;
  const int groups = a.groups > 0 ? a.groups : 1;
  s.PER = (NW + groups - 1) / groups;
  s.uniform = 1;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s.W[r] = a.slot_w[r];
    if (r * kSimdsPerCu < s.PER) {
      if (s.W[r] != s.W[0]) s.uniform = 0;
    }
  }
  s.SP = group_weight(s, s.PER);
  s.S = weight_before(s, NW);
  s.qT = T / NW;
  s.rT = T - s.qT * NW;
  return s;
}
// First block of wave w's slice (w <= NW).  Equal weights: floor(T w / NW)
// = qT w + floor(rT w / NW), in 32 bits while NW^2 fits.
__host__ __device__ __forceinline__ int slice_begin(const Slices& s, int w) {
  if (s.uniform) {
    if (s.NW <= 32768) return s.qT * w + (s.rT * w) / s.NW;
    return (int)qdiv((int64_t)s.T * w, s.NW);
  }
  return (int)qdiv((int64_t)s.T * weight_before(s, w), s.S);
}
// The wave whose slice holds block x (0 <= x < T): the largest w with
// slice_begin(w) <= x, i.e. with weight_before(w) <= ((x + 1) S - 1) / T.
// That weight is inverted in closed form: whole groups first, then the
// group's waves slot by slot (weights are positive).
__host__ __device__ __forceinline__ int slice_of(const Slices& s, int64_t x) {
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
__host__ __device__ __forceinline__ UnitPieces unit_pieces(const Slices& s, int64_t vs, int seg_cost,
                                                  int nblk) {
  UnitPieces p;
  p.w0 = slice_of(s, vs + seg_cost);
  p.n = slice_of(s, vs + seg_cost + nblk - 1) - p.w0 + 1;
  return p;
}
// Slot of candidate c, and whether it holds a partial state of this call.
__host__ __device__ __forceinline__ int candidate_slot(const UnitPieces& p, const Slices& s, int64_t vs,
                                              int c, bool& written) {
  const int w = p.w0 + c;
  const int b0 = slice_begin(s, w);
  written = b0 < slice_begin(s, w + 1);
  return 2 * w + (b0 >= vs ? 0 : 1);
}

// Waves that take part: at most one per min_wave_blocks blocks, and >= 1.
__host__ __device__ __forceinline__ int wave_count(const DecodeArgs& a, int T) {
  int nw = T / a.min_wave_blocks;
  return nw < 1 ? 1 : (nw > a.num_waves ? a.num_waves : nw);
}

// The host's part of the full grid's slicing (DecodeArgs::full_*).
__host__ __device__ __forceinline__ void set_full_grid(DecodeArgs& a) {
  const int64_t t = (int64_t)a.num_waves * a.min_wave_blocks;
  a.full_T = t < 0x7FFFFFFF ? (int32_t)t : 0x7FFFFFFF;
  const Slices f = make_slices(a, 0, a.num_waves > 0 ? a.num_waves : 1);
  a.full_per = f.PER;
  a.full_uniform = f.uniform;
  a.full_sp = f.SP;
  a.full_s = f.S;
}
// NW = wave_count(a, T) and make_slices(a, TV, NW), with the full grid's
// length-independent parts taken from the host (one division left).
__host__ __device__ __forceinline__ Slices grid_slices(const DecodeArgs& a, int TV, int T, int& NW) {
  if (T < a.full_T || a.full_per <= 0) {
    NW = wave_count(a, T);
    return make_slices(a, TV, NW);
  }
  NW = a.num_waves;
  Slices s;
  s.T = TV;
  s.NW = NW;
  s.uniform = a.full_uniform;
  s.PER = a.full_per;
#pragma unroll
  for (int r = 0; r < 4; ++r) s.W[r] = a.slot_w[r];
  s.SP = a.full_sp;
  s.S = a.full_s;
  s.qT = TV / NW;
  s.rT = TV - s.qT * NW;
  return s;
}

// Dynamic LDS of a workgroup of NT threads, in 32-bit words: the scan scratch
// (2 NT), the block prefixes (2 (B + 1)), the raw lengths (B), the blocks per
// unit (B), the clamped
// packed query offsets (B + 1, packed rows only) and the sink logits (NS).
// Host (launch size) and kernel (carve-up) both take the offsets from here.
struct LdsLayout {
  int scan, vscan, pref, vpref, nlen, nb, qo, sink, total;
};
// NS: sink logits staged in LDS (Hq when they are, else 0).
__host__ __device__ inline LdsLayout lds_layout(int B, int NT, int NS, bool packed) {
  LdsLayout l;
  l.scan = 0;
  l.vscan = l.scan + NT;
  l.pref = l.vscan + NT;
  l.vpref = l.pref + B + 1;
  l.nlen = l.vpref + B + 1;
  l.nb = l.nlen + B;
  l.qo = l.nb + B;
  l.sink = l.qo + (packed ? B + 1 : 0);
  l.total = l.sink + NS;
  return l;
}

// The blocks and units (Hkv x row tiles) of request b, from its raw length
// and its clamped packed offsets c0, c1 (ignored for fixed rows).
__host__ __device__ __forceinline__ ReqRows req_blocks(const DecodeArgs& a, int b, int nraw, int c0,
                                                       int c1, int& nb, int& units) {
  const ReqRows rr = rows_of(a, c0, c1, b);
  nb = unit_range_n(a, nraw, rr.lq).nblk;
  units = a.qo ? a.Hkv * tiles_of(a, rr.lq) : a.Hkv * a.row_tiles;
  return rr;
}

// Virtual blocks one unit of nb real blocks spans in the space the waves'
// slices divide: seg_cost blocks that are never streamed ahead of its nb
// real ones, or, with unit_mode, exactly one (the slices then count whole
// units, so NW waves over NW units give one unit to each wave).
__host__ __device__ __forceinline__ int unit_vspan(const DecodeArgs& a, int nb) {
  return nb <= 0 ? 0 : (a.unit_mode ? 1 : nb + a.seg_cost);
}

// The real block at virtual block v of a request whose blocks start at real
// block pref_b and virtual block vpref_b, nb blocks per unit: the unit's
// first real block for its virtual blocks.  With unit_mode each virtual
// block is one whole unit, so every slice bound is a unit start and no unit
// is cut.
// real_off: the same for the request's virtual offset off = v - vpref_b,
// relative to the request's first real block, and the unit ul (of the
// request) that holds it.
__host__ __device__ __forceinline__ int real_off(const DecodeArgs& a, int nb, int off, int& ul) {
  if (a.unit_mode) {
    ul = off;
    return off * nb;
  }
  const int vu = nb + a.seg_cost;
  ul = vu > 0 ? off / vu : 0;
  const int o = off - ul * vu - a.seg_cost;
  return ul * nb + (o > 0 ? o : 0);
}
__host__ __device__ __forceinline__ int real_block(const DecodeArgs& a, int pref_b, int vpref_b,
                                                   int nb, int v) {
  int ul;
  return pref_b + real_off(a, nb, v - vpref_b, ul);
}

}  // namespace dev
}  // namespace pkvd
