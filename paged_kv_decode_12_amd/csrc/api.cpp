// api.cpp -- C ABI of the paged-KV decode library: argument validation,
// shape-only launch planning, the split-KV workspace and kernel launches.
//
// Planning never reads device data (sequence lengths stay on the device), so
// a call is safe to capture in a HIP graph once its workspace exists; this is
// the capture-safe alternative to a planner that reads the lengths on the host
// (flashinfer.attention.prims_ts.batch_decode_with_paged_kv_cache, summary).
#include "pkvd.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include <hip/hip_runtime.h>

#include "decode_args.h"
#include "merge_states.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return atoi(s);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

struct Shapes {
  int64_t R, Hq, D, P, Hkv, ps, B, C;
  bool bf16;
};

struct Plan {
  int path;             // pkvd::kPathValu or pkvd::kPathMfma; -1: not plannable
  int rows_per_tile;
  int row_tiles;
  int num_waves;        // waves of the persistent grid
  int min_wave_blocks;  // minimum 16-key blocks per participating wave
  int64_t workgroups;
  int64_t units;        // (request, kv head, row tile) triples: one arrival counter each
  int merge_kernel;      // 1: cut units are merged by a second kernel
  int seg_cost;          // virtual blocks ahead of each unit in the sliced block space
  int slot_w[4];         // slice weights of the waves at position 0..3 on their SIMD
  int64_t slots;         // partial-state slots: two per wave
  // Workspace: one allocation whose first eighth (int_area) holds int32
  // state that is zero when allocated and that every call leaves at zero:
  // the arrival counters (at 0).  The
  // partial LSEs, outputs and the request prefix follow the int area.  The
  // int area's size belongs to the allocation, not the plan, so floats of
  // one plan never lie where another plan keeps int state.  Offsets are
  // relative to each area's start; ws_bytes is the allocation size needed.
  size_t int_bytes;
  size_t ws_lse, ws_o, ws_pref, ws_vpref, float_bytes;
  size_t ws_bytes;
};

// Bytes of the int area of an allocation of `bytes`.
size_t int_area(size_t bytes) { return bytes / 8 / 256 * 256; }

// Shape checks shared by every entry point.  Returns PKVD_OK or an error.
int check_shapes(const pkvd_tensor* q, const pkvd_tensor* k, const pkvd_tensor* bt,
                 int32_t Lq, int32_t wl, Shapes* s) {
  if (!q || !k || !bt) return fail(PKVD_ERR_INVALID_ARG, "q, k_cache and block_tables are required");
  if (q->ndim != 3) return fail(PKVD_ERR_INVALID_ARG, "q must be 3-D (B*q_len_per_req, Hq, D)");
  if (q->dtype != PKVD_BF16 && q->dtype != PKVD_F16)
    return fail(PKVD_ERR_INVALID_ARG, "q must be bf16 or fp16");
  if (k->ndim != 4) return fail(PKVD_ERR_INVALID_ARG, "k_cache must be 4-D (pages, Hkv, page_size, D)");
  if (bt->ndim != 2 || bt->dtype != PKVD_I32)
    return fail(PKVD_ERR_INVALID_ARG, "block_tables must be a 2-D int32 tensor (B, C)");
  if (Lq < 1) return fail(PKVD_ERR_INVALID_ARG, "q_len_per_req must be >= 1");
  if (wl < -1) return fail(PKVD_ERR_INVALID_ARG, "window_left must be -1 or >= 0");
  s->R = q->shape[0];
  s->Hq = q->shape[1];
  s->D = q->shape[2];
  s->P = k->shape[0];
  s->Hkv = k->shape[1];
  s->ps = k->shape[2];
  s->B = bt->shape[0];
  s->C = bt->shape[1];
  s->bf16 = q->dtype == PKVD_BF16;
  if (s->R < 1 || s->Hq < 1 || s->D < 1 || s->P < 1 || s->Hkv < 1 || s->ps < 1 || s->B < 1 ||
      s->C < 1)
    return fail(PKVD_ERR_INVALID_ARG, "every dimension must be >= 1");
  if (k->shape[3] != s->D) return fail(PKVD_ERR_INVALID_ARG, "k_cache head_dim differs from q");
  if (s->R != s->B * Lq)
    return fail(PKVD_ERR_INVALID_ARG, "q.shape[0]=%lld is not B*q_len_per_req=%lld",
                (long long)s->R, (long long)(s->B * Lq));
  if (s->Hq % s->Hkv)
    return fail(PKVD_ERR_INVALID_ARG, "num_heads_qo=%lld is not a multiple of num_heads_kv=%lld",
                (long long)s->Hq, (long long)s->Hkv);
  if (s->D != 64 && s->D != 128)
    return fail(PKVD_ERR_UNSUPPORTED, "head_dim=%lld not built (64 and 128 are)", (long long)s->D);
  if (s->ps > 256) return fail(PKVD_ERR_UNSUPPORTED, "page_size=%lld > 256", (long long)s->ps);
  if (s->B > pkvd::kMaxBatch)
    return fail(PKVD_ERR_UNSUPPORTED, "batch of %lld requests > %d", (long long)s->B,
                pkvd::kMaxBatch);
  if (s->P > INT32_MAX || s->C * s->ps > (1LL << 30) || s->R * s->Hq > (1LL << 30) ||
      s->Hq > 65535)
    return fail(PKVD_ERR_UNSUPPORTED, "problem dimensions exceed the built index ranges");
  return PKVD_OK;
}

// CUs of the current device, waves per workgroup and resident workgroups per
// CU for a kernel; an MI355X (256 CUs, one workgroup per CU) is assumed when
// no device answers.
struct DeviceFit {
  int cus = 256;
  int group_waves = 8;
  int blocks_per_cu = 1;
};

DeviceFit device_fit(int path, int rt, const Shapes& s) {
  DeviceFit f;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return f;
  }
  static std::mutex mu;
  static int cached_cus[64] = {0};
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && dev < 64) {
    if (!cached_cus[dev]) {
      int n = 0;
      if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
          n > 0)
        cached_cus[dev] = n;
      else
        (void)hipGetLastError();
    }
    if (cached_cus[dev]) f.cus = cached_cus[dev];
  }
  const bool pow2 = s.ps >= pkvd::kBlockKeys && (s.ps & (s.ps - 1)) == 0;
  const int gw = pkvd::decode_group_waves(path, rt, (int)s.D);
  if (gw > 0) f.group_waves = gw;
  // One workgroup per CU, holding the WPE waves per SIMD the kernel's
  // register budget was fitted to.  The occupancy query can report room for
  // a second workgroup when the kernel needs fewer registers than that
  // budget, but on MI355X the second one did not become resident alongside
  // (per-wave start stamps: half the waves began only when the first half
  // was done), so the grid is never sized for more than one.
  const int n = pkvd::decode_blocks_per_cu(path, rt, (int)s.D, s.bf16, pow2,
                                           pkvd::decode_lds_bytes((int)s.B, 64 * f.group_waves, 0));
  if (n <= 0) (void)hipGetLastError();
  f.blocks_per_cu = 1;
  return f;
}

// Virtual blocks ahead of each unit in the sliced block space (see make_plan),
// per engine, measured on MI355X (llama3_8b-shaped batch, VALU engine with a
// 6-deep ring: 0 -> 114.3 us, 2 -> 109.9, 3 -> 108.3, 4 -> 106.7, 6 -> 107.1;
// with the 3-deep ring: 5 -> 103.1, 6 -> 103.4, 7 -> 104.5.  MFMA engine,
// spec_verify: 0 -> 118.5 us, 6 -> 116.6).
int default_seg_cost(int path) { return path == pkvd::kPathMfma ? 6 : 5; }

// Default slice weight of the waves at position `slot` on their SIMD.  Equal
// weights measured fastest for the default engines on MI355X (the MFMA
// engine at D = 128 runs one wave per SIMD; for the others the second wave
// finishes last with equal slices, but a CU's waves share one memory pipe,
// so moving blocks to the first wave did not shorten the call).
int default_slot_weight(int path, int rows_per_tile, int slot) {
  (void)path;
  (void)rows_per_tile;
  (void)slot;
  return 100;
}

Plan make_plan(const Shapes& s, int32_t Lq, int32_t wl) {
  Plan p{};
  const int64_t g = s.Hq / s.Hkv;
  const int64_t R = g * Lq;
  // Groups of more than 4 query rows per kv head run on MFMA in 16-row tiles
  // (a group of 8 leaves half of each tile as padding rows); groups of up to
  // 4 use VALU dot products.  The VALU engine issues about 27 vector
  // instructions per (key, kv head) at 4 rows and more at 8, so past 4 rows
  // the vector units, not HBM, set the pace, while the matrix cores are idle.
  // Measured on MI355X: 8 rows, D = 128 (131k-key requests) 248 -> 217 us;
  // 8 rows, D = 64 (window of 128) 50 -> 36 us; 4 rows, D = 128 (2k keys)
  // 118 us VALU vs 135 us MFMA.
  // PKVD_FORCE_PATH=0/1 overrides the choice (for measurements and tests).
  const int forced_path = env_int("PKVD_FORCE_PATH", -1);
  p.path = forced_path == pkvd::kPathValu || forced_path == pkvd::kPathMfma
               ? forced_path
               : (R > 4 ? pkvd::kPathMfma : pkvd::kPathValu);
  p.rows_per_tile = p.path == pkvd::kPathMfma ? 16 : (R <= 4 ? 4 : 8);
  p.row_tiles = (int)((R + p.rows_per_tile - 1) / p.rows_per_tile);
  p.units = s.B * s.Hkv * p.row_tiles;

  // the linear block space must fit int32: units * blocks per unit
  int64_t kcap = s.C * s.ps;
  if (wl >= 0) kcap = std::min<int64_t>(kcap, (int64_t)wl + Lq);
  const int64_t max_blocks = (kcap + pkvd::kBlockKeys - 1) / pkvd::kBlockKeys + 1;
  // Each unit is preceded by seg_cost virtual blocks in the space the waves'
  // slices divide, so a slice that starts a unit (a segment switch costs the
  // wave about as long as streaming a few blocks) holds that many fewer real
  // blocks.  PKVD_SEG_COST overrides the default (0 turns it off).
  int seg_default = default_seg_cost(p.path);
  p.seg_cost = 0;   // set below, once the grid size is known
  if (p.units * (max_blocks + 64) >= INT32_MAX) return Plan{-1};

  const DeviceFit f = device_fit(p.path, p.rows_per_tile, s);
  int64_t nw = (int64_t)f.cus * f.blocks_per_cu * f.group_waves;
  const int forced = env_int("PKVD_WAVES", 0);
  if (forced > 0) nw = forced;
  // at least 2 blocks per participating wave: short batches then spread
  // over many waves (tiny 4-request batch: 24.2 us at 8 blocks, 16.2 us at
  // 2), while long ones use every resident wave anyway
  p.min_wave_blocks = std::max(1, env_int("PKVD_MIN_WAVE_BLOCKS", 2));
  // no more waves than the largest possible work can occupy
  nw = std::min<int64_t>(nw, (p.units * max_blocks + p.min_wave_blocks - 1) / p.min_wave_blocks);
  nw = std::max<int64_t>(1, std::min<int64_t>(nw, 1 << 20));
  p.num_waves = (int)nw;
  // Short units (a window keeps at most 32 blocks) that are at least half as
  // many as the waves: virtual blocks as long as a unit snap every slice
  // boundary to a unit start, so each unit is streamed whole by one wave and
  // none needs a merge (sink + window batch, 1024 units of 9 blocks over
  // 2048 waves: 27.5 -> 23.6 us).  With few units (a 4-request batch) cutting
  // them over more waves is faster.
  if (max_blocks <= 32 && 2 * p.units >= nw) seg_default = (int)max_blocks;
  p.seg_cost = std::min(64, std::max(0, env_int("PKVD_SEG_COST", seg_default)));
  // one workgroup per resident slot (one per CU) even when waves are few,
  // so that they spread over the CUs; more if the waves need more
  p.workgroups = std::max<int64_t>((nw + f.group_waves - 1) / f.group_waves,
                                   std::min<int64_t>((int64_t)f.cus * f.blocks_per_cu, nw));
  // PKVD_GROUPS forces fewer, fuller workgroups (tests reach several waves
  // per SIMD, and so the slot weights, with small grids)
  const int forced_groups = env_int("PKVD_GROUPS", 0);
  if (forced_groups > 0)
    p.workgroups = std::max<int64_t>(forced_groups, (nw + f.group_waves - 1) / f.group_waves);
  // Where cut units leave large partial states (many pieces per unit or wide
  // tiles: over 32 KB per unit) one wave merging a unit at the end would be
  // slow; a second kernel merges them all in parallel instead.  Estimated
  // from shapes only (pieces per unit ~ waves / units + 1).
  const int64_t pieces = nw / std::max<int64_t>(p.units, 1) + 1;
  const int64_t unit_bytes = pieces * p.rows_per_tile * s.D * 4;
  p.merge_kernel = env_int("PKVD_MERGE_KERNEL", unit_bytes > 32768 ? 1 : 0) ? 1 : 0;
  // Slice weights by position on the SIMD: of the two waves a SIMD holds,
  // the first issues ahead of the second and streams faster (per-wave
  // timestamps: about 1.2x the blocks per microsecond, and it starts
  // earlier), so with equal slices the second waves finish last.  Weight
  // W[s] goes to the waves at position s on their SIMD.
  // PKVD_SLOT_W="w0,w1,w2,w3" (1..1024, max/min <= 4) overrides the default.
  for (int r = 0; r < 4; ++r) p.slot_w[r] = default_slot_weight(p.path, p.rows_per_tile, r);
  if (const char* e = getenv("PKVD_SLOT_W")) {
    int w[4] = {0, 0, 0, 0};
    const int n = sscanf(e, "%d,%d,%d,%d", &w[0], &w[1], &w[2], &w[3]);
    for (int r = n; r < 4; ++r) w[r] = n > 0 ? w[n - 1] : 1;
    int lo = 1 << 30, hi = 0;
    for (int r = 0; r < 4; ++r) {
      w[r] = std::min(1024, std::max(1, w[r]));
      lo = std::min(lo, w[r]);
      hi = std::max(hi, w[r]);
    }
    if (n > 0 && hi <= 4 * lo)
      for (int r = 0; r < 4; ++r) p.slot_w[r] = w[r];
  }
  // two partial slots per wave (its slice's first and last segments)
  p.slots = (int64_t)2 * nw;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t rows = (size_t)p.slots * p.rows_per_tile;
  p.int_bytes = up((size_t)p.units * 4);   // the arrival counters
  p.ws_lse = 0;
  p.ws_o = up(rows * 4);
  p.ws_pref = p.ws_o + up(rows * (size_t)s.D * 4);
  p.ws_vpref = p.ws_pref + up((size_t)(s.B + 1) * 4);
  p.float_bytes = p.ws_vpref + up((size_t)(s.B + 1) * 4);
  // smallest allocation whose int area and remainder hold both parts
  size_t S = std::max(8 * p.int_bytes + 2048, p.float_bytes + p.float_bytes / 7 + 2048);
  S = up(S);
  while (int_area(S) < p.int_bytes || S - int_area(S) < p.float_bytes) S += 256;
  p.ws_bytes = S;
  return p;
}

// Library-owned workspace, one per device (layout in Plan).  It is zeroed
// when allocated, and every call leaves its int32 state at zero again.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
Workspace g_ws[64];

int ensure_workspace(size_t bytes, void** out, size_t* size) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKVD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(PKVD_ERR_HIP, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[dev];
  if (w.bytes < bytes) {
    if (w.ptr) {
      e = hipFree(w.ptr);   // waits for work that may still use the old buffer
      w.ptr = nullptr;
      w.bytes = 0;
      if (e != hipSuccess) return fail(PKVD_ERR_HIP, "hipFree: %s", hipGetErrorString(e));
    }
    void* p = nullptr;
    e = hipMalloc(&p, bytes);
    if (e != hipSuccess) return fail(PKVD_ERR_WORKSPACE, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
    e = hipMemset(p, 0, bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      (void)hipFree(p);
      return fail(PKVD_ERR_HIP, "hipMemset(workspace): %s", hipGetErrorString(e));
    }
    w.ptr = p;
    w.bytes = bytes;
  }
  *out = w.ptr;
  *size = w.bytes;
  return PKVD_OK;
}

bool contiguous(const pkvd_tensor* t) {
  int64_t expect = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->strides[i] != expect) return false;
    expect *= t->shape[i];
  }
  return true;
}

}  // namespace

extern "C" {

const char* pkvd_version(void) { return "0.1.0"; }

const char* pkvd_last_error(void) { return g_last_error.c_str(); }

const char* pkvd_status_string(int status) {
  switch (status) {
    case PKVD_OK: return "ok";
    case PKVD_ERR_INVALID_ARG: return "invalid argument";
    case PKVD_ERR_UNSUPPORTED: return "unsupported";
    case PKVD_ERR_WORKSPACE: return "workspace allocation failed";
    case PKVD_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int pkvd_decode_plan(const pkvd_tensor* q, const pkvd_tensor* k_cache,
                     const pkvd_tensor* block_tables, int32_t q_len_per_req, int32_t window_left,
                     int64_t out[6]) {
  Shapes s;
  int st = check_shapes(q, k_cache, block_tables, q_len_per_req, window_left, &s);
  if (st != PKVD_OK) return st;
  if (!out) return fail(PKVD_ERR_INVALID_ARG, "out is NULL");
  Plan p = make_plan(s, q_len_per_req, window_left);
  if (p.path < 0) return fail(PKVD_ERR_UNSUPPORTED, "block-table capacity C * page_size too large");
  out[0] = p.path;
  out[1] = p.rows_per_tile;
  out[2] = p.row_tiles;
  out[3] = p.num_waves;
  out[4] = p.min_wave_blocks;
  out[5] = p.workgroups;
  return PKVD_OK;
}

int pkvd_decode_workspace_bytes(const pkvd_tensor* q, const pkvd_tensor* k_cache,
                                const pkvd_tensor* block_tables, int32_t q_len_per_req,
                                int32_t window_left, size_t* bytes) {
  Shapes s;
  int st = check_shapes(q, k_cache, block_tables, q_len_per_req, window_left, &s);
  if (st != PKVD_OK) return st;
  if (!bytes) return fail(PKVD_ERR_INVALID_ARG, "bytes is NULL");
  const Plan p = make_plan(s, q_len_per_req, window_left);
  if (p.path < 0) return fail(PKVD_ERR_UNSUPPORTED, "block-table capacity C * page_size too large");
  *bytes = p.ws_bytes;
  return PKVD_OK;
}

int pkvd_reserve_workspace(size_t bytes) {
  void* p = nullptr;
  size_t size = 0;
  g_last_error.clear();
  if (bytes == 0) return PKVD_OK;
  return ensure_workspace(bytes, &p, &size);
}

int pkvd_decode(const pkvd_tensor* q, const pkvd_tensor* k_cache, const pkvd_tensor* v_cache,
                const pkvd_tensor* block_tables, const pkvd_tensor* seq_lens_kv, float scale,
                int32_t q_len_per_req, int32_t window_left, const pkvd_tensor* sinks,
                pkvd_tensor* out, pkvd_tensor* lse, void* stream) {
  g_last_error.clear();
  Shapes s;
  int st = check_shapes(q, k_cache, block_tables, q_len_per_req, window_left, &s);
  if (st != PKVD_OK) return st;
  const pkvd_tensor* k = k_cache;
  const pkvd_tensor* v = v_cache;
  if (!v || !seq_lens_kv || !out) return fail(PKVD_ERR_INVALID_ARG, "v_cache, seq_lens_kv and out are required");
  if (!q->data || !k->data || !v->data || !block_tables->data || !seq_lens_kv->data || !out->data)
    return fail(PKVD_ERR_INVALID_ARG, "NULL data pointer");
  if (!isfinite(scale)) return fail(PKVD_ERR_INVALID_ARG, "scale must be finite");
  // q: head_dim innermost and dense, rows 16-byte aligned
  if (q->strides[2] != 1) return fail(PKVD_ERR_INVALID_ARG, "q must have head_dim innermost and dense");
  if (!aligned16(q->data) || q->strides[0] % 8 || q->strides[1] % 8)
    return fail(PKVD_ERR_INVALID_ARG, "q rows must start 16-byte aligned");
  // K / V
  for (const pkvd_tensor* t : {k, v}) {
    const char* nm = t == k ? "k_cache" : "v_cache";
    if (t->ndim != 4 || t->dtype != q->dtype)
      return fail(PKVD_ERR_INVALID_ARG, "%s must be 4-D with q's dtype", nm);
    if (t->shape[0] != s.P || t->shape[1] != s.Hkv || t->shape[2] != s.ps || t->shape[3] != s.D)
      return fail(PKVD_ERR_INVALID_ARG, "k_cache and v_cache shapes differ");
    if (t->strides[3] != 1 || (s.ps > 1 && t->strides[2] != s.D))
      return fail(PKVD_ERR_INVALID_ARG, "%s pages must hold contiguous [page_size, head_dim] tiles", nm);
    if (!aligned16(t->data) || t->strides[0] % 8 || t->strides[1] % 8)
      return fail(PKVD_ERR_INVALID_ARG, "%s tiles must be 16-byte aligned", nm);
    if (t->strides[0] < 0 || t->strides[1] < 0)
      return fail(PKVD_ERR_INVALID_ARG, "%s strides must be non-negative", nm);
  }
  if (s.Hq / s.Hkv < 1) return fail(PKVD_ERR_INVALID_ARG, "num_heads_qo < num_heads_kv");
  // tables
  if (block_tables->strides[1] != 1 || block_tables->strides[0] < s.C)
    return fail(PKVD_ERR_INVALID_ARG, "block_tables rows must be contiguous and not overlap");
  if (seq_lens_kv->ndim != 1 || seq_lens_kv->dtype != PKVD_I32 || seq_lens_kv->shape[0] != s.B ||
      (s.B > 1 && seq_lens_kv->strides[0] != 1))
    return fail(PKVD_ERR_INVALID_ARG, "seq_lens_kv must be a contiguous int32 (B,) tensor");
  if (sinks) {
    if (!sinks->data || sinks->ndim != 1 || sinks->dtype != PKVD_F32 || sinks->shape[0] != s.Hq ||
        (s.Hq > 1 && sinks->strides[0] != 1))
      return fail(PKVD_ERR_INVALID_ARG, "sinks must be a contiguous float32 (num_heads_qo,) tensor");
    // the decode kernel stages the sink logits in LDS
    if (s.Hq > pkvd::kMaxSinkHeads)
      return fail(PKVD_ERR_UNSUPPORTED, "sinks with num_heads_qo=%lld > %d", (long long)s.Hq,
                  pkvd::kMaxSinkHeads);
  }
  if (out->ndim != 3 || out->dtype != q->dtype || out->shape[0] != s.R || out->shape[1] != s.Hq ||
      out->shape[2] != s.D || !contiguous(out))
    return fail(PKVD_ERR_INVALID_ARG, "out must be contiguous (B*q_len_per_req, Hq, D) with q's dtype");
  if (lse) {
    if (!lse->data || lse->ndim != 2 || lse->dtype != PKVD_F32 || lse->shape[0] != s.R ||
        lse->shape[1] != s.Hq || !contiguous(lse))
      return fail(PKVD_ERR_INVALID_ARG, "lse must be contiguous float32 (B*q_len_per_req, Hq)");
  }

  const Plan p = make_plan(s, q_len_per_req, window_left);
  if (p.path < 0) return fail(PKVD_ERR_UNSUPPORTED, "block-table capacity C * page_size too large");
  pkvd::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q->data);
  a.q_sr = q->strides[0];
  a.q_sh = q->strides[1];
  a.k = static_cast<const uint16_t*>(k->data);
  a.k_sp = k->strides[0];
  a.k_sh = k->strides[1];
  a.v = static_cast<const uint16_t*>(v->data);
  a.v_sp = v->strides[0];
  a.v_sh = v->strides[1];
  a.bt = static_cast<const int32_t*>(block_tables->data);
  a.bt_sr = block_tables->strides[0];
  a.seq_lens = static_cast<const int32_t*>(seq_lens_kv->data);
  a.sinks = sinks ? static_cast<const float*>(sinks->data) : nullptr;
  a.out = static_cast<uint16_t*>(out->data);
  a.lse = lse ? static_cast<float*>(lse->data) : nullptr;
  a.B = (int32_t)s.B;
  a.Hq = (int32_t)s.Hq;
  a.Hkv = (int32_t)s.Hkv;
  a.g = (int32_t)(s.Hq / s.Hkv);
  a.Lq = q_len_per_req;
  a.ps = (int32_t)s.ps;
  a.P = (int32_t)s.P;
  a.C = (int32_t)s.C;
  a.window_left = window_left;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.D = (int32_t)s.D;
  a.row_tiles = p.row_tiles;
  a.num_waves = p.num_waves;
  a.groups = (int32_t)p.workgroups;
  a.min_wave_blocks = p.min_wave_blocks;
#ifdef PKVD_TRACE
  {
    const char* t = getenv("PKVD_TRACE_PTR");   // device buffer of >= waves * 16 uint64
    a.trace = t ? reinterpret_cast<uint64_t*>(strtoull(t, nullptr, 0)) : nullptr;
  }
#endif
  void* ws = nullptr;
  size_t ws_size = 0;
  st = ensure_workspace(p.ws_bytes, &ws, &ws_size);
  if (st != PKVD_OK) return st;
  char* wi = static_cast<char*>(ws);            // int area
  char* wf = wi + int_area(ws_size);            // floats follow it
  a.counters = reinterpret_cast<int32_t*>(wi);
  a.ws_lse = reinterpret_cast<float*>(wf + p.ws_lse);
  a.ws_o = reinterpret_cast<float*>(wf + p.ws_o);
  a.ws_pref = reinterpret_cast<int32_t*>(wf + p.ws_pref);
  a.ws_vpref = reinterpret_cast<int32_t*>(wf + p.ws_vpref);
  a.seg_cost = p.seg_cost;
  a.merge_kernel = p.merge_kernel;
  for (int r = 0; r < 4; ++r) a.slot_w[r] = p.slot_w[r];
  if (env_int("PKVD_LOG", 0))
    fprintf(stderr,
            "pkvd: path=%d rows/tile=%d tiles=%d waves=%d min_wave_blocks=%d merge=%d\n",
            p.path, p.rows_per_tile, p.row_tiles, p.num_waves, p.min_wave_blocks, p.merge_kernel);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = pkvd::launch_decode(a, p.path, p.rows_per_tile, s.bf16, hs);
  if (e != hipSuccess) return fail(PKVD_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return PKVD_OK;
}

int pkvd_merge_states(const pkvd_tensor* v, const pkvd_tensor* s, const pkvd_tensor* sinks,
                      pkvd_tensor* v_out, pkvd_tensor* s_out, void* stream) {
  g_last_error.clear();
  if (!v || !s || !v_out) return fail(PKVD_ERR_INVALID_ARG, "v, s and v_out are required");
  if (v->ndim != 4) return fail(PKVD_ERR_INVALID_ARG, "v must be 4-D (S, rows, heads, D)");
  if (v->dtype != PKVD_BF16 && v->dtype != PKVD_F16 && v->dtype != PKVD_F32)
    return fail(PKVD_ERR_INVALID_ARG, "v must be bf16, fp16 or fp32");
  const int64_t S = v->shape[0], R = v->shape[1], H = v->shape[2], D = v->shape[3];
  if (S < 1 || R < 0 || H < 1 || D < 1)
    return fail(PKVD_ERR_INVALID_ARG, "need S >= 1, heads >= 1, D >= 1");
  if (H > INT32_MAX || D > INT32_MAX || S > (1LL << 40) || R * H > (1LL << 40))
    return fail(PKVD_ERR_UNSUPPORTED, "merge dimensions exceed the built index ranges");
  if (!contiguous(v)) return fail(PKVD_ERR_INVALID_ARG, "v must be contiguous");
  if (s->ndim != 3 || s->dtype != PKVD_F32 || s->shape[0] != S || s->shape[1] != R ||
      s->shape[2] != H || !contiguous(s))
    return fail(PKVD_ERR_INVALID_ARG, "s must be contiguous float32 (S, rows, heads)");
  if (v_out->ndim != 3 || v_out->dtype != v->dtype || v_out->shape[0] != R ||
      v_out->shape[1] != H || v_out->shape[2] != D || !contiguous(v_out))
    return fail(PKVD_ERR_INVALID_ARG, "v_out must be contiguous (rows, heads, D) with v's dtype");
  if (s_out && (s_out->ndim != 2 || s_out->dtype != PKVD_F32 || s_out->shape[0] != R ||
                s_out->shape[1] != H || !contiguous(s_out)))
    return fail(PKVD_ERR_INVALID_ARG, "s_out must be contiguous float32 (rows, heads)");
  if (sinks && (sinks->ndim != 1 || sinks->dtype != PKVD_F32 || sinks->shape[0] != H ||
                !contiguous(sinks)))
    return fail(PKVD_ERR_INVALID_ARG, "sinks must be a contiguous float32 (heads,) tensor");
  const bool empty = R == 0;
  if (!empty && (!v->data || !s->data || !v_out->data || (s_out && !s_out->data) ||
                 (sinks && !sinks->data)))
    return fail(PKVD_ERR_INVALID_ARG, "NULL data pointer");
  if (empty) return PKVD_OK;
  pkvd::MergeArgs a{};
  a.v = v->data;
  a.s = static_cast<const float*>(s->data);
  a.sinks = sinks ? static_cast<const float*>(sinks->data) : nullptr;
  a.v_out = v_out->data;
  a.s_out = s_out ? static_cast<float*>(s_out->data) : nullptr;
  a.S = S;
  a.items = R * H;
  a.H = (int32_t)H;
  a.D = (int32_t)D;
  const int dt = v->dtype == PKVD_BF16 ? 0 : (v->dtype == PKVD_F16 ? 1 : 2);
  hipError_t e = pkvd::launch_merge_states(a, dt, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKVD_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
  return PKVD_OK;
}

}  // extern "C"
