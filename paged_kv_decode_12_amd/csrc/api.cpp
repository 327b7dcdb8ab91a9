// api.cpp -- C ABI of the paged-KV decode library: argument validation,
// shape-only launch planning, the split-KV workspace and kernel launches.
//
// Planning never reads device data (sequence lengths and packed query offsets
// stay on the device), so a call is safe to capture in a HIP graph once its
// workspace exists; this is the capture-safe alternative to a planner that
// reads the lengths on the host
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
#include <vector>

#include <hip/hip_runtime.h>

#include "decode_args.h"
#include "merge_states.h"
#include "api_util.h"
#include "schedule.h"

namespace pkvd {
namespace api {

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

void clear_error() { g_last_error.clear(); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool contiguous(const pkvd_tensor* t) {
  int64_t expect = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->strides[i] != expect) return false;
    expect *= t->shape[i];
  }
  return true;
}

namespace {
// [*lo, *hi): the bytes a tensor's elements may occupy; false when empty.
bool byte_span(const pkvd_tensor* t, uintptr_t* lo, uintptr_t* hi) {
  const uintptr_t elt = t->dtype == PKVD_F32 || t->dtype == PKVD_I32 ? 4 : 2;
  uintptr_t last = 0;   // offset of the last element, in elements
  for (int i = 0; i < t->ndim; ++i) {
    if (t->shape[i] <= 0) return false;
    last += (uintptr_t)(t->shape[i] - 1) * (uintptr_t)(t->strides[i] < 0 ? 0 : t->strides[i]);
  }
  *lo = reinterpret_cast<uintptr_t>(t->data);
  *hi = *lo + (last + 1) * elt;
  return true;
}
}  // namespace

bool overlaps(const pkvd_tensor* a, const pkvd_tensor* b) {
  uintptr_t a0, a1, b0, b1;
  if (!byte_span(a, &a0, &a1) || !byte_span(b, &b0, &b1)) return false;
  return a0 < b1 && b0 < a1;
}

// CUs of the current device (cached per device); an MI355X (256 CUs) is
// assumed when no device answers.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  static std::mutex mu;
  static int cached[64] = {0};
  if (dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cached[dev] = n;
    else
      (void)hipGetLastError();
  }
  return cached[dev] ? cached[dev] : 256;
}

}  // namespace api
}  // namespace pkvd

namespace {

using namespace pkvd::api;

constexpr size_t kMaxLdsBytes = 160 * 1024;   // LDS a workgroup may hold on gfx950

// ---------------------------------------------------------------------------
// tuning overrides (measurement and test knobs), read from the environment
// once, and again on pkvd_reload_tuning()
// ---------------------------------------------------------------------------
struct Tuning {
  int force_path = -1;       // PKVD_FORCE_PATH: 0 VALU, 1 MFMA
  int waves = 0;             // PKVD_WAVES: waves of the persistent grid
  int min_wave_blocks = 2;   // PKVD_MIN_WAVE_BLOCKS
  int seg_cost = -1;         // PKVD_SEG_COST: virtual blocks ahead of each unit
  int groups = 0;            // PKVD_GROUPS: workgroups
  int merge_kernel = -1;     // PKVD_MERGE_KERNEL: 0 in place, 1 second kernel
  int unit_mode = -1;        // PKVD_UNIT_MODE: 0 block slices, 1 whole units
  int slot_w[4] = {0, 0, 0, 0};   // PKVD_SLOT_W="w0,w1,w2,w3" (0: default)
  int log = 0;               // PKVD_LOG: print each plan to stderr
};

std::mutex g_tuning_mutex;
Tuning g_tuning;
bool g_tuning_loaded = false;

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return atoi(s);
}

Tuning read_tuning() {
  Tuning t;
  t.force_path = env_int("PKVD_FORCE_PATH", -1);
  t.waves = env_int("PKVD_WAVES", 0);
  t.min_wave_blocks = std::max(1, env_int("PKVD_MIN_WAVE_BLOCKS", 2));
  t.seg_cost = env_int("PKVD_SEG_COST", -1);
  t.groups = env_int("PKVD_GROUPS", 0);
  t.merge_kernel = env_int("PKVD_MERGE_KERNEL", -1);
  t.unit_mode = env_int("PKVD_UNIT_MODE", -1);
  t.log = env_int("PKVD_LOG", 0);
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
      for (int r = 0; r < 4; ++r) t.slot_w[r] = w[r];
  }
  return t;
}

Tuning tuning() {
  std::lock_guard<std::mutex> lock(g_tuning_mutex);
  if (!g_tuning_loaded) {
    g_tuning = read_tuning();
    g_tuning_loaded = true;
  }
  return g_tuning;
}

// ---------------------------------------------------------------------------
// shapes and plan
// ---------------------------------------------------------------------------
struct Shapes {
  int64_t rows, Hq, D, P, Hkv, ps, B, C;
  int64_t Lq;      // fixed rows per request, or the packed capacity
  bool packed;
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
  int merge_kernel;     // 1: cut units are merged by a second kernel
  int unit_mode;        // 1: slice bounds snap to unit starts (no unit is cut)
  int seg_cost;         // virtual blocks ahead of each unit in the sliced block space
  int slot_w[4];        // slice weights of the waves at position 0..3 on their SIMD
  int64_t slots;        // partial-state slots: two per wave
  int group_waves;      // waves per workgroup
  size_t lds_bytes;     // dynamic LDS of the decode kernel
  // Workspace: one allocation whose first eighth (int_area) holds int32
  // state that is zero when allocated and that every call leaves at zero:
  // the arrival counters.  The partial LSEs, outputs and the request
  // prefixes follow the int area.  The int area's size belongs to the
  // allocation, not the plan, so floats of one plan never lie where another
  // plan keeps int state.  Offsets are relative to each area's start;
  // ws_bytes is the allocation size needed.
  size_t int_bytes;
  size_t ws_lse, ws_o, ws_pref, ws_vpref, float_bytes;
  size_t ws_bytes;
};

// Bytes of the int area of an allocation of `bytes`.
size_t int_area(size_t bytes) { return bytes / 8 / 256 * 256; }

// Shape checks shared by every entry point: q (rows, Hq, D) or token-major
// (B, SQ, Hq, D), k_cache (pages, Hkv, page_size, D), block_tables (B, C).
int check_shapes(const pkvd_tensor* q, const pkvd_tensor* k, const pkvd_tensor* bt,
                 const pkvd_tensor* qo, int32_t Lq, int32_t wl, Shapes* s) {
  if (!q || !k || !bt) return fail(PKVD_ERR_INVALID_ARG, "q, k_cache and block_tables are required");
  if (q->ndim != 3 && q->ndim != 4)
    return fail(PKVD_ERR_INVALID_ARG, "q must be 3-D (rows, Hq, D) or 4-D (B, SQ, Hq, D)");
  if (q->dtype != PKVD_BF16 && q->dtype != PKVD_F16)
    return fail(PKVD_ERR_INVALID_ARG, "q must be bf16 or fp16");
  if (k->ndim != 4) return fail(PKVD_ERR_INVALID_ARG, "k_cache must be 4-D (pages, Hkv, page_size, D)");
  if (bt->ndim != 2 || bt->dtype != PKVD_I32)
    return fail(PKVD_ERR_INVALID_ARG, "block_tables must be a 2-D int32 tensor (B, C)");
  if (Lq < 1) return fail(PKVD_ERR_INVALID_ARG, "q_len_per_req must be >= 1");
  if (wl < -1) return fail(PKVD_ERR_INVALID_ARG, "window_left must be -1 or >= 0");
  const int o = q->ndim - 3;   // a 4-D q is (B, SQ) rows
  s->rows = o ? q->shape[0] * q->shape[1] : q->shape[0];
  s->Hq = q->shape[o + 1];
  s->D = q->shape[o + 2];
  s->P = k->shape[0];
  s->Hkv = k->shape[1];
  s->ps = k->shape[2];
  s->B = bt->shape[0];
  s->C = bt->shape[1];
  s->Lq = Lq;
  s->packed = qo != nullptr;
  s->bf16 = q->dtype == PKVD_BF16;
  if (s->rows < 1 || s->Hq < 1 || s->D < 1 || s->P < 1 || s->Hkv < 1 || s->ps < 1 || s->B < 1 ||
      s->C < 1)
    return fail(PKVD_ERR_INVALID_ARG, "every dimension must be >= 1");
  if (k->shape[3] != s->D) return fail(PKVD_ERR_INVALID_ARG, "k_cache head_dim differs from q");
  if (o && q->shape[0] != s->B)
    return fail(PKVD_ERR_INVALID_ARG, "a 4-D q must be (B, SQ, Hq, D) with B = block_tables rows");
  if (!s->packed && s->rows != s->B * Lq)
    return fail(PKVD_ERR_INVALID_ARG, "q holds %lld rows, not B*q_len_per_req=%lld",
                (long long)s->rows, (long long)(s->B * Lq));
  if (s->packed) {
    if (o) return fail(PKVD_ERR_INVALID_ARG, "packed rows (qo_indptr) need a 3-D q (total_q, Hq, D)");
    if (qo->ndim != 1 || qo->dtype != PKVD_I32 || qo->shape[0] != s->B + 1 ||
        qo->strides[0] != 1 || !qo->data)
      return fail(PKVD_ERR_INVALID_ARG, "qo_indptr must be a contiguous int32 (B + 1,) tensor");
  }
  if (s->Hq % s->Hkv)
    return fail(PKVD_ERR_INVALID_ARG, "num_heads_qo=%lld is not a multiple of num_heads_kv=%lld",
                (long long)s->Hq, (long long)s->Hkv);
  if (s->D != 64 && s->D != 128)
    return fail(PKVD_ERR_UNSUPPORTED, "head_dim=%lld not built (64 and 128 are)", (long long)s->D);
  if (s->ps > 256) return fail(PKVD_ERR_UNSUPPORTED, "page_size=%lld > 256", (long long)s->ps);
  if (s->B > pkvd::kMaxBatch)
    return fail(PKVD_ERR_UNSUPPORTED, "batch of %lld requests > %d", (long long)s->B,
                pkvd::kMaxBatch);
  if (s->P > INT32_MAX || s->C * s->ps > (1LL << 30) || s->rows * s->Hq > (1LL << 30) ||
      s->Hq > 65535 || (s->Hq / s->Hkv) * Lq > 65535)
    return fail(PKVD_ERR_UNSUPPORTED, "problem dimensions exceed the built index ranges");
  return PKVD_OK;
}

// Virtual blocks ahead of each unit in the sliced block space, per engine,
// measured on MI355X (llama3_8b-shaped batch, VALU engine with a 6-deep ring:
// 0 -> 114.3 us, 2 -> 109.9, 3 -> 108.3, 4 -> 106.7, 6 -> 107.1; with the
// 3-deep ring: 5 -> 103.1, 6 -> 103.4, 7 -> 104.5.  MFMA engine, spec_verify:
// 0 -> 118.5 us, 6 -> 116.6).
int default_seg_cost(int path) { return path == pkvd::kPathMfma ? 6 : 5; }

Plan make_plan(const Shapes& s, int32_t wl, const Tuning& tu) {
  Plan p{};
  const int64_t g = s.Hq / s.Hkv;
  const int64_t R = g * s.Lq;
  // Groups of more than 4 query rows per kv head run on MFMA in 16-row tiles
  // (a group of 8 leaves half of each tile as padding rows); groups of up to
  // 4 use VALU dot products.  The VALU engine issues about 27 vector
  // instructions per (key, kv head) at 4 rows and more at 8, so past 4 rows
  // the vector units, not HBM, set the pace, while the matrix cores are idle.
  // Measured on MI355X: 8 rows, D = 128 (131k-key requests) 248 -> 217 us;
  // 8 rows, D = 64 (window of 128) 50 -> 36 us; 4 rows, D = 128 (2k keys)
  // 118 us VALU vs 135 us MFMA.
  p.path = tu.force_path == pkvd::kPathValu || tu.force_path == pkvd::kPathMfma
               ? tu.force_path
               : (R > 4 ? pkvd::kPathMfma : pkvd::kPathValu);
  p.rows_per_tile = p.path == pkvd::kPathMfma ? 16 : (R <= 4 ? 4 : 8);
  p.row_tiles = (int)((R + p.rows_per_tile - 1) / p.rows_per_tile);
  p.units = s.B * s.Hkv * p.row_tiles;
  p.group_waves = pkvd::decode_group_waves(p.path, p.rows_per_tile, (int)s.D);
  if (p.group_waves <= 0) return Plan{-1};

  // the linear block space must fit int32: units * blocks per unit
  int64_t kcap = s.C * s.ps;
  if (wl >= 0) kcap = std::min<int64_t>(kcap, (int64_t)wl + s.Lq);
  const int64_t max_blocks = (kcap + pkvd::kBlockKeys - 1) / pkvd::kBlockKeys + 1;
  if (p.units * (max_blocks + 64) >= INT32_MAX) return Plan{-1};

  // One workgroup per CU, holding the waves per SIMD the kernel's register
  // budget was fitted to.  (The occupancy calculator can report room for a
  // second workgroup when the kernel needs fewer registers than that budget,
  // but on MI355X the second one did not become resident alongside: per-wave
  // start stamps showed half the waves beginning only when the first half
  // was done.)
  const int cus = device_cus();
  int64_t nw = (int64_t)cus * p.group_waves;
  if (tu.waves > 0) nw = tu.waves;
  // at least 2 blocks per participating wave: short batches then spread
  // over many waves (tiny 4-request batch: 24.2 us at 8 blocks, 16.2 us at
  // 2), while long ones use every resident wave anyway
  p.min_wave_blocks = tu.min_wave_blocks;
  // no more waves than the largest possible work can occupy
  nw = std::min<int64_t>(nw, (p.units * max_blocks + p.min_wave_blocks - 1) / p.min_wave_blocks);
  nw = std::max<int64_t>(1, std::min<int64_t>(nw, 1 << 20));
  // Short units (a window keeps at most 32 blocks) that are at least half as
  // many as the waves are streamed whole, one wave per unit: the slice
  // bounds snap to unit starts, so no unit is cut and nothing is merged.
  // (Cutting 1024 window units of 9 blocks over 2048 waves wrote 9 MB of
  // partial states per call.)  With few units (a 4-request batch) cutting
  // them over more waves is faster.
  p.unit_mode = max_blocks <= 32 && 2 * p.units >= nw ? 1 : 0;
  if (tu.unit_mode == 0 || tu.unit_mode == 1) p.unit_mode = tu.unit_mode;
  if (p.unit_mode && tu.waves <= 0) nw = std::min<int64_t>(nw, p.units);
  p.num_waves = (int)nw;
  p.seg_cost = p.unit_mode ? 0
                           : std::min(64, std::max(0, tu.seg_cost >= 0 ? tu.seg_cost
                                                                      : default_seg_cost(p.path)));
  // one workgroup per resident slot (one per CU) even when waves are few,
  // so that they spread over the CUs; more if the waves need more
  p.workgroups = std::max<int64_t>((nw + p.group_waves - 1) / p.group_waves,
                                   std::min<int64_t>((int64_t)cus, nw));
  // PKVD_GROUPS forces fewer, fuller workgroups (tests reach several waves
  // per SIMD, and so the slot weights, with small grids)
  if (tu.groups > 0)
    p.workgroups = std::max<int64_t>(tu.groups, (nw + p.group_waves - 1) / p.group_waves);
  // Where cut units leave large partial states (many pieces per unit or wide
  // tiles: over 32 KB per unit) one wave merging a unit at the end would be
  // slow; a second kernel merges them all in parallel instead.  Estimated
  // from shapes only (pieces per unit ~ waves / units + 1).
  const int64_t pieces = nw / std::max<int64_t>(p.units, 1) + 1;
  const int64_t unit_bytes = pieces * p.rows_per_tile * s.D * 4;
  p.merge_kernel = tu.merge_kernel >= 0 ? (tu.merge_kernel ? 1 : 0) : (unit_bytes > 32768 ? 1 : 0);
  if (p.unit_mode) p.merge_kernel = 0;   // nothing to merge
  // Slice weights by position on the SIMD (equal by default: they measured
  // fastest for the default engines).
  for (int r = 0; r < 4; ++r) p.slot_w[r] = tu.slot_w[0] > 0 ? tu.slot_w[r] : 100;
  p.lds_bytes = pkvd::decode_lds_bytes((int)s.B, 64 * p.group_waves, 0, s.packed);
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

// ---------------------------------------------------------------------------
// workspaces
// ---------------------------------------------------------------------------
// Library-owned, one per device.  It is zeroed when allocated, and every call
// leaves its int32 state at zero again.  It only grows; a buffer it replaces
// is kept (never freed) until the process ends, because a HIP graph captured
// earlier may still launch kernels on it.  It never grows while the stream is
// capturing (the call fails with PKVD_ERR_WORKSPACE instead).
struct DeviceWorkspace {
  void* ptr = nullptr;
  size_t bytes = 0;
  std::vector<void*> retired;
  void* bound = nullptr;     // pkvd_set_workspace: the caller's buffer (not owned)
  size_t bound_bytes = 0;
};
std::mutex g_ws_mutex;
DeviceWorkspace g_ws[64];

int current_device(int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return fail(PKVD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (*dev < 0 || *dev >= 64) return fail(PKVD_ERR_HIP, "device id %d out of range", *dev);
  return PKVD_OK;
}

bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs != hipStreamCaptureStatusNone;
}

// Grows the library-owned workspace of the current device to >= bytes.
int grow_library_workspace(int dev, size_t bytes, hipStream_t stream, bool may_capture) {
  DeviceWorkspace& w = g_ws[dev];
  if (w.bytes >= bytes) return PKVD_OK;
  if (may_capture && stream_capturing(stream))
    return fail(PKVD_ERR_WORKSPACE,
                "the workspace needs %zu bytes (it holds %zu) and the stream is capturing a "
                "graph: call pkvd_reserve_workspace (or pass a workspace) before the capture",
                bytes, w.bytes);
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PKVD_ERR_WORKSPACE, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
  }
  e = hipMemset(p, 0, bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(p);
    return fail(PKVD_ERR_HIP, "hipMemset(workspace): %s", hipGetErrorString(e));
  }
  if (w.ptr) w.retired.push_back(w.ptr);
  w.ptr = p;
  w.bytes = bytes;
  return PKVD_OK;
}

// The workspace of one call: the caller's per-call buffer, else the buffer
// bound to the device with pkvd_set_workspace, else the library's own.
int resolve_workspace(void* call_ws, size_t call_bytes, size_t need, hipStream_t stream,
                      void** out, size_t* size) {
  if (call_ws) {
    if (call_bytes < need)
      return fail(PKVD_ERR_WORKSPACE, "workspace of %zu bytes is too small: this call needs %zu",
                  call_bytes, need);
    *out = call_ws;
    *size = call_bytes;
    return PKVD_OK;
  }
  int dev = 0;
  int st = current_device(&dev);
  if (st != PKVD_OK) return st;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  DeviceWorkspace& w = g_ws[dev];
  if (w.bound) {
    if (w.bound_bytes < need)
      return fail(PKVD_ERR_WORKSPACE,
                  "the bound workspace of %zu bytes is too small: this call needs %zu",
                  w.bound_bytes, need);
    *out = w.bound;
    *size = w.bound_bytes;
    return PKVD_OK;
  }
  st = grow_library_workspace(dev, need, stream, true);
  if (st != PKVD_OK) return st;
  *out = w.ptr;
  *size = w.bytes;
  return PKVD_OK;
}

// Checks of everything a decode call reads or writes beyond the shapes.
int check_call(const pkvd_decode_args* x, const Shapes& s) {
  const pkvd_tensor* q = x->q;
  const pkvd_tensor* k = x->k_cache;
  const pkvd_tensor* v = x->v_cache;
  if (!v || !x->seq_lens_kv || !x->out)
    return fail(PKVD_ERR_INVALID_ARG, "v_cache, seq_lens_kv and out are required");
  if (!q->data || !k->data || !v->data || !x->block_tables->data || !x->seq_lens_kv->data ||
      !x->out->data)
    return fail(PKVD_ERR_INVALID_ARG, "NULL data pointer");
  if (!isfinite(x->scale)) return fail(PKVD_ERR_INVALID_ARG, "scale must be finite");
  if (!isfinite(x->out_scale)) return fail(PKVD_ERR_INVALID_ARG, "out_scale must be finite");
  if (x->mask != PKVD_MASK_CAUSAL && x->mask != PKVD_MASK_DENSE)
    return fail(PKVD_ERR_INVALID_ARG, "mask must be PKVD_MASK_CAUSAL or PKVD_MASK_DENSE");
  // q: head_dim innermost and dense, rows 16-byte aligned; a 4-D q must
  // step its SQ rows evenly (stride[0] = SQ * stride[1]) so that it is a
  // (B * SQ, Hq, D) row tensor
  const int o = q->ndim - 3;
  if (q->strides[o + 2] != 1) return fail(PKVD_ERR_INVALID_ARG, "q must have head_dim innermost and dense");
  if (o && q->shape[1] > 1 && q->strides[0] != q->shape[1] * q->strides[1])
    return fail(PKVD_ERR_INVALID_ARG, "a 4-D q must hold its SQ rows at one stride");
  const int64_t q_sr = o ? q->strides[1] : q->strides[0], q_sh = q->strides[o + 1];
  if (!aligned16(q->data) || q_sr % 8 || q_sh % 8)
    return fail(PKVD_ERR_INVALID_ARG, "q rows must start 16-byte aligned");
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
  const pkvd_tensor* bt = x->block_tables;
  if (bt->strides[1] != 1 || bt->strides[0] < s.C)
    return fail(PKVD_ERR_INVALID_ARG, "block_tables rows must be contiguous and not overlap");
  const pkvd_tensor* sl = x->seq_lens_kv;
  if (sl->ndim != 1 || sl->dtype != PKVD_I32 || sl->shape[0] != s.B ||
      (s.B > 1 && sl->strides[0] != 1))
    return fail(PKVD_ERR_INVALID_ARG, "seq_lens_kv must be a contiguous int32 (B,) tensor");
  if (x->sinks) {
    const pkvd_tensor* sk = x->sinks;
    if (!sk->data || sk->ndim != 1 || sk->dtype != PKVD_F32 || sk->shape[0] != s.Hq ||
        (s.Hq > 1 && sk->strides[0] != 1))
      return fail(PKVD_ERR_INVALID_ARG, "sinks must be a contiguous float32 (num_heads_qo,) tensor");
    // the decode kernel stages the sink logits in LDS
    if (s.Hq > pkvd::kMaxSinkHeads)
      return fail(PKVD_ERR_UNSUPPORTED, "sinks with num_heads_qo=%lld > %d", (long long)s.Hq,
                  pkvd::kMaxSinkHeads);
  }
  // out: q's shape (3-D rows or 4-D token-major), contiguous, bf16 / fp16 / fp32
  const pkvd_tensor* out = x->out;
  if (out->ndim != q->ndim || !contiguous(out))
    return fail(PKVD_ERR_INVALID_ARG, "out must be contiguous with q's shape");
  for (int i = 0; i < q->ndim; ++i)
    if (out->shape[i] != q->shape[i]) return fail(PKVD_ERR_INVALID_ARG, "out must have q's shape");
  if (out->dtype != PKVD_BF16 && out->dtype != PKVD_F16 && out->dtype != PKVD_F32)
    return fail(PKVD_ERR_INVALID_ARG, "out must be bf16, fp16 or fp32");
  if (!aligned16(out->data)) return fail(PKVD_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (x->lse) {
    const pkvd_tensor* l = x->lse;
    const bool two_d = l->ndim == 2 && l->shape[0] == s.rows && l->shape[1] == s.Hq;
    const bool three_d = o && l->ndim == 3 && l->shape[0] == q->shape[0] &&
                         l->shape[1] == q->shape[1] && l->shape[2] == s.Hq;
    if (!l->data || l->dtype != PKVD_F32 || !(two_d || three_d) || !contiguous(l))
      return fail(PKVD_ERR_INVALID_ARG, "lse must be contiguous float32 (rows, Hq)");
  }
  if (x->workspace && (reinterpret_cast<uintptr_t>(x->workspace) & 255))
    return fail(PKVD_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return PKVD_OK;
}

int shapes_of(const pkvd_decode_args* x, Shapes* s) {
  if (!x) return fail(PKVD_ERR_INVALID_ARG, "args is NULL");
  return check_shapes(x->q, x->k_cache, x->block_tables, x->qo_indptr, x->q_len, x->window_left, s);
}

int plan_of(const Shapes& s, int32_t wl, Plan* p) {
  *p = make_plan(s, wl, tuning());
  if (p->path < 0) return fail(PKVD_ERR_UNSUPPORTED, "block-table capacity C * page_size too large");
  return PKVD_OK;
}

// The kernel arguments of a call (everything but the workspace).
void fill_args(const pkvd_decode_args* x, const Shapes& s, const Plan& p, pkvd::DecodeArgs* out) {
  const pkvd_tensor* q = x->q;
  const int o = q->ndim - 3;
  pkvd::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q->data);
  a.q_sr = o ? q->strides[1] : q->strides[0];
  a.q_sh = q->strides[o + 1];
  a.k = static_cast<const uint16_t*>(x->k_cache->data);
  a.k_sp = x->k_cache->strides[0];
  a.k_sh = x->k_cache->strides[1];
  a.v = x->v_cache ? static_cast<const uint16_t*>(x->v_cache->data) : nullptr;
  a.v_sp = x->v_cache ? x->v_cache->strides[0] : 0;
  a.v_sh = x->v_cache ? x->v_cache->strides[1] : 0;
  a.bt = static_cast<const int32_t*>(x->block_tables->data);
  a.bt_sr = x->block_tables->strides[0];
  a.seq_lens = x->seq_lens_kv ? static_cast<const int32_t*>(x->seq_lens_kv->data) : nullptr;
  a.qo = x->qo_indptr ? static_cast<const int32_t*>(x->qo_indptr->data) : nullptr;
  a.sinks = x->sinks ? static_cast<const float*>(x->sinks->data) : nullptr;
  a.out = x->out ? x->out->data : nullptr;
  const int od = x->out ? x->out->dtype : x->q->dtype;
  a.out_type = od == PKVD_BF16 ? pkvd::kOutBf16 : od == PKVD_F16 ? pkvd::kOutF16 : pkvd::kOutF32;
  a.lse = x->lse ? static_cast<float*>(x->lse->data) : nullptr;
  a.B = (int32_t)s.B;
  a.Hq = (int32_t)s.Hq;
  a.Hkv = (int32_t)s.Hkv;
  a.g = (int32_t)(s.Hq / s.Hkv);
  a.Lq = x->q_len;
  a.rows = (int32_t)s.rows;
  a.ps = (int32_t)s.ps;
  a.P = (int32_t)s.P;
  a.C = (int32_t)s.C;
  a.window_left = x->window_left;
  a.causal = x->mask == PKVD_MASK_CAUSAL ? 1 : 0;
  a.scale_log2 = (float)((double)x->scale * 1.4426950408889634);
  a.out_scale = x->out_scale;
  a.D = (int32_t)s.D;
  a.row_tiles = p.row_tiles;
  a.rows_per_tile = p.rows_per_tile;
  a.num_waves = p.num_waves;
  a.groups = (int32_t)p.workgroups;
  a.min_wave_blocks = p.min_wave_blocks;
  a.seg_cost = p.seg_cost;
  a.unit_mode = p.unit_mode;
  a.merge_kernel = p.merge_kernel;
  for (int r = 0; r < 4; ++r) a.slot_w[r] = p.slot_w[r];
  pkvd::dev::set_full_grid(a);
  *out = a;
}

int run_decode(const pkvd_decode_args* x, void* stream) {
  g_last_error.clear();
  Shapes s;
  int st = shapes_of(x, &s);
  if (st != PKVD_OK) return st;
  st = check_call(x, s);
  if (st != PKVD_OK) return st;
  Plan p;
  st = plan_of(s, x->window_left, &p);
  if (st != PKVD_OK) return st;
  const size_t lds = pkvd::decode_lds_bytes((int)s.B, 64 * p.group_waves,
                                            x->sinks ? (int)s.Hq : 0, s.packed);
  if (lds > kMaxLdsBytes)
    return fail(PKVD_ERR_UNSUPPORTED, "%lld requests with these options need %zu bytes of LDS",
                (long long)s.B, lds);
  pkvd::DecodeArgs a;
  fill_args(x, s, p, &a);
#ifdef PKVD_TRACE
  {
    const char* t = getenv("PKVD_TRACE_PTR");   // device buffer of >= waves * 16 uint64
    a.trace = t ? reinterpret_cast<uint64_t*>(strtoull(t, nullptr, 0)) : nullptr;
  }
#endif
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  size_t ws_size = 0;
  st = resolve_workspace(x->workspace, x->workspace_bytes, p.ws_bytes, hs, &ws, &ws_size);
  if (st != PKVD_OK) return st;
  char* wi = static_cast<char*>(ws);            // int area
  char* wf = wi + int_area(ws_size);            // floats follow it
  a.counters = reinterpret_cast<int32_t*>(wi);
  a.ws_lse = reinterpret_cast<float*>(wf + p.ws_lse);
  a.ws_o = reinterpret_cast<float*>(wf + p.ws_o);
  a.ws_pref = reinterpret_cast<int32_t*>(wf + p.ws_pref);
  a.ws_vpref = reinterpret_cast<int32_t*>(wf + p.ws_vpref);
  if (tuning().log)
    fprintf(stderr,
            "pkvd: path=%d rows/tile=%d tiles=%d waves=%d min_wave_blocks=%d merge=%d unit=%d "
            "seg_cost=%d\n",
            p.path, p.rows_per_tile, p.row_tiles, p.num_waves, p.min_wave_blocks, p.merge_kernel,
            p.unit_mode, p.seg_cost);
  hipError_t e = pkvd::launch_decode(a, p.path, p.rows_per_tile, s.bf16, hs);
  if (e != hipSuccess) return fail(PKVD_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return PKVD_OK;
}

pkvd_decode_args fixed_args(const pkvd_tensor* q, const pkvd_tensor* k_cache,
                            const pkvd_tensor* v_cache, const pkvd_tensor* block_tables,
                            const pkvd_tensor* seq_lens_kv, float scale, int32_t q_len_per_req,
                            int32_t window_left, const pkvd_tensor* sinks, pkvd_tensor* out,
                            pkvd_tensor* lse) {
  pkvd_decode_args x;
  memset(&x, 0, sizeof x);
  x.q = q;
  x.k_cache = k_cache;
  x.v_cache = v_cache;
  x.block_tables = block_tables;
  x.seq_lens_kv = seq_lens_kv;
  x.qo_indptr = nullptr;
  x.q_len = q_len_per_req;
  x.mask = PKVD_MASK_CAUSAL;
  x.window_left = window_left;
  x.scale = scale;
  x.out_scale = 1.0f;
  x.sinks = sinks;
  x.out = out;
  x.lse = lse;
  x.workspace = nullptr;
  x.workspace_bytes = 0;
  return x;
}

void plan_array(const Plan& p, int64_t* out, int n) {
  const int64_t v[8] = {p.path,       p.rows_per_tile,   p.row_tiles,    p.num_waves,
                        p.min_wave_blocks, p.workgroups, p.merge_kernel, p.unit_mode};
  for (int i = 0; i < n && i < 8; ++i) out[i] = v[i];
}

}  // namespace

extern "C" {

const char* pkvd_version(void) { return "0.2.0"; }

const char* pkvd_last_error(void) { return g_last_error.c_str(); }

const char* pkvd_status_string(int status) {
  switch (status) {
    case PKVD_OK: return "ok";
    case PKVD_ERR_INVALID_ARG: return "invalid argument";
    case PKVD_ERR_UNSUPPORTED: return "unsupported";
    case PKVD_ERR_WORKSPACE: return "workspace missing, too small or not allocatable";
    case PKVD_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

void pkvd_reload_tuning(void) {
  std::lock_guard<std::mutex> lock(g_tuning_mutex);
  g_tuning = read_tuning();
  g_tuning_loaded = true;
}

int pkvd_decode_plan(const pkvd_tensor* q, const pkvd_tensor* k_cache,
                     const pkvd_tensor* block_tables, int32_t q_len_per_req, int32_t window_left,
                     int64_t out[6]) {
  g_last_error.clear();
  Shapes s;
  int st = check_shapes(q, k_cache, block_tables, nullptr, q_len_per_req, window_left, &s);
  if (st != PKVD_OK) return st;
  if (!out) return fail(PKVD_ERR_INVALID_ARG, "out is NULL");
  Plan p;
  st = plan_of(s, window_left, &p);
  if (st != PKVD_OK) return st;
  plan_array(p, out, 6);
  return PKVD_OK;
}

int pkvd_decode_workspace_bytes(const pkvd_tensor* q, const pkvd_tensor* k_cache,
                                const pkvd_tensor* block_tables, int32_t q_len_per_req,
                                int32_t window_left, size_t* bytes) {
  g_last_error.clear();
  Shapes s;
  int st = check_shapes(q, k_cache, block_tables, nullptr, q_len_per_req, window_left, &s);
  if (st != PKVD_OK) return st;
  if (!bytes) return fail(PKVD_ERR_INVALID_ARG, "bytes is NULL");
  Plan p;
  st = plan_of(s, window_left, &p);
  if (st != PKVD_OK) return st;
  *bytes = p.ws_bytes;
  return PKVD_OK;
}

int pkvd_decode_ex_plan(const pkvd_decode_args* args, int64_t plan[8], size_t* workspace_bytes) {
  g_last_error.clear();
  Shapes s;
  int st = shapes_of(args, &s);
  if (st != PKVD_OK) return st;
  Plan p;
  st = plan_of(s, args->window_left, &p);
  if (st != PKVD_OK) return st;
  if (plan) plan_array(p, plan, 8);
  if (workspace_bytes) *workspace_bytes = p.ws_bytes;
  return PKVD_OK;
}

int pkvd_reserve_workspace(size_t bytes) {
  g_last_error.clear();
  if (bytes == 0) return PKVD_OK;
  int dev = 0;
  int st = current_device(&dev);
  if (st != PKVD_OK) return st;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  return grow_library_workspace(dev, bytes, nullptr, false);
}

int pkvd_workspace_capacity(size_t* bytes) {
  g_last_error.clear();
  if (!bytes) return fail(PKVD_ERR_INVALID_ARG, "bytes is NULL");
  int dev = 0;
  int st = current_device(&dev);
  if (st != PKVD_OK) return st;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  const DeviceWorkspace& w = g_ws[dev];
  *bytes = w.bound ? w.bound_bytes : w.bytes;
  return PKVD_OK;
}

int pkvd_set_workspace(void* dev_ptr, size_t bytes) {
  g_last_error.clear();
  int dev = 0;
  int st = current_device(&dev);
  if (st != PKVD_OK) return st;
  if (dev_ptr && (reinterpret_cast<uintptr_t>(dev_ptr) & 255))
    return fail(PKVD_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (dev_ptr && bytes < 4096)
    return fail(PKVD_ERR_INVALID_ARG, "workspace of %zu bytes is below the 4096-byte minimum", bytes);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  DeviceWorkspace& w = g_ws[dev];
  if (!dev_ptr) {
    w.bound = nullptr;
    w.bound_bytes = 0;
    return PKVD_OK;
  }
  // the int area must start at zero; every call leaves it at zero again
  hipError_t e = hipMemset(dev_ptr, 0, bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(PKVD_ERR_HIP, "hipMemset(workspace): %s", hipGetErrorString(e));
  w.bound = dev_ptr;
  w.bound_bytes = bytes;
  return PKVD_OK;
}

int pkvd_decode(const pkvd_tensor* q, const pkvd_tensor* k_cache, const pkvd_tensor* v_cache,
                const pkvd_tensor* block_tables, const pkvd_tensor* seq_lens_kv, float scale,
                int32_t q_len_per_req, int32_t window_left, const pkvd_tensor* sinks,
                pkvd_tensor* out, pkvd_tensor* lse, void* stream) {
  const pkvd_decode_args x = fixed_args(q, k_cache, v_cache, block_tables, seq_lens_kv, scale,
                                        q_len_per_req, window_left, sinks, out, lse);
  if (out && q && out->dtype != q->dtype) {
    g_last_error.clear();
    return fail(PKVD_ERR_INVALID_ARG, "out must have q's dtype (pkvd_decode_ex takes others)");
  }
  return run_decode(&x, stream);
}

int pkvd_decode_ex(const pkvd_decode_args* args, void* stream) { return run_decode(args, stream); }

int pkvd_decode_static(const pkvd_tensor* q, const pkvd_tensor* k_cache,
                       const pkvd_tensor* v_cache, const pkvd_tensor* block_tables,
                       const pkvd_tensor* seq_lens_kv, float scale, int32_t q_len_per_req,
                       int32_t window_left, const pkvd_tensor* sinks, pkvd_tensor* out,
                       pkvd_tensor* lse, void* stream) {
  g_last_error.clear();
  pkvd_decode_args x = fixed_args(q, k_cache, v_cache, block_tables, seq_lens_kv, scale,
                                  q_len_per_req, window_left, sinks, out, lse);
  if (out && q && out->dtype != q->dtype)
    return fail(PKVD_ERR_INVALID_ARG, "out must have q's dtype");
  // the size check comes before any HIP call
  Shapes s;
  int st = shapes_of(&x, &s);
  if (st != PKVD_OK) return st;
  Plan p;
  st = plan_of(s, window_left, &p);
  if (st != PKVD_OK) return st;
  if (p.ws_bytes > pkvd::kStaticScratchBytes)
    return fail(PKVD_ERR_WORKSPACE,
                "this call needs %zu bytes of workspace, more than the %zu-byte static workspace "
                "of pkvd_decode_static",
                p.ws_bytes, pkvd::kStaticScratchBytes);
  void* ptr = nullptr;
  size_t bytes = 0;
  hipError_t e = pkvd::static_scratch(&ptr, &bytes);
  if (e != hipSuccess) return fail(PKVD_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  x.workspace = ptr;
  x.workspace_bytes = bytes;
  return run_decode(&x, stream);
}

int pkvd_schedule_stats(const pkvd_decode_args* args, const int32_t* seq_lens,
                        const int32_t* qo_indptr, int64_t stats[8]) {
  using namespace pkvd::dev;
  g_last_error.clear();
  Shapes s;
  int st = shapes_of(args, &s);
  if (st != PKVD_OK) return st;
  if (!seq_lens || !stats || (s.packed && !qo_indptr))
    return fail(PKVD_ERR_INVALID_ARG, "seq_lens, stats (and qo_indptr for packed rows) are required");
  Plan p;
  st = plan_of(s, args->window_left, &p);
  if (st != PKVD_OK) return st;
  pkvd::DecodeArgs a;
  fill_args(args, s, p, &a);
  a.qo = s.packed ? qo_indptr : nullptr;   // the host copy: the helpers below read it
  const int B = (int)s.B;
  // the block prefixes, as the kernel's prologue builds them
  std::vector<int64_t> pref(B + 1), vpref(B + 1);
  std::vector<int> nblk(B), units(B);
  int64_t T = 0, TV = 0;
  for (int b = 0; b < B; ++b) {
    const int c0 = s.packed ? clamp_row(a, qo_indptr[b]) : 0;
    const int c1 = s.packed ? clamp_row(a, qo_indptr[b + 1]) : 0;
    req_blocks(a, b, seq_lens[b], c0, c1, nblk[b], units[b]);
    pref[b] = T;
    vpref[b] = TV;
    T += (int64_t)nblk[b] * units[b];
    TV += (int64_t)unit_vspan(a, nblk[b]) * units[b];
  }
  pref[B] = T;
  vpref[B] = TV;
  if (TV >= INT32_MAX) return fail(PKVD_ERR_UNSUPPORTED, "block space beyond int32");
  int NW;
  const Slices sl = grid_slices(a, (int)TV, (int)T, NW);
  // the full grid's host-set constants give the same slices as the
  // general path
  const int NWg = wave_count(a, (int)T);
  const Slices slg = make_slices(a, (int)TV, NWg);
  int64_t errors = 0;
  if (NWg != NW) ++errors;
  else
    for (int w = 0; w <= NW; ++w)
      if (slice_begin(sl, w) != slice_begin(slg, w)) ++errors;
  // the real block at virtual block v: the request holding v is the last one
  // whose virtual prefix is <= v (as the kernel's search finds it)
  auto real_at = [&](int64_t v) -> int64_t {
    if (v >= TV) return T;
    const int b = (int)(std::upper_bound(vpref.begin(), vpref.begin() + B, v) - vpref.begin()) - 1;
    return real_block(a, (int)pref[b], (int)vpref[b], nblk[b], (int)v);
  };
  std::vector<int64_t> lo(NW + 1);
  for (int w = 0; w <= NW; ++w) lo[w] = T ? real_at(slice_begin(sl, w)) : 0;
  if (lo[0] != 0 || lo[NW] != T) ++errors;
  for (int w = 0; w < NW; ++w)
    if (lo[w] > lo[w + 1]) ++errors;
  // every unit: the waves whose slices hold its blocks, and whether the
  // merge's bookkeeping (unit_pieces, candidate_slot) names exactly those
  int64_t live = 0, cut = 0, pieces = 0, max_pieces = 0;
  for (int b = 0; b < B; ++b) {
    if (nblk[b] == 0) continue;
    for (int u = 0; u < units[b]; ++u) {
      ++live;
      const int64_t us = pref[b] + (int64_t)u * nblk[b], ue = us + nblk[b];
      const int64_t vs = vpref[b] + (int64_t)u * unit_vspan(a, nblk[b]);
      // first wave whose slice ends after us
      int w = (int)(std::upper_bound(lo.begin(), lo.end(), us) - lo.begin()) - 1;
      int n = 0;
      std::vector<int> holders;
      for (; w < NW && lo[w] < ue; ++w)
        if (lo[w + 1] > us && lo[w + 1] > lo[w]) holders.push_back(w);
      n = (int)holders.size();
      if (n == 0) ++errors;   // a unit nobody streams
      if (n > 1) {
        ++cut;
        pieces += n;
        max_pieces = std::max<int64_t>(max_pieces, n);
        const UnitPieces up = unit_pieces(sl, vs, a.seg_cost, nblk[b]);
        std::vector<int> named;
        for (int c = 0; c < up.n; ++c) {
          bool written = false;
          const int slot = candidate_slot(up, sl, vs, c, written);
          if (!written) continue;
          const int ww = up.w0 + c;
          named.push_back(ww);
          // side 0 exactly when the wave's slice starts inside this unit
          if ((slot & 1) != (lo[ww] >= us ? 0 : 1)) ++errors;
        }
        if (named != holders) ++errors;
      }
    }
  }
  stats[0] = T;
  stats[1] = NW;
  stats[2] = live;
  stats[3] = cut;
  stats[4] = pieces;
  stats[5] = max_pieces;
  stats[6] = errors;
  stats[7] = TV;
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

