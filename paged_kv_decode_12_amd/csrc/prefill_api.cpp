// prefill_api.cpp -- C ABI entry point of context attention (pkvd_prefill):
// argument validation and the launch of the prefill kernel.  The operation
// is that of flashinfer.attention.prims_ts.batch_prefill (summary and
// Parameters).
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include <hip/hip_runtime.h>

#include "api_util.h"
#include "decode_args.h"
#include "pkvd.h"
#include "prefill_args.h"

using namespace pkvd::api;

namespace {

// A (rows, heads, D) view of a fixed (B, S, H, D) or packed (total, H, D)
// tensor: its row and head strides.  Fixed tensors must step their S rows at
// one stride (stride[0] == S * stride[1]).
int rows_view(const pkvd_tensor* t, bool packed, const char* nm, int64_t* rows, int64_t* sr,
              int64_t* sh) {
  if (packed ? t->ndim != 3 : t->ndim != 4)
    return fail(PKVD_ERR_INVALID_ARG, "%s must be %s", nm,
                packed ? "3-D (total, H, D) with packed offsets" : "4-D (B, S, H, D)");
  const int o = packed ? 0 : 1;
  if (t->strides[o + 2] != 1)
    return fail(PKVD_ERR_INVALID_ARG, "%s must have head_dim innermost and dense", nm);
  // a fixed tensor's (b, s) rows are row b * S + s at one stride: with S == 1
  // that stride is the batch stride, with B == 1 the sequence stride
  *sr = t->strides[o];
  if (!packed && t->shape[1] == 1) *sr = t->strides[0];
  else if (!packed && t->shape[0] > 1 && t->strides[0] != t->shape[1] * t->strides[1])
    return fail(PKVD_ERR_INVALID_ARG, "%s must hold its S rows at one stride", nm);
  *rows = packed ? t->shape[0] : t->shape[0] * t->shape[1];
  *sh = t->strides[o + 1];
  if (!aligned16(t->data) || *sr % 8 || *sh % 8 || *sr < 0 || *sh < 0)
    return fail(PKVD_ERR_INVALID_ARG, "%s rows must start 16-byte aligned", nm);
  return PKVD_OK;
}

}  // namespace

extern "C" int pkvd_prefill(const pkvd_prefill_args* x, void* stream) {
  clear_error();
  if (!x || !x->q || !x->k || !x->v || !x->out)
    return fail(PKVD_ERR_INVALID_ARG, "q, k, v and out are required");
  const pkvd_tensor *q = x->q, *k = x->k, *v = x->v;
  if (!q->data || !k->data || !v->data || !x->out->data)
    return fail(PKVD_ERR_INVALID_ARG, "NULL data pointer");
  if (q->dtype != PKVD_BF16 && q->dtype != PKVD_F16)
    return fail(PKVD_ERR_INVALID_ARG, "q must be bf16 or fp16");
  if (k->dtype != q->dtype || v->dtype != q->dtype)
    return fail(PKVD_ERR_INVALID_ARG, "k and v must have q's dtype");
  const bool packed = x->qo_indptr != nullptr;
  if (packed != (x->kv_indptr != nullptr))
    return fail(PKVD_ERR_INVALID_ARG, "qo_indptr and kv_indptr are given together or not at all");
  int64_t rq, rk, rv, q_sr, q_sh, k_sr, k_sh, v_sr, v_sh;
  int st = rows_view(q, packed, "q", &rq, &q_sr, &q_sh);
  if (st == PKVD_OK) st = rows_view(k, packed, "k", &rk, &k_sr, &k_sh);
  if (st == PKVD_OK) st = rows_view(v, packed, "v", &rv, &v_sr, &v_sh);
  if (st != PKVD_OK) return st;
  const int o = packed ? 0 : 1;
  const int64_t Hq = q->shape[o + 1], D = q->shape[o + 2], Hkv = k->shape[o + 1];
  for (int i = 0; i < k->ndim; ++i)
    if (v->shape[i] != k->shape[i]) return fail(PKVD_ERR_INVALID_ARG, "k and v shapes differ");
  if (k->shape[o + 2] != D) return fail(PKVD_ERR_INVALID_ARG, "k head_dim differs from q");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv)
    return fail(PKVD_ERR_INVALID_ARG, "num q heads %lld is not a multiple of kv heads %lld",
                (long long)Hq, (long long)Hkv);
  if (D != 128 && D != 256)
    return fail(PKVD_ERR_UNSUPPORTED, "head_dim=%lld not built for prefill (128 and 256 are)",
                (long long)D);
  int64_t B, Sq, Sk;
  if (packed) {
    const pkvd_tensor *qo = x->qo_indptr, *ko = x->kv_indptr;
    if (qo->ndim != 1 || ko->ndim != 1 || qo->dtype != PKVD_I32 || ko->dtype != PKVD_I32 ||
        qo->shape[0] < 2 || ko->shape[0] != qo->shape[0] || qo->strides[0] != 1 ||
        ko->strides[0] != 1 || !qo->data || !ko->data)
      return fail(PKVD_ERR_INVALID_ARG,
                  "qo_indptr and kv_indptr must be contiguous int32 (B + 1,) tensors");
    B = qo->shape[0] - 1;
    if (x->max_seq_len_q < 1) return fail(PKVD_ERR_INVALID_ARG, "max_seq_len_q must be >= 1");
    Sq = x->max_seq_len_q;
    Sk = 0;
  } else {
    B = q->shape[0];
    Sq = q->shape[1];
    Sk = k->shape[1];
    if (k->shape[0] != B) return fail(PKVD_ERR_INVALID_ARG, "q and k batch sizes differ");
    if (Sq < 1 || Sk < 1 || B < 1) return fail(PKVD_ERR_INVALID_ARG, "every dimension must be >= 1");
  }
  if (x->mask != PKVD_MASK_CAUSAL && x->mask != PKVD_MASK_DENSE &&
      x->mask != PKVD_MASK_VARIABLE_WINDOW)
    return fail(PKVD_ERR_INVALID_ARG, "mask must be causal, dense or variable_window");
  if (x->window_left < -1) return fail(PKVD_ERR_INVALID_ARG, "window_left must be -1 or >= 0");
  if (x->mask == PKVD_MASK_VARIABLE_WINDOW) {
    if (packed) return fail(PKVD_ERR_INVALID_ARG, "variable_window needs fixed-shape inputs");
    if (x->window_left != -1)
      return fail(PKVD_ERR_INVALID_ARG, "variable_window takes window_left = -1");
    for (const pkvd_tensor* t : {x->window_starts, x->window_ends})
      if (!t || !t->data || t->ndim != 2 || t->dtype != PKVD_I32 || t->shape[0] != B ||
          t->shape[1] != Sq || !contiguous(t))
        return fail(PKVD_ERR_INVALID_ARG,
                    "variable_window needs contiguous int32 (B, Sq) window_starts and window_ends");
  }
  if (!isfinite(x->sm_scale) || !isfinite(x->output_scale))
    return fail(PKVD_ERR_INVALID_ARG, "sm_scale and output_scale must be finite");
  const pkvd_tensor* out = x->out;
  if (out->ndim != q->ndim || !contiguous(out))
    return fail(PKVD_ERR_INVALID_ARG, "out must be contiguous with q's shape");
  for (int i = 0; i < q->ndim; ++i)
    if (out->shape[i] != q->shape[i]) return fail(PKVD_ERR_INVALID_ARG, "out must have q's shape");
  if (out->dtype != PKVD_BF16 && out->dtype != PKVD_F16 && out->dtype != PKVD_F32)
    return fail(PKVD_ERR_INVALID_ARG, "out must be bf16, fp16 or fp32");
  if (!aligned16(out->data)) return fail(PKVD_ERR_INVALID_ARG, "out must be 16-byte aligned");
  // out is written while other workgroups still read q, k and v (and the
  // rescaling kernel reads q again after the first kernel's stores)
  if (overlaps(out, q) || overlaps(out, k) || overlaps(out, v))
    return fail(PKVD_ERR_INVALID_ARG, "out must not overlap q, k or v");
  // the kernel's per-lane offsets within a tile of keys are 32-bit
  if (k_sr > (INT32_MAX - 8 * D) / 64 || v_sr > (INT32_MAX - 8 * D) / 64)
    return fail(PKVD_ERR_UNSUPPORTED, "k/v row strides exceed the built index range");
  int hpw = 0, tt = 0;
  if (!pkvd::prefill_geometry((int)D, (int)(Hq / Hkv), &hpw, &tt))
    return fail(PKVD_ERR_UNSUPPORTED, "head_dim=%lld not built for prefill", (long long)D);
  const int64_t m_tiles = (Sq + tt - 1) / tt;
  const int64_t groups = B * Hkv * ((Hq / Hkv) / hpw);
  if (rq > INT32_MAX || rk > INT32_MAX || rq * Hq * D > (1LL << 40) || Sq > INT32_MAX ||
      Sk > INT32_MAX || groups * m_tiles > INT32_MAX - 8 || B * Sq > INT32_MAX)
    return fail(PKVD_ERR_UNSUPPORTED, "problem dimensions exceed the built index ranges");
  pkvd::PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q->data);
  a.q_sr = q_sr;
  a.q_sh = q_sh;
  a.k = static_cast<const uint16_t*>(k->data);
  a.k_sr = k_sr;
  a.k_sh = k_sh;
  a.v = static_cast<const uint16_t*>(v->data);
  a.v_sr = v_sr;
  a.v_sh = v_sh;
  a.qo = packed ? static_cast<const int32_t*>(x->qo_indptr->data) : nullptr;
  a.kvo = packed ? static_cast<const int32_t*>(x->kv_indptr->data) : nullptr;
  a.starts = x->mask == PKVD_MASK_VARIABLE_WINDOW ? static_cast<const int32_t*>(x->window_starts->data) : nullptr;
  a.ends = x->mask == PKVD_MASK_VARIABLE_WINDOW ? static_cast<const int32_t*>(x->window_ends->data) : nullptr;
  a.out = out->data;
  a.out_type = out->dtype == PKVD_BF16 ? pkvd::kOutBf16 : out->dtype == PKVD_F16 ? pkvd::kOutF16 : pkvd::kOutF32;
  a.B = (int32_t)B;
  a.Hq = (int32_t)Hq;
  a.Hkv = (int32_t)Hkv;
  a.g = (int32_t)(Hq / Hkv);
  a.D = (int32_t)D;
  a.Sq = (int32_t)Sq;
  a.Sk = (int32_t)Sk;
  a.rows_q = (int32_t)rq;
  a.rows_kv = (int32_t)rk;
  a.mask = x->mask == PKVD_MASK_CAUSAL ? pkvd::kPrefillCausal
           : x->mask == PKVD_MASK_DENSE ? pkvd::kPrefillDense : pkvd::kPrefillVariable;
  a.window_left = x->window_left;
  a.scale_log2 = (float)((double)x->sm_scale * 1.4426950408889634);
  a.out_scale = x->output_scale;
  a.hpw = hpw;
  a.tt = tt;
  a.groups = (int32_t)groups;
  a.m_tiles = (int32_t)m_tiles;
  a.items = (int32_t)(groups * m_tiles);
  // the rescaling kernel: one workgroup per CU (its LDS ring fits one)
  a.safe_grid = std::min(a.items, std::max(device_cus(), 1));
  hipError_t e = pkvd::launch_prefill(a, q->dtype == PKVD_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKVD_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return PKVD_OK;
}
