/*
 * oracle.c -- plain fp64 CPU reference for batched paged-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links or calls this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or constant with the HIP path.
 *
 * What it computes (one output row per (query row r, query head h)):
 *   flashinfer.cudnn.cudnn_batch_decode_with_kv_cache
 *     - Parameters / q: q is (batch_size * q_len_per_req, num_heads_qo, head_dim),
 *       the rows of one request are consecutive, so row r belongs to request
 *       b = r / Lq and is that request's i = r % Lq-th query token.
 *     - Parameters / k_cache, v_cache, block_tables: page p of request b's
 *       logical sequence is physical page block_tables[b, p]; key j lives in
 *       page floor(j / page_size), slot j mod page_size (the plain reading of
 *       the HND page layout; the page never states the map explicitly).
 *     - Parameters / q_len_per_req: row i of a request with n keys sees keys
 *       0 .. n - Lq + i (bottom-right causal diagonal p_i = n - Lq + i).
 *     - Parameters / window_left: -1 disables the window; otherwise the row
 *       also drops keys before p_i - window_left (window_left keys before the
 *       diagonal plus the diagonal itself).
 *     - Parameters / sinks: sinks[h] is one extra logit in the softmax
 *       denominator whose value row is zero.  Read as an unscaled logit,
 *       indexed by the query head.
 *     - Note / LSE convention: lse = log2 sum_j exp(scale * q . k_j) over the
 *       row's visible keys (the row's own masked score row); the key-value head
 *       of query head h is h / (Hq / Hkv).  The exported lse excludes the sink;
 *       lse_with_sink also counts it (diagnostic).
 *   flashinfer.attention.prims_ts.batch_decode_with_paged_kv_cache
 *     - summary and Parameters / qo_indptr, max_seq_len_q: with cumulative
 *       query offsets qo_indptr (B + 1 entries) the query rows are packed:
 *       request b owns rows qo_indptr[b] .. qo_indptr[b + 1] - 1, so its
 *       query length Lq_b varies per request and row r is its
 *       i = r - qo_indptr[b]-th token.  Without them every request has the
 *       fixed length Lq (a [B, SQ, Hq, D] token-major tensor is the same
 *       memory as the (B * SQ, Hq, D) rows above).
 *     - Parameters / mask_type: "causal" is the bottom-right diagonal above;
 *       "dense" lets every row see every key j < n (a window, if any, still
 *       starts window_left keys before the row's diagonal position p_i).
 *     - Parameters / bmm2_scale (and batch_prefill's output_scale): the
 *       output is multiplied by this factor; the LSE is not.
 *
 * The softmax is the plain two-pass form: first every visible score and their
 * maximum, then the exponentials, their sum and the weighted sum of V.
 * A row with no visible key (out of contract) gives out = 0, lse = -inf.
 *
 * Inputs stay in their storage format (bf16 or IEEE fp16 bit patterns); this
 * file decodes them itself.  All arithmetic is double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_F16 = 1 };

enum {
  ORACLE_OK = 0,
  ORACLE_BAD_ARG = 1,        /* inconsistent shape or dtype */
  ORACLE_BAD_PAGE = 2,       /* a visible key maps outside the page pool */
  ORACLE_NO_MEMORY = 3
};

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_decode_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int e = (bits >> 10) & 0x1f;
  int m = bits & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);                /* zero and subnormals: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);    /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

static double decode(uint16_t bits, int dtype) {
  return dtype == ORACLE_BF16 ? oracle_decode_bf16(bits) : oracle_decode_f16(bits);
}

typedef struct {
  const uint16_t* q;  int64_t q_sr, q_sh;            /* q[r*q_sr + h*q_sh + d] */
  const uint16_t* k;  int64_t k_sp, k_sh, k_ss;      /* k[p*k_sp + kvh*k_sh + s*k_ss + d] */
  const uint16_t* v;  int64_t v_sp, v_sh, v_ss;
  int dtype;
  int64_t B, Hq, Hkv, D, ps, P;
  const int32_t* bt;  int64_t bt_sr, C;              /* bt[b*bt_sr + c] */
  const int32_t* seq_lens;
  double scale;
  int64_t Lq, wl;                                    /* Lq: fixed query length */
  const int32_t* qo_indptr;                          /* NULL, or packed rows: (B + 1,) */
  int causal;                                        /* 1: bottom-right causal, 0: dense */
  double out_scale;                                  /* factor on the output */
  const float* sinks;                                /* may be NULL */
  int64_t key_lo, key_hi;                            /* extra key restriction [lo, hi) */
} problem_t;

/* Request b, its query length and the token index i of query row r. */
static void row_owner(const problem_t* pb, int64_t r, int64_t* b, int64_t* lq, int64_t* i) {
  if (!pb->qo_indptr) {
    *b = r / pb->Lq;
    *lq = pb->Lq;
    *i = r % pb->Lq;
    return;
  }
  int64_t bb = 0;   /* the request whose row range [qo[b], qo[b + 1]) holds r */
  while (bb + 1 < pb->B && pb->qo_indptr[bb + 1] <= r) ++bb;
  *b = bb;
  *lq = pb->qo_indptr[bb + 1] - pb->qo_indptr[bb];
  *i = r - pb->qo_indptr[bb];
}

/* One (row r, head h).  Returns ORACLE_OK or ORACLE_BAD_PAGE. */
static int one_row(const problem_t* pb, int64_t r, int64_t h, double* s_buf,
                   double* out, double* lse, double* lse_ws) {
  const int64_t D = pb->D;
  int64_t b, lq, i;
  row_owner(pb, r, &b, &lq, &i);
  const int64_t g = pb->Hq / pb->Hkv, kvh = h / g;
  const int64_t n = pb->seq_lens[b];

  /* visible keys: lo <= j <= hi, 0 <= j < n */
  const int64_t diag = n - lq + i;
  int64_t hi = pb->causal ? diag : n - 1;
  int64_t lo = (pb->wl < 0) ? 0 : diag - pb->wl;
  if (lo < 0) lo = 0;
  if (hi > n - 1) hi = n - 1;
  if (lo < pb->key_lo) lo = pb->key_lo;
  if (hi > pb->key_hi - 1) hi = pb->key_hi - 1;

  const uint16_t* qrow = pb->q + r * pb->q_sr + h * pb->q_sh;
  double* qd = s_buf;                /* D decoded query values, then scores */
  double* s = s_buf + D;
  for (int64_t d = 0; d < D; ++d) qd[d] = decode(qrow[d], pb->dtype);

  /* pass 1: scores and their maximum */
  int64_t cnt = 0;
  double m = -INFINITY;
  for (int64_t j = lo; j <= hi; ++j) {
    int64_t col = j / pb->ps, slot = j % pb->ps;
    if (col >= pb->C) return ORACLE_BAD_PAGE;
    int64_t page = pb->bt[b * pb->bt_sr + col];
    if (page < 0 || page >= pb->P) return ORACLE_BAD_PAGE;
    const uint16_t* krow = pb->k + page * pb->k_sp + kvh * pb->k_sh + slot * pb->k_ss;
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += qd[d] * decode(krow[d], pb->dtype);
    s[cnt] = pb->scale * dot;
    if (s[cnt] > m) m = s[cnt];
    ++cnt;
  }
  const int has_sink = pb->sinks != NULL;
  const double sink = has_sink ? (double)pb->sinks[h] : 0.0;

  if (cnt == 0) {
    for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
    *lse = -INFINITY;
    *lse_ws = has_sink ? sink / log(2.0) : -INFINITY;
    return ORACLE_OK;
  }
  const double m_all = (has_sink && sink > m) ? sink : m;

  /* pass 2: exponentials, their sum, weighted sum of V */
  for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
  double S = 0.0;
  cnt = 0;
  for (int64_t j = lo; j <= hi; ++j) {
    int64_t page = pb->bt[b * pb->bt_sr + j / pb->ps];
    const uint16_t* vrow = pb->v + page * pb->v_sp + kvh * pb->v_sh + (j % pb->ps) * pb->v_ss;
    double w = exp(s[cnt++] - m_all);
    S += w;
    for (int64_t d = 0; d < D; ++d) out[d] += w * decode(vrow[d], pb->dtype);
  }
  const double Z = S + (has_sink ? exp(sink - m_all) : 0.0);
  for (int64_t d = 0; d < D; ++d) out[d] = pb->out_scale * (out[d] / Z);
  *lse = (m_all + log(S)) / log(2.0);
  *lse_ws = (m_all + log(Z)) / log(2.0);
  return ORACLE_OK;
}

/*
 * oracle_decode: compute selected (row, head) outputs.
 *   sel   : NULL for every (r, h) in row-major order r * Hq + h, else nsel
 *           indices r * Hq + h.
 *   out   : [count, D] doubles;  lse, lse_with_sink : [count] doubles.
 *   key_lo, key_hi : additionally restrict keys to [key_lo, key_hi)
 *           (pass 0 and INT64_MAX for none); used to build partial states.
 *   qo_indptr : NULL (every request has Lq rows) or (B + 1,) cumulative row
 *           offsets of packed rows (Lq is then unused).
 *   causal : 1 bottom-right causal rows, 0 dense rows.
 *   out_scale : factor on the output (1 for none).
 *   nthreads : OpenMP threads (<= 0: library default).
 */
int oracle_decode(const uint16_t* q, int64_t q_sr, int64_t q_sh,
                  const uint16_t* k, int64_t k_sp, int64_t k_sh, int64_t k_ss,
                  const uint16_t* v, int64_t v_sp, int64_t v_sh, int64_t v_ss,
                  int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                  int64_t ps, int64_t P,
                  const int32_t* block_tables, int64_t bt_sr, int64_t C,
                  const int32_t* seq_lens, double scale, int64_t Lq, int64_t window_left,
                  const int32_t* qo_indptr, int causal, double out_scale,
                  const float* sinks, int64_t key_lo, int64_t key_hi,
                  const int64_t* sel, int64_t nsel,
                  double* out, double* lse, double* lse_with_sink, int nthreads) {
  if (!q || !k || !v || !block_tables || !seq_lens || !out || !lse || !lse_with_sink)
    return ORACLE_BAD_ARG;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_F16) return ORACLE_BAD_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || ps < 1 || P < 1 || C < 1 || Lq < 1)
    return ORACLE_BAD_ARG;
  if (Hq % Hkv != 0 || window_left < -1) return ORACLE_BAD_ARG;
  int64_t rows = B * Lq;
  if (qo_indptr) {
    if (qo_indptr[0] != 0) return ORACLE_BAD_ARG;
    for (int64_t b = 0; b < B; ++b)
      if (qo_indptr[b + 1] < qo_indptr[b]) return ORACLE_BAD_ARG;
    rows = qo_indptr[B];
  }

  problem_t pb = {q, q_sr, q_sh, k, k_sp, k_sh, k_ss, v, v_sp, v_sh, v_ss, dtype,
                  B, Hq, Hkv, D, ps, P, block_tables, bt_sr, C, seq_lens, scale,
                  Lq, window_left, qo_indptr, causal ? 1 : 0, out_scale,
                  sinks, key_lo, key_hi};
  int64_t nmax = 0;
  for (int64_t b = 0; b < B; ++b)
    if (seq_lens[b] > nmax) nmax = seq_lens[b];
  const int64_t count = sel ? nsel : rows * Hq;
  int status = ORACLE_OK;

#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

#pragma omp parallel
  {
    double* buf = (double*)malloc(sizeof(double) * (size_t)(D + nmax + 1));
    if (!buf) {
#pragma omp atomic write
      status = ORACLE_NO_MEMORY;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < count; ++t) {
      if (!buf) continue;
      int64_t idx = sel ? sel[t] : t;
      int64_t r = idx / Hq, h = idx % Hq;
      if (r < 0 || r >= rows) {
#pragma omp atomic write
        status = ORACLE_BAD_ARG;
        continue;
      }
      int st = one_row(&pb, r, h, buf, out + t * D, lse + t, lse_with_sink + t);
      if (st != ORACLE_OK) {
#pragma omp atomic write
        status = st;
      }
    }
    free(buf);
  }
  return status;
}

/*
 * oracle_merge_states: combine S partial attention states of one (row, head)
 * that cover disjoint key sets, each given as a normalised output o_s[D] and
 * its base-2 log-sum-exp lse_s (Note / LSE convention: the base-2 LSE is what
 * the cascade-merge kernels consume).  Weight of state s is 2^lse_s; the
 * optional sink adds e^sink to the denominator only (Parameters / sinks).
 *   out = sum_s 2^lse_s o_s / (sum_s 2^lse_s + e^sink),  lse = log2 sum_s 2^lse_s
 * Every quantity is shifted by the largest exponent before exponentiation.
 */
void oracle_merge_states(const double* o, const double* lse_s, int64_t S, int64_t D,
                         const double* sink, double* out, double* lse) {
  double M = -INFINITY;
  for (int64_t s = 0; s < S; ++s)
    if (lse_s[s] > M) M = lse_s[s];
  const double sink2 = sink ? *sink / log(2.0) : -INFINITY;   /* e^x = 2^(x/ln2) */
  if (M == -INFINITY) {
    for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
    *lse = -INFINITY;
    return;
  }
  const double top = sink2 > M ? sink2 : M;
  double W = 0.0;
  for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
  for (int64_t s = 0; s < S; ++s) {
    double w = exp2(lse_s[s] - top);
    W += w;
    for (int64_t d = 0; d < D; ++d) out[d] += w * o[s * D + d];
  }
  const double Z = W + (sink ? exp2(sink2 - top) : 0.0);
  for (int64_t d = 0; d < D; ++d) out[d] /= Z;
  *lse = top + log2(W);
}

/*
 * oracle_prefill: context attention of flashinfer.attention.prims_ts.batch_prefill
 * (summary and Parameters).  One output row per (query row r, query head h).
 *   - summary / Parameters q, k, v, qo_indptr, kv_indptr: fixed tensors are
 *     [B, S, H, D] (row r = b * Sq + i, key row b * Sk + j); with both
 *     cumulative offset tensors the rows are packed: request b owns query rows
 *     qo[b] .. qo[b + 1] - 1 and key/value rows kvo[b] .. kvo[b + 1] - 1.
 *     The key/value head of query head h is h / (Hq / Hkv).
 *   - summary: causal masking is bottom-right aligned: query token i of a
 *     request with Sq queries and Sk keys sits at diagonal p_i = Sk - Sq + i
 *     and sees keys j <= p_i.  mask_type dense: every key j < Sk.
 *   - summary / Parameters window_left: -1 disables the left window; otherwise
 *     keys before p_i - window_left are dropped (at most window_left + 1 keys
 *     per causal row, also when Sq < Sk).
 *   - Parameters variable_window_token_starts / _ends: with mask_type
 *     variable_window, query token i of request b sees exactly the keys
 *     starts[b, i] .. ends[b, i] (inclusive; int32 [B, Sq], fixed shapes only).
 *   - Parameters sm_scale (softmax scale) and output_scale (a factor on the
 *     output).
 * The softmax is the plain two-pass form in double precision.  A row with no
 * visible key gives out = 0.  mask: 0 causal, 1 dense, 2 variable window.
 */
typedef struct {
  const uint16_t* q;  int64_t q_sr, q_sh;
  const uint16_t* k;  int64_t k_sr, k_sh;
  const uint16_t* v;  int64_t v_sr, v_sh;
  int dtype;
  int64_t B, Hq, Hkv, D, Sq, Sk;             /* Sq, Sk: fixed lengths */
  const int32_t* qo;  const int32_t* kvo;    /* packed offsets or NULL */
  int mask;
  int64_t wl;
  const int32_t* starts;  const int32_t* ends;   /* [B, Sq] for mask 2 */
  double scale, out_scale;
} prefill_t;

static void prefill_row(const prefill_t* pb, int64_t r, int64_t h, double* buf, double* out) {
  const int64_t D = pb->D;
  int64_t b, i, sq, sk, q0, k0;
  if (pb->qo) {
    b = 0;
    while (b + 1 < pb->B && pb->qo[b + 1] <= r) ++b;
    q0 = pb->qo[b];
    k0 = pb->kvo[b];
    sq = pb->qo[b + 1] - q0;
    sk = pb->kvo[b + 1] - k0;
  } else {
    b = r / pb->Sq;
    q0 = b * pb->Sq;
    k0 = b * pb->Sk;
    sq = pb->Sq;
    sk = pb->Sk;
  }
  i = r - q0;
  const int64_t kvh = h / (pb->Hq / pb->Hkv);
  const int64_t diag = sk - sq + i;
  int64_t lo, hi;
  if (pb->mask == 2) {
    lo = pb->starts[b * pb->Sq + i];
    hi = pb->ends[b * pb->Sq + i];
  } else {
    hi = pb->mask == 0 ? diag : sk - 1;
    lo = pb->wl < 0 ? 0 : diag - pb->wl;
  }
  if (lo < 0) lo = 0;
  if (hi > sk - 1) hi = sk - 1;
  double* qd = buf;
  double* s = buf + D;
  const uint16_t* qrow = pb->q + r * pb->q_sr + h * pb->q_sh;
  for (int64_t d = 0; d < D; ++d) qd[d] = decode(qrow[d], pb->dtype);
  double m = -INFINITY;
  int64_t cnt = 0;
  for (int64_t j = lo; j <= hi; ++j) {
    const uint16_t* krow = pb->k + (k0 + j) * pb->k_sr + kvh * pb->k_sh;
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += qd[d] * decode(krow[d], pb->dtype);
    s[cnt] = pb->scale * dot;
    if (s[cnt] > m) m = s[cnt];
    ++cnt;
  }
  for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
  if (cnt == 0) return;
  double S = 0.0;
  cnt = 0;
  for (int64_t j = lo; j <= hi; ++j) {
    const uint16_t* vrow = pb->v + (k0 + j) * pb->v_sr + kvh * pb->v_sh;
    const double w = exp(s[cnt++] - m);
    S += w;
    for (int64_t d = 0; d < D; ++d) out[d] += w * decode(vrow[d], pb->dtype);
  }
  for (int64_t d = 0; d < D; ++d) out[d] = pb->out_scale * (out[d] / S);
}

/*
 * Rows are (total query rows) x Hq; sel: NULL for all in row-major order
 * r * Hq + h, else nsel such indices.  out: [count, D].  Returns ORACLE_OK or
 * ORACLE_BAD_ARG.
 */
int oracle_prefill(const uint16_t* q, int64_t q_sr, int64_t q_sh,
                   const uint16_t* k, int64_t k_sr, int64_t k_sh,
                   const uint16_t* v, int64_t v_sr, int64_t v_sh,
                   int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                   int64_t Sq, int64_t Sk, const int32_t* qo, const int32_t* kvo,
                   int mask, int64_t window_left, const int32_t* starts, const int32_t* ends,
                   double scale, double out_scale, const int64_t* sel, int64_t nsel,
                   double* out, int nthreads) {
  if (!q || !k || !v || !out || B < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv) return ORACLE_BAD_ARG;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_F16) return ORACLE_BAD_ARG;
  if ((qo == NULL) != (kvo == NULL) || mask < 0 || mask > 2 || window_left < -1) return ORACLE_BAD_ARG;
  if (mask == 2 && (qo || !starts || !ends)) return ORACLE_BAD_ARG;
  int64_t rows, kmax;
  if (qo) {
    if (qo[0] != 0 || kvo[0] != 0) return ORACLE_BAD_ARG;
    kmax = 0;
    for (int64_t b = 0; b < B; ++b) {
      if (qo[b + 1] < qo[b] || kvo[b + 1] < kvo[b]) return ORACLE_BAD_ARG;
      if (kvo[b + 1] - kvo[b] > kmax) kmax = kvo[b + 1] - kvo[b];
    }
    rows = qo[B];
  } else {
    if (Sq < 1 || Sk < 1) return ORACLE_BAD_ARG;
    rows = B * Sq;
    kmax = Sk;
  }
  prefill_t pb = {q, q_sr, q_sh, k, k_sr, k_sh, v, v_sr, v_sh, dtype, B, Hq, Hkv, D, Sq, Sk,
                  qo, kvo, mask, window_left, starts, ends, scale, out_scale};
  const int64_t count = sel ? nsel : rows * Hq;
  int status = ORACLE_OK;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* buf = (double*)malloc(sizeof(double) * (size_t)(D + kmax + 1));
    if (!buf) {
#pragma omp atomic write
      status = ORACLE_NO_MEMORY;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t t = 0; t < count; ++t) {
      if (!buf) continue;
      const int64_t idx = sel ? sel[t] : t;
      const int64_t r = idx / Hq, h = idx % Hq;
      if (r < 0 || r >= rows) {
#pragma omp atomic write
        status = ORACLE_BAD_ARG;
        continue;
      }
      prefill_row(&pb, r, h, buf, out + t * D);
    }
    free(buf);
  }
  return status;
}
