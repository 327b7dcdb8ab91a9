/*
 * pkvd.h -- C ABI of the batched paged-KV decode attention library for
 * AMD Instinct MI355X (gfx950).  Library: paged_kv_decode_12_amd/libpkvd.so
 *
 * The operation is the one documented by
 *   flashinfer.cudnn.cudnn_batch_decode_with_kv_cache (Parameters, Returns, Note)
 * and, for the page-table layout, packed query rows, the mask type and the
 * output scale and type, by
 *   flashinfer.attention.prims_ts.batch_decode_with_paged_kv_cache (summary,
 *   Parameters).
 *
 * For every request b, query token i < Lq_b and query head h:
 *   row r = row0_b + i  (row0_b = b * q_len_per_req, or qo_indptr[b] for
 *   packed rows), kv head = h / (Hq / Hkv), n = seq_lens_kv[b],
 *   diagonal p = n - Lq_b + i, visible keys j with
 *     max(0, p - window_left) <= j <= p        (causal mask)
 *     max(0, p - window_left) <= j <= n - 1    (dense mask)
 *   (no lower bound when window_left == -1);
 *   key j is slot j % page_size of page block_tables[b, j / page_size];
 *   s_j = scale * q[r, h, :] . k_j
 *   out[r, h, :] = out_scale * sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{sinks[h]})
 *   lse[r, h]    = log2 sum_j e^{s_j}          (keys only; see below)
 *
 * Readings taken where the documentation is silent (one line each):
 *   - the exported LSE of a masked row sums over that row's visible keys and
 *     never includes the sink logit;
 *   - sinks[h] is an unscaled logit indexed by the query head;
 *   - block_tables, seq_lens_kv and qo_indptr are int32;
 *   - pkvd_decode (fixed rows, q_len_per_req > 1) always uses the
 *     bottom-right causal mask;
 *   - with the dense mask a window still starts window_left keys before the
 *     row's diagonal position p;
 *   - a row with no visible key (only possible when n < Lq_b under the causal
 *     mask, which the contract forbids) yields out = 0 and lse = -inf.
 *
 * Threading: calls may come from any host thread.  Calls that share a
 * workspace (the library's per-device one, a buffer bound with
 * pkvd_set_workspace, or one passed per call) must be ordered by the caller
 * (same stream, or events between streams); calls with different
 * workspaces may overlap.
 */
#ifndef PKVD_H_
#define PKVD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of a tensor descriptor. */
typedef enum {
  PKVD_BF16 = 0, /* bfloat16 */
  PKVD_F16 = 1,  /* IEEE binary16 */
  PKVD_F32 = 2,  /* IEEE binary32 */
  PKVD_I32 = 3   /* int32 */
} pkvd_dtype;

/* Status codes.  Every entry point returns one; 0 is success. */
typedef enum {
  PKVD_OK = 0,
  PKVD_ERR_INVALID_ARG = 1, /* shape, dtype, stride, alignment or value mismatch */
  PKVD_ERR_UNSUPPORTED = 2, /* valid by the documentation, not built here
                               (head_dim other than 64/128, page_size > 256) */
  PKVD_ERR_WORKSPACE = 3,   /* workspace too small, or could not be allocated
                               (including: it would have to grow during a
                               graph capture) */
  PKVD_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} pkvd_status;

/* Mask of the query rows of a request (batch_decode_with_paged_kv_cache,
 * Parameters / mask_type). */
typedef enum {
  PKVD_MASK_CAUSAL = 0,          /* row i sees keys up to its diagonal n - Lq_b + i */
  PKVD_MASK_DENSE = 1,           /* every row sees keys up to n - 1 */
  PKVD_MASK_VARIABLE_WINDOW = 2  /* pkvd_prefill only: per-query [start, end] bounds */
} pkvd_mask;

/*
 * A strided view of device memory.  The caller owns `data`; the library never
 * frees it.  shape/strides beyond ndim are ignored.  Strides are in elements.
 */
typedef struct {
  void* data;
  int32_t dtype; /* pkvd_dtype */
  int32_t ndim;
  int64_t shape[4];
  int64_t strides[4];
} pkvd_tensor;

/*
 * pkvd_decode -- enqueue one batched paged-KV decode on `stream`.
 * (cudnn_batch_decode_with_kv_cache: Parameters, Returns, Note)
 *
 *   q            bf16 or fp16, shape (B * q_len_per_req, Hq, D).  The rows of
 *                one request are consecutive.  strides[2] must be 1; the row
 *                and head strides are free (a head slice of a packed QKV
 *                projection works) but every row must start 16-byte aligned.
 *                (Parameters / q; Note)
 *   k_cache,     dtype of q, shape (num_pages, Hkv, page_size, D).  Each
 *   v_cache      (page, kv head) tile [page_size, D] must be contiguous
 *                (strides[3] == 1, strides[2] == D); page and head strides are
 *                free, so K and V may be views into one combined tensor.
 *                16-byte aligned.  (Parameters / k_cache, v_cache; the HND
 *                layout of batch_decode_with_paged_kv_cache)
 *   block_tables int32, shape (B, C); strides[1] == 1, strides[0] >= C (rows
 *                may be padded apart).  (Parameters / block_tables)
 *   seq_lens_kv  int32, shape (B,), contiguous, device resident.  Entries must
 *                satisfy q_len_per_req <= n <= C * page_size and every page
 *                id a request reaches must be < num_pages; the kernels do not
 *                report violations but clamp every index, so out-of-contract
 *                data never causes an out-of-bounds access.
 *                (Parameters / actual_seq_lens_kv, q_len_per_req)
 *   scale        softmax scale folded into q . k (Parameters / scale).
 *   q_len_per_req >= 1; > 1 selects the bottom-right causal mask.
 *   window_left  -1 (no window) or >= 0.  (Parameters / window_left)
 *   sinks        NULL, or fp32 (Hq,) contiguous.  (Parameters / sinks)
 *   out          caller-owned, dtype of q, contiguous (B * q_len_per_req, Hq, D).
 *   lse          NULL, or caller-owned fp32 contiguous (B * q_len_per_req, Hq):
 *                base-2 log-sum-exp of each row's visible scaled scores
 *                (Note / LSE convention).
 *   stream       hipStream_t (passed as void*); NULL = the default stream.
 *
 * Supported: D in {64, 128}; 1 <= page_size <= 256; Hq % Hkv == 0;
 * B <= 8192 requests; with sinks, Hq <= 4096 (the kernel keeps the sink
 * logits in on-chip memory).  Others return PKVD_ERR_UNSUPPORTED.
 * Work is only enqueued; the call never synchronises and never reads device
 * data on the host: one persistent kernel splits the total work evenly over
 * its waves from seq_lens_kv on the device.  The workspace (partial states
 * of units cut between waves) is the buffer bound with pkvd_set_workspace,
 * else a library-owned one per device, allocated on the first call and grown
 * when a call needs more (never while the stream is capturing a graph:
 * that call fails with PKVD_ERR_WORKSPACE; see pkvd_reserve_workspace).
 * Errors: PKVD_ERR_INVALID_ARG / PKVD_ERR_UNSUPPORTED are detected before any
 * HIP call; the message is available from pkvd_last_error().
 */
int pkvd_decode(const pkvd_tensor* q, const pkvd_tensor* k_cache, const pkvd_tensor* v_cache,
                const pkvd_tensor* block_tables, const pkvd_tensor* seq_lens_kv, float scale,
                int32_t q_len_per_req, int32_t window_left, const pkvd_tensor* sinks,
                pkvd_tensor* out, pkvd_tensor* lse, void* stream);

/*
 * pkvd_decode_static -- pkvd_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments, layout, semantics and errors as
 * pkvd_decode, but the workspace is a static device array of the library
 * (32 MiB on each GPU the library runs on, held from load until the process
 * ends) instead of a buffer the library or the caller allocates.  The call
 * allocates and frees nothing (no hipMalloc, no library allocation) and
 * never synchronises.  A call whose plan needs more than 32 MiB of workspace
 * fails with PKVD_ERR_WORKSPACE before any HIP call.  Every call on one GPU
 * shares that GPU's array: calls that may overlap on one GPU (different
 * streams without events between them) race and must not be made; calls on
 * one stream are ordered.  pkvd_decode's own workspace is separate.
 */
int pkvd_decode_static(const pkvd_tensor* q, const pkvd_tensor* k_cache,
                       const pkvd_tensor* v_cache, const pkvd_tensor* block_tables,
                       const pkvd_tensor* seq_lens_kv, float scale, int32_t q_len_per_req,
                       int32_t window_left, const pkvd_tensor* sinks, pkvd_tensor* out,
                       pkvd_tensor* lse, void* stream);

/*
 * Arguments of pkvd_decode_ex: the pkvd_decode call plus packed query rows,
 * the mask type, the output scale and type, and a per-call workspace
 * (batch_decode_with_paged_kv_cache: summary; Parameters / q, paged_kv_cache,
 * qo_indptr, max_seq_len_q, seq_len_q, mask_type, bmm1_scale, bmm2_scale,
 * out, out_dtype; cudnn_batch_decode_with_kv_cache: Parameters /
 * workspace_buffer, is_cuda_graph_compatible).  Zero-fill the struct, then
 * set the fields.
 *
 *   q            bf16 or fp16: (rows, Hq, D) as for pkvd_decode, or
 *                token-major (B, SQ, Hq, D) for fixed SQ = q_len rows per
 *                request (its SQ rows at one stride), or packed
 *                (total_q, Hq, D) when qo_indptr is given.
 *   k_cache,     as for pkvd_decode (a combined K/V tensor is two views).
 *   v_cache,
 *   block_tables,
 *   seq_lens_kv
 *   qo_indptr    NULL for fixed rows, or int32 (B + 1,) contiguous device
 *                tensor of cumulative row offsets: request b owns rows
 *                qo_indptr[b] .. qo_indptr[b + 1] - 1 of q and out
 *                (qo_indptr[0] = 0, nondecreasing, qo_indptr[B] = total_q,
 *                at most q_len rows per request; device data, not checked:
 *                the kernels clamp offsets into [0, total_q] and counts to
 *                q_len).  A request with no rows is skipped.
 *   q_len        fixed: query rows per request (q_len_per_req / seq_len_q);
 *                packed: the largest number of rows of any request
 *                (max_seq_len_q), which sizes the plan.  >= 1.
 *   mask         pkvd_mask.  With one row per request both masks agree.
 *   window_left  -1 or >= 0, measured from each row's diagonal position.
 *   scale        bmm1 scale folded into q . k; finite.
 *   out_scale    bmm2 scale: a factor on the output (not on the LSE); finite.
 *   sinks        NULL, or fp32 (Hq,) contiguous.
 *   out          caller-owned, q's shape, contiguous, 16-byte aligned;
 *                bf16, fp16 or fp32 (out_dtype), rounded to nearest even.
 *   lse          NULL, or fp32 contiguous (rows, Hq) (or (B, SQ, Hq) for a
 *                4-D q).
 *   workspace    NULL: as for pkvd_decode.  Else a caller-owned device buffer
 *                of workspace_bytes (>= what pkvd_decode_ex_plan reports,
 *                else PKVD_ERR_WORKSPACE), 256-byte aligned, zero-filled
 *                before its first use; every call leaves it ready for the
 *                next.  Calls may overlap when their workspaces differ.
 * Supported sizes as for pkvd_decode; packed rows also need (Hq / Hkv) *
 * q_len <= 65535.  Returns a status as for pkvd_decode.
 */
typedef struct {
  const pkvd_tensor* q;
  const pkvd_tensor* k_cache;
  const pkvd_tensor* v_cache;
  const pkvd_tensor* block_tables;
  const pkvd_tensor* seq_lens_kv;
  const pkvd_tensor* qo_indptr;
  int32_t q_len;
  int32_t mask;
  int32_t window_left;
  float scale;
  float out_scale;
  const pkvd_tensor* sinks;
  pkvd_tensor* out;
  pkvd_tensor* lse;
  void* workspace;
  size_t workspace_bytes;
} pkvd_decode_args;

int pkvd_decode_ex(const pkvd_decode_args* args, void* stream);

/*
 * pkvd_decode_ex_plan -- the plan pkvd_decode_ex would use for these
 * arguments (only shapes are read; no data pointer is dereferenced):
 * plan[0] = path (0 = VALU dot products, 1 = MFMA), plan[1] = rows per tile,
 * plan[2] = row tiles per (request, kv head), plan[3] = waves of the
 * persistent grid, plan[4] = minimum 16-key blocks per participating wave,
 * plan[5] = workgroups of the decode kernel, plan[6] = 1 when cut units are
 * merged by a second kernel, plan[7] = 1 when every unit is streamed whole
 * by one wave.  *workspace_bytes = the workspace the call needs.  Either
 * output may be NULL.  Planning for a caller workspace happens here, before
 * any graph capture (cudnn_batch_decode_with_kv_cache, Parameters /
 * is_cuda_graph_compatible; batch_decode_with_paged_kv_cache, summary).
 */
int pkvd_decode_ex_plan(const pkvd_decode_args* args, int64_t plan[8], size_t* workspace_bytes);

/*
 * pkvd_schedule_stats -- a host replay of the persistent schedule that
 * pkvd_decode_ex would run for these arguments (shapes only; no data pointer
 * is dereferenced) and the given host copies of seq_lens_kv (B entries) and,
 * for packed rows, qo_indptr (B + 1 entries).  It runs the kernels' own
 * schedule arithmetic on the host: stats[0] = 16-key blocks of the call,
 * stats[1] = waves taking part, stats[2] = units (request, kv head, row tile)
 * with blocks, stats[3] = units cut between waves (each leaves one partial
 * state per piece, merged with the base-2 LSE rule of the Note / LSE
 * convention), stats[4] = pieces of the cut units, stats[5] = most pieces of
 * one unit, stats[6] = inconsistencies found (blocks not covered exactly
 * once, or a merge that would read the wrong partial states; 0 when the
 * schedule is sound), stats[7] = blocks of the sliced (virtual) space.
 * A planning diagnostic: it predicts the partial-state traffic of a call.
 */
int pkvd_schedule_stats(const pkvd_decode_args* args, const int32_t* seq_lens,
                        const int32_t* qo_indptr, int64_t stats[8]);

/*
 * pkvd_decode_workspace_bytes -- bytes of workspace the plan of a
 * pkvd_decode call with these shapes needs on the current device.  Same
 * arguments as pkvd_decode minus the data; only shapes are read.  Returns a
 * status; the size is written to *bytes.  (cudnn_batch_decode_with_kv_cache,
 * Parameters / workspace_buffer: the workspace scales with the batch.)
 */
int pkvd_decode_workspace_bytes(const pkvd_tensor* q, const pkvd_tensor* k_cache,
                                const pkvd_tensor* block_tables, int32_t q_len_per_req,
                                int32_t window_left, size_t* bytes);

/*
 * pkvd_reserve_workspace -- make sure the current device's library-owned
 * workspace holds at least `bytes` (allocates with hipMalloc and zero-fills
 * it, synchronously, when it must).  Call it before capturing pkvd_decode
 * into a HIP graph: a call inside a capture never allocates and fails with
 * PKVD_ERR_WORKSPACE when the workspace is too small.  A buffer the library
 * replaces is kept until the process ends (a captured graph may use it).
 * (batch_decode_with_paged_kv_cache, summary: plan before capture.)
 */
int pkvd_reserve_workspace(size_t bytes);

/*
 * pkvd_workspace_capacity -- bytes the workspace of the next pkvd_decode on
 * the current device holds: the bound caller-owned buffer's size when one is
 * bound, else the library-owned buffer's (0 before any call or
 * reservation).  A call whose pkvd_decode_workspace_bytes is at most this
 * needs no allocation, so it may be captured into a HIP graph
 * (batch_decode_with_paged_kv_cache, summary: plan before capture).
 * Returns a status; the size is written to *bytes.
 */
int pkvd_workspace_capacity(size_t* bytes);

/*
 * pkvd_set_workspace -- bind a caller-owned device buffer as the workspace of
 * every later pkvd_decode (and pkvd_decode_ex without its own workspace) on
 * the current device (cudnn_batch_decode_with_kv_cache, Parameters /
 * workspace_buffer).  dev_ptr: 256-byte aligned device memory of `bytes`
 * (>= 4096) that stays valid while bound; the call zero-fills it
 * synchronously (not inside a graph capture).  NULL unbinds it (the library's
 * own workspace is used again).  While a buffer is bound the library never
 * allocates; a call that needs more than `bytes` fails with
 * PKVD_ERR_WORKSPACE.  The caller keeps ownership.
 */
int pkvd_set_workspace(void* dev_ptr, size_t bytes);

/*
 * pkvd_decode_plan -- the first six entries of pkvd_decode_ex_plan's plan for
 * a pkvd_decode call with these shapes.  With no device present the plan
 * assumes an MI355X (256 CUs, one workgroup per CU).
 */
int pkvd_decode_plan(const pkvd_tensor* q, const pkvd_tensor* k_cache,
                     const pkvd_tensor* block_tables, int32_t q_len_per_req,
                     int32_t window_left, int64_t out[6]);

/*
 * pkvd_reload_tuning -- re-read the PKVD_* environment overrides of the
 * planner (measurement and test knobs: PKVD_FORCE_PATH, PKVD_WAVES,
 * PKVD_MIN_WAVE_BLOCKS, PKVD_SEG_COST, PKVD_GROUPS, PKVD_MERGE_KERNEL,
 * PKVD_UNIT_MODE, PKVD_SLOT_W, PKVD_LOG).  They are read once, at the first
 * call, otherwise.
 */
void pkvd_reload_tuning(void);

/*
 * pkvd_prefill -- context attention: every query row of a request attends to
 * that request's own keys, the operation of
 * flashinfer.attention.prims_ts.batch_prefill (summary, Parameters).  For
 * request b with Sq_b queries and Sk_b keys, query token i, query head h:
 *   diagonal p = Sk_b - Sq_b + i (bottom-right aligned), visible keys j with
 *     max(0, p - window_left) <= j <= p        (PKVD_MASK_CAUSAL)
 *     max(0, p - window_left) <= j <= Sk_b - 1 (PKVD_MASK_DENSE)
 *     starts[b, i] <= j <= ends[b, i]          (PKVD_MASK_VARIABLE_WINDOW)
 *   (no lower bound from the window when window_left == -1);
 *   out[row, h, :] = output_scale * softmax_j(sm_scale * q . k_j) . v_j with
 *   kv head h / (Hq / Hkv); a row with no visible key gives 0.
 *
 *   q        bf16 or fp16: fixed (B, Sq, Hq, D) or packed (total_q, Hq, D);
 *            head_dim innermost and dense, rows 16-byte aligned, the other
 *            strides free (a fixed tensor must step its S rows at one stride).
 *   k, v     q's dtype: fixed (B, Sk, Hkv, D) or packed (total_kv, Hkv, D),
 *            the same layout rules; Hq % Hkv == 0.
 *   qo_indptr, kv_indptr  NULL (fixed) or both int32 (B + 1,) contiguous
 *            device tensors of cumulative offsets: request b owns query rows
 *            qo_indptr[b] .. qo_indptr[b + 1] - 1 and key/value rows
 *            kv_indptr[b] .. kv_indptr[b + 1] - 1 (device data, not checked:
 *            offsets are clamped into the tensors, query counts to
 *            max_seq_len_q).
 *   max_seq_len_q  packed: the largest query count of any request (sizes the
 *            grid); fixed: ignored.
 *   mask     PKVD_MASK_CAUSAL, PKVD_MASK_DENSE or PKVD_MASK_VARIABLE_WINDOW
 *            (fixed shapes only, window_left must be -1).
 *   window_left  -1 or >= 0.
 *   window_starts, window_ends  variable window: int32 (B, Sq) contiguous
 *            device tensors, 0 <= starts <= ends < Sk (clamped on the device).
 *   sm_scale, output_scale  finite.
 *   out      caller-owned, q's shape, contiguous, 16-byte aligned; bf16,
 *            fp16 or fp32 (out_dtype); shares no byte with q, k or v.
 * Supported: D in {128, 256}.  Work is only enqueued on `stream` (two
 * kernels: the second recomputes, with a rescaling pass, the row groups whose
 * probabilities overflowed their format in the first, which marks them in
 * `out`; `out` is complete once both have run); nothing is allocated and
 * nothing is read back.  Errors as for pkvd_decode.
 */
typedef struct {
  const pkvd_tensor* q;
  const pkvd_tensor* k;
  const pkvd_tensor* v;
  const pkvd_tensor* qo_indptr;
  const pkvd_tensor* kv_indptr;
  int32_t max_seq_len_q;
  int32_t mask;
  int32_t window_left;
  const pkvd_tensor* window_starts;
  const pkvd_tensor* window_ends;
  float sm_scale;
  float output_scale;
  pkvd_tensor* out;
} pkvd_prefill_args;

int pkvd_prefill(const pkvd_prefill_args* args, void* stream);

/* Message of the last error on the calling thread ("" if none). */
const char* pkvd_last_error(void);

/* Short text for a status code. */
const char* pkvd_status_string(int status);

/* Library version, e.g. "0.2.0". */
const char* pkvd_version(void);

/*
 * pkvd_merge_states -- the cascade merge: combine S partial attention states
 * of the same (row, head), each computed over its own disjoint set of keys,
 * into the state over their union.  A state is the pair this library's
 * decode writes: a normalised output and its base-2 log-sum-exp, the form the
 * cascade-merge kernels consume (cudnn_batch_decode_with_kv_cache, Note /
 * LSE convention).  For every row r and head h:
 *   v_out[r, h, :] = sum_s 2^{s[s, r, h]} v[s, r, h, :]
 *                    / (sum_s 2^{s[s, r, h]} + e^{sinks[h]})
 *   s_out[r, h]    = log2 sum_s 2^{s[s, r, h]}
 * with every exponent taken relative to the largest.  A state with
 * s = -inf is empty and weighs 0 (its v is never read into the sum); rows
 * whose states are all empty give v_out = 0, s_out = -inf.
 *
 *   v      (S, R, H, D) bf16, fp16 or fp32, contiguous, device memory
 *   s      (S, R, H) fp32 contiguous: base-2 LSE of each state
 *   sinks  NULL, or fp32 (H,) contiguous: a logit added to the denominator
 *          only (Parameters / sinks)
 *   v_out  (R, H, D), v's dtype, contiguous; caller-owned
 *   s_out  NULL, or fp32 (R, H) contiguous; caller-owned
 *   stream hipStream_t (passed as void*); NULL = the default stream
 * S >= 1; D >= 1.  The library allocates nothing for this call and never
 * synchronises.  Errors: PKVD_ERR_INVALID_ARG before any HIP call;
 * PKVD_ERR_HIP when the launch fails (message from pkvd_last_error()).
 */
int pkvd_merge_states(const pkvd_tensor* v, const pkvd_tensor* s, const pkvd_tensor* sinks,
                      pkvd_tensor* v_out, pkvd_tensor* s_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKVD_H_ */
