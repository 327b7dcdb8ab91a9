/*
 * pkvd.h -- C ABI of the batched paged-KV decode attention library for
 * AMD Instinct MI355X (gfx950).  Library: paged_kv_decode_12_amd/libpkvd.so
 *
 * The operation is the one documented by
 *   flashinfer.cudnn.cudnn_batch_decode_with_kv_cache (Parameters, Returns, Note)
 * and, for the page-table layout, by
 *   flashinfer.attention.prims_ts.batch_decode_with_paged_kv_cache (Parameters).
 *
 * For every request b, query token i < q_len_per_req and query head h:
 *   row r = b * q_len_per_req + i, kv head = h / (Hq / Hkv), n = seq_lens_kv[b],
 *   diagonal p = n - q_len_per_req + i, visible keys j with
 *     max(0, p - window_left) <= j <= p      (window_left >= 0)
 *     0 <= j <= p                             (window_left == -1)
 *   key j is slot j % page_size of page block_tables[b, j / page_size];
 *   s_j = scale * q[r, h, :] . k_j
 *   out[r, h, :] = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{sinks[h]})
 *   lse[r, h]    = log2 sum_j e^{s_j}          (keys only; see below)
 *
 * Readings taken where the documentation is silent (one line each):
 *   - the exported LSE of a masked row sums over that row's visible keys and
 *     never includes the sink logit;
 *   - sinks[h] is an unscaled logit indexed by the query head;
 *   - block_tables and seq_lens_kv are int32;
 *   - q_len_per_req > 1 always means the bottom-right causal mask;
 *   - a row with no visible key (only possible when n < q_len_per_req, which
 *     the contract forbids) yields out = 0 and lse = -inf.
 *
 * Threading: calls may come from any host thread.  Calls that can overlap on
 * one device share that device's workspace and must be ordered by the caller
 * (same stream, or events between streams).
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
  PKVD_ERR_WORKSPACE = 3,   /* workspace could not be allocated */
  PKVD_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} pkvd_status;

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
 *
 *   q            bf16 or fp16, shape (B * q_len_per_req, Hq, D).  The rows of
 *                one request are consecutive.  strides[2] must be 1; the row
 *                and head strides are free (a head slice of a packed QKV
 *                projection works) but every row must start 16-byte aligned.
 *                (cudnn_batch_decode_with_kv_cache: Parameters / q; Note)
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
 * its waves from seq_lens_kv on the device.  A workspace for the partial
 * states of units cut between waves is allocated on the first call (and
 * grown later if needed); see pkvd_reserve_workspace.
 * Errors: PKVD_ERR_INVALID_ARG / PKVD_ERR_UNSUPPORTED are detected before any
 * HIP call; the message is available from pkvd_last_error().
 */
int pkvd_decode(const pkvd_tensor* q, const pkvd_tensor* k_cache, const pkvd_tensor* v_cache,
                const pkvd_tensor* block_tables, const pkvd_tensor* seq_lens_kv, float scale,
                int32_t q_len_per_req, int32_t window_left, const pkvd_tensor* sinks,
                pkvd_tensor* out, pkvd_tensor* lse, void* stream);

/*
 * pkvd_decode_workspace_bytes -- bytes of workspace (partial states, two per
 * wave of the persistent grid) the plan for these shapes needs on the current
 * device.  Same
 * arguments as pkvd_decode minus the data; only shapes are read.  Returns
 * a status; the size is written to *bytes.
 */
int pkvd_decode_workspace_bytes(const pkvd_tensor* q, const pkvd_tensor* k_cache,
                                const pkvd_tensor* block_tables, int32_t q_len_per_req,
                                int32_t window_left, size_t* bytes);

/*
 * pkvd_reserve_workspace -- make sure the current device's library-owned
 * workspace holds at least `bytes` (allocates with hipMalloc when it must).
 * Call it before capturing pkvd_decode into a HIP graph so the call inside
 * the capture does not allocate.
 */
int pkvd_reserve_workspace(size_t bytes);

/*
 * pkvd_decode_plan -- the launch plan pkvd_decode would use for these shapes:
 * out[0] = path (0 = VALU dot products, 1 = MFMA), out[1] = rows per tile,
 * out[2] = row tiles per (request, kv head), out[3] = waves of the persistent
 * grid, out[4] = minimum 16-key blocks per participating wave,
 * out[5] = workgroups of the decode kernel.  With no device present the plan
 * assumes an MI355X (256 CUs, two workgroups per CU).
 */
int pkvd_decode_plan(const pkvd_tensor* q, const pkvd_tensor* k_cache,
                     const pkvd_tensor* block_tables, int32_t q_len_per_req,
                     int32_t window_left, int64_t out[6]);

/* Message of the last error on the calling thread ("" if none). */
const char* pkvd_last_error(void);

/* Short text for a status code. */
const char* pkvd_status_string(int status);

/* Library version, e.g. "0.1.0". */
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
