/*
 * ckl.h -- C ABI of the fused chunked KL distillation loss for MI355X (gfx950).
 *
 * The loss compares a student's full-vocabulary distribution with an offline
 * cache of the teacher's top-K logits per position and returns the loss with
 * its gradients, without ever holding the student's vocabulary x sequence
 * logit grid: the sequence is processed in row chunks and each chunk's logits
 * are computed, turned into gradient and discarded before the next chunk
 * ("A New Trick Slashes the Cost of Shrinking Giant AI Models", sections
 * "What did the researchers change?" and "Does this matter for longer
 * documents?"; "Making Knowledge Distillation Cheap Enough to Run at Scale"
 * (aiphreaks.com), bullet "Fused Chunked KL Loss").
 *
 * Definition (the readings where the pages are silent are stated here):
 *   z_r      = H_r . W^T                        student logits of position r, length V
 *   log p_S  = z_r - logsumexp(z_r)             full-vocabulary log-softmax
 *   p_T      = softmax(T_r)                     over the K cached teacher logits only;
 *                                               the other V - K tokens get no mass
 *                                               (elseif.net page, limitations paragraph)
 *   KL_r     = sum_k p_T,k (log p_T,k - log p_S,id_k)
 *   loss     = (1 / n) sum_r mask_r KL_r,       n = number of valid positions
 *                                               (loss = 0 and all gradients 0 if n = 0)
 *   dL/dz_r  = (mask_r / n) (softmax(z_r) - scatter(p_T,r))
 *   dH       = G W,   dW = G^T H                with G the stacked dL/dz_r
 * Temperature 1.  Teacher ids within a row must be distinct and in [0, V).
 * The logit at each cached id is the very fp32 value the logits contraction
 * accumulated (copied out before any exponential), so log p_S at the ids is
 * that of the dense definition to fp32 rounding of the log-normaliser.
 *
 * Ids outside [0, V), and repeats within a row, are outside the supported
 * inputs: no kernel reads or writes at them (they are left out of the loss
 * and the gradient, so the result is not the definition's), and a device
 * flag records them.  With the environment variable CKL_DEBUG=1, each loss
 * call waits for its own kernels and then returns CKL_EINVAL if the flag is
 * set.
 *
 * Layout and ownership (every call):
 *   - all arrays are row-major and contiguous, in device memory of the device
 *     that is current on the calling thread, and `stream` belongs to it;
 *   - H, W, dH, dW must be 16-byte aligned; ids, logits, out_loss 4-byte;
 *   - the caller owns every buffer; the library keeps no pointer after the
 *     call returns.  Work is enqueued on `stream` with no host synchronisation,
 *     so inputs and outputs must stay alive until the stream has finished;
 *   - d must be a multiple of 8; 1 <= K <= min(V, 2048);
 *   - N = 0 is an empty batch: no row is read (H, ids, logits, mask, dH and
 *     the per-position arrays may be null), and a loss call writes 0 to
 *     out_loss and zeros to dW, the result for a batch with no valid
 *     position; ckl_plan gives chunk 0 and 0 bytes, ckl_topk does nothing;
 *   - the library holds one grow-only device workspace per (device, stream),
 *     sized by ckl_plan; ckl_release_workspace frees them all.
 *
 * Environment: CKL_WORKSPACE_BYTES (workspace budget, default 6 GiB);
 * CKL_DEBUG=1 (input checks reported by the call, see above); CKL_TRACE=1
 * (roctx ranges around every loss call and every chunk, for rocprofv3
 * --marker-trace; skipped if no roctx library can be opened).
 *
 * Errors: arguments that are invalid or not supported are reported before
 * anything is enqueued, and the outputs are untouched.  A HIP failure returns
 * CKL_EHIP or CKL_ENOMEM and leaves the outputs undefined; since every call
 * overwrites dW (it does not accumulate into it), the call can be repeated.
 * No C++ exception crosses this interface.
 */
#ifndef CKL_H_
#define CKL_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CKL_OK = 0,
  CKL_EINVAL = -1,       /* null or misaligned pointer, N < 0, d, V or K < 1, K > V, chunk < 0 */
  CKL_ENOMEM = -2,       /* device workspace allocation failed */
  CKL_EBUDGET = -3,      /* no chunk size fits the workspace budget (or the given chunk does not) */
  CKL_EHIP = -4,         /* a HIP runtime call failed */
  CKL_EUNSUPPORTED = -5  /* d % 8 != 0, K > 2048, V > 2^26, a chunk above 2^20 rows, or a size
                            beyond 32-bit grid limits */
} ckl_status;

typedef enum { CKL_DTYPE_BF16 = 0, CKL_DTYPE_F32 = 1 } ckl_dtype;

/* Fused forward + backward of the loss above (bf16 hidden states and weight).
 *   H          bf16 [N, d]   student final hidden states
 *   W          bf16 [V, d]   LM-head weight
 *   topk_idx   int32 [N, K]  cached teacher ids, distinct per row, in [0, V)
 *   topk_logit fp32 [N, K]   cached teacher logits
 *   mask       uint8 [N]     1 = position counts, 0 = ignored; NULL = all count
 *   chunk      rows per chunk; 0 lets ckl_plan choose under the workspace budget
 *              (environment CKL_WORKSPACE_BYTES, default 6 GiB)
 *   out_loss   fp32 device scalar
 *   dH         bf16 [N, d]   gradient of the loss with respect to H (overwritten)
 *   dW         fp32 [V, d]   gradient with respect to W (overwritten)
 * Masked positions contribute nothing and cost no GEMM work: with a mask,
 * each chunk's valid rows are gathered to the front of workspace buffers
 * before its contractions, so masked rows get no logits.  Their dH rows are
 * written as +0.
 * The pages' interface statement is that a training code only swaps in this
 * loss, fed by the precomputed top-K cache (elseif.net page, adoption paragraph). */
int ckl_fwd_bwd(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logit,
                const uint8_t* mask, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk,
                float* out_loss, void* dH, float* dW, hipStream_t stream);

/* Same as ckl_fwd_bwd with H, W and dH in fp32 (fp32 matrix cores). */
int ckl_fwd_bwd_f32(const float* H, const float* W, const int32_t* topk_idx, const float* topk_logit,
                    const uint8_t* mask, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk,
                    float* out_loss, float* dH, float* dW, hipStream_t stream);

/* ckl_fwd_bwd / ckl_fwd_bwd_f32 selected by `dtype` (ckl_dtype), with two
 * optional per-position outputs (device, caller-owned, may be NULL):
 *   row_kl   fp32 [N]  KL_r of each position (0 for masked positions)
 *   row_lse  fp32 [N]  logsumexp of the student logits of each position (0 for
 *                      masked positions)
 * The loss is the sum of row_kl divided by the valid count. */
int ckl_fwd_bwd_ex(int dtype, const void* H, const void* W, const int32_t* topk_idx, const float* topk_logit,
                   const uint8_t* mask, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk,
                   float* out_loss, void* dH, float* dW, float* row_kl, float* row_lse, hipStream_t stream);

/* Largest workspace ckl_fwd_bwd_noalloc can use, in bytes (256 MiB). */
#define CKL_NOALLOC_MAX_BYTES (256ull << 20)

/* ckl_fwd_bwd_ex for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as ckl_fwd_bwd_ex, except that the
 * workspace is a fixed array of CKL_NOALLOC_MAX_BYTES in the library's own
 * device memory, which every GPU the library runs on holds until the process
 * ends; the call itself allocates and frees nothing.
 *   - The chunk planner runs with that size as its budget: a shape whose
 *     smallest workspace (or whose given chunk) does not fit returns
 *     CKL_EBUDGET before anything is enqueued.  The tiled copy of W alone
 *     takes V x d x (2 or 4) bytes, so this fits heads up to about
 *     V x d = 60 M elements in bf16 (e.g. d = 2048, V = 32,000), not the
 *     largest vocabularies.
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind; nothing in it has to start at zero (each buffer is written
 *     before it is read within a call).  Calls that overlap on one GPU (on
 *     different streams, or from several threads) race on the array and give
 *     undefined results: the caller orders them.
 *   - With the same chunk, the results are bitwise those of ckl_fwd_bwd_ex. */
int ckl_fwd_bwd_noalloc(int dtype, const void* H, const void* W, const int32_t* topk_idx,
                        const float* topk_logit, const uint8_t* mask, int64_t N, int64_t d, int64_t V, int64_t K,
                        int64_t chunk, float* out_loss, void* dH, float* dW, float* row_kl, float* row_lse,
                        hipStream_t stream);

/* The two-pass form of the same loss, for a training code whose backward runs
 * apart from its forward: the forward keeps one number per position and the
 * backward recomputes each chunk's logits from H and W instead of storing them
 * ("A New Trick Slashes the Cost of Shrinking Giant AI Models", section "What
 * did the researchers change?": chunks are computed and discarded, and what the
 * backward pass needs is recomputed; the same page's table lists a
 * forward-chunked loss beside the fused one).  Together the two calls do four
 * d x V contractions per position instead of the fused call's three.
 *
 * ckl_fwd: loss and per-position log-normaliser, no gradients.
 *   dtype      ckl_dtype of H and W
 *   H, W, topk_idx, topk_logit, mask, N, d, V, K, chunk   as for ckl_fwd_bwd
 *   out_loss   fp32 device scalar
 *   row_lse    fp32 [N] (required)   logsumexp of each position's student logits
 *                                    (0 for masked positions)
 *   row_kl     fp32 [N] or NULL      KL_r (0 for masked positions)
 * With the same inputs and chunk, loss, row_lse and row_kl are bitwise equal
 * to those of ckl_fwd_bwd_ex (and they do not depend on the chunk).  No exp
 * values are kept, so the workspace per row is a small fraction of the fused
 * call's and the planner's chunk is correspondingly longer. */
int ckl_fwd(int dtype, const void* H, const void* W, const int32_t* topk_idx, const float* topk_logit,
            const uint8_t* mask, int64_t N, int64_t d, int64_t V, int64_t K, int64_t chunk, float* out_loss,
            float* row_lse, float* row_kl, hipStream_t stream);

/* ckl_bwd: dH and dW of `grad_loss` x loss, recomputing every chunk's logits.
 *   row_lse    fp32 [N] (required)   the values ckl_fwd wrote for these inputs
 *   grad_loss  fp32 device scalar multiplying both gradients, or NULL for 1
 *   dH         [N, d] in dtype (overwritten);  dW  fp32 [V, d] (overwritten)
 * The log-normaliser is read from row_lse rather than recomputed.  With
 * grad_loss NULL and the same chunk, dH and dW are bitwise equal to those of
 * ckl_fwd_bwd. */
int ckl_bwd(int dtype, const void* H, const void* W, const int32_t* topk_idx, const float* topk_logit,
            const uint8_t* mask, const float* row_lse, const float* grad_loss, int64_t N, int64_t d, int64_t V,
            int64_t K, int64_t chunk, void* dH, float* dW, hipStream_t stream);

typedef enum { CKL_PASS_FUSED = 0, CKL_PASS_FWD = 1, CKL_PASS_BWD = 2 } ckl_pass;

/* Offline top-K cache writer: the step that produces topk_idx / topk_logit from
 * the teacher's logits, run once per training corpus ("A New Trick...",
 * section "What did the researchers change?": the teacher is run once and only
 * its top 100 predictions per position are saved; elseif.net page,
 * offline-cache paragraph).
 *   dtype     ckl_dtype of logits
 *   logits    [N, V] row-major, bf16 or fp32 (2- or 4-byte aligned); no NaN
 *   ids_out   int32 [N, K]   token ids of the K largest logits of each row
 *   vals_out  fp32 [N, K]    those logits (exact conversion of the inputs)
 * Each row's K pairs are ordered by value descending; equal values (-0 equals
 * +0) by id ascending, so the result is unique.  1 <= K <= min(V, 2048),
 * V < 2^31.  Enqueued on `stream`; no workspace.  Errors as for the other
 * calls; nothing is enqueued on an error. */
int ckl_topk(int dtype, const void* logits, int64_t N, int64_t V, int64_t K, int32_t* ids_out, float* vals_out,
             hipStream_t stream);

/* Chunk planner of the fused call (pure host computation, needs no GPU).  The
 * sequence is cut into chunks of C rows so that the loss's own device memory
 * stays bounded independently of N ("A New Trick...", section "Does this
 * matter for longer documents?": peak memory barely grows with input length).
 *   dtype         ckl_dtype of H and W
 *   budget_bytes  0 = CKL_WORKSPACE_BYTES or 6 GiB
 *   chunk_out, workspace_bytes_out  (may be NULL) the rows per chunk a call
 *                 with chunk = 0 uses, and the exact bytes it allocates for its
 *                 workspace: the largest multiple of 256 rows that fits (or N if
 *                 N < 256), evened out over the resulting chunk count, then
 *                 lowered by 256-row steps until it fits (the workspace is not
 *                 monotonic in the chunk: the dH split count depends on it)
 * Returns CKL_EBUDGET if not even 256 rows (or N) fit, CKL_EINVAL /
 * CKL_EUNSUPPORTED for shapes the calls reject. */
int ckl_plan(int64_t N, int64_t d, int64_t V, int64_t K, int dtype, uint64_t budget_bytes, int64_t* chunk_out,
             uint64_t* workspace_bytes_out);

/* The planner for one of the calls with a caller-given chunk: pass = ckl_pass
 * (the forward-only call needs no dH split-K slabs, so it can take longer
 * chunks); chunk > 0 checks min(chunk, N) rows against the budget
 * (CKL_EBUDGET if they do not fit), chunk = 0 plans as ckl_plan does. */
int ckl_plan_pass(int pass, int64_t N, int64_t d, int64_t V, int64_t K, int dtype, int64_t chunk,
                  uint64_t budget_bytes, int64_t* chunk_out, uint64_t* workspace_bytes_out);

/* Frees every cached workspace (after synchronising the device). */
void ckl_release_workspace(void);

/* Bytes currently held in cached workspaces (all devices and streams). */
uint64_t ckl_workspace_bytes_held(void);

/* Human-readable name of a status code. */
const char* ckl_strerror(int status);

/* Test entry: the row pass alone on caller-given fp32 logits Z [R, V]
 * (row stride V): log-normaliser, teacher softmax, gather, KL and the logit
 * gradient with weight `scale` for rows whose mask is 1 (or all rows if mask
 * is NULL).  Z is first turned into what the logits GEMM leaves in the
 * workspace (per 128-id slice: max m and exp(z - m) in the gradient's element
 * type), then the production row kernels run.  Outputs (device, caller-owned):
 *   zg_out          fp32 [R, K]  the logits at the teacher ids as the row pass read them
 *                                (copied from Z through the same id tables the
 *                                logits contraction fills: Z[r, id] bit for bit)
 *   scatter_ids_out int32 [R, K] the ids the top-K values were scattered to
 *   G_out           [R, V]       gradient, bf16 if g_bf16 else fp32
 *   kl_out, lse_out fp32 [R]     per-row KL and logsumexp (both 0 for masked rows)
 * Synchronises `stream` before returning. */
int ckl_debug_rows(const float* Z, const int32_t* idx, const float* tlogit, const uint8_t* mask, int64_t R,
                   int64_t V, int64_t K, float scale, int g_bf16, float* zg_out, int32_t* scatter_ids_out,
                   void* G_out, float* kl_out, float* lse_out, hipStream_t stream);

/* Measurement support.  While enabled, every kernel launch of a loss call
 * (ckl_fwd_bwd*, ckl_fwd, ckl_bwd, ckl_topk) is bracketed by HIP events on the call's
 * stream.  ckl_timing_query waits for the recorded events and returns the
 * summed milliseconds and launch count of one kernel kind: 0 logits GEMM,
 * 1 row pass, 2 dH GEMM, 3 dH split reduce, 4 dW GEMM, 5 other, 6 top-K
 * (ckl_topk).  Not for concurrent use from several threads. */
int ckl_timing_enable(int on);
int ckl_timing_query(int kind, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* CKL_H_ */
