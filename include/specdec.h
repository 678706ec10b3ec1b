/*
 * specdec.h - batched speculative-decoding verification and paged KV append / rollback
 * on AMD Instinct MI355X (gfx950). C ABI, plain pointers and sizes.
 *
 * One speculative cycle, as the pages describe it, is three stream-ordered calls:
 *
 *   kv_paged_append  - provisional append of the K/V the target pass produced for the
 *                      pending token and the k_b proposals of every request
 *                      ("Walk through KV-cache updates when speculative decoding rejects
 *                      some draft tokens", both paragraphs: K/V are appended as part of
 *                      the verifying forward pass, before the accept test);
 *   specdec_verify   - left-to-right modified rejection sampling with replacement /
 *                      bonus sampling ("Speculative decoding: accelerate LLM generation
 *                      without changing its answers", section 2 "Draft, verify, correct");
 *   kv_rollback      - truncate every request back to its committed prefix, freeing the
 *                      blocks past it ("Walk through KV-cache updates ...", paragraph 1;
 *                      "Keep cache validity aligned with the committed token history",
 *                      paragraphs 1-4).
 *   kv_rollback_draft - the same for the draft model's cache under its own processed-
 *                      state convention ("Keep cache validity ...", paragraph 5).
 *
 * Conventions for every entry point:
 *   - Pointers named device are device memory owned by the caller; the library never
 *     allocates, never frees, never synchronizes the stream and keeps no global mutable
 *     state. All work is enqueued on `stream`; outputs are valid once the stream reaches
 *     that point.
 *   - Arguments the host can see are checked before anything is enqueued; on failure the
 *     call returns SPECDEC_EINVAL and no device memory is touched.
 *   - Problems only the device can see (bad token ids, non-finite logits, too few free
 *     blocks, ...) set sticky bits in a caller-owned device word (OR-ed, never cleared by
 *     the library) and are handled per request as documented below.
 *   - No random numbers are drawn inside: every random decision uses the caller's
 *     uniforms, so results are a deterministic function of the inputs.
 */
#ifndef SPECDEC_H
#define SPECDEC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------------------ */
#define SPECDEC_OK          0
#define SPECDEC_EINVAL     (-1)   /* a host-visible argument is invalid; nothing enqueued */
#define SPECDEC_EHIP       (-3)   /* a HIP launch / runtime call failed                    */
#define SPECDEC_EWORKSPACE (-4)   /* workspace missing, misaligned or too small            */
#define SPECDEC_ESCRATCH   (-5)   /* specdec_cycle_static: the call needs more scratch than
                                     SPECDEC_STATIC_SCRATCH_BYTES; nothing enqueued       */

/* ---- logits element type ----------------------------------------------------------- */
#define SPECDEC_F32  0
#define SPECDEC_BF16 1

/* ---- device-side bits of specdec_verify's err_word and req_flags --------------------- */
#define SPECDEC_ERR_TOKEN      1   /* a draft token id outside [0, V)                      */
#define SPECDEC_ERR_K          2   /* cu_draft inconsistent: k_b<0, k_b>max_k, cu[0]!=0,
                                      cu[B]!=K                                            */
#define SPECDEC_ERR_NONFINITE  4   /* NaN / +inf logit in one of the request's rows, or a
                                      row with no finite kept logit                       */
#define SPECDEC_ERR_QZERO      8   /* flag only: q_i(y_i) == 0 at an evaluated position    */
#define SPECDEC_ERR_ZFALLBACK 16   /* flag only: residual mass was 0 after a rejection;
                                      the replacement was drawn from p_i                   */
#define SPECDEC_ERR_UNIFORM   32   /* a uniform outside [0, 1) (or NaN)                   */
#define SPECDEC_ERR_TREE     128   /* a draft tree's parent index outside {-1, .., j-1}   */
#define SPECDEC_ERR_TEAM     256   /* a tree walk's workgroup waited past its bound for the
                                      others of its request (not expected); request failed */
#define SPECDEC_ERR_PARAM     64   /* per-request parameters invalid: temperature <= 0 or
                                      not finite, top_p NaN, or an active top_k above
                                      specdec_params.top_k_max                            */

/* ---- device-side bits of kv_paged_cache.state --------------------------------------- */
#define KV_ERR_NOMEM       64        /* append needed more blocks than free: not applied   */
#define KV_ERR_APPEND     128        /* append argument invalid on device: not applied     */
#define KV_ERR_ROLLBACK   256        /* rollback request invalid (skipped) or corrupt meta */
#define KV_APPEND_REJECTED (1 << 16) /* not sticky: the latest append was not applied, so
                                        the next kv_rollback is a no-op                    */

/* Largest proposal count per request, batch size for the KV calls, and vocabulary. */
#define SPECDEC_MAX_K      64
#define SPECDEC_MAX_TREE   64         /* nodes of one request's draft tree               */
#define SPECDEC_MAX_KV_BATCH 4096
#define SPECDEC_MAX_V      2097152
/* positions the early-exit calls read one launch at a time before one launch reads the
 * rest of every request still live */
#define SPECDEC_EARLY_EXIT_SEQUENTIAL 2

/* Short English text for a return code. Never NULL. */
const char* specdec_status_string(int status);

/* =====================================================================================
 * Verification
 * ===================================================================================== */

/* Optional per-call diagnostics and scheduling hooks; any field may be NULL / 0. Row
 * arrays are indexed with the target rows first (0 .. K+B-1) and then the draft rows
 * (K+B .. 2K+B-1). */
typedef struct specdec_debug {
    double*  p_y;          /* [K]  p_i(y_i) after the transform                           */
    double*  q_y;          /* [K]  q_i(y_i)                                               */
    float*   row_max;      /* [2K+B] max kept logit of the row                            */
    double*  row_sum;      /* [2K+B] S = sum over kept x of exp((z(x) - max) / T)         */
    float*   row_thr;      /* [2K+B] top-k threshold logit (-inf when top-k is off)       */
    int32_t* row_nkept;    /* [2K+B] kept tokens with finite logit (-1 when top-k and
                                   top-p are off)                                         */
    double*  resid_mass;   /* [B]  W the final token was drawn from: residual mass, or
                                   sum of p for the bonus                                  */
    double*  picked_prob;  /* [B]  w(x*) / W                                               */
    int32_t* req_flags;    /* [B]  SPECDEC_ERR_* bits of the request                       */
    hipEvent_t ev_stats_begin;  /* timing events attached to the launch of the kernel    */
    hipEvent_t ev_stats_end;    /* that streams the logit rows (both or neither)         */
    hipEvent_t ev_stats_done;   /* recorded on `stream` once the logit rows have been
                                   streamed: independent bandwidth-bound work (the K/V
                                   scatter) can start on another stream while the
                                   latency-bound sampling kernel runs                     */
    /* Acceptance analytics ("Speculative decoding ...", section 3: a proposal drawn from q_i
     * is accepted with probability beta_i = sum_x min(p_i(x), q_i(x)) = 1 - (the residual
     * mass); section 4: E[A], the expected output of a cycle). Either pointer non-NULL adds
     * one pass over every proposal's row pair after the draw (the kept-token lists of bf16
     * top-k / top-p rows instead, where they exist). NaN for a failed request. */
    double*  accept_prob;       /* [K] beta_i of every proposal position                  */
    double*  expected_emitted;  /* [B] E[A] = 1 + sum_j prod_{i<=j} beta_i                */
} specdec_debug;

/* Per-request decoding transform ("Speculative decoding ...", sections 3 and 4: the same
 * transform on p and q of a request; requests of one batch may differ). Each array holds
 * B device values and replaces the scalar argument of the same name for every request;
 * NULL keeps the scalar. A request whose values are invalid fails with SPECDEC_ERR_PARAM
 * (num_accepted = -1) without affecting the others. Host struct, read during the call. */
typedef struct specdec_params {
    const float*   temperature;  /* [B] > 0 and finite                                   */
    const int32_t* top_k;        /* [B] any value; <= 0 or >= V: off                     */
    const float*   top_p;        /* [B] not NaN; <= 0 or >= 1: off                       */
    int32_t        top_k_max;    /* with top_k: the largest active top_k[b] allowed; the
                                    workspace is sized for it (>= 0; above 1024 those
                                    rows take the multi-pass select)                    */
    /* Stopping ("Keep cache validity aligned with the committed token history",
     * paragraph 6 lists EOS and output caps among the cases to test): when the accepted
     * proposals contain the request's end-of-sequence token, or the request may emit
     * fewer tokens than the cycle would, the output ends there: y_1 .. y_L with
     * L = the first EOS position (inclusive), or the cap, whichever is smaller, if that
     * falls within the accepted proposals; then nothing is drawn, num_emitted = L and
     * num_accepted = L (the cache keeps the pending token and y_1 .. y_L). A drawn
     * replacement or bonus token equal to EOS just ends the output naturally. Neither
     * array changes the transform or the path the rows take. */
    const int32_t* eos_token;    /* [B] device or NULL; < 0: none                        */
    const int32_t* max_emit;     /* [B] device or NULL; <= 0: no cap                     */
} specdec_params;

/* Bytes of device workspace specdec_verify needs for these sizes (16-byte aligned); 0
 * for sizes the call rejects (B < 1, K < 0, V outside [1, SPECDEC_MAX_V], bad dtype,
 * top_p NaN). */
size_t specdec_verify_workspace_size(int32_t B, int32_t K, int32_t V, int32_t dtype,
                                     int32_t top_k, float top_p,
                                     const specdec_params* per_request);

/*
 * specdec_verify - one verification step for a batch of B requests.
 *
 * For request b with k_b = cu_draft[b+1] - cu_draft[b] proposals y_1..y_k (draft_tokens
 * [cu_draft[b] .. cu_draft[b+1])):
 *   p_i = transform(target row i), i = 0..k_b (row k_b is the position after the block),
 *   q_i = transform(draft row i),  i = 0..k_b-1,
 * where transform keeps the tokens whose logit is >= the top_k-th largest logit of the row
 * (ties inclusive; all finite tokens when top_k <= 0 or top_k >= V) and applies a
 * max-subtracted softmax at temperature T ("Speculative decoding ...", section 6: stable
 * softmax, identical transform on both sides); then, when 0 < top_p < 1, keeps only the
 * nucleus: the tokens whose probability is >= the largest v such that the tokens of
 * probability >= v carry at least top_p of the mass (ties inclusive), and renormalizes
 * (sections 3 and 4 name temperature, top-k and top-p truncation among the transforms
 * applied alike to p and q). Proposal i is accepted iff
 * u_accept[cu_draft[b]+i] * q_i(y_i) < p_i(y_i), i.e. with probability
 * min(1, p_i(y_i)/q_i(y_i)) (section 2). The first rejection j ends the run; the
 * replacement is drawn from normalize(max(0, p_j - q_j)), or, when all k_b are accepted,
 * the bonus token from p_{k_b}; both by inverse CDF over ascending token ids with
 * u_sample[b]: the smallest x whose running sum exceeds u * W (section 2; section 3
 * shows the emitted token then has law p).
 *
 * Layout (all device, row-major, packed ragged):
 *   target_logits [K+B][V] dtype: rows of request b are cu_draft[b] + b + i, i = 0..k_b
 *   draft_logits  [K][V]   dtype: rows cu_draft[b] + i, i < k_b
 *   draft_tokens  [K] int32,  cu_draft [B+1] int32 (exclusive prefix of k_b)
 *   u_accept [K] fp32, u_sample [B] fp32, caller-drawn uniforms in [0, 1)
 * Outputs (device):
 *   out_tokens   [K+B] int32: request b writes num_emitted[b] tokens at cu_draft[b] + b
 *                (the accepted proposals, then the replacement or bonus token); other
 *                entries are left untouched
 *   num_accepted [B] int32 (-1 on a request error), num_emitted [B] int32 (0 on error)
 *   err_word     [1] int32, SPECDEC_ERR_* bits OR-ed in (not cleared)
 * Host scalars: B >= 1, K = cu_draft[B] (the packed row count the caller allocated),
 * 0 <= max_k <= SPECDEC_MAX_K, 1 <= V <= SPECDEC_MAX_V, dtype SPECDEC_F32 or SPECDEC_BF16,
 * temperature > 0 and finite, top_k any value (<= 0 or >= V disables it), top_p any
 * value but NaN (<= 0 or >= 1 disables it); a scalar that per_request replaces is not
 * checked. per_request: NULL, or per-request arrays (specdec_params; top_k_max >= 0 when
 * top_k is given). The nucleus mass decision is made with fp32
 * exponentials summed in fixed point (2^-42 units): a row whose boundary mass lies within
 * about 1e-6 of top_p may keep one group of equal logits more or less than exact
 * arithmetic would.
 * workspace: device, 16-byte aligned, >= specdec_verify_workspace_size(B, K, V, dtype,
 * top_k, top_p, per_request) bytes, owned by the caller; its contents need no initialization and are
 * scratch between calls. Calls that share a workspace must not overlap.
 * Returns SPECDEC_OK once enqueued, or SPECDEC_EINVAL / SPECDEC_EWORKSPACE /
 * SPECDEC_EHIP without enqueuing anything that writes outputs.
 */
int specdec_verify(const void* target_logits, const void* draft_logits, int32_t dtype,
                   const int32_t* draft_tokens, const int32_t* cu_draft,
                   const float* u_accept, const float* u_sample,
                   int32_t B, int32_t K, int32_t max_k, int32_t V,
                   float temperature, int32_t top_k, float top_p,
                   const specdec_params* per_request,
                   int32_t* out_tokens, int32_t* num_accepted, int32_t* num_emitted,
                   int32_t* err_word, const specdec_debug* dbg,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* specdec_verify_early_exit: specdec_verify without the rows past a request's first
 * rejection ("Speculative decoding: accelerate LLM generation without changing its
 * answers" §2-3: nothing after the first rejected proposal decides anything). The row
 * statistics of positions 0 .. SPECDEC_EARLY_EXIT_SEQUENTIAL - 1 run one launch per
 * position, each reading the rows of the requests whose earlier proposals were all
 * accepted; one more launch reads every later row of the requests still live then (ahead
 * of their decisions: few requests get that far, and one launch costs less than one per
 * position). A request rejected at an earlier position reads none of them. With a top-k /
 * top-p transform (scalar or per request) each of these is a chunk-select launch followed
 * by a merge launch over the rows it selected. The decision and the draw follow.
 * Arguments, layouts, ownership and workspace (specdec_verify_workspace_size with the same
 * arguments): as specdec_verify, and the same results bit for bit for every request whose
 * read rows are finite. A non-finite row past the first rejection is not reported; debug
 * p_y / q_y past the first rejection and row_max / row_sum / row_thr of rows not read are
 * NaN (row_nkept -1); ev_stats_begin / ev_stats_end bracket all the statistics launches.
 * Every transform specdec_verify takes (temperature, top-k, top-p, scalar or per request).
 * Host: every specdec_verify check, and also EINVAL, before anything is enqueued, when dbg
 * asks for the acceptance analytics (they need every row).
 */
int specdec_verify_early_exit(const void* target_logits, const void* draft_logits, int32_t dtype,
                              const int32_t* draft_tokens, const int32_t* cu_draft,
                              const float* u_accept, const float* u_sample,
                              int32_t B, int32_t K, int32_t max_k, int32_t V,
                              float temperature, int32_t top_k, float top_p,
                              const specdec_params* per_request,
                              int32_t* out_tokens, int32_t* num_accepted, int32_t* num_emitted,
                              int32_t* err_word, const specdec_debug* dbg,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* =====================================================================================
 * Paged KV cache
 * ===================================================================================== */

/* Cache metadata and storage, all device memory owned by the caller. Physical block X of
 * layer l holds block_size slots of K then V: pool[l][0][X] and pool[l][1][X], each slot
 * num_kv_heads * head_dim bf16 values. Logical block lb of request b is
 * block_tables[b][lb]; it is valid iff lb < ceil(seq_lens[b] / block_size), and entries
 * past that are -1. refcount[X] counts the table entries that reference X; a block is on
 * the free list iff its refcount is 0. The free list is a stack: free_list[0 ..
 * *free_count) with the top at *free_count - 1 ("Keep cache validity ...", paragraph 3:
 * block tables, ownership and reference counts decide which physical memory is valid). */
typedef struct kv_paged_cache {
    void*    pool;            /* bf16 [L][2][num_blocks][block_size][H][D]             */
    int32_t  num_layers;      /* L >= 1                                                */
    int32_t  num_kv_heads;    /* H >= 1                                                */
    int32_t  head_dim;        /* D >= 1; H*D*2 bytes must be a multiple of 16          */
    int32_t  block_size;      /* slots per block, >= 1                                 */
    int32_t  num_blocks;      /* NB >= 1                                               */
    int32_t  max_blocks_per_req;  /* MBR: columns of block_tables                      */
    int32_t* block_tables;    /* [B][MBR] int32                                        */
    int32_t* seq_lens;        /* [B] valid K/V entries; the committed length is one more
                                 (the last committed token is pending)                  */
    int32_t* refcount;        /* [NB]                                                  */
    int32_t* free_list;       /* [NB]                                                  */
    int32_t* free_count;      /* [1]                                                   */
    int32_t* state;           /* [1] KV_ERR_* sticky bits and KV_APPEND_REJECTED       */
} kv_paged_cache;

/* Bytes of device workspace kv_paged_append needs for B requests and N new entries. */
size_t kv_paged_append_workspace_size(int32_t B, int32_t N);

/*
 * kv_paged_append - provisional append of n_b = cu_new[b+1] - cu_new[b] entries per
 * request (in a cycle: the pending token and the k_b proposals, n_b = k_b + 1) at slots
 * seq_lens[b] .. seq_lens[b] + n_b - 1.
 * k_new, v_new: device bf16 [L][N][H][D] with N = cu_new[B]; entry t of request b is row
 * cu_new[b] + t. cu_new: device int32 [B+1].
 * Blocks are popped from the top of the free list in ascending request order, then
 * ascending logical block. When the receiving partial block is shared (refcount > 1) it
 * is first copied into a fresh block (copy-on-write, slots below seq_len) and the old
 * block is released ("Keep cache validity ...", paragraph 4: shared-prefix isolation).
 * All-or-nothing: if the batch needs more blocks than are free (KV_ERR_NOMEM) or an
 * argument is invalid on device (KV_ERR_APPEND: n_b < 0, cu_new[0] != 0, cu_new[B] != N,
 * capacity MBR * block_size exceeded, no block for a partial tail), no request changes
 * and KV_APPEND_REJECTED is set; a successful append clears KV_APPEND_REJECTED.
 * Host checks: 1 <= B <= SPECDEC_MAX_KV_BATCH, N >= 0, pointers non-NULL, geometry > 0.
 * workspace: device, 16-byte aligned, >= kv_paged_append_workspace_size(B, N) bytes;
 * scratch between calls, no initialization needed; calls sharing it must not overlap.
 */
int kv_paged_append(const kv_paged_cache* cache, int32_t B,
                    const void* k_new, const void* v_new, const int32_t* cu_new, int32_t N,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kv_rollback - truncate every request to its committed prefix after verification:
 * drop_b = k_b - num_accepted[b] trailing entries (k_b = cu_draft[b+1] - cu_draft[b]),
 * so that after a cycle seq_lens[b] = old length + 1 + num_accepted[b] (the pending token
 * and the accepted proposals stay; the replacement / bonus token becomes the new pending
 * token: "Keep cache validity ...", paragraphs 1-2). For every logical block from
 * ceil(new / block_size) to ceil(old / block_size) - 1 the refcount is decremented, the
 * block is pushed on the free list when it reaches 0 (ascending request, then logical
 * block order), and the table entry becomes -1. Only metadata changes: slots past the new
 * length inside a retained block keep their bytes ("rejected speculative tokens remain in
 * KV", paragraph 2). A request with num_accepted < 0, num_accepted > k_b or drop > seq_len
 * is skipped and KV_ERR_ROLLBACK set; a table entry out of range or a refcount already 0
 * sets KV_ERR_ROLLBACK and that entry is only cleared. The call is a no-op when the
 * latest append was rejected (KV_APPEND_REJECTED). B <= SPECDEC_MAX_KV_BATCH.
 * num_accepted [B] and cu_draft [B+1]: device int32 (specdec_verify's outputs / inputs).
 */
int kv_rollback(const kv_paged_cache* cache, int32_t B, const int32_t* num_accepted,
                const int32_t* cu_draft, hipStream_t stream);

/*
 * kv_rollback_draft - realign the draft model's cache with the committed history after
 * verification ("Keep cache validity aligned with the committed token history",
 * paragraph 5: the draft advanced along its own proposals and is realigned under its own
 * processed-state convention). To propose k_b tokens the draft processed its pending
 * token(s) and y_1 .. y_{k_b-1}, never y_{k_b}, which it only sampled; so it keeps the
 * states of y_1 .. y_{min(a_b, k_b-1)} and drops max(0, k_b - 1 - num_accepted[b]) trailing
 * entries (none when k_b = 0). Its pending tokens are then the replacement, or y_{k_b} and
 * the bonus token after a fully accepted round. Block release, error handling and the
 * no-op after a rejected append are those of kv_rollback; arguments likewise.
 */
int kv_rollback_draft(const kv_paged_cache* cache, int32_t B, const int32_t* num_accepted,
                      const int32_t* cu_draft, hipStream_t stream);

/* =====================================================================================
 * One whole cycle
 * ===================================================================================== */

/* Bytes of device workspace specdec_cycle needs (16-byte aligned); 0 where
 * specdec_verify_workspace_size gives 0. */
size_t specdec_cycle_workspace_size(int32_t B, int32_t K, int32_t V, int32_t dtype,
                                    int32_t top_k, float top_p,
                                    const specdec_params* per_request);

/*
 * specdec_cycle - one speculative cycle with the same effect as the three calls
 *   kv_paged_append(cache, B, k_new, v_new, cu_new, K + B, ...)   with cu_new[b] = cu_draft[b] + b
 *   specdec_verify(target_logits, ..., num_accepted, ...)
 *   kv_rollback(cache, B, num_accepted, cu_draft)
 * on `stream`: the pending token and the k_b proposals of every request are appended
 * (entry t of request b is row cu_draft[b] + b + t of k_new / v_new, bf16 [L][K+B][H][D]),
 * verified, and the cache truncated to the pending token plus the accepted proposals
 * ("Walk through KV-cache updates when speculative decoding rejects some draft tokens",
 * paragraph 1; "Keep cache validity aligned with the committed token history",
 * paragraphs 1-2). Outputs, error bits and cache state are bit-identical to the three
 * calls. The launches are fused so that block allocation overlaps the logit stream and the
 * K/V scatter overlaps the per-request sampling. Arguments and their checks are those of
 * the three calls (B <= SPECDEC_MAX_KV_BATCH); workspace >=
 * specdec_cycle_workspace_size(B, K, V, dtype, top_k, top_p, per_request) bytes, 16-byte
 * aligned.
 */
int specdec_cycle(const kv_paged_cache* cache, const void* k_new, const void* v_new,
                  const void* target_logits, const void* draft_logits, int32_t dtype,
                  const int32_t* draft_tokens, const int32_t* cu_draft,
                  const float* u_accept, const float* u_sample,
                  int32_t B, int32_t K, int32_t max_k, int32_t V,
                  float temperature, int32_t top_k, float top_p,
                  const specdec_params* per_request,
                  int32_t* out_tokens, int32_t* num_accepted, int32_t* num_emitted,
                  int32_t* err_word, const specdec_debug* dbg,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * specdec_cycle_static - specdec_cycle without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Its scratch is one array of
 * SPECDEC_STATIC_SCRATCH_BYTES in the library's device image: each GPU the library runs
 * on holds its own copy until the process ends; the library takes its address once per
 * device on the first call there. The call allocates nothing and frees nothing. Arguments,
 * layouts, ownership, host checks and results: as specdec_cycle with a workspace of that
 * size, bit for bit. A call whose workspace (specdec_cycle_workspace_size with the same
 * arguments) exceeds the array returns SPECDEC_ESCRATCH before anything is enqueued
 * (temperature-only cycles fit up to several hundred requests at V = 152064; top-k and
 * top-p candidate lists do not fit past small batches). Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (other streams, other threads) race and must
 * be serialized by the caller. Nothing in the array must start at zero (every launch
 * writes what it reads).
 */
#define SPECDEC_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
int specdec_cycle_static(const kv_paged_cache* cache, const void* k_new, const void* v_new,
                         const void* target_logits, const void* draft_logits, int32_t dtype,
                         const int32_t* draft_tokens, const int32_t* cu_draft,
                         const float* u_accept, const float* u_sample,
                         int32_t B, int32_t K, int32_t max_k, int32_t V,
                         float temperature, int32_t top_k, float top_p,
                         const specdec_params* per_request,
                         int32_t* out_tokens, int32_t* num_accepted, int32_t* num_emitted,
                         int32_t* err_word, const specdec_debug* dbg, hipStream_t stream);

/* specdec_cycle_early_exit: the same cycle without the rows past a request's first
 * rejection. "Speculative decoding: accelerate LLM generation without changing its
 * answers" §2-3: once proposal i is rejected, nothing after it is looked at; the accepted
 * count, the emitted tokens, the draw and the cache step depend only on the rows of
 * positions 0..j (j the first rejection, or k_b with the bonus row).
 *
 * Arguments, layouts, ownership, workspace (specdec_cycle_workspace_size with the same
 * arguments) and results: as specdec_cycle, bit for bit, for every request whose rows are
 * finite. Differences, all from the rows that are not read:
 *   - the row statistics of positions 0 .. SPECDEC_EARLY_EXIT_SEQUENTIAL - 1 run one launch
 *     per position p, each reading the rows of position p of the requests whose proposals
 *     before p were all accepted; one more launch reads every later row of the requests
 *     live at SPECDEC_EARLY_EXIT_SEQUENTIAL (ahead of their decisions); with a top-k /
 *     top-p transform each of these is a chunk-select launch followed by a merge launch
 *     over the rows it selected; the K/V scatter is spread over the launches after the
 *     first;
 *   - SPECDEC_ERR_NONFINITE covers the rows read (a non-finite row after the first
 *     rejection is not seen);
 *   - debug p_y / q_y after the first rejection, and row_max / row_sum / row_thr of rows
 *     not read, are NaN (row_nkept -1);
 *   - events: ev_stats_begin / ev_stats_end bracket all the statistics launches.
 * Every transform specdec_cycle takes: temperature, top-k and top-p, scalar or per request
 * (a request with invalid parameters reads no row and fails with SPECDEC_ERR_PARAM as in
 * specdec_cycle). Host: every specdec_cycle check, and also EINVAL, before anything is
 * enqueued, when dbg asks for the acceptance analytics (accept_prob, expected_emitted:
 * they need every row).
 */
int specdec_cycle_early_exit(const kv_paged_cache* cache, const void* k_new, const void* v_new,
                             const void* target_logits, const void* draft_logits, int32_t dtype,
                             const int32_t* draft_tokens, const int32_t* cu_draft,
                             const float* u_accept, const float* u_sample,
                             int32_t B, int32_t K, int32_t max_k, int32_t V,
                             float temperature, int32_t top_k, float top_p,
                             const specdec_params* per_request,
                             int32_t* out_tokens, int32_t* num_accepted, int32_t* num_emitted,
                             int32_t* err_word, const specdec_debug* dbg,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* =====================================================================================
 * Contiguous KV cache
 * ===================================================================================== */

/* One contiguous buffer per request with a write pointer ("Walk through KV-cache updates
 * when speculative decoding rejects some draft tokens": on a contiguous buffer rollback
 * rewinds the write pointer). All device memory owned by the caller. Entry t of request b
 * (layer l, K or V) lives at pool[l][kv][b][t]. */
typedef struct kv_contig_cache {
    void*    pool;            /* bf16 [L][2][batch][max_len][H][D]                     */
    int32_t  num_layers;      /* L >= 1                                                */
    int32_t  num_kv_heads;    /* H >= 1                                                */
    int32_t  head_dim;        /* D >= 1; H*D*2 bytes must be a multiple of 16          */
    int32_t  max_len;         /* entries per request, >= 1                             */
    int32_t  batch;           /* requests the pool holds, >= B of every call           */
    int32_t* seq_lens;        /* [batch] valid entries (the write pointer)             */
    int32_t* state;           /* [1] KV_ERR_* sticky bits and KV_APPEND_REJECTED       */
} kv_contig_cache;

/*
 * kv_contig_append - provisional append of n_b = cu_new[b+1] - cu_new[b] entries per
 * request at seq_lens[b] .. seq_lens[b] + n_b - 1 (same k_new / v_new / cu_new layout as
 * kv_paged_append). All-or-nothing: an entry past max_len (KV_ERR_NOMEM) or an invalid
 * argument on device (KV_ERR_APPEND: n_b < 0, cu_new[0] != 0, cu_new[B] != N, seq_len
 * outside [0, max_len]) leaves every request unchanged and sets KV_APPEND_REJECTED, which
 * a successful append clears. Host checks as kv_paged_append (B <= batch). Three launches
 * on `stream` (check, copy, commit); no workspace.
 */
int kv_contig_append(const kv_contig_cache* cache, int32_t B, const void* k_new,
                     const void* v_new, const int32_t* cu_new, int32_t N, hipStream_t stream);

/*
 * kv_contig_rollback - rewind every request's write pointer to its committed prefix:
 * drop k_b - a_b entries (draft = 0, the target's cache after a cycle that appended
 * k_b + 1), or max(0, k_b - 1 - a_b) (draft = 1, the draft's convention as in
 * kv_rollback_draft). Invalid requests (a_b < 0, a_b > k_b, more dropped than held) are
 * skipped and set KV_ERR_ROLLBACK; no-op after an append that was not applied. One launch.
 */
int kv_contig_rollback(const kv_contig_cache* cache, int32_t B, const int32_t* num_accepted,
                       const int32_t* cu_draft, int32_t draft, hipStream_t stream);

/* =====================================================================================
 * Draft trees
 * ===================================================================================== */

/*
 * specdec_tree_verify - verification of one draft tree per request.
 *
 * Request b owns nodes cu_nodes[b] .. cu_nodes[b+1]-1 (n_b <= max_nodes <= SPECDEC_MAX_TREE);
 * node j (local index) has token tree_tokens[cu_nodes[b] + j] and parent
 * tree_parent[cu_nodes[b] + j] in {-1, 0, .., j-1} (-1: a child of the root, the position
 * after the committed prefix). Positions: 0 the root, 1 + j the position after node j;
 * target_logits / draft_logits [N+B][V] hold the rows of request b's positions at
 * cu_nodes[b] + b + v (draft rows of nodes without children are not read).
 * The children of a position are alternatives for the next token, each drawn by the draft
 * from that position's q; they are tried in node order, child j accepted iff
 * u_accept[cu_nodes[b] + j] * q(y_j) < p'(y_j), where p' starts as the position's p and
 * after each rejected child becomes normalize(max(0, p' - q)) ("Speculative decoding ...",
 * sections 2-3: the linear rule, with the residual applied sibling after sibling). The first
 * accepted child continues the walk from its position; when every child is rejected the
 * replacement is drawn from the last residual, and a position reached by acceptance with
 * no children yields the bonus token from its p; both by inverse CDF with u_sample[b]
 * (ascending ids). Every target and draft row the walk reads takes the same transform as
 * in specdec_verify: temperature, then top_k (0 or >= V: off; ties at the k-th value
 * kept), then top_p (<= 0 or >= 1: off; the nucleus of the top-k set, ties kept); with
 * either filter on, the call first selects over every target row and the draft row of
 * every position with children (the draft rows of leaves are never read) and the walk
 * reads the kept tokens' statistics from there. per_request (or
 * NULL) replaces any of the three scalars by [B] arrays as in specdec_verify (a request
 * whose values are invalid fails with SPECDEC_ERR_PARAM alone); its stopping arrays
 * (eos_token, max_emit) are not taken on trees (EINVAL).
 * Outputs (device): num_accepted [B] = the accepted path's length (-1 on error),
 * num_emitted [B] = that + 1; out_tokens [N+B]: request b writes the path's tokens then
 * the drawn token at cu_nodes[b] + b; accepted_nodes [N]: the path's local node indices,
 * root first, at cu_nodes[b]; err_word [1] OR-ed SPECDEC_ERR_* bits (SPECDEC_ERR_TREE for a
 * bad parent); req_flags [B] (or NULL) each request's bits.
 * team: workgroups that share one request's walk (each pass over a row is split among
 * them); 0 picks min(16, max(1, CUs / B)), otherwise 1..16. The outputs do not depend on
 * it: partial sums are combined in a fixed order.
 * workspace: device, 16-byte aligned, >= specdec_tree_verify_workspace_size(B, N, V,
 * dtype, top_k, top_p, per_request) bytes, owned by the caller, contents need not be
 * initialized (the call resets its counters first); not used by other calls while this
 * one runs.
 * Host: B >= 1, N = cu_nodes[B], 0 <= max_nodes <= SPECDEC_MAX_TREE, 1 <= V <=
 * SPECDEC_MAX_V, temperature > 0 and finite and top_p not NaN (unless replaced per
 * request), per_request->top_k_max >= 0 with a top_k array, 0 <= team <= 16; EINVAL
 * otherwise, EWORKSPACE for a missing / small / misaligned workspace, before anything is
 * enqueued. Two launches on `stream` (counter reset, walk), three more before the walk
 * with top-k / top-p (the marking of the draft rows read, the chunk select, the per-row
 * merge; no chunk select with top_k above 1024), one more with per-request arrays (each
 * row's parameters). Testing only: the environment variable
 * SPECDEC_TREE_SPIN_LIMIT (a decimal integer in [0, 2^20], read at each call; anything
 * else is ignored) lowers the bound on the polls a member makes while it waits for the
 * rest of its team (default 2^20); a member that reaches the bound gives up, and its
 * request fails with SPECDEC_ERR_TEAM (the other requests are unaffected).
 */
size_t specdec_tree_verify_workspace_size(int32_t B, int32_t N, int32_t V, int32_t dtype,
                                          int32_t top_k, float top_p,
                                          const specdec_params* per_request);
int specdec_tree_verify(const void* target_logits, const void* draft_logits, int32_t dtype,
                        const int32_t* tree_tokens, const int32_t* tree_parent,
                        const int32_t* cu_nodes, const float* u_accept, const float* u_sample,
                        int32_t B, int32_t N, int32_t max_nodes, int32_t V, float temperature,
                        int32_t top_k, float top_p, const specdec_params* per_request,
                        int32_t* out_tokens, int32_t* accepted_nodes, int32_t* num_accepted,
                        int32_t* num_emitted, int32_t* err_word, int32_t* req_flags,
                        int32_t team, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * kv_tree_commit - keep the accepted path of every request's tree in the cache ("Keep cache
 * validity aligned with the committed token history", paragraph 3: gather the accepted
 * path into the cache layout, drop the siblings). The cycle appended n_b + 1 entries per
 * request with kv_paged_append (the pending token, then node j at the pending slot + 1 + j;
 * cu_new[b] = cu_nodes[b] + b). Path node i (i = 1..a_b, from accepted_nodes) moves to the
 * pending slot + i, in increasing i; then the cache is truncated to the pending slot + 1 +
 * a_b and blocks past the end are released as kv_rollback does (n_b - a_b dropped). A
 * request with a_b < 0 or > n_b, a path not strictly increasing within [0, n_b), offsets
 * outside [0, N] (N: the length of accepted_nodes, = cu_nodes[B]), or fewer than n_b + 1
 * entries is left as it is and flagged (KV_ERR_ROLLBACK). Nothing is done after an append
 * that was not applied. Two launches on `stream`; no workspace.
 */
int kv_tree_commit(const kv_paged_cache* cache, int32_t B, const int32_t* num_accepted,
                   const int32_t* accepted_nodes, const int32_t* cu_nodes, int32_t N,
                   hipStream_t stream);

/*
 * Bandwidth probes (measurement only, not part of the verification path): the ceilings
 * against which the launches above are read. specdec_probe_read streams `bytes` from `src`
 * once with the statistics launches' access pattern (256-thread workgroups, eight 16-byte
 * non-temporal loads in flight per thread, one 32 KB span per workgroup) and stores into
 * *sink only when the data fold to one particular word. specdec_probe_copy copies `bytes`
 * from `src` to `dst` with non-temporal 16-byte loads and stores, four in flight per thread
 * (the fastest copy shape measured on MI355X). Device pointers, 16-byte aligned, `bytes` a
 * positive multiple of 16,
 * buffers not overlapping; EINVAL otherwise, before anything is enqueued. One launch on
 * `stream`.
 */
int specdec_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
int specdec_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECDEC_H */
