/*
 * attn.h -- C ABI of the MI355X (gfx950) exact scaled-dot-product attention
 * forward library, libattn.so.
 *
 * Operation (every entry point computes the same thing):
 *
 *   O = softmax(scale * Q K^T + mask) V,   LSE = log of the softmax normaliser
 *
 * over tensors laid out as [B, H, N, d].  This is the attention of "Tensor
 * Parallelism with CUDA - Standard Attention" (S = Q K^T / sqrt(d), row-wise
 * softmax, O = P V) with the scale as an argument, and the masked five-step
 * form of "Naive Attention Kernel" (section 1), where the mask here is
 * structural (masked keys get probability exactly 0):
 *
 *   - key padding: per sequence b a valid key length L_b; keys j >= L_b are
 *     masked (the key-side mask of "cuda-reranker");
 *   - causal: key j is visible to query i only when j <= i (equal query and
 *     key lengths, top-left aligned).
 *
 * For each (b, h, i):  S_ij = scale * (q_i . k_j) over visible keys j,
 *   LSE_i = log(sum_j exp(S_ij)),  O_i = sum_j exp(S_ij - LSE_i) v_j.
 * A row with no visible key gets O_i = 0 and LSE_i = -inf.
 *
 * The attn_fwd_gqa* entry points take the general shapes: Q and O
 * [B, H, Nq, d], K and V [B, Hkv, Nk, d], H a multiple of Hkv.  Query head h
 * reads key/value head h / (H / Hkv) (consecutive query heads share one:
 * grouped-query attention; Hkv = 1 is multi-query attention), and queries and
 * keys may differ in length (cross-attention, or new queries against a longer
 * key/value history).  "cuda-reranker" lists cross-attention and
 * grouped-query attention as extensions without defining them; these are the
 * usual readings.  Causal masking is then aligned at the end: key j is
 * visible to query i only when j <= i + (Nk - Nq), so the last query sees
 * every key; with Nq = Nk this is the j <= i above, and rows with
 * i < Nq - Nk see no key.  The self-attention entry points are the case
 * Hkv = H, Nq = Nk = N.
 *
 * Conventions common to all entry points
 * --------------------------------------
 *  dtype    ATTN_F16 (IEEE binary16) or ATTN_BF16 (bfloat16) for Q, K, V and
 *           O.  Arithmetic is fp32 on the GPU (fp16/bf16 matrix-core inputs,
 *           fp32 accumulation); O is rounded to nearest-even into dtype.
 *  layout   Q, K, V, O: contiguous row-major [B, H, N, d] device arrays,
 *           16-byte aligned.  LSE: contiguous fp32 [B, H, N] device array,
 *           4-byte aligned, or NULL when not wanted.
 *  sizes    B, H, N >= 0; d in {32, 64, 128}.  B*H*N == 0 is a no-op.
 *           B*H <= 2^31 - 1 and N <= 2^30.  General shapes: Nq, Nk <= 2^30,
 *           (H / Hkv) * Nq <= 2^30; B*H*Nq == 0 is a no-op, and Nk == 0
 *           gives every row O = 0, LSE = -inf (K and V may then be NULL).
 *  scale    finite and >= 0 (normally 1/sqrt(d)).
 *  key_len  NULL (no padding mask) or a device int32 array [B]; values are
 *           clamped to [0, N] on the device.  K and V rows j >= L_b are never
 *           read, so they may hold anything (including NaN).
 *  stream   a hipStream_t passed as void* (NULL = the null stream).  Work is
 *           enqueued asynchronously; the call does not synchronise.
 *  ownership  the caller owns every buffer.  The library allocates no device
 *           memory, keeps no per-call state, and caches only device
 *           properties.  Calls are reentrant; calls on different streams may
 *           run concurrently.
 *  aliasing O and LSE must not overlap Q, K, V, key_len or each other.
 *  errors   argument errors are returned synchronously before anything is
 *           enqueued; ATTN_ERR_LAUNCH reports a failed kernel launch.  Faults
 *           inside a kernel surface at the caller's next synchronisation.
 *  determinism  identical inputs give bitwise identical outputs.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_F16 = 0,
    ATTN_BF16 = 1
} attn_dtype_t;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,  /* bad size, scale, pointer or aliasing */
    ATTN_ERR_UNSUPPORTED = 2,  /* d not in {32, 64, 128} or unknown dtype */
    ATTN_ERR_MISALIGNED = 3,   /* a pointer is not aligned as required */
    ATTN_ERR_WORKSPACE = 4,    /* workspace missing or too small */
    ATTN_ERR_LAUNCH = 5,       /* the HIP runtime rejected a launch */
    ATTN_ERR_DEVICE = 6        /* no usable gfx950 device is current */
} attn_status_t;

/*
 * attn_fwd -- fused, tiled forward pass.
 *
 * One kernel launch.  Each workgroup owns a tile of query rows of one (b, h),
 * keeps them in registers, streams the visible key/value tiles through LDS,
 * and keeps a running row maximum, running normaliser and rescaled output
 * accumulator (the online-softmax recurrence of "Self-Attention Kernel &
 * Inference Engine from Scratch", section "Online Softmax Formulation"), so
 * the N x N score matrix never reaches device memory.  Key tiles that are
 * wholly masked (past L_b, or after the query tile under causal masking) are
 * skipped (same page, "Engineering Decisions & Trade-offs"; "cuda-reranker",
 * the padding tile skip).
 *
 * Q, K, V: inputs as above.  O: output [B, H, N, d] in dtype.  LSE: optional
 * fp32 output [B, H, N] (natural log).  Returns ATTN_OK or an error code.
 */
attn_status_t attn_fwd(attn_dtype_t dtype,
                       const void *Q, const void *K, const void *V,
                       void *O, float *LSE,
                       int64_t B, int64_t H, int64_t N, int64_t d,
                       float scale, int causal, const int32_t *key_len,
                       void *stream);

/*
 * attn_fwd_gqa -- attn_fwd for the general shapes (see the top of this
 * file): Q [B, H, Nq, d], K and V [B, Hkv, Nk, d], O [B, H, Nq, d], LSE
 * [B, H, Nq] or NULL, key_len [B] (clamped to [0, Nk]) or NULL.
 *
 * One kernel launch.  A workgroup takes query rows of the H / Hkv heads that
 * share a key/value head together (their rows are contiguous in Q and O), so
 * each key/value tile it streams serves all of them.  Returns
 * ATTN_ERR_INVALID_ARG when Hkv does not divide H (or Hkv is 0 with H > 0),
 * otherwise as attn_fwd.  attn_fwd(..., N, ...) is
 * attn_fwd_gqa(..., H, N, N, ...).
 */
attn_status_t attn_fwd_gqa(attn_dtype_t dtype,
                           const void *Q, const void *K, const void *V,
                           void *O, float *LSE,
                           int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk,
                           int64_t d, float scale, int causal, const int32_t *key_len,
                           void *stream);

/*
 * attn_fwd_masked -- attn_fwd_gqa with an additive score mask: the scores
 * become S_ij = scale * (q_i . k_j) + mask_ij before the softmax, the
 * five-step form of "Naive Attention Kernel" (section 1: scores, scale, add
 * the mask, softmax, product with V) with its float mask.
 *
 * mask: device fp32 array, 4-byte aligned, element (b, h, i, j) at
 * b * mask_stride_b + h * mask_stride_h + i * Nk + j (strides in elements,
 * >= 0; rows of one (b, h) are contiguous).  Strides of 0 share one
 * [Nq, Nk] mask (the pages' [S, S]) across batch and heads.  One batch's
 * part, ((H - 1) * mask_stride_h + Nq * Nk) * 4 bytes, must be below 2 GiB.
 * An element of -inf removes that key as the structural masks do; a row all
 * of whose visible keys are -inf gets O = 0 and LSE = -inf.  +inf or NaN
 * elements give undefined results.  causal and key_len still apply.  The
 * mask is read, never written; it must not overlap O or LSE.
 *
 * One kernel launch (the streaming kernel for every Nk).  Returns
 * ATTN_ERR_INVALID_ARG for a NULL mask, negative strides, an oversized mask
 * or an overlap, ATTN_ERR_MISALIGNED for a misaligned mask, otherwise as
 * attn_fwd_gqa.
 */
attn_status_t attn_fwd_masked(attn_dtype_t dtype,
                              const void *Q, const void *K, const void *V,
                              void *O, float *LSE,
                              int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk,
                              int64_t d, float scale, int causal, const int32_t *key_len,
                              const float *mask, int64_t mask_stride_b, int64_t mask_stride_h,
                              void *stream);

/*
 * attn_fwd_naive -- unfused baseline that materialises scores and
 * probabilities ("Naive Attention Kernel", sections 1 and 3; "Tensor
 * Parallelism with CUDA - Standard Attention", sections "Why This
 * Ordering?" and "The Naive HBM Algorithm").
 *
 * Three launches per group of heads: scores S = scale Q K^T (fp32, masked
 * entries -inf) written to the workspace; a row-wise softmax in place
 * (max, exponential sum, normalise; also writes LSE); then O = P V.
 * workspace: device memory of workspace_bytes, 16-byte aligned, owned by the
 * caller and overwritten.  It must hold at least one head's fp32 N x N matrix
 * (attn_fwd_naive_workspace_bytes(1, 1, N)); with less than
 * attn_fwd_naive_workspace_bytes(B, H, N) the heads are processed in groups.
 * Returns ATTN_ERR_WORKSPACE when the workspace is NULL or too small.
 */
attn_status_t attn_fwd_naive(attn_dtype_t dtype,
                             const void *Q, const void *K, const void *V,
                             void *O, float *LSE,
                             int64_t B, int64_t H, int64_t N, int64_t d,
                             float scale, int causal, const int32_t *key_len,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/* Bytes of workspace that let attn_fwd_naive process all B*H heads at once:
 * B * H * N * N * 4.  Returns 0 for negative sizes or on overflow. */
size_t attn_fwd_naive_workspace_bytes(int64_t B, int64_t H, int64_t N);

/*
 * attn_fwd_splitkv -- the fused forward with each row's key range cut into
 * splits, for shapes whose (b, h, 256-row query tile) work items are too
 * few to occupy the GPU (few heads, long sequences).
 *
 * The visible keys of every row are divided into up to n_splits ranges of
 * whole 64-key tiles; workgroups compute each range as attn_fwd does and
 * write its normalised partial output O_s and log-sum-exp LSE_s (fp32) to
 * the workspace; a second launch merges them per row with the identity of
 * "Self-Attention Kernel & Inference Engine from Scratch" ("Online Softmax
 * Formulation") applied to whole blocks: LSE = log sum_s exp(LSE_s) and
 * O = sum_s exp(LSE_s - LSE) O_s.  The result equals attn_fwd's up to
 * rounding (O is rounded to dtype once, after the merge).
 *
 * Arguments as attn_fwd, plus: n_splits >= 1 (at most 4096; splits beyond
 * the key tiles a row has are empty and cost nothing); workspace: device
 * memory of at least attn_fwd_splitkv_workspace_bytes(B, H, N, d, n_splits)
 * bytes, 16-byte aligned, owned by the caller, overwritten, and overlapping
 * no tensor.  Returns ATTN_ERR_WORKSPACE when it is NULL or too small,
 * ATTN_ERR_INVALID_ARG for n_splits out of range or an overlap, otherwise
 * as attn_fwd.  Two launches on stream, asynchronous.
 */
attn_status_t attn_fwd_splitkv(attn_dtype_t dtype,
                               const void *Q, const void *K, const void *V,
                               void *O, float *LSE,
                               int64_t B, int64_t H, int64_t N, int64_t d,
                               float scale, int causal, const int32_t *key_len,
                               int64_t n_splits, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * attn_fwd_gqa_splitkv -- attn_fwd_splitkv for the general shapes of
 * attn_fwd_gqa: the key range [0, Nk) is cut into up to n_splits runs of
 * whole 64-key tiles.  The workspace must hold
 * attn_fwd_splitkv_workspace_bytes(B, H, Nq, d, n_splits) bytes (the
 * partials are per query row).  Errors as attn_fwd_gqa and attn_fwd_splitkv.
 */
attn_status_t attn_fwd_gqa_splitkv(attn_dtype_t dtype,
                                   const void *Q, const void *K, const void *V,
                                   void *O, float *LSE,
                                   int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk,
                                   int64_t d, float scale, int causal, const int32_t *key_len,
                                   int64_t n_splits, void *workspace, size_t workspace_bytes,
                                   void *stream);

/*
 * attn_fwd_gqa_splitkv_static -- attn_fwd_gqa_splitkv without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid it).  The split partials go to a scratch array inside the
 * library of ATTN_STATIC_SCRATCH_BYTES (64 MiB) per device, which every
 * device the library runs on holds until the process ends.
 *
 * Arguments, results and errors as attn_fwd_gqa_splitkv; the caller still
 * owns and passes Q, K, V, O, LSE and key_len.  Returns ATTN_ERR_WORKSPACE
 * when attn_fwd_splitkv_workspace_bytes(B, H, Nq, d, n_splits) exceeds
 * ATTN_STATIC_SCRATCH_BYTES (use fewer splits, or attn_fwd_gqa_splitkv with
 * a workspace), ATTN_ERR_DEVICE when the scratch address cannot be looked
 * up.  The first call on a device looks the address up once.  All calls on
 * one device share the one scratch array: calls that overlap in time on
 * one device (different streams, or host threads without ordering) race
 * and give wrong results; calls ordered on one stream are safe.  Nothing in
 * the scratch needs to start at zero (every partial read is written first
 * in the same call).
 */
#define ATTN_STATIC_SCRATCH_BYTES (64u << 20)
attn_status_t attn_fwd_gqa_splitkv_static(attn_dtype_t dtype,
                                          const void *Q, const void *K, const void *V,
                                          void *O, float *LSE,
                                          int64_t B, int64_t H, int64_t Hkv, int64_t Nq,
                                          int64_t Nk, int64_t d, float scale, int causal,
                                          const int32_t *key_len, int64_t n_splits,
                                          void *stream);

/*
 * attn_fwd_masked_splitkv -- attn_fwd_masked over up to n_splits key
 * ranges, merged as attn_fwd_splitkv does.  Workspace and errors as
 * attn_fwd_gqa_splitkv and attn_fwd_masked; the workspace must not overlap
 * the mask either.
 */
attn_status_t attn_fwd_masked_splitkv(attn_dtype_t dtype,
                                      const void *Q, const void *K, const void *V,
                                      void *O, float *LSE,
                                      int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk,
                                      int64_t d, float scale, int causal,
                                      const int32_t *key_len, const float *mask,
                                      int64_t mask_stride_b, int64_t mask_stride_h,
                                      int64_t n_splits, void *workspace, size_t workspace_bytes,
                                      void *stream);

/* Workspace bytes attn_fwd_splitkv needs: n_splits * B * H * N * (d + 1) * 4
 * (N = Nq for attn_fwd_gqa_splitkv).  Returns 0 for sizes out of range or on
 * overflow. */
size_t attn_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d,
                                        int64_t n_splits);

/* A split count that lets the work items of (dtype, B, H, N, d, causal)
 * occupy the compute units of the current device: 1 when the unsplit kernel
 * already fills its resident workgroups, else the largest count (at most
 * half the key tiles) whose workgroups with work all fit in one resident
 * round.  Under the causal mask an early query tile sees few keys, so most
 * of its later splits have no work and are not launched.  Returns 1 on any
 * error. */
int64_t attn_fwd_splitkv_default_splits(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N,
                                        int64_t d, int causal);

/* The same for the general shapes of attn_fwd_gqa_splitkv: the work items
 * are 256-row tiles of the (H / Hkv) * Nq query rows of each of the B * Hkv
 * key/value heads, and a split keeps at least two of the Nk keys' tiles.
 * Returns 1 on any error. */
int64_t attn_fwd_gqa_splitkv_default_splits(attn_dtype_t dtype, int64_t B, int64_t H,
                                            int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                                            int causal);

/* Static, NUL-terminated description of a status code. */
const char *attn_status_string(attn_status_t status);

/*
 * Name of the kernel instance attn_fwd launches for these arguments (for
 * profilers), written into buf (NUL-terminated, truncated to buf_len).  N is
 * the key length (Nk for attn_fwd_gqa, which chooses its kernel the same
 * way).
 * Returns the same status attn_fwd would return for an argument error,
 * else ATTN_OK.  Touches no device state.
 */
attn_status_t attn_fwd_kernel_name(attn_dtype_t dtype, int64_t d, int64_t N,
                                   int causal, int has_key_len,
                                   char *buf, size_t buf_len);

/*
 * Name of the kernel instance the general entry points launch for these
 * arguments (for profilers): attn_fwd_gqa (masked = 0, n_splits = 0),
 * attn_fwd_gqa_splitkv (n_splits > 0) or the masked forms (masked != 0);
 * with splits the merge kernel runs after it.  Written into buf
 * (NUL-terminated, truncated to buf_len).  Returns ATTN_ERR_UNSUPPORTED or
 * ATTN_ERR_INVALID_ARG for arguments those entry points reject, else
 * ATTN_OK.  Touches no device state.
 */
attn_status_t attn_fwd_gqa_kernel_name(attn_dtype_t dtype, int64_t d, int64_t H, int64_t Hkv,
                                       int64_t Nq, int64_t Nk, int causal, int masked,
                                       int64_t n_splits, char *buf, size_t buf_len);

/* Library ABI version (major * 100 + minor). */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
