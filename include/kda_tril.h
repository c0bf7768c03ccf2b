/*
 * kda_tril.h - C ABI of the MI355X (gfx950) KDA prefill chunk solver.
 *
 * Operation (LightLLM PR #1703, "perf(kda): parallelize diagonal solves in
 * Prefill", PR description, method paragraph): the sequence is cut into
 * 64-token chunks; for every chunk and every head the solver returns
 *
 *     X = (I + A)^-1,
 *
 * where A is the 64 x 64 strictly-lower-triangular intra-chunk matrix of
 * that head. The page's scheme inverts the four 16 x 16 diagonal blocks of
 * I + A independently and then merges them into the 64 x 64 inverse, keeping
 * the inverse tiles in FP32 until the final store (same PR, commit summary).
 * This library follows that scheme on CDNA4: every kernel computes in FP32;
 * inputs and outputs may be FP32, bfloat16 or binary16.
 *
 * Layout (both A and X, contiguous, row-major, 64 columns innermost):
 *   packed: [T, H, 64]; requests are concatenated along T and described by
 *           cu_seqlens. Chunks restart at every request's first token, so the
 *           last chunk of a request may hold fewer than 64 valid rows (L).
 *   dense:  [B, T, H, 64]; every batch element is one request of T tokens.
 * Element (token t, head h, column j) of A is entry (t - chunk_start, j) of
 * that chunk-head's matrix. Entries on or above the diagonal, and columns
 * >= L of a partial chunk, are ignored (never used in arithmetic, so NaN or
 * Inf there cannot reach X). For each valid row i < L of a chunk, X is
 * written in full: X[i][i] = 1, X[i][j] = 0 for j > i (including j >= L),
 * and the inverse below the diagonal. Rows that belong to no chunk (packed
 * tokens past cu_seqlens[num_seqs]) are not written.
 *
 * Memory: every pointer argument is DEVICE memory unless marked (host). The
 * caller owns A, X, cu_seqlens, chunk_indices and the workspace. The library
 * allocates nothing, frees nothing, keeps no pointer after a call returns,
 * never synchronises and never copies between host and device: every call
 * only enqueues kernels on `stream` and returns. A and X must not overlap,
 * and A, X and the workspace must be 16-byte aligned (KDA_ERR_INVALID_ARG
 * otherwise).
 *
 * Errors: plain status codes; nothing is thrown across the ABI. Problems that
 * the host can see (null pointers with nonzero sizes, H <= 0, unknown dtype,
 * forced SPLIT with too little workspace; KDA_ERR_UNSUPPORTED for sizes past
 * the int32 token range, H > 4096, or chunk slots x H past 2^26 - 4, the
 * wavefronts one launch can hold) are reported before any launch.
 * Device-side cu_seqlens are not validated (that would need a
 * synchronisation): they must start at 0, be non-decreasing and end at
 * <= total_tokens; kernels clamp every row index to [0, total_tokens) so a
 * bad cu_seqlens cannot write outside X.
 * KDA_ERR_HIP reports a failed launch (hipGetLastError after the launch).
 * Zero tokens, zero batch or zero requests is a no-op returning KDA_OK.
 *
 * Thread safety: stateless. Concurrent calls on different streams need
 * different workspaces.
 */
#ifndef KDA_TRIL_H
#define KDA_TRIL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of A or X. BF16 is bfloat16 (8 exponent, 7 mantissa bits),
 * F16 is IEEE binary16 (5 exponent, 10 mantissa bits); a 16-bit X is the
 * round-to-nearest-even of the FP32 result (binary16 overflows to +-inf past
 * 65504 and keeps subnormals). 16-bit inputs are widened to FP32 exactly. */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1, KDA_F16 = 2 } kda_dtype;

/* Kernel plan.
 *   AUTO   - pick SPLIT when it is eligible and the tuned rule prefers it,
 *            else FUSED (same PR, PR description: splitting is selected by
 *            the FP32 workspace budget and a minimum input length; commit
 *            summary: by chunk occupancy, to bound scratch). An ineligible
 *            SPLIT silently falls back to FUSED.
 *   FUSED  - one kernel: diagonal inverses and merges of a chunk-head in one
 *            wavefront (small launches: two wavefronts, each merging two
 *            block columns), merge products on the FP32 matrix cores
 *            (MFMA); every form gives the same bits.
 *   SPLIT  - two kernels: the diagonal kernel writes the four FP32 16 x 16
 *            inverse tiles of every chunk-head to the workspace, the merge
 *            kernel reads them back with A and writes X. Needs workspace of
 *            kda_tril_inv_workspace_size bytes; it must not exceed the FP32
 *            input size (T x H x 64 x 4 bytes), i.e. mean chunk occupancy
 *            T / num_chunks >= 16.
 *   FUSED_VALU - like FUSED, but the merge products run as FP32 vector FMAs
 *            instead of matrix-core instructions (the other precision mode:
 *            both are IEEE FP32 products and sums, in different orders). */
typedef enum {
    KDA_ALGO_AUTO = 0,
    KDA_ALGO_FUSED = 1,
    KDA_ALGO_SPLIT = 2,
    KDA_ALGO_FUSED_VALU = 3
} kda_algo;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = -1,
    KDA_ERR_UNSUPPORTED = -2,
    KDA_ERR_WORKSPACE = -3,
    KDA_ERR_HIP = -4
} kda_status;

/*
 * Workspace query and plan choice. Host only: never touches the GPU.
 *   total_tokens  T (packed) or B * T (dense), >= 0.
 *   num_seqs      number of requests (packed) or B (dense), >= 0.
 *   num_chunks    exact number of chunks if known, else 0: the bound
 *                 floor(total_tokens / 64) + num_seqs is then used.
 *   num_heads     H > 0.
 *   algo          requested plan.
 *   bytes (host out)   workspace bytes the call with this plan needs
 *                      (0 for FUSED / FUSED_VALU).
 *   chosen (host out, nullable)  plan that a call with a workspace of
 *                      *bytes bytes would run (AUTO resolved).
 * The SPLIT workspace is 4 tiles x 16 x 16 FP32 = 4096 bytes per chunk-head.
 * Returns KDA_ERR_WORKSPACE when SPLIT is forced but ineligible (its scratch
 * would exceed the FP32 input size). A call that runs SPLIT returns
 * KDA_ERR_INVALID_ARG when the workspace is not 16-byte aligned or overlaps A
 * or X.
 */
kda_status kda_tril_inv_workspace_size(int64_t total_tokens, int64_t num_seqs,
                                       int64_t num_chunks, int32_t num_heads, kda_algo algo,
                                       size_t *bytes, kda_algo *chosen);

/*
 * Dense batch: A [B, T, H, 64] of a_dtype, X [B, T, H, 64] of x_dtype.
 * B * T must fit in int32. workspace may be NULL when workspace_bytes is 0.
 */
kda_status kda_tril_inv_dense(const void *A, kda_dtype a_dtype, void *X, kda_dtype x_dtype,
                              int64_t B, int64_t T, int32_t H, void *workspace,
                              size_t workspace_bytes, kda_algo algo, hipStream_t stream);

/*
 * Packed varlen batch: A [total_tokens, H, 64], X [total_tokens, H, 64].
 *   cu_seqlens     int32 [num_seqs + 1] (device): 0 = cu[0] <= cu[1] <= ...
 *                  <= cu[num_seqs] <= total_tokens.
 *   chunk_indices  optional int32 [num_chunks][2] (device) of (request,
 *                  chunk-within-request) pairs in packed order, as a caller
 *                  that reuses one map across layers would keep it; NULL to
 *                  let the kernels resolve chunks from cu_seqlens on the
 *                  device (grid sized by the bound floor(T/64) + num_seqs).
 *                  The device scan costs each chunk one dependent memory
 *                  round trip per 64 requests before it, so with hundreds of
 *                  requests a map is much faster (64 heads, 2,000 requests of
 *                  1-20 tokens on MI355X: 126 us with a map, 301 us without).
 *   num_chunks     length of chunk_indices (0 when it is NULL).
 */
kda_status kda_tril_inv_packed(const void *A, kda_dtype a_dtype, void *X, kda_dtype x_dtype,
                               const int32_t *cu_seqlens, int64_t num_seqs,
                               int64_t total_tokens, int32_t H, const int32_t *chunk_indices,
                               int64_t num_chunks, void *workspace, size_t workspace_bytes,
                               kda_algo algo, hipStream_t stream);

/*
 * The shared chunk solver's other branches (same PR, PR description: the
 * 64-token kernel is the 64-token branch of a solver shared across chunk
 * sizes). chunk_size C is 16, 32 or 64; A and X are [B, T, H, C] (dense) or
 * [total_tokens, H, C] (packed), every chunk-head matrix is C x C, chunks of
 * C tokens restart at every request's first token, and chunk_indices (if
 * given) pairs count chunks of C tokens. Everything else (layout of a row,
 * ignored entries, full-row output, dtypes, ownership, errors) is as above.
 *   C = 64       identical to kda_tril_inv_dense / kda_tril_inv_packed.
 *   C = 16, 32   one kernel: the 16-token branch is the diagonal solve alone,
 *                the 32-token branch two diagonal solves and one merge on the
 *                matrix cores. Only AUTO and FUSED are accepted (SPLIT and
 *                FUSED_VALU return KDA_ERR_UNSUPPORTED); no workspace is used
 *                (pass NULL, 0).
 * Any other chunk_size returns KDA_ERR_INVALID_ARG.
 */
kda_status kda_tril_inv_dense_chunk(const void *A, kda_dtype a_dtype, void *X,
                                    kda_dtype x_dtype, int64_t B, int64_t T, int32_t H,
                                    int32_t chunk_size, void *workspace,
                                    size_t workspace_bytes, kda_algo algo, hipStream_t stream);

kda_status kda_tril_inv_packed_chunk(const void *A, kda_dtype a_dtype, void *X,
                                     kda_dtype x_dtype, const int32_t *cu_seqlens,
                                     int64_t num_seqs, int64_t total_tokens, int32_t H,
                                     int32_t chunk_size, const int32_t *chunk_indices,
                                     int64_t num_chunks, void *workspace,
                                     size_t workspace_bytes, kda_algo algo,
                                     hipStream_t stream);

/*
 * The matrix built inside the solver. KDA prefill hands the 64-token branch
 * (same PR, PR description) its delta-rule intra-chunk matrix; for tokens
 * i > j of one 64-token chunk and one head
 *
 *     A[i][j] = -beta_i * sum_d k[i][d] * k[j][d] * exp(g[i][d] - g[j][d]),
 *
 * and A[i][j] = 0 for j >= i. These calls take the keys, decays and write
 * strengths instead of A:
 *   k      [rows, H, K] of k_dtype: key rows, K channels; K a multiple of 16,
 *          16 <= K <= 256 (other K: KDA_ERR_UNSUPPORTED).
 *   g      [rows, H, K] FP32: cumulative log-decay of each channel,
 *          non-increasing along a chunk (log-gates <= 0, as in KDA). Only
 *          differences within a chunk enter, so g may restart at every chunk
 *          or run over a whole request; each is taken in FP32 before it is
 *          scaled, and evaluated as exp(g_i - g_ri) exp(g_ri - g_rj)
 *          exp(g_rj - g_j) with r_i, r_j the first rows of the 16-row blocks of
 *          i and j. Domain: a channel may fall by up to 5.4 per token for a
 *          whole chunk (tested to the fp32 bounds, alone, mixed with slow
 *          channels and in partial chunks). Past a fall of about 87 over 16
 *          consecutive tokens (5.45 per token) the factor between adjacent
 *          16-token blocks drops below 2^-126 and is flushed to 0, so entries
 *          of A between those blocks lose that channel's term.
 *   beta   [rows, H] of k_dtype: write strengths.
 * rows = total_tokens (packed, with cu_seqlens and optional chunk_indices as
 * for kda_tril_inv_packed) or B * T (dense, [B, T, H, ...]). k, g and the
 * output must be 16-byte aligned, beta aligned to its element size, and the
 * output must not overlap the inputs. All arithmetic is FP32 (k and beta
 * widened exactly); A is never rounded before the inverse.
 *
 *   kda_kkt_tril_inv_*  X = (I + A)^-1, [rows, H, 64] of x_dtype, written as
 *                       kda_tril_inv_* writes it. A never goes to memory.
 *   kda_kkt_*           A itself, [rows, H, 64] of a_dtype: every valid row
 *                       in full, exact zeros on and above the diagonal and in
 *                       columns >= L (the input of kda_tril_inv_*).
 * No workspace; the fused/split plans do not apply.
 */
kda_status kda_kkt_tril_inv_packed(const void *k, const float *g, const void *beta,
                                   kda_dtype k_dtype, void *X, kda_dtype x_dtype,
                                   const int32_t *cu_seqlens, int64_t num_seqs,
                                   int64_t total_tokens, int32_t H, int32_t K,
                                   const int32_t *chunk_indices, int64_t num_chunks,
                                   hipStream_t stream);

kda_status kda_kkt_tril_inv_dense(const void *k, const float *g, const void *beta,
                                  kda_dtype k_dtype, void *X, kda_dtype x_dtype, int64_t B,
                                  int64_t T, int32_t H, int32_t K, hipStream_t stream);

kda_status kda_kkt_packed(const void *k, const float *g, const void *beta, kda_dtype k_dtype,
                          void *A, kda_dtype a_dtype, const int32_t *cu_seqlens,
                          int64_t num_seqs, int64_t total_tokens, int32_t H, int32_t K,
                          const int32_t *chunk_indices, int64_t num_chunks,
                          hipStream_t stream);

kda_status kda_kkt_dense(const void *k, const float *g, const void *beta, kda_dtype k_dtype,
                         void *A, kda_dtype a_dtype, int64_t B, int64_t T, int32_t H, int32_t K,
                         hipStream_t stream);

/*
 * Fused KDA decode core: one decode step (one new token per sequence) of
 * the causal convolution with its rolling state, the KDA recurrent update and
 * gated RMSNorm, in one kernel (tokenspeed PR #1086, "perf(kimi3): fuse KDA
 * decode core", PR description; its test plan names convolution, paged-state,
 * padding and gated-RMSNorm references). The page gives no formulas; per
 * sequence b and head h (head dim d = head_dim, conv width W = conv_width)
 * the step is:
 *   for p in (q, k, v): y_p = silu(sum_{w<W} conv_w[p][w] * win_p[w]), where
 *       win_p = (the W-1 previous inputs, oldest first; then the new x_p);
 *       the window then drops its oldest entry and appends x_p
 *   q = y_q / sqrt(|y_q|^2 + eps_l2) / sqrt(d),  k = y_k / sqrt(|y_k|^2 + eps_l2),  v = y_v
 *   S = diag(exp(g)) S;  u = beta * (v - S^T k);  S = S + k u^T;  o = S^T q
 *   out = o / sqrt(mean(o^2) + eps_norm) * norm_w * sigmoid(z)
 * with S the d x d FP32 state (key rows, value columns). All arithmetic FP32.
 *
 *   qkv         [B, 3, H, d] of in_dtype: the new token's q, k, v before the
 *               convolution.
 *   z           [B, H, d] of in_dtype: output gate (before the sigmoid).
 *   g           [B, H, d] FP32: log-decay of each key channel (<= 0 in KDA).
 *   beta        [B, H] FP32: write strength.
 *   norm_w      [d] FP32: RMSNorm weight.
 *   conv_w      [3, W, H, d] FP32: depthwise taps, tap-major.
 *   slot        [B] int32 (device): the state slot of each sequence. A slot
 *               < 0 or >= num_slots marks a padding entry: its output is 0
 *               and no state is touched. Slots of non-padding entries must
 *               be distinct (entries sharing a slot race).
 *   state       [num_slots, H, d, d] FP32, updated in place (16-byte aligned).
 *   conv_state  [num_slots, 3, H, W - 1, d] FP32, updated in place.
 *   out         [B, H, d] of out_dtype.
 * head_dim must be 128, 2 <= conv_width <= 4 and B x H < 2^24 (one workgroup
 * of 256 threads per sequence and head), else KDA_ERR_UNSUPPORTED;
 * eps_l2, eps_norm must be finite and >= 0. out must not overlap the state
 * pools. B = 0 is a no-op.
 */
kda_status kda_decode_step(const void *qkv, const void *z, kda_dtype in_dtype, const float *g,
                           const float *beta, const float *norm_w, const float *conv_w,
                           const int32_t *slot, float *state, float *conv_state,
                           int64_t num_slots, void *out, kda_dtype out_dtype, int64_t B,
                           int32_t H, int32_t head_dim, int32_t conv_width, float eps_l2,
                           float eps_norm, hipStream_t stream);

/*
 * Allocation-free form of kda_tril_inv_packed, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It always runs the SPLIT plan, with the
 * workspace taken from a scratch array the library keeps in device memory:
 * KDA_TRIL_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU the library runs on,
 * held until the process ends, found on a device's first call. The call
 * itself allocates and frees nothing.
 *   Arguments, layout, ownership of A, X, cu_seqlens and chunk_indices, and
 *   results: as kda_tril_inv_packed with algo = KDA_ALGO_SPLIT (X bit for bit
 *   equal to it).
 *   Size limit: the split workspace, 4096 bytes x H x chunk slots (num_chunks
 *   when chunk_indices is given, else floor(total_tokens / 64) + num_seqs),
 *   must not exceed KDA_TRIL_NOALLOC_SCRATCH_BYTES (16,384 chunk-heads), and
 *   the split plan must be eligible (workspace <= FP32 input size); otherwise
 *   KDA_ERR_WORKSPACE before any device call.
 *   Concurrency: every call on one GPU uses that GPU's one array. Calls in
 *   order on one stream are safe; calls that overlap in time on one GPU (on
 *   different streams or from different host threads) race on it and give
 *   wrong results. Nothing in the array needs to start at zero: each call
 *   writes every tile it later reads.
 *   KDA_ERR_HIP: the device address of the array could not be found, or a
 *   launch failed.
 */
#define KDA_TRIL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_tril_inv_packed_noalloc(const void *A, kda_dtype a_dtype, void *X,
                                       kda_dtype x_dtype, const int32_t *cu_seqlens,
                                       int64_t num_seqs, int64_t total_tokens, int32_t H,
                                       const int32_t *chunk_indices, int64_t num_chunks,
                                       hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char *kda_status_string(kda_status s);

/* Plan AUTO would choose for a problem with these sizes and workspace
 * (host only; same rule the calls apply). The rule follows LightLLM PR #1703,
 * "perf(kda): parallelize diagonal solves in Prefill": the PR description
 * selects splitting by an FP32 workspace budget (scratch at most the FP32
 * input size) and a minimum input length; the commit summary selects it by
 * chunk occupancy, to bound scratch. SPLIT is chosen when the scratch of
 * 4096 bytes per chunk-head fits both the budget and workspace_bytes and
 * total_tokens reaches the minimum length, else FUSED. The minimum length is
 * the fused/split crossover measured on MI355X (none was found, so by default
 * AUTO never splits); two environment variables, read on every call, tune the
 * rule: KDA_TRIL_SPLIT_MIN_TOKENS sets the minimum length, and KDA_TRIL_ALGO
 * (fused, split or fused_valu) replaces the rule's choice for calls that ask
 * for AUTO (an ineligible split still falls back to FUSED). */
kda_algo kda_tril_auto_plan(int64_t total_tokens, int64_t num_chunks, int32_t num_heads,
                            size_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* KDA_TRIL_H */
