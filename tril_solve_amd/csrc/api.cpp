// C ABI of the KDA chunk solver (declared in include/kda_tril.h).
//
// Validates arguments on the host, resolves the plan, fills the kernels'
// Problem and enqueues them on the caller's stream. Never allocates, copies
// or synchronises.
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include "kda_tril.h"
#include "plan.h"
#include "tril_launch.h"

using namespace kda;

namespace {

// Token counts are int32 inside the kernels; keep room for +64 arithmetic.
constexpr int64_t kMaxTokens = (int64_t)INT32_MAX - 64;
// Heads: keeps every byte offset inside one chunk's rows (64 rows of H x 64
// elements) below 2^31, which the kernels' 32-bit buffer offsets rely on.
constexpr int32_t kMaxHeads = 4096;
// Key channels of the "build A from keys" path (64 rows x H x K elements of
// one chunk also stay below 2^31 bytes).
constexpr int32_t kMaxKeyDim = 256;

bool valid_dtype(kda_dtype d) { return d == KDA_F32 || d == KDA_BF16 || d == KDA_F16; }
bool valid_algo(kda_algo a) { return a >= KDA_ALGO_AUTO && a <= KDA_ALGO_FUSED_VALU; }
bool valid_chunk(int32_t c) { return c == 16 || c == 32 || c == 64; }
size_t dtype_bytes(kda_dtype d) { return d == KDA_F32 ? 4 : 2; }

// One wavefront of 64 lanes per chunk slot and head, in workgroups of up to
// four wavefronts: the launch, rounded up to whole workgroups, must stay
// below 2^32 threads.
bool grid_fits(int64_t slots, int32_t H) {
    const int64_t waves = slots * (int64_t)H;
    return slots <= kMaxTokens && (waves + 3) / 4 * 256 <= (int64_t)UINT32_MAX;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

kda_status run(const Problem &p, kda_algo algo, int a_dt, int x_dt, hipStream_t stream) {
    hipError_t e = hipSuccess;
    switch (algo) {
        case KDA_ALGO_FUSED:
            e = launch_fused_mfma(p, a_dt, x_dt, stream);
            break;
        case KDA_ALGO_SPLIT:
            e = launch_split(p, a_dt, x_dt, stream);
            break;
        case KDA_ALGO_FUSED_VALU:
            e = launch_fused_valu(p, a_dt, x_dt, stream);
            break;
        default:
            return KDA_ERR_INVALID_ARG;
    }
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Checks shared by both layouts; rows = tokens covered by A and X, C = chunk
// size (row length of A and X).
kda_status check_common(const void *A, kda_dtype a_dtype, const void *X, kda_dtype x_dtype,
                        int64_t rows, int32_t H, int32_t C, kda_algo algo) {
    if (!valid_dtype(a_dtype) || !valid_dtype(x_dtype) || !valid_algo(algo) || !valid_chunk(C))
        return KDA_ERR_INVALID_ARG;
    if (H <= 0) return KDA_ERR_INVALID_ARG;
    if (rows > kMaxTokens || H > kMaxHeads) return KDA_ERR_UNSUPPORTED;
    // the 16- and 32-token branches have a single kernel (no split, no
    // second merge engine)
    if (C != 64 && algo != KDA_ALGO_AUTO && algo != KDA_ALGO_FUSED) return KDA_ERR_UNSUPPORTED;
    if (rows == 0) return KDA_OK;
    if (A == nullptr || X == nullptr) return KDA_ERR_INVALID_ARG;
    if (!aligned16(A) || !aligned16(X)) return KDA_ERR_INVALID_ARG;
    const size_t elems = (size_t)rows * (size_t)H * (size_t)C;
    if (overlap(A, elems * dtype_bytes(a_dtype), X, elems * dtype_bytes(x_dtype)))
        return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

// Plan of a call. A SPLIT plan's workspace must be aligned and must not
// overlap A or X: the diagonal kernel writes it before the merge kernel reads
// A, so an overlap would corrupt the input with no error.
kda_status plan_call(int64_t rows, int64_t slots, int32_t H, int32_t C, kda_algo algo,
                     const void *A, size_t a_bytes, const void *X, size_t x_bytes,
                     void *workspace, size_t workspace_bytes, kda_algo *chosen) {
    if (C != 64) {  // one kernel per small chunk size, no workspace
        *chosen = KDA_ALGO_FUSED;
        return KDA_OK;
    }
    const size_t offered = workspace ? workspace_bytes : 0;
    kda_status st = resolve_plan(rows, slots, H, algo, offered, chosen);
    if (st != KDA_OK) return st;
    if (*chosen == KDA_ALGO_SPLIT) {
        const size_t need = (size_t)split_workspace_bytes(slots, H);
        if (!aligned16(workspace)) return KDA_ERR_INVALID_ARG;
        if (overlap(workspace, need, A, a_bytes) || overlap(workspace, need, X, x_bytes))
            return KDA_ERR_INVALID_ARG;
    }
    return KDA_OK;
}

size_t tensor_bytes(int64_t rows, int32_t H, int32_t C, kda_dtype d) {
    return (size_t)rows * (size_t)H * (size_t)C * dtype_bytes(d);
}

kda_status dense_call(const void *A, kda_dtype a_dtype, void *X, kda_dtype x_dtype, int64_t B,
                      int64_t T, int32_t H, int32_t C, void *workspace, size_t workspace_bytes,
                      kda_algo algo, hipStream_t stream) {
    if (B < 0 || T < 0) return KDA_ERR_INVALID_ARG;
    if (B > 0 && T > kMaxTokens / B) return KDA_ERR_UNSUPPORTED;
    const int64_t rows = B * T;
    kda_status st = check_common(A, a_dtype, X, x_dtype, rows, H, C, algo);
    if (st != KDA_OK || rows == 0) return st;
    const int64_t slots = B * ((T + C - 1) / C);
    if (!grid_fits(slots, H)) return KDA_ERR_UNSUPPORTED;
    kda_algo chosen = KDA_ALGO_FUSED;
    st = plan_call(rows, slots, H, C, algo, A, tensor_bytes(rows, H, C, a_dtype), X,
                   tensor_bytes(rows, H, C, x_dtype), workspace, workspace_bytes, &chosen);
    if (st != KDA_OK) return st;
    Problem p;
    memset(&p, 0, sizeof(p));
    p.A = A;
    p.X = X;
    p.ws = static_cast<float *>(workspace);
    p.num_seqs = (int32_t)B;
    p.seq_len = (int32_t)T;
    p.total_tokens = (int32_t)rows;
    p.heads = H;
    p.slots = (int32_t)slots;
    if (C != 64)
        return launch_small(p, C, (int)a_dtype, (int)x_dtype, stream) == hipSuccess ? KDA_OK
                                                                                   : KDA_ERR_HIP;
    return run(p, chosen, (int)a_dtype, (int)x_dtype, stream);
}

kda_status packed_call(const void *A, kda_dtype a_dtype, void *X, kda_dtype x_dtype,
                       const int32_t *cu_seqlens, int64_t num_seqs, int64_t total_tokens,
                       int32_t H, int32_t C, const int32_t *chunk_indices, int64_t num_chunks,
                       void *workspace, size_t workspace_bytes, kda_algo algo,
                       hipStream_t stream) {
    if (num_seqs < 0 || total_tokens < 0 || num_chunks < 0) return KDA_ERR_INVALID_ARG;
    if ((chunk_indices == nullptr) != (num_chunks == 0)) return KDA_ERR_INVALID_ARG;
    if (num_seqs > kMaxTokens || num_chunks > kMaxTokens) return KDA_ERR_UNSUPPORTED;
    kda_status st = check_common(A, a_dtype, X, x_dtype, total_tokens, H, C, algo);
    if (st != KDA_OK) return st;
    if (total_tokens == 0 || num_seqs == 0) return KDA_OK;
    if (cu_seqlens == nullptr) return KDA_ERR_INVALID_ARG;
    const int64_t slots = chunk_slots(total_tokens, num_seqs, num_chunks, C);
    if (!grid_fits(slots, H)) return KDA_ERR_UNSUPPORTED;
    kda_algo chosen = KDA_ALGO_FUSED;
    st = plan_call(total_tokens, slots, H, C, algo, A, tensor_bytes(total_tokens, H, C, a_dtype),
                   X, tensor_bytes(total_tokens, H, C, x_dtype), workspace, workspace_bytes,
                   &chosen);
    if (st != KDA_OK) return st;
    Problem p;
    memset(&p, 0, sizeof(p));
    p.A = A;
    p.X = X;
    p.cu = cu_seqlens;
    p.cmap = chunk_indices;
    p.ws = static_cast<float *>(workspace);
    p.num_seqs = (int32_t)num_seqs;
    p.total_tokens = (int32_t)total_tokens;
    p.heads = H;
    p.slots = (int32_t)slots;
    if (C != 64)
        return launch_small(p, C, (int)a_dtype, (int)x_dtype, stream) == hipSuccess ? KDA_OK
                                                                                   : KDA_ERR_HIP;
    return run(p, chosen, (int)a_dtype, (int)x_dtype, stream);
}

// The "build A from keys" path: k [rows, H, K] and beta [rows, H] of k_dtype,
// g [rows, H, K] FP32, out [rows, H, 64] of x_dtype.
kda_status check_kkt(const void *k, const float *g, const void *beta, kda_dtype k_dtype,
                     const void *out, kda_dtype x_dtype, int64_t rows, int32_t H, int32_t K) {
    if (!valid_dtype(k_dtype) || !valid_dtype(x_dtype) || H <= 0 || K <= 0)
        return KDA_ERR_INVALID_ARG;
    if (rows > kMaxTokens || H > kMaxHeads) return KDA_ERR_UNSUPPORTED;
    if (K % 16 != 0 || K > kMaxKeyDim) return KDA_ERR_UNSUPPORTED;
    if (rows == 0) return KDA_OK;
    if (!k || !g || !beta || !out) return KDA_ERR_INVALID_ARG;
    const size_t eb = dtype_bytes(k_dtype);
    if (!aligned16(k) || !aligned16(g) || !aligned16(out) || ((uintptr_t)beta % eb) != 0)
        return KDA_ERR_INVALID_ARG;
    const size_t nk = (size_t)rows * (size_t)H * (size_t)K;
    const size_t no = (size_t)rows * (size_t)H * 64 * dtype_bytes(x_dtype);
    if (overlap(out, no, k, nk * eb) || overlap(out, no, g, nk * 4) ||
        overlap(out, no, beta, (size_t)rows * (size_t)H * eb))
        return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

kda_status kkt_call(const void *k, const float *g, const void *beta, kda_dtype k_dtype, void *out,
                    kda_dtype x_dtype, const int32_t *cu_seqlens, int64_t num_seqs,
                    int64_t rows, int64_t dense_T, int32_t H, int32_t K,
                    const int32_t *chunk_indices, int64_t num_chunks, bool solve,
                    hipStream_t stream) {
    kda_status st = check_kkt(k, g, beta, k_dtype, out, x_dtype, rows, H, K);
    if (st != KDA_OK || rows == 0 || num_seqs == 0) return st;
    int64_t slots;
    if (dense_T >= 0) {
        slots = num_seqs * ((dense_T + 63) / 64);
    } else {
        if (cu_seqlens == nullptr) return KDA_ERR_INVALID_ARG;
        slots = chunk_slots(rows, num_seqs, num_chunks, 64);
    }
    if (!grid_fits(slots, H)) return KDA_ERR_UNSUPPORTED;
    KktProblem q;
    memset(&q, 0, sizeof(q));
    q.p.X = out;
    q.p.cu = dense_T >= 0 ? nullptr : cu_seqlens;
    q.p.cmap = dense_T >= 0 ? nullptr : chunk_indices;
    q.p.num_seqs = (int32_t)num_seqs;
    q.p.seq_len = dense_T >= 0 ? (int32_t)dense_T : 0;
    q.p.total_tokens = (int32_t)rows;
    q.p.heads = H;
    q.p.slots = (int32_t)slots;
    q.k = k;
    q.g = g;
    q.beta = beta;
    q.K = K;
    return launch_kkt(q, solve, (int)k_dtype, (int)x_dtype, stream) == hipSuccess ? KDA_OK
                                                                                 : KDA_ERR_HIP;
}

kda_status kkt_packed(const void *k, const float *g, const void *beta, kda_dtype k_dtype,
                      void *out, kda_dtype x_dtype, const int32_t *cu_seqlens, int64_t num_seqs,
                      int64_t total_tokens, int32_t H, int32_t K, const int32_t *chunk_indices,
                      int64_t num_chunks, bool solve, hipStream_t stream) {
    if (num_seqs < 0 || total_tokens < 0 || num_chunks < 0) return KDA_ERR_INVALID_ARG;
    if ((chunk_indices == nullptr) != (num_chunks == 0)) return KDA_ERR_INVALID_ARG;
    if (num_seqs > kMaxTokens || num_chunks > kMaxTokens) return KDA_ERR_UNSUPPORTED;
    return kkt_call(k, g, beta, k_dtype, out, x_dtype, cu_seqlens, num_seqs, total_tokens, -1, H,
                    K, chunk_indices, num_chunks, solve, stream);
}

kda_status kkt_dense(const void *k, const float *g, const void *beta, kda_dtype k_dtype,
                     void *out, kda_dtype x_dtype, int64_t B, int64_t T, int32_t H, int32_t K,
                     bool solve, hipStream_t stream) {
    if (B < 0 || T < 0) return KDA_ERR_INVALID_ARG;
    if (B > 0 && T > kMaxTokens / B) return KDA_ERR_UNSUPPORTED;
    return kkt_call(k, g, beta, k_dtype, out, x_dtype, nullptr, B, B * T, T, H, K, nullptr, 0,
                    solve, stream);
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK:
            return "KDA_OK";
        case KDA_ERR_INVALID_ARG:
            return "KDA_ERR_INVALID_ARG: invalid argument";
        case KDA_ERR_UNSUPPORTED:
            return "KDA_ERR_UNSUPPORTED: unsupported size or configuration";
        case KDA_ERR_WORKSPACE:
            return "KDA_ERR_WORKSPACE: split path not allowed or workspace too small";
        case KDA_ERR_HIP:
            return "KDA_ERR_HIP: kernel launch failed";
    }
    return "KDA_ERR_UNKNOWN: unknown status code";
}

kda_algo kda_tril_auto_plan(int64_t total_tokens, int64_t num_chunks, int32_t num_heads,
                            size_t workspace_bytes) {
    kda_algo chosen = KDA_ALGO_FUSED;
    if (total_tokens <= 0 || num_chunks <= 0 || num_heads <= 0) return KDA_ALGO_FUSED;
    if (resolve_plan(total_tokens, num_chunks, num_heads, KDA_ALGO_AUTO, workspace_bytes,
                     &chosen) != KDA_OK)
        return KDA_ALGO_FUSED;
    return chosen;
}

kda_status kda_tril_inv_workspace_size(int64_t total_tokens, int64_t num_seqs,
                                       int64_t num_chunks, int32_t num_heads, kda_algo algo,
                                       size_t *bytes, kda_algo *chosen) {
    if (bytes == nullptr || !valid_algo(algo)) return KDA_ERR_INVALID_ARG;
    if (total_tokens < 0 || num_seqs < 0 || num_chunks < 0 || num_heads <= 0)
        return KDA_ERR_INVALID_ARG;
    if (total_tokens > kMaxTokens || num_heads > kMaxHeads) return KDA_ERR_UNSUPPORTED;
    const int64_t slots = chunk_slots(total_tokens, num_seqs, num_chunks, 64);
    kda_algo c = KDA_ALGO_FUSED;
    kda_status st = resolve_plan(total_tokens, slots, num_heads, algo, SIZE_MAX, &c);
    if (st != KDA_OK) return st;
    *bytes = (c == KDA_ALGO_SPLIT) ? (size_t)split_workspace_bytes(slots, num_heads) : 0;
    if (chosen) *chosen = c;
    return KDA_OK;
}

kda_status kda_tril_inv_dense(const void *A, kda_dtype a_dtype, void *X, kda_dtype x_dtype,
                              int64_t B, int64_t T, int32_t H, void *workspace,
                              size_t workspace_bytes, kda_algo algo, hipStream_t stream) {
    return dense_call(A, a_dtype, X, x_dtype, B, T, H, 64, workspace, workspace_bytes, algo,
                      stream);
}

kda_status kda_tril_inv_packed(const void *A, kda_dtype a_dtype, void *X, kda_dtype x_dtype,
                               const int32_t *cu_seqlens, int64_t num_seqs,
                               int64_t total_tokens, int32_t H, const int32_t *chunk_indices,
                               int64_t num_chunks, void *workspace, size_t workspace_bytes,
                               kda_algo algo, hipStream_t stream) {
    return packed_call(A, a_dtype, X, x_dtype, cu_seqlens, num_seqs, total_tokens, H, 64,
                       chunk_indices, num_chunks, workspace, workspace_bytes, algo, stream);
}

kda_status kda_tril_inv_dense_chunk(const void *A, kda_dtype a_dtype, void *X,
                                    kda_dtype x_dtype, int64_t B, int64_t T, int32_t H,
                                    int32_t chunk_size, void *workspace,
                                    size_t workspace_bytes, kda_algo algo, hipStream_t stream) {
    return dense_call(A, a_dtype, X, x_dtype, B, T, H, chunk_size, workspace, workspace_bytes,
                      algo, stream);
}

kda_status kda_tril_inv_packed_chunk(const void *A, kda_dtype a_dtype, void *X,
                                     kda_dtype x_dtype, const int32_t *cu_seqlens,
                                     int64_t num_seqs, int64_t total_tokens, int32_t H,
                                     int32_t chunk_size, const int32_t *chunk_indices,
                                     int64_t num_chunks, void *workspace,
                                     size_t workspace_bytes, kda_algo algo,
                                     hipStream_t stream) {
    return packed_call(A, a_dtype, X, x_dtype, cu_seqlens, num_seqs, total_tokens, H,
                       chunk_size, chunk_indices, num_chunks, workspace, workspace_bytes, algo,
                       stream);
}

kda_status kda_tril_inv_packed_noalloc(const void *A, kda_dtype a_dtype, void *X,
                                       kda_dtype x_dtype, const int32_t *cu_seqlens,
                                       int64_t num_seqs, int64_t total_tokens, int32_t H,
                                       const int32_t *chunk_indices, int64_t num_chunks,
                                       hipStream_t stream) {
    // every host check first, so that a refused call never touches the device
    if (num_seqs < 0 || total_tokens < 0 || num_chunks < 0) return KDA_ERR_INVALID_ARG;
    if ((chunk_indices == nullptr) != (num_chunks == 0)) return KDA_ERR_INVALID_ARG;
    if (num_seqs > kMaxTokens || num_chunks > kMaxTokens) return KDA_ERR_UNSUPPORTED;
    kda_status st = check_common(A, a_dtype, X, x_dtype, total_tokens, H, 64, KDA_ALGO_SPLIT);
    if (st != KDA_OK || total_tokens == 0 || num_seqs == 0) return st;
    if (cu_seqlens == nullptr) return KDA_ERR_INVALID_ARG;
    const int64_t slots = chunk_slots(total_tokens, num_seqs, num_chunks, 64);
    if (!grid_fits(slots, H)) return KDA_ERR_UNSUPPORTED;
    if (split_workspace_bytes(slots, H) > (int64_t)KDA_TRIL_NOALLOC_SCRATCH_BYTES ||
        !split_within_budget(total_tokens, slots, H))
        return KDA_ERR_WORKSPACE;
    float *ws = nullptr;
    if (noalloc_scratch(&ws) != hipSuccess) return KDA_ERR_HIP;
    return packed_call(A, a_dtype, X, x_dtype, cu_seqlens, num_seqs, total_tokens, H, 64,
                       chunk_indices, num_chunks, ws, KDA_TRIL_NOALLOC_SCRATCH_BYTES,
                       KDA_ALGO_SPLIT, stream);
}

kda_status kda_kkt_tril_inv_packed(const void *k, const float *g, const void *beta,
                                   kda_dtype k_dtype, void *X, kda_dtype x_dtype,
                                   const int32_t *cu_seqlens, int64_t num_seqs,
                                   int64_t total_tokens, int32_t H, int32_t K,
                                   const int32_t *chunk_indices, int64_t num_chunks,
                                   hipStream_t stream) {
    return kkt_packed(k, g, beta, k_dtype, X, x_dtype, cu_seqlens, num_seqs, total_tokens, H, K,
                      chunk_indices, num_chunks, true, stream);
}

kda_status kda_kkt_tril_inv_dense(const void *k, const float *g, const void *beta,
                                  kda_dtype k_dtype, void *X, kda_dtype x_dtype, int64_t B,
                                  int64_t T, int32_t H, int32_t K, hipStream_t stream) {
    return kkt_dense(k, g, beta, k_dtype, X, x_dtype, B, T, H, K, true, stream);
}

kda_status kda_kkt_packed(const void *k, const float *g, const void *beta, kda_dtype k_dtype,
                          void *A, kda_dtype a_dtype, const int32_t *cu_seqlens,
                          int64_t num_seqs, int64_t total_tokens, int32_t H, int32_t K,
                          const int32_t *chunk_indices, int64_t num_chunks,
                          hipStream_t stream) {
    return kkt_packed(k, g, beta, k_dtype, A, a_dtype, cu_seqlens, num_seqs, total_tokens, H, K,
                      chunk_indices, num_chunks, false, stream);
}

kda_status kda_kkt_dense(const void *k, const float *g, const void *beta, kda_dtype k_dtype,
                         void *A, kda_dtype a_dtype, int64_t B, int64_t T, int32_t H, int32_t K,
                         hipStream_t stream) {
    return kkt_dense(k, g, beta, k_dtype, A, a_dtype, B, T, H, K, false, stream);
}

kda_status kda_decode_step(const void *qkv, const void *z, kda_dtype in_dtype, const float *g,
                           const float *beta, const float *norm_w, const float *conv_w,
                           const int32_t *slot, float *state, float *conv_state,
                           int64_t num_slots, void *out, kda_dtype out_dtype, int64_t B,
                           int32_t H, int32_t head_dim, int32_t conv_width, float eps_l2,
                           float eps_norm, hipStream_t stream) {
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return KDA_ERR_INVALID_ARG;
    if (B < 0 || H <= 0 || num_slots < 0) return KDA_ERR_INVALID_ARG;
    if (!(eps_l2 >= 0.0f) || !(eps_norm >= 0.0f) || eps_l2 > 1e30f || eps_norm > 1e30f)
        return KDA_ERR_INVALID_ARG;  // negative, NaN or infinite
    if (head_dim != 128 || conv_width < 2 || conv_width > 4) return KDA_ERR_UNSUPPORTED;
    // one workgroup of 256 threads per (sequence, head): the launch must stay
    // below 2^32 threads
    if (B > (int64_t)(UINT32_MAX / 256) / H || num_slots > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    if (B == 0) return KDA_OK;
    if (num_slots == 0) return KDA_ERR_INVALID_ARG;
    if (!qkv || !z || !g || !beta || !norm_w || !conv_w || !slot || !state || !conv_state || !out)
        return KDA_ERR_INVALID_ARG;
    const size_t ib = dtype_bytes(in_dtype), ob = dtype_bytes(out_dtype);
    if (!aligned16(state) || ((uintptr_t)conv_state & 3u) || ((uintptr_t)g & 3u) ||
        ((uintptr_t)beta & 3u) || ((uintptr_t)norm_w & 3u) || ((uintptr_t)conv_w & 3u) ||
        ((uintptr_t)slot & 3u) || ((uintptr_t)qkv % ib) || ((uintptr_t)z % ib) ||
        ((uintptr_t)out % ob))
        return KDA_ERR_INVALID_ARG;
    const size_t n_state = (size_t)num_slots * (size_t)H * 128 * 128 * 4;
    const size_t n_conv = (size_t)num_slots * 3 * (size_t)H * (size_t)(conv_width - 1) * 128 * 4;
    const size_t n_out = (size_t)B * (size_t)H * 128 * ob;
    if (overlap(out, n_out, state, n_state) || overlap(out, n_out, conv_state, n_conv) ||
        overlap(state, n_state, conv_state, n_conv))
        return KDA_ERR_INVALID_ARG;
    DecodeProblem p;
    memset(&p, 0, sizeof(p));
    p.qkv = qkv;
    p.z = z;
    p.g = g;
    p.beta = beta;
    p.norm_w = norm_w;
    p.conv_w = conv_w;
    p.slot = slot;
    p.state = state;
    p.conv_state = conv_state;
    p.out = out;
    p.B = (int32_t)B;
    p.H = H;
    p.W = conv_width;
    p.num_slots = (int32_t)num_slots;
    p.eps_l2 = eps_l2;
    p.eps_norm = eps_norm;
    return launch_decode(p, (int)in_dtype, (int)out_dtype, stream) == hipSuccess ? KDA_OK
                                                                               : KDA_ERR_HIP;
}

}  // extern "C"
