/*
 * Plain CPU oracle for the KDA prefill chunk solver.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it. It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (LightLLM PR #1703, "perf(kda): parallelize diagonal solves
 * in Prefill", PR description, method paragraph): for every 64-token chunk of
 * every request and every head (and, for the shared solver's other branches,
 * every 16- or 32-token chunk), the inverse X = (I + A)^-1 of the unit
 * lower-triangular matrix I + A, where A holds the strictly-lower
 * intra-chunk entries. The page computes it with four 16x16 diagonal inverses
 * and a blocked merge; that is only an evaluation order of the same unique
 * inverse (det(I + A) = 1), so this oracle evaluates the plain definition:
 * column-by-column forward substitution of (I + A) X = I in double precision,
 * one chunk-head at a time, with no blocking.
 *
 * Readings where the page is silent (each also recorded in the design notes):
 *  - chunks restart at every request's first token, so a request of length n
 *    has ceil(n / 64) chunks and only its last one may be partial;
 *  - only rows i < L of a chunk with L valid tokens exist; the result is the
 *    L x L inverse, i.e. the leading block of the zero-padded 64x64 one;
 *  - entries of A on or above the diagonal are ignored (never read);
 *  - every valid row of X is written in full: 1 on the diagonal, 0 above it
 *    and in columns >= L;
 *  - rows that belong to no chunk are not touched.
 *
 * Layouts: packed A and X are [T, H, C] row-major (token, head, column) for
 * chunks of C tokens; dense ones are [B, T, H, C]. Element (token t, head h,
 * column j) is the entry (t - chunk_start, j) of that chunk-head's matrix.
 *
 * For the fused path that builds A from keys, decays and write strengths
 * before inverting it, oracle_kkt_* evaluate that A from its definition (see
 * there); the oracle of the fused path is that A, kept in double precision,
 * followed by the inverse above.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_CHUNK 64

/*
 * Chunk enumeration of a packed batch (same PR, PR description: the solver
 * accepts packed varlen batches described by cumulative sequence lengths).
 * Request s covers tokens [cu[s], cu[s+1]); its chunks of C tokens start at
 * cu[s] + C*c. Writes up to `cap` entries and returns the total number of
 * chunks, or -1 when cu is not non-decreasing, cu[0] < 0 or C < 1.
 */
int64_t oracle_chunks_packed_c(const int32_t *cu, int64_t nseq, int C, int64_t *seq_out,
                               int64_t *start_out, int32_t *len_out, int64_t cap) {
    int64_t n = 0;
    if (C < 1 || (nseq > 0 && cu[0] < 0)) return -1;
    for (int64_t s = 0; s < nseq; ++s) {
        int64_t bos = cu[s], eos = cu[s + 1];
        if (eos < bos) return -1;
        for (int64_t p = bos; p < eos; p += C) {
            int64_t len = eos - p < C ? eos - p : C;
            if (n < cap) {
                if (seq_out) seq_out[n] = s;
                if (start_out) start_out[n] = p;
                if (len_out) len_out[n] = (int32_t)len;
            }
            ++n;
        }
    }
    return n;
}

int64_t oracle_chunks_packed(const int32_t *cu, int64_t nseq, int64_t *seq_out,
                             int64_t *start_out, int32_t *len_out, int64_t cap) {
    return oracle_chunks_packed_c(cu, nseq, ORACLE_CHUNK, seq_out, start_out, len_out, cap);
}

/*
 * X = (I + M)^-1 for one L x L matrix, L <= W <= 64. M and X are row-major
 * with leading dimensions ldm and ldx (in elements). Only M[i][j] with j < i
 * is read. X is written for rows i < L and columns j < W (columns >= L are
 * 0), matching a full output row of a W-wide chunk.
 *
 * Column c of X solves (I + M) x = e_c: x_i = 0 for i < c, x_c = 1, and for
 * i > c, x_i = -sum_{j=c}^{i-1} M[i][j] x_j, summed in increasing j.
 */
void oracle_inv_unit_lower_w(const double *M, int64_t ldm, int L, int W, double *X, int64_t ldx) {
    double col[ORACLE_CHUNK];
    for (int i = 0; i < L; ++i)
        for (int j = 0; j < W; ++j) X[(int64_t)i * ldx + j] = 0.0;
    for (int c = 0; c < L; ++c) {
        for (int i = 0; i < c; ++i) col[i] = 0.0;
        col[c] = 1.0;
        for (int i = c + 1; i < L; ++i) {
            double s = 0.0;
            for (int j = c; j < i; ++j) s += M[(int64_t)i * ldm + j] * col[j];
            col[i] = -s;
        }
        for (int i = c; i < L; ++i) X[(int64_t)i * ldx + c] = col[i];
    }
}

void oracle_inv_unit_lower(const double *M, int64_t ldm, int L, double *X, int64_t ldx) {
    oracle_inv_unit_lower_w(M, ldm, L, ORACLE_CHUNK, X, ldx);
}

static int oracle_threads(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Packed layout with chunks of C tokens (C in 1..64): A, X are [T, H, C]
 * doubles; cu has nseq + 1 entries with cu[nseq] <= T. Returns the number of
 * chunk-head matrices solved, or -1 on a malformed problem. nthreads <= 0
 * uses the OpenMP default.
 */
int64_t oracle_tril_inv_packed_c(const double *A, double *X, const int32_t *cu, int64_t nseq,
                                 int64_t T, int32_t H, int C, int nthreads) {
    if (H <= 0 || nseq < 0 || C < 1 || C > ORACLE_CHUNK) return -1;
    int64_t nt = oracle_chunks_packed_c(cu, nseq, C, NULL, NULL, NULL, 0);
    if (nt < 0 || (nseq > 0 && cu[nseq] > T)) return -1;
    int64_t *start = (int64_t *)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(int64_t));
    int32_t *len = (int32_t *)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(int32_t));
    if (!start || !len) { free(start); free(len); return -1; }
    oracle_chunks_packed_c(cu, nseq, C, NULL, start, len, nt);
    const int64_t rs = (int64_t)H * C; /* elements between consecutive tokens */
    const int64_t work = nt * (int64_t)H;
#pragma omp parallel for schedule(static) num_threads(oracle_threads(nthreads))
    for (int64_t w = 0; w < work; ++w) {
        int64_t k = w / H, h = w % H;
        int64_t off = start[k] * rs + h * C;
        oracle_inv_unit_lower_w(A + off, rs, len[k], C, X + off, rs);
    }
    free(start);
    free(len);
    return work;
}

int64_t oracle_tril_inv_packed(const double *A, double *X, const int32_t *cu, int64_t nseq,
                               int64_t T, int32_t H, int nthreads) {
    return oracle_tril_inv_packed_c(A, X, cu, nseq, T, H, ORACLE_CHUNK, nthreads);
}

/*
 * Dense batch layout (same PR, PR description: the solver also takes dense
 * [B, T, H] batches) with chunks of C tokens: A, X are [B, T, H, C] doubles;
 * every batch element is one request of T tokens, so its chunks start at Cc
 * and the last has T - Cc valid rows. Returns the number of matrices solved.
 */
int64_t oracle_tril_inv_dense_c(const double *A, double *X, int64_t B, int64_t T, int32_t H,
                                int C, int nthreads) {
    if (H <= 0 || B < 0 || T < 0 || C < 1 || C > ORACLE_CHUNK) return -1;
    const int64_t rs = (int64_t)H * C;
    const int64_t per_b = (T + C - 1) / C;
    const int64_t work = B * per_b * (int64_t)H;
#pragma omp parallel for schedule(static) num_threads(oracle_threads(nthreads))
    for (int64_t w = 0; w < work; ++w) {
        int64_t h = w % H, k = w / H;
        int64_t b = k / per_b, c = k % per_b;
        int64_t row0 = b * T + c * C;
        int L = (int)(T - c * C < C ? T - c * C : C);
        int64_t off = row0 * rs + h * C;
        oracle_inv_unit_lower_w(A + off, rs, L, C, X + off, rs);
    }
    return work;
}

int64_t oracle_tril_inv_dense(const double *A, double *X, int64_t B, int64_t T, int32_t H,
                              int nthreads) {
    return oracle_tril_inv_dense_c(A, X, B, T, H, ORACLE_CHUNK, nthreads);
}

/*
 * Round-to-nearest-even from binary32 to bfloat16. The same PR keeps the
 * inverse tiles in FP32 through the merge (commit summary), so a bfloat16
 * output is read as one rounding of the final FP32 value at the store; this is
 * the CPU side of that rounding, used to check it. bfloat16 is
 * the upper 16 bits of a binary32; the value is rounded to the nearer of the
 * two representable neighbours, and a tie goes to the one whose last kept bit
 * is 0. NaNs stay NaN (quiet bit forced). Overflow rounds to infinity, as the
 * definition gives.
 */
void oracle_rne_bf16(const uint32_t *f32bits, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b = f32bits[i];
        if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu) != 0u) {
            out[i] = (uint16_t)((b >> 16) | 0x0040u);
            continue;
        }
        uint32_t kept = b >> 16;
        uint32_t rest = b & 0xFFFFu;
        if (rest > 0x8000u || (rest == 0x8000u && (kept & 1u))) kept += 1u;
        out[i] = (uint16_t)kept;
    }
}

int oracle_num_threads(void) { return oracle_threads(0); }

/*
 * The matrix A itself, for the fused "build A, then invert" path. KDA prefill
 * hands the solver its delta-rule intra-chunk matrix (same PR, PR
 * description: KDA Prefill uses the shared solver's 64-token branch); for
 * tokens i > j of one chunk and one head it is
 *
 *     A[i][j] = -beta_i * sum_d k[i][d] * k[j][d] * exp(g[i][d] - g[j][d]),
 *
 * with k the key rows (K channels), g the cumulative log-decay of each
 * channel and beta_i the token's write strength; A[i][j] = 0 for j >= i.
 * Evaluated from this definition in double precision: one exp per
 * difference, the sum over d in increasing d.
 *
 * One chunk of L rows: k, g are row-major with rs_kg elements between
 * consecutive tokens (H * K in [T, H, K]), beta has rs_b between tokens (H);
 * A gets L full rows of 64 entries, rs_a apart.
 */
static void oracle_kkt_chunk(const double *k, const double *g, const double *beta,
                             int64_t rs_kg, int64_t rs_b, int L, int K, double *A,
                             int64_t rs_a) {
    for (int i = 0; i < L; ++i) {
        for (int j = 0; j < ORACLE_CHUNK; ++j) A[(int64_t)i * rs_a + j] = 0.0;
        for (int j = 0; j < i; ++j) {
            double s = 0.0;
            for (int d = 0; d < K; ++d)
                s += k[(int64_t)i * rs_kg + d] * k[(int64_t)j * rs_kg + d] *
                     exp(g[(int64_t)i * rs_kg + d] - g[(int64_t)j * rs_kg + d]);
            A[(int64_t)i * rs_a + j] = -beta[(int64_t)i * rs_b] * s;
        }
    }
}

/*
 * Packed layout, 64-token chunks: k, g [T, H, K], beta [T, H], A out
 * [T, H, 64] (doubles). Rows of every chunk are written in full; rows outside
 * all chunks are untouched. Returns the number of chunk-head matrices, or -1
 * on a malformed problem.
 */
int64_t oracle_kkt_packed(const double *k, const double *g, const double *beta, double *A,
                          const int32_t *cu, int64_t nseq, int64_t T, int32_t H, int K,
                          int nthreads) {
    if (H <= 0 || nseq < 0 || K < 1) return -1;
    int64_t nt = oracle_chunks_packed_c(cu, nseq, ORACLE_CHUNK, NULL, NULL, NULL, 0);
    if (nt < 0 || (nseq > 0 && cu[nseq] > T)) return -1;
    int64_t *start = (int64_t *)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(int64_t));
    int32_t *len = (int32_t *)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(int32_t));
    if (!start || !len) { free(start); free(len); return -1; }
    oracle_chunks_packed_c(cu, nseq, ORACLE_CHUNK, NULL, start, len, nt);
    const int64_t work = nt * (int64_t)H;
#pragma omp parallel for schedule(static) num_threads(oracle_threads(nthreads))
    for (int64_t w = 0; w < work; ++w) {
        int64_t c = w / H, h = w % H;
        int64_t t0 = start[c];
        oracle_kkt_chunk(k + (t0 * H + h) * K, g + (t0 * H + h) * K, beta + t0 * H + h,
                         (int64_t)H * K, H, len[c], K, A + (t0 * H + h) * ORACLE_CHUNK,
                         (int64_t)H * ORACLE_CHUNK);
    }
    free(start);
    free(len);
    return work;
}

/* Dense layout: k, g [B, T, H, K], beta [B, T, H], A [B, T, H, 64]; every
 * batch element is one request of T tokens. */
int64_t oracle_kkt_dense(const double *k, const double *g, const double *beta, double *A,
                         int64_t B, int64_t T, int32_t H, int K, int nthreads) {
    if (H <= 0 || B < 0 || T < 0 || K < 1) return -1;
    const int64_t per_b = (T + ORACLE_CHUNK - 1) / ORACLE_CHUNK;
    const int64_t work = B * per_b * (int64_t)H;
#pragma omp parallel for schedule(static) num_threads(oracle_threads(nthreads))
    for (int64_t w = 0; w < work; ++w) {
        int64_t h = w % H, c = (w / H) % per_b, b = w / H / per_b;
        int64_t t0 = b * T + c * ORACLE_CHUNK;
        int L = (int)(T - c * ORACLE_CHUNK < ORACLE_CHUNK ? T - c * ORACLE_CHUNK : ORACLE_CHUNK);
        oracle_kkt_chunk(k + (t0 * H + h) * K, g + (t0 * H + h) * K, beta + t0 * H + h,
                         (int64_t)H * K, H, L, K, A + (t0 * H + h) * ORACLE_CHUNK,
                         (int64_t)H * ORACLE_CHUNK);
    }
    return work;
}

/*
 * One decode step of the fused KDA decode core (tokenspeed PR #1086,
 * "perf(kimi3): fuse KDA decode core", PR description: single-token causal
 * convolution with its state update, the KDA recurrent update and gated
 * RMSNorm; its test plan names convolution, paged-state, padding and
 * gated-RMSNorm references). The page gives no formulas; this is the plain
 * reading of those parts for one new token per sequence, evaluated from the
 * definitions in double precision:
 *
 *   for each projection p in (q, k, v) and channel c of head h:
 *     y_c = sum_{w < W-1} cw[p][w][c] * cs[p][w][c] + cw[p][W-1][c] * x[p][c]
 *     (cs: the W-1 previous inputs, oldest first), then cs shifts by one
 *     and x becomes its newest entry; y_c = silu(y_c) = y_c / (1 + exp(-y_c))
 *   q = y_q / sqrt(|y_q|^2 + eps_l2) / sqrt(d),  k = y_k / sqrt(|y_k|^2 + eps_l2),
 *   v = y_v
 *   S <- diag(exp(g)) S                  (S: d x d, key rows i, value columns j)
 *   u_j = beta * (v_j - sum_i S[i][j] k_i)
 *   S[i][j] <- S[i][j] + k_i u_j
 *   o_j = sum_i S[i][j] q_i
 *   out_j = o_j / sqrt(mean_j o_j^2 + eps_norm) * wn_j * sigmoid(z_j)
 *
 * Layouts (doubles): qkv [B, 3, H, d]; g [B, H, d]; beta [B, H]; z [B, H, d];
 * wn [d]; cw [3, W, H, d] (tap-major); slot [B] (int32): the state slot of
 * each batch entry, < 0 for padding; S [slots, H, d, d]; cs [slots, 3, H,
 * W - 1, d]; out [B, H, d]. Padding entries get out = 0 and touch no state.
 * S and cs are updated in place. Returns 0, or -1 on bad sizes.
 */
int oracle_kda_decode(const double *qkv, const double *g, const double *beta, const double *z,
                      const double *wn, const double *cw, const int32_t *slot, double *S,
                      double *cs, double *out, int64_t B, int32_t H, int d, int W,
                      double eps_l2, double eps_norm) {
    if (B < 0 || H <= 0 || d <= 0 || d > 256 || W < 2 || W > 8) return -1;
    for (int64_t b = 0; b < B; ++b) {
        for (int32_t h = 0; h < H; ++h) {
            double *o_out = out + (b * H + h) * d;
            const int32_t s = slot[b];
            if (s < 0) {
                for (int j = 0; j < d; ++j) o_out[j] = 0.0;
                continue;
            }
            double y[3][256];
            for (int p = 0; p < 3; ++p) {
                double *st = cs + (((int64_t)s * 3 + p) * H + h) * (int64_t)(W - 1) * d;
                const double *x = qkv + ((b * 3 + p) * H + h) * d;
                for (int c = 0; c < d; ++c) {
                    double acc = 0.0;
                    for (int w = 0; w < W - 1; ++w)
                        acc += cw[(((int64_t)p * W + w) * H + h) * d + c] * st[(int64_t)w * d + c];
                    acc += cw[(((int64_t)p * W + (W - 1)) * H + h) * d + c] * x[c];
                    for (int w = 0; w < W - 2; ++w) st[(int64_t)w * d + c] = st[(int64_t)(w + 1) * d + c];
                    st[(int64_t)(W - 2) * d + c] = x[c];
                    y[p][c] = acc / (1.0 + exp(-acc));
                }
            }
            double nq = 0.0, nk = 0.0;
            for (int c = 0; c < d; ++c) {
                nq += y[0][c] * y[0][c];
                nk += y[1][c] * y[1][c];
            }
            const double sq = 1.0 / sqrt(nq + eps_l2) / sqrt((double)d);
            const double sk = 1.0 / sqrt(nk + eps_l2);
            double q[256], k[256];
            for (int c = 0; c < d; ++c) {
                q[c] = y[0][c] * sq;
                k[c] = y[1][c] * sk;
            }
            double *M = S + ((int64_t)s * H + h) * (int64_t)d * d;
            const double *gg = g + (b * H + h) * d;
            for (int i = 0; i < d; ++i) {
                const double a = exp(gg[i]);
                for (int j = 0; j < d; ++j) M[(int64_t)i * d + j] *= a;
            }
            const double bt = beta[b * H + h];
            double u[256];
            for (int j = 0; j < d; ++j) {
                double r = 0.0;
                for (int i = 0; i < d; ++i) r += M[(int64_t)i * d + j] * k[i];
                u[j] = bt * (y[2][j] - r);
            }
            for (int i = 0; i < d; ++i)
                for (int j = 0; j < d; ++j) M[(int64_t)i * d + j] += k[i] * u[j];
            double o[256], ms = 0.0;
            for (int j = 0; j < d; ++j) {
                double r = 0.0;
                for (int i = 0; i < d; ++i) r += M[(int64_t)i * d + j] * q[i];
                o[j] = r;
                ms += r * r;
            }
            const double rn = 1.0 / sqrt(ms / d + eps_norm);
            const double *zz = z + (b * H + h) * d;
            for (int j = 0; j < d; ++j) o_out[j] = o[j] * rn * wn[j] / (1.0 + exp(-zz[j]));
        }
    }
    return 0;
}
