// Delta-rule matrix built inside the 64-token chunk solver, for gfx950.
//
// KDA prefill hands the shared solver's 64-token branch (LightLLM PR #1703,
// "perf(kda): parallelize diagonal solves in Prefill", PR description) its
// delta-rule intra-chunk matrix: for tokens i > j of one chunk and one head,
//
//     A[i][j] = -beta_i * sum_d k[i][d] k[j][d] exp(g[i][d] - g[j][d]),
//
// with k the keys (K channels), g the cumulative log-decay of each channel
// and beta_i the token's write strength. These kernels form A from k, g and
// beta in registers and either invert it at once (the fused path: A never
// goes to memory) or store it (the matrix alone, for callers that keep the
// two steps apart).
//
// One wavefront per chunk-head, grid-stride walk as in the 64-token solver.
// A is formed as ten 16 x 16 blocks A_IJ (J <= I, blocks of 16 rows), each a
// K-long contraction on the FP32 matrix cores, K in slices of 16 channels:
//
//   A_IJ = -diag(beta_I) Q_I Kx_J^T,  Q_I[i][d] = k[i][d] e^{g[i][d] - g[r][d]},
//                                     Kx_J[j][d] = k[j][d] e^{g[r][d] - g[j][d]},
//
// with the reference row r = 16 I, the first row of block row I. The
// factors exp(g_i - g_r) and exp(g_r - g_j) multiply to exp(g_i - g_j); for
// blocks below the diagonal (j < r <= i) both are at most 1 when the decay
// does not grow along the chunk, and on the diagonal block the second spans at
// most 15 tokens of decay, so neither factor overflows for any realistic
// gate. Each product is computed transposed, D = Kx_J Q_I^T: the MFMA
// accumulator then holds row i of A_IJ, columns 4g..4g+3, in lane (g, i),
// which is the layout the merge consumes (OPND_A) with no data movement.
// The diagonal blocks go through LDS once to become the row-per-lane layout
// of the diagonal solve.
#include "tril_device.h"
#include "tril_launch.h"

namespace kda {

// Keys and write strengths share one element type EK; decays are FP32.
template <class EK>
struct KktViews {
    TileView<EK> k;
    TileView<F32> g;
    TileView<EK> beta;
};

// a * exp(x), with x already the decay difference (a = 0 rows stay 0 by
// select, so an overflowing factor on a row past the chunk cannot make NaN).
__device__ __forceinline__ f4 scaled(f4 a, f4 x, bool keep) {
    f4 r;
#pragma unroll
    for (int s = 0; s < 4; ++s) r[s] = keep ? a[s] * __expf(x[s]) : 0.0f;
    return r;
}

// acc + Kx Q^T over one 16-channel slice (lane (g, n): Kx row n and Q row n,
// channels 4g..4g+3; the reduction index is permuted as d = 4g + s).
__device__ __forceinline__ f4 mma_kq(f4 Kx, f4 Q, f4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Kx[0], Q[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Kx[1], Q[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Kx[2], Q[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Kx[3], Q[3], acc, 0, 0, 0);
    return acc;
}

// The ten blocks A_IJ (J <= I) of one chunk-head in OPND_A layout: row n of
// block row I in lane (g, n), columns 16J + 4g..+3. Entries on and above the
// diagonal are exact zeros; rows past the chunk are zero.
template <class EK>
__device__ __forceinline__ void build_blocks(const KktViews<EK> &v, int K, int len,
                                             f4 (&acc)[4][4], int lane) {
    const int g4 = lane >> 4, n = lane & 15;
    const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int J = 0; J < 4; ++J) acc[I][J] = z;
    bool valid[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) valid[b] = 16 * b + n < len;
    // one descriptor per tensor over all rows of the chunk-head (few SGPRs);
    // block b's rows are 16 b rows further in the per-lane offset
    const Rsrc rk = v.k.rows_from(0), rg = v.g.rows_from(0);
    const uint32_t offk = (uint32_t)(n * v.k.rstride + 4 * g4) * EK::kBytes;
    const uint32_t offg = (uint32_t)(n * v.g.rstride + 4 * g4) * F32::kBytes;
    const uint32_t blk_k = (uint32_t)(16 * v.k.rstride) * EK::kBytes;
    const uint32_t blk_g = (uint32_t)(16 * v.g.rstride) * F32::kBytes;
#pragma unroll 1
    for (int d0 = 0; d0 < K; d0 += 16) {
        f4 kb[4], gb[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            kb[b] = load4<EK>(rk, offk + b * blk_k + d0 * EK::kBytes);
            gb[b] = load4<F32>(rg, offg + b * blk_g + d0 * F32::kBytes);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (16 * I >= len) break;  // uniform: block row I lies past the chunk
            f4 gref;
#pragma unroll
            for (int s = 0; s < 4; ++s) gref[s] = row_bcast<0>(gb[I][s]);
            const f4 Q = scaled(kb[I], gb[I] - gref, valid[I]);
#pragma unroll
            for (int J = 0; J <= I; ++J) {
                const f4 Kx = scaled(kb[J], gref - gb[J], valid[J]);
                acc[I][J] = mma_kq(Kx, Q, acc[I][J]);
            }
        }
    }
    // -beta of this lane's row in each block row; strictly-lower mask on the
    // diagonal blocks (column 4g + s < row n), by select
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const float nb = -load1<EK>(v.beta.rows_from(16 * I), (uint32_t)(n * v.beta.rstride) *
                                                                   EK::kBytes);
#pragma unroll
        for (int J = 0; J <= I; ++J)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float a = acc[I][J][s] * nb;
                acc[I][J][s] = (J < I || 4 * g4 + s < n) ? a : 0.0f;
            }
    }
}

// Writes rows 16I..16I+15 of A (those inside the view) from blocks in OPND_A
// layout: staged through LDS so every store covers four whole 64-column rows.
template <class E, int I>
__device__ __forceinline__ void store_rows_a(const TileView<E> &X, const f4 (&blk)[4],
                                             float *stage, int lane) {
    constexpr int S = stage_row(I);
    const int g4 = lane >> 4, n = lane & 15;
    wave_sync();
#pragma unroll
    for (int J = 0; J <= I; ++J)
        *reinterpret_cast<f4 *>(&stage[n * S + 16 * J + 4 * g4]) = blk[J];
    wave_sync();
    const int r4 = lane >> 4, c4 = (lane & 15) * 4;
    const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t off = (uint32_t)(r4 * X.rstride + c4) * E::kBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + r4;
        f4 v = z;
        if (c4 < 16 * (I + 1)) v = *reinterpret_cast<const f4 *>(&stage[row * S + c4]);
        store4<E>(X.rows_from(16 * I + 4 * i), off, v);
    }
    wave_sync();
}

template <class EK, class EO, bool SOLVE>
__global__ __launch_bounds__(kFusedThreads) void tril_kkt(KktProblem q) {
    __shared__ float lds_all[kFusedWaves * kLdsPerWave];
    const Problem &p = q.p;
    const int lane0 = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float *xs = lds_all + wid * kLdsPerWave;
    const long total = (long)p.slots * p.heads;
    const long G = (long)gridDim.x * kFusedWaves;
    for (long w = (long)blockIdx.x * kFusedWaves + wid; w < total; w += G) {
        const int slot = (int)(w / p.heads);
        const int h = (int)(w - (long)slot * p.heads);
        const Chunk ch = uniform(resolve_chunk<kChunk>(p, slot, lane0));
        if (ch.len <= 0) continue;
        const int lane = opaque_lane(lane0);
        const long row0 = (long)ch.start * p.heads + h;  // (token, head) index of row 0
        const KktViews<EK> v{
            {static_cast<const typename EK::T *>(q.k) + row0 * q.K, p.heads * q.K, ch.len, q.K},
            {q.g + row0 * q.K, p.heads * q.K, ch.len, q.K},
            {static_cast<const typename EK::T *>(q.beta) + row0, p.heads, ch.len, 1}};
        f4 acc[4][4];
        build_blocks<EK>(v, q.K, ch.len, acc, lane);
        const TileView<EO> X{static_cast<typename EO::T *>(p.X) + row0 * kChunk,
                             p.heads * kChunk, ch.len, kChunk};
        if constexpr (SOLVE) {
            // diagonal blocks to the row-per-lane layout of the diagonal solve
            const int g4 = lane >> 4, n = lane & 15;
            wave_sync();
#pragma unroll
            for (int b = 0; b < 4; ++b)
                *reinterpret_cast<f4 *>(&xs[b * kXsBlock + n * kXsCol + 4 * g4]) = acc[b][b];
            wave_sync();
            float arow[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f4 r = *reinterpret_cast<const f4 *>(&xs[g4 * kXsBlock + n * kXsCol + 4 * q4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) arow[4 * q4 + e] = r[e];
            }
            wave_sync();
            const MfmaEngine<kXsBlock, kXsCol> eng{xs, lane};
            diag_inverses(xs, arow, lane);
            merge_and_store<EO, kXsBlock, kXsCol>(eng, acc, xs, xs, X, lane);
        } else {
            store_rows_a<EO, 0>(X, acc[0], xs, lane);
            if (ch.len <= 16) continue;
            store_rows_a<EO, 1>(X, acc[1], xs, lane);
            if (ch.len <= 32) continue;
            store_rows_a<EO, 2>(X, acc[2], xs, lane);
            if (ch.len <= 48) continue;
            store_rows_a<EO, 3>(X, acc[3], xs, lane);
        }
    }
}

// ------------------------------------------------------------------ launch

template <class Kern>
static hipError_t launch_kkt_kernel(Kern kernel, const KktProblem &q, hipStream_t stream) {
    const long waves = (long)q.p.slots * q.p.heads;
    const long need = (waves + kFusedWaves - 1) / kFusedWaves;
    const long cap = resident_blocks(reinterpret_cast<const void *>(kernel), kFusedThreads);
    const long blocks = cap > 0 && cap < need ? cap : need;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kFusedThreads), 0, stream, q);
    return hipGetLastError();
}

hipError_t launch_kkt(const KktProblem &q, bool solve, int k_dt, int x_dt, hipStream_t stream) {
    return dispatch_dtypes<F32, BF16, F16>(k_dt, x_dt, [&]<class EK, class EO>() {
        return solve ? launch_kkt_kernel(tril_kkt<EK, EO, true>, q, stream)
                     : launch_kkt_kernel(tril_kkt<EK, EO, false>, q, stream);
    });
}

}  // namespace kda
