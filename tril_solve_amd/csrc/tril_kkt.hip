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
// One wavefront per chunk-head, a grid of one wavefront per item as in the
// 64-token solver (a grid forced smaller walks them with a grid stride).
// A is formed as ten 16 x 16 blocks A_IJ (J <= I, blocks of 16 rows), each a
// K-long contraction on the FP32 matrix cores, K in slices of 16 channels.
// With r_I = 16 I the first row of block I, exp(g_i - g_j) factors as
//
//   exp(g_i - g_rI) * exp(g_rI - g_rJ) * exp(g_rJ - g_j)   (i in block I, j in J)
//
// so A_IJ = -diag(beta_I) Q_I (P_J * c_IJ)^T with Q_I = k_I e^{g_I - g_rI},
// P_J = k_J e^{g_rJ - g_J} and c_IJ = e^{g_rI - g_rJ} per channel (c_II = 1).
// When the decay does not grow along the chunk, Q and c are at most 1 and P
// spans at most 15 tokens of decay, so no factor overflows for any realistic
// gate; exponentials per lane and 16-channel slice drop from 56 (one per
// block pair and row) to 36: 16 for Q, 16 for P and 4 for the six c_IJ, which
// depend on the channel only and are spread over the lanes of a 16-lane row
// and shared by DPP broadcasts. Each exponent (a decay difference) is scaled
// by log2(e) so every exponential is a bare v_exp_f32. That instruction
// returns no subnormal results: a factor below 2^-126 is 0, which bounds the
// domain (c for adjacent blocks spans 16 tokens of decay, so falls up to
// about 87 over 16 consecutive tokens, 5.45 per token, are represented).
//
// Each product is computed transposed, D = (P_J c_IJ) Q_I^T: the MFMA
// accumulator then holds row i of A_IJ, columns 4g..4g+3, in lane (g, i),
// which is the layout the merge consumes (OPND_A) with no data movement.
// The diagonal blocks reach the row-per-lane layout of the diagonal solve by
// lane swaps between registers.
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

constexpr float kLog2e = 1.4426950408889634f;

// Four elements as loaded (no conversion), so that a load issued a slice
// ahead is not waited for at once by its widening; widen4 converts at use.
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
template <class E>
struct Raw4 {
    typedef u2 T;  // four 16-bit elements
    static __device__ __forceinline__ T load(Rsrc r, uint32_t off) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    }
};
template <>
struct Raw4<F32> {
    typedef u4 T;
    static __device__ __forceinline__ T load(Rsrc r, uint32_t off) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
};
// The FP32 decays as loaded. Each decay line is used up by the iteration
// that loads it; a 16-bit key line is only half used by one slice, so with
// 16-bit keys the decays take the nontemporal policy and L2 evicts them
// first, which keeps more key lines for the next slice (HBM reads per launch
// at 16 x 512 tokens, 64 heads, K = 128: 510 -> 448 MB). FP32 key lines are
// used up in one slice, and the default policy stays.
template <class EK>
__device__ __forceinline__ u4 load_decays(Rsrc r, uint32_t off) {
    constexpr int policy = EK::kBytes == 2 ? kNontemporal : 0;
    return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, policy));
}
template <class E>
__device__ __forceinline__ f4 widen4(typename Raw4<E>::T v);
template <>
__device__ __forceinline__ f4 widen4<F32>(u4 v) {
    return __builtin_bit_cast(f4, v);
}
template <>
__device__ __forceinline__ f4 widen4<BF16>(u2 v) {
    f4 o;
    o[0] = bf16_to_f32(v[0] & 0xFFFFu);
    o[1] = bf16_to_f32(v[0] >> 16);
    o[2] = bf16_to_f32(v[1] & 0xFFFFu);
    o[3] = bf16_to_f32(v[1] >> 16);
    return o;
}
template <>
__device__ __forceinline__ f4 widen4<F16>(u2 v) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 h = __builtin_bit_cast(h4, v);
    f4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (float)h[e];  // exact widening
    return o;
}

// a * 2^x (x a decay difference already scaled by log2 e).
__device__ __forceinline__ f4 scaled(f4 a, f4 x) {
    f4 r;
#pragma unroll
    for (int s = 0; s < 4; ++s) r[s] = a[s] * __builtin_amdgcn_exp2f(x[s]);
    return r;
}

// Block pairs I > J get numbers p = 0..5 in the order (1,0), (2,0), (2,1),
// (3,0), (3,1), (3,2); lane p of every 16-lane row evaluates c for pair p
// (its four channels), and pair_factor<p> hands it to the whole row.
template <int P>
__device__ __forceinline__ f4 pair_factor(const f4 &cv) {
    f4 r;
#pragma unroll
    for (int s = 0; s < 4; ++s) r[s] = row_bcast<P>(cv[s]);
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

// One 32-channel slice of the keys and decays of a chunk-head as loaded:
// lane (g, n) holds row n of each 16-row block, channels 8g..8g+7 of the
// slice, so the four lanes of a row cover 128 contiguous bytes of the FP32
// decays (one whole cache line) and 64 or 128 bytes of the keys. Lines are
// then used up within one iteration instead of being fetched again from HBM
// by a later one (rows lie H x K elements apart, so a partly used line
// rarely survives in L2 until the next slice). It is consumed as two
// 16-channel sub-slices t = 0, 1 of channels 8g + 4t + s (s = 0..3).
template <class EK>
struct Slice {
    typename Raw4<EK>::T k[4][2];
    u4 g[4][2];
};

// Where a lane's loads go: one descriptor per tensor over all rows of the
// chunk-head (few SGPRs), block b's rows 16 b rows further in the offset.
template <class EK>
struct SliceSrc {
    Rsrc rk, rg;
    uint32_t offk, blk_k;
    uint32_t offgb[4];
    bool upper;  // this lane holds channels 16..31 of a slice (g >= 2)

    // Loads the slice at channel d0. With `half` (K % 32 = 16: only 16
    // channels are left) the lanes of channels 16..31 read 0 keys and, so
    // that their factors stay finite, the decays 16 channels lower.
    __device__ __forceinline__ void load(Slice<EK> &s, int d0, bool half) const {
        const bool off = half && upper;
        const uint32_t kmask = off ? kOffMasked : 0u;
        const uint32_t gback = off ? 16u * F32::kBytes : 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                s.g[b][t] = load_decays<EK>(rg, offgb[b] + (d0 + 4 * t) * F32::kBytes - gback);
                s.k[b][t] =
                    Raw4<EK>::load(rk, (offk + b * blk_k + (d0 + 4 * t) * EK::kBytes) | kmask);
            }
    }
};

// Adds one 16-channel sub-slice to the ten blocks. Block by block: P_b is
// kept for the blocks below it, Q_b is used at once, so few factors are live
// together.
template <class EK>
__device__ __forceinline__ void accumulate_sub(const typename Raw4<EK>::T (&kr)[4],
                                               const u4 (&graw)[4], const f4 &wsel,
                                               f4 (&acc)[4][4]) {
    f4 gl[4], gr[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        gl[b] = widen4<F32>(graw[b]);
        // decay of the block's reference row (its row 0) in every lane
#pragma unroll
        for (int s = 0; s < 4; ++s) gr[b][s] = row_bcast<0>(gl[b][s]);
    }
    // Every exponent is a difference of decays taken first and scaled by
    // log2 e after: decays a few tokens apart subtract exactly, so a caller's
    // cumulative decays may run far from zero (over a whole request rather
    // than restarting at each chunk) without their rounding entering.
    // c for this lane's pair (I, J), every pair's c reaching the row by
    // broadcast: the difference gr[I] - gr[J] as sum_b wsel[b] gr[b] with
    // wsel[b] = [b == I] - [b == J], which for finite decays is that
    // difference bit for bit (the zero terms add exact zeros, the two others
    // round once); a select on the lane's pair compiled to divergent branches.
    f4 cv;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        float a = wsel[0] * gr[0][s];
#pragma unroll
        for (int b = 1; b < 4; ++b) a = __builtin_fmaf(wsel[b], gr[b][s], a);
        cv[s] = __builtin_amdgcn_exp2f(a * kLog2e);
    }
    f4 P[4];
    // all ten products, also for blocks past a partial chunk (their P and Q
    // are zero): no branches
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const f4 kb = widen4<EK>(kr[b]);
        // the two exponents are exact negations of each other: one
        // subtraction, the second exponential takes it negated
        const f4 t = (gr[b] - gl[b]) * kLog2e;
        P[b] = scaled(kb, t);
        const f4 Q = scaled(kb, -t);
        acc[b][b] = mma_kq(P[b], Q, acc[b][b]);
        if (b == 1) acc[1][0] = mma_kq(P[0] * pair_factor<0>(cv), Q, acc[1][0]);
        if (b == 2) {
            acc[2][0] = mma_kq(P[0] * pair_factor<1>(cv), Q, acc[2][0]);
            acc[2][1] = mma_kq(P[1] * pair_factor<2>(cv), Q, acc[2][1]);
        }
        if (b == 3) {
            acc[3][0] = mma_kq(P[0] * pair_factor<3>(cv), Q, acc[3][0]);
            acc[3][1] = mma_kq(P[1] * pair_factor<4>(cv), Q, acc[3][1]);
            acc[3][2] = mma_kq(P[2] * pair_factor<5>(cv), Q, acc[3][2]);
        }
    }
}

template <class EK>
__device__ __forceinline__ void accumulate_slice(const Slice<EK> &sl, const f4 &wsel,
                                                 f4 (&acc)[4][4]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        typename Raw4<EK>::T kr[4];
        u4 graw[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            kr[b] = sl.k[b][t];
            graw[b] = sl.g[b][t];
        }
        accumulate_sub<EK>(kr, graw, wsel, acc);
    }
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
    SliceSrc<EK> src;
    src.rk = v.k.rows_from(0);
    src.rg = v.g.rows_from(0);
    src.offk = (uint32_t)(n * v.k.rstride + 8 * g4) * EK::kBytes;
    src.blk_k = (uint32_t)(16 * v.k.rstride) * EK::kBytes;
    src.upper = g4 >= 2;
    const uint32_t offg = (uint32_t)(n * v.g.rstride + 8 * g4) * F32::kBytes;
    const uint32_t blk_g = (uint32_t)(16 * v.g.rstride) * F32::kBytes;
    // Rows past a partial chunk read 0 keys (out of the descriptor's range)
    // and, instead of their own decays, those of their block's first row:
    // their factors are then 0 * 2^0 = 0 with no select, whatever the
    // decays' magnitude (a block wholly past the chunk reads 0 for both).
#pragma unroll
    for (int b = 0; b < 4; ++b)
        src.offgb[b] = (16 * b + n < len ? offg : (uint32_t)(8 * g4) * F32::kBytes) + b * blk_g;
    // the pair whose c_IJ this lane evaluates (lanes 6..15 of a row repeat
    // pair 0; nobody reads them)
    const int pn = n < 6 ? n : 0;
    const int pI = pn == 0 ? 1 : pn < 3 ? 2 : 3;
    const int pJ = pn == 0 || pn == 1 || pn == 3 ? 0 : pn == 2 || pn == 4 ? 1 : 2;
    f4 wsel;  // +1 at block I, -1 at block J of this lane's pair
#pragma unroll
    for (int b = 0; b < 4; ++b) wsel[b] = (float)((b == pI) - (b == pJ));
    // Each iteration issues all loads of a 32-channel slice (whole lines)
    // before any use; other wavefronts cover their latency.
#pragma unroll 1
    for (int d0 = 0; d0 < K; d0 += 32) {
        Slice<EK> sl;
        src.load(sl, d0, d0 + 32 > K);
        __builtin_amdgcn_sched_barrier(0);
        accumulate_slice<EK>(sl, wsel, acc);
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
    // Lanes right of the block row read column 0 of the staging (any value
    // in the wave's LDS would do) and store zeros: the read is unconditional,
    // so the compiler does not split each store into two partial-wave
    // stores under exec masks (each store instruction covers four whole rows).
    const bool in_row = c4 < 16 * (I + 1);
    const int cs = in_row ? c4 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + r4;
        const f4 sv = *reinterpret_cast<const f4 *>(&stage[row * S + cs]);
        store4<E>(X.rows_from(16 * I + 4 * i), off, in_row ? sv : z);
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
            // diagonal blocks to the row-per-lane layout of the diagonal solve:
            // acc[b][b] holds row n, columns 4g..4g+3 of block b in lane (g, n),
            // the layout diag_rows_from_blocks transposes with lane swaps
            const f4 dg[4] = {acc[0][0], acc[1][1], acc[2][2], acc[3][3]};
            float arow[16];
            diag_rows_from_blocks(dg, arow);
            wave_sync();  // the previous item's last LDS reads are done
            const MfmaEngine<kXsBlock, kXsCol> eng{xs, lane};
            diag_inverses(xs, arow, lane);
            merge_and_store<EO>(eng, acc, xs, X, lane);
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

// One wavefront per chunk-head, so the hardware dispatcher hands each free
// slot the next one (a grid of what the GPU holds at once, each wavefront
// walking a fixed share, was 1-3% slower with the same bits: 16 x 512 tokens,
// 64 heads, K = 128, bf16 keys 114.8-118.3 against 113.5-114.0 us, f32 keys
// 133.0-133.3 against 129.4-130.1); wavefronts walk only on a grid that
// KDA_TRIL_BLOCKS_PER_CU forces.
template <class Kern>
static hipError_t launch_kkt_kernel(Kern kernel, const KktProblem &q, hipStream_t stream) {
    const long waves = (long)q.p.slots * q.p.heads;
    const long blocks = blocks_forced() ? walk_blocks(reinterpret_cast<const void *>(kernel), waves,
                                                      min_chunks(q.p, kChunk) * q.p.heads)
                                        : (waves + kFusedWaves - 1) / kFusedWaves;
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
