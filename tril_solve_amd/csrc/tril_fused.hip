// Fused KDA chunk solver kernel for gfx950: one wavefront per chunk-head.
//
// LightLLM PR #1703 ("perf(kda): parallelize diagonal solves in Prefill",
// PR description): invert the four 16x16 diagonal blocks of every 64x64
// chunk matrix independently, then merge into the 64x64 inverse with FP32
// tiles. Everything for one chunk-head happens inside one wavefront: the
// tile goes HBM -> VGPRs (diagonal blocks also -> LDS), the inverse goes
// VGPRs -> HBM, and nothing else touches memory.
//
// Traffic per full chunk-head: the ten blocks on or below the diagonal of A
// are read (the six upper blocks are never needed, so never loaded) and all
// 64 rows x 64 columns of X are written.
#include "tril_device.h"
#include "tril_launch.h"

namespace kda {

template <class EI, class EO>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_fused_mfma(Problem p) {
    __shared__ float lds_all[kFusedWaves * kLdsPerWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    float *lds = lds_all + wid * kLdsPerWave;
    const long w = (long)blockIdx.x * kFusedWaves + wid;
    const int slot = (int)(w / p.heads);
    const int h = (int)(w - (long)slot * p.heads);
    if (slot >= p.slots) return;
    const Chunk ch = resolve_chunk(p, slot, lane);
    if (ch.len <= 0) return;

    const long rstride = (long)p.heads * kChunk;  // elements between tokens
    const long base = ((long)ch.start * p.heads + h) * kChunk;
    const typename EI::T *A = static_cast<const typename EI::T *>(p.A) + base;
    typename EO::T *X = static_cast<typename EO::T *>(p.X) + base;

    f4 blk[4][4];
    load_lower_blocks<EI>(blk, A, rstride, ch.len, lane, true, true);
    const f4 dA[4] = {blk[0][0], blk[1][1], blk[2][2], blk[3][3]};
    diag_inverses(lds, dA, lane);
    const MergeOut o = merge_mfma<kXsBlock, kXsCol>(lds, blk[1][0], blk[2][0], blk[2][1],
                                                    blk[3][0], blk[3][1], blk[3][2], lane);
    store_x<EO, kXsBlock, kXsCol>(X, rstride, ch.len, o, lds, lane);
}

// ------------------------------------------------------------------------
// Same kernel with the merge products on the vector ALUs (FP32 FMA) instead
// of the matrix cores; kept as the second precision mode and as the
// comparison point for the matrix-core merge.

constexpr int kScr = 20;                        // padded row stride of scratch
constexpr int kLdsPerWaveValu = kLdsPerWave + 2 * 16 * kScr;

// acc + P * Q for P in OPND_A, Q in OPND_O; result in OPND_O. Both operands
// go through LDS: lane (g, n) needs rows 4g..4g+3 of P and column n of Q.
__device__ __forceinline__ f4 valu_mm(float *ps, float *qs, f4 P, f4 Q, f4 acc, int lane) {
    const int g = lane >> 4, m = lane & 15;
    *reinterpret_cast<f4 *>(&ps[m * kScr + 4 * g]) = P;  // row m
    *reinterpret_cast<f4 *>(&qs[m * kScr + 4 * g]) = Q;  // column m
    wave_sync();
    f4 qc[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) qc[kq] = *reinterpret_cast<const f4 *>(&qs[m * kScr + 4 * kq]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float a = acc[r];
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            const f4 pr = *reinterpret_cast<const f4 *>(&ps[(4 * g + r) * kScr + 4 * kq]);
#pragma unroll
            for (int e = 0; e < 4; ++e) a = __builtin_fmaf(pr[e], qc[kq][e], a);
        }
        acc[r] = a;
    }
    wave_sync();
    return acc;
}

// -X_II * S with X_II read from its column-major LDS copy; S in OPND_O.
__device__ __forceinline__ f4 valu_neg_xii(const float *xs, float *qs, int I, f4 S, int lane) {
    const int g = lane >> 4, m = lane & 15;
    *reinterpret_cast<f4 *>(&qs[m * kScr + 4 * g]) = S;
    wave_sync();
    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
        const f4 sc = *reinterpret_cast<const f4 *>(&qs[m * kScr + 4 * kq]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = 4 * kq + e;
            const f4 col = *reinterpret_cast<const f4 *>(&xs[I * kXsBlock + k * kXsCol + 4 * g]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(-col[r], sc[e], acc[r]);
        }
    }
    wave_sync();
    return acc;
}

template <class EI, class EO>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_fused_valu(Problem p) {
    __shared__ float lds_all[kFusedWaves * kLdsPerWaveValu];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    float *lds = lds_all + wid * kLdsPerWaveValu;
    float *ps = lds + kLdsPerWave;
    float *qs = ps + 16 * kScr;
    const long w = (long)blockIdx.x * kFusedWaves + wid;
    const int slot = (int)(w / p.heads);
    const int h = (int)(w - (long)slot * p.heads);
    if (slot >= p.slots) return;
    const Chunk ch = resolve_chunk(p, slot, lane);
    if (ch.len <= 0) return;

    const long rstride = (long)p.heads * kChunk;
    const long base = ((long)ch.start * p.heads + h) * kChunk;
    const typename EI::T *A = static_cast<const typename EI::T *>(p.A) + base;
    typename EO::T *X = static_cast<typename EO::T *>(p.X) + base;

    f4 blk[4][4];
    load_lower_blocks<EI>(blk, A, rstride, ch.len, lane, true, true);
    const f4 dA[4] = {blk[0][0], blk[1][1], blk[2][2], blk[3][3]};
    diag_inverses(lds, dA, lane);

    const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    const f4 x00 = xs_opnd_o<kXsBlock, kXsCol>(lds, 0, lane);
    const f4 x11 = xs_opnd_o<kXsBlock, kXsCol>(lds, 1, lane);
    const f4 x22 = xs_opnd_o<kXsBlock, kXsCol>(lds, 2, lane);
    MergeOut o;
    const f4 s10 = valu_mm(ps, qs, blk[1][0], x00, z, lane);
    const f4 s21 = valu_mm(ps, qs, blk[2][1], x11, z, lane);
    const f4 s32 = valu_mm(ps, qs, blk[3][2], x22, z, lane);
    f4 s20 = valu_mm(ps, qs, blk[2][0], x00, z, lane);
    f4 s31 = valu_mm(ps, qs, blk[3][1], x11, z, lane);
    f4 s30 = valu_mm(ps, qs, blk[3][0], x00, z, lane);
    o.x10 = valu_neg_xii(lds, qs, 1, s10, lane);
    o.x21 = valu_neg_xii(lds, qs, 2, s21, lane);
    o.x32 = valu_neg_xii(lds, qs, 3, s32, lane);
    s20 = valu_mm(ps, qs, blk[2][1], o.x10, s20, lane);
    s31 = valu_mm(ps, qs, blk[3][2], o.x21, s31, lane);
    s30 = valu_mm(ps, qs, blk[3][1], o.x10, s30, lane);
    o.x20 = valu_neg_xii(lds, qs, 2, s20, lane);
    o.x31 = valu_neg_xii(lds, qs, 3, s31, lane);
    s30 = valu_mm(ps, qs, blk[3][2], o.x20, s30, lane);
    o.x30 = valu_neg_xii(lds, qs, 3, s30, lane);
    store_x<EO, kXsBlock, kXsCol>(X, rstride, ch.len, o, lds, lane);
}

template <class EI, class EO>
static hipError_t launch_valu_t(const Problem &p, hipStream_t stream) {
    const long waves = (long)p.slots * p.heads;
    const long blocks = (waves + kFusedWaves - 1) / kFusedWaves;
    hipLaunchKernelGGL((tril_inv_fused_valu<EI, EO>), dim3((unsigned)blocks), dim3(kFusedThreads),
                       0, stream, p);
    return hipGetLastError();
}

hipError_t launch_fused_valu(const Problem &p, int a_bf16, int x_bf16, hipStream_t stream) {
    if (!a_bf16 && !x_bf16) return launch_valu_t<F32, F32>(p, stream);
    if (!a_bf16 && x_bf16) return launch_valu_t<F32, BF16>(p, stream);
    if (a_bf16 && !x_bf16) return launch_valu_t<BF16, F32>(p, stream);
    return launch_valu_t<BF16, BF16>(p, stream);
}

template <class EI, class EO>
static hipError_t launch_fused_t(const Problem &p, hipStream_t stream) {
    const long waves = (long)p.slots * p.heads;
    const long blocks = (waves + kFusedWaves - 1) / kFusedWaves;
    hipLaunchKernelGGL((tril_inv_fused_mfma<EI, EO>), dim3((unsigned)blocks), dim3(kFusedThreads),
                       0, stream, p);
    return hipGetLastError();
}

hipError_t launch_fused_mfma(const Problem &p, int a_bf16, int x_bf16, hipStream_t stream) {
    if (!a_bf16 && !x_bf16) return launch_fused_t<F32, F32>(p, stream);
    if (!a_bf16 && x_bf16) return launch_fused_t<F32, BF16>(p, stream);
    if (a_bf16 && !x_bf16) return launch_fused_t<BF16, F32>(p, stream);
    return launch_fused_t<BF16, BF16>(p, stream);
}

}  // namespace kda
