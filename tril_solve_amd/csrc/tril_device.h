// Device-side building blocks of the KDA chunk solver for gfx950 (CDNA4).
//
// One wavefront (64 lanes) owns one chunk-head matrix M = I + A, 64 x 64,
// split into 4 x 4 blocks of 16 x 16 (block row I, block column K, 0-based).
// LightLLM PR #1703 ("perf(kda): parallelize diagonal solves in Prefill",
// commit summary and PR description) inverts the four diagonal blocks
// independently and then merges, keeping FP32 tiles until the store. Here:
//
//   * the four diagonal inverses X_KK = (I + A_KK)^-1 run at once, one lane
//     per (block K, column c) doing a 16-step forward substitution with the
//     block's rows broadcast from LDS;
//   * the merge uses X_IJ = -X_II * sum_{K=J}^{I-1} A_IK X_KJ for I > J, in
//     three levels ({X10, X21, X32}, {X20, X31}, {X30}), every 16 x 16 x 16
//     product being four v_mfma_f32_16x16x4_f32 (or VALU FMAs);
//   * the tiles stay FP32 and are rounded once at the store.
//
// Register layouts (lane l, g = l / 16, m = l % 16):
//   OPND_A  lane (g, m) holds row m, columns 4g..4g+3 of a block (float4).
//           It is the A operand of the 16x16x4 MFMA at step s (reg s),
//           with the reduction index permuted as k = 4g + s.
//   OPND_O  lane (g, n) holds rows 4g..4g+3 of column n (float4). It is the
//           MFMA accumulator layout, and with the same permutation of k it is
//           directly the B operand: reg s = row 4g + s. So a product result
//           feeds the next product with no data movement.
//   STORE   lane (g, 4q + t) holds row 4g + t, columns 4q..4q+3 (float4),
//           obtained from OPND_O by a 4 x 4 transpose inside each lane quad.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tril_launch.h"

namespace kda {

constexpr int kChunk = 64;
constexpr int kWave = 64;

typedef float f4 __attribute__((ext_vector_type(4)));

// LDS per wave (floats). The diagonal A blocks (row-major, block stride
// kDiagStride) and, after the substitution, the diagonal inverses
// (column-major: column c of block K at K * kXsBlock + c * kXsCol) share it.
constexpr int kDiagStride = 16 * 16 + 4;
constexpr int kXsCol = 20;
constexpr int kXsBlock = 16 * kXsCol;
constexpr int kLdsPerWave = 4 * kXsBlock;  // 1280 floats = 5 KiB
static_assert(4 * kDiagStride <= kLdsPerWave, "diag A must fit in the wave's LDS");

// Orders LDS traffic between lanes of one wavefront (no s_barrier: LDS is
// processed in order per wave; this stops the compiler from moving accesses).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- element I/O

struct F32 {
    typedef float T;
    static constexpr int kBytes = 4;
};
struct BF16 {
    typedef uint16_t T;
    static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
    return __builtin_bit_cast(float, b << 16);
}

// Four consecutive elements -> float4 (bf16 -> f32 is exact).
template <class E>
__device__ __forceinline__ f4 load4(const typename E::T *p);
template <>
__device__ __forceinline__ f4 load4<F32>(const float *p) {
    return *reinterpret_cast<const f4 *>(p);
}
template <>
__device__ __forceinline__ f4 load4<BF16>(const uint16_t *p) {
    uint2 v = *reinterpret_cast<const uint2 *>(p);
    f4 r;
    r[0] = bf16_to_f32(v.x & 0xFFFFu);
    r[1] = bf16_to_f32(v.x >> 16);
    r[2] = bf16_to_f32(v.y & 0xFFFFu);
    r[3] = bf16_to_f32(v.y >> 16);
    return r;
}

// float4 -> four consecutive elements. bf16 uses the hardware round to
// nearest even (v_cvt_pk_bf16_f32).
template <class E>
__device__ __forceinline__ void store4(typename E::T *p, f4 v);
template <>
__device__ __forceinline__ void store4<F32>(float *p, f4 v) {
    *reinterpret_cast<f4 *>(p) = v;
}
template <>
__device__ __forceinline__ void store4<BF16>(uint16_t *p, f4 v) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 lo = {(__bf16)v[0], (__bf16)v[1]};
    b2 hi = {(__bf16)v[2], (__bf16)v[3]};
    uint2 o;
    o.x = __builtin_bit_cast(uint32_t, lo);
    o.y = __builtin_bit_cast(uint32_t, hi);
    *reinterpret_cast<uint2 *>(p) = o;
}

// ------------------------------------------------------------ chunk resolution

struct Chunk {
    int32_t start;  // first token (row) of the chunk
    int32_t len;    // valid rows, 1..64 (0: nothing to do)
};

// wave-wide inclusive prefix sum of an int
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// Resolve chunk slot k (wave-uniform) to rows of A/X. Returns len 0 when the
// slot is past the last chunk. Dense: chunk c of batch b starts at b*T + 64c.
// Packed: slots enumerate chunks in packed order; with a chunk map the slot
// indexes it, else the wave scans cu_seqlens 64 requests at a time.
__device__ __forceinline__ Chunk resolve_chunk(const Problem &p, int k, int lane) {
    Chunk ch{0, 0};
    if (p.cu == nullptr) {
        const int per = (p.seq_len + kChunk - 1) / kChunk;
        const int b = k / per, c = k - b * per;
        if (b < p.num_seqs) {
            ch.start = b * p.seq_len + c * kChunk;
            ch.len = min(kChunk, p.seq_len - c * kChunk);
        }
        return ch;
    }
    int bos = 0, eos = 0;
    if (p.cmap != nullptr) {
        const int s = p.cmap[2 * k], c = p.cmap[2 * k + 1];
        if (s < 0 || s >= p.num_seqs || c < 0) return ch;
        bos = p.cu[s] + c * kChunk;
        eos = p.cu[s + 1];
    } else {
        int base = 0;
        bool found = false;
        for (int s0 = 0; s0 < p.num_seqs; s0 += kWave) {
            const int s = s0 + lane;
            int cnt = 0, b0 = 0, e0 = 0;
            if (s < p.num_seqs) {
                b0 = p.cu[s];
                e0 = p.cu[s + 1];
                cnt = e0 > b0 ? (e0 - b0 + kChunk - 1) / kChunk : 0;
            }
            const int incl = wave_incl_scan(cnt, lane);
            const int total = __shfl(incl, kWave - 1, kWave);
            if (k < base + total) {
                const bool hit = (k >= base + incl - cnt) && (k < base + incl);
                const unsigned long long m = __ballot(hit);
                const int src = __builtin_ctzll(m);
                const int first = base + __shfl(incl - cnt, src, kWave);
                bos = __shfl(b0, src, kWave) + (k - first) * kChunk;
                eos = __shfl(e0, src, kWave);
                found = true;
                break;
            }
            base += total;
        }
        if (!found) return ch;
    }
    // Clamp to the rows of the tensors so a malformed cu_seqlens cannot
    // address memory outside A and X.
    if (bos < 0 || bos >= p.total_tokens || eos <= bos) return ch;
    eos = min(eos, p.total_tokens);
    ch.start = bos;
    ch.len = min(kChunk, eos - bos);
    return ch;
}

// ------------------------------------------------------------ small helpers

// 4 x 4 transpose inside each lane quad: in reg r of lane t (t = l % 4) the
// value V[t][r]; out reg r of lane t holds V[r][t]. Two DPP swap stages.
__device__ __forceinline__ float dpp_swap1(float v) {  // quad_perm [1,0,3,2]
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1,
                                                              0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_swap2(float v) {  // quad_perm [2,3,0,1]
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E,
                                                              0xF, 0xF, false));
}
__device__ __forceinline__ f4 quad_transpose(f4 v, int lane) {
    const bool t0 = lane & 1, t1 = lane & 2;
    f4 u;
    {
        const float a0 = dpp_swap1(v[0]), a1 = dpp_swap1(v[1]);
        const float a2 = dpp_swap1(v[2]), a3 = dpp_swap1(v[3]);
        u[0] = t0 ? a1 : v[0];
        u[1] = t0 ? v[1] : a0;
        u[2] = t0 ? a3 : v[2];
        u[3] = t0 ? v[3] : a2;
    }
    f4 w;
    {
        const float b0 = dpp_swap2(u[0]), b1 = dpp_swap2(u[1]);
        const float b2 = dpp_swap2(u[2]), b3 = dpp_swap2(u[3]);
        w[0] = t1 ? b2 : u[0];
        w[1] = t1 ? b3 : u[1];
        w[2] = t1 ? u[2] : b0;
        w[3] = t1 ? u[3] : b1;
    }
    return w;
}

// 16 x 16 x 16 product on the matrix cores: acc + P * Q with P in OPND_A and
// Q in OPND_O layout (reduction index k = 4g + s at step s).
__device__ __forceinline__ f4 mma16(f4 P, f4 Q, f4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(P[0], Q[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(P[1], Q[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(P[2], Q[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(P[3], Q[3], acc, 0, 0, 0);
    return acc;
}

// --------------------------------------------------- diagonal block inverses

// Input: lane (g, i) holds row i, columns 4g..4g+3 of each diagonal block
// A_KK (OPND_A layout, rows past the chunk already zero). Stores the strictly
// lower part (others forced to 0 by select, so NaN/Inf there cannot leak) to
// LDS, runs the four 16-step forward substitutions, one lane per
// (block b = lane / 16, column c = lane % 16), and leaves X_KK column-major in
// LDS: column c of block K at lds[K * kXsBlock + c * kXsCol + row].
__device__ __forceinline__ void diag_inverses(float *lds, const f4 dA[4], int lane) {
    const int g = lane >> 4, m = lane & 15;
#pragma unroll
    for (int K = 0; K < 4; ++K) {
        f4 v;
#pragma unroll
        for (int s = 0; s < 4; ++s) v[s] = (4 * g + s < m) ? dA[K][s] : 0.0f;
        *reinterpret_cast<f4 *>(&lds[K * kDiagStride + m * 16 + 4 * g]) = v;
    }
    wave_sync();
    const int b = g, c = m;
    const float *row = lds + b * kDiagStride;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.0f : 0.0f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int q = 0; q < (i + 3) / 4; ++q) {
            const f4 a = *reinterpret_cast<const f4 *>(&row[i * 16 + 4 * q]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * q + e < i) acc = __builtin_fmaf(a[e], x[4 * q + e], acc);
        }
        x[i] = (i > c) ? -acc : x[i];
    }
    wave_sync();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f4 v = {x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
        *reinterpret_cast<f4 *>(&lds[b * kXsBlock + c * kXsCol + 4 * q]) = v;
    }
    wave_sync();
}

// X_KK from a column-major copy (LDS or the split workspace) in the three
// register layouts. Column c of block K starts at K * BS + c * CS.
template <int BS, int CS>
__device__ __forceinline__ f4 xs_opnd_o(const float *xs, int K, int lane) {
    const int g = lane >> 4, n = lane & 15;
    return *reinterpret_cast<const f4 *>(&xs[K * BS + n * CS + 4 * g]);
}
template <int BS, int CS>
__device__ __forceinline__ f4 xs_opnd_a_neg(const float *xs, int K, int lane) {
    const int g = lane >> 4, m = lane & 15;
    f4 r;
#pragma unroll
    for (int s = 0; s < 4; ++s) r[s] = -xs[K * BS + (4 * g + s) * CS + m];
    return r;
}
template <int BS, int CS>
__device__ __forceinline__ f4 xs_store(const float *xs, int K, int lane) {
    const int g = lane >> 4, q = (lane >> 2) & 3, t = lane & 3;
    f4 r;
#pragma unroll
    for (int s = 0; s < 4; ++s) r[s] = xs[K * BS + (4 * q + s) * CS + 4 * g + t];
    return r;
}

// Merge products on the matrix cores: A blocks in OPND_A layout, diagonal
// inverses from a column-major copy; results X_IJ (I > J) in OPND_O layout.
struct MergeOut {
    f4 x10, x21, x32, x20, x31, x30;
};

template <int BS, int CS>
__device__ __forceinline__ MergeOut merge_mfma(const float *xs, const f4 a10, const f4 a20,
                                               const f4 a21, const f4 a30, const f4 a31,
                                               const f4 a32, int lane) {
    const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    const f4 x00 = xs_opnd_o<BS, CS>(xs, 0, lane);
    const f4 x11 = xs_opnd_o<BS, CS>(xs, 1, lane);
    const f4 x22 = xs_opnd_o<BS, CS>(xs, 2, lane);
    const f4 n11 = xs_opnd_a_neg<BS, CS>(xs, 1, lane);
    const f4 n22 = xs_opnd_a_neg<BS, CS>(xs, 2, lane);
    const f4 n33 = xs_opnd_a_neg<BS, CS>(xs, 3, lane);
    MergeOut o;
    // level 1, plus the first terms of levels 2 and 3 (they need only X_KK)
    const f4 s10 = mma16(a10, x00, z);
    const f4 s21 = mma16(a21, x11, z);
    const f4 s32 = mma16(a32, x22, z);
    f4 s20 = mma16(a20, x00, z);
    f4 s31 = mma16(a31, x11, z);
    f4 s30 = mma16(a30, x00, z);
    o.x10 = mma16(n11, s10, z);
    o.x21 = mma16(n22, s21, z);
    o.x32 = mma16(n33, s32, z);
    // level 2
    s20 = mma16(a21, o.x10, s20);
    s31 = mma16(a32, o.x21, s31);
    s30 = mma16(a31, o.x10, s30);
    o.x20 = mma16(n22, s20, z);
    o.x31 = mma16(n33, s31, z);
    // level 3
    s30 = mma16(a32, o.x20, s30);
    o.x30 = mma16(n33, s30, z);
    return o;
}

// Loads of the blocks on and below the diagonal: lane (g, m) takes row
// 16I + m, columns 16K + 4g..+3 of block (I, K), K <= I (and K >= kmin).
// Rows at or past `len` read as 0.
template <class E>
__device__ __forceinline__ void load_lower_blocks(f4 blk[4][4], const typename E::T *A, long rstride,
                                                  int len, int lane, bool diag, bool offdiag) {
    const int g = lane >> 4, m = lane & 15;
    const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        const int r = 16 * I + m;
        const bool ok = r < len;
        const typename E::T *row = A + (long)r * rstride + 4 * g;
#pragma unroll
        for (int K = 0; K <= I; ++K) {
            const bool want = (K == I) ? diag : offdiag;
            blk[I][K] = (want && ok) ? load4<E>(row + 16 * K) : z;
        }
    }
}

// Writes the 64 rows of X for one chunk-head: row-block I gets X_IJ (J < I)
// from OPND_O registers, X_II from the column-major copy, zeros for J > I.
// Lane (g, 4q + t) writes row 16I + 4g + t, columns 16J + 4q..+3; rows at or
// past `len` are not written.
template <class E, int BS, int CS>
__device__ __forceinline__ void store_x(typename E::T *X, long rstride, int len, const MergeOut &o,
                                        const float *xs, int lane) {
    const int g = lane >> 4, q = (lane >> 2) & 3, t = lane & 3;
    const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    const f4 xo[4][4] = {
        {z, z, z, z},
        {o.x10, z, z, z},
        {o.x20, o.x21, z, z},
        {o.x30, o.x31, o.x32, z},
    };
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        // DPP transposes read neighbouring lanes, so they run with every lane
        // active; only the stores are masked by row.
        f4 v[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            if (J < I)
                v[J] = quad_transpose(xo[I][J], lane);
            else if (J == I)
                v[J] = xs_store<BS, CS>(xs, I, lane);
            else
                v[J] = z;
        }
        const int r = 16 * I + 4 * g + t;
        if (r < len) {
            typename E::T *row = X + (long)r * rstride + 4 * q;
#pragma unroll
            for (int J = 0; J < 4; ++J) store4<E>(row + 16 * J, v[J]);
        }
    }
}

}  // namespace kda
