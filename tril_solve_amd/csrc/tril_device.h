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

// LDS per wave (floats): the diagonal inverses, column-major (column c of
// block K at K * kXsBlock + c * kXsCol). The output staging of block row I
// (16 rows x 16(I + 1) columns, row stride 16(I + 1) + 4) reuses the same
// region: by the time block row I is staged, every value of blocks 0..I that
// is still needed has been read into registers.
constexpr int kXsCol = 20;
constexpr int kXsBlock = 16 * kXsCol;
constexpr int kXsFloats = 4 * kXsBlock;  // 1280 floats = 5 KiB
constexpr int kLdsPerWave = kXsFloats;
__host__ __device__ constexpr int stage_row(int I) { return 16 * (I + 1) + 4; }
static_assert(16 * stage_row(3) <= kXsFloats, "the staging of a block row must fit");

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
struct F16 {
    typedef uint16_t T;
    static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
    return __builtin_bit_cast(float, b << 16);
}

// Tile I/O goes through buffer resources: a 128-bit descriptor (kept in
// SGPRs) whose num_records ends right after the last valid row of the
// chunk-head. The hardware range check then returns 0 for loads of rows past
// the chunk and drops stores to them, so loads and stores need no per-row
// branches (and the wave's memory-counter waits stay exact).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) access, gfx9-family layout

// Rows 0..len-1 (len >= 1) of one chunk-head (or of a few adjacent heads of
// one chunk), row r at base + r * rstride elements, `width` elements used per
// row. Descriptors are made per group of rows at the point of use (a few
// scalar instructions) so the row part of every address lives in SGPRs and a
// single per-lane offset VGPR serves all loads or stores of a tile.
template <class E>
struct TileView {
    const typename E::T *base;
    int rstride;  // elements between consecutive rows
    int len;      // valid rows
    int width;    // elements of a row that belong to the view (<= rstride)

    // Descriptor whose byte 0 is row r0; its range ends after the `width`
    // elements of row len-1, so rows at or past len (relative offsets from
    // row r0 onward) are out of range: loads return 0, stores are dropped.
    __device__ __forceinline__ Rsrc rows_from(int r0) const {
        const int valid = len - r0;  // rows from r0 on that exist
        const uint32_t n =
            valid > 0 ? (uint32_t)((valid - 1) * rstride + width) * E::kBytes : 0u;
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<typename E::T *>(base + (long)r0 * rstride), 0, n, kRsrcWord3);
    }
};

// Four consecutive elements at byte offset `off` -> float4 (bf16 -> f32 is
// exact); 0 past the descriptor's range.
template <class E>
__device__ __forceinline__ f4 load4(Rsrc r, uint32_t off);
template <>
__device__ __forceinline__ f4 load4<F32>(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <>
__device__ __forceinline__ f4 load4<BF16>(Rsrc r, uint32_t off) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    f4 o;
    o[0] = bf16_to_f32(v[0] & 0xFFFFu);
    o[1] = bf16_to_f32(v[0] >> 16);
    o[2] = bf16_to_f32(v[1] & 0xFFFFu);
    o[3] = bf16_to_f32(v[1] >> 16);
    return o;
}

template <>
__device__ __forceinline__ f4 load4<F16>(Rsrc r, uint32_t off) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 v = __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    f4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (float)v[e];  // exact widening
    return o;
}

// float4 -> four consecutive elements at byte offset `off`; dropped past the
// descriptor's range. X is written once and never read again here: the stores
// carry the nontemporal bit and device scope, so the lines go out through L2
// without displacing cached lines (on 16 x 512 tokens, 64 heads: 1.6% faster
// than nontemporal alone, 4% faster than the default write-back policy; device
// scope alone was no better than the default). bf16 uses the hardware round
// to nearest even (v_cvt_pk_bf16_f32), binary16 the IEEE conversion in the
// default round-to-nearest-even mode.
constexpr int kNontemporal = 2;   // cache-policy bit: nontemporal (loads and stores)
constexpr int kScopeDevice = 16;  // cache-policy bit: device scope
constexpr int kStorePolicy = kScopeDevice | kNontemporal;
template <class E>
__device__ __forceinline__ void store4(Rsrc r, uint32_t off, f4 v);
template <>
__device__ __forceinline__ void store4<F32>(Rsrc r, uint32_t off, f4 v) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, kStorePolicy);
}
template <>
__device__ __forceinline__ void store4<BF16>(Rsrc r, uint32_t off, f4 v) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const b2 lo = {(__bf16)v[0], (__bf16)v[1]};
    const b2 hi = {(__bf16)v[2], (__bf16)v[3]};
    const u2 o = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    __builtin_amdgcn_raw_buffer_store_b64(o, r, off, 0, kStorePolicy);
}
template <>
__device__ __forceinline__ void store4<F16>(Rsrc r, uint32_t off, f4 v) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    h4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (_Float16)v[e];  // v_cvt_f16_f32, round to nearest even
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, h), r, off, 0, kStorePolicy);
}

// Single elements, for the kernels that give every lane one column of a
// matrix (each load or store instruction then covers whole adjacent rows).
template <class E>
__device__ __forceinline__ float load1(Rsrc r, uint32_t off);
template <>
__device__ __forceinline__ float load1<F32>(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <>
__device__ __forceinline__ float load1<BF16>(Rsrc r, uint32_t off) {
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}
template <>
__device__ __forceinline__ float load1<F16>(Rsrc r, uint32_t off) {
    return (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}

template <class E>
__device__ __forceinline__ void store1(Rsrc r, uint32_t off, float v);
template <>
__device__ __forceinline__ void store1<F32>(Rsrc r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0,
                                          kStorePolicy);
}
template <>
__device__ __forceinline__ void store1<BF16>(Rsrc r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)v), r, off, 0,
                                          kStorePolicy);
}
template <>
__device__ __forceinline__ void store1<F16>(Rsrc r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)v), r, off, 0,
                                          kStorePolicy);
}

// Byte offset that is out of range of every descriptor above (their ranges
// stay below 2 GiB): OR-ed into the offsets of lanes that must not touch
// memory, so their loads return 0 and their stores are dropped.
constexpr uint32_t kOffMasked = 0x80000000u;

// ------------------------------------------------------------ chunk resolution

struct Chunk {
    int32_t start;  // first token (row) of the chunk
    int32_t len;    // valid rows, 1..C (0: nothing to do)
};

// Wave-wide inclusive prefix sum of an int, on DPP lane moves (no LDS round
// trips): a Hillis-Steele scan inside each 16-lane row (row_shr by 1, 2, 4,
// 8; lanes shifted in from outside the row read 0), then the last lane of
// row 0 / 2 is added to row 1 / 3 (row_bcast:15) and the last lane of row 1
// to rows 2 and 3 (row_bcast:31). Lanes a move does not write keep 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_or_zero(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += dpp_or_zero<0x111, 0xF>(v);  // row_shr:1
    v += dpp_or_zero<0x112, 0xF>(v);  // row_shr:2
    v += dpp_or_zero<0x114, 0xF>(v);  // row_shr:4
    v += dpp_or_zero<0x118, 0xF>(v);  // row_shr:8
    v += dpp_or_zero<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_or_zero<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Value of v in lane `src` (wave-uniform) for the whole wave.
__device__ __forceinline__ int lane_value(int v, int src) {
    return __builtin_amdgcn_readlane(v, src);
}

// Resolve chunk slot k (wave-uniform) to rows of A/X for chunks of C tokens.
// Returns len 0 when the slot is past the last chunk. Dense: chunk c of batch
// b starts at b*T + C*c. Packed: slots enumerate chunks in packed order; with
// a chunk map the slot indexes it, else the wave scans cu_seqlens 64 requests
// at a time.
template <int C>
__device__ __forceinline__ Chunk resolve_chunk(const Problem &p, int k, int lane) {
    Chunk ch{0, 0};
    if (p.cu == nullptr) {
        const int per = (p.seq_len + C - 1) / C;
        const int b = k / per, c = k - b * per;
        if (b < p.num_seqs) {
            ch.start = b * p.seq_len + c * C;
            ch.len = min(C, p.seq_len - c * C);
        }
        return ch;
    }
    int bos = 0, eos = 0;
    if (p.cmap != nullptr) {
        const int s = p.cmap[2 * k], c = p.cmap[2 * k + 1];
        if (s < 0 || s >= p.num_seqs || c < 0) return ch;
        bos = p.cu[s] + c * C;
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
                cnt = e0 > b0 ? (e0 - b0 + C - 1) / C : 0;
            }
            const int incl = wave_incl_scan(cnt);
            const int total = lane_value(incl, kWave - 1);
            if (k < base + total) {
                const bool hit = (k >= base + incl - cnt) && (k < base + incl);
                const unsigned long long m = __ballot(hit);
                const int src = __builtin_ctzll(m);
                const int first = base + lane_value(incl - cnt, src);
                bos = lane_value(b0, src) + (k - first) * C;
                eos = lane_value(e0, src);
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
    ch.len = min(C, eos - bos);
    return ch;
}

// The chunk is the same for every lane of the wave: keep it in SGPRs so the
// tile's base pointers and row arithmetic stay scalar.
__device__ __forceinline__ Chunk uniform(Chunk c) {
    c.start = __builtin_amdgcn_readfirstlane(c.start);
    c.len = __builtin_amdgcn_readfirstlane(c.len);
    return c;
}

// The lane index made opaque to the optimiser: values derived from it are
// then recomputed where used instead of being hoisted out of the walk over
// work items and held in registers for the kernel's lifetime.
__device__ __forceinline__ int opaque_lane(int lane) {
    asm volatile("" : "+v"(lane));
    return lane;
}

// ------------------------------------------------------------ small helpers

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

// Value of v in lane I of this lane's 16-lane row (DPP row_newbcast). Every
// lane's source lane exists, so no "old" value is needed (an explicit one
// costs a move and a hazard wait per broadcast).
template <int I>
__device__ __forceinline__ float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                              0x150 + I, 0xF, 0xF, true));
}

// Row I of the substitution: x_I = -sum_{j<I} A[I][j] x_j (j increasing),
// kept only below the diagonal (x_I stays 0 above it and 1 on it).
template <int I>
__device__ __forceinline__ void subst_row(const float (&arow)[16], float (&x)[16], int c) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < I; ++j) acc = __builtin_fmaf(row_bcast<I>(arow[j]), x[j], acc);
    x[I] = (I > c) ? -acc : x[I];
}

// Four 16x16 forward substitutions at once, one lane per (block b, column
// c), b = lane / 16, c = lane % 16. Input: lane (b, i) holds row i of the
// diagonal block A_bb (16 floats, rows past the chunk already 0); entry
// A_bb[i][j] reaches the lanes of row b through a DPP broadcast from lane i,
// and only j < i is ever broadcast, so whatever is stored on or above the
// diagonal of A never enters the arithmetic. Output: X_bb column-major in
// LDS, column c of block b at xs[b * kXsBlock + c * kXsCol + row].
__device__ __forceinline__ void diag_inverses(float *xs, const float (&arow)[16], int lane) {
    const int b = lane >> 4, c = lane & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.0f : 0.0f;
    subst_row<1>(arow, x, c);
    subst_row<2>(arow, x, c);
    subst_row<3>(arow, x, c);
    subst_row<4>(arow, x, c);
    subst_row<5>(arow, x, c);
    subst_row<6>(arow, x, c);
    subst_row<7>(arow, x, c);
    subst_row<8>(arow, x, c);
    subst_row<9>(arow, x, c);
    subst_row<10>(arow, x, c);
    subst_row<11>(arow, x, c);
    subst_row<12>(arow, x, c);
    subst_row<13>(arow, x, c);
    subst_row<14>(arow, x, c);
    subst_row<15>(arow, x, c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f4 v = {x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
        *reinterpret_cast<f4 *>(&xs[b * kXsBlock + c * kXsCol + 4 * q]) = v;
    }
    wave_sync();
}

// Lane (g, m) loads row 16b + m, columns 16b + 4g..16b + 4g + 3 of diagonal
// block b into d[b], b = 0..3, so every load instruction covers 16 rows x 64
// contiguous bytes (as the off-diagonal loads do) rather than 64 rows x 16
// bytes. Rows past the chunk read as 0.
template <class E>
__device__ __forceinline__ void load_diag_blocks(f4 (&d)[4], const TileView<E> &A, int lane) {
    const int g = lane >> 4, m = lane & 15;
    const uint32_t off = (uint32_t)(m * A.rstride + 4 * g) * E::kBytes;
#pragma unroll
    for (int b = 0; b < 4; ++b) d[b] = load4<E>(A.rows_from(16 * b), off + 16 * b * E::kBytes);
}

// load_diag_blocks' layout -> one row per lane: lane (b, i) gets row i of
// diagonal block b, column c in arow[c]. Taking d[b] in 16-lane row g as
// entry (g, b) of a 4 x 4 matrix (each entry a float4), this is the matrix's
// transpose, done by lane swaps between registers without LDS:
// v_permlane32_swap exchanges lane rows 2-3 of d[b] with lane rows 0-1 of
// d[b + 2] (b = 0, 1), then v_permlane16_swap exchanges lane rows 1 and 3 of
// d[b] with lane rows 0 and 2 of d[b + 1] (b = 0, 2).
//
// The swaps are written as instructions rather than through the compiler's
// two-result builtins, whose second result this compiler lost (it folded the
// swapped values of elements 1-3 away). Both registers are read and written
// by each swap; the s_nop pairs keep two wait states around it (the hardware
// needs them between a swap's results and their next read).
__device__ __forceinline__ void lane_swap32(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void lane_swap16(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void diag_rows_from_blocks(const f4 (&d)[4], float (&arow)[16]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float r0 = d[0][e], r1 = d[1][e], r2 = d[2][e], r3 = d[3][e];
        lane_swap32(r0, r2);
        lane_swap32(r1, r3);
        lane_swap16(r0, r1);
        lane_swap16(r2, r3);
        arow[e] = r0;
        arow[4 + e] = r1;
        arow[8 + e] = r2;
        arow[12 + e] = r3;
    }
}

// Lane (b, i) loads row 16b + i, columns 16b + 4q..16b + 4q + 3 into r[q]
// (the row of diagonal block b as four float4): one row per lane, so each of
// the four load instructions touches 64 rows, and the rows need no transpose.
template <class E>
__device__ __forceinline__ void load_diag_row_quads(f4 (&r)[4], const TileView<E> &A, int lane) {
    const int b = lane >> 4, i = lane & 15;
    const Rsrc rs = A.rows_from(0);
    const uint32_t off = (uint32_t)((16 * b + i) * A.rstride + 16 * b) * E::kBytes;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = load4<E>(rs, off + 4 * q * E::kBytes);
}

// Lane (b, i) gets row 16b + i, columns 16b..16b+15 (the row of diagonal
// block b); rows past the chunk read as 0.
template <class E>
__device__ __forceinline__ void load_diag_rows(float (&arow)[16], const TileView<E> &A, int lane) {
    f4 d[4];
    load_diag_blocks<E>(d, A, lane);
    diag_rows_from_blocks(d, arow);
}

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
// Loads of the six blocks below the diagonal: lane (g, m) takes row
// 16I + m, columns 16K + 4g..+3 of block (I, K), K < I (OPND_A layout).
// Rows past the chunk read as 0.
template <class E>
__device__ __forceinline__ void load_offdiag_blocks(f4 (&blk)[4][4], const TileView<E> &A,
                                                    int lane) {
    const int g = lane >> 4, m = lane & 15;
    const uint32_t off = (uint32_t)(m * A.rstride + 4 * g) * E::kBytes;
#pragma unroll
    for (int I = 1; I < 4; ++I) {
        const Rsrc r = A.rows_from(16 * I);
#pragma unroll
        for (int K = 0; K < I; ++K) blk[I][K] = load4<E>(r, off + 16 * K * E::kBytes);
    }
}

// Registers of one chunk-head's input tile as loaded: the diagonal blocks and
// the six blocks below the diagonal (OPND_A). Two layouts of the diagonal
// blocks, chosen per launch by measurement (the fused kernel's launcher):
//   ROWS = false: load_diag_blocks (16 rows x 64 bytes per load instruction);
//     diag_rows_from_blocks turns them into rows once they have arrived.
//   ROWS = true: load_diag_row_quads (one row per lane, no transpose): fewer
//     dependent steps between the loads and the diagonal solve.
struct Tile {
    f4 dg[4];
    f4 blk[4][4];  // blk[I][K] for K < I
};

template <class E, bool ROWS>
__device__ __forceinline__ void load_tile(Tile &t, const TileView<E> &A, int lane) {
    if constexpr (ROWS)
        load_diag_row_quads<E>(t.dg, A, lane);
    else
        load_diag_blocks<E>(t.dg, A, lane);
    // the diagonal blocks are issued first, so that the diagonal solve waits
    // for four loads and not for the ones it does not need (otherwise the
    // compiler groups the loads by descriptor)
    __builtin_amdgcn_sched_barrier(0);
    load_offdiag_blocks<E>(t.blk, A, lane);
}

// The diagonal rows of a loaded tile in the layout of diag_inverses.
template <bool ROWS>
__device__ __forceinline__ void tile_diag_rows(const Tile &t, float (&arow)[16]) {
    if constexpr (ROWS) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) arow[4 * q + e] = t.dg[q][e];
    } else {
        diag_rows_from_blocks(t.dg, arow);
    }
}

// Writes rows 16I..16I+15 of X (those inside the descriptor) through the LDS
// staging tile so that every store instruction covers four whole 64-column
// rows (16 lanes x 16 bytes per row for fp32): X_IJ (J <= I) come in OPND_O
// registers xo[J]; the zero upper triangle (columns past 16(I + 1)) is
// stored without touching LDS.
template <class E, int I>
__device__ __forceinline__ void store_block_row(const TileView<E> &X, const f4 (&xo)[4],
                                                float *stage, int lane) {
    constexpr int S = stage_row(I);
    const int g = lane >> 4, n = lane & 15;
    wave_sync();  // every earlier read of this LDS region has completed
#pragma unroll
    for (int J = 0; J <= I; ++J)
#pragma unroll
        for (int r = 0; r < 4; ++r) stage[(4 * g + r) * S + 16 * J + n] = xo[J][r];
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

// Merge products on the matrix cores: mm(P, Q, acc) = acc + P Q with P in
// OPND_A and Q in OPND_O; negx(I, S) = -X_II S with X_II read (negated, in
// OPND_A) from the column-major copy xs; xkk(K) = X_KK in OPND_O.
template <int BS, int CS>
struct MfmaEngine {
    const float *xs;
    int lane;
    __device__ __forceinline__ f4 mm(f4 P, f4 Q, f4 acc) const { return mma16(P, Q, acc); }
    __device__ __forceinline__ f4 negx(int I, f4 S) const {
        const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        return mma16(xs_opnd_a_neg<BS, CS>(xs, I, lane), S, z);
    }
    __device__ __forceinline__ f4 xkk(int K) const { return xs_opnd_o<BS, CS>(xs, K, lane); }
};

// Block merge and stores, one block row at a time (the rows of block row I
// are written as soon as X_I0..X_II are known):
//   X_IJ = -X_II * sum_{K=J}^{I-1} A_IK X_KJ,  I > J,
// FP32 throughout. X_KK come from the engine (eng.xkk, eng.negx: a
// column-major copy in LDS in the fused kernel, the workspace in the split
// path); the products run in the same order in both, so their results agree
// bit for bit. `stage` may alias the engine's LDS copy (the fused kernel):
// everything block row I needs from blocks 0..I of it is read before block
// row I is staged, and block row I's staging covers at most the first
// 16 * stage_row(I) floats, which ends inside block I.
template <class E, class Eng>
__device__ __forceinline__ void merge_and_store(const Eng &eng, const f4 (&blk)[4][4],
                                                float *stage, const TileView<E> &X, int lane) {
    const int len = X.len;
    const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    f4 xo[4] = {z, z, z, z};
    // block row 0
    const f4 x00 = eng.xkk(0);
    xo[0] = x00;
    store_block_row<E, 0>(X, xo, stage, lane);
    if (len <= 16) return;
    // block row 1
    const f4 x11 = eng.xkk(1);
    const f4 x10 = eng.negx(1, eng.mm(blk[1][0], x00, z));
    xo[0] = x10;
    xo[1] = x11;
    store_block_row<E, 1>(X, xo, stage, lane);
    if (len <= 32) return;
    // block row 2
    const f4 x22 = eng.xkk(2);
    const f4 s21 = eng.mm(blk[2][1], x11, z);
    const f4 s20 = eng.mm(blk[2][1], x10, eng.mm(blk[2][0], x00, z));
    const f4 x21 = eng.negx(2, s21);
    const f4 x20 = eng.negx(2, s20);
    xo[0] = x20;
    xo[1] = x21;
    xo[2] = x22;
    store_block_row<E, 2>(X, xo, stage, lane);
    if (len <= 48) return;
    // block row 3
    const f4 x33 = eng.xkk(3);
    const f4 s32 = eng.mm(blk[3][2], x22, z);
    const f4 s31 = eng.mm(blk[3][2], x21, eng.mm(blk[3][1], x11, z));
    const f4 s30 = eng.mm(blk[3][2], x20, eng.mm(blk[3][1], x10, eng.mm(blk[3][0], x00, z)));
    xo[0] = eng.negx(3, s30);
    xo[1] = eng.negx(3, s31);
    xo[2] = eng.negx(3, s32);
    xo[3] = x33;
    store_block_row<E, 3>(X, xo, stage, lane);
}

}  // namespace kda
