// The shared chunk solver's 16- and 32-token branches for gfx950.
//
// LightLLM PR #1703 ("perf(kda): parallelize diagonal solves in Prefill", PR
// description) describes the 64-token kernel as one branch of a solver that
// also serves smaller chunks. With chunks of C tokens every chunk-head matrix
// is C x C, A and X are [T, H, C] (packed) or [B, T, H, C] (dense), and:
//
//   * C = 16: the matrix is a single diagonal block, so the solve is the
//     diagonal step alone. A wavefront takes four heads of one chunk and
//     gives every lane one column (lane = 16 * head + column): a row of the
//     four heads is 64 adjacent elements, so each load or store instruction
//     covers one whole such row, and the columns never leave their lanes.
//   * C = 32: two diagonal 16 x 16 inverses and one merge level,
//     X_10 = -X_11 (A_10 X_00), on the matrix cores. A wavefront takes two
//     heads of one chunk: its four 16-lane rows run the four diagonal
//     substitutions of both heads at once, then both merges follow, and the
//     rows are written through LDS staging as whole 2-head rows. Launches of
//     several rounds with 32 heads or more give a workgroup one chunk and
//     eight heads instead, their rows loaded straight into LDS (the group
//     kernel below), with the same arithmetic.
//
// The per-wavefront kernels walk their work items (chunk, group of heads)
// with a grid stride like the 64-token kernel (the group kernel's grid has
// one workgroup per item). All compute in FP32 with the same
// operation order as the 64-token kernel's corresponding blocks, so a 16- or
// 32-token chunk gives bit for bit the leading block of the 64-token result
// on the same (zero-padded) rows.
#include <utility>

#include <stdlib.h>
#include <string.h>

#include "tril_device.h"
#include "tril_launch.h"

namespace kda {

typedef __attribute__((address_space(3))) void *LdsPtr32;

// load1 with the nontemporal policy, for the 16-token kernel whose every
// line is read by exactly one load instruction (a line read again by a later
// instruction would be fetched twice, so the other kernels keep the default
// policy).
template <class E>
__device__ __forceinline__ float load1_once(Rsrc r, uint32_t off);
template <>
__device__ __forceinline__ float load1_once<F32>(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNontemporal));
}
template <>
__device__ __forceinline__ float load1_once<BF16>(Rsrc r, uint32_t off) {
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kNontemporal));
}
template <>
__device__ __forceinline__ float load1_once<F16>(Rsrc r, uint32_t off) {
    return (float)__builtin_bit_cast(_Float16,
                                     __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kNontemporal));
}

// --------------------------------------------------------------- 16 tokens

constexpr int kHeads16 = 4;  // heads per wavefront (4 x 16 columns = 64 lanes)

// -sum_{j<I} A[I][j] x[j] (j increasing) for the lane's column: A[I][j] is
// element I of column j, held by lane j of this 16-lane row.
template <int I, int... J>
__device__ __forceinline__ float col_dot(const float (&a)[16], const float (&x)[16],
                                         std::integer_sequence<int, J...>) {
    float acc = 0.0f;
    ((acc = __builtin_fmaf(row_bcast<J>(a[I]), x[J], acc)), ...);
    return acc;
}

template <int I>
__device__ __forceinline__ float select_below(float v, float keep, int c) {
    return (I > c) ? v : keep;
}

// Forward substitution for column c of (I + A)^-1 (rows in increasing order;
// only rows below the diagonal are computed, so A's own diagonal and upper
// part are never read).
template <int... I>
__device__ __forceinline__ void col_subst(const float (&a)[16], float (&x)[16], int c,
                                          std::integer_sequence<int, I...>) {
    // the dot product is taken on every lane and then selected (same bits):
    // a conditional evaluation compiled to one exec-masked branch per row
    ((x[I] = select_below<I>(-col_dot<I>(a, x, std::make_integer_sequence<int, I>{}), x[I], c)),
     ...);
}

template <class EI, class EO>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_c16(Problem p) {
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane0 = threadIdx.x & (kWave - 1);
    const int groups = (p.heads + kHeads16 - 1) / kHeads16;
    const long total = (long)p.slots * groups;
    const long G = (long)gridDim.x * kFusedWaves;
    for (long w = (long)blockIdx.x * kFusedWaves + wid; w < total; w += G) {
        const int slot = (int)(w / groups);
        const int hg = (int)(w - (long)slot * groups);
        const Chunk ch = uniform(resolve_chunk<16>(p, slot, lane0));
        if (ch.len <= 0) continue;
        const int lane = opaque_lane(lane0);
        const int c = lane & 15;
        const int h0 = kHeads16 * hg;
        const int hv = min(kHeads16, p.heads - h0);  // heads of this group that exist
        const int rstride = p.heads * 16;
        const long base = ((long)ch.start * p.heads + h0) * 16;
        const TileView<EI> A{static_cast<const typename EI::T *>(p.A) + base, rstride, ch.len,
                             16 * hv};
        const TileView<EO> X{static_cast<typename EO::T *>(p.X) + base, rstride, ch.len,
                             16 * hv};
        const uint32_t mask = (lane >> 4) < hv ? 0u : kOffMasked;

        // a[i] = A[i][c] of this lane's head; rows past the chunk read as 0
        float a[16];
        const Rsrc ra = A.rows_from(0);
        const uint32_t offa = (uint32_t)lane * EI::kBytes | mask;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            a[i] = load1_once<EI>(ra, offa + (uint32_t)(i * rstride * EI::kBytes));

        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.0f : 0.0f;
        col_subst(a, x, c, std::make_integer_sequence<int, 16>{});

        // row i of the four heads is one 64-element store; rows past the
        // chunk are dropped by the descriptor
        const Rsrc rx = X.rows_from(0);
        const uint32_t offx = (uint32_t)lane * EO::kBytes | mask;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            store1<EO>(rx, offx + (uint32_t)(i * rstride * EO::kBytes), x[i]);
    }
}

// --------------------------------------------------------------- 32 tokens

constexpr int kHeads32 = 2;  // heads per wavefront (2 heads x 2 diagonal blocks)
constexpr int kStage32 = 2 * 32 + 4;  // LDS row stride of the 2-head staging
static_assert(16 * kStage32 <= kLdsPerWave, "the staging of a block row must fit");

// Rows 16I..16I+15 of both heads through LDS: xo[m][J] is block (I, J) of
// head m in OPND_O layout (J <= I); columns past the diagonal block are 0.
// Each store instruction then covers four whole 2-head rows.
template <class E, int I>
__device__ __forceinline__ void store_pair_rows(const TileView<E> &X, const f4 (&xo)[2][2],
                                                float *stage, uint32_t mask_hi, int lane) {
    const int g = lane >> 4, n = lane & 15;
    wave_sync();  // earlier reads of this LDS region have completed
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int J = 0; J <= I; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) stage[(4 * g + r) * kStage32 + 32 * m + 16 * J + n] = xo[m][J][r];
    wave_sync();
    const int r4 = lane >> 4, c4 = (lane & 15) * 4;
    const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t off = (uint32_t)(r4 * X.rstride + c4) * E::kBytes | (c4 >= 32 ? mask_hi : 0u);
    // unconditional staging read (lanes right of the block row read column 0
    // and store zeros), so each store stays one full-wave instruction
    const bool in_row = (c4 & 31) < 16 * (I + 1);
    const int cs = in_row ? c4 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + r4;
        const f4 sv = *reinterpret_cast<const f4 *>(&stage[row * kStage32 + cs]);
        store4<E>(X.rows_from(16 * I + 4 * i), off, in_row ? sv : z);
    }
    wave_sync();
}

template <class EI, class EO, bool ROWS>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_c32(Problem p) {
    __shared__ float lds_all[kFusedWaves * kLdsPerWave];
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane0 = threadIdx.x & (kWave - 1);
    float *xs = lds_all + wid * kLdsPerWave;
    const int groups = (p.heads + kHeads32 - 1) / kHeads32;
    const long total = (long)p.slots * groups;
    const long G = (long)gridDim.x * kFusedWaves;
    for (long w = (long)blockIdx.x * kFusedWaves + wid; w < total; w += G) {
        const int slot = (int)(w / groups);
        const int hg = (int)(w - (long)slot * groups);
        const Chunk ch = uniform(resolve_chunk<32>(p, slot, lane0));
        if (ch.len <= 0) continue;
        const int lane = opaque_lane(lane0);
        const int h0 = kHeads32 * hg;
        const int hv = min(kHeads32, p.heads - h0);
        const int rstride = p.heads * 32;
        const long base = ((long)ch.start * p.heads + h0) * 32;
        const TileView<EI> A{static_cast<const typename EI::T *>(p.A) + base, rstride, ch.len,
                             32 * hv};
        const TileView<EO> X{static_cast<typename EO::T *>(p.X) + base, rstride, ch.len,
                             32 * hv};
        const uint32_t mask_hi = hv > 1 ? 0u : kOffMasked;  // second head missing

        // Diagonal rows: lane (b, i), b = 2m + d, holds row 16d + i, columns
        // 16d..16d+15 of head m (block d of head m goes to LDS block b). As in
        // the 64-token kernel, launches in which wavefronts walk several items
        // load each block as 16 rows x 64 bytes per instruction and transpose
        // with lane swaps (ROWS = false); one-round launches load one row per
        // lane (ROWS = true).
        f4 dgb[4];
        if constexpr (ROWS) {
            const int b = lane >> 4, i = lane & 15, m = b >> 1, d = b & 1;
            const uint32_t off =
                (uint32_t)((16 * d + i) * rstride + 32 * m + 16 * d) * EI::kBytes |
                (m > 0 ? mask_hi : 0u);
            const Rsrc r = A.rows_from(0);
#pragma unroll
            for (int q = 0; q < 4; ++q) dgb[q] = load4<EI>(r, off + 4 * q * EI::kBytes);
        } else {
            const int g = lane >> 4, mr = lane & 15;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int m = b >> 1, d = b & 1;
                const uint32_t off =
                    (uint32_t)(mr * rstride + 32 * m + 16 * d + 4 * g) * EI::kBytes |
                    (m > 0 ? mask_hi : 0u);
                dgb[b] = load4<EI>(A.rows_from(16 * d), off);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // diagonal loads first
        // A_10 of both heads in OPND_A layout (row 16 + m', columns 4g..4g+3)
        f4 a10[2];
        {
            const int g = lane >> 4, mr = lane & 15;
            const Rsrc r = A.rows_from(16);
            const uint32_t off = (uint32_t)(mr * rstride + 4 * g) * EI::kBytes;
            a10[0] = load4<EI>(r, off);
            a10[1] = load4<EI>(r, (off + 32 * EI::kBytes) | mask_hi);
        }

        float arow[16];
        if constexpr (ROWS) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) arow[4 * q + e] = dgb[q][e];
        } else {
            diag_rows_from_blocks(dgb, arow);
        }
        diag_inverses(xs, arow, lane);
        // Everything the merge needs from the diagonal copies is read into
        // registers before the first staging, which reuses the same LDS.
        const MfmaEngine<kXsBlock, kXsCol> eng{xs, lane};
        const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        f4 x00[2], row1[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m) x00[m] = xs_opnd_o<kXsBlock, kXsCol>(xs, 2 * m, lane);
        const bool two_rows = ch.len > 16;
        if (two_rows) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                row1[m][1] = xs_opnd_o<kXsBlock, kXsCol>(xs, 2 * m + 1, lane);
                row1[m][0] = eng.negx(2 * m + 1, eng.mm(a10[m], x00[m], z));
            }
        }
        const f4 row0[2][2] = {{x00[0], z}, {x00[1], z}};
        store_pair_rows<EO, 0>(X, row0, xs, mask_hi, lane);
        if (two_rows) store_pair_rows<EO, 1>(X, row1, xs, mask_hi, lane);
    }
}

// ------------------------------------------------------------------------
// 32 tokens, group form (launches in which wavefronts walk several items): a
// workgroup of four wavefronts owns one chunk and eight adjacent heads, whose
// rows are 8 x 32 elements, 1 KiB (FP32) or 512 bytes (16-bit) of adjacent
// bytes; they go from HBM straight into LDS (16-byte buffer loads with the
// LDS bit, every byte read by one instruction, so nontemporal), and then each
// wavefront takes its two heads from LDS in the layouts of the kernel above
// (diagonal rows one per lane, A_10 in OPND_A) and runs the same arithmetic.
//
// LDS: slots of 1040 bytes (1 KiB + 16, so 16 consecutive rows fall on
// different banks), each holding what one load instruction brings: one FP32
// row of the eight heads, or two 16-bit rows 2j and 2j + 1, the second with
// its heads rotated by two positions (128 bytes) for the same reason.

constexpr int kHeadsGroup32 = 8;
// Groups (chunks with rows x groups of eight heads, a lower bound) per
// compute unit above which the group kernel takes over from the
// per-wavefront kernel. Measured on cold buffers (rotations past 1 GB), 64
// heads, same bits (us, per-wavefront / group): 16 requests of 128 tokens (2
// groups per CU) 6.75 / 7.40, of 192 (3) 11.46 / 9.48, of 256 (4) 15.17 /
// 14.34, 32 of 128 (4) 15.13 / 14.30; 32 heads, 16 of 256 (2) 6.83 / 7.38, of
// 512 (4) 15.15 / 14.93. (The rule once asked for more items than the walking
// grid held, which left 3-6 groups per CU on the per-wavefront kernel.)
constexpr long kGroup32PerCu = 2;
// Heads from which multi-round launches take the group kernel: with fewer the
// per-wavefront kernel reads nearly adjacent rows anyway and groups of eight
// run partly empty. Single long requests of 16,384 chunk-heads, same box (µs,
// per-wavefront / group): H = 1 27.0 / 77.7, 2 26.0 / 37.6, 4 26.2 / 26.3,
// 8 25.6 / 25.4, 12 26.0 / 28.6, 16 26.0 / 25.8, 32 26.0 / 25.8, 64 26.0 / 25.1:
// below 32 heads the two are within noise of each other or the group loses.
// It also needs mostly full chunks (the tokens would fill at least half the
// chunk slots): for many requests of a few tokens its tile loads and
// barriers cost more than they save (64 heads, 200 requests of 1-3 tokens
// 9.4-9.6 us against 8.1-8.4; 400 requests of 1-10 tokens 19.8-20.1 against
// 16.1-16.7).
constexpr int kGroup32MinHeads = 32;
constexpr int kSlot32 = 1040;

template <class EI>
struct Tile32 {
    static constexpr int kRowsPerSlot = 4 / EI::kBytes;      // 1 or 2
    static constexpr int kHeadBytes = 32 * EI::kBytes;       // a head's row
    static constexpr int kSlots = 32 / kRowsPerSlot;
    static constexpr int kBytes = kSlots * kSlot32 > kFusedWaves * kLdsPerWave * 4
                                      ? kSlots * kSlot32
                                      : kFusedWaves * kLdsPerWave * 4;
    // LDS byte of row R, head position hh (0..7), byte column bc of its row
    __host__ __device__ static __forceinline__ int addr(int R, int hh, int bc) {
        const int k = R % kRowsPerSlot;
        const int pos = (hh - 2 * k) & 7;
        return (R / kRowsPerSlot) * kSlot32 + k * 8 * kHeadBytes + pos * kHeadBytes + bc;
    }
};

// Columns c..c+3 of row R of head position hh, widened to FP32.
template <class EI>
__device__ __forceinline__ f4 lds_quad32(const char *lds, int R, int hh, int c) {
    typedef Tile32<EI> L;
    if constexpr (EI::kBytes == 4) {
        return *reinterpret_cast<const f4 *>(lds + L::addr(R, hh, 4 * c));
    } else if constexpr (__is_same(EI, BF16)) {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 v = *reinterpret_cast<const u2 *>(lds + L::addr(R, hh, 2 * c));
        f4 o;
        o[0] = bf16_to_f32(v[0] & 0xFFFFu);
        o[1] = bf16_to_f32(v[0] >> 16);
        o[2] = bf16_to_f32(v[1] & 0xFFFFu);
        o[3] = bf16_to_f32(v[1] >> 16);
        return o;
    } else {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 v = *reinterpret_cast<const h4 *>(lds + L::addr(R, hh, 2 * c));
        f4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (float)v[e];  // exact widening
        return o;
    }
}

template <class EI, class EO>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_c32_group(Problem p) {
    typedef Tile32<EI> L;
    __shared__ __attribute__((aligned(16))) char lds[L::kBytes];
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane0 = threadIdx.x & (kWave - 1);
    // once the group's rows are read, the tile holds each wavefront's
    // diagonal inverses and staging
    float *xs = reinterpret_cast<float *>(lds) + wid * kLdsPerWave;
    const int groups = (p.heads + kHeadsGroup32 - 1) / kHeadsGroup32;
    const long total = (long)p.slots * groups;
    for (long gi = blockIdx.x; gi < total; gi += gridDim.x) {
        const int slot = (int)(gi / groups);
        const int hg = (int)(gi - (long)slot * groups);
        // the same chunk for the whole workgroup: every wavefront takes the
        // same branches and meets the same barriers
        const Chunk ch = uniform(resolve_chunk<32>(p, slot, lane0));
        if (ch.len <= 0) continue;
        const int lane = opaque_lane(lane0);
        const int h0 = kHeadsGroup32 * hg;
        const int nh = min(kHeadsGroup32, p.heads - h0);
        const int rstride = p.heads * 32;
        const long gbase = ((long)ch.start * p.heads + h0) * 32;
        {
            const TileView<EI> A{static_cast<const typename EI::T *>(p.A) + gbase, rstride,
                                 ch.len, 32 * nh};
            const Rsrc r = A.rows_from(0);
            // lane l: row k = l / (64 / rows per slot) of the slot, position
            // and 16-byte piece of that row; the position holds head
            // (pos + 2k) mod 8
            constexpr int lanes_row = 64 / L::kRowsPerSlot, pieces = L::kHeadBytes / 16;
            const int k = lane / lanes_row, w = lane % lanes_row;
            const int pos = w / pieces, pc = w % pieces;
            const int ph = (pos + 2 * k) & 7;
            const uint32_t hmask = ph < nh ? 0u : kOffMasked;
#pragma unroll
            for (int q = 0; q < L::kSlots / kFusedWaves; ++q) {
                const int s = wid + kFusedWaves * q;
                const int row = s * L::kRowsPerSlot + k;
                const uint32_t off =
                    ((uint32_t)(row * rstride + ph * 32) * EI::kBytes + 16 * pc) | hmask;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr32)(lds + s * kSlot32), 16,
                                                         off, 0, 0, kNontemporal);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // every wavefront's share of the group has arrived
        // this wavefront's heads: positions 2 wid (+1)
        f4 dgb[4], a10[2];
        {
            const int b = lane >> 4, i = lane & 15, m = b >> 1, d = b & 1;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                dgb[q] = lds_quad32<EI>(lds, 16 * d + i, 2 * wid + m, 16 * d + 4 * q);
            const int g = lane >> 4, mr = lane & 15;
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) a10[mm] = lds_quad32<EI>(lds, 16 + mr, 2 * wid + mm, 4 * g);
        }
        __syncthreads();  // every wavefront has its rows: the tile is free
        const int hv = nh - 2 * wid;  // heads of this wavefront that exist
        if (hv > 0) {
            const uint32_t mask_hi = hv > 1 ? 0u : kOffMasked;
            const long base = gbase + 2 * wid * 32;
            const TileView<EO> X{static_cast<typename EO::T *>(p.X) + base, rstride, ch.len,
                                 32 * min(hv, 2)};
            float arow[16];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) arow[4 * q + e] = dgb[q][e];
            diag_inverses(xs, arow, lane);
            const MfmaEngine<kXsBlock, kXsCol> eng{xs, lane};
            const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            f4 x00[2], row1[2][2];
#pragma unroll
            for (int m = 0; m < 2; ++m) x00[m] = xs_opnd_o<kXsBlock, kXsCol>(xs, 2 * m, lane);
            const bool two_rows = ch.len > 16;
            if (two_rows) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    row1[m][1] = xs_opnd_o<kXsBlock, kXsCol>(xs, 2 * m + 1, lane);
                    row1[m][0] = eng.negx(2 * m + 1, eng.mm(a10[m], x00[m], z));
                }
            }
            const f4 row0[2][2] = {{x00[0], z}, {x00[1], z}};
            store_pair_rows<EO, 0>(X, row0, xs, mask_hi, lane);
            if (two_rows) store_pair_rows<EO, 1>(X, row1, xs, mask_hi, lane);
        }
        __syncthreads();  // staging reads done before the next group's loads land
    }
}

// ------------------------------------------------------------------ launch

// KDA_TRIL_SMALL_LAYOUT (read on every call): "wave" runs the per-wavefront
// 32-token kernel for every launch, "group" the 8-head group kernel for every
// launch (the tests use it to reach its edge cases on small problems);
// anything else, or unset, the group kernel from more than two groups per
// compute unit (32 heads or more, mostly full chunks).
static int small_layout() {
    const char *e = getenv("KDA_TRIL_SMALL_LAYOUT");
    if (e && strcmp(e, "wave") == 0) return 1;
    if (e && strcmp(e, "group") == 0) return 2;
    return 0;
}

template <class K>
static hipError_t launch_groups(K kernel, const Problem &p, int chunk, int heads_per_wave,
                                hipStream_t stream) {
    const long groups = (p.heads + heads_per_wave - 1) / heads_per_wave;
    const long blocks = walk_blocks(reinterpret_cast<const void *>(kernel), (long)p.slots * groups,
                                    min_chunks(p, chunk) * groups);
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kFusedThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_small(const Problem &p, int chunk, int a_dt, int x_dt, hipStream_t stream) {
    return dispatch_dtypes<F32, BF16, F16>(a_dt, x_dt, [&]<class EI, class EO>() {
        if (chunk == 16) return launch_groups(tril_inv_c16<EI, EO>, p, 16, kHeads16, stream);
        if (chunk == 32) {
            // the group kernel from more than two groups per CU when there
            // are enough heads and the chunks are mostly full; else the
            // ROWS = false variant sizes the grid, one-round launches run the
            // row-per-lane variant and longer ones the ROWS = false variant (the row-per-lane one when the chunks are
            // mostly empty: 200 requests of 1-3 tokens over 64 heads 7.7-7.9
            // against 8.0-8.3 us; single long requests at 4 and 16 heads
            // 25.7-26.1 against 26.3-26.5 the other way)
            const long groups = (p.heads + kHeads32 - 1) / kHeads32;
            const long items = (long)p.slots * groups;
            const long blocks =
                walk_blocks(reinterpret_cast<const void *>(tril_inv_c32<EI, EO, false>), items,
                            min_chunks(p, 32) * groups);
            const bool multi = blocks * kFusedWaves < items;
            const bool full = chunks_mostly_full(p, 32);
            const int lay = small_layout();
            const long heads8 = (p.heads + kHeadsGroup32 - 1) / kHeadsGroup32;
            if (lay == 2 || (lay == 0 && full && p.heads >= kGroup32MinHeads &&
                             min_chunks(p, 32) * heads8 > kGroup32PerCu * device_cus())) {
                const long g8 = (long)p.slots * heads8;
                const long gb = group_blocks(
                    reinterpret_cast<const void *>(tril_inv_c32_group<EI, EO>), g8);
                hipLaunchKernelGGL((tril_inv_c32_group<EI, EO>), dim3((unsigned)gb),
                                   dim3(kFusedThreads), 0, stream, p);
                return hipGetLastError();
            }
            if (multi && (lay == 1 || full))
                return launch_groups(tril_inv_c32<EI, EO, false>, p, 32, kHeads32, stream);
            return launch_groups(tril_inv_c32<EI, EO, true>, p, 32, kHeads32, stream);
        }
        return hipErrorInvalidValue;
    });
}

}  // namespace kda
