// Fused KDA chunk solver kernels for gfx950, in three forms: one wavefront
// per chunk-head at a time (the basis of the others), four adjacent heads of a
// chunk per workgroup with their tiles loaded into LDS (launches of several
// rounds), and two or four wavefronts per chunk-head, one per pair of block
// columns or per column (launches that leave compute units idle).
//
// LightLLM PR #1703 ("perf(kda): parallelize diagonal solves in Prefill",
// PR description): invert the four 16x16 diagonal blocks of every 64x64
// chunk matrix independently, then merge into the 64x64 inverse with FP32
// tiles. In the one-wavefront form everything for one chunk-head happens
// inside one wavefront: the tile goes HBM -> VGPRs, the diagonal inverses go
// through a small LDS copy, the inverse goes VGPRs -> LDS staging -> HBM as
// whole rows. Its grid has one wavefront per chunk-head (a grid that is
// forced smaller walks them with a stride of the grid size), so consecutive
// wavefronts work on neighbouring heads of the same chunk (adjacent 256-byte
// rows in HBM).
//
// Traffic per full chunk-head: the ten blocks on or below the diagonal of A
// are read (the six upper blocks are never needed, so never loaded) and all
// 64 rows x 64 columns of X are written.
#include <stdlib.h>
#include <string.h>

#include "tril_device.h"
#include "tril_group.h"
#include "tril_launch.h"

namespace kda {

// Work item w (wave-uniform) = chunk slot w / H, head w % H.
struct Item {
    Chunk ch;
    int32_t h;
};

template <class EI, bool ROWS>
__device__ __forceinline__ Item fetch(const Problem &p, long w, Tile &t, int lane) {
    Item it;
    const int slot = (int)(w / p.heads);
    it.h = (int)(w - (long)slot * p.heads);
    it.ch = uniform(resolve_chunk<kChunk>(p, slot, lane));
    if (it.ch.len > 0) {
        const TileView<EI> A{static_cast<const typename EI::T *>(p.A) +
                                 ((long)it.ch.start * p.heads + it.h) * kChunk,
                             p.heads * kChunk, it.ch.len, kChunk};
        load_tile<EI, ROWS>(t, A, opaque_lane(lane));
    }
    return it;
}

template <class EI, class EO, bool ROWS, class Eng>
__device__ __forceinline__ void solve(const Problem &p, const Item &it, const Tile &t, float *xs,
                                      float *stage, const Eng &eng, int lane) {
    if (it.ch.len <= 0) return;
    lane = opaque_lane(lane);
    const TileView<EO> X{static_cast<typename EO::T *>(p.X) +
                             ((long)it.ch.start * p.heads + it.h) * kChunk,
                         p.heads * kChunk, it.ch.len, kChunk};
    float arow[16];
    tile_diag_rows<ROWS>(t, arow);
    diag_inverses(xs, arow, lane);
    merge_and_store<EO>(eng, t.blk, stage, X, lane);
}

// Wavefronts per workgroup: four independent ones for the launches that walk
// several items each; one for the launches in which every item has its own
// wavefront (ROWS), so that those items spread over as many compute units as
// possible (64 matrices: 64 CUs instead of 16). (Workgroups of four for
// one-round launches past two chunk-heads per CU measured level: 1,024
// chunk-heads 6.70-6.90 against 6.58-6.74 us, 2,048 10.88-11.14 against
// 11.08-11.43.)
template <bool ROWS>
__host__ __device__ constexpr int waves_per_block() {
    return ROWS ? 1 : kFusedWaves;
}

// Grid-stride walk over the work items. (Loading the next tile before
// solving the current one was measured too: the second register tile costs
// more occupancy than the overlap gains on MI355X, so each item is loaded
// when its wavefront reaches it, and other wavefronts cover the latency.)
template <class EI, class EO, bool ROWS, class Eng>
__device__ __forceinline__ void walk(const Problem &p, float *xs, float *stage, const Eng &eng,
                                     long w, int lane) {
    const long total = (long)p.slots * p.heads;
    const long G = (long)gridDim.x * waves_per_block<ROWS>();
    for (; w < total; w += G) {
        Tile t;
        const Item it = fetch<EI, ROWS>(p, w, t, lane);
        solve<EI, EO, ROWS>(p, it, t, xs, stage, eng, lane);
    }
}

template <class EI, class EO, bool ROWS>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_fused_mfma(Problem p) {
    __shared__ float lds_all[waves_per_block<ROWS>() * kLdsPerWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = ROWS ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float *xs = lds_all + wid * kLdsPerWave;
    float *stage = xs;  // the staging reuses the diagonal-inverse region
    const MfmaEngine<kXsBlock, kXsCol> eng{xs, lane};
    walk<EI, EO, ROWS>(p, xs, stage, eng, (long)blockIdx.x * waves_per_block<ROWS>() + wid, lane);
}

// ------------------------------------------------------------------------
// Latency form for launches that leave compute units idle (at most two
// chunk-heads per compute unit, e.g. one 64-token request over 64 heads): W =
// 2 (or 4) wavefronts per chunk-head, each for two (or one) block columns, in
// workgroups of one chunk-head (two when there are more chunk-heads than
// CUs, so that no CU runs a second workgroup). The merge
// X_IJ = -X_II * sum_{K=J}^{I-1} A_IK X_KJ reads only blocks of column J
// above row I and the diagonal inverses, so the columns need nothing from
// each other: each wavefront inverts the four
// diagonal blocks itself (the same lanes and steps as the one-wavefront
// kernel, at the same cost as one block), runs its columns' products in the
// one-wavefront kernel's order, and writes X_JJ..X_3J into the staging rows
// of their block rows; after one barrier the wavefronts store the block
// rows. The longest chain of products is 36 instead of all 64 in one
// wavefront (two wavefronts: columns 0 and 3, beside columns 1 and 2's 28;
// four: column 0, beside 20, 8 and none), the block rows are stored at once,
// and X is the same bit for bit.

// Columns of wavefront w out of W: one each for W = 4; for W = 2, columns 0
// and 3 (36 products) and columns 1 and 2 (28).
__host__ __device__ constexpr int column_mask(int W, int w) {
    return W == 4 ? 1 << w : (w == 0 ? 0x9 : 0x6);
}
__host__ __device__ constexpr int lowest_column(int mask) {
    return (mask & 1) ? 0 : (mask & 2) ? 1 : (mask & 4) ? 2 : 3;
}

// The diagonal rows and the blocks below the diagonal from column J0 on.
template <class EI, int J0>
__device__ __forceinline__ void load_column_tile(Tile &t, const TileView<EI> &A, int lane) {
    load_diag_row_quads<EI>(t.dg, A, lane);
    __builtin_amdgcn_sched_barrier(0);  // the diagonal solve waits for these only
    const int g = lane >> 4, m = lane & 15;
    const uint32_t off = (uint32_t)(m * A.rstride + 4 * g) * EI::kBytes;
#pragma unroll
    for (int I = J0 + 1; I < 4; ++I) {
        const Rsrc r = A.rows_from(16 * I);
#pragma unroll
        for (int K = J0; K < I; ++K) t.blk[I][K] = load4<EI>(r, off + 16 * K * EI::kBytes);
    }
}

// Floats of block row I's staging (16 rows of stage_row(I)) and where it
// starts in the workgroup's staging region.
__host__ __device__ constexpr int col_stage_floats(int I) { return 16 * stage_row(I); }
__host__ __device__ constexpr int col_stage_base(int I) {
    return I == 0 ? 0 : col_stage_base(I - 1) + col_stage_floats(I - 1);
}
constexpr int kColStageFloats = col_stage_base(4);

// Block column J of X, staged into the rows of its block rows
// (store_block_row's layout).
template <int J, class Eng>
__device__ __forceinline__ void merge_column(const Eng &eng, const Tile &t, float *stage,
                                             int lane) {
    const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    f4 x[4];
    x[J] = eng.xkk(J);
#pragma unroll
    for (int I = J + 1; I < 4; ++I) {
        f4 acc = z;
#pragma unroll
        for (int K = J; K < I; ++K) acc = eng.mm(t.blk[I][K], x[K], acc);
        x[I] = eng.negx(I, acc);
    }
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int I = J; I < 4; ++I) {
        float *st = stage + col_stage_base(I);
#pragma unroll
        for (int r = 0; r < 4; ++r) st[(4 * g + r) * stage_row(I) + 16 * J + n] = x[I][r];
    }
}

template <class EI, int MASK>
__device__ __forceinline__ void merge_columns(const Problem &p, const Chunk &ch, int h,
                                              float *xs, float *stage, int lane) {
    const TileView<EI> A{static_cast<const typename EI::T *>(p.A) +
                             ((long)ch.start * p.heads + h) * kChunk,
                         p.heads * kChunk, ch.len, kChunk};
    Tile t;
    load_column_tile<EI, lowest_column(MASK)>(t, A, opaque_lane(lane));
    float arow[16];
    tile_diag_rows<true>(t, arow);
    diag_inverses(xs, arow, opaque_lane(lane));
    const MfmaEngine<kXsBlock, kXsCol> eng{xs, lane};
    if constexpr ((MASK & 1) != 0) merge_column<0>(eng, t, stage, lane);
    if constexpr ((MASK & 2) != 0) merge_column<1>(eng, t, stage, lane);
    if constexpr ((MASK & 4) != 0) merge_column<2>(eng, t, stage, lane);
    if constexpr ((MASK & 8) != 0) merge_column<3>(eng, t, stage, lane);
}

// Rows 16I..16I+15 of X from block row I's staging: four whole rows per store
// instruction, zeros right of the block row (as in store_block_row).
template <class EO, int I>
__device__ __forceinline__ void store_staged_row(const TileView<EO> &X, const float *stage,
                                                 int lane) {
    constexpr int S = stage_row(I);
    const float *st = stage + col_stage_base(I);
    const int r4 = lane >> 4, c4 = (lane & 15) * 4;
    const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t off = (uint32_t)(r4 * X.rstride + c4) * EO::kBytes;
    const bool in_row = c4 < 16 * (I + 1);
    const int cs = in_row ? c4 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f4 sv = *reinterpret_cast<const f4 *>(&st[(4 * i + r4) * S + cs]);
        store4<EO>(X.rows_from(16 * I + 4 * i), off, in_row ? sv : z);
    }
}

// W wavefronts per chunk-head, P chunk-heads per workgroup (consecutive work
// items); wavefront W * q + j works on the workgroup's q-th chunk-head.
template <class EI, class EO, int W, int P>
__global__ __launch_bounds__(kWave * W * P) void tril_inv_fused_cols(Problem p) {
    static_assert((W == 2 && (P == 1 || P == 2)) || (W == 4 && P == 1),
                  "two wavefronts per chunk-head, one or two chunk-heads per workgroup, or four");
    __shared__ __attribute__((aligned(16))) float xs_all[W * P * kLdsPerWave];
    __shared__ __attribute__((aligned(16))) float stage_all[P * kColStageFloats];
    const int lane = threadIdx.x & (kWave - 1);
    const int wall = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int q = wall / W, wid = wall - q * W;
    float *xs = xs_all + wall * kLdsPerWave;
    float *stage = stage_all + q * kColStageFloats;
    const long w = (long)blockIdx.x * P + q;
    Chunk ch{0, 0};
    int h = 0;
    if (w < (long)p.slots * p.heads) {
        const int slot = (int)(w / p.heads);
        h = (int)(w - (long)slot * p.heads);
        ch = uniform(resolve_chunk<kChunk>(p, slot, lane));
    }
    if (ch.len > 0) {
        if constexpr (W == 4) {
            switch (wid) {
                case 0: merge_columns<EI, column_mask(4, 0)>(p, ch, h, xs, stage, lane); break;
                case 1: merge_columns<EI, column_mask(4, 1)>(p, ch, h, xs, stage, lane); break;
                case 2: merge_columns<EI, column_mask(4, 2)>(p, ch, h, xs, stage, lane); break;
                default: merge_columns<EI, column_mask(4, 3)>(p, ch, h, xs, stage, lane); break;
            }
        } else if (wid == 0) {
            merge_columns<EI, column_mask(2, 0)>(p, ch, h, xs, stage, lane);
        } else {
            merge_columns<EI, column_mask(2, 1)>(p, ch, h, xs, stage, lane);
        }
    }
    __syncthreads();  // every wavefront of the workgroup, with work or not
    if (ch.len <= 0) return;
    // block row I is stored by wavefront I mod W of its chunk-head (rows past
    // the chunk: none)
    const TileView<EO> X{static_cast<typename EO::T *>(p.X) +
                             ((long)ch.start * p.heads + h) * kChunk,
                         p.heads * kChunk, ch.len, kChunk};
    if (wid == 0) store_staged_row<EO, 0>(X, stage, lane);
    if (wid == 1 % W && ch.len > 16) store_staged_row<EO, 1>(X, stage, lane);
    if (wid == 2 % W && ch.len > 32) store_staged_row<EO, 2>(X, stage, lane);
    if (wid == 3 % W && ch.len > 48) store_staged_row<EO, 3>(X, stage, lane);
}

// ------------------------------------------------------------------------
// Multi-head form of the same kernel, for launches of several rounds. A
// workgroup of four wavefronts owns a group (chunk, four adjacent heads): the
// lines of the four heads' tiles that the solve needs go from HBM straight
// into LDS, each load instruction covering one token's row of the four heads
// (1 KiB of adjacent bytes) or two tokens' first lines of the four heads;
// then every wavefront reads its own head's blocks from LDS in the layouts of
// the solve and runs the same diagonal solve, merge and stores as the kernel
// above. The grid has one workgroup per group, so the hardware dispatcher
// hands every free workgroup slot the next group (a grid of what the GPU
// holds at once, each workgroup walking a fixed share, was 2-8% slower). Measured with loads and stores alone on 16 x
// 512 tokens, 64 heads, this load pattern takes 40.0-40.4 us against 42.2 us
// for the per-wavefront one.
//
// The tile is FusedPlan's (tril_group.h).

// Head position hh's tile from the group's LDS copy, in the registers of the
// solve: diagonal blocks one row per lane, blocks below the diagonal in
// OPND_A.
template <class EI>
__device__ __forceinline__ void read_tile(Tile &t, const char *lds, int hh, int lane) {
    read_diag_rows<EI, FusedPlan<EI>>(t.dg, lds, hh, lane);
    read_offdiag_blocks<EI, FusedPlan<EI>>(t.blk, lds, hh, lane);
}

// (Issuing the next group's loads as soon as every wavefront has read the
// current tile, with the inverses and staging in LDS of their own so that
// the loads land while the tile is solved, was measured too: 70,400 bytes of
// LDS per workgroup leave two workgroups per CU, and on the same box and
// buffers 16 x 512 tokens took 42.3 against 42.0 us, 48 ragged requests
// 117.9 against 117.2 us, 131,072 tokens 607 against 582 us.)
template <class EI, class EO>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_fused_heads4(Problem p) {
    typedef FusedPlan<EI> Plan;
    static_assert(Plan::kBytes >= kGroupHeads * kLdsPerWave * 4,
                  "the solve's LDS regions must fit in the tile's");
    __shared__ __attribute__((aligned(16))) char lds[Plan::kBytes];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // once a group's tiles are in registers, the tile region holds each
    // wavefront's diagonal inverses and output staging
    float *xs = reinterpret_cast<float *>(lds) + wid * kLdsPerWave;
    const MfmaEngine<kXsBlock, kXsCol> eng{xs, lane};
    // fewer than 2^26 groups: the launch checks slots x H x 64 < 2^32
    const int hg = (p.heads + kGroupHeads - 1) / kGroupHeads;
    const int groups = p.slots * hg;
    for (int gi = blockIdx.x; gi < groups; gi += gridDim.x) {
        const Group gr = group_of(p, gi, hg, lane);
        if (gr.ch.len <= 0) continue;
        load_group_of<EI, Plan>(p, gr, lds, wid, opaque_lane(lane));
        group_arrived();
        Tile t;
        read_tile<EI>(t, lds, wid, opaque_lane(lane));
        __syncthreads();  // every wavefront has its tile: the region is free
        if (wid < gr.nh) solve<EI, EO, true>(p, Item{gr.ch, gr.h0 + wid}, t, xs, xs, eng, lane);
        __syncthreads();  // staging reads done before the next group's loads land
    }
}

// ------------------------------------------------------------------------
// Same kernel with the merge products on the vector ALUs (FP32 FMA) instead
// of the matrix cores; kept as the second precision mode and as the
// comparison point for the matrix-core merge.

constexpr int kScr = 20;  // padded row stride of the product scratch
constexpr int kLdsPerWaveValu = kLdsPerWave + 2 * 16 * kScr;

struct ValuEngine {
    const float *xs;
    float *ps;
    float *qs;
    int lane;

    // acc + P Q for P in OPND_A, Q in OPND_O; result in OPND_O. Both operands
    // go through LDS: lane (g, n) needs rows 4g..4g+3 of P and column n of Q.
    __device__ __forceinline__ f4 mm(f4 P, f4 Q, f4 acc) const {
        const int g = lane >> 4, m = lane & 15;
        *reinterpret_cast<f4 *>(&ps[m * kScr + 4 * g]) = P;  // row m
        *reinterpret_cast<f4 *>(&qs[m * kScr + 4 * g]) = Q;  // column m
        wave_sync();
        // one reduction quarter per iteration; not unrolled, so that the LDS
        // reads are not all hoisted into registers at once
#pragma unroll 1
        for (int kq = 0; kq < 4; ++kq) {
            const f4 qc = *reinterpret_cast<const f4 *>(&qs[m * kScr + 4 * kq]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f4 pr = *reinterpret_cast<const f4 *>(&ps[(4 * g + r) * kScr + 4 * kq]);
                float a = acc[r];
#pragma unroll
                for (int e = 0; e < 4; ++e) a = __builtin_fmaf(pr[e], qc[e], a);
                acc[r] = a;
            }
        }
        wave_sync();
        return acc;
    }

    // -X_II S with X_II read from its column-major LDS copy; S in OPND_O.
    __device__ __forceinline__ f4 negx(int I, f4 S) const {
        const int g = lane >> 4, m = lane & 15;
        *reinterpret_cast<f4 *>(&qs[m * kScr + 4 * g]) = S;
        wave_sync();
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 1
        for (int kq = 0; kq < 4; ++kq) {
            const f4 sc = *reinterpret_cast<const f4 *>(&qs[m * kScr + 4 * kq]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = 4 * kq + e;
                const f4 col =
                    *reinterpret_cast<const f4 *>(&xs[I * kXsBlock + k * kXsCol + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(-col[r], sc[e], acc[r]);
            }
        }
        wave_sync();
        return acc;
    }

    __device__ __forceinline__ f4 xkk(int K) const {
        return xs_opnd_o<kXsBlock, kXsCol>(xs, K, lane);
    }
};

template <class EI, class EO, bool ROWS>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_fused_valu(Problem p) {
    __shared__ float lds_all[waves_per_block<ROWS>() * kLdsPerWaveValu];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = ROWS ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float *xs = lds_all + wid * kLdsPerWaveValu;
    float *stage = xs;
    float *ps = xs + kLdsPerWave;
    const ValuEngine eng{xs, ps, ps + 16 * kScr, lane};
    walk<EI, EO, ROWS>(p, xs, stage, eng, (long)blockIdx.x * waves_per_block<ROWS>() + wid, lane);
}

// ------------------------------------------------------------------ launch

// The layout of the diagonal-block loads (ROWS, see Tile) is chosen per
// launch. When every item has its own wavefront in one round, latency
// decides and the row-per-lane loads win (64 matrices: 5.7 against 6.3 us on
// MI355X). Past one round, with one wavefront per item, the 16-row loads
// with lane swaps in 4-wavefront workgroups are faster (same bits, us): 16 x
// 512 tokens 44.4 against 51.7, one request of 131,072 tokens 632 against
// 756, the 48 ragged requests 116.9 against 135.3, 8 heads, 4 requests of
// 32,768 tokens 75.6 against 86.5 (level at 2 heads). Mostly empty chunks
// (many requests, or dense rows, of a few tokens) take the row-per-lane
// variant in workgroups of one wavefront there too: 64 heads, 200 requests of
// 1-3 tokens 12.6-13.1 against 14.5-15.3 us, 100 of 1-20 tokens 8.2-8.7
// against 9.0-9.8, 400 of 1-10 tokens 27.7-27.9 against 30.2-31.4 (same bits). Every launch has one
// wavefront per item, so the hardware dispatcher hands each free slot the
// next one; a grid of what the GPU holds at once, each wavefront walking a
// fixed share, was slower (same bits): 8 heads, 4 requests of 32,768 tokens
// 78.6 against 74.9 us; 64 heads, 2,000 requests of 1-20 tokens 333.9
// against 301.9; the VALU merge on 131,072 tokens 758 against 632, on the 48
// ragged requests 158.3 against 148.1. Wavefronts walk only on a grid that
// KDA_TRIL_BLOCKS_PER_CU forces.
template <class KT, class KR>
static hipError_t launch_walk(KT ktput, KR krows, const Problem &p, hipStream_t stream) {
    const long waves = (long)p.slots * p.heads;
    const long blocks = walk_blocks(reinterpret_cast<const void *>(ktput), waves,
                                    min_chunks(p, kChunk) * p.heads);
    const bool one_round = blocks * kFusedWaves >= waves;
    const bool walk = blocks_forced();
    if (one_round)  // one item per workgroup of one wavefront
        hipLaunchKernelGGL(krows, dim3((unsigned)waves), dim3(kWave), 0, stream, p);
    else if (!chunks_mostly_full(p, kChunk))  // the same wavefronts
        hipLaunchKernelGGL(krows, dim3((unsigned)(walk ? blocks * kFusedWaves : waves)),
                           dim3(kWave), 0, stream, p);
    else
        hipLaunchKernelGGL(ktput,
                           dim3((unsigned)(walk ? blocks : (waves + kFusedWaves - 1) / kFusedWaves)),
                           dim3(kFusedThreads), 0, stream, p);
    return hipGetLastError();
}

// KDA_TRIL_FUSED_LAYOUT (read on every call): "wave" runs the per-wavefront
// kernel for every launch, "heads4" the 4-head kernel for every launch (one
// round or not; the tests use it to reach its edge cases on small problems),
// "cols2", "cols2p" and "cols4" the column kernel for every launch, with two
// wavefronts per chunk-head and one or two chunk-heads per workgroup, or with
// four wavefronts per chunk-head (kept as the comparison point: at every
// size measured it was at most level with two); anything else, or unset,
// chooses by the number of rounds, of chunk-heads per CU and of heads.
enum class Layout { kAuto, kWave, kHeads4, kCols2, kCols2P, kCols4 };

// The 4-head kernel takes launches whose chunk-heads (the lower bound: for a
// packed scan ceil(T / 64) chunks) exceed what the per-wavefront kernel
// holds at once at its occupancy, from this many heads. Below that bound
// the two are level on cold buffers (64 heads, same bits: 16 requests of 256
// tokens 23.83 us either way, 48 of 64 tokens 18.40 against 18.35) and the
// per-wavefront kernel is faster when A is partly in the 256 MB cache, as
// when it was just written (19.7 against 23.8, 15.1 against 17.4); above it
// the 4-head kernel wins (1.2-1.5 times as many chunk-heads: 32.6-32.7
// against 34.5-34.7 us; C3, 1.6 times: 41.7 against 44.1). (The bound once came from the walking grid, one workgroup per CU
// below the occupancy and over the chunk slots, which sent launches of one
// round to the 4-head kernel.) With few
// heads the rows of a chunk's heads are close together anyway, so the
// per-wavefront loads cover nearly adjacent bytes, and groups of four run
// partly empty when H is not a multiple of four. Measured on single long
// requests (same box, six rotating buffer sets; µs, per-wavefront / 4-head):
// 8,192 chunk-heads at H = 2 44.5 / 45.1, 4 45.4 / 46.5, 5 45.8 / 52.3,
// 8 45.6 / 46.5, 9 45.7 / 44.1, 10 46.0 / 44.5, 12 46.7 / 45.7, 13 45.4 / 46.3,
// 16 52.5 / 46.9, 32 47.6 / 44.5, 64 44.6 / 42.6; 4,096 at H = 1 22.8 / 32.9;
// 6,144 at H = 6 34.2 / 38.7.
constexpr int kHeads4MinHeads = 9;
// ... and only while the chunks are mostly full: when the tokens would fill
// fewer than half the chunk slots, as for many requests of a few tokens,
// the tile loads and barriers of the
// 4-head kernel cost more than they save (200 requests of 1-3 tokens over 64
// heads: 18.6 us against 14.6-15.2; 100 requests of 1-20 tokens: 12.1
// against 9.0-9.4).

// Launches of at most one chunk-head per compute unit take the column kernel
// with two wavefronts per chunk-head, and launches of at most two per CU the
// same kernel with two chunk-heads per workgroup (four wavefronts): a second
// workgroup on a CU costs about as much as the shorter chains save. Requests
// of 64 tokens over 64 heads, one box, µs per call back to back (one-wavefront
// kernel / column kernel with two wavefronts per chunk-head, one chunk-head
// per workgroup / two per workgroup / four wavefronts per chunk-head):
//   64 chunk-heads   4.92-4.98 / 4.03-4.05 / 4.31-4.33 / 4.04-4.07
//   256              4.96-5.08 / 4.18-4.25 / 4.66-4.69 / 4.31-4.40
//   320              5.27-5.39 / 5.42-5.50 / 4.76-4.80 / 5.27-5.29
//   512              5.64-5.75 / 5.73-5.84 / 5.31-5.35 / 5.59-5.65
//   640              5.88-6.02 / 6.06-6.16 / 6.18-6.26 / 6.15-6.24
//   1,024            6.47-6.83 / 7.24-8.31 / 6.79-7.02 / 7.27-7.57
// and dense 4 x 512 tokens, 16 heads, bf16 A (512 chunk-heads): 5.56-5.70 /
// 5.69-5.79 / 5.30-5.37 / 5.67-5.72.
// The rules count the chunk-heads that have rows (a lower bound for packed
// inputs without a chunk map: ceil(T / 64) chunks per head) and also bound
// the chunk slots (an upper bound), so that many short requests, whose
// chunks the lower bound undercounts, keep the per-wavefront kernel.
constexpr long kColsPerCu = 1;
constexpr long kCols2PPerCu = 2;
constexpr long kColsSlotsPerCu = 2;  // chunk slots x heads per CU (x 2 with two per workgroup)

static Layout fused_layout() {
    const char *e = getenv("KDA_TRIL_FUSED_LAYOUT");
    if (e && strcmp(e, "wave") == 0) return Layout::kWave;
    if (e && strcmp(e, "heads4") == 0) return Layout::kHeads4;
    if (e && strcmp(e, "cols2") == 0) return Layout::kCols2;
    if (e && strcmp(e, "cols2p") == 0) return Layout::kCols2P;
    if (e && strcmp(e, "cols4") == 0) return Layout::kCols4;
    return Layout::kAuto;
}

template <class K>
static hipError_t launch_cols(K kernel, long chunk_heads, int per_block, int threads,
                              hipStream_t stream, const Problem &p) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)((chunk_heads + per_block - 1) / per_block)),
                       dim3(threads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_fused_mfma(const Problem &p, int a_dt, int x_dt, hipStream_t stream) {
    return dispatch_dtypes<F32, BF16, F16>(a_dt, x_dt, [&]<class EI, class EO>() {
        // chunk slots x heads (for packed inputs without a chunk map the slots
        // are an upper bound on the chunks), and chunk-heads that have rows
        // (a lower bound: exact for dense inputs and chunk maps)
        const long waves = (long)p.slots * p.heads;
        const long items = min_chunks(p, kChunk) * p.heads;
        const long held = resident_blocks(
                              reinterpret_cast<const void *>(tril_inv_fused_mfma<EI, EO, false>),
                              kFusedThreads) *
                          kFusedWaves;
        const Layout lay = fused_layout();
        if (lay == Layout::kHeads4 ||
            (lay == Layout::kAuto && p.heads >= kHeads4MinHeads && chunks_mostly_full(p, kChunk) &&
             items > held)) {
            const long groups = (long)p.slots * ((p.heads + kGroupHeads - 1) / kGroupHeads);
            const long g = group_blocks(
                reinterpret_cast<const void *>(tril_inv_fused_heads4<EI, EO>), groups);
            hipLaunchKernelGGL((tril_inv_fused_heads4<EI, EO>), dim3((unsigned)g),
                               dim3(kFusedThreads), 0, stream, p);
            return hipGetLastError();
        }
        // (one workgroup per one or two chunk-heads: forced launches keep the
        // grid below 2^24 workgroups, larger ones take the walking kernel)
        const bool small = waves < (1L << 24);
        const long cus = lay == Layout::kAuto ? device_cus() : 0;
        if ((lay == Layout::kCols2 && small) ||
            (lay == Layout::kAuto && items <= kColsPerCu * cus && waves <= kColsSlotsPerCu * cus))
            return launch_cols(tril_inv_fused_cols<EI, EO, 2, 1>, waves, 1, 2 * kWave, stream, p);
        if ((lay == Layout::kCols2P && small) ||
            (lay == Layout::kAuto && items <= kCols2PPerCu * cus &&
             waves <= 2 * kColsSlotsPerCu * cus))
            return launch_cols(tril_inv_fused_cols<EI, EO, 2, 2>, waves, 2, 4 * kWave, stream, p);
        if (lay == Layout::kCols4 && small)
            return launch_cols(tril_inv_fused_cols<EI, EO, 4, 1>, waves, 1, 4 * kWave, stream, p);
        return launch_walk(tril_inv_fused_mfma<EI, EO, false>, tril_inv_fused_mfma<EI, EO, true>,
                           p, stream);
    });
}

hipError_t launch_fused_valu(const Problem &p, int a_dt, int x_dt, hipStream_t stream) {
    return dispatch_dtypes<F32, BF16, F16>(a_dt, x_dt, [&]<class EI, class EO>() {
        return launch_walk(tril_inv_fused_valu<EI, EO, false>, tril_inv_fused_valu<EI, EO, true>,
                           p, stream);
    });
}

}  // namespace kda
