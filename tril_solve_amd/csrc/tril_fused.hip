// Fused KDA chunk solver kernels for gfx950: one wavefront per chunk-head at
// a time.
//
// LightLLM PR #1703 ("perf(kda): parallelize diagonal solves in Prefill",
// PR description): invert the four 16x16 diagonal blocks of every 64x64
// chunk matrix independently, then merge into the 64x64 inverse with FP32
// tiles. Everything for one chunk-head happens inside one wavefront: the
// tile goes HBM -> VGPRs, the diagonal inverses go through a small LDS copy,
// the inverse goes VGPRs -> LDS staging -> HBM as whole rows.
//
// The grid is sized to what the GPU holds at once and every wavefront walks
// chunk-heads with a stride of the grid size, so consecutive wavefronts work
// on neighbouring heads of the same chunk (adjacent 256-byte rows in HBM).
//
// Traffic per full chunk-head: the ten blocks on or below the diagonal of A
// are read (the six upper blocks are never needed, so never loaded) and all
// 64 rows x 64 columns of X are written.
#include <stdlib.h>
#include <string.h>

#include "tril_device.h"
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
    merge_and_store<EO, kXsBlock, kXsCol>(eng, t.blk, xs, stage, X, lane);
}

// Wavefronts per workgroup: four independent ones for the launches that walk
// several items each; one for the launches in which every item has its own
// wavefront (ROWS), so that those items spread over as many compute units as
// possible (64 matrices: 64 CUs instead of 16).
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
// Multi-head form of the same kernel, for launches in which wavefronts walk
// several items. A workgroup of four wavefronts owns (chunk, four adjacent
// heads): the lines of the four heads' tiles that the solve needs go from HBM
// straight into LDS (buffer loads with the LDS bit, no VGPRs), each load
// instruction covering one token's row of the four heads (1 KiB of adjacent
// bytes) or two tokens' first lines of the four heads; then every wavefront
// reads its own head's blocks from LDS in the layouts of the solve and runs
// the same diagonal solve, merge and stores as the kernel above. Four heads'
// rows are adjacent in HBM, so each load instruction covers long runs instead
// of 64-byte pieces 16 KiB apart: measured with loads and stores alone on 16 x
// 512 tokens, 64 heads, the pattern takes 40.0-40.4 us against 42.2 us.
//
// LDS tile layout (bytes), in slots of kSlotBytes (1 KiB plus 16 bytes, so
// the 16 rows a block read touches fall on different banks):
//   pair slots: two tokens r and r + 8 of one block row, each as the first
//     128 bytes of heads 0..3 (512 bytes); the second token's heads are
//     rotated by one position so that the two rows sit 128 bytes apart in
//     bank order. FP32 input: the 32 rows of block rows 0 and 1 (they need
//     columns 0..31, one line per head); 16-bit input: all 64 rows (a head's
//     row is one 128-byte line).
//   row slots (FP32 only): rows 32..63, all 256 bytes of heads 0..3.
constexpr int kGroupHeads = 4;
constexpr int kSlotBytes = 1040;

template <class EI>
struct GroupTile {
    static constexpr int kPairSlots = EI::kBytes == 4 ? 16 : 32;
    static constexpr int kRowSlots = EI::kBytes == 4 ? 32 : 0;
    static constexpr int kBytes = (kPairSlots + kRowSlots) * kSlotBytes;
    static_assert(kBytes >= kGroupHeads * kLdsPerWave * 4,
                  "the solve's LDS regions must fit in the tile's");

    // byte address of row R, head position hh, byte column bc of that head
    __device__ static __forceinline__ int addr(int R, int hh, int bc) {
        if (EI::kBytes == 4 && R >= 32)
            return (kPairSlots + R - 32) * kSlotBytes + hh * 256 + bc;
        const int p = (R >> 4) * 8 + (R & 7), half = (R >> 3) & 1;
        const int pos = half ? (hh + 3) & 3 : hh;
        return p * kSlotBytes + half * 512 + pos * 128 + bc;
    }
};

typedef __attribute__((address_space(3))) void *LdsPtr;

// This wavefront's share of a group's loads: pair slots wid, wid + 4, ... and
// (FP32) the row slots of rows 32 + wid, 36 + wid, ... Lanes of heads past
// the last head (nh < 4) use an out-of-range offset: their LDS bytes get 0.
// Every line is read by exactly one instruction, so the loads carry the
// nontemporal bit (same-box A/B: 16 x 512 tokens 42.9 -> 42.2 us, 48 ragged
// requests 121.9 -> 117.9 us, 131,072 tokens 607 -> 583 us).
template <class EI>
__device__ __forceinline__ void load_group(Rsrc r, int rstride, int nh, char *lds, int wid,
                                           int lane) {
    typedef GroupTile<EI> L;
    const int half = lane >> 5, pos = (lane >> 3) & 3, piece = lane & 7;
    const int ph = half ? (pos + 1) & 3 : pos;  // head whose bytes land at this position
    const uint32_t pmask = ph < nh ? 0u : kOffMasked;
#pragma unroll
    for (int q = 0; q < L::kPairSlots / 4; ++q) {
        const int p = wid + 4 * q;
        const int row = 16 * (p >> 3) + (p & 7) + 8 * half;
        const uint32_t off = ((uint32_t)(row * rstride + ph * 64) * EI::kBytes + 16 * piece) | pmask;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(lds + p * kSlotBytes), 16, off, 0, 0, kNontemporal);
    }
    const uint32_t rmask = (lane >> 4) < nh ? 0u : kOffMasked;
#pragma unroll
    for (int q = 0; q < L::kRowSlots / 4; ++q) {
        const int row = 32 + wid + 4 * q;
        const uint32_t off = ((uint32_t)(row * rstride) * EI::kBytes + 16 * lane) | rmask;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (LdsPtr)(lds + (L::kPairSlots + row - 32) * kSlotBytes), 16, off, 0, 0, kNontemporal);
    }
}

// Columns c..c+3 of row R of head position hh, widened to FP32.
template <class EI>
__device__ __forceinline__ f4 lds_quad(const char *lds, int R, int hh, int c);
template <>
__device__ __forceinline__ f4 lds_quad<F32>(const char *lds, int R, int hh, int c) {
    return *reinterpret_cast<const f4 *>(lds + GroupTile<F32>::addr(R, hh, 4 * c));
}
template <>
__device__ __forceinline__ f4 lds_quad<BF16>(const char *lds, int R, int hh, int c) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 v = *reinterpret_cast<const u2 *>(lds + GroupTile<BF16>::addr(R, hh, 2 * c));
    f4 o;
    o[0] = bf16_to_f32(v[0] & 0xFFFFu);
    o[1] = bf16_to_f32(v[0] >> 16);
    o[2] = bf16_to_f32(v[1] & 0xFFFFu);
    o[3] = bf16_to_f32(v[1] >> 16);
    return o;
}
// (A vector of binary16 values, as the global loads widen them: converting
// single 16-bit lanes of an integer vector through bit casts lost three of
// every four elements in this compiler's output.)
template <>
__device__ __forceinline__ f4 lds_quad<F16>(const char *lds, int R, int hh, int c) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 v = *reinterpret_cast<const h4 *>(lds + GroupTile<F16>::addr(R, hh, 2 * c));
    f4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (float)v[e];  // exact widening
    return o;
}

// Head position hh's tile from the group's LDS copy, in the registers of the
// solve: diagonal blocks one row per lane (lane (b, i): row 16b + i, columns
// 16b + 4q..+3 in dg[q]), blocks below the diagonal in OPND_A.
template <class EI>
__device__ __forceinline__ void read_tile(Tile &t, const char *lds, int hh, int lane) {
    const int hi = lane >> 4, lo = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) t.dg[q] = lds_quad<EI>(lds, 16 * hi + lo, hh, 16 * hi + 4 * q);
#pragma unroll
    for (int I = 1; I < 4; ++I)
#pragma unroll
        for (int K = 0; K < I; ++K) t.blk[I][K] = lds_quad<EI>(lds, 16 * I + lo, hh, 16 * K + 4 * hi);
}

// A group of four heads of one chunk slot (len 0: nothing to do).
struct Group {
    Chunk ch;
    int h0, nh;
};

template <class EI>
__device__ __forceinline__ Group group_of(const Problem &p, int gi, int hg, int lane) {
    Group gr;
    const int slot = gi / hg;
    gr.h0 = (gi - slot * hg) * kGroupHeads;
    gr.nh = min(kGroupHeads, p.heads - gr.h0);
    gr.ch = uniform(resolve_chunk<kChunk>(p, slot, lane));
    return gr;
}

template <class EI>
__device__ __forceinline__ void load_group_of(const Problem &p, const Group &gr, char *lds,
                                              int wid, int lane) {
    const long row0 = (long)gr.ch.start * p.heads + gr.h0;
    const TileView<EI> A{static_cast<const typename EI::T *>(p.A) + row0 * kChunk,
                         p.heads * kChunk, gr.ch.len, gr.nh * kChunk};
    load_group<EI>(A.rows_from(0), A.rstride, gr.nh, lds, wid, lane);
}

template <class EI, class EO>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_fused_heads4(Problem p) {
    __shared__ __attribute__((aligned(16))) char lds[GroupTile<EI>::kBytes];
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
        // the same chunk for the whole workgroup: every wavefront takes the
        // same branches and meets the same barriers
        const Group gr = group_of<EI>(p, gi, hg, lane);
        if (gr.ch.len <= 0) continue;
        load_group_of<EI>(p, gr, lds, wid, opaque_lane(lane));
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // every wavefront's share of the group has arrived
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
// launch. When every item has its own wavefront (one round), latency decides
// and the row-per-lane loads win (64 matrices: 5.7 against 6.3 us on
// MI355X). When wavefronts walk several items, the 16-row loads with lane
// swaps were faster on 16 x 512 tokens (0.9%) and on the 48 ragged requests
// (1.3-3.5%); on long single requests the two measured within 2% of each
// other, in either order depending on the machine. The ROWS = false variant
// sizes the grid (its registers allow fewer wavefronts).
template <class KT, class KR>
static hipError_t launch_walk(KT ktput, KR krows, const Problem &p, hipStream_t stream) {
    const long waves = (long)p.slots * p.heads;
    const long blocks = walk_blocks(reinterpret_cast<const void *>(ktput), waves,
                                    min_chunks(p, kChunk) * p.heads);
    const bool one_round = blocks * kFusedWaves >= waves;
    if (one_round)  // one item per workgroup of one wavefront
        hipLaunchKernelGGL(krows, dim3((unsigned)waves), dim3(kWave), 0, stream, p);
    else
        hipLaunchKernelGGL(ktput, dim3((unsigned)blocks), dim3(kFusedThreads), 0, stream, p);
    return hipGetLastError();
}

// KDA_TRIL_FUSED_LAYOUT (read on every call): "wave" runs the per-wavefront
// kernel for every launch, "heads4" the 4-head kernel for every launch (one
// round or not; the tests use it to reach its edge cases on small problems);
// anything else, or unset, chooses by the number of rounds.
enum class Layout { kAuto, kWave, kHeads4 };
static Layout fused_layout() {
    const char *e = getenv("KDA_TRIL_FUSED_LAYOUT");
    if (e && strcmp(e, "wave") == 0) return Layout::kWave;
    if (e && strcmp(e, "heads4") == 0) return Layout::kHeads4;
    return Layout::kAuto;
}

hipError_t launch_fused_mfma(const Problem &p, int a_dt, int x_dt, hipStream_t stream) {
    return dispatch_dtypes<F32, BF16, F16>(a_dt, x_dt, [&]<class EI, class EO>() {
        const long waves = (long)p.slots * p.heads;
        const long blocks = walk_blocks(
            reinterpret_cast<const void *>(tril_inv_fused_mfma<EI, EO, false>), waves,
            min_chunks(p, kChunk) * p.heads);
        const Layout lay = fused_layout();
        if (lay == Layout::kHeads4 || (lay == Layout::kAuto && blocks * kFusedWaves < waves)) {
            const long groups = (long)p.slots * ((p.heads + kGroupHeads - 1) / kGroupHeads);
            const long g = group_blocks(
                reinterpret_cast<const void *>(tril_inv_fused_heads4<EI, EO>), groups);
            hipLaunchKernelGGL((tril_inv_fused_heads4<EI, EO>), dim3((unsigned)g),
                               dim3(kFusedThreads), 0, stream, p);
            return hipGetLastError();
        }
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
