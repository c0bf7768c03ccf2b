// Split variant of the KDA chunk solver for gfx950: two kernels in stream
// order with an FP32 workspace between them.
//
// LightLLM PR #1703 ("perf(kda): parallelize diagonal solves in Prefill",
// commit summary and PR description) keeps FP32 inverse tiles through the
// merge and bounds the extra scratch by the FP32 input size, choosing the
// split path by chunk occupancy. Here the diagonal kernel writes the four
// FP32 16x16 inverse tiles of every chunk-head (4 KiB) to the workspace
// [slots * H, 4, 16, 16], each tile column-major; the merge kernel reads them
// with the off-diagonal blocks of A and writes X. Per full chunk-head this
// moves 8 KiB more than the fused kernel (tiles written once, read once).
// Both kernels come in two forms with the same arithmetic: one wavefront per
// chunk-head, and four adjacent heads of a chunk per workgroup with their
// tiles loaded into LDS (launches of several rounds with two heads or more).
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <utility>
#include <vector>

#include "kda_tril.h"
#include "tril_device.h"
#include "tril_group.h"
#include "tril_launch.h"

// Workspace of the allocation-free entry point (kda_tril_inv_packed_noalloc):
// the split plan's tiles in device memory the library holds, one copy per GPU
// for as long as the process runs. Host code never uses this name as an
// address (on the host it is only a stand-in); it uses the device address
// that noalloc_scratch looks up per device.
static __device__ __align__(256) float scratch[KDA_TRIL_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace kda {

constexpr int kWsTile = 256;   // floats per 16x16 tile
constexpr int kWsCol = 16;     // column stride inside a tile (column-major)

template <class EI>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_split_diag(Problem p) {
    __shared__ float lds_all[kFusedWaves * kXsFloats];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float *lds = lds_all + wid * kXsFloats;
    const long w = (long)blockIdx.x * kFusedWaves + wid;
    const int slot = (int)(w / p.heads);
    const int h = (int)(w - (long)slot * p.heads);
    if (slot >= p.slots) return;
    const Chunk ch = uniform(resolve_chunk<kChunk>(p, slot, lane));
    if (ch.len <= 0) return;

    const int rstride = p.heads * kChunk;
    const long base = ((long)ch.start * p.heads + h) * kChunk;
    const typename EI::T *A = static_cast<const typename EI::T *>(p.A) + base;
    float arow[16];
    load_diag_rows<EI>(arow, TileView<EI>{A, rstride, ch.len, kChunk}, lane);
    diag_inverses(lds, arow, lane);

    // lane (b, c) copies column c of tile b: 64 contiguous bytes per lane,
    // 4 KiB contiguous per wavefront.
    const int b = lane >> 4, c = lane & 15;
    float *tile = p.ws + (((long)slot * p.heads + h) * 4 + b) * kWsTile + c * kWsCol;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f4 *>(tile + 4 * q) =
            *reinterpret_cast<const f4 *>(&lds[b * kXsBlock + c * kXsCol + 4 * q]);
}

template <class EI, class EO>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_split_merge(Problem p) {
    __shared__ float stage_all[kFusedWaves * kLdsPerWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float *stage = stage_all + wid * kLdsPerWave;
    const long w = (long)blockIdx.x * kFusedWaves + wid;
    const int slot = (int)(w / p.heads);
    const int h = (int)(w - (long)slot * p.heads);
    if (slot >= p.slots) return;
    const Chunk ch = uniform(resolve_chunk<kChunk>(p, slot, lane));
    if (ch.len <= 0) return;

    const int rstride = p.heads * kChunk;
    const long base = ((long)ch.start * p.heads + h) * kChunk;
    const typename EI::T *A = static_cast<const typename EI::T *>(p.A) + base;
    typename EO::T *X = static_cast<typename EO::T *>(p.X) + base;
    const float *tiles = p.ws + ((long)slot * p.heads + h) * 4 * kWsTile;

    f4 blk[4][4];
    load_offdiag_blocks<EI>(blk, TileView<EI>{A, rstride, ch.len, kChunk}, lane);
    const MfmaEngine<kWsTile, kWsCol> eng{tiles, lane};
    merge_and_store<EO>(eng, blk, stage, TileView<EO>{X, rstride, ch.len, kChunk}, lane);
}

// Merge products on the matrix cores with the diagonal operands of one
// chunk-head loaded from the workspace up front (X_KK in OPND_O, -X_II in
// OPND_A), so that their loads are in flight together with the group's tile
// loads instead of one after another inside the merge. Same values, same
// products as MfmaEngine on the workspace.
struct WsEngine {
    f4 o[4], an[4];  // an[0] unused
    __device__ __forceinline__ void load(const float *tiles, int lane) {
#pragma unroll
        for (int K = 0; K < 4; ++K) o[K] = xs_opnd_o<kWsTile, kWsCol>(tiles, K, lane);
        an[0] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int I = 1; I < 4; ++I) an[I] = xs_opnd_a_neg<kWsTile, kWsCol>(tiles, I, lane);
    }
    __device__ __forceinline__ f4 mm(f4 P, f4 Q, f4 acc) const { return mma16(P, Q, acc); }
    __device__ __forceinline__ f4 negx(int I, f4 S) const {
        const f4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        return mma16(an[I], S, z);
    }
    __device__ __forceinline__ f4 xkk(int K) const { return o[K]; }
};

// ------------------------------------------------------------------------
// The same two kernels in 4-head form, for launches in which wavefronts walk
// several items: a workgroup of four wavefronts owns a group (chunk, four
// adjacent heads) whose tiles of A go from HBM straight into LDS with
// instructions covering long runs of adjacent bytes; each wavefront then
// reads its head's blocks from LDS and computes what the kernels above
// compute for it, with the same arithmetic (same results, bit for bit).

// The tiles are DiagPlan's and MergePlan's (tril_group.h).

// LDS of a 4-head split kernel: the group's tile, reused, once every
// wavefront has read it, for each wavefront's region of kLdsPerWave floats
// (diagonal inverses, or output staging).
template <class Plan>
constexpr int split_lds_bytes() {
    return Plan::kBytes > kGroupHeads * kLdsPerWave * 4 ? Plan::kBytes
                                                        : kGroupHeads * kLdsPerWave * 4;
}

template <class EI>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_split_diag_heads4(Problem p) {
    typedef DiagPlan<EI> Plan;
    __shared__ __attribute__((aligned(16))) char lds[split_lds_bytes<Plan>()];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float *xs = reinterpret_cast<float *>(lds) + wid * kLdsPerWave;
    // fewer than 2^26 groups: the launch checks slots x H x 64 < 2^32
    const int hg = (p.heads + kGroupHeads - 1) / kGroupHeads;
    const int groups = p.slots * hg;
    for (int gi = blockIdx.x; gi < groups; gi += gridDim.x) {
        const Group gr = group_of(p, gi, hg, lane);
        if (gr.ch.len <= 0) continue;
        load_group_of<EI, Plan>(p, gr, lds, wid, opaque_lane(lane));
        group_arrived();
        f4 dg[4];
        read_diag_rows<EI, Plan>(dg, lds, wid, opaque_lane(lane));
        __syncthreads();  // every wavefront has its rows: the region is free
        if (wid < gr.nh) {
            float arow[16];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) arow[4 * q + e] = dg[q][e];
            diag_inverses(xs, arow, lane);
            // store q writes tile q: 1 KiB of adjacent bytes, lane (c, r)
            // columns c's rows 4r..4r+3
            const long item = (long)(gi / hg) * p.heads + gr.h0 + wid;
            float *tiles = p.ws + item * 4 * kWsTile + 4 * lane;
            const int c = lane >> 2, r = lane & 3;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<f4 *>(tiles + q * kWsTile) =
                    *reinterpret_cast<const f4 *>(&xs[q * kXsBlock + c * kXsCol + 4 * r]);
        }
        __syncthreads();  // the copies are read before the next group's loads land
    }
}

template <class EI, class EO>
__global__ __launch_bounds__(kFusedThreads) void tril_inv_split_merge_heads4(Problem p) {
    typedef MergePlan<EI> Plan;
    __shared__ __attribute__((aligned(16))) char lds[split_lds_bytes<Plan>()];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    float *stage = reinterpret_cast<float *>(lds) + wid * kLdsPerWave;
    const int hg = (p.heads + kGroupHeads - 1) / kGroupHeads;
    const int groups = p.slots * hg;
    const int rstride = p.heads * kChunk;
    for (int gi = blockIdx.x; gi < groups; gi += gridDim.x) {
        const Group gr = group_of(p, gi, hg, lane);
        if (gr.ch.len <= 0) continue;
        load_group_of<EI, Plan>(p, gr, lds, wid, opaque_lane(lane));
        const bool mine = wid < gr.nh;
        const int h = gr.h0 + wid;
        WsEngine eng;
        if (mine) eng.load(p.ws + ((long)(gi / hg) * p.heads + h) * 4 * kWsTile, lane);
        group_arrived();
        f4 blk[4][4];
        read_offdiag_blocks<EI, Plan>(blk, lds, wid, opaque_lane(lane));
        __syncthreads();  // every wavefront has its blocks: the region is free
        if (mine) {
            typename EO::T *X =
                static_cast<typename EO::T *>(p.X) + ((long)gr.ch.start * p.heads + h) * kChunk;
            merge_and_store<EO>(eng, blk, stage, TileView<EO>{X, rstride, gr.ch.len, kChunk},
                                lane);
        }
        __syncthreads();  // staging reads done before the next group's loads land
    }
}

// KDA_TRIL_SPLIT_LAYOUT (read on every call): "wave" runs the per-wavefront
// kernels for every launch, "heads4" the 4-head ones for every launch;
// anything else, or unset, the 4-head ones from more than two chunk-heads
// with rows per compute unit when there are two heads or more.
constexpr long kSplitHeads4PerCu = 2;

static int split_layout() {
    const char *e = getenv("KDA_TRIL_SPLIT_LAYOUT");
    if (e && strcmp(e, "wave") == 0) return 1;
    if (e && strcmp(e, "heads4") == 0) return 2;
    return 0;
}

template <class EI, class EO>
static hipError_t launch_split_t(const Problem &p, hipStream_t stream) {
    const long waves = (long)p.slots * p.heads;
    const long blocks = (waves + kFusedWaves - 1) / kFusedWaves;
    const int lay = split_layout();
    // (A single head leaves three of a group's four wavefronts idle: on a
    // 524,288-token request the per-wavefront kernels took 63-65 µs against
    // 75-76; from two heads on the 4-head ones win, 60 against 63 at H = 2.)
    // The 4-head kernels take over from more than two chunk-heads per CU,
    // well before the per-wavefront launch stops fitting on the GPU at once
    // (cold buffers, 64 heads, same bits, us, per-wavefront / 4-head: 512
    // chunk-heads 10.12 / 10.47, 1,024 12.57 / 11.98, 2,048 19.36 / 17.44,
    // 4,096 34.40 / 31.66; 16 heads, 512: 10.31 / 10.53).
    const bool heads4 =
        lay == 2 || (lay == 0 && p.heads >= 2 &&
                     min_chunks(p, kChunk) * p.heads > kSplitHeads4PerCu * device_cus());
    if (heads4) {
        const long groups = (long)p.slots * ((p.heads + kGroupHeads - 1) / kGroupHeads);
        const long gd = group_blocks(
            reinterpret_cast<const void *>(tril_inv_split_diag_heads4<EI>), groups);
        hipLaunchKernelGGL((tril_inv_split_diag_heads4<EI>), dim3((unsigned)gd),
                           dim3(kFusedThreads), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const long gm = group_blocks(
            reinterpret_cast<const void *>(tril_inv_split_merge_heads4<EI, EO>), groups);
        hipLaunchKernelGGL((tril_inv_split_merge_heads4<EI, EO>), dim3((unsigned)gm),
                           dim3(kFusedThreads), 0, stream, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((tril_inv_split_diag<EI>), dim3((unsigned)blocks), dim3(kFusedThreads), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((tril_inv_split_merge<EI, EO>), dim3((unsigned)blocks),
                       dim3(kFusedThreads), 0, stream, p);
    return hipGetLastError();
}

namespace {
std::mutex g_scratch_mu;
std::vector<std::pair<int, float *>> g_scratch;  // (device, address of `scratch` there)
}  // namespace

hipError_t noalloc_scratch(float **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    for (const auto &d : g_scratch)
        if (d.first == dev) {
            *ptr = d.second;
            return hipSuccess;
        }
    void *addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    g_scratch.emplace_back(dev, static_cast<float *>(addr));
    *ptr = static_cast<float *>(addr);
    return hipSuccess;
}

hipError_t launch_split(const Problem &p, int a_dt, int x_dt, hipStream_t stream) {
    return dispatch_dtypes<F32, BF16, F16>(a_dt, x_dt, [&]<class EI, class EO>() {
        return launch_split_t<EI, EO>(p, stream);
    });
}

}  // namespace kda
