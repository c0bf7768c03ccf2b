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
#include <mutex>
#include <utility>
#include <vector>

#include "kda_tril.h"
#include "tril_device.h"
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
    merge_and_store<EO, kWsTile, kWsCol>(eng, blk, tiles, stage,
                                         TileView<EO>{X, rstride, ch.len, kChunk}, lane);
}

template <class EI, class EO>
static hipError_t launch_split_t(const Problem &p, hipStream_t stream) {
    const long waves = (long)p.slots * p.heads;
    const long blocks = (waves + kFusedWaves - 1) / kFusedWaves;
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
