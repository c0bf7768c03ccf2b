// Kernel-facing problem description and the host-side launchers (internal to
// the library; the public interface is include/kda_tril.h).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace kda {

// One solver call as the kernels see it (passed by value to every kernel).
struct Problem {
    const void *A;
    void *X;
    const int32_t *cu;     // packed: cu_seqlens [num_seqs + 1]; dense: null
    const int32_t *cmap;   // packed: optional (request, chunk) pairs; else null
    float *ws;             // split workspace [slots * H, 4, 16, 16] or null
    int32_t num_seqs;      // packed requests, or dense batch B
    int32_t seq_len;       // dense T
    int32_t total_tokens;  // rows of A and X
    int32_t heads;         // H
    int32_t slots;         // chunk slots in the grid (>= number of chunks)
};

constexpr int kFusedWaves = 4;  // independent wavefronts per workgroup
constexpr int kFusedThreads = 64 * kFusedWaves;

// Workgroups of `threads` threads of kernel `fn` that the current device
// holds at once (occupancy x compute units); 0 when unknown. Cached.
long resident_blocks(const void *fn, int threads);

hipError_t launch_fused_mfma(const Problem &p, int a_bf16, int x_bf16, hipStream_t stream);
hipError_t launch_split(const Problem &p, int a_bf16, int x_bf16, hipStream_t stream);
hipError_t launch_fused_valu(const Problem &p, int a_bf16, int x_bf16, hipStream_t stream);

}  // namespace kda
