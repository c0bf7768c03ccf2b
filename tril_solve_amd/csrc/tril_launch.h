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

// The fused "build A, then invert" path: A is formed from keys, cumulative
// log-decays and write strengths instead of being read (p.A unused; p.X is X,
// or A itself when only the matrix is wanted).
struct KktProblem {
    Problem p;
    const void *k;     // [rows, H, K], element type k_dt
    const float *g;    // [rows, H, K], FP32
    const void *beta;  // [rows, H], element type k_dt
    int32_t K;         // channels, a multiple of 16
};

// One step of the fused KDA decode core (head dim 128), layouts as in the
// C ABI's kda_decode_step.
struct DecodeProblem {
    const void *qkv;       // [B, 3, H, 128], element type in_dt
    const void *z;         // [B, H, 128], element type in_dt
    const float *g;        // [B, H, 128]
    const float *beta;     // [B, H]
    const float *norm_w;   // [128]
    const float *conv_w;   // [3, W, H, 128]
    const int32_t *slot;   // [B]
    float *state;          // [num_slots, H, 128, 128]
    float *conv_state;     // [num_slots, 3, H, W - 1, 128]
    void *out;             // [B, H, 128], element type out_dt
    int32_t B, H, W, num_slots;
    float eps_l2, eps_norm;
};

constexpr int kFusedWaves = 4;  // independent wavefronts per workgroup
constexpr int kFusedThreads = 64 * kFusedWaves;

// Workgroups of `threads` threads of kernel `fn` that the current device
// holds at once (occupancy x compute units; KDA_TRIL_BLOCKS_PER_CU, when set,
// replaces the occupancy, read on every call); 0 when unknown. The device's
// occupancy is cached per kernel and device.
long resident_blocks(const void *fn, int threads);

// Compute units of the current device (0 when unknown).
long device_cus();

// Grid of a grid-stride kernel with kFusedWaves independent wavefronts per
// workgroup and at most `waves` wavefront work items (at least `min_waves` of
// them real; the rest are chunk slots past the last chunk, which end after
// the lookup): one wavefront per item, capped at what the device holds at
// once, the wavefronts then walking the items in rounds. When the device
// holds b workgroups per compute unit, b - 1 is used instead if that leaves
// fewer idle wavefront slots in the last round and still 16 or more
// wavefronts per CU: wavefronts with one item fewer than the rest leave the
// memory system with fewer requests in flight while the others finish. The
// 16- and 32-token and split per-wavefront kernels launch this grid; the
// 64-token and build-A launchers use it to tell one-round launches from
// longer ones and launch it only when KDA_TRIL_BLOCKS_PER_CU is set (else one
// wavefront per item).
long walk_blocks(const void *fn, long waves, long min_waves);

// Whether KDA_TRIL_BLOCKS_PER_CU forces the grid size (read on every call).
bool blocks_forced();

// Grid of a grid-stride kernel whose workgroups (kFusedThreads threads) walk
// `groups` work items together: one workgroup per group, so that the
// hardware dispatcher hands each free workgroup slot the next group and no
// compute unit is left with a fixed share that it finishes late (same bits,
// 2-8% faster than a grid of what the device holds at once, one workgroup per
// CU fewer for long problems: 64 heads, 16 x 512 tokens 42.1 -> 41.4 us, 48
// ragged requests 117.6 -> 107.6, one request of 131,072 tokens 585 -> 571;
// the split plan's pair of kernels 920 -> 864 us on the last). Walks only past
// 2^22 groups, or on the grid KDA_TRIL_BLOCKS_PER_CU asks for.
long group_blocks(const void *fn, long groups);

// Element-type codes of A and X: the kda_dtype values (0 f32, 1 bf16, 2 f16).
hipError_t launch_fused_mfma(const Problem &p, int a_dt, int x_dt, hipStream_t stream);
hipError_t launch_split(const Problem &p, int a_dt, int x_dt, hipStream_t stream);
// Device address, on the current device, of the library-held split workspace
// of KDA_TRIL_NOALLOC_SCRATCH_BYTES (looked up once per device, then cached).
hipError_t noalloc_scratch(float **ptr);
hipError_t launch_fused_valu(const Problem &p, int a_dt, int x_dt, hipStream_t stream);
// Chunks of 16 or 32 tokens (A and X rows of `chunk` elements).
hipError_t launch_small(const Problem &p, int chunk, int a_dt, int x_dt, hipStream_t stream);
// A from keys, decays and write strengths; inverted (solve) or stored.
hipError_t launch_kkt(const KktProblem &q, bool solve, int k_dt, int x_dt, hipStream_t stream);
// One decode step of the fused KDA decode core.
hipError_t launch_decode(const DecodeProblem &p, int in_dt, int out_dt, hipStream_t stream);

// Lower bound on the chunks of a call with chunks of C tokens: exact for the
// dense layout and for a caller chunk map (p.slots); for packed inputs without
// a map, every chunk holds at most C tokens.
inline long min_chunks(const Problem &p, int C) {
    if (p.cu != nullptr && p.cmap == nullptr) return ((long)p.total_tokens + C - 1) / C;
    return p.slots;
}

// Whether the chunks of a call are mostly full: its tokens would fill at
// least half of its chunk slots (many requests, or dense rows, of a few
// tokens are not).
inline bool chunks_mostly_full(const Problem &p, int C) {
    return 2 * (((long)p.total_tokens + C - 1) / C) >= p.slots;
}

// Calls f.template operator()<EI, EO>() for the element types of the codes.
template <class EF32, class EBF16, class EF16, class F>
hipError_t dispatch_dtypes(int a_dt, int x_dt, F &&f) {
    auto with_out = [&](auto ein) -> hipError_t {
        using EI = decltype(ein);
        switch (x_dt) {
            case 0: return f.template operator()<EI, EF32>();
            case 1: return f.template operator()<EI, EBF16>();
            case 2: return f.template operator()<EI, EF16>();
        }
        return hipErrorInvalidValue;
    };
    switch (a_dt) {
        case 0: return with_out(EF32{});
        case 1: return with_out(EBF16{});
        case 2: return with_out(EF16{});
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
