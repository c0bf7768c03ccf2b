// Host-side planning of a solver call: workspace size and the fused/split
// choice. Pure host code, no HIP calls, so it runs on machines without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kda_tril.h"

namespace kda {

// FP32 scratch of the split path per chunk-head: four 16x16 FP32 tiles.
constexpr int64_t kSplitBytesPerMatrix = 4 * 16 * 16 * 4;
// FP32 input bytes per token and head (one 64-wide row), the budget unit.
constexpr int64_t kF32RowBytes = 64 * 4;

// Smallest packed/dense token count at which AUTO prefers the split path.
// Measured on MI355X; overridable with KDA_TRIL_SPLIT_MIN_TOKENS.
int64_t split_min_tokens();

// Chunk slots the kernels cover for chunks of `chunk` tokens: the exact count
// when known, else the bound floor(T / chunk) + num_seqs (each request adds at
// most one partial chunk).
int64_t chunk_slots(int64_t total_tokens, int64_t num_seqs, int64_t num_chunks, int chunk);

// Workspace bytes of the split path for this many chunk slots.
int64_t split_workspace_bytes(int64_t slots, int32_t heads);

// Split is allowed when its scratch does not exceed the FP32 input size
// (T x H x 64 x 4 bytes), i.e. mean chunk occupancy T / slots >= 16.
bool split_within_budget(int64_t total_tokens, int64_t slots, int32_t heads);

// Resolve a requested plan. `ws_bytes` is the workspace the caller offers
// (use SIZE_MAX to ask what AUTO would pick with unlimited workspace).
// Returns KDA_ERR_WORKSPACE when SPLIT is forced but not allowed or not
// given enough workspace; *chosen is set on success.
kda_status resolve_plan(int64_t total_tokens, int64_t slots, int32_t heads, kda_algo requested,
                        size_t ws_bytes, kda_algo *chosen);

}  // namespace kda
