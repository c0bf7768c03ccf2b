// Host-side planning: workspace sizes and the fused/split choice.
//
// LightLLM PR #1703 ("perf(kda): parallelize diagonal solves in Prefill")
// selects splitting by an FP32 workspace budget and a minimum input length
// (PR description) and bounds scratch by chunk occupancy (commit summary).
// Here the budget is the FP32 input size T x H x 256 bytes, the split scratch
// is 4096 bytes per chunk slot and head, and AUTO splits only when the call
// offers that much workspace, fits the budget, and has at least
// split_min_tokens() tokens.
#include "plan.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

namespace kda {

// No input size has been measured on MI355X at which the split path beats the
// fused kernel (the fused kernel already runs the four diagonal solves in
// parallel and moves 8 KiB less per chunk-head), so by default AUTO does not
// split. KDA_TRIL_SPLIT_MIN_TOKENS lowers the threshold for experiments.
static constexpr int64_t kDefaultSplitMinTokens = INT64_MAX;

int64_t split_min_tokens() {
    const char *e = getenv("KDA_TRIL_SPLIT_MIN_TOKENS");
    if (e && *e) {
        char *end = nullptr;
        long long v = strtoll(e, &end, 10);
        if (end && *end == '\0' && v >= 0) return (int64_t)v;
    }
    return kDefaultSplitMinTokens;
}

// Tuning override of AUTO: KDA_TRIL_ALGO = fused | split | fused_valu makes
// calls that ask for AUTO run that plan instead (a split that is not eligible
// still falls back to fused, as AUTO does); unset, empty or "auto" keeps the
// rule. Calls that name a plan are never overridden.
static kda_algo auto_override() {
    const char *e = getenv("KDA_TRIL_ALGO");
    if (e == nullptr || *e == '\0') return KDA_ALGO_AUTO;
    if (strcmp(e, "fused") == 0) return KDA_ALGO_FUSED;
    if (strcmp(e, "split") == 0) return KDA_ALGO_SPLIT;
    if (strcmp(e, "fused_valu") == 0) return KDA_ALGO_FUSED_VALU;
    return KDA_ALGO_AUTO;
}

int64_t chunk_slots(int64_t total_tokens, int64_t num_seqs, int64_t num_chunks, int chunk) {
    if (num_chunks > 0) return num_chunks;
    return total_tokens / chunk + num_seqs;
}

int64_t split_workspace_bytes(int64_t slots, int32_t heads) {
    return slots * (int64_t)heads * kSplitBytesPerMatrix;
}

bool split_within_budget(int64_t total_tokens, int64_t slots, int32_t heads) {
    return split_workspace_bytes(slots, heads) <= total_tokens * (int64_t)heads * kF32RowBytes;
}

kda_status resolve_plan(int64_t total_tokens, int64_t slots, int32_t heads, kda_algo requested,
                        size_t ws_bytes, kda_algo *chosen) {
    const int64_t need = split_workspace_bytes(slots, heads);
    const bool budget_ok = split_within_budget(total_tokens, slots, heads);
    const bool ws_ok = ws_bytes >= (size_t)need;
    kda_algo out = requested;
    switch (requested) {
        case KDA_ALGO_FUSED:
        case KDA_ALGO_FUSED_VALU:
            break;
        case KDA_ALGO_SPLIT:
            if (!budget_ok || !ws_ok) return KDA_ERR_WORKSPACE;
            break;
        case KDA_ALGO_AUTO: {
            const kda_algo forced = auto_override();
            if (forced == KDA_ALGO_SPLIT)
                out = (budget_ok && ws_ok) ? KDA_ALGO_SPLIT : KDA_ALGO_FUSED;
            else if (forced != KDA_ALGO_AUTO)
                out = forced;
            else
                out = (budget_ok && ws_ok && total_tokens >= split_min_tokens())
                          ? KDA_ALGO_SPLIT
                          : KDA_ALGO_FUSED;
            break;
        }
        default:
            return KDA_ERR_INVALID_ARG;
    }
    const char *log = getenv("KDA_TRIL_LOG");
    if (log && *log && *log != '0')
        fprintf(stderr,
                "kda_tril: T=%lld slots=%lld H=%d requested=%d -> %d (split scratch %lld B, "
                "budget %s, workspace %s)\n",
                (long long)total_tokens, (long long)slots, (int)heads, (int)requested, (int)out,
                (long long)need, budget_ok ? "ok" : "exceeded", ws_ok ? "ok" : "short");
    *chosen = out;
    return KDA_OK;
}

}  // namespace kda
