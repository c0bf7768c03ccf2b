// Host helpers shared by the launchers.
#include <hip/hip_runtime.h>
#include <stdlib.h>

#include <mutex>
#include <vector>

#include "tril_launch.h"

namespace kda {

namespace {
// Wavefronts per compute unit below which the grid is never cut: the solver's
// memory pattern reaches the same rate with 16 and with 32 wavefronts per CU,
// and fewer leave too few bytes in flight.
constexpr long kMinWavesPerCu = 16;
// Largest grid of a multi-head launch: its 256-thread workgroups stay far
// below the 2^32 work-items of one dispatch; larger problems walk.
constexpr long kMaxGroupGrid = 1L << 22;

struct OccEntry {
    const void *fn;
    int dev;
    long per_cu;  // workgroups per compute unit
    long cus;
    bool forced;  // per_cu set by KDA_TRIL_BLOCKS_PER_CU
};
std::mutex g_occ_mu;
std::vector<OccEntry> g_occ;  // what the device reports, per kernel and device

OccEntry residency(const void *fn, int threads) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return {fn, 0, 0, 0, false};
    OccEntry r{fn, dev, 0, 0, false};
    bool cached = false;
    {
        std::lock_guard<std::mutex> lk(g_occ_mu);
        for (const OccEntry &e : g_occ)
            if (e.fn == fn && e.dev == dev) {
                r = e;
                cached = true;
                break;
            }
    }
    if (!cached) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess)
            per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        r.per_cu = per_cu;
        r.cus = cus;
        std::lock_guard<std::mutex> lk(g_occ_mu);
        g_occ.push_back(r);
    }
    // Tuning and testing override, read on every call (so one process can
    // launch the same problem on different grids): workgroups per compute
    // unit the grid is sized for.
    if (const char *e = getenv("KDA_TRIL_BLOCKS_PER_CU")) {
        const int v = atoi(e);
        if (v > 0) {
            r.per_cu = v;
            r.forced = true;
        }
    }
    return r;
}
}  // namespace

long device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus;
}

bool blocks_forced() {
    const char *e = getenv("KDA_TRIL_BLOCKS_PER_CU");
    return e != nullptr && atoi(e) > 0;
}

long resident_blocks(const void *fn, int threads) {
    const OccEntry r = residency(fn, threads);
    return r.per_cu * r.cus;
}

long walk_blocks(const void *fn, long waves, long min_waves) {
    const long need = (waves + kFusedWaves - 1) / kFusedWaves;
    const OccEntry r = residency(fn, kFusedThreads);
    if (r.per_cu <= 0 || r.cus <= 0) return need;
    long per_cu = r.per_cu;
    if (!r.forced && (per_cu - 1) * kFusedWaves >= kMinWavesPerCu && min_waves > 0) {
        // share of the last round's wavefront slots that has real items, for
        // b workgroups per CU; one fewer than the occupancy allows is taken
        // when it fills the last round better and still keeps kMinWavesPerCu
        // wavefronts on every compute unit
        auto fill = [&](long b) {
            const long slots = b * r.cus * kFusedWaves;
            const long rounds = (min_waves + slots - 1) / slots;
            return (double)min_waves / (double)(rounds * slots);
        };
        if (fill(per_cu - 1) > fill(per_cu)) per_cu -= 1;
    }
    const long cap = per_cu * r.cus;
    return cap < need ? cap : need;
}

long group_blocks(const void *fn, long groups) {
    long cap = kMaxGroupGrid;
    const OccEntry r = residency(fn, kFusedThreads);
    if (r.forced && r.cus > 0 && r.per_cu * r.cus < cap) cap = r.per_cu * r.cus;
    return cap < groups ? cap : groups;
}

}  // namespace kda
