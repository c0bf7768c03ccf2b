// Host helpers shared by the launchers.
#include <hip/hip_runtime.h>
#include <stdlib.h>

#include <mutex>
#include <vector>

#include "tril_launch.h"

namespace kda {

namespace {
struct OccEntry {
    const void *fn;
    int dev;
    long blocks;
};
std::mutex g_occ_mu;
std::vector<OccEntry> g_occ;
}  // namespace

long resident_blocks(const void *fn, int threads) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    {
        std::lock_guard<std::mutex> lk(g_occ_mu);
        for (const OccEntry &e : g_occ)
            if (e.fn == fn && e.dev == dev) return e.blocks;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess)
        per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 0;
    // Tuning override: workgroups per compute unit the grid is sized for.
    if (const char *e = getenv("KDA_TRIL_BLOCKS_PER_CU")) {
        const int v = atoi(e);
        if (v > 0) per_cu = v;
    }
    const long blocks = (long)per_cu * cus;
    std::lock_guard<std::mutex> lk(g_occ_mu);
    g_occ.push_back({fn, dev, blocks});
    return blocks;
}

}  // namespace kda
