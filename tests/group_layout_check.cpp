// Host-side check of the 4-head group tiles (tril_group.h), for every plan the
// solver kernels use and every input element type. It runs the header's own
// address arithmetic on the CPU, no GPU involved:
//   - the loads: every lane of every load instruction (GroupPlan::load_src)
//     brings 16 bytes of the rows, heads and columns the plan holds, lands
//     inside the tile, and no two lanes write the same LDS byte; every byte
//     the plan holds is loaded exactly once;
//   - the reads: every byte the solve reads through GroupPlan::addr (the
//     diagonal rows, one per lane, and the blocks below the diagonal, in the
//     layouts of read_diag_rows and read_offdiag_blocks) holds the element of
//     A it stands for;
//   - the banks: within each 16-lane group of such a read, the lanes' bytes
//     fall on different banks (64 banks of 4 bytes), the property the slot
//     padding and the head rotation are there for.
// Prints one line per plan and "ok" at the end; exits non-zero on the first
// violation.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tril_group.h"

using namespace kda;

namespace {

struct Elem {
    int row, head, byte;
};

[[noreturn]] void fail(const char *plan, const char *what, int a, int b, int c) {
    std::printf("FAIL %s: %s (%d, %d, %d)\n", plan, what, a, b, c);
    std::exit(1);
}

long key(int row, int head, int byte) { return ((long)row * 4 + head) * 512 + byte; }

template <class EI, class Plan>
void check(const char *name, bool diag, bool offdiag) {
    constexpr int E = EI::kBytes;
    std::vector<long> owner(Plan::kBytes, -1);
    std::vector<int> times(64 * 4 * 512, 0);
    for (int s = 0; s < Plan::kSlots; ++s) {
        const int I = Plan::block_of(s);
        for (int lane = 0; lane < 64; ++lane) {
            const typename Plan::Src src = Plan::load_src(I, s - Plan::base(I), lane);
            if (src.row < 16 * I || src.row >= 16 * I + 16 || src.head < 0 || src.head > 3 ||
                src.byte < Plan::lo(I) || src.byte + 16 > Plan::lo(I) + Plan::piece(I) ||
                src.byte % 16 != 0)
                fail(name, "load outside the plan's columns", s, lane, src.byte);
            for (int b = 0; b < 16; ++b) {
                const int L = s * kSlotBytes + 16 * lane + b;
                if (L >= Plan::kBytes) fail(name, "load past the tile", s, lane, L);
                if (owner[L] != -1) fail(name, "two loads write one LDS byte", s, lane, L);
                owner[L] = key(src.row, src.head, src.byte + b);
                ++times[key(src.row, src.head, src.byte + b)];
            }
        }
    }
    for (int I = 0; I < 4; ++I)
        for (int r = 16 * I; r < 16 * I + 16; ++r)
            for (int h = 0; h < 4; ++h)
                for (int b = 0; b < kChunk * E; ++b) {
                    const bool held = b >= Plan::lo(I) && b < Plan::lo(I) + Plan::piece(I);
                    if (times[key(r, h, b)] != (held ? 1 : 0))
                        fail(name, "byte not loaded exactly once", r, h, b);
                }
    // one read instruction: lane -> (row, column of its 4 elements)
    auto check_read = [&](int hh, auto where) {
        std::vector<int> banks;
        for (int lane = 0; lane < 64; ++lane) {
            int R, c;
            where(lane, R, c);
            for (int b = 0; b < 4 * E; ++b) {
                const int a = Plan::addr(R, hh, c * E + b);
                if (a < 0 || a >= Plan::kBytes || owner[a] != key(R, hh, c * E + b))
                    fail(name, "read finds another element", R, hh, c * E + b);
            }
            if (lane % 16 == 0) banks.assign(64, 0);
            for (int d = 0; d < E; ++d)
                if (++banks[(Plan::addr(R, hh, c * E) / 4 + d) % 64] > 1)
                    fail(name, "two lanes of a 16-lane group on one bank", R, hh, c);
        }
    };
    for (int hh = 0; hh < 4; ++hh) {
        if (diag)
            for (int q = 0; q < 4; ++q)
                check_read(hh, [&](int lane, int &R, int &c) {
                    const int b = lane >> 4, i = lane & 15;
                    R = 16 * b + i;
                    c = 16 * b + 4 * q;
                });
        if (offdiag)
            for (int I = 1; I < 4; ++I)
                for (int K = 0; K < I; ++K)
                    check_read(hh, [&](int lane, int &R, int &c) {
                        const int g = lane >> 4, m = lane & 15;
                        R = 16 * I + m;
                        c = 16 * K + 4 * g;
                    });
    }
    std::printf("%s: %d slots, %d bytes\n", name, Plan::kSlots, Plan::kBytes);
}

}  // namespace

int main() {
    check<F32, FusedPlan<F32>>("fused f32", true, true);
    check<BF16, FusedPlan<BF16>>("fused bf16", true, true);
    check<F16, FusedPlan<F16>>("fused f16", true, true);
    check<F32, DiagPlan<F32>>("split diagonal f32", true, false);
    check<BF16, DiagPlan<BF16>>("split diagonal bf16", true, false);
    check<F32, MergePlan<F32>>("split merge f32", false, true);
    check<BF16, MergePlan<BF16>>("split merge bf16", false, true);
    std::printf("ok\n");
    return 0;
}
