// Tiles of four adjacent heads of one chunk, loaded from HBM straight into
// LDS, for the solver kernels in which a workgroup of four wavefronts owns a
// *group* (one chunk, four heads) and each wavefront one head of it.
//
// The four heads' rows of a token are adjacent in HBM (4 x 256 bytes for
// FP32, 4 x 128 for 16-bit elements), so a group's lines can be fetched with
// load instructions that each cover long runs of adjacent bytes, instead of
// 64-byte pieces 16 KiB apart as when each wavefront loads its own head. The
// loads are buffer loads with the LDS bit (gfx950's 16-byte direct-to-LDS
// form): the data go to LDS without passing through VGPRs, and every line is
// read by exactly one instruction, so they carry the nontemporal bit (same
// box, same buffers, the solver on 16 x 512 tokens: 42.9 -> 42.2 us; 48
// ragged requests 121.9 -> 117.9 us; 131,072 tokens 607 -> 583 us).
//
// Which lines a tile holds is a per-kernel plan over the four block rows
// (rows 16I..16I+15), per head: one 128-byte line of each row (columns 0..31
// or 32..63 of an FP32 row; a 16-bit row is one line), both lines, or none.
//
// LDS layout (bytes), in slots of kSlotBytes (1 KiB plus 16 bytes, so the 16
// rows one block read touches fall on different banks):
//   pair slot: rows r and r + 8 of one block row, each as one line of heads
//     0..3 (512 bytes); the second row's heads are rotated by one position,
//     so that the two rows sit 128 bytes apart in bank order. A block row
//     with one line per row takes 8 pair slots.
//   row slot: one FP32 row, all 256 bytes of heads 0..3. A block row with
//     both lines takes 16 row slots.
// Slots follow block-row order; wavefront w issues the loads of slots w,
// w + 4, w + 8, ... (every block row takes a multiple of four slots, so the
// kind of slot the q-th load fills is the same for all four wavefronts).
#pragma once

#include "tril_device.h"

namespace kda {

constexpr int kGroupHeads = 4;
constexpr int kSlotBytes = 1040;

// Lines of a block row's rows that a group tile holds (per head).
enum LineSel : int { kNone = 0, kLine0 = 1, kLine1 = 2, kBoth = 3 };

template <class EI, int M0, int M1, int M2, int M3>
struct GroupPlan {
    // a 16-bit row is a single line: any selection holds all of it
    __host__ __device__ static constexpr int mode(int I) {
        const int m = I == 0 ? M0 : I == 1 ? M1 : I == 2 ? M2 : M3;
        return (EI::kBytes == 2 && m != kNone) ? kLine0 : m;
    }
    __host__ __device__ static constexpr bool paired(int I) {
        return mode(I) == kLine0 || mode(I) == kLine1;
    }
    __host__ __device__ static constexpr int slots(int I) {
        return mode(I) == kNone ? 0 : paired(I) ? 8 : 16;
    }
    // (closed forms, so that a block row known only at run time costs a few
    // selects rather than a loop)
    __host__ __device__ static constexpr int base(int I) {
        return (I > 0 ? slots(0) : 0) + (I > 1 ? slots(1) : 0) + (I > 2 ? slots(2) : 0) +
               (I > 3 ? slots(3) : 0);
    }
    __host__ __device__ static constexpr int line_bytes(int I) {
        return mode(I) == kLine1 ? 128 : 0;
    }
    // the block row whose slots include slot s
    __host__ __device__ static constexpr int block_of(int s) {
        int I = 0;
        while (I < 3 && s >= base(I + 1)) ++I;
        return I;
    }
    static constexpr int kSlots = base(4);
    static constexpr int kBytes = kSlots * kSlotBytes;

    // LDS byte address of row R, head position hh, byte column bc of that
    // head's row (bc inside the lines the plan holds for R's block row)
    // (one address expression with selects, not two branches: R's block row
    // is not always known at compile time)
    __device__ static __forceinline__ int addr(int R, int hh, int bc) {
        const int I = R >> 4;
        const bool pr = paired(I);
        const int half = (R >> 3) & 1;
        const int pos = half ? (hh + 3) & 3 : hh;
        const int slot = base(I) + (pr ? (R & 7) : (R & 15));
        const int inner = pr ? half * 512 + pos * 128 - line_bytes(I) : hh * 256;
        return slot * kSlotBytes + inner + bc;
    }
};

typedef __attribute__((address_space(3))) void *LdsPtr;

// This wavefront's share of a group's loads (slots wid, wid + 4, ...). Lanes
// of heads past the last head (nh < 4) use an out-of-range offset: their LDS
// bytes get 0 and no memory is read for them.
template <class EI, class Plan>
__device__ __forceinline__ void load_group(Rsrc r, int rstride, int nh, char *lds, int wid,
                                           int lane) {
    const int half = lane >> 5, pos = (lane >> 3) & 3, piece = lane & 7;
    const int ph = half ? (pos + 1) & 3 : pos;  // head whose bytes land at this position
    const uint32_t pmask = ph < nh ? 0u : kOffMasked;
    const uint32_t rmask = (lane >> 4) < nh ? 0u : kOffMasked;
#pragma unroll
    for (int q = 0; q < Plan::kSlots / 4; ++q) {
        const int I = Plan::block_of(4 * q);
        const int s = wid + 4 * q;
        const int j = s - Plan::base(I);  // slot within the block row
        uint32_t off;
        if (Plan::paired(I)) {
            const int row = 16 * I + j + 8 * half;
            off = ((uint32_t)(row * rstride + ph * 64) * EI::kBytes + Plan::line_bytes(I) +
                   16 * piece) | pmask;
        } else {
            const int row = 16 * I + j;
            off = ((uint32_t)(row * rstride) * EI::kBytes + 16 * lane) | rmask;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(lds + s * kSlotBytes), 16, off, 0,
                                                 0, kNontemporal);
    }
}

// Columns c..c+3 of row R of head position hh, widened to FP32.
template <class EI, class Plan>
__device__ __forceinline__ f4 lds_quad(const char *lds, int R, int hh, int c) {
    if constexpr (EI::kBytes == 4) {
        return *reinterpret_cast<const f4 *>(lds + Plan::addr(R, hh, 4 * c));
    } else if constexpr (__is_same(EI, BF16)) {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 v = *reinterpret_cast<const u2 *>(lds + Plan::addr(R, hh, 2 * c));
        f4 o;
        o[0] = bf16_to_f32(v[0] & 0xFFFFu);
        o[1] = bf16_to_f32(v[0] >> 16);
        o[2] = bf16_to_f32(v[1] & 0xFFFFu);
        o[3] = bf16_to_f32(v[1] >> 16);
        return o;
    } else {
        // a vector of binary16 values, as the global loads widen them
        // (converting single 16-bit lanes of an integer vector through bit
        // casts lost three of every four elements in this compiler's output)
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 v = *reinterpret_cast<const h4 *>(lds + Plan::addr(R, hh, 2 * c));
        f4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (float)v[e];  // exact widening
        return o;
    }
}

// Head position hh's diagonal blocks, one row per lane (lane (b, i): row
// 16b + i, columns 16b + 4q..+3 in dg[q]).
template <class EI, class Plan>
__device__ __forceinline__ void read_diag_rows(f4 (&dg)[4], const char *lds, int hh, int lane) {
    const int b = lane >> 4, i = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) dg[q] = lds_quad<EI, Plan>(lds, 16 * b + i, hh, 16 * b + 4 * q);
}

// Head position hh's six blocks below the diagonal in OPND_A (lane (g, m):
// row 16I + m, columns 16K + 4g..+3).
template <class EI, class Plan>
__device__ __forceinline__ void read_offdiag_blocks(f4 (&blk)[4][4], const char *lds, int hh,
                                                    int lane) {
    const int g = lane >> 4, m = lane & 15;
#pragma unroll
    for (int I = 1; I < 4; ++I)
#pragma unroll
        for (int K = 0; K < I; ++K) blk[I][K] = lds_quad<EI, Plan>(lds, 16 * I + m, hh, 16 * K + 4 * g);
}

// A group of four heads of one chunk slot (len 0: nothing to do).
struct Group {
    Chunk ch;
    int h0, nh;
};

// Group gi of a launch over slots x hg groups (hg = heads / 4, rounded up).
// The chunk is the same for the whole workgroup, so every wavefront takes the
// same branches and meets the same barriers.
__device__ __forceinline__ Group group_of(const Problem &p, int gi, int hg, int lane) {
    Group gr;
    const int slot = gi / hg;
    gr.h0 = (gi - slot * hg) * kGroupHeads;
    gr.nh = min(kGroupHeads, p.heads - gr.h0);
    gr.ch = uniform(resolve_chunk<kChunk>(p, slot, lane));
    return gr;
}

// The group's tiles of A into LDS, as the plan says.
template <class EI, class Plan>
__device__ __forceinline__ void load_group_of(const Problem &p, const Group &gr, char *lds,
                                              int wid, int lane) {
    const long row0 = (long)gr.ch.start * p.heads + gr.h0;
    const TileView<EI> A{static_cast<const typename EI::T *>(p.A) + row0 * kChunk,
                         p.heads * kChunk, gr.ch.len, gr.nh * kChunk};
    load_group<EI, Plan>(A.rows_from(0), A.rstride, gr.nh, lds, wid, lane);
}

// Waits for this wavefront's share of the group's loads, then for every
// wavefront's (the loads are counted by vmcnt and done once it is 0).
__device__ __forceinline__ void group_arrived() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

}  // namespace kda
