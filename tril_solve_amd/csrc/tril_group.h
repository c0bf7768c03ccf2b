// Tiles of four adjacent heads of one chunk, loaded from HBM straight into
// LDS, for the solver kernels in which a workgroup of four wavefronts owns a
// *group* (one chunk, four heads) and each wavefront one head of it.
//
// The four heads' rows of a token are adjacent in HBM (4 x 256 bytes for
// FP32, 4 x 128 for 16-bit elements), so a group's rows can be fetched with
// load instructions that each cover long runs of adjacent bytes, instead of
// 64-byte pieces 16 KiB apart as when each wavefront loads its own head. The
// loads are buffer loads with the LDS bit (gfx950's 16-byte direct-to-LDS
// form): the data go to LDS without passing through VGPRs, and every byte is
// read by exactly one instruction, so they carry the nontemporal bit (same
// box, same buffers, the fused solver on 16 x 512 tokens: 42.9 -> 42.2 us;
// 48 ragged requests 121.9 -> 117.9 us; 131,072 tokens 607 -> 583 us).
//
// Which columns a tile holds is a per-kernel plan over the four block rows
// (rows 16I..16I+15): for each block row, columns c0..c0+nc-1 of every row of
// every head, where nc x element size is 64, 128 or 256 bytes (a quarter,
// half or whole FP32 row; a half or whole 16-bit row), or nothing.
//
// LDS layout (bytes), in slots of kSlotBytes (1 KiB plus 16 bytes, so the 16
// rows one block read touches fall on different banks). A slot is what one
// load instruction fills: n = 256 / piece rows of the four heads, where piece
// is the bytes of a row the plan holds. Block row I takes 16 / n slots; its
// slot j holds rows j, j + 16/n, j + 2*16/n, ... of the block row, the k-th
// of them at byte k * 4 * piece with its heads rotated by k positions (head
// hh at position (hh - k) mod 4), so that the rows a 16-lane read touches sit
// on different banks. Slots follow block-row order; wavefront w issues the
// loads of slots w, w + 4, w + 8, ... (every block row takes a multiple of
// four slots, so what the q-th load of a wavefront fills is known at compile
// time).
#pragma once

#include "tril_device.h"

namespace kda {

constexpr int kGroupHeads = 4;
constexpr int kSlotBytes = 1040;

// A block row's columns c0..c0+nc-1 (nc = 0: none), as a plan's argument.
__host__ __device__ constexpr int cols(int c0, int nc) { return (c0 << 8) | nc; }

template <class EI, int S0, int S1, int S2, int S3>
struct GroupPlan {
    __host__ __device__ static constexpr int sel(int I) {
        return I == 0 ? S0 : I == 1 ? S1 : I == 2 ? S2 : S3;
    }
    // bytes of a row held, and the byte column where they start
    __host__ __device__ static constexpr int piece(int I) { return (sel(I) & 255) * EI::kBytes; }
    __host__ __device__ static constexpr int lo(int I) { return (sel(I) >> 8) * EI::kBytes; }
    // rows per slot, and slots of block row I
    __host__ __device__ static constexpr int rows(int I) {
        return piece(I) == 0 ? 1 : 256 / piece(I);
    }
    __host__ __device__ static constexpr int slots(int I) {
        return piece(I) == 0 ? 0 : 16 / rows(I);
    }
    __host__ __device__ static constexpr bool valid(int I) {
        return piece(I) == 0 ||
               ((piece(I) == 64 || piece(I) == 128 || piece(I) == 256) &&
                lo(I) % piece(I) == 0 && lo(I) + piece(I) <= kChunk * EI::kBytes);
    }
    static_assert(valid(0) && valid(1) && valid(2) && valid(3),
                  "a block row holds an aligned quarter, half or whole FP32 row, or an "
                  "aligned half or whole 16-bit row");
    // (closed forms, so that a block row known only at run time costs a few
    // selects rather than a loop)
    __host__ __device__ static constexpr int base(int I) {
        return (I > 0 ? slots(0) : 0) + (I > 1 ? slots(1) : 0) + (I > 2 ? slots(2) : 0) +
               (I > 3 ? slots(3) : 0);
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
    // head's row (bc inside the columns the plan holds for R's block row);
    // one expression with selects, not branches, as R's block row is not
    // always known at compile time
    __host__ __device__ static __forceinline__ int addr(int R, int hh, int bc) {
        const int I = R >> 4, r = R & 15;
        const int per = slots(I);  // a power of two
        const int j = r & (per - 1), k = r / per;
        const int pos = (hh - k) & 3;
        return (base(I) + j) * kSlotBytes + (4 * k + pos) * piece(I) + bc - lo(I);
    }

    // What lane `lane` of the load that fills slot j of block row I (LDS
    // slot base(I) + j) brings: 16 bytes of row `row` of the chunk, head
    // position `head`, from byte column `byte` of that head's row, landing at
    // byte 16 * lane of the slot. Lane l of a load that fills n rows takes
    // row k = l / (64 / n) of the slot, and a position and 16-byte piece in
    // it; the position holds head (pos + k) mod 4.
    struct Src {
        int row, head, byte;
    };
    __host__ __device__ static __forceinline__ Src load_src(int I, int j, int lane) {
        const int n = rows(I), per = slots(I);
        const int pieces = piece(I) / 16;  // lanes per (row, head)
        const int k = lane / (64 / n);
        const int w = lane % (64 / n);
        const int pos = w / pieces, pc = w % pieces;
        return Src{16 * I + j + k * per, (pos + k) & 3, lo(I) + 16 * pc};
    }
};

// The plans of the solver kernels.
// The fused kernel needs columns 0..31 of block rows 0 and 1 and columns
// 0..63 of block rows 2 and 3; rows of 16-bit elements are loaded whole, as
// one 128-byte line each.
template <class EI>
using FusedPlan = GroupPlan<EI, cols(0, EI::kBytes == 4 ? 32 : 64),
                            cols(0, EI::kBytes == 4 ? 32 : 64), cols(0, 64), cols(0, 64)>;
// The split plan's diagonal kernel reads the diagonal blocks alone: columns
// 16I..16I+15 of block row I, a quarter FP32 row; 16-bit rows in halves
// (columns 0..31 for block rows 0 and 1, 32..63 for 2 and 3), 64 bytes each.
template <class EI>
using DiagPlan = GroupPlan<EI, EI::kBytes == 4 ? cols(0, 16) : cols(0, 32),
                           EI::kBytes == 4 ? cols(16, 16) : cols(0, 32),
                           EI::kBytes == 4 ? cols(32, 16) : cols(32, 32),
                           EI::kBytes == 4 ? cols(48, 16) : cols(32, 32)>;
// The split plan's merge kernel reads the blocks below the diagonal: columns
// 0..15 of block row 1 (16-bit: 0..31, 64 bytes), 0..31 of block row 2,
// whole rows of block row 3.
template <class EI>
using MergePlan = GroupPlan<EI, cols(0, 0), cols(0, EI::kBytes == 4 ? 16 : 32), cols(0, 32),
                            cols(0, 64)>;

typedef __attribute__((address_space(3))) void *LdsPtr;

// This wavefront's share of a group's loads (slots wid, wid + 4, ...), each
// lane's 16 bytes as Plan::load_src says. Lanes of heads past the last head
// (nh < 4) use an out-of-range offset: their LDS bytes get 0 and no memory is
// read for them.
template <class EI, class Plan>
__device__ __forceinline__ void load_group(Rsrc r, int rstride, int nh, char *lds, int wid,
                                           int lane) {
#pragma unroll
    for (int q = 0; q < Plan::kSlots / 4; ++q) {
        // the slot's block row depends on q alone (every block row takes a
        // multiple of four slots), so it is known at compile time
        const int I = Plan::block_of(4 * q);
        const int s = wid + 4 * q;
        const typename Plan::Src src = Plan::load_src(I, s - Plan::base(I), lane);
        const uint32_t off =
            ((uint32_t)(src.row * rstride + src.head * kChunk) * EI::kBytes + src.byte) |
            (src.head < nh ? 0u : kOffMasked);
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
        for (int K = 0; K < I; ++K)
            blk[I][K] = lds_quad<EI, Plan>(lds, 16 * I + m, hh, 16 * K + 4 * g);
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
