// Fused KDA decode core for gfx950: one decode step (one new token per
// sequence) of the causal convolution with its state, the KDA recurrent
// update and gated RMSNorm, in one kernel.
//
// tokenspeed PR #1086 ("perf(kimi3): fuse KDA decode core", PR description)
// fuses exactly these parts into one kernel for GFX950 and tests them against
// convolution, paged-state, padding and gated-RMSNorm references. The page
// states no formulas; the step computed here, per sequence b and head h
// (head dim D = 128, conv width W), is:
//
//   y_p = silu(sum_w cw[p][w] * window_p[w]),  window_p = (W-1 previous inputs, x_p)
//   q = y_q / sqrt(|y_q|^2 + eps_l2) / sqrt(D),  k = y_k / sqrt(|y_k|^2 + eps_l2),  v = y_v
//   S <- diag(exp(g)) S;  u = beta (v - S^T k);  S <- S + k u^T;  o = S^T q
//   out = o / sqrt(mean(o^2) + eps_norm) * wn * sigmoid(z)
//
// with S (D x D FP32, key rows, value columns) and the conv windows kept in
// paged pools indexed by a per-sequence slot (negative or past the pool: a
// padding entry).
//
// One workgroup of 256 threads per (sequence, head). The state dominates the
// traffic (64 KiB read and 64 KiB written per step), so every other input is
// loaded first and the state tile right after, before any wait; the
// convolution and the norms then run while the tile is in flight. Two ways
// to split the state over the four wavefronts (S_new^T q = (decayed S)^T q +
// (k . q) u, so either way the state is read and written exactly once):
//   - by value columns (larger batches): wavefront w owns columns
//     32w..32w+31 of all 128 key rows (lane l: columns 32w + 4(l % 8) .. +3
//     of rows 16(l / 8) .. +15), so the reductions over key rows (S^T k and
//     S^T q of the decayed state) stay inside the wavefront (per-lane sums
//     over 16 rows, then lanes xor 8, 16, 32) and each wavefront updates and
//     writes back its columns as soon as its own tile has arrived, with no
//     barrier in between;
//   - by pairs of key rows (up to one (sequence, head) pair per compute
//     unit, where latency rules): wavefront w owns row pairs 4i + w (lanes
//     0..31 the even row, 32..63 the odd one; lane l: columns 4(l % 32) .. +3),
//     so every load and store instruction covers two whole rows, 1 KiB of
//     adjacent bytes instead of eight 128-byte pieces; the row sums of the
//     four wavefronts meet in LDS after one barrier.
// Same box, same state pools, B sequences x 32 heads (µs per step, columns /
// row pairs): B = 2 6.44 / 6.24-6.25, 4 7.31-7.35 / 7.10-7.17, 8 8.98-8.99 /
// 8.45-8.49, 16 14.98-14.99 / 15.14-15.19 (another box: 14.94-14.96 /
// 14.52-14.60), 32 27.59-27.60 / 28.41-28.50.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "tril_device.h"
#include "tril_launch.h"

namespace kda {

constexpr int kDecD = 128;         // head dim (keys = values)
constexpr int kDecThreads = 256;
constexpr int kDecRows = 16;       // state rows per lane
constexpr int kDecPad = kDecD + kDecD / 16;

__device__ __forceinline__ int pad_row(int r) { return r + (r >> 4); }

template <class E>
__device__ __forceinline__ float ld_elem(const typename E::T *p, long i);
template <>
__device__ __forceinline__ float ld_elem<F32>(const float *p, long i) {
    return p[i];
}
template <>
__device__ __forceinline__ float ld_elem<BF16>(const uint16_t *p, long i) {
    return bf16_to_f32(p[i]);
}
template <>
__device__ __forceinline__ float ld_elem<F16>(const uint16_t *p, long i) {
    return (float)__builtin_bit_cast(_Float16, p[i]);
}

template <class E>
__device__ __forceinline__ void st_elem(typename E::T *p, long i, float v);
template <>
__device__ __forceinline__ void st_elem<F32>(float *p, long i, float v) {
    p[i] = v;
}
template <>
__device__ __forceinline__ void st_elem<BF16>(uint16_t *p, long i, float v) {
    p[i] = __builtin_bit_cast(uint16_t, (__bf16)v);
}
template <>
__device__ __forceinline__ void st_elem<F16>(uint16_t *p, long i, float v) {
    p[i] = __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Cross-lane sums on DPP moves and lane swaps (no LDS round trips; the
// shuffle-based butterflies compiled to one ds_bpermute per step). Each step
// adds the value of a partner lane; partners are paired both ways, so every
// lane of a group ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                                  0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141;   // lane i <-> 7 - i within each 8 lanes
constexpr int kRowMirror = 0x140;    // lane i <-> 15 - i within each 16-lane row
constexpr int kRowRor8 = 0x128;      // lane i <-> i + 8 (mod 16) within each row
// 16-lane rows 0 + 1 and 2 + 3, lanes at the same position in their rows
__device__ __forceinline__ float rows_pair_add(float v) {
    float a = v, b = v;
    lane_swap16(a, b);
    return a + b;
}
// rows 0 + 2 and 1 + 3
__device__ __forceinline__ float rows_half_add(float v) {
    float a = v, b = v;
    lane_swap32(a, b);
    return a + b;
}

// Sum over the 64 lanes of a wavefront (result in every lane).
__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_add<kQuadXor1>(v);
    v = dpp_add<kQuadXor2>(v);
    v = dpp_add<kHalfMirror>(v);
    v = dpp_add<kRowMirror>(v);
    v = rows_pair_add(v);
    return rows_half_add(v);
}

// One step for one (sequence, head); layouts as in the C ABI. PAIRS: the
// state split by pairs of key rows, else by value columns.
template <class EI, class EO, bool PAIRS>
__global__ __launch_bounds__(kDecThreads) void kda_decode_step_kernel(DecodeProblem p) {
    // per key row: padded (row r at r + r / 16), so the 8 rows a wavefront
    // reads at once (16 apart) fall in distinct banks
    __shared__ float yq[kDecPad], yk[kDecPad], gq[kDecPad];
    __shared__ __align__(16) float yv[kDecD], zs[kDecD], nws[kDecD];  // per value column
    // row sums of each wavefront (PAIRS), or each wavefront's sum of o^2
    __shared__ __align__(16) float red_k[kDecThreads / kWave][kDecD];
    __shared__ __align__(16) float red_q[kDecThreads / kWave][kDecD];

    const int t = threadIdx.x;
    const int b = blockIdx.x / p.H, h = blockIdx.x - b * p.H;
    const long bh = (long)b * p.H + h;
    const int slot = p.slot[b];
    typename EO::T *out = static_cast<typename EO::T *>(p.out) + bh * kDecD;
    if (slot < 0 || slot >= p.num_slots) {  // padding (or a slot outside the pool)
        if (t < kDecD) st_elem<EO>(out, t, 0.0f);
        return;
    }

    // 1. every small input first: the memory counter waits in issue order, so
    //    a load issued after the state tile could only be used once the whole
    //    tile had arrived. Threads 0..127 handle the q and k channels of the
    //    convolution, threads 128..255 the v channels; conv widths 2..4. The
    //    loads are unconditional (indices past the width or the thread's
    //    projections are clamped to valid ones and their values unused), so
    //    they form one block that the state loads follow with no wait between.
    const int c = t & (kDecD - 1);
    const int W = p.W;
    const int wv = __builtin_amdgcn_readfirstlane(t) / kWave;  // wavefront index
    const bool low = wv < 2;
    const int pfirst = low ? 0 : 2, pn = low ? 2 : 1;
    const typename EI::T *qkv = static_cast<const typename EI::T *>(p.qkv);
    float xin[2], win[2][3], tap[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int p3 = k < pn ? pfirst + k : pfirst;
        xin[k] = ld_elem<EI>(qkv, ((long)b * 3 + p3) * p.H * kDecD + (long)h * kDecD + c);
        const float *ws = p.conv_state + (((long)slot * 3 + p3) * p.H + h) * (long)(W - 1) * kDecD;
        const float *cw = p.conv_w + ((long)p3 * W * p.H + h) * kDecD + c;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (w < 3) win[k][w] = ws[(long)(w < W - 1 ? w : 0) * kDecD + c];
            tap[k][w] = cw[(long)(w < W ? w : 0) * p.H * kDecD];
        }
    }
    const float graw = p.g[bh * kDecD + c];
    const float beta = p.beta[bh];
    // z (threads 0..127) and norm_w (threads 128..255), kept in LDS until the end
    const float zraw = ld_elem<EI>(static_cast<const typename EI::T *>(p.z), bh * kDecD + c);
    const float nwraw = p.norm_w[c];
    // this lane's 4 value columns and its 16 key rows
    const int l = t & (kWave - 1);
    const int col = PAIRS ? 4 * (l & 31) : 32 * wv + 4 * (l & 7);
    const int half = l >> 5;  // PAIRS: the row of the pair
    auto key_row = [&](int i) { return PAIRS ? 2 * (4 * i + wv) + half : 16 * (l >> 3) + i; };

    // 2. then the state tile of this lane
    float *S = p.state + ((long)slot * p.H + h) * kDecD * kDecD + col;
    f4 s[kDecRows];
#pragma unroll
    for (int i = 0; i < kDecRows; ++i)
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(&S[(long)key_row(i) * kDecD]));
    __builtin_amdgcn_sched_barrier(0);  // keep every use of the loads below this point

    // 3. causal convolution over the window of the W - 1 previous inputs and
    //    the new one; the window then shifts by one (oldest entry dropped)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (k < pn) {
            const int p3 = pfirst + k;
            float *ws = p.conv_state + (((long)slot * 3 + p3) * p.H + h) * (long)(W - 1) * kDecD;
            float acc = 0.0f;
#pragma unroll
            for (int w = 0; w < 3; ++w)
                if (w < W - 1) acc = __builtin_fmaf(tap[k][w], win[k][w], acc);
#pragma unroll
            for (int w = 0; w < 4; ++w)
                if (w == W - 1) acc = __builtin_fmaf(tap[k][w], xin[k], acc);
#pragma unroll
            for (int w = 1; w < 3; ++w)
                if (w < W - 1) ws[(long)(w - 1) * kDecD + c] = win[k][w];
            ws[(long)(W - 2) * kDecD + c] = xin[k];
            const float y = acc / (1.0f + __expf(-acc));  // silu
            if (p3 == 0) yq[pad_row(c)] = y;
            if (p3 == 1) yk[pad_row(c)] = y;
            if (p3 == 2) yv[c] = y;
        }
    }
    if (low) {
        gq[pad_row(c)] = __expf(graw);
        zs[c] = zraw;
    } else {
        nws[c] = nwraw;
    }
    __syncthreads();

    // 4. squared norms of y_q, y_k and their dot product, in every wavefront
    float sq, sk, dqk;
    {
        const float a0 = yq[pad_row(l)], a1 = yq[pad_row(l + kWave)];
        const float k0 = yk[pad_row(l)], k1 = yk[pad_row(l + kWave)];
        const float nq = wave_sum(a0 * a0 + a1 * a1), nk = wave_sum(k0 * k0 + k1 * k1);
        dqk = wave_sum(a0 * k0 + a1 * k1);
        sq = 1.0f / (__builtin_sqrtf(nq + p.eps_l2) * __builtin_sqrtf((float)kDecD));
        sk = 1.0f / __builtin_sqrtf(nk + p.eps_l2);
    }

    // 5. decay, then S^T k and S^T q over the 128 rows of this lane's columns
    f4 pa = {0.0f, 0.0f, 0.0f, 0.0f}, pb = pa;
#pragma unroll
    for (int i = 0; i < kDecRows; ++i) {
        const int r = pad_row(key_row(i));
        s[i] *= gq[r];
        pa += s[i] * yk[r];
        pb += s[i] * yq[r];
    }
    if constexpr (PAIRS) {
        // the two rows of each pair (lanes l and l ^ 32), then the four
        // wavefronts in order, so every lane of a column gets the same bits
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pa[j] = rows_half_add(pa[j]);
            pb[j] = rows_half_add(pb[j]);
        }
        if (half == 0) {
            *reinterpret_cast<f4 *>(&red_k[wv][col]) = pa;
            *reinterpret_cast<f4 *>(&red_q[wv][col]) = pb;
        }
        __syncthreads();
        pa = *reinterpret_cast<const f4 *>(&red_k[0][col]);
        pb = *reinterpret_cast<const f4 *>(&red_q[0][col]);
#pragma unroll
        for (int w = 1; w < kDecThreads / kWave; ++w) {
            pa += *reinterpret_cast<const f4 *>(&red_k[w][col]);
            pb += *reinterpret_cast<const f4 *>(&red_q[w][col]);
        }
    } else {
        // sums over the eight lanes with the same l % 8 (l, l ^ 8, l ^ 16, ...)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pa[j] = rows_half_add(rows_pair_add(dpp_add<kRowRor8>(pa[j])));
            pb[j] = rows_half_add(rows_pair_add(dpp_add<kRowRor8>(pb[j])));
        }
    }

    // 6. u = beta (v - S^T k), state update S += k u^T written back in place,
    //    o = S^T q + (k . q) u
    const f4 v4 = *reinterpret_cast<const f4 *>(&yv[col]);
    const f4 u = beta * (v4 - pa * sk);
#pragma unroll
    for (int i = 0; i < kDecRows; ++i) {
        const float ki = yk[pad_row(key_row(i))] * sk;
        __builtin_nontemporal_store(s[i] + ki * u, reinterpret_cast<f4 *>(&S[(long)key_row(i) * kDecD]));
    }
    const f4 o = pb * sq + (dqk * sq * sk) * u;

    // 7. gated RMSNorm of o over the 128 value columns: PAIRS, lanes 0..31 of
    //    every wavefront hold all of them and wavefront 0 writes the output;
    //    else lanes 0..7 of each wavefront hold its 32, and each writes those
    float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
    ss = dpp_add<kHalfMirror>(dpp_add<kQuadXor2>(dpp_add<kQuadXor1>(ss)));  // over 8 lanes
    float ms;
    if constexpr (PAIRS) {
        if (wv != 0 || half != 0) return;
        ms = rows_pair_add(dpp_add<kRowMirror>(ss)) / kDecD;  // lanes 0..31
    } else {
        if (l == 0) red_k[0][wv] = ss;
        __syncthreads();
        if (l >= 8) return;
        ms = (red_k[0][0] + red_k[0][1] + red_k[0][2] + red_k[0][3]) / kDecD;
    }
    {
        const float rn = 1.0f / __builtin_sqrtf(ms + p.eps_norm);
        const f4 z4 = *reinterpret_cast<const f4 *>(&zs[col]);
        const f4 w4 = *reinterpret_cast<const f4 *>(&nws[col]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float gate = 1.0f / (1.0f + __expf(-z4[j]));
            st_elem<EO>(out, col + j, o[j] * rn * w4[j] * gate);
        }
    }
}

// The state split by row pairs up to one (sequence, head) pair per compute
// unit. (At two per CU the two splits measured level: 14.5-15.2 µs either
// way, by box.) KDA_TRIL_DECODE_LAYOUT (read on every call) = "pairs" or
// "cols" forces one split for every launch (the tests reach both on small
// problems).
constexpr long kDecPairsPerCu = 1;

hipError_t launch_decode(const DecodeProblem &p, int in_dt, int out_dt, hipStream_t stream) {
    const char *e = getenv("KDA_TRIL_DECODE_LAYOUT");
    const bool pairs = e && strcmp(e, "pairs") == 0   ? true
                       : e && strcmp(e, "cols") == 0 ? false
                                                     : (long)p.B * p.H <= kDecPairsPerCu * device_cus();
    return dispatch_dtypes<F32, BF16, F16>(in_dt, out_dt, [&]<class EI, class EO>() {
        if (pairs)
            hipLaunchKernelGGL((kda_decode_step_kernel<EI, EO, true>), dim3((unsigned)(p.B * p.H)),
                               dim3(kDecThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((kda_decode_step_kernel<EI, EO, false>), dim3((unsigned)(p.B * p.H)),
                               dim3(kDecThreads), 0, stream, p);
        return hipGetLastError();
    });
}

}  // namespace kda
