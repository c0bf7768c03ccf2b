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
// paged pools indexed by a per-sequence slot (negative: padding entry).
//
// One workgroup of 256 threads per (sequence, head). The state dominates the
// traffic (64 KiB read and 64 KiB written per step), so its loads are issued
// right after the convolution's few inputs, and the convolution and norms run
// while they are in flight. Thread
// (c, r), c = t % 32, r = t / 32, holds columns 4c..4c+3 of rows 16r..16r+15
// in registers for the whole step: one pass gives both reductions S^T k and
// S^T q of the decayed state (partial sums over its 16 rows, combined over
// the 8 row groups through LDS), then the update is applied to the same
// registers and written back. Since S_new^T q = (decayed S)^T q + (k . q) u,
// the state is read and written exactly once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tril_device.h"
#include "tril_launch.h"

namespace kda {

constexpr int kDecD = 128;         // head dim (keys = values)
constexpr int kDecThreads = 256;
constexpr int kDecRows = 16;       // state rows per thread
constexpr int kDecGroups = 8;      // row groups (16 rows each)

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

// Sum over the 64 lanes of a wavefront (result in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// One step for one (sequence, head); layouts as in the C ABI.
template <class EI, class EO>
__global__ __launch_bounds__(kDecThreads) void kda_decode_step_kernel(DecodeProblem p) {
    __shared__ float yq[kDecD], yk[kDecD], yv[kDecD], gq[kDecD];
    __shared__ float part[2][kDecGroups][kDecD];
    __shared__ float red[4][4];
    __shared__ float uo[2][kDecD];

    const int t = threadIdx.x;
    const int b = blockIdx.x / p.H, h = blockIdx.x - b * p.H;
    const int slot = p.slot[b];
    typename EO::T *out = static_cast<typename EO::T *>(p.out) + ((long)b * p.H + h) * kDecD;
    if (slot < 0 || slot >= p.num_slots) {  // padding (or a slot outside the pool)
        if (t < kDecD) st_elem<EO>(out, t, 0.0f);
        return;
    }

    // 1. the small inputs of the convolution first: the memory counter waits
    //    in issue order, so loads issued after the state tile could only be
    //    used once the whole tile had arrived. Threads 0..127 handle the q
    //    and k channels, threads 128..255 the v channels; conv widths 2..4.
    //    The loads are unconditional (indices past the width or the thread's
    //    projections are clamped to valid ones and their values unused), so
    //    they form one block the state loads can follow with no wait between.
    const int c = t & (kDecD - 1);
    const int W = p.W;
    // wavefront-uniform (waves 0-1 vs 2-3)
    const bool low = __builtin_amdgcn_readfirstlane(t) < kDecD;
    const int pfirst = low ? 0 : 2, pn = low ? 2 : 1;
    const typename EI::T *qkv = static_cast<const typename EI::T *>(p.qkv);
    float xin[2], win[2][3], tap[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int p3 = k < pn ? pfirst + k : pfirst;
        xin[k] = ld_elem<EI>(qkv, (((long)b * 3 + p3) * p.H + h) * kDecD + c);
        const float *ws = p.conv_state + (((long)slot * 3 + p3) * p.H + h) * (long)(W - 1) * kDecD;
        const float *cw = p.conv_w + ((long)p3 * W * p.H + h) * kDecD + c;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (w < 3) win[k][w] = ws[(long)(w < W - 1 ? w : 0) * kDecD + c];
            tap[k][w] = cw[(long)(w < W ? w : 0) * p.H * kDecD];
        }
    }
    const float graw = p.g[((long)b * p.H + h) * kDecD + c];

    // 2. then the state tile of this thread
    const int c4 = (t & 31) * 4, r0 = (t >> 5) * kDecRows;
    float *S = p.state + ((long)slot * p.H + h) * kDecD * kDecD;
    f4 s[kDecRows];
#pragma unroll
    for (int r = 0; r < kDecRows; ++r)
        s[r] = *reinterpret_cast<const f4 *>(&S[(long)(r0 + r) * kDecD + c4]);
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
            if (p3 == 0) yq[c] = y;
            if (p3 == 1) yk[c] = y;
            if (p3 == 2) yv[c] = y;
        }
    }
    if (low) gq[c] = __expf(graw);
    __syncthreads();

    // 4. squared norms of y_q, y_k and their dot product (waves 0 and 1)
    if (t < kDecD) {
        const float a = yq[t], bk = yk[t];
        const float s0 = wave_sum(a * a), s1 = wave_sum(bk * bk), s2 = wave_sum(a * bk);
        if ((t & (kWave - 1)) == 0) {
            red[t / kWave][0] = s0;
            red[t / kWave][1] = s1;
            red[t / kWave][2] = s2;
        }
    }
    __syncthreads();
    const float nq = red[0][0] + red[1][0], nk = red[0][1] + red[1][1];
    const float dqk = red[0][2] + red[1][2];
    const float sq = 1.0f / (__builtin_sqrtf(nq + p.eps_l2) * __builtin_sqrtf((float)kDecD));
    const float sk = 1.0f / __builtin_sqrtf(nk + p.eps_l2);

    // 5. decay, then partial S^T k and S^T q over this thread's 16 rows
    f4 pa = {0.0f, 0.0f, 0.0f, 0.0f}, pb = pa;
#pragma unroll
    for (int r = 0; r < kDecRows; ++r) {
        const int i = r0 + r;
        s[r] *= gq[i];
        const float ki = yk[i] * sk, qi = yq[i] * sq;
        pa += s[r] * ki;
        pb += s[r] * qi;
    }
    *reinterpret_cast<f4 *>(&part[0][t >> 5][c4]) = pa;
    *reinterpret_cast<f4 *>(&part[1][t >> 5][c4]) = pb;
    __syncthreads();

    // 6. u = beta (v - S^T k) and o = S^T q + (k . q) u per value column
    if (t < kDecD) {
        float a = 0.0f, bq = 0.0f;
#pragma unroll
        for (int r = 0; r < kDecGroups; ++r) {
            a += part[0][r][t];
            bq += part[1][r][t];
        }
        const float u = p.beta[(long)b * p.H + h] * (yv[t] - a);
        uo[0][t] = u;
        uo[1][t] = bq + dqk * sq * sk * u;
    }
    __syncthreads();

    // 7. state update S += k u^T, written back in place
    {
        const f4 u4 = *reinterpret_cast<const f4 *>(&uo[0][c4]);
#pragma unroll
        for (int r = 0; r < kDecRows; ++r) {
            const float ki = yk[r0 + r] * sk;
            *reinterpret_cast<f4 *>(&S[(long)(r0 + r) * kDecD + c4]) = s[r] + ki * u4;
        }
    }

    // 8. gated RMSNorm of o
    if (t < kDecD) {
        const float o = uo[1][t];
        const float ss = wave_sum(o * o);
        if ((t & (kWave - 1)) == 0) red[t / kWave][3] = ss;
    }
    __syncthreads();
    if (t < kDecD) {
        const float ms = (red[0][3] + red[1][3]) / kDecD;
        const float rn = 1.0f / __builtin_sqrtf(ms + p.eps_norm);
        const typename EI::T *z = static_cast<const typename EI::T *>(p.z);
        const float zz = ld_elem<EI>(z, ((long)b * p.H + h) * kDecD + t);
        const float gate = 1.0f / (1.0f + __expf(-zz));
        st_elem<EO>(out, t, uo[1][t] * rn * p.norm_w[t] * gate);
    }
}

hipError_t launch_decode(const DecodeProblem &p, int in_dt, int out_dt, hipStream_t stream) {
    return dispatch_dtypes<F32, BF16, F16>(in_dt, out_dt, [&]<class EI, class EO>() {
        auto kernel = kda_decode_step_kernel<EI, EO>;
        hipLaunchKernelGGL(kernel, dim3((unsigned)(p.B * p.H)), dim3(kDecThreads), 0, stream, p);
        return hipGetLastError();
    });
}

}  // namespace kda
