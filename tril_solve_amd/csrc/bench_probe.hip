// Measurement helpers for the benchmark (not part of the solver's C ABI):
//   * a plain streaming copy, the known-size reference that scales the HBM
//     byte counters of rocprofv3;
//   * streaming probes of what HBM delivers on this GPU: a copy, a read-only
//     sum and a write-only fill, each with a chosen unroll (independent
//     16-byte accesses in flight per thread), cache policy and grid size, so
//     the benchmark can sweep them and report the fastest as the measured
//     ceiling next to the 8 TB/s published peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kda_probe_copy_kernel(const f4 *__restrict__ src,
                                                             f4 *__restrict__ dst, int64_t n4) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (; i < n4; i += step) dst[i] = src[i];
}

// Copies n floats (n a multiple of 4, both pointers 16-byte aligned) on
// `stream`. Returns 0, or -1 on bad arguments, -4 on a launch failure.
extern "C" int kda_probe_copy_f32(const float *src, float *dst, int64_t n, hipStream_t stream) {
    if (n < 0 || (n & 3) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return -1;
    if (n == 0) return 0;
    const int64_t n4 = n / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(kda_probe_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const f4 *>(src), reinterpret_cast<f4 *>(dst), n4);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// ------------------------------------------------------------------ sweeps

// Cache policy of the probes' accesses: 0 the default, 1 nontemporal loads
// and stores, 2 nontemporal stores only.
template <int POL>
__device__ __forceinline__ f4 ld(const f4 *p) {
    if constexpr (POL == 1) return __builtin_nontemporal_load(p);
    return *p;
}
template <int POL>
__device__ __forceinline__ void st(f4 *p, f4 v) {
    if constexpr (POL == 1 || POL == 2)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

constexpr int kProbeThreads = 256;

// Grid-stride passes of U accesses per thread, the U accesses of a pass
// `stride` apart (so each instruction still covers 4 KiB of adjacent lines
// per workgroup); a tail pass handles what does not fill U.
template <int U, int POL>
__global__ __launch_bounds__(kProbeThreads) void kda_probe_copy_u(const f4 *__restrict__ src,
                                                                  f4 *__restrict__ dst,
                                                                  int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    for (; i + (U - 1) * stride < n4; i += U * stride) {
        f4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld<POL>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) st<POL>(dst + i + u * stride, v[u]);
    }
    for (; i < n4; i += stride) st<POL>(dst + i, ld<POL>(src + i));
}

// Sum of all elements a thread reads, written to out[thread] (out holds
// gridDim.x * kProbeThreads floats), so the loads cannot be dropped.
template <int U, int POL>
__global__ __launch_bounds__(kProbeThreads) void kda_probe_read_u(const f4 *__restrict__ src,
                                                                  float *__restrict__ out,
                                                                  int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    const int64_t t = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    int64_t i = t;
    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (; i + (U - 1) * stride < n4; i += U * stride) {
        f4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld<POL>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc += v[u];
    }
    for (; i < n4; i += stride) acc += ld<POL>(src + i);
    out[t] = acc[0] + acc[1] + acc[2] + acc[3];
}

template <int U, int POL>
__global__ __launch_bounds__(kProbeThreads) void kda_probe_fill_u(f4 *__restrict__ dst,
                                                                  int64_t n4, float value) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    const f4 v = {value, value, value, value};
    for (; i + (U - 1) * stride < n4; i += U * stride) {
#pragma unroll
        for (int u = 0; u < U; ++u) st<POL>(dst + i + u * stride, v);
    }
    for (; i < n4; i += stride) st<POL>(dst + i, v);
}

template <int U, int POL>
static hipError_t run_probe(int kind, const float *src, float *dst, int64_t n4, int64_t blocks,
                            hipStream_t stream) {
    const dim3 g((unsigned)blocks), b(kProbeThreads);
    const f4 *s = reinterpret_cast<const f4 *>(src);
    f4 *d = reinterpret_cast<f4 *>(dst);
    switch (kind) {
        case 0: hipLaunchKernelGGL((kda_probe_copy_u<U, POL>), g, b, 0, stream, s, d, n4); break;
        case 1: hipLaunchKernelGGL((kda_probe_read_u<U, POL>), g, b, 0, stream, s, dst, n4); break;
        case 2:
            hipLaunchKernelGGL((kda_probe_fill_u<U, POL>), g, b, 0, stream, d, n4, 1.0f);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int POL>
static hipError_t run_unroll(int unroll, int kind, const float *src, float *dst, int64_t n4,
                             int64_t blocks, hipStream_t stream) {
    switch (unroll) {
        case 1: return run_probe<1, POL>(kind, src, dst, n4, blocks, stream);
        case 2: return run_probe<2, POL>(kind, src, dst, n4, blocks, stream);
        case 4: return run_probe<4, POL>(kind, src, dst, n4, blocks, stream);
        case 8: return run_probe<8, POL>(kind, src, dst, n4, blocks, stream);
    }
    return hipErrorInvalidValue;
}

// One streaming probe over n floats (a multiple of 4; 16-byte aligned
// pointers):
//   kind 0 copy src -> dst (dst holds n floats),
//   kind 1 read src, one float per thread to dst (dst_n >= blocks * 256),
//   kind 2 fill dst (n floats; src unused).
// unroll 1, 2, 4 or 8; policy 0 default, 1 nontemporal, 2 nontemporal stores;
// blocks of 256 threads, 1 .. 2^20. Returns 0, -1 on bad arguments, -4 on a
// launch failure.
extern "C" int kda_probe_stream(int kind, int unroll, int policy, const float *src, float *dst,
                                int64_t n, int64_t dst_n, int64_t blocks, hipStream_t stream) {
    if (n <= 0 || (n & 3) || blocks < 1 || blocks > (1 << 20)) return -1;
    if (((uintptr_t)src & 15) || ((uintptr_t)dst & 15) || dst == nullptr) return -1;
    if (kind != 2 && src == nullptr) return -1;
    if ((kind == 0 || kind == 2) && dst_n < n) return -1;
    if (kind == 1 && dst_n < blocks * kProbeThreads) return -1;
    const int64_t n4 = n / 4;
    hipError_t e;
    switch (policy) {
        case 0: e = run_unroll<0>(unroll, kind, src, dst, n4, blocks, stream); break;
        case 1: e = run_unroll<1>(unroll, kind, src, dst, n4, blocks, stream); break;
        case 2: e = run_unroll<2>(unroll, kind, src, dst, n4, blocks, stream); break;
        default: return -1;
    }
    if (e == hipErrorInvalidValue) return -1;
    return e == hipSuccess ? 0 : -4;
}
