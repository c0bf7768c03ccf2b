// Measurement helper for the benchmark (not part of the solver's C ABI): a
// plain streaming copy, used as the measured copy roofline and as the
// known-size reference that scales the HBM byte counters of rocprofv3.
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
