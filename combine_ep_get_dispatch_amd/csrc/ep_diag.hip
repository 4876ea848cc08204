// Diagnostic kernels: element-wise runs of the conversions the path uses, so
// they can be checked value by value, and a plain streaming copy used as the
// reference kernel for HBM traffic counters and the copy ceiling.
#include "ep_internal.h"
#include "ep_device.h"

namespace ep {
namespace {

// Four values per thread, so the hardware path converts exactly as the
// dispatch kernel does (packed pairs into one dword).
__global__ void convert_e4m3_kernel(const float* __restrict__ in, uint8_t* __restrict__ out,
                                    int64_t n, int mode) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= n) return;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (i + j < n) ? in[i + j] : 0.0f;
    const uint32_t w = mode == 0 ? e4m3x4_hw(v[0], v[1], v[2], v[3])
                                 : e4m3x4_sw(v[0], v[1], v[2], v[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (i + j < n) out[i + j] = (uint8_t)(w >> (8 * j));
}

__global__ void convert_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out,
                                    int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 2;
    if (i >= n) return;
    const float a = in[i];
    const float b = (i + 1 < n) ? in[i + 1] : 0.0f;
    const uint32_t w = pack_bf16x2(a, b);
    out[i] = (uint16_t)w;
    if (i + 1 < n) out[i + 1] = (uint16_t)(w >> 16);
}

// Grid-stride copy of 16-byte vectors.  With 65536 workgroups of 256 threads
// (16.7M threads, a few vectors each) it measured the highest copy rate among
// the grid sizes and unroll depths tried on MI355X.
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, int64_t nvec) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride)
        dst[i] = src[i];
}

}  // namespace

hipError_t launch_convert_e4m3(const float* in, uint8_t* out, int64_t n, int mode,
                               hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int64_t threads = (n + 3) / 4;
    hipLaunchKernelGGL(convert_e4m3_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, s, in, out, n, mode);
    return hipGetLastError();
}

hipError_t launch_convert_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int64_t threads = (n + 1) / 2;
    hipLaunchKernelGGL(convert_bf16_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, s, in, out, n);
    return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
    const int64_t nvec = (int64_t)(bytes / 16);
    if (nvec == 0) return hipSuccess;
    int64_t blocks = (nvec + 255) / 256;
    if (blocks > 65536) blocks = 65536;          // grid-stride beyond 16.7M vectors
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), nvec);
    return hipGetLastError();
}

}  // namespace ep
