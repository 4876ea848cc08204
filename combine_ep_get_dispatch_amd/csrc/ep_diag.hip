// Diagnostic kernels: element-wise runs of the conversions the path uses, so
// they can be checked value by value, and a streaming copy used as the
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

// Streaming copy, the measured copy ceiling: every wave copies whole 4 KiB
// spans (each lane four 16-byte non-temporal loads in flight, then four
// non-temporal stores), waves striding over the spans; workgroup 0 copies the
// last partial span 16 bytes per thread.  Among the span sizes (1-16 KiB),
// cache policies and grid sizes tried on MI355X, 4 KiB spans with
// non-temporal loads and stores over 32768 workgroups of 256 threads copied
// fastest (6.3 TB/s of reads plus writes, against 5.4 TB/s for one 16-byte
// vector per thread and iteration).
constexpr int kCopySpan = 4096;
constexpr int kCopyThreads = 256;
constexpr int kCopyMaxBlocks = 32768;

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const char* __restrict__ src,
                                                            char* __restrict__ dst,
                                                            int64_t nspan, int64_t tail) {
    const int lane = threadIdx.x & 63;
    constexpr int wpb = kCopyThreads / 64;
    constexpr int V = kCopySpan / 1024;        // 16-byte vectors per lane per span
    const int64_t nw = (int64_t)gridDim.x * wpb;
    for (int64_t sp = (int64_t)blockIdx.x * wpb + (threadIdx.x >> 6); sp < nspan; sp += nw) {
        const int64_t off = sp * kCopySpan + lane * 16;
        uint4 v[V];
#pragma unroll
        for (int i = 0; i < V; ++i) v[i] = load_nt(src + off + i * 1024);
#pragma unroll
        for (int i = 0; i < V; ++i) store_nt(dst + off + i * 1024, v[i]);
    }
    if (blockIdx.x == 0)                       // the last partial span, tail bytes
        for (int64_t i = threadIdx.x * 16; i < tail; i += kCopyThreads * 16) {
            const int64_t off = nspan * kCopySpan + i;
            store_nt(dst + off, load_nt(src + off));
        }
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
    if (bytes == 0) return hipSuccess;
    const int64_t nspan = (int64_t)(bytes / kCopySpan);
    const int64_t tail = (int64_t)(bytes % kCopySpan);   // a multiple of 16
    int64_t blocks = (nspan + kCopyThreads / 64 - 1) / (kCopyThreads / 64);
    if (blocks > kCopyMaxBlocks) blocks = kCopyMaxBlocks;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s,
                       static_cast<const char*>(src), static_cast<char*>(dst), nspan, tail);
    return hipGetLastError();
}

}  // namespace ep
