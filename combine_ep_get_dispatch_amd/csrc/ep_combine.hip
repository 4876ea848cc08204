// Combine on gfx950: gather each token's expert outputs back from the
// receive rows and reduce them with the token's gate weights,
//   out[t,h] = bf16_rne( fma chain over k of w[t,k] * y[dst_row[t,k], h] ),
// accumulated in fp32 from +0 in slot order, masked slots (dst_row < 0)
// skipped.
//
// Combine is the second half of the expert-parallel all-to-all ("DeepSeek
// releases DeepEP, an efficient communication library for MoE models",
// section "DeepEP: Optimizing MoE Communication"); the weighting and the
// accumulation order are this library's reading.
//
// Design.  The kernel is HBM-bound (about 1 flop per byte), so the goal is to
// keep enough independent 16-byte loads in flight: one wave per (token,
// 512-channel chunk), 8 channels per lane; lane k first fetches dst_row and
// the weight of slot k, then every slot's 16-byte row segment is loaded
// before the first FMA (K loads in flight per lane), and the result is
// rounded with v_cvt_pk_bf16_f32 and written as one 16-byte store.  y and
// out are streamed with the non-temporal hint (each byte is touched once), so
// they do not displace the receive buffers that dispatch has just written.  The slot
// count is a template parameter for the common top-k values so the loads
// unroll; other K take a loop over groups of 8 slots.
//
// Large top-8 batches take a tiled form: a workgroup of 16 waves owns a tile
// of consecutive tokens, computes the tile's chunks as above into LDS and
// then writes the tile's outputs, which are contiguous in `out`, as one
// burst (112 KiB at 7168 channels) instead of interleaving 1 KiB result
// stores with the gathers.  At 4096 tokens x 7168 channels the step with
// dispatch took 139.8 against 143.9 us at top-8, but 114.6 / 115.0 at top-6,
// 90.4 / 87.0 at top-4, 62.9 / 61.6 at top-2 and 52.0 / 51.8 at top-1: with
// fewer slots the burst is a larger share of a tile's traffic, and the CU
// waits for it before its next tile starts.
#include "ep_internal.h"
#include "ep_device.h"

namespace ep {
namespace {

__device__ __forceinline__ void fma8(float (&acc)[8], float w, const uint4& v) {
    acc[0] = __builtin_fmaf(w, bf16_lo(v.x), acc[0]);
    acc[1] = __builtin_fmaf(w, bf16_hi(v.x), acc[1]);
    acc[2] = __builtin_fmaf(w, bf16_lo(v.y), acc[2]);
    acc[3] = __builtin_fmaf(w, bf16_hi(v.y), acc[3]);
    acc[4] = __builtin_fmaf(w, bf16_lo(v.z), acc[4]);
    acc[5] = __builtin_fmaf(w, bf16_hi(v.z), acc[5]);
    acc[6] = __builtin_fmaf(w, bf16_lo(v.w), acc[6]);
    acc[7] = __builtin_fmaf(w, bf16_hi(v.w), acc[7]);
}

// Slots [k0, k0 + KN) of the token: load all, then accumulate in order.
template <int KN>
__device__ __forceinline__ void combine_slots(float (&acc)[8], const uint16_t* __restrict__ y,
                                              int H, int h0, bool act, int drow, float wl,
                                              int k0, int kend) {
    uint4 v[KN];
#pragma unroll
    for (int i = 0; i < KN; ++i) {
        const int d = __builtin_amdgcn_readlane(drow, k0 + i);
        v[i] = make_uint4(0, 0, 0, 0);
        if (k0 + i < kend && d >= 0 && act)
            v[i] = load_nt(y + (int64_t)d * H + h0);
    }
#pragma unroll
    for (int i = 0; i < KN; ++i) {
        const int d = __builtin_amdgcn_readlane(drow, k0 + i);
        const float w = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), k0 + i));
        if (k0 + i < kend && d >= 0) fma8(acc, w, v[i]);
    }
}

// One wave's task: token t = task / nchunk, channel chunk task % nchunk.
template <int KT>   // KT > 0: exactly KT slots; KT == 0: any K <= 64
__device__ __forceinline__ void combine_task(const uint16_t* __restrict__ y, int64_t nrows,
                                             const int32_t* __restrict__ dst_row,
                                             const float* __restrict__ w, int K, int H,
                                             uint16_t* __restrict__ out, int nchunk,
                                             int64_t task) {
    const int lane = threadIdx.x & 63;
    const int t = (int)(task / nchunk);
    const int c = (int)(task - (int64_t)t * nchunk);
    const int h0 = c * kCombineChunk + lane * 8;
    const bool act = h0 < H;

    const int kk = KT > 0 ? KT : K;
    int drow = -1;
    float wl = 0.0f;
    if (lane < kk) {
        drow = dst_row[(int64_t)t * kk + lane];
        wl = w[(int64_t)t * kk + lane];
        if (drow >= nrows) drow = -1;   // outside y: skipped like a masked slot
    }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    if constexpr (KT > 0) {
        combine_slots<KT>(acc, y, H, h0, act, drow, wl, 0, KT);
    } else {
        for (int k0 = 0; k0 < K; k0 += 8) combine_slots<8>(acc, y, H, h0, act, drow, wl, k0, K);
    }
    if (act) {
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        store_nt(out + (int64_t)t * H + h0, o);
    }
}

template <int KT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const uint16_t* __restrict__ y, int64_t nrows, const int32_t* __restrict__ dst_row,
    const float* __restrict__ w, int K, int H, uint16_t* __restrict__ out, int nchunk,
    int64_t ntask) {
    const int64_t task = (int64_t)blockIdx.x * (kCombineThreads / 64) +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (task >= ntask) return;
    combine_task<KT>(y, nrows, dst_row, w, K, H, out, nchunk, task);
}

// Tiled form: workgroup b owns tokens [b*tile, b*tile + nt).  Lane j < nt*KT
// holds slot j % KT of the tile's token j / KT.  The waves take the tile's
// (token, chunk) tasks wave, wave + waves, ..., each with its KT row loads in
// flight before the FMAs as in the untiled form, and put each rounded 16-byte
// result at its place in the tile's LDS copy of `out`; after the barrier
// every thread stores 16-byte pieces i, i + blockDim, ... of the tile.
template <int KT>
__global__ __launch_bounds__(kCombineTileThreads) void combine_tile_kernel(
    const uint16_t* __restrict__ y, int64_t nrows, const int32_t* __restrict__ dst_row,
    const float* __restrict__ w, int T, int H, uint16_t* __restrict__ out, int nchunk,
    int tile) {
    extern __shared__ EP_LDS_ALIGN uint4 s_out[];   // [nt * H / 8]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int t0 = blockIdx.x * tile;
    const int nt = min(tile, T - t0);
    int drow = -1;
    float wl = 0.0f;
    if (lane < nt * KT) {
        drow = dst_row[(int64_t)t0 * KT + lane];
        wl = w[(int64_t)t0 * KT + lane];
        if (drow >= nrows) drow = -1;   // outside y: skipped like a masked slot
    }
    const int ntask = nt * nchunk;
    for (int task = wave; task < ntask; task += nw) {
        const int tt = task / nchunk;
        const int h0 = (task - tt * nchunk) * kCombineChunk + lane * 8;
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        combine_slots<KT>(acc, y, H, h0, h0 < H, drow, wl, tt * KT, tt * KT + KT);
        if (h0 < H) {
            uint4 o;
            o.x = pack_bf16x2(acc[0], acc[1]);
            o.y = pack_bf16x2(acc[2], acc[3]);
            o.z = pack_bf16x2(acc[4], acc[5]);
            o.w = pack_bf16x2(acc[6], acc[7]);
            s_out[(tt * H + h0) >> 3] = o;          // H % 8 == 0
        }
    }
    __syncthreads();
    uint4* o = reinterpret_cast<uint4*>(out + (int64_t)t0 * H);
    const int n16 = nt * (H >> 3);
    for (int i = threadIdx.x; i < n16; i += blockDim.x) store_nt(o + i, s_out[i]);
}

// CU-budget form: a grid of at most num_cus workgroups of kBudgetThreads,
// every wave striding over the tasks, so the hardware places the work on at
// most num_cus CUs and leaves the others to concurrent kernels.
template <int KT>
__global__ __launch_bounds__(kBudgetThreads) void combine_budget_kernel(
    const uint16_t* __restrict__ y, int64_t nrows, const int32_t* __restrict__ dst_row,
    const float* __restrict__ w, int K, int H, uint16_t* __restrict__ out, int nchunk,
    int64_t ntask) {
    const int wpb = kBudgetThreads / 64;
    for (int64_t task = (int64_t)blockIdx.x * wpb + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
         task < ntask; task += (int64_t)gridDim.x * wpb)
        combine_task<KT>(y, nrows, dst_row, w, K, H, out, nchunk, task);
}

template <int KT>
hipError_t launch_k(dim3 grid, bool budget, hipStream_t s, const uint16_t* y, int64_t nrows,
                    const int32_t* dst_row, const float* w, int K, int H, uint16_t* out,
                    int nchunk, int64_t ntask, int T, int tile) {
    if constexpr (KT == kCombineTileK) {
        if (tile > 0) {
            const size_t lds = sizeof(uint4) * (size_t)tile * (size_t)(H / 8);
            if (lds > 64 * 1024) {
                hipError_t e = allow_large_lds(
                    reinterpret_cast<const void*>(combine_tile_kernel<KT>), kCombineTileLdsSlot,
                    (int)kCombineTileLds);
                if (e != hipSuccess) return e;
            }
            hipLaunchKernelGGL(combine_tile_kernel<KT>, dim3((unsigned)((T + tile - 1) / tile)),
                               dim3(kCombineTileThreads), lds, s, y, nrows, dst_row, w, T, H, out,
                               nchunk, tile);
            return hipGetLastError();
        }
    }
    if (budget)
        hipLaunchKernelGGL(combine_budget_kernel<KT>, grid, dim3(kBudgetThreads), 0, s, y, nrows,
                           dst_row, w, K, H, out, nchunk, ntask);
    else
        hipLaunchKernelGGL(combine_kernel<KT>, grid, dim3(kCombineThreads), 0, s, y, nrows,
                           dst_row, w, K, H, out, nchunk, ntask);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const uint16_t* y, int64_t nrows, const int32_t* dst_row,
                          const float* w, int T, int K, int H, uint16_t* out, int num_cus,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int nchunk = (H + kCombineChunk - 1) / kCombineChunk;
    const int64_t ntask = (int64_t)T * nchunk;
    int64_t nblk = (ntask + kCombineThreads / 64 - 1) / (kCombineThreads / 64);
    bool budget = false;
    if (num_cus > 0) {
        const int64_t bblk = (ntask + kBudgetThreads / 64 - 1) / (kBudgetThreads / 64);
        budget = true;
        nblk = bblk < num_cus ? bblk : num_cus;
    }
    const dim3 grid((unsigned)nblk);
    // Top-8 in tiles of as many tokens as the LDS budget allows, while the
    // batch still gives every CU two tiles; else one wave per task.
    int tile = 0;
    if (!budget && K == kCombineTileK) {
        tile = (int)(kCombineTileLds / ((size_t)H * sizeof(uint16_t)));
        if (tile > 64 / K) tile = 64 / K;
        if (tile > T / kCombineTileMinBlocks) tile = T / kCombineTileMinBlocks;
        if (tile < 2) tile = 0;
    }
#define EP_C_ARGS grid, budget, s, y, nrows, dst_row, w, K, H, out, nchunk, ntask, T, tile
    switch (K) {
        case 1: return launch_k<1>(EP_C_ARGS);
        case 2: return launch_k<2>(EP_C_ARGS);
        case 4: return launch_k<4>(EP_C_ARGS);
        case 6: return launch_k<6>(EP_C_ARGS);
        case 8: return launch_k<8>(EP_C_ARGS);
        default: return launch_k<0>(EP_C_ARGS);
    }
#undef EP_C_ARGS
}

}  // namespace ep
