// Dispatch on gfx950: scatter every token's hidden vector into the receive
// rows of the experts its router picked, optionally quantised to OCP E4M3
// with one fp32 scale per 128 channels.
//
// Dispatch is the first half of the expert-parallel all-to-all ("DeepSeek
// releases DeepEP, an efficient communication library for MoE models",
// section "DeepEP: Optimizing MoE Communication"); FP8 for dispatch is in the
// feature list of "DeepSeek Open Source Weekly Review - 2", and the same
// page's comment list credits the library with doing its reads and writes as
// 64/128-bit instructions, which gfx950 has as global_load/store_dwordx4.
//
// Design.  Work is split by SOURCE token, so it is balanced whatever the
// routing skew: one wave per (token, 1024-channel chunk), 16 channels per
// lane, i.e. two 16-byte loads of x per lane and, per destination, one
// 16-byte store of codes (FP8) or two of bf16.  The K destination rows come
// from the layout workspace: lane k computes row(k) = base[e][block(t)] +
// rank(t,k) with ordinary vector loads, and the store loop reads it back as a
// scalar with readlane.  For FP8 a 128-channel group is 8 lanes; its amax is
// a 3-step xor shuffle, then 448/a_c and a_c/448 are correctly rounded fp32
// divisions and the codes come from v_cvt_pk_fp8_f32.  x is read once and the
// quantisation is done once per token, not once per copy.
#include "ep_internal.h"
#include "ep_device.h"

namespace ep {
namespace {

template <bool FP8>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(
    const uint16_t* __restrict__ x, int H, const int64_t* __restrict__ idx, int K, int E,
    int TB, int nb, const WsHeader* __restrict__ hdr, const int* __restrict__ base,
    const int* __restrict__ rank, void* __restrict__ recv_x, float* __restrict__ recv_scales,
    int32_t* __restrict__ recv_src, int32_t* __restrict__ dst_row, int nchunk, int64_t ntask,
    int nrows) {
    const int lane = threadIdx.x & 63;
    const int64_t task = (int64_t)blockIdx.x * (kDispatchThreads / 64) +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (task >= ntask) return;
    const int t = (int)(task / nchunk);
    const int c = (int)(task - (int64_t)t * nchunk);
    const int h0 = c * kDispatchChunk + lane * 16;
    const bool act0 = h0 < H;          // channels h0 .. h0+7
    const bool act1 = h0 + 8 < H;      // channels h0+8 .. h0+15

    // Destination row of slot k = lane (K <= 64).
    int drow = -1;
    if (lane < K) {
        const int64_t e = idx[(int64_t)t * K + lane];
        if (e >= 0 && e < E)
            drow = base[e * nb + t / TB] + rank[(int64_t)t * K + lane];
        if (drow >= nrows) drow = -1;   // only with a workspace from another layout
    }
    if (c == 0) {
        if (lane < K) {
            dst_row[(int64_t)t * K + lane] = drow;
            if (drow >= 0) recv_src[drow] = t;
            // rows past the last valid one belong to no token
            const int r = t * K + lane;
            if (r >= hdr->num_valid) recv_src[r] = -1;
        }
    }

    const uint16_t* xs = x + (int64_t)t * H + h0;
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
    if (act0) v0 = *reinterpret_cast<const uint4*>(xs);
    if (act1) v1 = *reinterpret_cast<const uint4*>(xs + 8);

    if constexpr (FP8) {
        const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        float f[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            f[2 * i] = bf16_lo(w[i]);
            f[2 * i + 1] = bf16_hi(w[i]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
        amax = group8_max(amax);
        const float ac = fmaxf(amax, 1e-4f);
        const float inv = 448.0f / ac;
        const float scale = ac / 448.0f;
        uint4 q;
        q.x = e4m3x4_hw(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
        q.y = e4m3x4_hw(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
        q.z = e4m3x4_hw(f[8] * inv, f[9] * inv, f[10] * inv, f[11] * inv);
        q.w = e4m3x4_hw(f[12] * inv, f[13] * inv, f[14] * inv, f[15] * inv);
        const int G = H >> 7;
        for (int k = 0; k < K; ++k) {
            const int d = __builtin_amdgcn_readlane(drow, k);
            if (d < 0) continue;
            if (act0) {
                uint8_t* dst = static_cast<uint8_t*>(recv_x) + (int64_t)d * H + h0;
                *reinterpret_cast<uint4*>(dst) = q;
                if ((lane & 7) == 0) recv_scales[(int64_t)d * G + (h0 >> 7)] = scale;
            }
        }
    } else {
        for (int k = 0; k < K; ++k) {
            const int d = __builtin_amdgcn_readlane(drow, k);
            if (d < 0) continue;
            uint16_t* dst = static_cast<uint16_t*>(recv_x) + (int64_t)d * H + h0;
            if (act0) *reinterpret_cast<uint4*>(dst) = v0;
            if (act1) *reinterpret_cast<uint4*>(dst + 8) = v1;
        }
    }
}

}  // namespace

hipError_t launch_dispatch(const uint16_t* x, int T, int H, const int64_t* idx, int K, int E,
                           bool fp8, void* recv_x, float* recv_scales, int32_t* recv_src,
                           int32_t* dst_row, const void* ws, const WsMap& m, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const char* base = static_cast<const char*>(ws);
    const WsHeader* hdr = reinterpret_cast<const WsHeader*>(base);
    const int* cntb = reinterpret_cast<const int*>(base + m.cnt_off);
    const int* rank = reinterpret_cast<const int*>(base + m.rank_off);
    const int nchunk = (H + kDispatchChunk - 1) / kDispatchChunk;
    const int64_t ntask = (int64_t)T * nchunk;
    const int waves_per_block = kDispatchThreads / 64;
    const int64_t blocks = (ntask + waves_per_block - 1) / waves_per_block;
    if (fp8)
        hipLaunchKernelGGL(dispatch_kernel<true>, dim3((unsigned)blocks), dim3(kDispatchThreads),
                           0, s, x, H, idx, K, E, m.tb, m.nb, hdr, cntb, rank, recv_x,
                           recv_scales, recv_src, dst_row, nchunk, ntask, T * K);
    else
        hipLaunchKernelGGL(dispatch_kernel<false>, dim3((unsigned)blocks), dim3(kDispatchThreads),
                           0, s, x, H, idx, K, E, m.tb, m.nb, hdr, cntb, rank, recv_x,
                           recv_scales, recv_src, dst_row, nchunk, ntask, T * K);
    return hipGetLastError();
}

}  // namespace ep
