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
// routing skew: one workgroup per token, one wave per 1024-channel chunk, 16
// channels per lane -- two 16-byte loads of x per lane and, per destination,
// one 16-byte store of codes (FP8) or two of bf16, so every destination row is
// written in whole 1 KiB runs.  The K destination rows come from the layout
// workspace (lane k loads row(k); the store loop reads it back as a scalar
// with readlane).  For FP8 a 128-channel group is 8 lanes: its amax is a
// 3-step xor shuffle, 448/a_c and a_c/448 are correctly rounded fp32
// divisions, and the codes come from v_cvt_pk_fp8_f32.  The token's G scales
// are gathered in LDS and each destination's scale row goes out as one
// contiguous G*4-byte store.  x is read once (non-temporal: each byte is
// used once) and quantised once per token, not once per copy; the receive
// rows are written through L2 (device-scope stores), which measured faster
// than ordinary and than non-temporal stores here.
#include "ep_internal.h"
#include "ep_device.h"

namespace ep {
namespace {

// Scatter token t (one workgroup): quantise or copy its H channels and write
// them to the K destination rows held by lanes 0..K-1 of `drow` (-1 = none).
// s_scale is G floats of LDS (FP8 only).
template <bool FP8>
__device__ __forceinline__ void scatter_token(const uint16_t* __restrict__ x, int H, int K, int t,
                                              int drow, void* __restrict__ recv_x,
                                              float* __restrict__ recv_scales, float* s_scale,
                                              int nchunk) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    if constexpr (FP8) {
        // Lane l quantises channels [16l, 16l + 16) of the chunk: its 128-channel
        // group is lanes 8g .. 8g+7, and its 16 codes are one 16-byte store.
        for (int c = wave; c < nchunk; c += nw) {
            const int h0 = c * kDispatchChunk + lane * 16;
            const bool act = h0 < H;       // H % 128 == 0: all 16 channels or none
            const uint16_t* xs = x + (int64_t)t * H + h0;
            uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
            if (act) {
                v0 = load_nt(xs);
                v1 = load_nt(xs + 8);
            }
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
            if (act && (lane & 7) == 0) s_scale[h0 >> 7] = scale;
            for (int k = 0; k < K; ++k) {
                const int d = __builtin_amdgcn_readlane(drow, k);
                if (d < 0) continue;
                if (act) store_wt(static_cast<uint8_t*>(recv_x) + (int64_t)d * H + h0, q);
            }
        }
    } else {
        // Lane l copies channels [8l, 8l + 8) and [512 + 8l, 512 + 8l + 8) of
        // the chunk, so every load and store instruction covers 1 KiB of
        // consecutive bytes (whole cache lines).  Non-temporal stores measured
        // fastest for these rows (bf16 receive rows are twice the FP8 bytes).
        for (int c = wave; c < nchunk; c += nw) {
            const int ha = c * kDispatchChunk + lane * 8;
            const int hb = ha + kDispatchChunk / 2;
            const bool act_a = ha < H;     // H % 8 == 0: all 8 channels or none
            const bool act_b = hb < H;
            const uint16_t* xs = x + (int64_t)t * H;
            uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
            if (act_a) va = *reinterpret_cast<const uint4*>(xs + ha);
            if (act_b) vb = *reinterpret_cast<const uint4*>(xs + hb);
            for (int k = 0; k < K; ++k) {
                const int d = __builtin_amdgcn_readlane(drow, k);
                if (d < 0) continue;
                uint16_t* dst = static_cast<uint16_t*>(recv_x) + (int64_t)d * H;
                if (act_a) store_nt(dst + ha, va);
                if (act_b) store_nt(dst + hb, vb);
            }
        }
    }
    if constexpr (FP8) {
        __syncthreads();
        const int G = H >> 7;
        for (int k = wave; k < K; k += nw) {   // one wave per destination scale row
            const int d = __builtin_amdgcn_readlane(drow, k);
            if (d < 0) continue;
            for (int g = lane; g < G; g += 64) recv_scales[(int64_t)d * G + g] = s_scale[g];
        }
    }
}

template <bool FP8>
__global__ __launch_bounds__(kDispatchMaxThreads) void dispatch_kernel(
    const uint16_t* __restrict__ x, int H, int K, const WsHeader* __restrict__ hdr,
    const int* __restrict__ rows, void* __restrict__ recv_x, float* __restrict__ recv_scales,
    int32_t* __restrict__ recv_src, int32_t* __restrict__ dst_row, int nchunk, int nrows) {
    extern __shared__ float s_scale[];   // [G] scales of this token (FP8)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = blockIdx.x;

    // Destination row of slot k = lane (K <= 64).
    int drow = -1;
    if (lane < K) {
        drow = rows[(int64_t)t * K + lane];
        if (drow >= nrows) drow = -1;   // only with a workspace from another layout
    }
    if (wave == 0 && lane < K) {
        dst_row[(int64_t)t * K + lane] = drow;
        if (drow >= 0) recv_src[drow] = t;
        // rows past the last valid one belong to no token
        const int r = t * K + lane;
        if (r >= hdr->num_valid) recv_src[r] = -1;
    }
    scatter_token<FP8>(x, H, K, t, drow, recv_x, recv_scales, s_scale, nchunk);
}

// Decode dispatch into fixed-capacity receive rows, in one launch (expert e
// owns rows [e*C, (e+1)*C); a slot whose rank in its expert reaches C is
// dropped).  No row number depends on another expert's count, so nothing has
// to be summed over all experts before data moves: every workgroup reads the
// whole (small) routing tensor, builds in LDS the per-expert counts of all
// slots and of the slots of earlier tokens, takes its own rows from the
// latter, and then scatters its token exactly as dispatch_kernel does.
// Workgroup b also writes the counts of experts b, b + grid, ... and marks
// their unfilled rows with -1, so the whole result comes from this launch.
// Each workgroup reads T*K routing entries, so the cost grows as T^2*K: this
// is the small-batch path.
template <bool FP8>
__global__ __launch_bounds__(kDispatchMaxThreads) void ll_dispatch_kernel(
    const uint16_t* __restrict__ x, const int64_t* __restrict__ idx, int T, int H, int K, int E,
    int C, int32_t* __restrict__ cnt_e, void* __restrict__ recv_x,
    float* __restrict__ recv_scales, int32_t* __restrict__ recv_src,
    int32_t* __restrict__ dst_row, int64_t* __restrict__ num_invalid, int nchunk) {
    extern __shared__ int smem[];
    int* h_pre = smem;                                      // [E] slots of tokens < t
    int* h_all = smem + E;                                  // [E] all valid slots
    float* s_scale = reinterpret_cast<float*>(smem + 2 * E); // [G] (FP8)
    __shared__ int s_inv;
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = blockIdx.x;

    for (int e = tid; e < E; e += nthr) {
        h_pre[e] = 0;
        h_all[e] = 0;
    }
    if (tid == 0) s_inv = 0;
    __syncthreads();

    const int n = T * K;
    const int before = t * K;
    int inv = 0;
    for (int i = tid; i < n; i += nthr) {
        const int64_t v = idx[i];
        if (v >= 0 && v < E) {
            atomicAdd(&h_all[v], 1);
            if (i < before) atomicAdd(&h_pre[v], 1);
        } else if (v != -1) {
            ++inv;
        }
    }
    if (blockIdx.x == 0 && inv != 0) atomicAdd(&s_inv, inv);
    __syncthreads();

    // Row of slot k = lane: expert e's slots of earlier tokens, plus the
    // earlier slots of this token with the same expert.
    int drow = -1;
    if (t < T) {
        int e = -1;
        if (lane < K) {
            const int64_t v = idx[(int64_t)t * K + lane];
            if (v >= 0 && v < E) e = (int)v;
        }
        int dup = 0;
        for (int j = 0; j < K; ++j) {
            const int ej = __builtin_amdgcn_readlane(e, j);
            if (j < lane && ej == e) ++dup;
        }
        if (e >= 0) {
            const int r = h_pre[e] + dup;
            if (r < C) drow = e * C + r;
        }
        if (wave == 0 && lane < K) {
            dst_row[(int64_t)t * K + lane] = drow;
            if (drow >= 0) recv_src[drow] = t;
        }
    }

    for (int e = blockIdx.x; e < E; e += gridDim.x) {
        const int c = h_all[e];
        if (tid == 0) cnt_e[e] = c;
        for (int r = (c < C ? c : C) + tid; r < C; r += nthr) recv_src[(int64_t)e * C + r] = -1;
    }
    if (blockIdx.x == 0 && tid == 0 && num_invalid) *num_invalid = s_inv;

    if (t < T) scatter_token<FP8>(x, H, K, t, drow, recv_x, recv_scales, s_scale, nchunk);
}

}  // namespace

hipError_t launch_dispatch(const uint16_t* x, int T, int H, int K, bool fp8, void* recv_x,
                           float* recv_scales, int32_t* recv_src, int32_t* dst_row,
                           const void* ws, const WsMap& m, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const char* base = static_cast<const char*>(ws);
    const WsHeader* hdr = reinterpret_cast<const WsHeader*>(base);
    const int* rows = reinterpret_cast<const int*>(base + m.rows_off);
    const int nchunk = (H + kDispatchChunk - 1) / kDispatchChunk;
    const int nw = nchunk < kDispatchMaxThreads / 64 ? nchunk : kDispatchMaxThreads / 64;
    const size_t lds = fp8 ? sizeof(float) * (size_t)(H / 128) : 0;
    if (fp8)
        hipLaunchKernelGGL(dispatch_kernel<true>, dim3(T), dim3(64 * nw), lds, s, x, H, K, hdr,
                           rows, recv_x, recv_scales, recv_src, dst_row, nchunk, T * K);
    else
        hipLaunchKernelGGL(dispatch_kernel<false>, dim3(T), dim3(64 * nw), 0, s, x, H, K, hdr,
                           rows, recv_x, recv_scales, recv_src, dst_row, nchunk, T * K);
    return hipGetLastError();
}

size_t ll_dispatch_lds_bytes(int E, int H, bool fp8) {
    return sizeof(int) * 2 * (size_t)E + (fp8 ? sizeof(float) * (size_t)(H / 128) : 0);
}

hipError_t launch_ll_dispatch(const uint16_t* x, const int64_t* idx, int T, int H, int K, int E,
                              int C, bool fp8, int32_t* cnt_e, void* recv_x, float* recv_scales,
                              int32_t* recv_src, int32_t* dst_row, int64_t* num_invalid,
                              hipStream_t s) {
    const int nchunk = (H + kDispatchChunk - 1) / kDispatchChunk;
    int nw = nchunk < kDispatchMaxThreads / 64 ? nchunk : kDispatchMaxThreads / 64;
    if (nw < kLlMinWaves) nw = kLlMinWaves;     // more threads for the routing scan
    const size_t lds = ll_dispatch_lds_bytes(E, H, fp8);
    const unsigned grid = T > 0 ? (unsigned)T : 1u;
    if (fp8)
        hipLaunchKernelGGL(ll_dispatch_kernel<true>, dim3(grid), dim3(64 * nw), lds, s, x, idx, T,
                           H, K, E, C, cnt_e, recv_x, recv_scales, recv_src, dst_row,
                           num_invalid, nchunk);
    else
        hipLaunchKernelGGL(ll_dispatch_kernel<false>, dim3(grid), dim3(64 * nw), lds, s, x, idx,
                           T, H, K, E, C, cnt_e, recv_x, recv_scales, recv_src, dst_row,
                           num_invalid, nchunk);
    return hipGetLastError();
}

}  // namespace ep
