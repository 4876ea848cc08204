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
// routing skew: one workgroup per token and one wave per chunk of the row --
// FP8: 1024 channels, 16 per lane, two 16-byte loads of x per lane and one
// 16-byte store of codes per destination; bf16: 512 channels, 8 per lane, one
// 16-byte load and one 16-byte store per destination -- so every destination
// row is written in whole 1 KiB runs.  The K destination rows come from the layout
// workspace (lane k loads row(k); the store loop reads it back as a scalar
// with readlane).  For FP8 a 128-channel group is 8 lanes: its amax is a
// 3-step xor shuffle, 448/a_c and a_c/448 are correctly rounded fp32
// divisions, and the codes come from v_cvt_pk_fp8_f32.  The token's G scales
// are gathered in LDS and each destination's scale row goes out as one
// contiguous G*4-byte store.  x is read once (FP8: non-temporal, each byte
// is used once) and quantised once per token, not once per copy; receive rows
// are written through L2 (device-scope stores).  The bf16 chunk is half the
// FP8 one so that a token's copy runs on twice as many waves: its rows are
// twice as wide, and with 1024-channel chunks the bf16 scatter of 8192 tokens
// x 7168 channels, top-8, measured 4% slower.
//
// Kernels: dispatch_kernel (rows from the two-launch layout), the
// layout-finishing layout_dispatch_kernel (one call: each workgroup sums its
// token's rows over the count launch's per-block tables), dedup_dispatch_kernel
// (one copy per token and partition) and ll_dispatch_kernel (fixed capacity
// per expert, one launch); the first two also have a CU-budget form whose
// workgroups loop over the tokens.
#include "ep_internal.h"
#include "ep_device.h"

namespace ep {
namespace {

// Partition of expert e: (e * ceil(2^32 / Ep)) >> 32, exact for E <= 1024.
__device__ __forceinline__ int partition_of_expert(int e, uint64_t pmagic) {
    return (int)(((uint64_t)(uint32_t)e * pmagic) >> 32);
}

// One lane's share of one chunk of a token, ready to store.  FP8 (1024-channel
// chunks): lane l holds the 16 codes of channels [16l, 16l + 16) of the chunk
// in .a (its 128-channel group is lanes 8g .. 8g+7; the group's scale goes to
// s_scale and, as bits, to .b.x).  bf16 (512-channel chunks): lane l holds
// channels [8l, 8l + 8) in .a, so every load and store instruction covers
// 1 KiB of consecutive bytes.
struct ChunkData {
    uint4 a, b;
};

// The chunk's raw bf16 words as loaded (FP8: 16 channels per lane; bf16:
// 8 channels per lane), kept apart from the conversion so that a kernel
// can issue the loads early and convert once it has waited for them.  The
// loads are branch-free: a lane past the end of the row loads the row's last
// 16 bytes instead (always in bounds), and everything downstream ignores it
// (finish_chunk and store_chunk test h < H), so the compiler can wait for
// other loads without waiting for these.
template <bool FP8>
__device__ __forceinline__ ChunkData load_raw(const uint16_t* __restrict__ x, int H, int t,
                                              int c) {
    const int lane = threadIdx.x & 63;
    const uint16_t* xs = x + (int64_t)t * H;
    ChunkData d;
    if constexpr (FP8) {
        const int h0 = c * kDispatchChunk + lane * 16;
        const int hc = h0 < H ? h0 : H - 16;   // H % 128 == 0
        d.a = load_nt(xs + hc);                // each byte of x is used once
        d.b = load_nt(xs + hc + 8);
    } else {
        const int h0 = c * kDispatchChunkBf16 + lane * 8;
        d.a = *reinterpret_cast<const uint4*>(xs + (h0 < H ? h0 : H - 8));   // H % 8 == 0
        d.b = make_uint4(0, 0, 0, 0);
    }
    return d;
}

// Largest of the 2N bf16 magnitudes (sign bit cleared) packed in w, as bits:
// for non-negative values integer order is numeric order, and NaNs (above
// 0x7F80 = +inf) come out above every number.  With nan_out, NaNs count as 0.
template <int N>
__device__ __forceinline__ uint32_t max_bf16_magnitude(const uint32_t (&w)[N], bool nan_out) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
        if (nan_out) {
            lo = lo > 0x7F80u ? 0u : lo;
            hi = hi > 0x7F80u ? 0u : hi;
        }
        m = max(m, max(lo, hi));
    }
    return m;
}

// The E4M3 codes of the 2N bf16 values packed in w, each multiplied by inv
// first (byte j of q[i] = value 4i + j).  Unless the group is finite, every
// infinite or NaN x gets the NaN code S.1111.111 with the sign of x, whatever
// sign the hardware gives the NaN of x * inv.
template <int N>
__device__ __forceinline__ void e4m3_codes(const uint32_t (&w)[N], float inv, bool finite,
                                           uint32_t (&q)[N / 2]) {
    float f[2 * N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
    }
#pragma unroll
    for (int i = 0; i < N / 2; ++i)
        q[i] = e4m3x4_hw(f[4 * i] * inv, f[4 * i + 1] * inv, f[4 * i + 2] * inv,
                         f[4 * i + 3] * inv);
    if (!finite) {
#pragma unroll
        for (int i = 0; i < 2 * N; ++i) {
            const uint32_t b = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
            if ((b & 0x7F80u) == 0x7F80u) {             // infinite or NaN x
                const uint32_t code = ((b >> 8) & 0x80u) | 0x7Fu;
                const int sh = 8 * (i & 3);
                q[i >> 2] = (q[i >> 2] & ~(0xFFu << sh)) | (code << sh);
            }
        }
    }
}

// Raw words -> what store_chunk writes: the E4M3 codes in .a (and the group
// scale in s_scale) for FP8; unchanged for bf16.  A group that holds an
// infinity or a NaN (rare; found from the integer maximum of its magnitudes)
// takes a slower path: its maximum leaves the NaNs out (an infinity makes the
// scale +inf and the inverse 0, so its finite values become signed zeros),
// and its infinite or NaN values get the NaN code (e4m3_codes).
template <bool FP8>
__device__ __forceinline__ ChunkData finish_chunk(const ChunkData& raw, int H, int c,
                                                  float* s_scale) {
    if constexpr (!FP8) {
        return raw;
    } else {
        const int lane = threadIdx.x & 63;
        const int h0 = c * kDispatchChunk + lane * 16;
        const uint32_t w[8] = {raw.a.x, raw.a.y, raw.a.z, raw.a.w,
                               raw.b.x, raw.b.y, raw.b.z, raw.b.w};
        // the group's largest |x| as bf16 bits (exact); the 8 lanes of a
        // group agree on `finite`, so the branches split whole groups
        uint32_t mbits = group8_max_u32(max_bf16_magnitude(w, false));
        const bool finite = mbits < 0x7F80u;
        if (!finite) mbits = group8_max_u32(max_bf16_magnitude(w, true));
        const float ac = fmaxf(__uint_as_float(mbits << 16), 1e-4f);
        const float inv = 448.0f / ac;
        const float scale = ac / 448.0f;
        uint32_t q[4];
        e4m3_codes(w, inv, finite, q);
        ChunkData d;
        d.a = make_uint4(q[0], q[1], q[2], q[3]);
        d.b = make_uint4(__float_as_uint(scale), 0, 0, 0);
        if (h0 < H && (lane & 7) == 0) s_scale[h0 >> 7] = scale;
        return d;
    }
}

// The decode dispatch's FP8 chunk is 512 channels (kLlChunk): lane l holds
// channels [8l, 8l + 8) (one 16-byte load, the bf16 chunk's), its 128-channel
// group is the 16 lanes of its DPP row, and its 8 codes go out as one 8-byte
// store per destination.  Half the 1024-channel chunk's quantiser work per
// wave, so a small batch spreads it over twice as many waves.
struct HalfChunk {
    uint2 q;        // the 8 codes
    float scale;    // the group's scale
};

__device__ __forceinline__ HalfChunk quantise_half(const uint4& raw) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t mbits = group16_max_u32(max_bf16_magnitude(w, false));
    const bool finite = mbits < 0x7F80u;
    if (!finite) mbits = group16_max_u32(max_bf16_magnitude(w, true));
    const float ac = fmaxf(__uint_as_float(mbits << 16), 1e-4f);
    uint32_t q[2];
    e4m3_codes(w, 448.0f / ac, finite, q);
    HalfChunk d;
    d.q = make_uint2(q[0], q[1]);
    d.scale = ac / 448.0f;
    return d;
}

// Store a 512-channel FP8 chunk of codes and its 4 group scales to the K
// destination rows held by lanes 0..K-1 of `drow` (-1 = none).
__device__ __forceinline__ void store_half_chunk(const HalfChunk& d, int H, int K, int c,
                                                 int drow, void* __restrict__ recv_x,
                                                 float* __restrict__ recv_scales) {
    const int lane = threadIdx.x & 63;
    const int h0 = c * kLlChunk + lane * 8;
    const bool act = h0 < H;
    const bool lead = act && (lane & 15) == 0;
    const int G = H >> 7;
    for (int k = 0; k < K; ++k) {
        const int r = __builtin_amdgcn_readlane(drow, k);
        if (r < 0) continue;
        if (act) store_wt8(static_cast<uint8_t*>(recv_x) + (int64_t)r * H + h0, d.q);
        if (lead) recv_scales[(int64_t)r * G + (h0 >> 7)] = d.scale;
    }
}

template <bool FP8>
__device__ __forceinline__ ChunkData load_chunk(const uint16_t* __restrict__ x, int H, int t,
                                                int c, float* s_scale) {
    return finish_chunk<FP8>(load_raw<FP8>(x, H, t, c), H, c, s_scale);
}

// Store one chunk to the K destination rows held by lanes 0..K-1 of `drow`
// (-1 = none).  Rows of both formats are written through L2 (device-scope
// stores), which measured fastest for each in a steady loop of steps whose
// tokens are not left in a cache by earlier ones (non-temporal bf16 stores
// look faster only while the tokens stay cached).
template <bool FP8>
__device__ __forceinline__ void store_chunk(const ChunkData& d, int H, int K, int c, int drow,
                                            void* __restrict__ recv_x) {
    const int lane = threadIdx.x & 63;
    if constexpr (FP8) {
        const int h0 = c * kDispatchChunk + lane * 16;
        const bool act = h0 < H;
        for (int k = 0; k < K; ++k) {
            const int r = __builtin_amdgcn_readlane(drow, k);
            if (r < 0) continue;
            if (act) store_wt(static_cast<uint8_t*>(recv_x) + (int64_t)r * H + h0, d.a);
        }
    } else {
        const int h0 = c * kDispatchChunkBf16 + lane * 8;
        const bool act = h0 < H;
        for (int k = 0; k < K; ++k) {
            const int r = __builtin_amdgcn_readlane(drow, k);
            if (r < 0) continue;
            if (act) store_wt(static_cast<uint16_t*>(recv_x) + (int64_t)r * H + h0, d.a);
        }
    }
}

// Scatter token t with a group of nw waves (the whole workgroup, or one of
// several groups of a workgroup that carries several tokens at once; wave =
// the wave's index inside its group): wave w handles chunks w, w+nw, ...;
// `first` is chunk `wave`, already loaded (when wave < nchunk).  FP8: the
// token's G scales are gathered in s_scale (LDS) and each destination's scale
// row then goes out as one contiguous store.  `active` is false for a group
// without a token, which still takes part in the barrier.
template <bool FP8>
__device__ __forceinline__ void scatter_token_group(const uint16_t* __restrict__ x, int H, int K,
                                                    int t, int drow, const ChunkData& first,
                                                    void* __restrict__ recv_x,
                                                    float* __restrict__ recv_scales,
                                                    float* s_scale, int nchunk, bool active,
                                                    int wave, int nw) {
    const int lane = threadIdx.x & 63;
    if (active) {
        if (wave < nchunk) store_chunk<FP8>(first, H, K, wave, drow, recv_x);
        for (int c = wave + nw; c < nchunk; c += nw)
            store_chunk<FP8>(load_chunk<FP8>(x, H, t, c, s_scale), H, K, c, drow, recv_x);
    }
    if constexpr (FP8) {
        __syncthreads();
        if (active) {
            const int G = H >> 7;
            for (int k = wave; k < K; k += nw) {   // one wave per destination scale row
                const int r = __builtin_amdgcn_readlane(drow, k);
                if (r < 0) continue;
                for (int g = lane; g < G; g += 64) recv_scales[(int64_t)r * G + g] = s_scale[g];
            }
        }
    }
}

// scatter_token_group for a whole workgroup.
template <bool FP8>
__device__ __forceinline__ void scatter_token(const uint16_t* __restrict__ x, int H, int K, int t,
                                              int drow, const ChunkData& first,
                                              void* __restrict__ recv_x,
                                              float* __restrict__ recv_scales, float* s_scale,
                                              int nchunk) {
    scatter_token_group<FP8>(x, H, K, t, drow, first, recv_x, recv_scales, s_scale, nchunk, true,
                             __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), blockDim.x >> 6);
}

template <bool FP8>
__device__ __forceinline__ void dispatch_token(
    int t, const uint16_t* __restrict__ x, int H, int K, const WsHeader* __restrict__ hdr,
    const int* __restrict__ rows, void* __restrict__ recv_x, float* __restrict__ recv_scales,
    int32_t* __restrict__ recv_src, int32_t* __restrict__ dst_row, int nchunk, int nrows,
    float* s_scale) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // Destination row of slot k = lane (K <= 64).  (Loading x before these
    // rows are known measured slower, here and in the decode kernel.)
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
    ChunkData first;
    if (wave < nchunk) first = load_chunk<FP8>(x, H, t, wave, s_scale);
    scatter_token<FP8>(x, H, K, t, drow, first, recv_x, recv_scales, s_scale, nchunk);
}

// One workgroup per token, or (LOOP, the CU-budget form) a smaller grid whose
// workgroups take tokens blockIdx.x, blockIdx.x + gridDim.x, ...
template <bool FP8, bool LOOP>
__global__ __launch_bounds__(kDispatchMaxThreads) void dispatch_kernel(
    const uint16_t* __restrict__ x, int T, int H, int K, const WsHeader* __restrict__ hdr,
    const int* __restrict__ rows, void* __restrict__ recv_x, float* __restrict__ recv_scales,
    int32_t* __restrict__ recv_src, int32_t* __restrict__ dst_row, int nchunk, int nrows) {
    extern __shared__ EP_LDS_ALIGN float s_scale[];   // [G] scales of this token (FP8)
    if constexpr (!LOOP) {
        dispatch_token<FP8>(blockIdx.x, x, H, K, hdr, rows, recv_x, recv_scales, recv_src,
                            dst_row, nchunk, nrows, s_scale);
    } else {
        for (int t = blockIdx.x; t < T; t += gridDim.x) {
            dispatch_token<FP8>(t, x, H, K, hdr, rows, recv_x, recv_scales, recv_src, dst_row,
                                nchunk, nrows, s_scale);
            __syncthreads();               // the next token reuses the LDS
        }
    }
}

// Dispatch that also finishes the layout (after the count launch in kCountPre mode).
// Slot (t,k) of expert e, in token block b, with rank r inside the block:
//   row = expert_offsets[e] + (rows of e in blocks < b) + r
//       = sum over blocks j of pre[j][e] + sum over j < b of cnt[j][e] + r,
// and N = sum over j of pre[j][E].  Thread i = k * S + j (S = blocks rounded
// up to a power of two) loads slot k's packed row and then block j's term
// for it (k = K: block j's term of N): one round of L2 loads after the row
// load, spread over (K+1)*S threads.  A sum over each S-lane segment
// (segment_sum: DPP moves inside a 16-lane row) gives the row, which reaches
// the other waves through LDS (one barrier).  The workgroup handling token 0 also writes the counts, offsets
// and header.  s_scale ([G]), s_row ([64]) and s_n are the workgroup's LDS.
template <bool FP8>
__device__ __forceinline__ void layout_dispatch_token(
    int t, const uint16_t* __restrict__ x, int H, int K, int E, int P, int Ep, int TB, int nb,
    int seg_log2, const int* __restrict__ cnt, const int* __restrict__ pre,
    const int* __restrict__ pcnt, const int* __restrict__ inv, const int* __restrict__ rows,
    WsHeader* __restrict__ hdr, int32_t* __restrict__ cnt_e, int32_t* __restrict__ cnt_p,
    int32_t* __restrict__ off_e, int32_t* __restrict__ off_p, void* __restrict__ recv_x,
    float* __restrict__ recv_scales, int32_t* __restrict__ recv_src,
    int32_t* __restrict__ dst_row, int nchunk, int nrows, float* s_scale, int* s_row,
    int& s_n, bool active, int tid, int gsize) {
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = gsize >> 6;

    {
        const int b = t / TB;
        const int S = 1 << seg_log2;     // segment lanes, S >= nb, S <= 64
        const int k = tid >> seg_log2;
        const int j = tid & (S - 1);
        int pk = -1, v = 0;
        if (!active) {
        } else if (k < K) {
            pk = rows[(int64_t)t * K + k];
            if (pk >= 0 && j < nb) {
                const int e = pk >> kRankBits;
                v = pre[(int64_t)j * (E + 1) + e];
                if (j < b) v += cnt[(int64_t)j * E + e];
            }
        } else if (k == K && j < nb) {
            v = pre[(int64_t)j * (E + 1) + E];
        }
        v = segment_sum(v, S);
        if (active && j == 0) {
            if (k < K) {
                int r = pk >= 0 ? v + (pk & ((1 << kRankBits) - 1)) : -1;
                if (r >= nrows) r = -1;    // only with a workspace from another layout
                s_row[k] = r;
            } else if (k == K) {
                s_n = v;
            }
        }
    }
    __syncthreads();
    const int drow = (active && lane < K) ? s_row[lane] : -1;
    if (active && wave == 0 && lane < K) {
        dst_row[(int64_t)t * K + lane] = drow;
        if (drow >= 0) recv_src[drow] = t;
        const int r = t * K + lane;        // rows past the last valid one belong to no token
        if (r >= s_n) recv_src[r] = -1;
    }
    if (active && t == 0 && tid == 0) hdr->num_valid = s_n;

    if (active && t == 0) {                // the layout's own outputs
        for (int e = tid; e <= E; e += gsize) {
            int c = 0, o = 0;
            for (int j = 0; j < nb; ++j) {
                o += pre[(int64_t)j * (E + 1) + e];
                if (e < E) c += cnt[(int64_t)j * E + e];
            }
            off_e[e] = o;
            if (e < E) cnt_e[e] = c;
            if (e % Ep == 0) off_p[e / Ep] = o;     // e = P*Ep = E gives off_p[P] = N
        }
        for (int p = tid; p < P; p += gsize) {
            int c = 0;
            for (int j = 0; j < nb; ++j) c += pcnt[(int64_t)j * P + p];
            cnt_p[p] = c;
        }
        if (tid == 0) {
            int64_t nerr = 0;
            for (int j = 0; j < nb; ++j) nerr += inv[j];
            hdr->num_invalid = nerr;
        }
    }

    ChunkData first;
    if (active && wave < nchunk) first = load_chunk<FP8>(x, H, t, wave, s_scale);
    scatter_token_group<FP8>(x, H, K, t, drow, first, recv_x, recv_scales, s_scale, nchunk,
                             active, wave, nw);
}

// One workgroup per token, or (LOOP, the CU-budget form) a smaller grid whose
// workgroups take tokens blockIdx.x, blockIdx.x + gridDim.x, ...
template <bool FP8, bool LOOP>
__global__ __launch_bounds__(kDispatchMaxThreads) void layout_dispatch_kernel(
    const uint16_t* __restrict__ x, int T, int H, int K, int E, int P, int Ep, int TB, int nb,
    int seg_log2, const int* __restrict__ cnt, const int* __restrict__ pre,
    const int* __restrict__ pcnt, const int* __restrict__ inv, const int* __restrict__ rows,
    WsHeader* __restrict__ hdr, int32_t* __restrict__ cnt_e, int32_t* __restrict__ cnt_p,
    int32_t* __restrict__ off_e, int32_t* __restrict__ off_p, void* __restrict__ recv_x,
    float* __restrict__ recv_scales, int32_t* __restrict__ recv_src,
    int32_t* __restrict__ dst_row, int nchunk, int nrows, int gsize_loop) {
    extern __shared__ EP_LDS_ALIGN float s_scale[];   // [groups][G] scales of the group's token (FP8)
    __shared__ int s_row[kBudgetGroups][64];   // receive row of slot k (K <= 64)
    __shared__ int s_n[kBudgetGroups];         // N
    if constexpr (!LOOP) {
        layout_dispatch_token<FP8>(blockIdx.x, x, H, K, E, P, Ep, TB, nb, seg_log2, cnt, pre,
                                   pcnt, inv, rows, hdr, cnt_e, cnt_p, off_e, off_p, recv_x,
                                   recv_scales, recv_src, dst_row, nchunk, nrows, s_scale,
                                   s_row[0], s_n[0], true, threadIdx.x, blockDim.x);
    } else {
        // groups of gsize threads, one token each, in lockstep through the
        // barriers; the workgroup's groups take tokens base + g
        const int groups = blockDim.x / gsize_loop;
        const int g = threadIdx.x / gsize_loop;
        const int G = H >> 7;
        for (int base = blockIdx.x * groups; base < T; base += gridDim.x * groups) {
            const int t = base + g;
            layout_dispatch_token<FP8>(t < T ? t : T - 1, x, H, K, E, P, Ep, TB, nb, seg_log2, cnt,
                                       pre, pcnt, inv, rows, hdr, cnt_e, cnt_p, off_e, off_p,
                                       recv_x, recv_scales, recv_src, dst_row, nchunk, nrows,
                                       s_scale + (FP8 ? g * G : 0), s_row[g], s_n[g], t < T,
                                       threadIdx.x - g * gsize_loop, gsize_loop);
            __syncthreads();               // the next tokens reuse the LDS
        }
    }
}

// De-duplicated per-partition dispatch (after the count launch in kCountDedup
// mode): one copy of the token per partition it reaches, at partition p's
// row  sum over blocks j of ppre[j][p] + sum over j < b of pcnt[j][p] + (the
// token's rank among its block's member tokens of p), and the expert-major
// row of every slot as in layout_dispatch_kernel (only as an index: the
// data goes to the de-duplicated rows).  Thread i = g * S + j sums block j's
// terms (and every S-th block's after it) for slot g (g < K: its expert row
// and its partition row) or for the totals (g = K: N and the number of
// de-duplicated rows); sums over S-lane segments (segment_sum) close the
// sums.  A slot stores the token's data only if it is the first of
// the token's slots in its partition.  Workgroup 0 writes the counts, offsets
// and header.
template <bool FP8>
__global__ __launch_bounds__(kDispatchMaxThreads) void dedup_dispatch_kernel(
    const uint16_t* __restrict__ x, int H, int K, int E, int P, int Ep, uint64_t pmagic, int TB,
    int nb, int seg_log2, int Kp, const int* __restrict__ cnt, const int* __restrict__ pre,
    const int* __restrict__ pcnt, const int* __restrict__ ppre, const int* __restrict__ inv,
    const int* __restrict__ rows, const int* __restrict__ prank, WsHeader* __restrict__ hdr,
    int32_t* __restrict__ cnt_e, int32_t* __restrict__ cnt_p, int32_t* __restrict__ off_e,
    int32_t* __restrict__ off_p, int32_t* __restrict__ ptok_off, void* __restrict__ recv_x,
    float* __restrict__ recv_scales, int32_t* __restrict__ recv_src,
    int32_t* __restrict__ recv_topk_idx, int32_t* __restrict__ slot_src,
    int32_t* __restrict__ dst_row, int nchunk, int nrows, int ndrows) {
    extern __shared__ EP_LDS_ALIGN float s_scale[];   // [G] scales of this token (FP8)
    __shared__ int s_pk[64];             // packed slot k (K <= 64)
    __shared__ int s_erow[64];           // expert-major row of slot k
    __shared__ int s_drow[64];           // de-duplicated row of slot k's partition
    __shared__ int s_n, s_nd;            // N and the number of de-duplicated rows
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = blockIdx.x;

    {
        const int b = t / TB;
        const int S = 1 << seg_log2;
        const int g = tid >> seg_log2;       // slot g (g < K), or the totals (g == K)
        const int j0 = tid & (S - 1);
        int ve = 0, vp = 0, pk = -1, pr = -1;
        if (g < K) {
            pk = rows[(int64_t)t * K + g];
            if (pk >= 0) {
                const int e = pk >> kRankBits;
                const int p = partition_of_expert(e, pmagic);
                pr = prank[(int64_t)t * K + g];
                for (int j = j0; j < nb; j += S) {
                    ve += pre[(int64_t)j * (E + 1) + e];
                    vp += ppre[(int64_t)j * (P + 1) + p];
                    if (j < b) {
                        ve += cnt[(int64_t)j * E + e];
                        vp += pcnt[(int64_t)j * P + p];
                    }
                }
            }
        } else if (g == K) {
            for (int j = j0; j < nb; j += S) {
                ve += pre[(int64_t)j * (E + 1) + E];
                vp += ppre[(int64_t)j * (P + 1) + P];
            }
        }
        ve = segment_sum(ve, S);
        vp = segment_sum(vp, S);
        if (j0 == 0) {
            if (g < K) {
                int r = pk >= 0 ? ve + (pk & ((1 << kRankBits) - 1)) : -1;
                if (r >= nrows) r = -1;    // only with a workspace from another layout
                s_erow[g] = r;
                s_pk[g] = pk;
                int d = (pk >= 0 && pr >= 0) ? vp + pr : -1;
                if (d >= ndrows) d = -1;
                s_drow[g] = d;
            } else if (g == K) {
                s_n = ve;
                s_nd = vp;
            }
        }
    }
    __syncthreads();
    // The token's first chunk is requested before the slots' partitions are
    // sorted out (their readlane loop would otherwise delay it): 53.1 -> 51.5
    // us at 4096 x 7168, top-8 of 256.  (In the other dispatch kernels, whose
    // index stores or marks come before the data, the same order measured
    // slower.)
    ChunkData raw_chunk;
    if (wave < nchunk) raw_chunk = load_raw<FP8>(x, H, t, wave);
    const int N = s_n;
    const int ND = s_nd;
    const int pk = lane < K ? s_pk[lane] : -1;
    const int e = pk >= 0 ? pk >> kRankBits : -1;
    const int part = e >= 0 ? partition_of_expert(e, pmagic) : -1;
    const int erow = lane < K ? s_erow[lane] : -1;
    const int drow = lane < K ? s_drow[lane] : -1;
    bool first = part >= 0;
    for (int j = 0; j < K; ++j) {
        const int pj = __builtin_amdgcn_readlane(part, j);
        if (j < lane && pj == part) first = false;
    }
    const int store_row = first ? drow : -1;

    if (t == 0) {                          // the layout's own outputs
        for (int ee = tid; ee <= E; ee += blockDim.x) {
            int c = 0, o = 0;
            for (int j = 0; j < nb; ++j) {
                o += pre[(int64_t)j * (E + 1) + ee];
                if (ee < E) c += cnt[(int64_t)j * E + ee];
            }
            off_e[ee] = o;
            if (ee < E) cnt_e[ee] = c;
            if (ee % Ep == 0) off_p[ee / Ep] = o;
        }
        for (int p = tid; p <= P; p += blockDim.x) {
            int c = 0, o = 0;
            for (int j = 0; j < nb; ++j) {
                o += ppre[(int64_t)j * (P + 1) + p];
                if (p < P) c += pcnt[(int64_t)j * P + p];
            }
            ptok_off[p] = o;
            if (p < P) cnt_p[p] = c;
        }
        if (tid == 0) {
            int64_t nerr = 0;
            for (int j = 0; j < nb; ++j) nerr += inv[j];
            hdr->num_valid = N;
            hdr->num_invalid = nerr;
        }
    }

    ChunkData first_chunk;
    if (wave < nchunk) first_chunk = finish_chunk<FP8>(raw_chunk, H, wave, s_scale);
    scatter_token<FP8>(x, H, K, t, store_row, first_chunk, recv_x, recv_scales, s_scale, nchunk);

    // The token's index outputs go after its data: issued first, they delay
    // wave 0's loads (the launch took 56.4 instead of 52.8 us at 4096 x 7168,
    // top-8 of 256 experts).
    if (wave == 0) {
        if (lane < K) {
            dst_row[(int64_t)t * K + lane] = erow;
            if (erow >= 0) slot_src[erow] = drow;
            const int r = t * K + lane;    // expert rows past N belong to no slot
            if (r >= N) slot_src[r] = -1;
            if (store_row >= 0) recv_src[store_row] = t;
        }
        // Local expert ids of the token's rows, one (row owner k, column c)
        // pair per lane: the row of slot k (if it owns one) holds at column c
        // slot c's expert minus the partition's first expert when slot c is
        // in slot k's partition, else -1.
        for (int l0 = 0; l0 < K * K; l0 += 64) {
            const int l = l0 + lane;
            const int k = l < K * K ? l / K : 0;
            const int c = l - k * K;
            const int rk = __shfl(store_row, k);
            const int k_part = __shfl(part, k);
            const int c_part = __shfl(part, c < K ? c : 0);
            const int ec = __shfl(e, c < K ? c : 0);
            if (l < K * K && rk >= 0)
                recv_topk_idx[(int64_t)rk * K + c] = (c_part == k_part) ? ec - k_part * Ep : -1;
        }
    }
    // Rows past the last de-duplicated one among [t*Kp, (t+1)*Kp) are unused.
    for (int i = tid; i < Kp * (K + 1); i += blockDim.x) {
        const int q = i / (K + 1);
        const int c = i - q * (K + 1);
        const int64_t r = (int64_t)t * Kp + q;
        if (r < ND) continue;
        if (c == K) recv_src[r] = -1;
        else recv_topk_idx[r * K + c] = -1;
    }
}

// T = 0 for the de-duplicated dispatch: every partition token offset is 0.
__global__ void dedup_empty_kernel(int P, int32_t* __restrict__ ptok_off) {
    for (int i = threadIdx.x; i <= P; i += blockDim.x) ptok_off[i] = 0;
}

// Decode dispatch into fixed-capacity receive rows, in one launch (expert e
// owns rows [e*C, (e+1)*C); a slot whose rank in its expert reaches C is
// dropped).  No row number depends on another expert's count, so nothing has
// to be summed over all experts before data moves: every workgroup reads the
// whole (small) routing tensor, builds in LDS the per-expert counts of all
// slots and of the slots of earlier tokens, takes its token's rows from the
// latter, and then scatters its share of the token in 512-channel chunks
// (bf16: dispatch_kernel's chunk; FP8: the half-size chunk of quantise_half,
// whose group maximum spans a DPP row).  A token's row is split over `split`
// workgroups (workgroup b takes token b / split and the b % split-th
// contiguous range of its channel chunks, with the matching scale groups):
// with fewer tokens than CUs this spreads the stores over more CUs, whose
// individual store rate is what bounds a small batch.  Workgroup b also
// writes the counts of experts b, b + grid, ... and marks their unfilled rows
// with -1, so the whole result comes from this launch.  Each workgroup reads
// T*K routing entries, so the cost grows as T^2*K*split: this is the
// small-batch path.
template <bool FP8>
__global__ __launch_bounds__(kDispatchMaxThreads) void ll_dispatch_kernel(
    const uint16_t* __restrict__ x, const int64_t* __restrict__ idx, int T, int H, int K, int E,
    int C, int32_t* __restrict__ cnt_e, void* __restrict__ recv_x,
    float* __restrict__ recv_scales, int32_t* __restrict__ recv_src,
    int32_t* __restrict__ dst_row, int64_t* __restrict__ num_invalid, int nchunk, int split,
    int cps) {
    extern __shared__ EP_LDS_ALIGN int smem[];
    int* h_pre = smem;                                      // [E] slots of tokens < t
    int* h_all = smem + E;                                  // [E] all valid slots
    __shared__ int s_inv;
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = blockIdx.x / split;
    const int part = blockIdx.x - t * split;   // this workgroup's share of the token
    const int c0 = part * cps;                 // its chunks [c0, c1)
    const int c1 = min(c0 + cps, nchunk);

    // This token's own ids (lane k holds slot k) and the first round of the
    // routing scan are loaded together (T >= 1 here and t < T; branch-free,
    // clamped in-bounds loads whose extra lanes are discarded).  The token's
    // row is loaded only once its destinations are known: loading it first
    // measured slower.
    int64_t own = idx[(int64_t)t * K + (lane < K ? lane : K - 1)];
    if (lane >= K) own = -1;
    const int n = T * K;
    const int before = t * K;
    int64_t v[kLlScanUnroll];
#pragma unroll
    for (int j = 0; j < kLlScanUnroll; ++j) {
        const int i = tid + j * nthr;
        v[j] = idx[i < n ? i : n - 1];
        if (i >= n) v[j] = -1;
    }
    // The wave's first chunk of the token is requested right after the
    // routing loads, so that its latency overlaps the scan (branch-free,
    // in-bounds loads).  (Issued after the histograms, the loads left the
    // kernel 1.5 us longer at 128 tokens x 7168, top-8 of 256 experts.)
    const int cfirst = c0 + wave;
    ChunkData raw;
    if (cfirst < c1) raw = load_raw<false>(x, H, t, cfirst);   // 512 channels, either dtype

    for (int e = tid; e < E; e += nthr) {
        h_pre[e] = 0;
        h_all[e] = 0;
    }
    if (tid == 0) s_inv = 0;
    __syncthreads();

    // The first round (all of it up to kLlScanUnroll * blockDim slots) is
    // straight-line code; larger inputs loop for the rest.
    int inv = 0;
    auto count = [&](int i0) {
#pragma unroll
        for (int j = 0; j < kLlScanUnroll; ++j) {
            const int i = i0 + j * nthr;
            if (v[j] >= 0 && v[j] < E) {
                atomicAdd(&h_all[v[j]], 1);
                if (i < before) atomicAdd(&h_pre[v[j]], 1);
            } else if (v[j] != -1) {
                ++inv;
            }
        }
    };
    count(tid);
    for (int i0 = tid + kLlScanUnroll * nthr; i0 < n; i0 += kLlScanUnroll * nthr) {
#pragma unroll
        for (int j = 0; j < kLlScanUnroll; ++j) {
            const int i = i0 + j * nthr;
            v[j] = idx[i < n ? i : n - 1];
            if (i >= n) v[j] = -1;
        }
        count(i0);
    }
    if (blockIdx.x == 0 && inv != 0) atomicAdd(&s_inv, inv);
    __syncthreads();

    // Row of slot k = lane: expert e's slots of earlier tokens, plus the
    // earlier slots of this token with the same expert.
    int drow = -1;
    {
        const int e = (own >= 0 && own < E) ? (int)own : -1;
        int dup = 0;
        for (int j = 0; j < K; ++j) {
            const int ej = __builtin_amdgcn_readlane(e, j);
            if (j < lane && ej == e) ++dup;
        }
        if (e >= 0) {
            const int r = h_pre[e] + dup;
            if (r < C) drow = e * C + r;
        }
        if (part == 0 && wave == 0 && lane < K) {
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

    // This workgroup's 512-channel chunks c0 .. c1-1: wave w takes c0 + w,
    // c0 + w + nw, ...  FP8: each wave writes its own chunk's codes and 4
    // scales (no barrier and no LDS round trip, which the decode batch's
    // latency would pay for).
    const int nw = nthr >> 6;
    for (int c = cfirst; c < c1; c += nw) {
        const ChunkData r = c == cfirst ? raw : load_raw<false>(x, H, t, c);
        if constexpr (FP8)
            store_half_chunk(quantise_half(r.a), H, K, c, drow, recv_x, recv_scales);
        else
            store_chunk<false>(r, H, K, c, drow, recv_x);
    }
}

// T = 0: every count is 0, every row unfilled, nothing invalid.
__global__ void ll_empty_kernel(int E, int C, int32_t* __restrict__ cnt_e,
                                int32_t* __restrict__ recv_src,
                                int64_t* __restrict__ num_invalid) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < E) cnt_e[i] = 0;
    if (i < (int64_t)E * C) recv_src[i] = -1;
    if (i == 0 && num_invalid) *num_invalid = 0;
}

}  // namespace

hipError_t launch_dispatch(const uint16_t* x, int T, int H, int K, bool fp8, void* recv_x,
                           float* recv_scales, int32_t* recv_src, int32_t* dst_row,
                           const void* ws, const WsMap& m, int num_cus, int nrows,
                           hipStream_t s) {
    if (T == 0) return hipSuccess;
    const char* base = static_cast<const char*>(ws);
    const WsHeader* hdr = reinterpret_cast<const WsHeader*>(base);
    const int* rows = reinterpret_cast<const int*>(base + m.rows_off);
    const int nchunk = (H + dispatch_chunk(fp8) - 1) / dispatch_chunk(fp8);
    const int nw = nchunk < kDispatchMaxThreads / 64 ? nchunk : kDispatchMaxThreads / 64;
    const size_t lds = fp8 ? sizeof(float) * (size_t)(H / 128) : 0;
    const bool loop = num_cus > 0 && num_cus < T;
    const dim3 grid(loop ? (unsigned)num_cus : (unsigned)T);
#define EP_D_ARGS x, T, H, K, hdr, rows, recv_x, recv_scales, recv_src, dst_row, nchunk, nrows
    if (fp8 && loop)
        hipLaunchKernelGGL((dispatch_kernel<true, true>), grid, dim3(64 * nw), lds, s, EP_D_ARGS);
    else if (fp8)
        hipLaunchKernelGGL((dispatch_kernel<true, false>), grid, dim3(64 * nw), lds, s, EP_D_ARGS);
    else if (loop)
        hipLaunchKernelGGL((dispatch_kernel<false, true>), grid, dim3(64 * nw), 0, s, EP_D_ARGS);
    else
        hipLaunchKernelGGL((dispatch_kernel<false, false>), grid, dim3(64 * nw), 0, s, EP_D_ARGS);
#undef EP_D_ARGS
    return hipGetLastError();
}

size_t ll_dispatch_lds_bytes(int E) { return sizeof(int) * 2 * (size_t)E; }

hipError_t launch_ll_dispatch(const uint16_t* x, const int64_t* idx, int T, int H, int K, int E,
                              int C, bool fp8, int32_t* cnt_e, void* recv_x, float* recv_scales,
                              int32_t* recv_src, int32_t* dst_row, int64_t* num_invalid,
                              hipStream_t s) {
    const int nchunk = (H + kLlChunk - 1) / kLlChunk;
    const int nw = kLlWaves;
    static_assert(kLlWaves * 64 <= kDispatchMaxThreads, "block too large");
    const size_t lds = ll_dispatch_lds_bytes(E);
    if (T == 0) {
        const int64_t rows = (int64_t)E * C > E ? (int64_t)E * C : E;
        hipLaunchKernelGGL(ll_empty_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s,
                           E, C, cnt_e, recv_src, num_invalid);
        return hipGetLastError();
    }
    // Workgroups per token: enough to put every CU to work when the batch is
    // small, each with at least one chunk (cps chunks each, the last fewer).
    int split = kLlTargetWorkgroups / T;
    if (split > nchunk) split = nchunk;
    if (split < 1) split = 1;
    const int cps = (nchunk + split - 1) / split;
    split = (nchunk + cps - 1) / cps;
    const unsigned grid = (unsigned)((int64_t)T * split);
    if (fp8)
        hipLaunchKernelGGL(ll_dispatch_kernel<true>, dim3(grid), dim3(64 * nw), lds, s, x, idx, T,
                           H, K, E, C, cnt_e, recv_x, recv_scales, recv_src, dst_row,
                           num_invalid, nchunk, split, cps);
    else
        hipLaunchKernelGGL(ll_dispatch_kernel<false>, dim3(grid), dim3(64 * nw), lds, s, x, idx,
                           T, H, K, E, C, cnt_e, recv_x, recv_scales, recv_src, dst_row,
                           num_invalid, nchunk, split, cps);
    return hipGetLastError();
}

hipError_t launch_layout_dispatch(const uint16_t* x, const int64_t* idx, int T, int H, int K,
                                  int E, int P, bool fp8, void* ws, const WsMap& m,
                                  int32_t* cnt_e, int32_t* cnt_p, uint8_t* in_part,
                                  int32_t* off_e, int32_t* off_p, void* recv_x,
                                  float* recv_scales, int32_t* recv_src, int32_t* dst_row,
                                  int num_cus, hipStream_t s) {
    const int nchunk = (H + dispatch_chunk(fp8) - 1) / dispatch_chunk(fp8);
    const int nw = nchunk < kDispatchMaxThreads / 64 ? nchunk : kDispatchMaxThreads / 64;
    // The finishing sums are one round of loads per token workgroup and a
    // bounded amount of work for workgroup 0; other shapes (and those with a
    // single-launch layout) take the layout and the plain dispatch.
    int seg_log2 = 0;                    // segment of 2^seg_log2 >= nb lanes per slot
    while ((1 << seg_log2) < m.nb) ++seg_log2;
    const bool fused = T > 0 && !layout_single_launch(T, K, E, P, m) && seg_log2 <= 6 &&
                       ((int64_t)(K + 1) << seg_log2) <= 64 * nw &&
                       (int64_t)(E + 1) * m.nb <= kLayoutDispatchMaxTerms;
    if (!fused) {
        hipError_t e = launch_layout(idx, T, K, E, P, ws, m, cnt_e, cnt_p, in_part, off_e, off_p,
                                     s);
        if (e != hipSuccess) return e;
        return launch_dispatch(x, T, H, K, fp8, recv_x, recv_scales, recv_src, dst_row, ws, m,
                               num_cus, T * K, s);
    }
    hipError_t e = launch_layout_count(idx, T, K, E, P, ws, m, in_part, kCountPre, s);
    if (e != hipSuccess) return e;
    char* base = static_cast<char*>(ws);
    WsHeader* hdr = reinterpret_cast<WsHeader*>(base);
    const int* cnt = reinterpret_cast<const int*>(base + m.cnt_off);
    const int* pcnt = reinterpret_cast<const int*>(base + m.pcnt_off);
    const int* inv = reinterpret_cast<const int*>(base + m.inv_off);
    const int* pre = reinterpret_cast<const int*>(base + m.pre_off);
    const int* rows = reinterpret_cast<const int*>(base + m.rows_off);
    const size_t lds = fp8 ? sizeof(float) * (size_t)(H / 128) : 0;
    // CU budget: num_cus workgroups, each carrying `groups` tokens at a time
    // (as many groups of nw waves as fit in one workgroup, up to
    // kBudgetGroups), so that a CU keeps several tokens' loads in flight.
    int groups = kDispatchMaxThreads / (64 * nw);
    if (groups > kBudgetGroups) groups = kBudgetGroups;
    const bool loop = num_cus > 0 && (int64_t)num_cus * groups < T;
    const dim3 grid(loop ? (unsigned)num_cus : (unsigned)T);
    const dim3 block(loop ? 64 * nw * groups : 64 * nw);
    const size_t lds_all = loop ? lds * groups : lds;
#define EP_LD_ARGS x, T, H, K, E, P, E / P, m.tb, m.nb, seg_log2, cnt, pre, pcnt, inv, rows, hdr, \
                   cnt_e, cnt_p, off_e, off_p, recv_x, recv_scales, recv_src, dst_row, nchunk, \
                   T * K, 64 * nw
    if (fp8 && loop)
        hipLaunchKernelGGL((layout_dispatch_kernel<true, true>), grid, block, lds_all, s,
                           EP_LD_ARGS);
    else if (fp8)
        hipLaunchKernelGGL((layout_dispatch_kernel<true, false>), grid, block, lds_all, s,
                           EP_LD_ARGS);
    else if (loop)
        hipLaunchKernelGGL((layout_dispatch_kernel<false, true>), grid, block, lds_all, s,
                           EP_LD_ARGS);
    else
        hipLaunchKernelGGL((layout_dispatch_kernel<false, false>), grid, block, lds_all, s,
                           EP_LD_ARGS);
#undef EP_LD_ARGS
    return hipGetLastError();
}

hipError_t launch_dispatch_dedup(const uint16_t* x, const int64_t* idx, int T, int H, int K,
                                 int E, int P, bool fp8, void* ws, const WsMap& m, int32_t* cnt_e,
                                 int32_t* cnt_p, uint8_t* in_part, int32_t* off_e, int32_t* off_p,
                                 int32_t* ptok_off, void* recv_x, float* recv_scales,
                                 int32_t* recv_src, int32_t* recv_topk_idx, int32_t* slot_src,
                                 int32_t* dst_row, hipStream_t s) {
    if (T == 0) {
        hipError_t e = launch_layout(idx, T, K, E, P, ws, m, cnt_e, cnt_p, in_part, off_e, off_p,
                                     s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(dedup_empty_kernel, dim3(1), dim3(256), 0, s, P, ptok_off);
        return hipGetLastError();
    }
    hipError_t e = launch_layout_count(idx, T, K, E, P, ws, m, in_part, kCountDedup, s);
    if (e != hipSuccess) return e;
    char* base = static_cast<char*>(ws);
    WsHeader* hdr = reinterpret_cast<WsHeader*>(base);
    const int* cnt = reinterpret_cast<const int*>(base + m.cnt_off);
    const int* pcnt = reinterpret_cast<const int*>(base + m.pcnt_off);
    const int* inv = reinterpret_cast<const int*>(base + m.inv_off);
    const int* pre = reinterpret_cast<const int*>(base + m.pre_off);
    const int* ppre = reinterpret_cast<const int*>(base + m.ppre_off);
    const int* prank = reinterpret_cast<const int*>(base + m.prank_off);
    const int* rows = reinterpret_cast<const int*>(base + m.rows_off);
    const int nchunk = (H + dispatch_chunk(fp8) - 1) / dispatch_chunk(fp8);
    const int nw = nchunk < kDispatchMaxThreads / 64 ? nchunk : kDispatchMaxThreads / 64;
    // Enough threads for at least one lane per term group, and segments of S
    // lanes (a power of two, <= 64, no wider than the blocks need).
    const int groups = K + 1;
    int threads = 64 * nw;
    if (threads < groups) threads = (groups + 63) / 64 * 64;
    int seg_log2 = 0;
    while ((1 << (seg_log2 + 1)) <= 64 && (groups << (seg_log2 + 1)) <= threads &&
           (1 << seg_log2) < m.nb)
        ++seg_log2;
    const int Kp = K < P ? K : P;
    const size_t lds = fp8 ? sizeof(float) * (size_t)(H / 128) : 0;
    const uint64_t pmagic = ((uint64_t)1 << 32) / (uint64_t)(E / P) +
                            ((((uint64_t)1 << 32) % (uint64_t)(E / P)) ? 1 : 0);
    if (fp8)
        hipLaunchKernelGGL(dedup_dispatch_kernel<true>, dim3(T), dim3(threads), lds, s, x, H, K,
                           E, P, E / P, pmagic, m.tb, m.nb, seg_log2, Kp, cnt, pre, pcnt, ppre,
                           inv, rows, prank, hdr, cnt_e, cnt_p, off_e, off_p, ptok_off, recv_x,
                           recv_scales, recv_src, recv_topk_idx, slot_src, dst_row, nchunk,
                           T * K, T * Kp);
    else
        hipLaunchKernelGGL(dedup_dispatch_kernel<false>, dim3(T), dim3(threads), lds, s, x, H, K,
                           E, P, E / P, pmagic, m.tb, m.nb, seg_log2, Kp, cnt, pre, pcnt, ppre,
                           inv, rows, prank, hdr, cnt_e, cnt_p, off_e, off_p, ptok_off, recv_x,
                           recv_scales, recv_src, recv_topk_idx, slot_src, dst_row, nchunk,
                           T * K, T * Kp);
    return hipGetLastError();
}

}  // namespace ep
