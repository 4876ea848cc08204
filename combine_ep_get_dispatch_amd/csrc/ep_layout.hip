// Dispatch layout on gfx950: per-expert and per-partition counts and offsets
// from the router's top-k expert ids, plus each slot's stable rank inside its
// expert, in one launch.
//
// The all-to-all of expert parallelism needs this bookkeeping before any
// token moves ("DeepSeek releases DeepEP, an efficient communication library
// for MoE models", section "DeepEP: Optimizing MoE Communication"); the pages
// do not describe it, so the definitions follow include/ep.h.
//
// Design.  Workgroup b owns the tokens [b*TB, b*TB + TB), about 2048 (token,
// slot) entries, split into 8 contiguous wave ranges.  Each wave walks its
// range 64 entries at a time and ranks every entry among the equal expert
// ids seen so far in that range: lanes with the same id are found with one
// ballot per id bit (AND of the matching ballots), so the rank is
// "count so far" (a per-wave LDS counter) plus the number of lower lanes in
// the match -- no atomics, so the order is deterministic and stable.  After a
// barrier the per-wave counters are prefix-summed across waves, giving each
// entry its rank inside the block, and the block's per-expert count goes to
// the workspace in expert-major order cnt[e][b].
//
// The last workgroup to finish (a ticket counter in the workspace header)
// then turns the counts into offsets: expert totals, their exclusive scan,
// and in place the per-(expert, block) bases
//     base[e][b] = expert_offsets[e] + sum_{b' < b} cnt[e][b'],
// from which dispatch computes every slot's receive row as
// base[e][block(t)] + rank.  The same last workgroup writes all the small
// outputs and resets the header for the next call.
#include "ep_internal.h"
#include "ep_device.h"

namespace ep {
namespace {

// Exclusive scan of a[0..n) in LDS by the whole workgroup; returns the total
// to every thread.  `red` is kLayoutWaves + 1 ints of LDS scratch.
__device__ int block_exclusive_scan(int* a, int n, int* red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (n + kLayoutThreads - 1) / kLayoutThreads;
    const int i0 = tid * per;
    const int i1 = min(i0 + per, n);
    int local = 0;
    for (int i = i0; i < i1; ++i) local += a[i];
    // inclusive scan of `local` across the wave
    int inc = local;
    for (int d = 1; d < 64; d <<= 1) {
        int up = __shfl_up(inc, d);
        if (lane >= d) inc += up;
    }
    if (lane == 63) red[wave] = inc;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int w = 0; w < kLayoutWaves; ++w) {
            int v = red[w];
            red[w] = run;
            run += v;
        }
        red[kLayoutWaves] = run;
    }
    __syncthreads();
    int run = red[wave] + inc - local;
    for (int i = i0; i < i1; ++i) {
        int v = a[i];
        a[i] = run;
        run += v;
    }
    const int total = red[kLayoutWaves];
    __syncthreads();
    return total;
}

__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(
    const int64_t* __restrict__ idx, int T, int K, int E, int P, int Ep, int TB, int nb,
    int ebits, WsHeader* __restrict__ hdr, int* __restrict__ cnt, int* __restrict__ pcnt,
    int* __restrict__ rank, int32_t* __restrict__ cnt_e, int32_t* __restrict__ cnt_p,
    uint8_t* __restrict__ in_part, int32_t* __restrict__ off_e, int32_t* __restrict__ off_p,
    int vec_rows) {
    extern __shared__ int smem[];
    int* wcnt = smem;                              // [waves][E] running counts
    int* ent = wcnt + kLayoutWaves * E;            // [kLayoutEntries] expert id or -1
    int* rnk = ent + kLayoutEntries;               // [kLayoutEntries] rank in wave range
    int* pc = rnk + kLayoutEntries;                // [P] distinct tokens per partition
    __shared__ int red[kLayoutWaves + 1];
    __shared__ int s_err;
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x;
    const int t0 = b * TB;
    const int tb = min(TB, T - t0);
    const int n = tb * K;
    const int64_t* my = idx + (int64_t)t0 * K;

    for (int i = tid; i < kLayoutWaves * E; i += kLayoutThreads) wcnt[i] = 0;
    for (int i = tid; i < P; i += kLayoutThreads) pc[i] = 0;
    if (tid == 0) s_err = 0;
    __syncthreads();

    // ---- stable ranks inside each wave's contiguous range of entries -------
    const int nchunks = (n + 63) >> 6;
    const int per = (nchunks + kLayoutWaves - 1) / kLayoutWaves;
    const int c0 = wave * per;
    const int c1 = min(c0 + per, nchunks);
    int* myw = wcnt + wave * E;
    int nerr = 0;
    for (int c = c0; c < c1; ++c) {
        const int j = (c << 6) + lane;
        const int64_t v = (j < n) ? my[j] : -1;
        const bool valid = v >= 0 && v < E;
        nerr += (j < n && !valid && v != -1) ? 1 : 0;
        const int e = valid ? (int)v : 0;
        uint64_t m = __ballot(valid);
        for (int bit = 0; bit < ebits; ++bit) {
            const bool on = (e >> bit) & 1;
            const uint64_t bb = __ballot(on);
            m &= on ? bb : ~bb;
        }
        int r = -1;
        if (valid) {
            r = myw[e] + __popcll(m & ((1ull << lane) - 1ull));
            if ((m >> lane) == 1ull) myw[e] += __popcll(m);   // highest lane of the match
        }
        if (j < n) {
            ent[j] = valid ? e : -1;
            rnk[j] = r;
        }
    }
    if (nerr) atomicAdd(&s_err, nerr);
    __syncthreads();

    // ---- prefix over waves; the block's per-expert count -------------------
    for (int e = tid; e < E; e += kLayoutThreads) {
        int run = 0;
        for (int w = 0; w < kLayoutWaves; ++w) {
            const int c = wcnt[w * E + e];
            wcnt[w * E + e] = run;
            run += c;
        }
        cnt[(int64_t)e * nb + b] = run;
    }
    __syncthreads();
    for (int j = tid; j < n; j += kLayoutThreads) {
        const int e = ent[j];
        const int w = (j >> 6) / per;
        rank[(int64_t)t0 * K + j] = (e >= 0) ? wcnt[w * E + e] + rnk[j] : -1;
    }

    // ---- partition membership rows, 16 partitions per work item -----------
    const int nwords = (P + 15) >> 4;
    for (int it = tid; it < tb * nwords; it += kLayoutThreads) {
        const int tl = it / nwords;
        const int pbeg = (it - tl * nwords) << 4;
        const int pend = min(pbeg + 16, P);
        uint64_t lo = 0, hi = 0;
        for (int k = 0; k < K; ++k) {
            const int e = ent[tl * K + k];
            if (e < 0) continue;
            const int p = e / Ep;
            if (p < pbeg || p >= pend) continue;
            const int q = p - pbeg;
            const uint64_t bit = 1ull << ((q & 7) * 8);
            const uint64_t word = (q < 8) ? lo : hi;
            if (!(word & bit)) {
                if (q < 8) lo |= bit; else hi |= bit;
                atomicAdd(&pc[p], 1);
            }
        }
        uint8_t* row = in_part + (int64_t)(t0 + tl) * P + pbeg;
        if (vec_rows) {
            *reinterpret_cast<uint4*>(row) =
                make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
        } else {
            for (int q = 0; q < pend - pbeg; ++q)
                row[q] = (uint8_t)(((q < 8 ? lo : hi) >> ((q & 7) * 8)) & 1u);
        }
    }
    __syncthreads();
    for (int p = tid; p < P; p += kLayoutThreads) pcnt[(int64_t)p * nb + b] = pc[p];
    if (tid == 0 && s_err)
        __hip_atomic_fetch_add(&hdr->invalid_accum, (int64_t)s_err, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);

    // ---- the last workgroup to finish turns counts into offsets -----------
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&hdr->ticket, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (uint32_t)(nb - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    int* tot = smem;   // [E] expert totals, then offsets (LDS reused)
    for (int e = tid; e < E; e += kLayoutThreads) {
        int s = 0;
        const int* col = cnt + (int64_t)e * nb;
        for (int bb = 0; bb < nb; ++bb) s += col[bb];
        tot[e] = s;
    }
    __syncthreads();
    const int total = block_exclusive_scan(tot, E, red);
    for (int e = tid; e < E; e += kLayoutThreads) {
        int run = tot[e];
        int* col = cnt + (int64_t)e * nb;
        for (int bb = 0; bb < nb; ++bb) {
            const int c = col[bb];
            col[bb] = run;
            run += c;
        }
        off_e[e] = tot[e];
        cnt_e[e] = run - tot[e];
    }
    for (int p = tid; p <= P; p += kLayoutThreads) off_p[p] = (p < P) ? tot[p * Ep] : total;
    for (int p = tid; p < P; p += kLayoutThreads) {
        int s = 0;
        const int* col = pcnt + (int64_t)p * nb;
        for (int bb = 0; bb < nb; ++bb) s += col[bb];
        cnt_p[p] = s;
    }
    if (tid == 0) {
        off_e[E] = total;
        hdr->num_valid = total;
        hdr->invalid_published =
            __hip_atomic_load(&hdr->invalid_accum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&hdr->invalid_accum, (int64_t)0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&hdr->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// T == 0: every count and offset is zero and no slot is invalid.
__global__ void layout_empty_kernel(int E, int P, WsHeader* __restrict__ hdr,
                                    int32_t* __restrict__ cnt_e, int32_t* __restrict__ cnt_p,
                                    int32_t* __restrict__ off_e, int32_t* __restrict__ off_p) {
    for (int i = threadIdx.x; i <= E; i += blockDim.x) {
        off_e[i] = 0;
        if (i < E) cnt_e[i] = 0;
    }
    for (int i = threadIdx.x; i <= P; i += blockDim.x) {
        off_p[i] = 0;
        if (i < P) cnt_p[i] = 0;
    }
    if (threadIdx.x == 0) {
        hdr->num_valid = 0;
        hdr->invalid_published = 0;
    }
}

}  // namespace

hipError_t launch_layout(const int64_t* idx, int T, int K, int E, int P, void* ws,
                         const WsMap& m, int32_t* cnt_e, int32_t* cnt_p, uint8_t* in_part,
                         int32_t* off_e, int32_t* off_p, hipStream_t s) {
    char* base = static_cast<char*>(ws);
    WsHeader* hdr = reinterpret_cast<WsHeader*>(base);
    if (T == 0) {
        hipLaunchKernelGGL(layout_empty_kernel, dim3(1), dim3(256), 0, s, E, P, hdr, cnt_e,
                           cnt_p, off_e, off_p);
        return hipGetLastError();
    }
    int ebits = 0;
    while ((1 << ebits) < E) ++ebits;
    const size_t lds = sizeof(int) * ((size_t)kLayoutWaves * E + 2 * kLayoutEntries + P);
    const int vec_rows = (P % 16 == 0) && (reinterpret_cast<uintptr_t>(in_part) % 16 == 0);
    hipLaunchKernelGGL(layout_kernel, dim3(m.nb), dim3(kLayoutThreads), lds, s, idx, T, K, E, P,
                       E / P, m.tb, m.nb, ebits, hdr, reinterpret_cast<int*>(base + m.cnt_off),
                       reinterpret_cast<int*>(base + m.pcnt_off),
                       reinterpret_cast<int*>(base + m.rank_off), cnt_e, cnt_p, in_part, off_e,
                       off_p, vec_rows);
    return hipGetLastError();
}

}  // namespace ep
