// Dispatch layout on gfx950: per-expert and per-partition counts and offsets
// from the router's top-k expert ids, and every valid slot's receive row.
//
// The all-to-all of expert parallelism needs this bookkeeping before any
// token moves ("DeepSeek releases DeepEP, an efficient communication library
// for MoE models", section "DeepEP: Optimizing MoE Communication"); the pages
// do not describe it, so the definitions follow include/ep.h.
//
// Every slot's rank among the earlier slots of its expert is found inside
// the workgroup that owns the slot's token: waves take contiguous ranges of
// its (token, slot) entries and walk them 64 at a time (in the count launch
// 12 of the 16 waves rank while the other 4 write the partition rows); the
// lanes holding the same expert id come from a per-wave LDS match table (E <=
// 256) or from one ballot per id bit (AND of the matching ballots), so a
// slot's rank is its wave's running count (LDS) plus the number of lower
// lanes in the match -- deterministic and stable, no atomics between
// workgroups -- and a prefix over the waves makes it the rank inside the
// workgroup.  What a workgroup cannot see alone is how many rows the earlier
// workgroups and the lower experts take.  Three forms provide it, with no
// atomics or fences between workgroups in any:
//
// * fused (one launch, for inputs of at most kFusedMaxBlocks token blocks,
//   e.g. decode batches): each workgroup stages ALL expert ids in LDS while
//   histogramming the slots before and after its own (its own slots are
//   counted by the ranking), scans the totals and writes final receive rows
//   for its own slots directly.  Workgroup 0 also counts the distinct tokens
//   per partition and writes the small outputs and the header.  Each
//   workgroup re-reads and re-counts every slot, so this only pays off while
//   the blocks are few: at 4096 x 8 (16 blocks) it measured 27 us against 14
//   us for the two launches.
//
// * count + finalize (ep_get_dispatch_layout, ep_layout_dispatch_aligned):
//   count writes per-workgroup expert counts cnt[b][*], partition rows and
//   counts, invalid counts, and for each slot (expert << 12 | rank in block);
//   finalize sums the count matrix per workgroup (E * nb ints), scans the
//   totals (rounded up to the alignment for the aligned layout) and rewrites
//   the slots as receive rows
//     row = expert_offsets[e] + (rows of e in blocks < b) + rank.
//
// * count + the dispatch launch (ep_layout_dispatch, ep_dispatch_dedup): the
//   count launch also writes each block's exclusive prefix of its counts over
//   the experts (and, de-duplicating, the tokens' ranks inside their
//   partitions and the prefix of the block's partition counts), and every
//   dispatch workgroup finishes its own token's rows from sums over the
//   blocks (ep_dispatch.hip).
#include "ep.h"
#include "ep_internal.h"
#include "ep_device.h"

#include <atomic>

namespace ep {
namespace {


// Stored form of an expert id: the id itself, -1 for a masked slot, -2 for an
// invalid one.
__device__ __forceinline__ int stored_id(int64_t v, int E) {
    return (v >= 0 && v < E) ? (int)v : (v == -1 ? -1 : -2);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (row
// shifts by 1, 2, 4, 8 inside each 16-lane row, then the row broadcasts of
// lanes 15 and 31); no LDS traffic.  Lanes a move has no source for take 0.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    const int lane = threadIdx.x & 63;
    int t;
    t = __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    if ((lane & 15) >= 1) x += t;
    t = __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    if ((lane & 15) >= 2) x += t;
    t = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    if ((lane & 15) >= 4) x += t;
    t = __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    if ((lane & 15) >= 8) x += t;
    t = __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
    if (lane & 16) x += t;
    t = __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
    if (lane & 32) x += t;
    return x;
}

// Exclusive scan of a[0..n) in LDS, called by the whole workgroup; returns
// the total to every thread.  Wave 0 alone scans: lane l sums its
// ceil(n / 64) consecutive values, a DPP inclusive sum joins the lanes, and
// the lane writes its values' exclusive prefixes back; one barrier publishes
// them and the total (`red`: one int of LDS scratch).
__device__ int block_exclusive_scan(int* a, int n, int* red) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int per = (n + 63) >> 6;
        const int i0 = lane * per;
        const int i1 = min(i0 + per, n);
        int local = 0;
        for (int i = i0; i < i1; ++i) local += a[i];
        const int inc = wave_inclusive_sum(local);
        int run = inc - local;
        for (int i = i0; i < i1; ++i) {
            const int v = a[i];
            a[i] = run;
            run += v;
        }
        if (lane == 63) red[0] = inc;
    }
    __syncthreads();
    return red[0];
}

// Stable ranks of the workgroup's own entries ids[0..n) (stored ids, < 0 =
// no expert).  wcnt is [kLayoutWaves][E] zeroed LDS, rnk [n] LDS.  After the
// call rnk[j] is the number of entries before j (inside the workgroup) with
// the same expert, -1 for entries without one; if blk_cnt is given,
// blk_cnt[e] receives the workgroup's count of expert e.
//
// The lanes of a 64-entry chunk that hold the same expert (the "match" mask)
// come either from one ballot per id bit (ebits ballots, each a handful of
// VALU instructions per lane) or, when mtab is given ([kLayoutWaves][E][2]
// zeroed 32-bit LDS words, for E <= kMatchTableMaxE), from the wave's own
// table: every lane ORs its bit into mtab[e] (lanes 0-31 the first word,
// 32-63 the second), reads both words back and clears them -- one wave's LDS
// operations complete in issue order, so the reads see the whole chunk's
// bits and the clears follow every read.  (32-bit words: the tables start at
// an offset of the dynamic area that is only a multiple of 4 bytes.)  The
// table costs a few LDS operations per chunk instead of the ballots' VALU
// work, which is what bounds this loop on the few workgroups a layout uses.
//
// Only the first nrw waves rank; the others run side() meanwhile (work that
// needs the staged ids but not the ranks), and everything after the first
// barrier is shared by the whole workgroup.  mid() runs on every thread
// between the first and the second barrier (it sees what side() wrote, and
// what it writes is seen by everything after the call).
//
// FINAL = false stops after the second barrier, before the ranks are made
// block-wide: rnk[j] is then the rank inside its wave's range and the caller
// adds wcnt[w * E + e] (by then each wave's exclusive prefix over the ranking
// waves) with w = (j >> 6) / rank_chunks_per_wave(n, nrw) -- one LDS pass and
// one barrier fewer when the caller reads every rank once anyway.
struct NoSideWork {
    __device__ void operator()() const {}
};

__device__ __forceinline__ int rank_chunks_per_wave(int n, int nrw) {
    return (((n + 63) >> 6) + nrw - 1) / nrw;
}

template <bool FINAL = true, typename Id, typename Side = NoSideWork, typename Mid = NoSideWork>
__device__ void rank_entries(const Id* ids, int n, int E, int ebits, int* wcnt, int* rnk,
                             int* blk_cnt, unsigned* mtab = nullptr, int nrw = kLayoutWaves,
                             Side side = Side(), Mid mid = Mid()) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nchunks = (n + 63) >> 6;
    const int per = rank_chunks_per_wave(n, nrw);
    const int c0 = wave < nrw ? wave * per : nchunks;
    const int c1 = min(c0 + per, nchunks);
    int* myw = wcnt + wave * E;
    unsigned* myt = mtab ? mtab + (size_t)wave * 2 * E : nullptr;
    for (int c = c0; c < c1; ++c) {          // wave-uniform loop: ballots are safe
        const int j = (c << 6) + lane;
        const int e0 = (j < n) ? (int)ids[j] : -1;
        const bool valid = e0 >= 0;
        const int e = valid ? e0 : 0;
        uint64_t m;
        if (myt) {
            unsigned* w = myt + 2 * e;
            // The three phases touch different words of the table (a lane ORs
            // one word, reads two), so nothing but these compiler fences keeps
            // their LDS operations in the order written; the hardware then
            // completes one wave's LDS operations in issue order.
            if (valid) __hip_atomic_fetch_or(w + (lane >> 5), 1u << (lane & 31), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_WAVEFRONT);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            unsigned lo = 0, hi = 0;
            if (valid) {
                lo = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
                hi = __hip_atomic_load(w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (valid) {
                __hip_atomic_store(w, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
                __hip_atomic_store(w + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the next chunk's ORs follow the clears
            m = ((uint64_t)hi << 32) | lo;
        } else {
            m = __ballot(valid);
            for (int bit = 0; bit < ebits; ++bit) {
                const bool on = (e >> bit) & 1;
                const uint64_t bb = __ballot(on);
                m &= on ? bb : ~bb;
            }
        }
        if (valid) {
            rnk[j] = myw[e] + __popcll(m & ((1ull << lane) - 1ull));
            if ((m >> lane) == 1ull) myw[e] += __popcll(m);   // highest lane of the match
        } else if (j < n) {
            rnk[j] = -1;
        }
    }
    if (wave >= nrw) side();
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kLayoutThreads) {   // prefix over waves
        int run = 0;
        for (int w = 0; w < nrw; ++w) {
            const int c = wcnt[w * E + e];
            wcnt[w * E + e] = run;
            run += c;
        }
        if (blk_cnt) blk_cnt[e] = run;
    }
    mid();
    __syncthreads();
    if constexpr (FINAL) {
        for (int j = threadIdx.x; j < n; j += kLayoutThreads) {
            const int e = ids[j];
            if (e >= 0) rnk[j] += wcnt[((j >> 6) / per) * E + e];
        }
        __syncthreads();
    }
}

// One wave writes the block's expert counts cnt[0..E) and their exclusive
// prefix pre[0..E] (pre[E] = total) from bc, which holds 64*PER ints (zero
// past E); lane l owns experts [l*PER, l*PER + PER).
template <int PER>
__device__ void scan_block_counts(const int* bc, int E, int* cnt, int* pre) {
    const int lane = threadIdx.x & 63;
    const int e0 = lane * PER;
    int v[PER];
    int local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        v[i] = bc[e0 + i];
        local += v[i];
    }
    const int inc = wave_inclusive_sum(local);
    int run = inc - local;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (e0 + i < E) {
            cnt[e0 + i] = v[i];
            pre[e0 + i] = run;
        }
        run += v[i];
    }
    if (lane == 63) pre[E] = inc;
}

// Per-lane share of experts for scan_block_counts: ceil(E / 64) rounded up to
// a power of two (<= 16 for E <= 1024).
__host__ __device__ constexpr int scan_per(int E) {
    int per = 1;
    while (per * 64 < E) per <<= 1;
    return per;
}

// Match tables are used up to this many experts ([waves][E][2] 32-bit words).
constexpr int kMatchTableMaxE = 256;

// Waves of the count launch that rank; the others (side waves) write the
// partition rows meanwhile.  In the de-duplicating mode the kCountSideWaves
// side waves also rank the tokens inside their partitions, which needs their
// LDS tables; the other modes give half the waves to the partition rows,
// which measured 0.3 us faster than four (12.3 against 12.6 us for the
// two-launch layout of 4096 tokens, top-8 of 256 experts, 64 partitions).
constexpr int kCountRankWaves = 8;
constexpr int kDedupRankWaves = 12;
constexpr int kCountSideWaves = kLayoutWaves - kDedupRankWaves;
static_assert(kCountSideWaves > 0 && kCountRankWaves < kLayoutWaves,
              "no waves left for the partition rows");

// Flag on a side wave's partition rank: the token is the highest member of
// its pass in the slot's partition (ranks stay below kLayoutEntries).
constexpr int kSideTop = 1 << 30;

// Ints of layout_count_kernel's partition-count array pc: P, padded with
// zeros to 64 * scan_per(P) when it is scanned (kCountDedup).
__host__ __device__ constexpr int count_pc_ints(int P, int mode) {
    return mode == kCountDedup ? 64 * scan_per(P) : P;
}

// layout_count_kernel's dynamic LDS, in ints: wcnt [waves][E], ids and rnk
// [kLayoutEntries] each, pc [count_pc_ints], with kCountPre or kCountDedup bc
// [64 * scan_per(E)], with kCountDedup the side waves' partition match tables
// ptab [kCountSideWaves][P][2], their member counts prun [kCountSideWaves][P]
// and the slots' partition ranks psr [kLayoutEntries]; the expert match
// tables follow at the returned offset.
__host__ __device__ constexpr int count_table_offset(int E, int P, int mode) {
    return kLayoutWaves * E + 2 * kLayoutEntries + count_pc_ints(P, mode) +
           (mode != kCountPlain ? 64 * scan_per(E) : 0) +
           (mode == kCountDedup ? 3 * kCountSideWaves * P + kLayoutEntries : 0);
}

// Partition of expert e: e / Ep computed as (e * ceil(2^32 / Ep)) >> 32,
// which is exact for e, Ep <= 2^10 (the error e * (ceil(2^32/Ep) - 2^32/Ep)
// / 2^32 < 2^-22 stays below the 1/Ep gap to the next integer).
__device__ __forceinline__ int partition_of(int e, uint64_t pmagic) {
    return (int)(((uint64_t)(uint32_t)e * pmagic) >> 32);
}

// Four membership bits (bit i of x, i < 4) as four bytes 0/1.
__device__ __forceinline__ uint32_t spread4(uint32_t x) {
    return (x & 1u) | ((x & 2u) << 7) | ((x & 4u) << 14) | ((x & 8u) << 21);
}

// One token's membership bytes for 64 partitions or fewer (nbytes), from
// their bit mask; 16-byte stores when vec (nbytes a multiple of 16, row
// 16-byte aligned).
__device__ __forceinline__ void write_member_row(uint8_t* row, uint64_t mask, int nbytes,
                                                 bool vec) {
    if (vec) {
        for (int q = 0; q < nbytes; q += 16) {
            const uint32_t b16 = (uint32_t)(mask >> q) & 0xffffu;
            *reinterpret_cast<uint4*>(row + q) =
                make_uint4(spread4(b16), spread4(b16 >> 4), spread4(b16 >> 8), spread4(b16 >> 12));
        }
    } else {
        for (int q = 0; q < nbytes; ++q) row[q] = (uint8_t)((mask >> q) & 1u);
    }
}

// Partition-membership rows of tokens [0, ntok) (thread per token; ids are
// their K stored ids each, token-major): for every window of 64 partitions
// the token's membership is a 64-bit mask, written out as bytes to
// out_rows (row stride P; 16-byte stores when `vec`) and, if pc is given,
// counted into pc (one LDS atomic per member partition).
template <typename Id>
__device__ void partition_rows(const Id* ids, int ntok, int K, int P, uint64_t pmagic,
                               uint8_t* out_rows, bool vec, int* pc,
                               int first = -1, int stride = kLayoutThreads) {
    for (int tl = first < 0 ? (int)threadIdx.x : first; tl < ntok; tl += stride) {
        for (int w0 = 0; w0 < P; w0 += 64) {
            uint64_t mask = 0;
            for (int k = 0; k < K; ++k) {
                const int e = ids[tl * K + k];
                if (e < 0) continue;
                const int q = partition_of(e, pmagic) - w0;
                if (q >= 0 && q < 64) mask |= 1ull << q;
            }
            if (pc) {
                for (uint64_t m = mask; m; m &= m - 1) atomicAdd(&pc[w0 + __builtin_ctzll(m)], 1);
            }
            if (out_rows)
                write_member_row(out_rows + (int64_t)tl * P + w0, mask, min(64, P - w0), vec);
        }
    }
}

// Tokens per side wave in the de-duplicating count launch: the block's ntok
// tokens in ns contiguous spans, whole passes of 64.
__host__ __device__ inline int side_span(int ntok, int ns) {
    return ((ntok + ns - 1) / ns + 63) & ~63;
}

// Slots a side wave handles at once (their partitions and ranks in registers).
constexpr int kSideChunk = 8;

// Side wave s (of ns) of the de-duplicating count launch: the partition rows
// of tokens [s*span, (s+1)*span) (as partition_rows writes them) and, for
// each of their slots, the token's rank among the span's member tokens of
// the slot's partition (token order).  Tokens go in passes of 64, lane =
// token.  Within a pass the members of partition p come from the wave's LDS
// match table tab[p] (two 32-bit words: lanes 0-31 and 32-63): every slot
// ORs its lane's bit into its partition's entry, reads the entry back and
// takes run[p] (the span's members of p in the earlier passes) plus the
// members below its lane; then every slot clears its entry, and the highest
// member stores run[p] = its rank + 1.  A token with several slots in p sets
// the same bit and stores the same values, so no slot needs to know whether
// it is its token's first in p.  One wave's LDS operations complete in issue
// order, so each read sees all of the pass's bits and the clears and stores
// follow every read.  Slots go kSideChunk at a time so that their LDS loads
// are issued together; with K <= kSideChunk a token's partitions and ranks
// stay in registers through the pass (and, with P <= 64, give its membership
// row too).  srank[slot] gets the rank (with kSideTop on the highest member's
// slots); run[s][p] ends holding the span's member count of p.  tab and run
// start zeroed; tab ends zeroed.
template <typename Id>
__device__ void partition_ranks_side(const Id* ids, int ntok, int K, int P, uint64_t pmagic,
                                     uint8_t* out_rows, bool vec, unsigned* tab, int* run,
                                     int* srank, int s, int ns) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    const int span = side_span(ntok, ns);
    const int t_end = min(ntok, (s + 1) * span);
    unsigned* mytab = tab + (size_t)s * 2 * P;
    int* myrun = run + (size_t)s * P;
    const bool one = K <= kSideChunk;
    if (!(one && P <= 64))
        partition_rows(ids, t_end, K, P, pmagic, out_rows, vec, nullptr, s * span + lane, 64);
    for (int base = s * span; base < t_end; base += 64) {
        const int tl = base + lane;
        if (tl >= t_end) continue;
        const Id* tok_ids = ids + tl * K;
        int* tok_rank = srank + tl * K;
        int pp[kSideChunk];                // partitions of slots k0 .. k0 + 7 (-1: none)
        int rr[kSideChunk];                // their ranks (| kSideTop)
        const auto parts = [&](int k0) {
#pragma unroll
            for (int i = 0; i < kSideChunk; ++i) {
                const int e = k0 + i < K ? (int)tok_ids[k0 + i] : -1;
                pp[i] = e >= 0 ? partition_of(e, pmagic) : -1;
            }
        };
        const auto set_bits = [&]() {
#pragma unroll
            for (int i = 0; i < kSideChunk; ++i)
                if (pp[i] >= 0)
                    __hip_atomic_fetch_or(mytab + 2 * pp[i] + (lane >> 5), 1u << (lane & 31),
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        };
        const auto read_ranks = [&](int k0) {
#pragma unroll
            for (int i = 0; i < kSideChunk; ++i) {
                if (pp[i] < 0) continue;
                const unsigned lo = __hip_atomic_load(mytab + 2 * pp[i], __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_WAVEFRONT);
                const unsigned hi = __hip_atomic_load(mytab + 2 * pp[i] + 1, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_WAVEFRONT);
                const uint64_t m = ((uint64_t)hi << 32) | lo;
                const int r = __hip_atomic_load(myrun + pp[i], __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_WAVEFRONT) +
                              __popcll(m & below);
                rr[i] = (m >> lane) == 1ull ? r | kSideTop : r;
                __hip_atomic_store(tok_rank + k0 + i, rr[i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WAVEFRONT);
            }
        };
        const auto clear = [&]() {
#pragma unroll
            for (int i = 0; i < kSideChunk; ++i) {
                if (pp[i] < 0) continue;
                __hip_atomic_store(mytab + 2 * pp[i], 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WAVEFRONT);
                __hip_atomic_store(mytab + 2 * pp[i] + 1, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WAVEFRONT);
                if (rr[i] & kSideTop)
                    __hip_atomic_store(myrun + pp[i], (rr[i] & ~kSideTop) + 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WAVEFRONT);
            }
        };
        if (one) {
            parts(0);
            if (P <= 64) {
                uint64_t mask = 0;
#pragma unroll
                for (int i = 0; i < kSideChunk; ++i)
                    if (pp[i] >= 0) mask |= 1ull << pp[i];
                write_member_row(out_rows + (int64_t)tl * P, mask, P, vec);
            }
            set_bits();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);   // keep the phases in issue order
            read_ranks(0);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            clear();
        } else {
            for (int k0 = 0; k0 < K; k0 += kSideChunk) {
                parts(k0);
                set_bits();
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            for (int k0 = 0; k0 < K; k0 += kSideChunk) {
                parts(k0);
                read_ranks(k0);
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            for (int k0 = 0; k0 < K; k0 += kSideChunk) {
                parts(k0);
#pragma unroll
                for (int i = 0; i < kSideChunk; ++i)
                    if (pp[i] >= 0)
                        rr[i] = __hip_atomic_load(tok_rank + k0 + i, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_WAVEFRONT);
                clear();
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
}

// ---------------------------------------------------------------- fused ----

__global__ __launch_bounds__(kLayoutThreads) void layout_fused_kernel(
    const int64_t* __restrict__ idx, int T, int K, int E, int P, int Ep, uint64_t pmagic,
    int TB, int ebits, int* __restrict__ rows, uint8_t* __restrict__ in_part, int vec_rows,
    WsHeader* __restrict__ hdr, int32_t* __restrict__ cnt_e, int32_t* __restrict__ cnt_p,
    int32_t* __restrict__ off_e, int32_t* __restrict__ off_p) {
    extern __shared__ EP_LDS_ALIGN int smem[];
    int* bef = smem;                               // [E] slots of e before this block's
    int* aft = bef + E;                            // [E] ... after this block's
    int* own = aft + E;                            // [E] ... in this block
    int* off = own + E;                            // [E] expert offsets
    int* wcnt = off + E;                           // [waves][E]
    int* rnk = wcnt + kLayoutWaves * E;            // [kLayoutEntries]
    int* pc = rnk + kLayoutEntries;                // [P]
    int16_t* ids = reinterpret_cast<int16_t*>(pc + P);   // [T*K] stored ids
    __shared__ int red[1];
    __shared__ int s_err;

    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int TK = T * K;
    const int t0 = b * TB;
    const int tb = min(TB, T - t0);
    const int j0 = t0 * K;
    const int n = tb * K;

    for (int i = tid; i < (4 + kLayoutWaves) * E; i += kLayoutThreads) smem[i] = 0;
    for (int i = tid; i < P; i += kLayoutThreads) pc[i] = 0;
    if (tid == 0) s_err = 0;
    __syncthreads();

    // ---- stage every expert id in LDS; histogram the slots outside the
    //      block (before / after); 16 loads in flight per thread ------------
    int nerr = 0;
    constexpr int U = 16;
    for (int base = 0; base < TK; base += U * kLayoutThreads) {
        int64_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * kLayoutThreads + tid;
            v[u] = (j < TK) ? idx[j] : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * kLayoutThreads + tid;
            if (j < TK) {
                const int id = stored_id(v[u], E);
                if (id >= 0 && (j < j0 || j >= j0 + n)) atomicAdd(j < j0 ? &bef[id] : &aft[id], 1);
                nerr += (id == -2);
                ids[j] = (int16_t)id;
            }
        }
    }
    if (nerr) atomicAdd(&s_err, nerr);
    __syncthreads();

    // ---- own slots: stable ranks and the block's own counts ----------------
    rank_entries(ids + j0, n, E, ebits, wcnt, rnk, own);

    // ---- offsets ------------------------------------------------------------
    for (int e = tid; e < E; e += kLayoutThreads) off[e] = bef[e] + own[e] + aft[e];
    __syncthreads();
    const int total = block_exclusive_scan(off, E, red);

    for (int j = tid; j < n; j += kLayoutThreads) {
        const int e = ids[j0 + j];
        rows[(int64_t)j0 + j] = (e >= 0) ? off[e] + bef[e] + rnk[j] : -1;
    }
    partition_rows(ids + j0, tb, K, P, pmagic, in_part + (int64_t)t0 * P, vec_rows != 0,
                   (int*)nullptr);

    if (b != 0) return;
    // ---- workgroup 0: distinct tokens per partition and the small outputs ---
    partition_rows(ids, T, K, P, pmagic, (uint8_t*)nullptr, false, pc);
    for (int e = tid; e < E; e += kLayoutThreads) {
        off_e[e] = off[e];
        cnt_e[e] = bef[e] + own[e] + aft[e];
    }
    for (int p = tid; p <= P; p += kLayoutThreads) off_p[p] = (p < P) ? off[p * Ep] : total;
    __syncthreads();
    for (int p = tid; p < P; p += kLayoutThreads) cnt_p[p] = pc[p];
    if (tid == 0) {
        off_e[E] = total;
        hdr->num_valid = total;
        hdr->num_invalid = s_err;
    }
}

// ------------------------------------------------------------ two launches --

// MODE >= kCountPre: also write pre[b][0..E] = the block's exclusive prefix
// of its expert counts over the experts (pre[b][E] = the block's valid
// slots), so that a later kernel can form any expert offset as a sum over
// blocks instead of a scan over experts (the one-call layout + dispatch uses
// this).  MODE == kCountDedup: also prank (in-block partition ranks of every
// slot) and ppre[b][0..P] (prefix of the block's partition counts).
template <int MODE>
__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(
    const int64_t* __restrict__ idx, int T, int K, int E, int P, uint64_t pmagic, int TB,
    int ebits,
    int* __restrict__ cnt, int* __restrict__ pcnt, int* __restrict__ inv,
    int* __restrict__ rows, uint8_t* __restrict__ in_part, int vec_rows,
    int* __restrict__ pre, int* __restrict__ prank, int* __restrict__ ppre) {
    constexpr bool PRE = MODE != kCountPlain;
    extern __shared__ EP_LDS_ALIGN int smem[];
    int* wcnt = smem;                              // [waves][E]
    int* ids = wcnt + kLayoutWaves * E;            // [kLayoutEntries] stored ids
    int* rnk = ids + kLayoutEntries;               // [kLayoutEntries]
    int* pc = rnk + kLayoutEntries;                // [count_pc_ints(P, MODE)]
    int* bc = pc + count_pc_ints(P, MODE);         // [64 * scan_per(E)] block counts (PRE)
    // kCountDedup: the side waves' partition tables, member counts and ranks
    unsigned* ptab = reinterpret_cast<unsigned*>(bc + (PRE ? 64 * scan_per(E) : 0));
    int* prun = reinterpret_cast<int*>(ptab + 2 * kCountSideWaves * P);   // [side waves][P]
    int* psr = prun + kCountSideWaves * P;                                // [kLayoutEntries]
    // [waves][E][2] match tables (E <= kMatchTableMaxE)
    unsigned* mtab = reinterpret_cast<unsigned*>(smem + count_table_offset(E, P, MODE));
    const bool use_mtab = E <= kMatchTableMaxE;
    __shared__ int s_err;

    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int t0 = b * TB;
    const int tb = min(TB, T - t0);
    const int n = tb * K;                          // <= kLayoutEntries
    const int64_t* my = idx + (int64_t)t0 * K;

    // All (at most 4) loads per thread are issued before anything else.
    constexpr int U = kLayoutEntries / kLayoutThreads;
    int64_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = u * kLayoutThreads + tid;
        v[u] = (j < n) ? my[j] : -1;
    }
    for (int i = tid; i < kLayoutWaves * E; i += kLayoutThreads) wcnt[i] = 0;
    for (int i = tid; i < count_pc_ints(P, MODE); i += kLayoutThreads) pc[i] = 0;
    if (PRE)
        for (int i = E + tid; i < 64 * scan_per(E); i += kLayoutThreads) bc[i] = 0;
    if (use_mtab)
        for (int i = tid; i < 2 * kLayoutWaves * E; i += kLayoutThreads) mtab[i] = 0u;
    if (MODE == kCountDedup)                       // ptab and prun
        for (int i = tid; i < 3 * kCountSideWaves * P; i += kLayoutThreads) ptab[i] = 0u;
    if (tid == 0) s_err = 0;
    int nerr = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = u * kLayoutThreads + tid;
        if (j < n) {
            const int id = stored_id(v[u], E);
            nerr += (id == -2);
            ids[j] = id;
        }
    }
    __syncthreads();
    if (nerr) atomicAdd(&s_err, nerr);

    unsigned* tab = use_mtab ? mtab : nullptr;
    // The waves after the first nrw write the partition rows (which need
    // only the staged ids) while the first ones rank; in the de-duplicating
    // mode they also rank the tokens inside their partitions, and between
    // the ranking's barriers every thread turns their per-span member counts
    // into prefixes over the spans (pc = the block's totals).
    constexpr int nrw = MODE == kCountDedup ? kDedupRankWaves : kCountRankWaves;
    [[maybe_unused]] const int side_tok = side_span(tb, kCountSideWaves);
    const auto side = [&]() {
        if constexpr (MODE == kCountDedup)
            partition_ranks_side(ids, tb, K, P, pmagic, in_part + (int64_t)t0 * P,
                                 vec_rows != 0, ptab, prun, psr,
                                 __builtin_amdgcn_readfirstlane(tid >> 6) - nrw, kCountSideWaves);
        else
            partition_rows(ids, tb, K, P, pmagic, in_part + (int64_t)t0 * P, vec_rows != 0, pc,
                           tid - nrw * 64, kLayoutThreads - nrw * 64);
    };
    const auto mid = [&]() {
        if constexpr (MODE == kCountDedup) {
            for (int p = tid; p < P; p += kLayoutThreads) {
                int run = 0;
                for (int w = 0; w < kCountSideWaves; ++w) {
                    const int c = prun[w * P + p];
                    prun[w * P + p] = run;
                    run += c;
                }
                pc[p] = run;
            }
        }
    };
    if constexpr (PRE) {
        rank_entries<false>(ids, n, E, ebits, wcnt, rnk, bc, tab, nrw, side, mid);   // ends with a barrier
        // One wave scans the block's expert counts and (de-duplicating mode)
        // another its partition counts; the other waves go on with the rows.
        if (tid < 64) {
            int* cb = cnt + (int64_t)b * E;
            int* pb = pre + (int64_t)b * (E + 1);
            switch (scan_per(E)) {
                case 1: scan_block_counts<1>(bc, E, cb, pb); break;
                case 2: scan_block_counts<2>(bc, E, cb, pb); break;
                case 4: scan_block_counts<4>(bc, E, cb, pb); break;
                case 8: scan_block_counts<8>(bc, E, cb, pb); break;
                default: scan_block_counts<16>(bc, E, cb, pb); break;
            }
        } else if (MODE == kCountDedup && tid < 128) {
            int* cb = pcnt + (int64_t)b * P;
            int* pb = ppre + (int64_t)b * (P + 1);
            switch (scan_per(P)) {
                case 1: scan_block_counts<1>(pc, P, cb, pb); break;
                case 2: scan_block_counts<2>(pc, P, cb, pb); break;
                case 4: scan_block_counts<4>(pc, P, cb, pb); break;
                case 8: scan_block_counts<8>(pc, P, cb, pb); break;
                default: scan_block_counts<16>(pc, P, cb, pb); break;
            }
        }
    } else {
        rank_entries<false>(ids, n, E, ebits, wcnt, rnk, cnt + (int64_t)b * E, tab, nrw, side);
    }
    // The packed slots, the in-wave ranks made block-wide on the way; the
    // waves scanning the block's counts above stay out.
    const int per = rank_chunks_per_wave(n, nrw);
    constexpr int busy = MODE == kCountDedup ? 128 : (MODE == kCountPre ? 64 : 0);
    if (tid >= busy) {
        for (int j = tid - busy; j < n; j += kLayoutThreads - busy) {
            const int e = ids[j];
            rows[(int64_t)t0 * K + j] =
                (e >= 0) ? (e << kRankBits) | (rnk[j] + wcnt[((j >> 6) / per) * E + e]) : -1;
            if constexpr (MODE == kCountDedup) {
                const int w = (j / K) / side_tok;  // the side wave that ranked the token
                prank[(int64_t)t0 * K + j] =
                    e >= 0 ? prun[w * P + partition_of(e, pmagic)] + (psr[j] & ~kSideTop) : -1;
            }
        }
    }
    if constexpr (MODE != kCountDedup)
        for (int p = tid; p < P; p += kLayoutThreads) pcnt[(int64_t)b * P + p] = pc[p];
    if (tid == 0) inv[b] = s_err;
}

// align > 1: every expert's run is padded to a multiple of align rows, and
// (recv_src given) the padding rows and the rows [used, R) get source -1 --
// workgroup b marks the padding of experts b, b + nb, ..., and all
// workgroups stride over the rows past the last run.
__global__ __launch_bounds__(kLayoutThreads) void layout_finalize_kernel(
    int T, int K, int E, int P, int Ep, int TB, int nb, const int* __restrict__ cnt,
    const int* __restrict__ pcnt, const int* __restrict__ inv, int* __restrict__ rows,
    WsHeader* __restrict__ hdr, int32_t* __restrict__ cnt_e, int32_t* __restrict__ cnt_p,
    int32_t* __restrict__ off_e, int32_t* __restrict__ off_p, int align,
    int32_t* __restrict__ recv_src, int64_t R) {
    extern __shared__ EP_LDS_ALIGN int smem[];
    int* off = smem;          // [E] totals, then exclusive offsets
    int* bef = off + E;       // [E] rows of e in blocks before this one
    int* tot = bef + E;       // [E] totals (kept for the outputs)
    __shared__ int red[1];

    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    // The block's packed slots (at most kLayoutEntries) are loaded first:
    // they do not depend on the sums below.
    const int t0 = b * TB;
    const int n = min(TB, T - t0) * K;
    constexpr int U = kLayoutEntries / kLayoutThreads;
    static_assert(kLayoutEntries % kLayoutThreads == 0, "whole rounds of slots");
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = u * kLayoutThreads + tid;
        v[u] = j < n ? rows[(int64_t)t0 * K + j] : -1;
    }
    for (int e = tid; e < E; e += kLayoutThreads) {
        int s_all = 0, s_bef = 0;
#pragma unroll 8
        for (int bb = 0; bb < nb; ++bb) {
            const int c = cnt[(int64_t)bb * E + e];
            s_all += c;
            s_bef += (bb < b) ? c : 0;
        }
        off[e] = align > 1 ? (s_all + align - 1) / align * align : s_all;
        tot[e] = s_all;
        bef[e] = s_bef;
    }
    __syncthreads();
    const int total = block_exclusive_scan(off, E, red);

    if (recv_src) {
        for (int e = b; e < E; e += nb) {
            const int r1 = e + 1 < E ? off[e + 1] : total;
            for (int r = off[e] + tot[e] + tid; r < r1; r += kLayoutThreads) recv_src[r] = -1;
        }
        for (int64_t r = total + (int64_t)b * kLayoutThreads + tid; r < R;
             r += (int64_t)nb * kLayoutThreads)
            recv_src[r] = -1;
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = u * kLayoutThreads + tid;
        if (v[u] >= 0) {
            const int e = v[u] >> kRankBits;
            rows[(int64_t)t0 * K + j] = off[e] + bef[e] + (v[u] & ((1 << kRankBits) - 1));
        }
    }

    if (b != 0) return;
    for (int e = tid; e < E; e += kLayoutThreads) {
        off_e[e] = off[e];
        cnt_e[e] = tot[e];
    }
    for (int p = tid; p <= P; p += kLayoutThreads) off_p[p] = (p < P) ? off[p * Ep] : total;
    for (int p = tid; p < P; p += kLayoutThreads) {
        int s = 0;
#pragma unroll 8
        for (int bb = 0; bb < nb; ++bb) s += pcnt[(int64_t)bb * P + p];
        cnt_p[p] = s;
    }
    if (tid == 0) {
        int64_t nerr = 0;
        for (int bb = 0; bb < nb; ++bb) nerr += inv[bb];
        off_e[E] = total;
        hdr->num_valid = total;
        hdr->num_invalid = nerr;
    }
}

// n ints of p set to v.
__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
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
        hdr->num_invalid = 0;
    }
}

}  // namespace

size_t layout_fused_lds_bytes(int T, int K, int E, int P) {
    const size_t ids = align256(sizeof(int16_t) * (size_t)T * (size_t)K);
    return sizeof(int) * ((size_t)(4 + kLayoutWaves) * E + kLayoutEntries + P) + ids;
}

// Raising a kernel's dynamic-LDS cap is a per-device attribute of the
// function: it is set once per (kernel, device) -- remembered in one bit per
// device of an atomic word per kernel slot, so concurrent callers and several
// devices are safe.  Devices past 63 set it on every call.
namespace {
std::atomic<uint64_t> g_lds_raised[kLdsSlots];
}  // namespace

hipError_t allow_large_lds(const void* fn, int slot, int bytes) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (g_lds_raised[slot].load(std::memory_order_acquire) & bit)) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) g_lds_raised[slot].fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

namespace {
// The layout kernels raise their cap to the largest LDS any launch here asks for.
constexpr int kLdsCap = (int)kFusedLdsLimit;
}  // namespace

bool layout_single_launch(int T, int K, int E, int P, const WsMap& m) {
    return T > 0 && m.nb <= kFusedMaxBlocks && layout_fused_lds_bytes(T, K, E, P) <= kFusedLdsLimit;
}

namespace {

int expert_bits(int E) {
    int ebits = 0;
    while ((1 << ebits) < E) ++ebits;
    return ebits;
}

uint64_t partition_magic(int Ep) {   // ceil(2^32 / Ep)
    return ((uint64_t)1 << 32) / (uint64_t)Ep + ((((uint64_t)1 << 32) % (uint64_t)Ep) ? 1 : 0);
}

bool vector_rows(int P, const uint8_t* in_part) {
    return (P % 16 == 0) && (reinterpret_cast<uintptr_t>(in_part) % 16 == 0);
}

}  // namespace

// Dynamic LDS of layout_count_kernel; the largest shapes of each kind fit.
static_assert(sizeof(int) * count_table_offset(EP_MAX_EXPERTS, EP_MAX_EXPERTS, kCountDedup) <=
                  (size_t)kLdsCap, "count launch LDS");
static_assert(sizeof(int) * (count_table_offset(kMatchTableMaxE, kMatchTableMaxE, kCountDedup) +
                             2 * kLayoutWaves * kMatchTableMaxE) <= (size_t)kLdsCap,
              "count launch LDS with match tables");
size_t count_lds_bytes(int E, int P, int mode) {
    size_t bytes = sizeof(int) * (size_t)count_table_offset(E, P, mode);
    if (E <= kMatchTableMaxE) bytes += sizeof(unsigned) * 2 * (size_t)kLayoutWaves * E;
    return bytes;
}

hipError_t launch_layout_count(const int64_t* idx, int T, int K, int E, int P, void* ws,
                               const WsMap& m, uint8_t* in_part, int mode, hipStream_t s) {
    char* base = static_cast<char*>(ws);
    int* cnt = reinterpret_cast<int*>(base + m.cnt_off);
    int* pcnt = reinterpret_cast<int*>(base + m.pcnt_off);
    int* inv = reinterpret_cast<int*>(base + m.inv_off);
    int* pre = reinterpret_cast<int*>(base + m.pre_off);
    int* ppre = reinterpret_cast<int*>(base + m.ppre_off);
    int* prank = reinterpret_cast<int*>(base + m.prank_off);
    int* rows = reinterpret_cast<int*>(base + m.rows_off);
    const int ebits = expert_bits(E);
    const uint64_t pmagic = partition_magic(E / P);
    const int vec = vector_rows(P, in_part);
    const size_t lds = count_lds_bytes(E, P, mode);
    if (lds > 64 * 1024) {
        const void* fn = mode == kCountDedup
                             ? reinterpret_cast<const void*>(layout_count_kernel<kCountDedup>)
                         : mode == kCountPre
                             ? reinterpret_cast<const void*>(layout_count_kernel<kCountPre>)
                             : reinterpret_cast<const void*>(layout_count_kernel<kCountPlain>);
        hipError_t e = allow_large_lds(fn, kCountLdsSlot + mode, kLdsCap);
        if (e != hipSuccess) return e;
    }
    if (mode == kCountDedup)
        hipLaunchKernelGGL(layout_count_kernel<kCountDedup>, dim3(m.nb), dim3(kLayoutThreads), lds,
                           s, idx, T, K, E, P, pmagic, m.tb, ebits, cnt, pcnt, inv, rows, in_part,
                           vec, pre, prank, ppre);
    else if (mode == kCountPre)
        hipLaunchKernelGGL(layout_count_kernel<kCountPre>, dim3(m.nb), dim3(kLayoutThreads), lds,
                           s, idx, T, K, E, P, pmagic, m.tb, ebits, cnt, pcnt, inv, rows, in_part,
                           vec, pre, prank, ppre);
    else
        hipLaunchKernelGGL(layout_count_kernel<kCountPlain>, dim3(m.nb), dim3(kLayoutThreads), lds,
                           s, idx, T, K, E, P, pmagic, m.tb, ebits, cnt, pcnt, inv, rows, in_part,
                           vec, pre, prank, ppre);
    return hipGetLastError();
}

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
    const int ebits = expert_bits(E);
    const int Ep = E / P;
    const uint64_t pmagic = partition_magic(Ep);
    int* rows = reinterpret_cast<int*>(base + m.rows_off);
    const int vec_rows = vector_rows(P, in_part);

    const size_t fused_lds = layout_fused_lds_bytes(T, K, E, P);
    if (layout_single_launch(T, K, E, P, m)) {
        if (fused_lds > 64 * 1024) {
            hipError_t e = allow_large_lds(reinterpret_cast<const void*>(layout_fused_kernel),
                                           kFusedLdsSlot, kLdsCap);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(layout_fused_kernel, dim3(m.nb), dim3(kLayoutThreads), fused_lds, s,
                           idx, T, K, E, P, Ep, pmagic, m.tb, ebits, rows, in_part, vec_rows, hdr,
                           cnt_e, cnt_p, off_e, off_p);
        return hipGetLastError();
    }

    hipError_t err = launch_layout_count(idx, T, K, E, P, ws, m, in_part, kCountPlain, s);
    if (err != hipSuccess) return err;
    int* cnt = reinterpret_cast<int*>(base + m.cnt_off);
    int* pcnt = reinterpret_cast<int*>(base + m.pcnt_off);
    int* inv = reinterpret_cast<int*>(base + m.inv_off);
    const size_t lds2 = sizeof(int) * 3 * (size_t)E;
    hipLaunchKernelGGL(layout_finalize_kernel, dim3(m.nb), dim3(kLayoutThreads), lds2, s, T, K, E,
                       P, E / P, m.tb, m.nb, cnt, pcnt, inv, rows, hdr, cnt_e, cnt_p, off_e,
                       off_p, 1, nullptr, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_layout_aligned(const int64_t* idx, int T, int K, int E, int P, int align,
                                 void* ws, const WsMap& m, int32_t* cnt_e, int32_t* cnt_p,
                                 uint8_t* in_part, int32_t* off_e, int32_t* off_p,
                                 int32_t* recv_src, int64_t R, hipStream_t s) {
    char* base = static_cast<char*>(ws);
    WsHeader* hdr = reinterpret_cast<WsHeader*>(base);
    if (T == 0) {
        hipLaunchKernelGGL(layout_empty_kernel, dim3(1), dim3(256), 0, s, E, P, hdr, cnt_e,
                           cnt_p, off_e, off_p);
        if (R > 0) {
            const int64_t blocks = (R + 255) / 256 < 1024 ? (R + 255) / 256 : 1024;
            hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                               recv_src, R, -1);
        }
        return hipGetLastError();
    }
    hipError_t err = launch_layout_count(idx, T, K, E, P, ws, m, in_part, kCountPlain, s);
    if (err != hipSuccess) return err;
    int* rows = reinterpret_cast<int*>(base + m.rows_off);
    int* cnt = reinterpret_cast<int*>(base + m.cnt_off);
    int* pcnt = reinterpret_cast<int*>(base + m.pcnt_off);
    int* inv = reinterpret_cast<int*>(base + m.inv_off);
    const size_t lds2 = sizeof(int) * 3 * (size_t)E;
    hipLaunchKernelGGL(layout_finalize_kernel, dim3(m.nb), dim3(kLayoutThreads), lds2, s, T, K, E,
                       P, E / P, m.tb, m.nb, cnt, pcnt, inv, rows, hdr, cnt_e, cnt_p, off_e,
                       off_p, align, recv_src, R);
    return hipGetLastError();
}

}  // namespace ep
