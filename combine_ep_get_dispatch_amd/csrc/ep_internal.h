// Internal interface between the C-ABI entry points (ep_api.hip) and the
// gfx950 kernels.  Not installed; the public interface is include/ep.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

// Alignment of every dynamic-LDS array (extern __shared__).  The dynamic area
// follows a kernel's static LDS, which may end at any 4-byte boundary; the
// attribute makes the compiler pad the static part so that the dynamic base
// is 16-byte aligned.  Views carved out of a dynamic array may then use LDS
// accesses up to 16 bytes wide, provided their offsets are multiples of their
// access width; an 8- or 16-byte access to a less aligned LDS address faults.
#define EP_LDS_ALIGN __attribute__((aligned(16)))

// CU budget: the *_cu entry points launch at most num_cus workgroups of this
// size (or the kernel's own size) that loop over their work, so that the
// hardware places them on at most num_cus CUs.
constexpr int kBudgetThreads = 1024;
// Tokens a CU-budget dispatch workgroup carries at once (at most).
constexpr int kBudgetGroups = 4;

// ---------------------------------------------------------------- layout ---
// The layout kernels give each workgroup one block of consecutive tokens
// holding about kLayoutEntries (token, slot) entries and 16 waves (the
// ranking is a chain of LDS round trips per 64-entry chunk, so more waves
// with fewer chunks each finish sooner: 16 measured 0.5 us faster than 8 at
// 4096 x 8; the count launch ranks with 12 of them, three chunks each at
// K = 8, while the other 4 write the partition rows).
constexpr int kLayoutThreads = 1024;
constexpr int kLayoutWaves = kLayoutThreads / 64;
constexpr int kLayoutEntries = 2048;

// Dynamic LDS the single-launch layout may use (gfx950 gives a workgroup up to
// 160 KiB; a little is left for the kernel's static LDS).
constexpr size_t kFusedLdsLimit = 156 * 1024;

// A launch asking for more than 64 KiB of dynamic LDS first raises the
// kernel's cap (hipFuncAttributeMaxDynamicSharedMemorySize) to `bytes` on the
// current device, once per (slot, device); each kernel has its own slot.
constexpr int kFusedLdsSlot = 0;
constexpr int kCountLdsSlot = 1;          // + count mode (3 slots)
constexpr int kCombineTileLdsSlot = 4;
constexpr int kLdsSlots = 5;
hipError_t allow_large_lds(const void* fn, int slot, int bytes);
// ... and only for inputs of at most this many token blocks.
constexpr int kFusedMaxBlocks = 2;

// Packed slot after the count launch: (expert << kRankBits) | rank in block.
constexpr int kRankBits = 12;     // rank inside a block < kLayoutEntries = 2^11
static_assert(kLayoutEntries <= (1 << kRankBits), "rank field too narrow");

__host__ __device__ inline int layout_tokens_per_block(int K) {
    int tb = kLayoutEntries / K;
    return tb < 1 ? 1 : tb;
}

// First 256 bytes of the caller's workspace, written by every layout call.
struct WsHeader {
    int32_t num_valid;     // N = valid slots of the last layout
    int32_t pad;
    int64_t num_invalid;   // invalid slots of the last layout
};
constexpr size_t kWsHeaderBytes = 256;
static_assert(sizeof(WsHeader) <= kWsHeaderBytes, "header too large");

// Workspace map for one shape (offsets in bytes from the workspace start):
//   [0, 256)           WsHeader
//   cnt  int32 [nb][E] per-block expert counts
//   pcnt int32 [nb][P] per-block distinct-token counts per partition
//   inv  int32 [nb]    per-block invalid-slot counts
//   pre  int32 [nb][E+1] per-block exclusive prefix of the expert counts over
//                      the experts, pre[b][E] = the block's valid slots
//                      (written only by the one-call and de-duplicated paths)
//   ppre int32 [nb][P+1] per-block exclusive prefix of the partition token
//                      counts over the partitions (de-duplicated path)
//   prank int32 [T*K]  each slot's rank among its block's member tokens of
//                      the slot's partition (de-duplicated path)
//   rows int32 [T*K]   receive row of every slot (-1 if masked/invalid); the
//                      count kernel leaves (expert << 12 | rank in block)
//                      there and the finalize kernel turns it into the row
struct WsMap {
    int nb = 0;        // token blocks
    int tb = 1;        // tokens per block
    size_t cnt_off = 0, pcnt_off = 0, inv_off = 0, pre_off = 0, ppre_off = 0, prank_off = 0;
    size_t rows_off = 0, total = 0;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline WsMap ws_map(int T, int K, int E, int P) {
    WsMap m;
    m.tb = layout_tokens_per_block(K);
    m.nb = (T + m.tb - 1) / m.tb;
    m.cnt_off = kWsHeaderBytes;
    m.pcnt_off = m.cnt_off + align256(sizeof(int32_t) * (size_t)E * (size_t)m.nb);
    m.inv_off = m.pcnt_off + align256(sizeof(int32_t) * (size_t)P * (size_t)m.nb);
    m.pre_off = m.inv_off + align256(sizeof(int32_t) * (size_t)m.nb);
    m.ppre_off = m.pre_off + align256(sizeof(int32_t) * (size_t)(E + 1) * (size_t)m.nb);
    m.prank_off = m.ppre_off + align256(sizeof(int32_t) * (size_t)(P + 1) * (size_t)m.nb);
    m.rows_off = m.prank_off + align256(sizeof(int32_t) * (size_t)T * (size_t)K);
    m.total = m.rows_off + align256(sizeof(int32_t) * (size_t)T * (size_t)K);
    return m;
}

// LDS the single-launch layout needs for this shape (it is used when this
// fits in kFusedLdsLimit; larger inputs take the two-launch form).
size_t layout_fused_lds_bytes(int T, int K, int E, int P);

hipError_t launch_layout(const int64_t* idx, int T, int K, int E, int P, void* ws,
                         const WsMap& m, int32_t* cnt_e, int32_t* cnt_p, uint8_t* in_part,
                         int32_t* off_e, int32_t* off_p, hipStream_t s);

// The two-launch layout with every expert's run padded to a multiple of
// align rows (expert_offsets are the padded ones, num_valid in the header the
// rows in use); the finalize launch also sets recv_src = -1 on every padding
// row and on rows [used, R).  T = 0 writes zeros and fills recv_src[0, R).
hipError_t launch_layout_aligned(const int64_t* idx, int T, int K, int E, int P, int align,
                                 void* ws, const WsMap& m, int32_t* cnt_e, int32_t* cnt_p,
                                 uint8_t* in_part, int32_t* off_e, int32_t* off_p,
                                 int32_t* recv_src, int64_t R, hipStream_t s);

// True when launch_layout takes its single-launch form for this shape.
bool layout_single_launch(int T, int K, int E, int P, const WsMap& m);

// What the count launch writes besides the per-block counts, partition rows
// and counts, invalid counts and packed (expert << 12 | rank) slots:
// kCountPlain nothing more; kCountPre each block's prefix of its expert
// counts; kCountDedup also every slot's in-block rank among its partition's
// member tokens and each block's prefix of its partition counts.
constexpr int kCountPlain = 0;
constexpr int kCountPre = 1;
constexpr int kCountDedup = 2;

// The first of the two layout launches alone (T > 0), in one of the modes above.
hipError_t launch_layout_count(const int64_t* idx, int T, int K, int E, int P, void* ws,
                               const WsMap& m, uint8_t* in_part, int mode, hipStream_t s);

// ---------------------------------------------------------------- dispatch --
// One workgroup per token, one wave per chunk of the row, at most 16 waves;
// wider rows loop over their chunks.  FP8: 1024-channel chunks (16 channels
// per lane); bf16: 512-channel chunks (8 channels per lane).
constexpr int kDispatchMaxThreads = 1024;
constexpr int kDispatchChunk = 1024;
constexpr int kDispatchChunkBf16 = 512;
__host__ __device__ constexpr int dispatch_chunk(bool fp8) {
    return fp8 ? kDispatchChunk : kDispatchChunkBf16;
}

// num_cus > 0 (and < T): the CU-budget form, num_cus workgroups looping over
// the tokens; otherwise one workgroup per token.  nrows: receive rows (T*K,
// or more for an aligned layout); a workspace row outside it is dropped.
hipError_t launch_dispatch(const uint16_t* x, int T, int H, int K, bool fp8, void* recv_x,
                           float* recv_scales, int32_t* recv_src, int32_t* dst_row,
                           const void* ws, const WsMap& m, int num_cus, int nrows,
                           hipStream_t s);

// Largest (E + 1) * blocks that workgroup 0 of the one-call layout + dispatch
// sums (beyond it the call takes the two-step form).
constexpr int64_t kLayoutDispatchMaxTerms = 32768;

// Layout and dispatch in one call: the count launch (with the prefix matrix),
// then one dispatch launch whose workgroups finish the layout themselves --
// each token's rows from sums over the blocks, workgroup 0 the counts,
// offsets and header.  Shapes with a single-launch layout run that layout and
// the ordinary dispatch instead.  Same outputs as launch_layout followed by
// launch_dispatch, except that the workspace's per-slot rows are left in
// their packed form.
hipError_t launch_layout_dispatch(const uint16_t* x, const int64_t* idx, int T, int H, int K,
                                  int E, int P, bool fp8, void* ws, const WsMap& m,
                                  int32_t* cnt_e, int32_t* cnt_p, uint8_t* in_part,
                                  int32_t* off_e, int32_t* off_p, void* recv_x,
                                  float* recv_scales, int32_t* recv_src, int32_t* dst_row,
                                  int num_cus, hipStream_t s);

// Fixed-capacity (decode) dispatch: one launch, one or more workgroups per
// token (T = 0 takes a small fill kernel instead) of kLlWaves waves; the
// routing scan that every workgroup does takes few rounds of loads
// (kLlScanUnroll in flight per thread: one round up to 2048 slots), and
// waves past the workgroup's channel chunks only take part in the scan.
// Eight waves rather than sixteen start sooner and scan sooner (the kernel
// ended 0.3 us earlier at 128 tokens x 7168, top-8 of 256 experts).  LDS:
// two [E] int histograms.  Both dtypes move 512-channel chunks (FP8 too,
// so that the quantiser of a small batch is spread over more waves).
constexpr int kLlWaves = 8;
constexpr int kLlScanUnroll = 4;
constexpr int kLlChunk = 512;
static_assert(kLlChunk == kDispatchChunkBf16, "the decode kernel loads and stores bf16 chunks");
// Workgroups the decode dispatch aims for (one per CU of MI355X): a batch of
// T < this many tokens splits each token over up to this / T workgroups.
constexpr int kLlTargetWorkgroups = 256;

size_t ll_dispatch_lds_bytes(int E);

hipError_t launch_ll_dispatch(const uint16_t* x, const int64_t* idx, int T, int H, int K, int E,
                              int C, bool fp8, int32_t* cnt_e, void* recv_x, float* recv_scales,
                              int32_t* recv_src, int32_t* dst_row, int64_t* num_invalid,
                              hipStream_t s);

// De-duplicated per-partition dispatch: the count launch in kCountDedup mode,
// then one dispatch launch that finishes both layouts (expert-major slot rows
// and de-duplicated partition rows) and writes one copy of each token per
// partition it reaches.
hipError_t launch_dispatch_dedup(const uint16_t* x, const int64_t* idx, int T, int H, int K,
                                 int E, int P, bool fp8, void* ws, const WsMap& m, int32_t* cnt_e,
                                 int32_t* cnt_p, uint8_t* in_part, int32_t* off_e, int32_t* off_p,
                                 int32_t* ptok_off, void* recv_x, float* recv_scales,
                                 int32_t* recv_src, int32_t* recv_topk_idx, int32_t* slot_src,
                                 int32_t* dst_row, hipStream_t s);

// ---------------------------------------------------------------- combine ---
// One wave per (token, 512-channel chunk); 8 channels per lane; two waves per
// workgroup (measured ~3% faster than 4 or 8 and slightly faster than 1).
constexpr int kCombineThreads = 128;
constexpr int kCombineChunk = 512;
// Tiled form for large top-8 batches: workgroups of 16 waves, each owning a
// tile of consecutive tokens whose outputs (at most kCombineTileLds bytes,
// one workgroup per CU) are staged in LDS and written as one burst; used
// while the batch gives every CU of a 256-CU part at least two tiles.  (Two
// workgroups per CU, with 72 or 56 KiB tiles, or 8 waves measured slower or
// no faster.)
constexpr int kCombineTileK = 8;
constexpr int kCombineTileThreads = 1024;
constexpr size_t kCombineTileLds = 112 * 1024;
constexpr int kCombineTileMinBlocks = 512;

// num_cus > 0: the CU-budget form (at most num_cus workgroups of
// kBudgetThreads striding over the tasks); otherwise the ordinary launch.
hipError_t launch_combine(const uint16_t* y, int64_t nrows, const int32_t* dst_row,
                          const float* w, int T, int K, int H, uint16_t* out, int num_cus,
                          hipStream_t s);

// ------------------------------------------------------------ diagnostics ---
hipError_t launch_convert_e4m3(const float* in, uint8_t* out, int64_t n, int mode, hipStream_t s);
hipError_t launch_convert_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

}  // namespace ep
