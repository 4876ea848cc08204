/*
 * ep.h -- C ABI of the MoE token dispatch / combine library for AMD MI355X
 * (gfx950, CDNA4).  Built as libep_mi355x.so from hand-written HIP kernels.
 *
 * The operations.  In expert parallelism every token is sent to the experts
 * its router picked ("dispatch") and the experts' outputs are brought back to
 * the token ("combine"); the two form an all-to-all exchange between the GPUs
 * that host the experts ("DeepSeek releases DeepEP, an efficient communication
 * library for MoE models", section "DeepEP: Optimizing MoE Communication").
 * Dispatch may carry FP8 payloads (FP8 for dispatch is in the feature list of
 * "DeepSeek Open Source Weekly Review - 2").  This library computes one GPU's
 * share of that exchange with the destination partitions laid out as
 * contiguous runs of one local receive buffer, so that partition p's rows are
 * exactly what would be sent to GPU p.
 *
 * Notation: T tokens, H hidden size, K router slots per token (top-k),
 * E experts, P destination partitions (E % P == 0; expert e belongs to
 * partition e / (E/P)), G = H/128 scale groups, R = T*K receive rows.
 *
 * Conventions shared by every entry point:
 *  - Array arguments are device pointers on the current HIP device, row-major
 *    and contiguous, owned by the caller.  The library never allocates or
 *    frees memory.  Its only device state is the static scratch array of
 *    ep_layout_dispatch_static (one per GPU); every other call works in the
 *    caller's workspace.  Its host-side globals are a per-device flag, set
 *    once and thread-safe, recording that a kernel's larger dynamic-LDS
 *    limit has been raised, and the per-device address of that scratch.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously; nothing synchronises except
 *    ep_get_device_error.
 *  - Arguments are validated on the host; on any error the call returns a
 *    non-zero ep_status_t and enqueues nothing.  EP_ERR_HIP reports a failed
 *    launch (hipGetLastError after the launch).
 *  - Buffers must not overlap.  x, recv_x, y and out must be 16-byte aligned.
 *  - topk_idx entries: a value in [0, E) selects that expert; -1 is a masked
 *    slot (skipped everywhere); any other value is an invalid slot: it is
 *    skipped like a masked one and counted in the workspace's error word
 *    (see ep_get_device_error).
 */
#ifndef EP_MI355X_H
#define EP_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the two enums get int32_t as their fixed underlying type, so that
 * every int a C caller passes (an unknown status code, a bad dtype that the
 * call must reject) is a valid value of the parameter's type; the size and
 * the calling convention are those of the C enums. */
#ifdef __cplusplus
#define EP_ENUM_BASE : int32_t
#else
#define EP_ENUM_BASE
#endif

typedef enum EP_ENUM_BASE {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = 1,  /* null pointer, bad size or inconsistent shape */
    EP_ERR_UNSUPPORTED = 2,  /* valid but outside the library's limits     */
    EP_ERR_WORKSPACE = 3,    /* workspace smaller than ep_workspace_bytes() */
    EP_ERR_HIP = 4           /* a HIP call or kernel launch failed          */
} ep_status_t;

typedef enum EP_ENUM_BASE {
    EP_DTYPE_BF16 = 0,       /* receive rows are bf16 copies of the tokens  */
    EP_DTYPE_FP8_E4M3 = 1    /* receive rows are OCP E4M3 codes + scales    */
} ep_dtype_t;

/* Limits of the library (EP_ERR_UNSUPPORTED beyond them). */
#define EP_MAX_EXPERTS 1024
#define EP_MAX_TOPK 64
#define EP_LL_MAX_SLOTS 8192   /* T*K of one ep_low_latency_dispatch call */
#define EP_MAX_EXPERT_ALIGNMENT 1024   /* of ep_layout_dispatch_aligned */
#define EP_STATIC_SCRATCH_BYTES (8u << 20)   /* per GPU, of ep_layout_dispatch_static */

/*
 * Bytes of device workspace that ep_get_dispatch_layout and ep_dispatch need
 * for this shape; 0 if the shape is invalid.  The workspace needs no
 * initialisation: ep_get_dispatch_layout writes everything ep_dispatch and
 * ep_get_device_error read from it.  A workspace may be reused for any shape
 * it is large enough for; one workspace serves one layout -> dispatch
 * sequence at a time.
 */
size_t ep_workspace_bytes(int32_t num_tokens, int32_t num_topk, int32_t num_experts,
                          int32_t num_partitions);

/*
 * Dispatch layout: the counts and offsets that the all-to-all needs before
 * any data moves (the bookkeeping behind the exchange of "DeepEP: Optimizing
 * MoE Communication"; the pages do not spell it out, the definitions below
 * are this library's):
 *   num_tokens_per_expert    [E]   valid slots routed to expert e
 *   num_tokens_per_partition [P]   distinct tokens with a valid slot in p
 *   is_token_in_partition  [T*P]   uint8, 1 iff token t has a valid slot in p
 *   expert_offsets         [E+1]   exclusive prefix sum of the expert counts;
 *                                  expert_offsets[E] = N = number of valid slots
 *   partition_offsets      [P+1]   expert_offsets[p * (E/P)]: partition p owns
 *                                  receive rows [partition_offsets[p],
 *                                  partition_offsets[p+1])
 * It also records, in the workspace, the receive row of every slot (see
 * ep_dispatch), which ep_dispatch then uses.  topk_idx is int64 [T*K].
 * T may be 0 (all counts and offsets become 0).
 */
ep_status_t ep_get_dispatch_layout(const int64_t *topk_idx, int32_t num_tokens,
                                   int32_t num_topk, int32_t num_experts,
                                   int32_t num_partitions,
                                   int32_t *num_tokens_per_expert,
                                   int32_t *num_tokens_per_partition,
                                   uint8_t *is_token_in_partition,
                                   int32_t *expert_offsets, int32_t *partition_offsets,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dispatch (the "dispatch" half of "DeepEP: Optimizing MoE Communication"):
 * every valid slot (t,k) gets its own receive row
 *   dst_row[t*K+k] = expert_offsets[e] + (rank of (t,k) among the slots of
 *                    expert e, in token-major then slot order),  e = topk_idx
 * or -1 for a masked/invalid slot, and recv_src_token[dst_row] = t; receive
 * rows r >= N get recv_src_token[r] = -1 and their recv_x/recv_scales rows are
 * left untouched.  (A row the workspace would place outside [0, R) -- only
 * possible when the workspace does not come from the matching layout call --
 * is dropped and its slot reported as -1, so no write leaves the buffers.)
 * Rows are therefore grouped by expert in ascending order and partition p's
 * rows are one contiguous run.
 *   out_dtype == EP_DTYPE_BF16:  recv_x is bf16 [R*H], row r a bitwise copy of
 *     x[recv_src_token[r]]; recv_scales is ignored (may be NULL).
 *   out_dtype == EP_DTYPE_FP8_E4M3 (H % 128 == 0): for each token and each
 *     group of 128 consecutive channels, a = max|x|, a_c = max(a, 1e-4f),
 *     s = a_c / 448 and the codes are E4M3(x * (448 / a_c)) (OCP E4M3, round
 *     to nearest even, saturating, sign kept); recv_x is uint8 [R*H] and
 *     recv_scales fp32 [R*G] holds s, so x ~= code * s.  (FP8 for dispatch:
 *     feature list of "DeepSeek Open Source Weekly Review - 2"; the format,
 *     granularity and scale rule are this library's.)  Non-finite x: a NaN
 *     takes no part in the maximum a; an infinity makes s = +inf and 448/a_c
 *     = 0, so the group's finite values get signed-zero codes; every infinite
 *     or NaN x gets the code S.1111.111 (0x7F / 0xFF) with the sign of x.
 * x is bf16 [T*H]; topk_idx int64 [T*K] and workspace must be the ones the
 * preceding ep_get_dispatch_layout call used, with the same T, K, E, P and on
 * the same stream (or ordered after it).  H % 8 == 0.
 */
ep_status_t ep_dispatch(const void *x, int32_t num_tokens, int32_t hidden,
                        const int64_t *topk_idx, int32_t num_topk, int32_t num_experts,
                        int32_t num_partitions, ep_dtype_t out_dtype,
                        void *recv_x, float *recv_scales, int32_t *recv_src_token,
                        int32_t *dst_row, const void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * Layout and dispatch in one call: exactly the outputs of
 * ep_get_dispatch_layout followed by ep_dispatch with the same arguments
 * (every argument has the meaning given there), computed with one kernel
 * launch fewer -- the dispatch kernel finishes the layout itself, so the
 * counts, offsets and the header are written by the same launch that moves
 * the rows.  The workspace afterwards serves ep_get_device_error, but not a
 * later ep_dispatch (its per-slot rows are left in an intermediate form).
 */
ep_status_t ep_layout_dispatch(const void *x, int32_t num_tokens, int32_t hidden,
                               const int64_t *topk_idx, int32_t num_topk, int32_t num_experts,
                               int32_t num_partitions, ep_dtype_t out_dtype,
                               int32_t *num_tokens_per_expert,
                               int32_t *num_tokens_per_partition,
                               uint8_t *is_token_in_partition, int32_t *expert_offsets,
                               int32_t *partition_offsets, void *recv_x, float *recv_scales,
                               int32_t *recv_src_token, int32_t *dst_row, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * ep_layout_dispatch for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments (minus the workspace), same checks, kernels and
 * outputs as ep_layout_dispatch; the workspace is instead a static device
 * array inside the library, EP_STATIC_SCRATCH_BYTES on every GPU that the
 * library runs on, held until the process ends.  Nothing is allocated; the
 * caller passes every input and output.  The first call on a device looks up
 * that device's copy of the array (hipGetSymbolAddress) and keeps its address.
 *   EP_ERR_UNSUPPORTED when ep_workspace_bytes(T, K, E, P) exceeds
 *   EP_STATIC_SCRATCH_BYTES (about T*K <= 1M slots at E <= 256), or when the
 *   current device's index is 64 or more.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap on one GPU (on different streams without
 * ordering between them, or from host threads that do not order them) race
 * and give undefined results; order them on one stream or with events.  The
 * invalid-id count of a call stays in the array and is not reported
 * (ep_layout_dispatch with a workspace and ep_get_device_error report it).
 */
ep_status_t ep_layout_dispatch_static(const void *x, int32_t num_tokens, int32_t hidden,
                                      const int64_t *topk_idx, int32_t num_topk,
                                      int32_t num_experts, int32_t num_partitions,
                                      ep_dtype_t out_dtype, int32_t *num_tokens_per_expert,
                                      int32_t *num_tokens_per_partition,
                                      uint8_t *is_token_in_partition, int32_t *expert_offsets,
                                      int32_t *partition_offsets, void *recv_x,
                                      float *recv_scales, int32_t *recv_src_token,
                                      int32_t *dst_row, void *stream);

/*
 * Receive rows of ep_layout_dispatch_aligned: T*K + E*(expert_alignment-1),
 * enough for any routing; 0 for a shape that call rejects.
 */
int64_t ep_aligned_rows(int32_t num_tokens, int32_t num_topk, int32_t num_experts,
                        int32_t expert_alignment);

/*
 * Layout and dispatch with every expert's run of receive rows padded to a
 * multiple of A = expert_alignment rows: the input form of a grouped expert
 * GEMM whose row tiles must not straddle two experts.  The pages give no
 * receive layout at all (their normal kernels serve training and prefill:
 * "DeepSeek releases DeepEP, an efficient communication library for MoE
 * models", section "Technical Details"); the padding is this library's
 * reading:
 *   expert_offsets[0] = 0,
 *   expert_offsets[e+1] = expert_offsets[e] + ceil(cnt_e / A) * A,
 *   partition_offsets[p] = expert_offsets[p * E/P];
 *   num_tokens_per_expert (unpadded), num_tokens_per_partition and
 *   is_token_in_partition as ep_get_dispatch_layout writes them;
 *   dst_row[t*K+k] = expert_offsets[e] + (rank of (t,k) among expert e's
 *   valid slots, token-major then slot order), -1 for masked/invalid slots;
 *   recv_src_token [R] (R = ep_aligned_rows(T, K, E, A)): the source token of
 *   each row holding one, -1 on the padding rows expert_offsets[e] + cnt_e ..
 *   expert_offsets[e+1] - 1 and on every row >= expert_offsets[E];
 *   recv_x [R*H] (bf16, or uint8 E4M3 codes) and recv_scales [R*G]: the rows
 *   holding a token exactly as ep_dispatch writes them (same copy, same
 *   quantiser); padding and unused rows are left untouched.
 * A = 1 gives exactly the outputs of ep_layout_dispatch.  ep_combine takes the
 * result unchanged with num_rows = R and y laid out like the receive rows.
 * Other arguments, conditions and errors as ep_layout_dispatch; in addition
 * 1 <= A <= EP_MAX_EXPERT_ALIGNMENT and R < 2^31 (else EP_ERR_INVALID_ARG).
 * Three launches on `stream`: the count launch, one that finishes the layout
 * and marks the padding rows, and the dispatch.  The workspace
 * (ep_workspace_bytes(T, K, E, P) bytes) afterwards serves
 * ep_get_device_error.  T may be 0 (counts 0, every row -1).
 */
ep_status_t ep_layout_dispatch_aligned(const void *x, int32_t num_tokens, int32_t hidden,
                                       const int64_t *topk_idx, int32_t num_topk,
                                       int32_t num_experts, int32_t num_partitions,
                                       int32_t expert_alignment, ep_dtype_t out_dtype,
                                       int32_t *num_tokens_per_expert,
                                       int32_t *num_tokens_per_partition,
                                       uint8_t *is_token_in_partition, int32_t *expert_offsets,
                                       int32_t *partition_offsets, void *recv_x,
                                       float *recv_scales, int32_t *recv_src_token,
                                       int32_t *dst_row, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * De-duplicated dispatch: one copy of a token per destination partition
 * instead of one per selected expert -- what goes to the same destination is
 * merged before it is sent ("DeepSeek Open Source Week: A carnival of
 * technology inclusion, the magic of improving the efficiency of large
 * models", section 4), and group-limited gating keeps the destinations per
 * token few ("DeepSeek releases DeepEP, an efficient communication library
 * for MoE models", section "DeepEP: Optimizing MoE Communication").  The
 * layout is this library's (the pages give none).  Kp = min(K, P),
 * RD = T * Kp rows (an upper bound on the rows used).
 *   The five layout outputs as in ep_get_dispatch_layout, and
 *   partition_token_offsets [P+1]: exclusive prefix of
 *     num_tokens_per_partition; partition p's rows are
 *     [partition_token_offsets[p], partition_token_offsets[p+1]), one per
 *     token with a valid slot in p, in token order; ND = offsets[P] rows used.
 *   recv_x [RD*H] (bf16, or E4M3 codes with recv_scales [RD*G] as in
 *     ep_dispatch): row r holds token recv_src_token[r]; rows >= ND are not
 *     written and get recv_src_token = -1.
 *   recv_topk_idx [RD*K] int32: for row r of (t, p) and each slot k of t, the
 *     local expert id e - p*(E/P) if slot k's expert e is in p, else -1 (all
 *     -1 for rows >= ND): the per-row local-expert selection.
 *   dst_row [T*K]: every valid slot's expert-major row, exactly as
 *     ep_dispatch numbers them (only an index here: no data is written there).
 *   slot_src_row [T*K] int32: for every expert-major row r, the
 *     de-duplicated row holding its token (-1 for r >= N), so expert e's
 *     inputs are the rows slot_src_row[expert_offsets[e] ..
 *     expert_offsets[e+1]) -- the per-partition local permutation.
 * ep_combine then runs unchanged on expert outputs y [T*K, H] in expert-major
 * order with dst_row.  Two kernel launches; the workspace is sized by
 * ep_workspace_bytes and afterwards serves ep_get_device_error (not a later
 * ep_dispatch).
 */
ep_status_t ep_dispatch_dedup(const void *x, int32_t num_tokens, int32_t hidden,
                              const int64_t *topk_idx, int32_t num_topk, int32_t num_experts,
                              int32_t num_partitions, ep_dtype_t out_dtype,
                              int32_t *num_tokens_per_expert, int32_t *num_tokens_per_partition,
                              uint8_t *is_token_in_partition, int32_t *expert_offsets,
                              int32_t *partition_offsets, int32_t *partition_token_offsets,
                              void *recv_x, float *recv_scales, int32_t *recv_src_token,
                              int32_t *recv_topk_idx, int32_t *slot_src_row, int32_t *dst_row,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Combine (the "combine" half of "DeepEP: Optimizing MoE Communication"):
 * bring each token's expert outputs back and reduce them with its gate
 * weights.  For every token t and channel h:
 *   acc = +0.0f;  for k = 0..K-1 with 0 <= dst_row[t*K+k] < num_rows:
 *       acc = fmaf(topk_weights[t*K+k], y[dst_row[t*K+k]*H + h], acc)
 *   out[t*H + h] = bf16(acc), rounded to nearest even.
 * y is bf16 [num_rows * H] (normally num_rows = T*K, the receive rows in
 * dispatch's order); dst_row int32 [T*K] as written by ep_dispatch; slots
 * whose dst_row lies outside [0, num_rows) are skipped like masked ones, so
 * no y row outside the buffer is ever read.  topk_weights fp32 [T*K]; out
 * bf16 [T*H].  H % 8 == 0.  T may be 0.  (The weighting and the fp32
 * accumulation order are this library's reading; the pages only name the
 * operation.)  y and topk_weights are expected finite: with an infinity or a
 * NaN the result is the IEEE result of the same chain (NaN, +-inf), with the
 * sign and payload of a NaN unspecified.
 */
ep_status_t ep_combine(const void *y, int64_t num_rows, const int32_t *dst_row,
                       const float *topk_weights, int32_t num_tokens, int32_t num_topk,
                       int32_t hidden, void *out, void *stream);

/*
 * Decode dispatch into fixed-capacity receive buffers, in a single kernel
 * launch.  Besides its throughput kernels the library family serves
 * inference decoding with kernels built for small batches and the lowest
 * latency ("DeepSeek releases DeepEP, an efficient communication library for
 * MoE models", section "Technical Details"; the 128-token, top-8 decode case
 * is in "Deepseek Ai Deepep: A library for an open-open EP for example
 * training", section "Technological Views and Benefits").  The pages give no
 * buffer layout for it; this library's is a fixed capacity C per expert, so
 * no receive row depends on a prefix sum over the experts and nothing has to
 * wait for one:
 *   expert e owns receive rows [e*C, (e+1)*C) (partition p, holding experts
 *   [p*E/P, (p+1)*E/P), owns the contiguous rows [p*(E/P)*C, (p+1)*(E/P)*C));
 *   a valid slot (t,k) of expert e whose rank among expert e's valid slots,
 *   in token-major then slot order, is r gets
 *     dst_row[t*K+k] = e*C + r   if r < C,
 *   and is dropped (dst_row = -1) if r >= C; masked and invalid slots get -1.
 *   num_tokens_per_expert [E] counts all valid slots of e, dropped ones
 *   included, so rows e*C .. e*C + min(count, C) - 1 are filled and
 *   count > C reports drops (C >= T can drop nothing unless a token repeats
 *   an expert).
 *   recv_src_token [E*C]: the source token of each filled row, -1 elsewhere.
 *   recv_x [E*C*H] (bf16, or uint8 E4M3 codes) and recv_scales [E*C*G] hold
 *   the filled rows exactly as ep_dispatch writes them (same copy and same
 *   quantiser); unfilled rows are left untouched.
 *   num_invalid: device pointer to one int64 that receives the number of
 *   invalid topk_idx entries (not -1 and outside [0, E)), or NULL.
 * ep_combine runs on the result unchanged, with y [E*C, H] laid out like the
 * receive rows and num_rows = E*C.  Every output is written by this one
 * launch; no workspace, no initialisation, no host synchronisation.
 * x bf16 [T*H], topk_idx int64 [T*K]; H % 8 == 0 (H % 128 == 0 for FP8);
 * capacity >= 1; E*C < 2^31.  T may be 0 (counts 0, every row -1).
 * EP_ERR_UNSUPPORTED when T*K > EP_LL_MAX_SLOTS (every workgroup reads the
 * whole routing tensor: use ep_get_dispatch_layout + ep_dispatch for large
 * batches), E > EP_MAX_EXPERTS or K > EP_MAX_TOPK.
 */
ep_status_t ep_low_latency_dispatch(const void *x, int32_t num_tokens, int32_t hidden,
                                    const int64_t *topk_idx, int32_t num_topk,
                                    int32_t num_experts, int32_t capacity,
                                    ep_dtype_t out_dtype, int32_t *num_tokens_per_expert,
                                    void *recv_x, float *recv_scales, int32_t *recv_src_token,
                                    int32_t *dst_row, int64_t *num_invalid, void *stream);

/*
 * CU budget: ep_layout_dispatch and ep_combine confined to at most num_cus
 * compute units, so that they can run beside other kernels (expert GEMMs)
 * on the same GPU -- the pages' "flexible GPU resource control" for
 * overlapping communication with computation ("DeepSeek releases DeepEP, an
 * efficient communication library for MoE models", feature list; users
 * choose the number of SMs the kernels use, "Deepseek Ai Deepep: A library
 * for an open-open EP for example training", section "Technological Views
 * and Benefits").  The dispatch launch (and combine) then runs as at most
 * num_cus workgroups that loop over the tokens (tasks); the hardware places
 * them on at most num_cus CUs.  Results are identical to the calls without
 * a budget; num_cus = 0 means no budget; num_cus < 0 is EP_ERR_INVALID_ARG.
 * The count launch of ep_layout_dispatch_cu already uses only
 * ceil(T / (2048 / K)) workgroups.
 */
ep_status_t ep_layout_dispatch_cu(const void *x, int32_t num_tokens, int32_t hidden,
                                  const int64_t *topk_idx, int32_t num_topk, int32_t num_experts,
                                  int32_t num_partitions, ep_dtype_t out_dtype,
                                  int32_t *num_tokens_per_expert,
                                  int32_t *num_tokens_per_partition,
                                  uint8_t *is_token_in_partition, int32_t *expert_offsets,
                                  int32_t *partition_offsets, void *recv_x, float *recv_scales,
                                  int32_t *recv_src_token, int32_t *dst_row, void *workspace,
                                  size_t workspace_bytes, int32_t num_cus, void *stream);

ep_status_t ep_combine_cu(const void *y, int64_t num_rows, const int32_t *dst_row,
                          const float *topk_weights, int32_t num_tokens, int32_t num_topk,
                          int32_t hidden, void *out, int32_t num_cus, void *stream);

/*
 * Waits for `stream`, then stores in *num_invalid the number of invalid
 * topk_idx entries (not -1 and outside [0, E)) that the most recent
 * ep_get_dispatch_layout on this workspace met.  num_invalid is a host
 * pointer.
 */
ep_status_t ep_get_device_error(const void *workspace, size_t workspace_bytes,
                                int64_t *num_invalid, void *stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char *ep_status_string(ep_status_t status);

/*
 * Diagnostics and measurement helpers.  They run the same device code as the
 * path above, so tests can check it value by value and benchmarks can
 * calibrate counters against a kernel of known traffic.
 */

/* out[i] = E4M3 code of in[i], with the conversion ep_dispatch uses (mode 0)
 * or the bit-exact software conversion (mode 1).  in fp32 [n], out uint8 [n]. */
ep_status_t ep_convert_e4m3(const float *in, uint8_t *out, int64_t n, int32_t mode,
                            void *stream);

/* out[i] = bf16 bits of in[i], rounded to nearest even, with the conversion
 * ep_combine uses.  in fp32 [n], out uint16 [n]. */
ep_status_t ep_convert_bf16(const float *in, uint16_t *out, int64_t n, void *stream);

/* Streaming copy of `bytes` bytes (multiple of 16, 16-byte aligned pointers,
 * non-overlapping): reads `bytes` and writes `bytes`, each wave moving whole
 * 4 KiB spans with non-temporal 16-byte loads and stores.  Used as the
 * reference kernel for HBM traffic counters and as the measured copy
 * ceiling. */
ep_status_t ep_copy(const void *src, void *dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_H */
