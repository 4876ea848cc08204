// C-ABI entry points (include/ep.h): host-side validation, workspace sizing
// and kernel launches.  Nothing here touches the device before validation
// has passed, and nothing here allocates.
#include "ep.h"
#include "ep_internal.h"

#include <atomic>
#include <mutex>

// Device scratch of ep_layout_dispatch_static: the workspace of callers that
// cannot allocate.  Every GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: only the pointer that hipGetSymbolAddress returns for the
// current device may reach a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[EP_STATIC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by the layout and dispatch calls.
ep_status_t check_routing_shape(int32_t T, int32_t K, int32_t E, int32_t P) {
    if (T < 0 || K <= 0 || E <= 0 || P <= 0) return EP_ERR_INVALID_ARG;
    if (E % P != 0 || K > E) return EP_ERR_INVALID_ARG;
    if ((int64_t)T * K >= kMaxRows) return EP_ERR_INVALID_ARG;
    if (E > EP_MAX_EXPERTS || K > EP_MAX_TOPK) return EP_ERR_UNSUPPORTED;
    return EP_OK;
}

ep_status_t from_hip(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

// Address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;

ep_status_t device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return EP_ERR_HIP;
    if (dev < 0 || dev >= kScratchDevices) return EP_ERR_UNSUPPORTED;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return EP_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return EP_OK;
}

}  // namespace

extern "C" {

size_t ep_workspace_bytes(int32_t num_tokens, int32_t num_topk, int32_t num_experts,
                          int32_t num_partitions) {
    if (check_routing_shape(num_tokens, num_topk, num_experts, num_partitions) != EP_OK)
        return 0;
    return ep::ws_map(num_tokens, num_topk, num_experts, num_partitions).total;
}

ep_status_t ep_get_dispatch_layout(const int64_t* topk_idx, int32_t num_tokens,
                                   int32_t num_topk, int32_t num_experts,
                                   int32_t num_partitions, int32_t* num_tokens_per_expert,
                                   int32_t* num_tokens_per_partition,
                                   uint8_t* is_token_in_partition, int32_t* expert_offsets,
                                   int32_t* partition_offsets, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    const int32_t T = num_tokens, K = num_topk, E = num_experts, P = num_partitions;
    ep_status_t st = check_routing_shape(T, K, E, P);
    if (st != EP_OK) return st;
    if (!num_tokens_per_expert || !num_tokens_per_partition || !expert_offsets ||
        !partition_offsets || !workspace)
        return EP_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !is_token_in_partition)) return EP_ERR_INVALID_ARG;
    const ep::WsMap m = ep::ws_map(T, K, E, P);
    if (workspace_bytes < m.total) return EP_ERR_WORKSPACE;
    return from_hip(ep::launch_layout(topk_idx, T, K, E, P, workspace, m, num_tokens_per_expert,
                                      num_tokens_per_partition, is_token_in_partition,
                                      expert_offsets, partition_offsets,
                                      static_cast<hipStream_t>(stream)));
}

ep_status_t ep_dispatch(const void* x, int32_t num_tokens, int32_t hidden,
                        const int64_t* topk_idx, int32_t num_topk, int32_t num_experts,
                        int32_t num_partitions, ep_dtype_t out_dtype, void* recv_x,
                        float* recv_scales, int32_t* recv_src_token, int32_t* dst_row,
                        const void* workspace, size_t workspace_bytes, void* stream) {
    const int32_t T = num_tokens, H = hidden, K = num_topk, E = num_experts, P = num_partitions;
    ep_status_t st = check_routing_shape(T, K, E, P);
    if (st != EP_OK) return st;
    if (out_dtype != EP_DTYPE_BF16 && out_dtype != EP_DTYPE_FP8_E4M3) return EP_ERR_INVALID_ARG;
    const bool fp8 = out_dtype == EP_DTYPE_FP8_E4M3;
    if (H <= 0 || H % 8 != 0 || (fp8 && H % 128 != 0)) return EP_ERR_INVALID_ARG;
    if (!workspace) return EP_ERR_INVALID_ARG;
    if (T > 0) {
        if (!x || !topk_idx || !recv_x || !recv_src_token || !dst_row) return EP_ERR_INVALID_ARG;
        if (fp8 && !recv_scales) return EP_ERR_INVALID_ARG;
        if (!aligned16(x) || !aligned16(recv_x)) return EP_ERR_INVALID_ARG;
    }
    const ep::WsMap m = ep::ws_map(T, K, E, P);
    if (workspace_bytes < m.total) return EP_ERR_WORKSPACE;
    return from_hip(ep::launch_dispatch(static_cast<const uint16_t*>(x), T, H, K, fp8, recv_x,
                                        recv_scales, recv_src_token, dst_row, workspace, m, 0,
                                        T * K, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Argument checks of the one-call layout + dispatch (the workspace apart).
ep_status_t check_layout_dispatch(const void* x, int32_t T, int32_t H, const int64_t* topk_idx,
                                  int32_t K, int32_t E, int32_t P, ep_dtype_t out_dtype,
                                  const int32_t* num_tokens_per_expert,
                                  const int32_t* num_tokens_per_partition,
                                  const uint8_t* is_token_in_partition,
                                  const int32_t* expert_offsets, const int32_t* partition_offsets,
                                  const void* recv_x, const float* recv_scales,
                                  const int32_t* recv_src_token, const int32_t* dst_row) {
    ep_status_t st = check_routing_shape(T, K, E, P);
    if (st != EP_OK) return st;
    if (out_dtype != EP_DTYPE_BF16 && out_dtype != EP_DTYPE_FP8_E4M3) return EP_ERR_INVALID_ARG;
    const bool fp8 = out_dtype == EP_DTYPE_FP8_E4M3;
    if (H <= 0 || H % 8 != 0 || (fp8 && H % 128 != 0)) return EP_ERR_INVALID_ARG;
    if (!num_tokens_per_expert || !num_tokens_per_partition || !expert_offsets ||
        !partition_offsets)
        return EP_ERR_INVALID_ARG;
    if (T > 0) {
        if (!x || !topk_idx || !is_token_in_partition || !recv_x || !recv_src_token || !dst_row)
            return EP_ERR_INVALID_ARG;
        if (fp8 && !recv_scales) return EP_ERR_INVALID_ARG;
        if (!aligned16(x) || !aligned16(recv_x)) return EP_ERR_INVALID_ARG;
    }
    return EP_OK;
}

}  // namespace

extern "C" {

ep_status_t ep_layout_dispatch_cu(const void* x, int32_t num_tokens, int32_t hidden,
                                  const int64_t* topk_idx, int32_t num_topk, int32_t num_experts,
                                  int32_t num_partitions, ep_dtype_t out_dtype,
                                  int32_t* num_tokens_per_expert,
                                  int32_t* num_tokens_per_partition,
                                  uint8_t* is_token_in_partition, int32_t* expert_offsets,
                                  int32_t* partition_offsets, void* recv_x, float* recv_scales,
                                  int32_t* recv_src_token, int32_t* dst_row, void* workspace,
                                  size_t workspace_bytes, int32_t num_cus, void* stream) {
    const int32_t T = num_tokens, H = hidden, K = num_topk, E = num_experts, P = num_partitions;
    ep_status_t st = check_layout_dispatch(x, T, H, topk_idx, K, E, P, out_dtype,
                                           num_tokens_per_expert, num_tokens_per_partition,
                                           is_token_in_partition, expert_offsets,
                                           partition_offsets, recv_x, recv_scales,
                                           recv_src_token, dst_row);
    if (st != EP_OK) return st;
    if (!workspace || num_cus < 0) return EP_ERR_INVALID_ARG;
    const bool fp8 = out_dtype == EP_DTYPE_FP8_E4M3;
    const ep::WsMap m = ep::ws_map(T, K, E, P);
    if (workspace_bytes < m.total) return EP_ERR_WORKSPACE;
    return from_hip(ep::launch_layout_dispatch(
        static_cast<const uint16_t*>(x), topk_idx, T, H, K, E, P, fp8, workspace, m,
        num_tokens_per_expert, num_tokens_per_partition, is_token_in_partition, expert_offsets,
        partition_offsets, recv_x, recv_scales, recv_src_token, dst_row, num_cus,
        static_cast<hipStream_t>(stream)));
}

ep_status_t ep_layout_dispatch(const void* x, int32_t num_tokens, int32_t hidden,
                               const int64_t* topk_idx, int32_t num_topk, int32_t num_experts,
                               int32_t num_partitions, ep_dtype_t out_dtype,
                               int32_t* num_tokens_per_expert, int32_t* num_tokens_per_partition,
                               uint8_t* is_token_in_partition, int32_t* expert_offsets,
                               int32_t* partition_offsets, void* recv_x, float* recv_scales,
                               int32_t* recv_src_token, int32_t* dst_row, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return ep_layout_dispatch_cu(x, num_tokens, hidden, topk_idx, num_topk, num_experts,
                                 num_partitions, out_dtype, num_tokens_per_expert,
                                 num_tokens_per_partition, is_token_in_partition, expert_offsets,
                                 partition_offsets, recv_x, recv_scales, recv_src_token, dst_row,
                                 workspace, workspace_bytes, 0, stream);
}

ep_status_t ep_layout_dispatch_static(const void* x, int32_t num_tokens, int32_t hidden,
                                      const int64_t* topk_idx, int32_t num_topk,
                                      int32_t num_experts, int32_t num_partitions,
                                      ep_dtype_t out_dtype, int32_t* num_tokens_per_expert,
                                      int32_t* num_tokens_per_partition,
                                      uint8_t* is_token_in_partition, int32_t* expert_offsets,
                                      int32_t* partition_offsets, void* recv_x,
                                      float* recv_scales, int32_t* recv_src_token,
                                      int32_t* dst_row, void* stream) {
    const int32_t T = num_tokens, H = hidden, K = num_topk, E = num_experts, P = num_partitions;
    ep_status_t st = check_layout_dispatch(x, T, H, topk_idx, K, E, P, out_dtype,
                                           num_tokens_per_expert, num_tokens_per_partition,
                                           is_token_in_partition, expert_offsets,
                                           partition_offsets, recv_x, recv_scales,
                                           recv_src_token, dst_row);
    if (st != EP_OK) return st;
    if (ep::ws_map(T, K, E, P).total > (size_t)EP_STATIC_SCRATCH_BYTES) return EP_ERR_UNSUPPORTED;
    void* ws = nullptr;
    st = device_scratch(&ws);
    if (st != EP_OK) return st;
    // The kernels and outputs of ep_layout_dispatch, with the device's scratch
    // as the workspace.  Nothing in it needs clearing: every layout call
    // writes all that its dispatch launch reads.
    return ep_layout_dispatch_cu(x, num_tokens, hidden, topk_idx, num_topk, num_experts,
                                 num_partitions, out_dtype, num_tokens_per_expert,
                                 num_tokens_per_partition, is_token_in_partition, expert_offsets,
                                 partition_offsets, recv_x, recv_scales, recv_src_token, dst_row,
                                 ws, (size_t)EP_STATIC_SCRATCH_BYTES, 0, stream);
}

int64_t ep_aligned_rows(int32_t num_tokens, int32_t num_topk, int32_t num_experts,
                        int32_t expert_alignment) {
    if (check_routing_shape(num_tokens, num_topk, num_experts, 1) != EP_OK) return 0;
    if (expert_alignment < 1 || expert_alignment > EP_MAX_EXPERT_ALIGNMENT) return 0;
    const int64_t R = (int64_t)num_tokens * num_topk +
                      (int64_t)num_experts * (expert_alignment - 1);
    return R < kMaxRows ? R : 0;
}

ep_status_t ep_layout_dispatch_aligned(const void* x, int32_t num_tokens, int32_t hidden,
                                       const int64_t* topk_idx, int32_t num_topk,
                                       int32_t num_experts, int32_t num_partitions,
                                       int32_t expert_alignment, ep_dtype_t out_dtype,
                                       int32_t* num_tokens_per_expert,
                                       int32_t* num_tokens_per_partition,
                                       uint8_t* is_token_in_partition, int32_t* expert_offsets,
                                       int32_t* partition_offsets, void* recv_x,
                                       float* recv_scales, int32_t* recv_src_token,
                                       int32_t* dst_row, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    const int32_t T = num_tokens, H = hidden, K = num_topk, E = num_experts, P = num_partitions;
    ep_status_t st = check_routing_shape(T, K, E, P);
    if (st != EP_OK) return st;
    const int64_t R = ep_aligned_rows(T, K, E, expert_alignment);
    if (R == 0 && T > 0) return EP_ERR_INVALID_ARG;
    if (expert_alignment < 1 || expert_alignment > EP_MAX_EXPERT_ALIGNMENT)
        return EP_ERR_INVALID_ARG;
    if (out_dtype != EP_DTYPE_BF16 && out_dtype != EP_DTYPE_FP8_E4M3) return EP_ERR_INVALID_ARG;
    const bool fp8 = out_dtype == EP_DTYPE_FP8_E4M3;
    if (H <= 0 || H % 8 != 0 || (fp8 && H % 128 != 0)) return EP_ERR_INVALID_ARG;
    if (!num_tokens_per_expert || !num_tokens_per_partition || !expert_offsets ||
        !partition_offsets || !workspace)
        return EP_ERR_INVALID_ARG;
    if (R > 0 && !recv_src_token) return EP_ERR_INVALID_ARG;
    if (T > 0) {
        if (!x || !topk_idx || !is_token_in_partition || !recv_x || !dst_row)
            return EP_ERR_INVALID_ARG;
        if (fp8 && !recv_scales) return EP_ERR_INVALID_ARG;
        if (!aligned16(x) || !aligned16(recv_x)) return EP_ERR_INVALID_ARG;
    }
    const ep::WsMap m = ep::ws_map(T, K, E, P);
    if (workspace_bytes < m.total) return EP_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = ep::launch_layout_aligned(topk_idx, T, K, E, P, expert_alignment, workspace, m,
                                             num_tokens_per_expert, num_tokens_per_partition,
                                             is_token_in_partition, expert_offsets,
                                             partition_offsets, recv_src_token, R, s);
    if (e != hipSuccess) return EP_ERR_HIP;
    return from_hip(ep::launch_dispatch(static_cast<const uint16_t*>(x), T, H, K, fp8, recv_x,
                                        recv_scales, recv_src_token, dst_row, workspace, m, 0,
                                        (int)R, s));
}

ep_status_t ep_dispatch_dedup(const void* x, int32_t num_tokens, int32_t hidden,
                              const int64_t* topk_idx, int32_t num_topk, int32_t num_experts,
                              int32_t num_partitions, ep_dtype_t out_dtype,
                              int32_t* num_tokens_per_expert, int32_t* num_tokens_per_partition,
                              uint8_t* is_token_in_partition, int32_t* expert_offsets,
                              int32_t* partition_offsets, int32_t* partition_token_offsets,
                              void* recv_x, float* recv_scales, int32_t* recv_src_token,
                              int32_t* recv_topk_idx, int32_t* slot_src_row, int32_t* dst_row,
                              void* workspace, size_t workspace_bytes, void* stream) {
    const int32_t T = num_tokens, H = hidden, K = num_topk, E = num_experts, P = num_partitions;
    ep_status_t st = check_routing_shape(T, K, E, P);
    if (st != EP_OK) return st;
    if (out_dtype != EP_DTYPE_BF16 && out_dtype != EP_DTYPE_FP8_E4M3) return EP_ERR_INVALID_ARG;
    const bool fp8 = out_dtype == EP_DTYPE_FP8_E4M3;
    if (H <= 0 || H % 8 != 0 || (fp8 && H % 128 != 0)) return EP_ERR_INVALID_ARG;
    if (!num_tokens_per_expert || !num_tokens_per_partition || !expert_offsets ||
        !partition_offsets || !partition_token_offsets || !workspace)
        return EP_ERR_INVALID_ARG;
    if (T > 0) {
        if (!x || !topk_idx || !is_token_in_partition || !recv_x || !recv_src_token ||
            !recv_topk_idx || !slot_src_row || !dst_row)
            return EP_ERR_INVALID_ARG;
        if (fp8 && !recv_scales) return EP_ERR_INVALID_ARG;
        if (!aligned16(x) || !aligned16(recv_x)) return EP_ERR_INVALID_ARG;
    }
    const ep::WsMap m = ep::ws_map(T, K, E, P);
    if (workspace_bytes < m.total) return EP_ERR_WORKSPACE;
    return from_hip(ep::launch_dispatch_dedup(
        static_cast<const uint16_t*>(x), topk_idx, T, H, K, E, P, fp8, workspace, m,
        num_tokens_per_expert, num_tokens_per_partition, is_token_in_partition, expert_offsets,
        partition_offsets, partition_token_offsets, recv_x, recv_scales, recv_src_token,
        recv_topk_idx, slot_src_row, dst_row, static_cast<hipStream_t>(stream)));
}

ep_status_t ep_low_latency_dispatch(const void* x, int32_t num_tokens, int32_t hidden,
                                    const int64_t* topk_idx, int32_t num_topk,
                                    int32_t num_experts, int32_t capacity, ep_dtype_t out_dtype,
                                    int32_t* num_tokens_per_expert, void* recv_x,
                                    float* recv_scales, int32_t* recv_src_token,
                                    int32_t* dst_row, int64_t* num_invalid, void* stream) {
    const int32_t T = num_tokens, H = hidden, K = num_topk, E = num_experts, C = capacity;
    ep_status_t st = check_routing_shape(T, K, E, 1);
    if (st != EP_OK) return st;
    if (C <= 0 || (int64_t)E * C >= kMaxRows) return EP_ERR_INVALID_ARG;
    if (out_dtype != EP_DTYPE_BF16 && out_dtype != EP_DTYPE_FP8_E4M3) return EP_ERR_INVALID_ARG;
    const bool fp8 = out_dtype == EP_DTYPE_FP8_E4M3;
    if (H <= 0 || H % 8 != 0 || (fp8 && H % 128 != 0)) return EP_ERR_INVALID_ARG;
    if (!num_tokens_per_expert || !recv_src_token) return EP_ERR_INVALID_ARG;
    if (T > 0) {
        if (!x || !topk_idx || !recv_x || !dst_row) return EP_ERR_INVALID_ARG;
        if (fp8 && !recv_scales) return EP_ERR_INVALID_ARG;
        if (!aligned16(x) || !aligned16(recv_x)) return EP_ERR_INVALID_ARG;
    }
    if ((int64_t)T * K > EP_LL_MAX_SLOTS) return EP_ERR_UNSUPPORTED;
    return from_hip(ep::launch_ll_dispatch(
        static_cast<const uint16_t*>(x), topk_idx, T, H, K, E, C, fp8, num_tokens_per_expert,
        recv_x, recv_scales, recv_src_token, dst_row, num_invalid,
        static_cast<hipStream_t>(stream)));
}

ep_status_t ep_combine_cu(const void* y, int64_t num_rows, const int32_t* dst_row,
                          const float* topk_weights, int32_t num_tokens, int32_t num_topk,
                          int32_t hidden, void* out, int32_t num_cus, void* stream) {
    const int32_t T = num_tokens, K = num_topk, H = hidden;
    if (T < 0 || K <= 0 || H <= 0 || H % 8 != 0 || num_rows < 0 || num_cus < 0)
        return EP_ERR_INVALID_ARG;
    if ((int64_t)T * K >= kMaxRows) return EP_ERR_INVALID_ARG;
    if (K > EP_MAX_TOPK) return EP_ERR_UNSUPPORTED;
    if (T > 0) {
        if (!dst_row || !topk_weights || !out) return EP_ERR_INVALID_ARG;
        if ((y && !aligned16(y)) || !aligned16(out)) return EP_ERR_INVALID_ARG;
    }
    if (T > 0 && num_rows > 0 && !y) return EP_ERR_INVALID_ARG;
    return from_hip(ep::launch_combine(static_cast<const uint16_t*>(y), num_rows, dst_row,
                                       topk_weights, T, K, H, static_cast<uint16_t*>(out),
                                       num_cus, static_cast<hipStream_t>(stream)));
}

ep_status_t ep_combine(const void* y, int64_t num_rows, const int32_t* dst_row,
                       const float* topk_weights, int32_t num_tokens, int32_t num_topk,
                       int32_t hidden, void* out, void* stream) {
    return ep_combine_cu(y, num_rows, dst_row, topk_weights, num_tokens, num_topk, hidden, out, 0,
                         stream);
}

ep_status_t ep_get_device_error(const void* workspace, size_t workspace_bytes,
                                int64_t* num_invalid, void* stream) {
    if (!workspace || !num_invalid || workspace_bytes < ep::kWsHeaderBytes)
        return EP_ERR_INVALID_ARG;
    const ep::WsHeader* hdr = static_cast<const ep::WsHeader*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int64_t v = 0;
    if (hipMemcpyAsync(&v, &hdr->num_invalid, sizeof v, hipMemcpyDeviceToHost, s) !=
        hipSuccess)
        return EP_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return EP_ERR_HIP;
    *num_invalid = v;
    return EP_OK;
}

const char* ep_status_string(ep_status_t status) {
    switch (status) {
        case EP_OK: return "EP_OK";
        case EP_ERR_INVALID_ARG: return "EP_ERR_INVALID_ARG";
        case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED";
        case EP_ERR_WORKSPACE: return "EP_ERR_WORKSPACE";
        case EP_ERR_HIP: return "EP_ERR_HIP";
    }
    return "EP_ERR_UNKNOWN";
}

ep_status_t ep_convert_e4m3(const float* in, uint8_t* out, int64_t n, int32_t mode,
                            void* stream) {
    if (n < 0 || (n > 0 && (!in || !out)) || (mode != 0 && mode != 1)) return EP_ERR_INVALID_ARG;
    return from_hip(ep::launch_convert_e4m3(in, out, n, mode, static_cast<hipStream_t>(stream)));
}

ep_status_t ep_convert_bf16(const float* in, uint16_t* out, int64_t n, void* stream) {
    if (n < 0 || (n > 0 && (!in || !out))) return EP_ERR_INVALID_ARG;
    return from_hip(ep::launch_convert_bf16(in, out, n, static_cast<hipStream_t>(stream)));
}

ep_status_t ep_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (bytes % 16 != 0) return EP_ERR_INVALID_ARG;
    if (bytes > 0 && (!src || !dst || !aligned16(src) || !aligned16(dst)))
        return EP_ERR_INVALID_ARG;
    return from_hip(ep::launch_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
