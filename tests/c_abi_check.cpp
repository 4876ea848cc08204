// A C++ caller of the C ABI alone (include/ep.h, hipMalloc, no torch): one
// offsets-layout step in bf16 and in FP8, each both as the two calls
// ep_get_dispatch_layout -> ep_dispatch and as the one call ep_layout_dispatch,
// then ep_combine and ep_get_device_error, with checks that need no reference
// implementation:
//   the expert counts equal a count taken on the host, the one invalid id is
//   reported and its slot gets no row, counts sum to the valid slots, offsets
//   are their exclusive prefix, every
//   valid slot gets a distinct row inside its expert's run, rows inside a run
//   are in token order, recv_src_token inverts dst_row, bf16 rows are bitwise
//   copies of their tokens, every FP8 group's largest element encodes to +-448
//   with scale = max|x| / 448, and combine with weight 1 on slot 0 (0 on the
//   others) of identity experts returns x bit for bit.  Bad arguments return
//   EP_ERR_INVALID_ARG without touching the device.
// Prints "c_abi_check ok" and exits 0, or names the first failure and exits 1.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <utility>
#include <vector>

#include "ep.h"

namespace {

int g_failures = 0;

void expect(bool ok, const char* what) {
    if (!ok && g_failures++ == 0) std::fprintf(stderr, "c_abi_check FAILED: %s\n", what);
}

#define HIP_OK(call)                                                             \
    do {                                                                         \
        hipError_t e_ = (call);                                                  \
        if (e_ != hipSuccess) {                                                  \
            std::fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));      \
            return 1;                                                            \
        }                                                                        \
    } while (0)

#define EP_OK_CALL(call)                                                         \
    do {                                                                         \
        ep_status_t s_ = (call);                                                 \
        if (s_ != EP_OK) {                                                       \
            std::fprintf(stderr, "%s: %s\n", #call, ep_status_string(s_));       \
            return 1;                                                            \
        }                                                                        \
    } while (0)

float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// E4M3 code -> value (bias 7, 3 mantissa bits, subnormals below 2^-6).
float e4m3_to_float(uint8_t c) {
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    const float v = e == 0 ? std::ldexp((float)m, -9) : std::ldexp(1.0f + m / 8.0f, e - 7);
    return s ? -v : v;
}

}  // namespace

int main() {
    const int32_t T = 512, H = 1024, E = 64, P = 8, K = 6, Ep = E / P, G = H / 128;
    const int32_t R = T * K;

    // Routing: six distinct experts per token, slot 5 masked on every 17th token,
    // and one invalid id (slot 4 of token 3).
    std::vector<int64_t> idx((size_t)T * K);
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k)
            idx[(size_t)t * K + k] = (k == 5 && t % 17 == 0) ? -1 : (t * 5 + k * 11) % E;
    idx[(size_t)3 * K + 4] = E + 5;
    std::vector<int> host_cnt(E, 0);
    int valid = 0;
    for (int64_t v : idx)
        if (v >= 0 && v < E) {
            ++host_cnt[v];
            ++valid;
        }
    // Tokens: bf16 values with a per-(token, group) range, exact small multiples of 1/8.
    std::vector<uint16_t> x((size_t)T * H);
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            const float v = (float)(((t * 31 + h * 7) % 23) - 11) / 8.0f * (1 + (h / 128 + t) % 3);
            uint32_t u;
            std::memcpy(&u, &v, 4);
            x[(size_t)t * H + h] = (uint16_t)(u >> 16);   // exact: at most 8 significant bits
        }
    std::vector<float> w((size_t)T * K, 0.0f);
    for (int t = 0; t < T; ++t) w[(size_t)t * K] = 1.0f;

    const size_t ws_bytes = ep_workspace_bytes(T, K, E, P);
    expect(ws_bytes > 0, "ep_workspace_bytes");
    void *d_ws, *d_x, *d_idx, *d_w, *d_rx8, *d_rx16, *d_rs, *d_out;
    int32_t *d_cnt_e, *d_cnt_p, *d_off_e, *d_off_p, *d_src, *d_dst;
    uint8_t* d_inp;
    HIP_OK(hipMalloc(&d_ws, ws_bytes));
    HIP_OK(hipMalloc(&d_x, x.size() * 2));
    HIP_OK(hipMalloc(&d_idx, idx.size() * 8));
    HIP_OK(hipMalloc(&d_w, w.size() * 4));
    HIP_OK(hipMalloc(&d_rx8, (size_t)R * H));
    HIP_OK(hipMalloc(&d_rx16, (size_t)R * H * 2));
    HIP_OK(hipMalloc(&d_rs, (size_t)R * G * 4));
    HIP_OK(hipMalloc(&d_out, (size_t)T * H * 2));
    HIP_OK(hipMalloc(&d_cnt_e, E * 4));
    HIP_OK(hipMalloc(&d_cnt_p, P * 4));
    HIP_OK(hipMalloc(&d_off_e, (E + 1) * 4));
    HIP_OK(hipMalloc(&d_off_p, (P + 1) * 4));
    HIP_OK(hipMalloc(&d_src, R * 4));
    HIP_OK(hipMalloc(&d_dst, R * 4));
    HIP_OK(hipMalloc(&d_inp, (size_t)T * P));
    HIP_OK(hipMemcpy(d_x, x.data(), x.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_idx, idx.data(), idx.size() * 8, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w, w.data(), w.size() * 4, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    // Bad arguments are refused on the host.
    expect(ep_layout_dispatch(d_x, T, H, (const int64_t*)d_idx, K, E, 7, EP_DTYPE_BF16, d_cnt_e,
                              d_cnt_p, d_inp, d_off_e, d_off_p, d_rx16, nullptr, d_src, d_dst,
                              d_ws, ws_bytes, stream) == EP_ERR_INVALID_ARG,
           "E % P != 0 accepted");
    expect(ep_layout_dispatch(d_x, T, H, (const int64_t*)d_idx, K, E, P, EP_DTYPE_FP8_E4M3,
                              d_cnt_e, d_cnt_p, d_inp, d_off_e, d_off_p, d_rx8, nullptr, d_src,
                              d_dst, d_ws, ws_bytes, stream) == EP_ERR_INVALID_ARG,
           "FP8 without scales accepted");
    expect(ep_layout_dispatch(d_x, T, H, (const int64_t*)d_idx, K, E, P, EP_DTYPE_BF16, d_cnt_e,
                              d_cnt_p, d_inp, d_off_e, d_off_p, d_rx16, nullptr, d_src, d_dst,
                              d_ws, 16, stream) == EP_ERR_WORKSPACE,
           "small workspace accepted");

    for (int run = 0; run < 4; ++run) {
        const int fp8 = run & 1, two_calls = run >> 1;
        void* rx = fp8 ? d_rx8 : d_rx16;
        const ep_dtype_t dt = fp8 ? EP_DTYPE_FP8_E4M3 : EP_DTYPE_BF16;
        // clear the outputs, so that every value checked below comes from this run
        const std::pair<void*, size_t> outs[] = {{d_cnt_e, E * 4}, {d_cnt_p, P * 4},
                                                 {d_off_e, (E + 1) * 4}, {d_off_p, (P + 1) * 4},
                                                 {d_src, R * 4}, {d_dst, R * 4}};
        for (const auto& o : outs) HIP_OK(hipMemset(o.first, 0x7f, o.second));
        if (two_calls) {
            EP_OK_CALL(ep_get_dispatch_layout((const int64_t*)d_idx, T, K, E, P, d_cnt_e, d_cnt_p,
                                              d_inp, d_off_e, d_off_p, d_ws, ws_bytes, stream));
            EP_OK_CALL(ep_dispatch(d_x, T, H, (const int64_t*)d_idx, K, E, P, dt, rx,
                                   fp8 ? (float*)d_rs : nullptr, d_src, d_dst, d_ws, ws_bytes,
                                   stream));
        } else {
            EP_OK_CALL(ep_layout_dispatch(d_x, T, H, (const int64_t*)d_idx, K, E, P, dt, d_cnt_e,
                                          d_cnt_p, d_inp, d_off_e, d_off_p, rx,
                                          fp8 ? (float*)d_rs : nullptr, d_src, d_dst, d_ws,
                                          ws_bytes, stream));
        }
        if (!fp8)   // identity experts: y = the bf16 receive rows
            EP_OK_CALL(ep_combine(d_rx16, R, d_dst, (const float*)d_w, T, K, H, d_out, stream));
        int64_t ninv = -1;
        EP_OK_CALL(ep_get_device_error(d_ws, ws_bytes, &ninv, stream));   // synchronises
        expect(ninv == 1, "the one invalid id is not reported");

        std::vector<int32_t> cnt_e(E), cnt_p(P), off_e(E + 1), off_p(P + 1), src(R), dst(R);
        std::vector<uint8_t> inp((size_t)T * P);
        HIP_OK(hipMemcpy(cnt_e.data(), d_cnt_e, E * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(cnt_p.data(), d_cnt_p, P * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(off_e.data(), d_off_e, (E + 1) * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(off_p.data(), d_off_p, (P + 1) * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(src.data(), d_src, R * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(dst.data(), d_dst, R * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(inp.data(), d_inp, (size_t)T * P, hipMemcpyDeviceToHost));

        int sum = 0;
        for (int e = 0; e < E; ++e) {
            expect(cnt_e[e] == host_cnt[e], "expert count differs from the host's count");
            expect(off_e[e] == sum, "expert offsets are not the prefix of the counts");
            sum += cnt_e[e];
        }
        expect(sum == valid && off_e[E] == valid, "counts do not sum to the valid slots");
        for (int p = 0; p <= P; ++p)
            expect(off_p[p] == off_e[p * Ep], "partition offsets");
        for (int p = 0; p < P; ++p) {
            int members = 0;
            for (int t = 0; t < T; ++t) members += inp[(size_t)t * P + p];
            expect(cnt_p[p] == members, "partition token counts");
        }
        std::vector<int> seen(R, 0), last_tok(R, -1);
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k) {
                const int64_t e = idx[(size_t)t * K + k];
                const int r = dst[(size_t)t * K + k];
                if (e < 0 || e >= E) {
                    expect(r == -1, "masked or invalid slot got a row");
                    continue;
                }
                expect(r >= off_e[e] && r < off_e[e + 1], "row outside its expert's run");
                if (r < 0 || r >= R) continue;
                expect(seen[r]++ == 0, "two slots share a row");
                expect(src[r] == t, "recv_src_token does not invert dst_row");
                expect(inp[(size_t)t * P + e / Ep] == 1, "partition mask");
            }
        for (int e = 0; e < E; ++e)
            for (int r = off_e[e] + 1; r < off_e[e + 1]; ++r)
                expect(src[r] >= src[r - 1], "rows of an expert out of token order");
        for (int r = valid; r < R; ++r) expect(src[r] == -1, "unused row has a source");

        if (!fp8) {
            std::vector<uint16_t> rx16((size_t)valid * H), out((size_t)T * H);
            HIP_OK(hipMemcpy(rx16.data(), d_rx16, rx16.size() * 2, hipMemcpyDeviceToHost));
            HIP_OK(hipMemcpy(out.data(), d_out, out.size() * 2, hipMemcpyDeviceToHost));
            for (int r = 0; r < valid; ++r)
                expect(std::memcmp(&rx16[(size_t)r * H], &x[(size_t)src[r] * H], H * 2) == 0,
                       "bf16 row is not a copy of its token");
            expect(std::memcmp(out.data(), x.data(), out.size() * 2) == 0,
                   "combine of identity experts with weight 1 on slot 0 is not x");
        } else {
            std::vector<uint8_t> rx8((size_t)valid * H);
            std::vector<float> rs((size_t)valid * G);
            HIP_OK(hipMemcpy(rx8.data(), d_rx8, rx8.size(), hipMemcpyDeviceToHost));
            HIP_OK(hipMemcpy(rs.data(), d_rs, rs.size() * 4, hipMemcpyDeviceToHost));
            for (int r = 0; r < valid; ++r)
                for (int g = 0; g < G; ++g) {
                    float amax = 0.0f, cmax = 0.0f;
                    for (int j = 0; j < 128; ++j) {
                        const size_t h = (size_t)g * 128 + j;
                        amax = std::fmax(amax, std::fabs(bf16_to_float(x[(size_t)src[r] * H + h])));
                        cmax = std::fmax(cmax, std::fabs(e4m3_to_float(rx8[(size_t)r * H + h])));
                    }
                    const float ac = amax > 1e-4f ? amax : 1e-4f;
                    expect(rs[(size_t)r * G + g] == ac / 448.0f, "scale is not max|x| / 448");
                    if (amax >= 1e-4f) expect(cmax == 448.0f, "group maximum does not encode to 448");
                }
        }
    }
    HIP_OK(hipStreamDestroy(stream));
    for (void* p : {d_ws, d_x, d_idx, d_w, d_rx8, d_rx16, d_rs, d_out, (void*)d_cnt_e,
                    (void*)d_cnt_p, (void*)d_off_e, (void*)d_off_p, (void*)d_src, (void*)d_dst,
                    (void*)d_inp})
        HIP_OK(hipFree(p));
    if (g_failures) {
        std::fprintf(stderr, "c_abi_check: %d failed checks\n", g_failures);
        return 1;
    }
    std::printf("c_abi_check ok\n");
    return 0;
}
