/*
 * ep_oracle.c -- plain, slow, single-threaded CPU oracle for MoE token
 * dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  The product
 * path (the HIP library and its Python binding) never calls it, and this file
 * shares no code, header, table or constant generator with that path.
 *
 * What is computed and where it comes from.
 *   DeepEP is the expert-parallel all-to-all library for Mixture-of-Experts
 *   models: "dispatch" sends each token to the experts that its router picked
 *   and "combine" brings the expert outputs back to the token
 *   ("DeepSeek releases DeepEP, an efficient communication library for MoE
 *   models", section "DeepEP: Optimizing MoE Communication"; the same two
 *   operations are named in the introduction of "Deepseek Ai Deepep: A library
 *   for an open-open EP for example training").  Dispatch may carry FP8
 *   payloads (the feature list of "DeepSeek Open Source Weekly Review - 2"
 *   names FP8 for dispatch).
 *
 *   The pages give neither the bookkeeping (layout) that an all-to-all needs,
 *   nor the receive-buffer order, nor the FP8 scale rule, nor the combine
 *   arithmetic.  This oracle takes the plainest reading of each, as listed
 *   in the repository's design notes:
 *     - expert e lives in partition floor(e / (E/P))              (contiguous)
 *     - one receive row per valid (token, slot) pair, rows grouped by expert
 *       in ascending expert order, so every partition is one contiguous run
 *     - inside one expert's rows the order is by source token, then by slot
 *     - topk_idx == -1 is a masked slot; any other value outside [0, E) is an
 *       invalid slot: it is masked too and counted as an error
 *     - per-partition token counts count distinct tokens
 *     - FP8 is OCP E4M3 (bias 7, max finite 448, one NaN pattern per sign),
 *       round to nearest even, saturating, sign kept; one fp32 scale per
 *       token and 128 consecutive channels: a = max|x|, a_c = max(a, 1e-4f),
 *       q = E4M3(x * (448 / a_c)), s = a_c / 448
 *     - combine: out = bf16_rne( fma chain over slots k = 0..K-1 of
 *       w[t][k] * y[dst[t][k]] in fp32, starting from +0, skipping masked
 *       slots )
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fPIC -shared.
 * Contraction is off so that every float product and sum below rounds on its
 * own, exactly as written; fmaf() is the only fused operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Scalar formats                                                           */
/* ------------------------------------------------------------------------ */

/* bf16 -> fp32 is exact: a bf16 value is the top half of an fp32 word. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * fp32 -> bf16, round to nearest, ties to even.
 * Written from the definition: take the two bf16 values that bracket |f|
 * (truncation and the next one up), measure both distances exactly in double,
 * keep the nearer, and on a tie keep the one whose last mantissa bit is 0.
 * The next value up from the largest finite bf16 is 2^128, which rounds to
 * infinity, as IEEE round-to-nearest prescribes.
 */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(f))
        return (uint16_t)(sign | 0x7F80u);

    uint16_t lo = (uint16_t)((u >> 16) & 0x7FFFu); /* |f| truncated */
    uint16_t hi = (uint16_t)(lo + 1u);             /* next bf16 magnitude up */
    double a = fabs((double)f);
    double vlo = (double)bf16_to_f32(lo);
    double vhi = (hi == 0x7F80u) ? ldexp(1.0, 128) : (double)bf16_to_f32(hi);
    double dlo = a - vlo, dhi = vhi - a;
    uint16_t mag;
    if (dlo < dhi)
        mag = lo;
    else if (dhi < dlo)
        mag = hi;
    else
        mag = (lo & 1u) ? hi : lo;
    return (uint16_t)(sign | mag);
}

/*
 * fp32 -> OCP E4M3 ("e4m3fn"), round to nearest even, saturating.
 * Format: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Normal
 * codes are (1 + m/8) * 2^(e-7) for e = 1..15; code S.1111.111 is NaN, so the
 * largest finite value is 1.75 * 2^8 = 448 (0x7E).  Subnormal codes
 * (e = 0) are (m/8) * 2^-6.
 *
 * Every finite E4M3 value is an integer multiple of the quantum of its
 * binade: 2^(E-3) for |v| in [2^E, 2^(E+1)), E >= -6, and the subnormals
 * share the quantum 2^-9 of binade -6.  So the encoder finds the binade,
 * divides by the quantum (exact: a power of two) and rounds to the nearest
 * integer with nearbyint() under the default ties-to-even mode.  A result of
 * 16 quanta carries into the next binade.  Magnitudes at or above 448
 * saturate to 448; the sign bit is always kept, so a negative value that
 * rounds to zero gives 0x80.
 */
uint8_t oracle_e4m3(float v)
{
    uint8_t sign = signbit(v) ? 0x80u : 0x00u;
    if (isnan(v))
        return (uint8_t)(sign | 0x7Fu);
    double a = fabs((double)v);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7Eu);
    if (a == 0.0)
        return sign;

    int ex;
    (void)frexp(a, &ex); /* a = f * 2^ex with f in [0.5, 1) */
    int E = ex - 1;      /* a in [2^E, 2^(E+1)) */
    if (E < -6)
        E = -6;          /* subnormal range: quantum of binade -6 */
    double q = nearbyint(a / ldexp(1.0, E - 3));
    if (q >= 16.0) {     /* rounded up into the next binade */
        E += 1;
        q = 8.0;
    }
    int code;
    if (E == -6 && q < 8.0)
        code = (int)q;                          /* subnormal */
    else
        code = ((E + 7) << 3) | ((int)q - 8);  /* normal */
    if (code > 0x7E)
        code = 0x7E;     /* unreachable for a < 448; kept as the saturation rule */
    return (uint8_t)(sign | (uint8_t)code);
}

/* Element-wise array forms, for the tests' sweeps. */
void oracle_bf16_rne_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(in[i]);
}

void oracle_e4m3_array(const float *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Layout: per-expert / per-partition counts and offsets                     */
/* ------------------------------------------------------------------------ */

/*
 * The bookkeeping every all-to-all dispatch needs before it can move data:
 * how many rows go to each expert and to each destination partition, and
 * where each run starts ("DeepSeek releases DeepEP ...", section "DeepEP:
 * Optimizing MoE Communication": efficient all-to-all between the GPUs that
 * host the experts).
 *
 *   idx          [T][K] int64, row-major
 *   cnt_e        [E]    rows routed to expert e (valid slots only)
 *   cnt_p        [P]    distinct tokens with at least one valid slot in p
 *   in_part      [T][P] 1 if token t has a valid slot in partition p, else 0
 *   off_e        [E+1]  exclusive prefix sum of cnt_e; off_e[E] = N
 *   off_p        [P+1]  off_p[p] = off_e[p * (E/P)]
 * Returns the number of invalid slots (outside [0, E) and not -1).
 */
int64_t oracle_layout(const int64_t *idx, int32_t T, int32_t K, int32_t E, int32_t P,
                      int32_t *cnt_e, int32_t *cnt_p, uint8_t *in_part,
                      int32_t *off_e, int32_t *off_p)
{
    int32_t Ep = E / P;
    int64_t nerr = 0;
    for (int32_t e = 0; e < E; ++e)
        cnt_e[e] = 0;
    for (int32_t p = 0; p < P; ++p)
        cnt_p[p] = 0;
    for (int64_t i = 0; i < (int64_t)T * P; ++i)
        in_part[i] = 0;

    for (int32_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t v = idx[(int64_t)t * K + k];
            if (v >= 0 && v < E) {
                cnt_e[v] += 1;
                in_part[(int64_t)t * P + v / Ep] = 1;
            } else if (v != -1) {
                nerr += 1;
            }
        }
    }
    for (int32_t t = 0; t < T; ++t)
        for (int32_t p = 0; p < P; ++p)
            cnt_p[p] += in_part[(int64_t)t * P + p];

    off_e[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        off_e[e + 1] = off_e[e] + cnt_e[e];
    for (int32_t p = 0; p <= P; ++p)
        off_p[p] = off_e[p * Ep];
    return nerr;
}

/*
 * Receive-row assignment.  Valid slots are visited in (token, slot) order and
 * each takes the next free row of its expert's run, so inside an expert the
 * rows are ordered by source token, then slot.
 *   dst [T][K]  receive row of slot (t,k), or -1 for a masked/invalid slot
 *   src [T*K]   source token of receive row r, or -1 for r >= N
 */
void oracle_permutation(const int64_t *idx, int32_t T, int32_t K, int32_t E,
                        const int32_t *off_e, int32_t *dst, int32_t *src)
{
    int32_t *next = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int32_t N = off_e[E];
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t v = idx[(int64_t)t * K + k];
            if (v >= 0 && v < E) {
                int32_t r = off_e[v] + next[v];
                next[v] += 1;
                dst[(int64_t)t * K + k] = r;
                src[r] = t;
            } else {
                dst[(int64_t)t * K + k] = -1;
            }
        }
    }
    for (int64_t r = N; r < (int64_t)T * K; ++r)
        src[r] = -1;
    free(next);
}

/* ------------------------------------------------------------------------ */
/* Dispatch                                                                  */
/* ------------------------------------------------------------------------ */

/* bf16 dispatch: receive row r is a bitwise copy of token src[r], r < N. */
void oracle_dispatch_bf16(const uint16_t *x, int32_t T, int32_t H,
                          const int32_t *src, int32_t N, uint16_t *recv_x)
{
    (void)T;
    for (int64_t r = 0; r < N; ++r) {
        int64_t t = src[r];
        for (int64_t h = 0; h < H; ++h)
            recv_x[r * H + h] = x[t * H + h];
    }
}

/*
 * Per-token FP8 quantisation with one scale per 128 consecutive channels
 * (FP8 for dispatch is in the feature list of "DeepSeek Open Source Weekly
 * Review - 2"; FP8 support is also listed in "DeepSeek releases DeepEP ...",
 * section "DeepEP: Optimizing MoE Communication").  For token t and group
 * g (channels 128g .. 128g+127):
 *   a    = max |x|                (exact in fp32)
 *   a_c  = max(a, 1e-4f)
 *   inv  = 448.0f / a_c           (one correctly rounded fp32 division)
 *   s    = a_c / 448.0f           (one correctly rounded fp32 division)
 *   q[h] = E4M3(x[h] * inv)       (one rounded fp32 product, then encode)
 *   q [T][H] bytes, s [T][H/128] fp32.  H must be a multiple of 128.
 * Non-finite x (the pages say nothing of them; this reading keeps the sign
 * of x in every code, as for zeros): a NaN is left out of the maximum (the
 * comparison below is false for it), an infinity makes a = a_c = s = +inf
 * and inv = 0, and the code of an infinite or NaN x is the NaN pattern
 * S.1111.111 with S the sign of x -- x * inv is a NaN for both, and IEEE
 * arithmetic leaves open the sign of the NaN that inf * 0 produces.
 */
void oracle_quantize(const uint16_t *x, int32_t T, int32_t H, uint8_t *q, float *s)
{
    int32_t G = H / 128;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t g = 0; g < G; ++g) {
            float a = 0.0f;
            for (int32_t j = 0; j < 128; ++j) {
                float v = fabsf(bf16_to_f32(x[t * H + 128 * g + j]));
                if (v > a)
                    a = v;
            }
            float ac = (a > 1e-4f) ? a : 1e-4f;
            float inv = 448.0f / ac;
            s[t * G + g] = ac / 448.0f;
            for (int32_t j = 0; j < 128; ++j) {
                float xv = bf16_to_f32(x[t * H + 128 * g + j]);
                if (isnan(xv) || isinf(xv))
                    q[t * H + 128 * g + j] = signbit(xv) ? 0xFFu : 0x7Fu;
                else
                    q[t * H + 128 * g + j] = oracle_e4m3(xv * inv);
            }
        }
    }
}

/* FP8 dispatch: receive row r (r < N) gets token src[r]'s codes and scales. */
void oracle_dispatch_fp8(const uint16_t *x, int32_t T, int32_t H,
                         const int32_t *src, int32_t N,
                         uint8_t *recv_x, float *recv_scales)
{
    int32_t G = H / 128;
    uint8_t *q = (uint8_t *)malloc((size_t)T * (size_t)H + 1);
    float *s = (float *)malloc(((size_t)T * (size_t)G + 1) * sizeof(float));
    oracle_quantize(x, T, H, q, s);
    for (int64_t r = 0; r < N; ++r) {
        int64_t t = src[r];
        for (int64_t h = 0; h < H; ++h)
            recv_x[r * H + h] = q[t * H + h];
        for (int32_t g = 0; g < G; ++g)
            recv_scales[r * G + g] = s[t * G + g];
    }
    free(q);
    free(s);
}

/* ------------------------------------------------------------------------ */
/* Fixed-capacity receive layout (decode variant)                            */
/* ------------------------------------------------------------------------ */

/*
 * Besides the throughput kernels, the library has a second family for
 * inference decoding: small batches, lowest latency ("DeepSeek releases
 * DeepEP ...", section "Technical Details"; the 128-token, top-8 decode case
 * is in "Deepseek Ai Deepep: A library for an open-open EP for example
 * training", section "Technological Views and Benefits").  The pages give no
 * buffer layout for it.  This oracle takes a fixed-capacity one, in which no
 * row number depends on the counts of other experts:
 *   expert e owns receive rows [e*C, (e+1)*C), C = capacity per expert
 *   a valid slot (t,k) of expert e whose rank among expert e's valid slots,
 *   in (token, slot) order, is r gets row e*C + r when r < C; when r >= C it
 *   is dropped (dst = -1)
 *   cnt_e [E]    valid slots routed to expert e (dropped ones included)
 *   dst   [T][K] receive row of slot (t,k), or -1 (masked, invalid, dropped)
 *   src   [E*C]  source token of each receive row, -1 where no slot landed
 * Returns the number of invalid slots (outside [0, E) and not -1).
 */
int64_t oracle_ll_layout(const int64_t *idx, int32_t T, int32_t K, int32_t E, int32_t C,
                         int32_t *cnt_e, int32_t *dst, int32_t *src)
{
    int64_t nerr = 0;
    for (int32_t e = 0; e < E; ++e)
        cnt_e[e] = 0;
    for (int64_t r = 0; r < (int64_t)E * C; ++r)
        src[r] = -1;
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t v = idx[(int64_t)t * K + k];
            int32_t row = -1;
            if (v >= 0 && v < E) {
                int32_t rank = cnt_e[v];
                cnt_e[v] += 1;
                if (rank < C) {
                    row = (int32_t)v * C + rank;
                    src[row] = t;
                }
            } else if (v != -1) {
                nerr += 1;
            }
            dst[(int64_t)t * K + k] = row;
        }
    }
    return nerr;
}

/*
 * Dispatch into receive rows named by a source-token map: each row r in
 * [0, R) with src[r] >= 0 becomes token src[r]'s row (bf16 bits, or FP8
 * codes and scales from oracle_quantize); rows with src[r] = -1 are left
 * unwritten.
 */
void oracle_dispatch_rows_bf16(const uint16_t *x, int32_t T, int32_t H,
                               const int32_t *src, int64_t R, uint16_t *recv_x)
{
    (void)T;
    for (int64_t r = 0; r < R; ++r) {
        int64_t t = src[r];
        if (t < 0)
            continue;
        for (int64_t h = 0; h < H; ++h)
            recv_x[r * H + h] = x[t * H + h];
    }
}

void oracle_dispatch_rows_fp8(const uint16_t *x, int32_t T, int32_t H,
                              const int32_t *src, int64_t R,
                              uint8_t *recv_x, float *recv_scales)
{
    int32_t G = H / 128;
    uint8_t *q = (uint8_t *)malloc((size_t)T * (size_t)H + 1);
    float *s = (float *)malloc(((size_t)T * (size_t)G + 1) * sizeof(float));
    oracle_quantize(x, T, H, q, s);
    for (int64_t r = 0; r < R; ++r) {
        int64_t t = src[r];
        if (t < 0)
            continue;
        for (int64_t h = 0; h < H; ++h)
            recv_x[r * H + h] = q[t * H + h];
        for (int32_t g = 0; g < G; ++g)
            recv_scales[r * G + g] = s[t * G + g];
    }
    free(q);
    free(s);
}

/* ------------------------------------------------------------------------ */
/* Expert runs aligned for grouped GEMMs                                     */
/* ------------------------------------------------------------------------ */

/*
 * The expert-major layout of oracle_layout / oracle_permutation with every
 * expert's run padded to a whole number of `align` rows, so that each
 * expert's first row sits on a tile boundary of a grouped expert GEMM.  The
 * pages give no receive layout at all (their normal kernels serve training
 * and prefill: "DeepSeek releases DeepEP ...", section "Technical Details");
 * this is the plainest reading of a padded one:
 *   cnt_e, cnt_p, in_part   as oracle_layout (unpadded counts)
 *   off_e [E+1]  off_e[0] = 0, off_e[e+1] = off_e[e] + ceil(cnt_e[e] / align) * align
 *   off_p [P+1]  off_p[p] = off_e[p * (E/P)]
 *   dst   [T][K] off_e[e] + (rank of slot (t,k) among expert e's valid slots
 *                in (token, slot) order), -1 for a masked/invalid slot
 *   src   [R]    R = T*K + E*(align-1) rows (enough for any routing): the
 *                source token of each row, -1 for padding and unused rows
 * align = 1 gives exactly oracle_layout and oracle_permutation.
 * Returns the number of invalid slots (outside [0, E) and not -1).
 */
int64_t oracle_aligned_layout(const int64_t *idx, int32_t T, int32_t K, int32_t E, int32_t P,
                              int32_t align, int32_t *cnt_e, int32_t *cnt_p, uint8_t *in_part,
                              int32_t *off_e, int32_t *off_p, int32_t *dst, int32_t *src)
{
    int32_t Ep = E / P;
    int64_t R = (int64_t)T * K + (int64_t)E * (align - 1);
    int64_t nerr = oracle_layout(idx, T, K, E, P, cnt_e, cnt_p, in_part, off_e, off_p);
    int32_t *next = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int32_t run = 0;

    for (int32_t e = 0; e < E; ++e) {
        off_e[e] = run;
        run += (cnt_e[e] + align - 1) / align * align;   /* the run padded to whole tiles */
    }
    off_e[E] = run;
    for (int32_t p = 0; p <= P; ++p)
        off_p[p] = off_e[Ep * p];

    for (int64_t r = 0; r < R; ++r)
        src[r] = -1;
    for (int64_t i = 0; i < (int64_t)T * K; ++i) {      /* row-major = (token, slot) order */
        int64_t v = idx[i];
        dst[i] = -1;
        if (v < 0 || v >= E)
            continue;
        dst[i] = off_e[v] + next[v];
        next[v] += 1;
        src[dst[i]] = (int32_t)(i / K);
    }
    free(next);
    return nerr;
}

/* ------------------------------------------------------------------------ */
/* De-duplicated per-partition dispatch                                      */
/* ------------------------------------------------------------------------ */

/*
 * One copy of a token per destination partition instead of one per selected
 * expert.  Group-limited gating keeps the number of partitions a token
 * reaches small ("DeepSeek releases DeepEP ...", section "DeepEP: Optimizing
 * MoE Communication"), and merging what goes to the same destination before
 * it is sent is how the library saves link traffic ("DeepSeek Open Source
 * Week: A carnival of technology inclusion ...", section 4).  The pages give
 * no layout; this oracle takes the plainest one:
 *   ptok_off [P+1]   exclusive prefix of the per-partition token counts
 *                    (cnt_p of oracle_layout)
 *   the rows of partition p are [ptok_off[p], ptok_off[p+1]), one per token
 *   with a valid slot in p, in token order
 *   dd_row   [T][P]  row of (t, p), -1 if t has no valid slot in p
 *   dd_src   [RD]    source token of each row, -1 for rows >= ptok_off[P]
 *                    (RD = T * min(K, P) rows, an upper bound)
 *   dd_idx   [RD][K] for row (t, p): the local expert id e - p*(E/P) of each
 *                    slot k of t whose expert is in p, else -1 (rows beyond
 *                    ptok_off[P] are -1 throughout)
 *   slot_src [T*K]   for every expert-major receive row r = dst[t][k] (as
 *                    oracle_permutation numbers them): the row of (t, part of
 *                    slot k), so an expert's inputs are dd rows
 *                    slot_src[expert_offsets[e] .. expert_offsets[e+1]);
 *                    -1 for r >= N
 * Returns the number of rows, ptok_off[P].
 */
int32_t oracle_dedup_layout(const int64_t *idx, int32_t T, int32_t K, int32_t E, int32_t P,
                            const int32_t *cnt_p, const int32_t *dst, int32_t *ptok_off,
                            int32_t *dd_row, int32_t *dd_src, int32_t *dd_idx,
                            int32_t *slot_src)
{
    int32_t Ep = E / P;
    int32_t Kp = K < P ? K : P;
    int64_t RD = (int64_t)T * Kp;
    int32_t *next = (int32_t *)calloc((size_t)P + 1, sizeof(int32_t));
    ptok_off[0] = 0;
    for (int32_t p = 0; p < P; ++p)
        ptok_off[p + 1] = ptok_off[p] + cnt_p[p];
    for (int64_t i = 0; i < (int64_t)T * P; ++i)
        dd_row[i] = -1;
    for (int64_t r = 0; r < RD; ++r) {
        dd_src[r] = -1;
        for (int32_t k = 0; k < K; ++k)
            dd_idx[r * K + k] = -1;
    }
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t p = 0; p < P; ++p) {
            int member = 0;
            for (int32_t k = 0; k < K; ++k) {
                int64_t v = idx[(int64_t)t * K + k];
                if (v >= 0 && v < E && v / Ep == p)
                    member = 1;
            }
            if (!member)
                continue;
            int32_t r = ptok_off[p] + next[p];
            next[p] += 1;
            dd_row[(int64_t)t * P + p] = r;
            dd_src[r] = t;
            for (int32_t k = 0; k < K; ++k) {
                int64_t v = idx[(int64_t)t * K + k];
                if (v >= 0 && v < E && v / Ep == p)
                    dd_idx[(int64_t)r * K + k] = (int32_t)(v - (int64_t)p * Ep);
            }
        }
    }
    for (int64_t r = 0; r < (int64_t)T * K; ++r)
        slot_src[r] = -1;
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int32_t r = dst[(int64_t)t * K + k];
            if (r < 0)
                continue;
            int64_t v = idx[(int64_t)t * K + k];
            slot_src[r] = dd_row[(int64_t)t * P + v / Ep];
        }
    }
    free(next);
    return ptok_off[P];
}

/* ------------------------------------------------------------------------ */
/* Combine                                                                   */
/* ------------------------------------------------------------------------ */

/*
 * Combine: bring the expert outputs of a token back and reduce them with the
 * token's gate weights ("DeepSeek releases DeepEP ...", section "DeepEP:
 * Optimizing MoE Communication").  For every token t and channel h:
 *   acc = +0.0f
 *   for k = 0 .. K-1 with dst[t][k] >= 0:  acc = fmaf(w[t][k], y[dst[t][k]][h], acc)
 *   out[t][h] = bf16_rne(acc)
 *   y [R][H] bf16 (R >= max dst + 1), w [T][K] fp32, out [T][H] bf16.
 */
void oracle_combine(const uint16_t *y, const int32_t *dst, const float *w,
                    int32_t T, int32_t K, int32_t H, uint16_t *out)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                int64_t r = dst[t * K + k];
                if (r < 0)
                    continue;
                acc = fmaf(w[t * K + k], bf16_to_f32(y[r * H + h]), acc);
            }
            out[t * H + h] = oracle_bf16_rne(acc);
        }
    }
}
