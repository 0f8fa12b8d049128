/*
 * CPU oracle for MoE token dispatch / combine.  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously-correct definition that the HIP
 * library is checked against.  Only the test suite, the smoke entry point and
 * the benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or helper with the HIP library: it has its own bf16 / E4M3 / UE8M0
 * codecs, written from the format definitions (IEEE-754 binary16-truncated
 * "bfloat16" with round-to-nearest-even, and the OCP 8-bit floating point
 * specification for E4M3 and E8M0), and its own layout arithmetic.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no fast-math, SSE float on
 * x86-64, so every float operation below is one correctly rounded IEEE
 * binary32 op).  OpenMP only splits the token loops of dispatch and combine
 * across threads for the timing baseline; one thread is the default.
 *
 * What is computed, and the passages it follows (pages cited by title and
 * section):
 *   - Layout inferred from top-k expert ids, with per-expert received-token
 *     counts carried on the dispatch handle: page "moe: add DeepEP V2
 *     ElasticBuffer support to MoE token dispatcher", Motivation and the
 *     _dispatch_core commit message.
 *   - Per-expert-contiguous ("expanded") layout for prefill and the
 *     fixed-capacity masked [experts, capacity, hidden] slab for decode:
 *     page "[Feature] Add DeepEPv2 (ElasticBuffer) MoE A2A backend",
 *     Supported scope / layouts paragraph and the review reply on layout
 *     following the inference phase; page vLLM tools/ep_kernels, commit
 *     message (do_expand, per-expert-contiguous layout).
 *   - FP8 block-quantized dispatch with fp32 (Hopper) or packed UE8M0
 *     (Blackwell) activation scales: page "[Feature] Add DeepEPv2
 *     (ElasticBuffer) MoE A2A backend", Implementation; page "deepep v2
 *     support?", quantization requirement (128x128 weight blocks, dynamic
 *     activation scaling => 1x128 activation groups).
 *   - Combine as the router-weighted top-k reduction back to token order,
 *     with no further reduction after it: page vLLM tools/ep_kernels, commit
 *     message (weighted reduction in combine); page "[Feature] Add DeepEPv2
 *     (ElasticBuffer) MoE A2A backend", review (extra post-expert reduction
 *     double-counts).
 *   - The per-rank deduplicated exchange of the V1 dispatch (its layout
 *     pre-pass, named on page "moe: add DeepEP V2 ElasticBuffer support to MoE
 *     token dispatcher", Motivation): each token sent once per destination
 *     rank, expanded to per-expert rows on the receiver, and combined as
 *     per-rank partial sums reduced again on the source (the multiple-
 *     reduction option on page vLLM tools/ep_kernels, commit message).
 *   - MXFP8 dispatch for 1x32 MXFP8 experts with dynamic activation scaling
 *     (page "[Feature] Add DeepEPv2 (ElasticBuffer) MoE A2A backend", format
 *     check), following the OCP Microscaling conversion.
 *   - Adapters for grouped-GEMM consumers: per-row expert indices, masked <->
 *     contiguous repack and MN-major scales (same page, Implementation:
 *     masked-slab repack kernels and GEMM adapters with fp32 and packed UE8M0
 *     scales).
 *
 * The pages leave row order, alignment, overflow handling, scale formulas and
 * rounding open; the readings taken here are stated in the comments of each
 * function.  Every function below is pinned by a CPU test
 * (brute force, closed forms, library routines, exhaustive codec sweeps or
 * hand-worked fixtures); none is "parity unpinned".
 */
#include <assert.h>
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Codecs                                                                   */
/* ------------------------------------------------------------------------ */

/* bfloat16 bits -> float: the bf16 pattern is the upper half of a binary32. */
float oracle_bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t float_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* Value of a bf16 magnitude pattern (sign cleared) as a double, with the
 * pattern one past the largest finite magnitude standing for 2^128 (where
 * IEEE rounding sends overflowing values, i.e. to infinity). */
static double bf16_mag_value(uint32_t mag)
{
    if (mag >= 0x7F80u)
        return ldexp(1.0, 128);
    return (double)oracle_bf16_to_float((uint16_t)mag);
}

/* float -> bfloat16 bits, round to nearest, ties to even.  Written as the
 * definition: of the two bf16 magnitudes that bracket |f| (the truncation and
 * its successor), take the nearer; on a tie take the one whose last mantissa
 * bit is 0.  Differences are exact in double.  Inputs are finite. */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u = float_bits(f);
    uint32_t sign = u & 0x80000000u;
    assert((u & 0x7F800000u) != 0x7F800000u); /* finite inputs only */
    uint32_t lo = (u & 0x7FFFFFFFu) >> 16;    /* truncated magnitude */
    uint32_t hi = lo + 1;
    double a = fabs((double)f);
    double dlo = a - bf16_mag_value(lo);
    double dhi = bf16_mag_value(hi) - a;
    uint32_t pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = (lo & 1u) ? hi : lo;
    return (uint16_t)((sign >> 16) | pick);
}

/* Value of a non-negative E4M3 code 0x00..0x7E (OCP FP8 E4M3: bias 7, three
 * mantissa bits, exponent field 0 = subnormal m/8 * 2^-6, no infinities,
 * 0x7F = NaN, largest finite 0x7E = 448). */
double oracle_e4m3_value(uint8_t code)
{
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    assert(code <= 0x7E);
    if (e == 0)
        return ldexp((double)m / 8.0, -6);
    return ldexp(1.0 + (double)m / 8.0, e - 7);
}

/* Values of the 127 non-negative finite codes, filled from the decode rule
 * above on first use. */
static double e4m3_values[0x7F];
static int e4m3_values_ready = 0;

static double e4m3_code_value(int code)
{
    if (!e4m3_values_ready) {
        for (int c = 0; c <= 0x7E; c++)
            e4m3_values[c] = oracle_e4m3_value((uint8_t)c);
        e4m3_values_ready = 1;
    }
    return e4m3_values[code];
}

/* float -> E4M3 byte, for finite |v| <= 448.  The definition: the code whose
 * value is nearest to |v|, ties to the code with even (zero) last mantissa
 * bit, sign bit = sign of v (so -0 and small negatives give 0x80).  The 127
 * non-negative finite codes are increasing in value, so the bracketing pair is
 * found by bisection over the code values. */
uint8_t oracle_e4m3_encode(float v)
{
    uint8_t sign = (float_bits(v) & 0x80000000u) ? 0x80 : 0x00;
    double a = fabs((double)v);
    assert(a <= 448.0);
    /* largest code c with value(c) <= a */
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (e4m3_code_value(mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int c = lo;
    if (c < 0x7E) {
        double dlo = a - e4m3_code_value(c);
        double dhi = e4m3_code_value(c + 1) - a;
        if (dhi < dlo || (dhi == dlo && (c & 1)))
            c = c + 1;
    }
    return (uint8_t)(sign | (uint8_t)c);
}

/* UE8M0 scale exponent: the smallest integer k with a <= 448 * 2^k, i.e. the
 * power-of-two scale rounded UP so that no element of the block can exceed
 * the E4M3 range after scaling.  Evaluated exactly in double by search. */
int oracle_ue8m0_exponent(float a)
{
    double ad = (double)a;
    int k = 0;
    assert(a > 0.0f);
    while (ad > ldexp(448.0, k))
        k++;
    while (ad <= ldexp(448.0, k - 1))
        k--;
    return k;
}

/* OCP MX shared exponent for E4M3 elements (OCP Microscaling Formats
 * specification, conversion to MX: the shared exponent is floor(log2(a))
 * minus the largest exponent of the element format, which is 8 for E4M3
 * since 448 = 1.75 * 2^8): the largest integer s with 2^(s+8) <= a.
 * Evaluated exactly in double by search. */
int oracle_mx_exponent(float a)
{
    double ad = (double)a;
    assert(ad > 0.0 && isfinite(ad));
    int s = 0;
    while (ldexp(1.0, s + 8) > ad)
        s--;
    while (ldexp(1.0, s + 9) <= ad)
        s++;
    return s;
}

/* ------------------------------------------------------------------------ */
/* Layout: counts, offsets, stable slots, source-index maps                 */
/* ------------------------------------------------------------------------ */

enum { ORACLE_CONTIGUOUS = 0, ORACLE_MASKED = 1 };

/*
 * Pairs p = t*K + k are visited in ascending p.  e = topk_idx[p]:
 *   0 <= e < E  routed;  e == -1 unrouted (skipped);  anything else invalid
 *   (skipped and counted in status[1]).
 * count[e]  = number of routed pairs with expert e.
 * slot(p)   = number of routed pairs q < p with the same expert (a stable
 *             counting sort: rows of one expert keep ascending pair order).
 * Contiguous: segment of e starts at expert_offset[e], segments are padded to
 *             a multiple of `align` rows; row(p) = expert_offset[e] + slot(p).
 * Masked:     expert e owns rows [e*C, (e+1)*C); row(p) = e*C + slot(p) when
 *             slot(p) < C, otherwise the pair is dropped and counted in
 *             status[0]; recv_count[e] = min(count[e], C).
 * rank_offset[r] = expert_offset[r * E/R]: virtual rank r owns experts
 *             [r*E/R, (r+1)*E/R), which are rows rank_offset[r]..[r+1].
 * pair_to_row[p] = row(p) or -1; row_to_pair[row] = p for kept pairs and -1
 *             for every other row in [0, rows_capacity).
 * Returns 0, or -1 if the rows needed exceed rows_capacity.
 */
int oracle_dispatch_layout(int32_t T, int32_t K, int32_t E, int32_t R,
                           int32_t layout, int32_t align, int32_t capacity,
                           int64_t rows_capacity, const int32_t *topk_idx,
                           int32_t *expert_count, int32_t *recv_count,
                           int32_t *expert_offset, int32_t *rank_offset,
                           int32_t *pair_to_row, int32_t *row_to_pair,
                           int32_t *status)
{
    int64_t P = (int64_t)T * K;
    int32_t L = E / R;
    int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    assert(seen != NULL);

    status[0] = 0;
    status[1] = 0;
    for (int32_t e = 0; e < E; e++)
        expert_count[e] = 0;

    /* counts */
    for (int64_t p = 0; p < P; p++) {
        int32_t e = topk_idx[p];
        if (e >= 0 && e < E)
            expert_count[e]++;
        else if (e != -1)
            status[1]++;
    }

    /* segment offsets */
    expert_offset[0] = 0;
    for (int32_t e = 0; e < E; e++) {
        if (layout == ORACLE_CONTIGUOUS) {
            int32_t padded = ((expert_count[e] + align - 1) / align) * align;
            expert_offset[e + 1] = expert_offset[e] + padded;
            recv_count[e] = expert_count[e];
        } else {
            expert_offset[e + 1] = (e + 1) * capacity;
            recv_count[e] = expert_count[e] < capacity ? expert_count[e] : capacity;
            if (expert_count[e] > capacity)
                status[0] += expert_count[e] - capacity;
        }
    }
    for (int32_t r = 0; r <= R; r++)
        rank_offset[r] = expert_offset[r * L];

    if ((int64_t)expert_offset[E] > rows_capacity) {
        free(seen);
        return -1;
    }

    for (int64_t row = 0; row < rows_capacity; row++)
        row_to_pair[row] = -1;

    /* stable slots and both maps */
    for (int64_t p = 0; p < P; p++) {
        int32_t e = topk_idx[p];
        if (!(e >= 0 && e < E)) {
            pair_to_row[p] = -1;
            continue;
        }
        int32_t slot = seen[e]++;
        int32_t row;
        if (layout == ORACLE_CONTIGUOUS)
            row = expert_offset[e] + slot;
        else
            row = slot < capacity ? e * capacity + slot : -1;
        pair_to_row[p] = row;
        if (row >= 0)
            row_to_pair[row] = (int32_t)p;
    }
    free(seen);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dispatch: row permutation, optional fused FP8 1x128 quantization          */
/* ------------------------------------------------------------------------ */

enum { ORACLE_QUANT_NONE = 0, ORACLE_QUANT_FP8_F32 = 1, ORACLE_QUANT_FP8_UE8M0 = 2, ORACLE_QUANT_MXFP8 = 3 };

#define ORACLE_BLOCK 128          /* activation quantization group, 1 x 128 */
#define ORACLE_AMAX_FLOOR 1e-10f  /* keeps the scale of an all-zero block finite */
#define ORACLE_MX_BLOCK 32        /* MXFP8 group, 1 x 32 */

/* Quantize one token row (H channels) into E4M3 bytes `q` and its per-block
 * scales.  For block b (channels 128b .. 128b+127):
 *   amax = max |x|, a = max(amax, 1e-10)
 *   fp32 scales : s = a / 448 (binary32 division), q = E4M3(clamp(x / s, +-448))
 *   UE8M0 scales: k = smallest integer with a <= 448 * 2^k, scale byte k + 127,
 *                 q = E4M3(x * 2^-k)  (exact scaling; the clamp cannot bind)
 * Scales go to s32[b] (fp32) or byte b of the packed little-endian words w32
 * (four blocks per word, unused high bytes zero). */
static void quantize_token_row(int32_t H, int32_t quant, const uint16_t *x,
                               uint8_t *q, float *s32, uint32_t *w32)
{
    if (quant == ORACLE_QUANT_MXFP8) {
        /* MXFP8 (1x32, OCP MX): per block of 32 channels, amax and the floor a
         * as above, shared exponent s = oracle_mx_exponent(a), scale byte
         * s + 127 (E8M0, byte b of the row's scale bytes, passed in w32),
         * q = E4M3(clamp(x * 2^-s, +-448)); the clamp binds when a * 2^-s
         * exceeds 448 (it lies in [256, 512)). */
        uint8_t *e8 = (uint8_t *)w32;
        for (int32_t b = 0; b < H / ORACLE_MX_BLOCK; b++) {
            const uint16_t *xb = x + (int64_t)b * ORACLE_MX_BLOCK;
            float amax = 0.0f;
            for (int j = 0; j < ORACLE_MX_BLOCK; j++) {
                float v = fabsf(oracle_bf16_to_float(xb[j]));
                assert(isfinite(v));
                if (v > amax)
                    amax = v;
            }
            float a = amax > ORACLE_AMAX_FLOOR ? amax : ORACLE_AMAX_FLOOR;
            int sx = oracle_mx_exponent(a);
            assert(sx + 127 >= 1 && sx + 127 <= 254);
            e8[b] = (uint8_t)(sx + 127);
            for (int j = 0; j < ORACLE_MX_BLOCK; j++) {
                float v = ldexpf(oracle_bf16_to_float(xb[j]), -sx);
                if (v > 448.0f)
                    v = 448.0f;
                if (v < -448.0f)
                    v = -448.0f;
                q[(int64_t)b * ORACLE_MX_BLOCK + j] = oracle_e4m3_encode(v);
            }
        }
        (void)s32;
        return;
    }
    int32_t NB = H / ORACLE_BLOCK;
    if (quant == ORACLE_QUANT_FP8_UE8M0)
        for (int32_t w = 0; w < (NB + 3) / 4; w++)
            w32[w] = 0;
    for (int32_t b = 0; b < NB; b++) {
        const uint16_t *xb = x + (int64_t)b * ORACLE_BLOCK;
        float amax = 0.0f;
        for (int j = 0; j < ORACLE_BLOCK; j++) {
            float v = fabsf(oracle_bf16_to_float(xb[j]));
            assert(isfinite(v));
            if (v > amax)
                amax = v;
        }
        float a = amax > ORACLE_AMAX_FLOOR ? amax : ORACLE_AMAX_FLOOR;
        if (quant == ORACLE_QUANT_FP8_F32) {
            float s = a / 448.0f;
            s32[b] = s;
            for (int j = 0; j < ORACLE_BLOCK; j++) {
                float v = oracle_bf16_to_float(xb[j]) / s;
                if (v > 448.0f)
                    v = 448.0f;
                if (v < -448.0f)
                    v = -448.0f;
                q[(int64_t)b * ORACLE_BLOCK + j] = oracle_e4m3_encode(v);
            }
        } else {
            int k = oracle_ue8m0_exponent(a);
            assert(k + 127 >= 0 && k + 127 <= 254);
            w32[b / 4] |= (uint32_t)(k + 127) << (8 * (b % 4));
            for (int j = 0; j < ORACLE_BLOCK; j++) {
                float v = ldexpf(oracle_bf16_to_float(xb[j]), -k);
                q[(int64_t)b * ORACLE_BLOCK + j] = oracle_e4m3_encode(v);
            }
        }
    }
}

/*
 * For every kept pair p (pair_to_row[p] >= 0) of token t = p / K:
 *   quant NONE : out_x[row, :] = x[t, :]           (bf16 bit copy, H*2 bytes)
 *   quant FP8  : out_x[row, :] = E4M3 bytes of x[t, :] (H bytes) and the
 *                row's scales in out_scale (fp32 [rows, H/128], packed
 *                UE8M0 uint32 [rows, ceil(H/512)], or MXFP8 E8M0 bytes
 *                uint8 [rows, H/32]).
 *   out_row_weight[row] = topk_w[p] when both pointers are given.
 * Quantization happens once per token; every kept row of the token receives
 * the same bytes.  Rows that no kept pair maps to are not written.
 */
void oracle_dispatch(int32_t T, int32_t K, int32_t H, int32_t quant,
                     const uint16_t *x, const float *topk_w,
                     const int32_t *pair_to_row, void *out_x, void *out_scale,
                     float *out_row_weight)
{
    int32_t NB = H / ORACLE_BLOCK;
    int32_t NW = (NB + 3) / 4;
    /* Tokens are independent (each writes only its own kept rows), so they
     * may be split over threads; the bytes do not depend on the split.  The
     * E4M3 value table is filled here, before any thread reads it. */
    (void)e4m3_code_value(0);
#pragma omp parallel
    {
    uint8_t *q = NULL;
    float *s32 = NULL;
    uint32_t *w32 = NULL;
    if (quant != ORACLE_QUANT_NONE) {
        q = (uint8_t *)malloc((size_t)H);
        s32 = (float *)malloc(sizeof(float) * (size_t)(NB > 0 ? NB : 1));
        /* packed UE8M0 words, or the MX scale bytes (H/32 <= 4 * NW words) */
        w32 = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(4 * NW > 0 ? 4 * NW : 1));
        assert(q && s32 && w32);
    }
#pragma omp for schedule(static)
    for (int32_t t = 0; t < T; t++) {
        const uint16_t *xt = x + (int64_t)t * H;
        int any = 0;
        for (int32_t k = 0; k < K; k++)
            any |= pair_to_row[(int64_t)t * K + k] >= 0;
        if (!any)
            continue;
        if (quant != ORACLE_QUANT_NONE)
            quantize_token_row(H, quant, xt, q, s32, w32);
        for (int32_t k = 0; k < K; k++) {
            int64_t p = (int64_t)t * K + k;
            int32_t row = pair_to_row[p];
            if (row < 0)
                continue;
            if (quant == ORACLE_QUANT_NONE) {
                uint16_t *dst = (uint16_t *)out_x + (int64_t)row * H;
                for (int32_t j = 0; j < H; j++)
                    dst[j] = xt[j];
            } else {
                uint8_t *dst = (uint8_t *)out_x + (int64_t)row * H;
                for (int32_t j = 0; j < H; j++)
                    dst[j] = q[j];
                if (quant == ORACLE_QUANT_FP8_F32) {
                    float *sd = (float *)out_scale + (int64_t)row * NB;
                    for (int32_t b = 0; b < NB; b++)
                        sd[b] = s32[b];
                } else if (quant == ORACLE_QUANT_MXFP8) {
                    int32_t NX = H / ORACLE_MX_BLOCK;
                    uint8_t *sd = (uint8_t *)out_scale + (int64_t)row * NX;
                    memcpy(sd, w32, (size_t)NX);
                } else {
                    uint32_t *wd = (uint32_t *)out_scale + (int64_t)row * NW;
                    for (int32_t w = 0; w < NW; w++)
                        wd[w] = w32[w];
                }
            }
            if (out_row_weight != NULL && topk_w != NULL)
                out_row_weight[row] = topk_w[p];
        }
    }
    free(q);
    free(s32);
    free(w32);
    }
}

/* ------------------------------------------------------------------------ */
/* Combine: router-weighted top-k reduction back to token order             */
/* ------------------------------------------------------------------------ */

/*
 * out[t, j] = bf16_RNE( sum over k = 0..K-1 with row = pair_to_row[t*K+k] >= 0
 *                        of topk_w[t*K+k] * y[row, j] )
 * accumulated in binary32 starting from +0, in ascending k, the product and the
 * sum each rounded to binary32 (no fused multiply-add).  A token with no kept
 * pair gives +0.  The weights are the caller's router weights as given (no
 * renormalisation over kept pairs), and nothing is reduced afterwards.
 */
void oracle_combine(int32_t T, int32_t K, int32_t H, const uint16_t *y,
                    const float *topk_w, const int32_t *pair_to_row,
                    uint16_t *out)
{
    /* tokens are independent: the same sums in the same order on any thread */
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; t++) {
        for (int32_t j = 0; j < H; j++) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; k++) {
                int64_t p = (int64_t)t * K + k;
                int32_t row = pair_to_row[p];
                if (row < 0)
                    continue;
                float prod = topk_w[p] * oracle_bf16_to_float(y[(int64_t)row * H + j]);
                acc = acc + prod;
            }
            out[(int64_t)t * H + j] = oracle_bf16_rne(acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Per-rank deduplicated exchange: send each token once per destination rank */
/* ------------------------------------------------------------------------ */

/*
 * The per-rank layout that the V1 dispatch computed in a separate pre-pass
 * (get_dispatch_layout, named on page "moe: add DeepEP V2 ElasticBuffer
 * support to MoE token dispatcher", Motivation): which ranks each token must
 * reach and how many tokens each rank receives.  Readings taken here:
 *   - expert e belongs to rank e / (E/R); token t is in rank r when at least
 *     one of its pairs has a valid id (0 <= id < E) of rank r.  Ids -1 and
 *     invalid ids make no rank; a masked-capacity drop on the receiver does
 *     not change membership (the sender does not know it).
 *   - rank r's rows are rank_token_offset[r] .. [r+1], its tokens in
 *     ascending t, with no padding: rank_token_offset is the exclusive scan
 *     of rank_token_count.
 *   - token_rank_row[t*R + r] = that row, or -1 when t is not in rank r
 *     (is_token_in_rank is token_rank_row >= 0); rank_row_to_token[row] = t,
 *     and -1 for every other row in [0, rank_rows_capacity).
 * Returns 0, or -1 if the rows exceed rank_rows_capacity.
 */
int oracle_rank_layout(int32_t T, int32_t K, int32_t E, int32_t R,
                       int64_t rank_rows_capacity, const int32_t *topk_idx,
                       int32_t *rank_token_count, int32_t *rank_token_offset,
                       int32_t *token_rank_row, int32_t *rank_row_to_token)
{
    int32_t L = E / R;
    for (int32_t r = 0; r < R; r++)
        rank_token_count[r] = 0;
    /* membership first: token_rank_row holds 1 / 0 until rows are assigned */
    for (int32_t t = 0; t < T; t++) {
        for (int32_t r = 0; r < R; r++)
            token_rank_row[(int64_t)t * R + r] = 0;
        for (int32_t k = 0; k < K; k++) {
            int32_t e = topk_idx[(int64_t)t * K + k];
            if (e >= 0 && e < E)
                token_rank_row[(int64_t)t * R + e / L] = 1;
        }
        for (int32_t r = 0; r < R; r++)
            rank_token_count[r] += token_rank_row[(int64_t)t * R + r];
    }
    rank_token_offset[0] = 0;
    for (int32_t r = 0; r < R; r++)
        rank_token_offset[r + 1] = rank_token_offset[r] + rank_token_count[r];
    if ((int64_t)rank_token_offset[R] > rank_rows_capacity)
        return -1;
    for (int64_t row = 0; row < rank_rows_capacity; row++)
        rank_row_to_token[row] = -1;
    for (int32_t r = 0; r < R; r++) {
        int32_t next = rank_token_offset[r];
        for (int32_t t = 0; t < T; t++) {
            int32_t *slot = &token_rank_row[(int64_t)t * R + r];
            if (*slot) {
                *slot = next;
                rank_row_to_token[next] = t;
                next++;
            } else {
                *slot = -1;
            }
        }
    }
    return 0;
}

/* Bytes of one dispatched row and of its scales, per quant mode. */
static int64_t row_bytes(int32_t H, int32_t quant)
{
    return quant == ORACLE_QUANT_NONE ? 2 * (int64_t)H : (int64_t)H;
}

static int64_t scale_bytes(int32_t H, int32_t quant)
{
    int32_t NB = H / ORACLE_BLOCK;
    if (quant == ORACLE_QUANT_FP8_F32)
        return 4 * (int64_t)NB;
    if (quant == ORACLE_QUANT_FP8_UE8M0)
        return 4 * (int64_t)((NB + 3) / 4);
    if (quant == ORACLE_QUANT_MXFP8)
        return (int64_t)(H / ORACLE_MX_BLOCK);
    return 0;
}

/*
 * Deduplicated dispatch (sender side): each token's row, quantized as in
 * oracle_dispatch, is written once per rank it is in, to row
 * token_rank_row[t*R + r] of the per-rank send buffer.  This is dispatch
 * with the R (token, rank) slots of a token in place of its K pairs.
 */
void oracle_dispatch_dedup(int32_t T, int32_t R, int32_t H, int32_t quant,
                           const uint16_t *x, const int32_t *token_rank_row,
                           void *send_x, void *send_scale)
{
    oracle_dispatch(T, R, H, quant, x, NULL, token_rank_row, send_x, send_scale, NULL);
}

/*
 * Receive-side expansion: every kept pair p = t*K+k of expert e (rank
 * r = e / (E/R)) gets the bytes of its token's row on rank r:
 *   out_x[pair_to_row[p], :] = send_x[token_rank_row[t*R + r], :]
 * and the same for the row's scales.  Other rows are not written.
 */
void oracle_expand(int32_t T, int32_t K, int32_t E, int32_t R, int32_t H, int32_t quant,
                   const int32_t *topk_idx, const void *send_x, const void *send_scale,
                   const int32_t *token_rank_row, const int32_t *pair_to_row,
                   void *out_x, void *out_scale)
{
    int32_t L = E / R;
    int64_t rb = row_bytes(H, quant), sb = scale_bytes(H, quant);
    for (int32_t t = 0; t < T; t++) {
        for (int32_t k = 0; k < K; k++) {
            int64_t p = (int64_t)t * K + k;
            int32_t row = pair_to_row[p];
            if (row < 0)
                continue;
            int32_t e = topk_idx[p];
            int32_t src = token_rank_row[(int64_t)t * R + e / L];
            assert(src >= 0);
            memcpy((uint8_t *)out_x + row * rb, (const uint8_t *)send_x + src * rb, (size_t)rb);
            if (sb > 0)
                memcpy((uint8_t *)out_scale + row * sb, (const uint8_t *)send_scale + src * sb, (size_t)sb);
        }
    }
}

/*
 * Partial combine (receiver side, before the return trip): for every token t
 * and rank r it is in,
 *   partial[token_rank_row[t*R+r], j] = bf16_RNE( sum over k ascending with
 *       valid id e of rank r and row = pair_to_row[t*K+k] >= 0
 *       of topk_w[t*K+k] * y[row, j] )
 * in binary32 from +0, product and sum each rounded.  A (token, rank) whose
 * pairs were all dropped gives +0.  The pages name the option of a second
 * reduction (the VLLM_DEEPEP_V2_ALLOW_MULTIPLE_REDUCTION switch on page vLLM
 * tools/ep_kernels, commit message); the bf16 partial sums are the reading
 * taken here.
 */
void oracle_combine_partial(int32_t T, int32_t K, int32_t E, int32_t R, int32_t H,
                            const int32_t *topk_idx, const uint16_t *y, const float *topk_w,
                            const int32_t *pair_to_row, const int32_t *token_rank_row,
                            uint16_t *partial)
{
    int32_t L = E / R;
    for (int32_t t = 0; t < T; t++) {
        for (int32_t r = 0; r < R; r++) {
            int32_t dst = token_rank_row[(int64_t)t * R + r];
            if (dst < 0)
                continue;
            for (int32_t j = 0; j < H; j++) {
                float acc = 0.0f;
                for (int32_t k = 0; k < K; k++) {
                    int64_t p = (int64_t)t * K + k;
                    int32_t e = topk_idx[p];
                    int32_t row = pair_to_row[p];
                    if (!(e >= 0 && e < E) || e / L != r || row < 0)
                        continue;
                    float prod = topk_w[p] * oracle_bf16_to_float(y[(int64_t)row * H + j]);
                    acc = acc + prod;
                }
                partial[(int64_t)dst * H + j] = oracle_bf16_rne(acc);
            }
        }
    }
}

/*
 * Final reduction on the source rank, after the return trip:
 *   out[t, j] = bf16_RNE( sum over r ascending with q = token_rank_row[t*R+r]
 *                          >= 0 of partial[q, j] )
 * in binary32 from +0.  A token in no rank gives +0.
 */
void oracle_combine_reduce(int32_t T, int32_t R, int32_t H, const uint16_t *partial,
                           const int32_t *token_rank_row, uint16_t *out)
{
    for (int32_t t = 0; t < T; t++) {
        for (int32_t j = 0; j < H; j++) {
            float acc = 0.0f;
            for (int32_t r = 0; r < R; r++) {
                int32_t q = token_rank_row[(int64_t)t * R + r];
                if (q >= 0)
                    acc = acc + oracle_bf16_to_float(partial[(int64_t)q * H + j]);
            }
            out[(int64_t)t * H + j] = oracle_bf16_rne(acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Adapters for grouped-GEMM consumers: per-row experts, masked <-> contiguous */
/* repack, MN-major scales                                                    */
/* ------------------------------------------------------------------------ */

/*
 * The pages add masked-slab repack kernels and grouped-GEMM adapters for
 * contiguous prefill and masked decode, with fp32 and packed UE8M0 scales
 * (page "[Feature] Add DeepEPv2 (ElasticBuffer) MoE A2A backend",
 * Implementation).  Readings taken here: a contiguous grouped GEMM reads one
 * expert index per row (-1 for rows it must skip); a masked slab is repacked
 * by moving expert e's first recv_count[e] rows back to back, each segment
 * padded to `align` rows, and expert outputs come back the same way; scales
 * are read in MN-major order (scale j of row r at j*ld + r) with the leading
 * dimension rounded up to 16 bytes.
 */

/* row_expert[r] = e for every row r that holds one of expert e's received
 * pairs (rows off[e] .. off[e] + recv_count[e] - 1, where off[e] =
 * expert_offset[e]), -1 for every other row in [0, rows). */
void oracle_row_expert(int32_t E, const int32_t *expert_offset, const int32_t *recv_count,
                       int64_t rows, int32_t *row_expert)
{
    for (int64_t r = 0; r < rows; r++)
        row_expert[r] = -1;
    for (int32_t e = 0; e < E; e++)
        for (int32_t s = 0; s < recv_count[e]; s++)
            row_expert[(int64_t)expert_offset[e] + s] = e;
}

/* Masked slab -> contiguous segments: out_offset[0] = 0, out_offset[e+1] =
 * out_offset[e] + recv_count[e] rounded up to `align`; row s < recv_count[e]
 * of expert e moves from e*C + s to out_offset[e] + s, with its scales.
 * Padding rows are not written; out_row_expert covers [0, out_rows).
 * Returns -1 if the segments exceed out_rows. */
int oracle_repack_masked_to_contiguous(int32_t E, int32_t C, int32_t align, int32_t H, int32_t quant,
                                       const int32_t *recv_count, const void *x, const void *scale,
                                       int64_t out_rows, void *out_x, void *out_scale,
                                       int32_t *out_offset, int32_t *out_row_expert)
{
    int64_t rb = row_bytes(H, quant), sb = scale_bytes(H, quant);
    out_offset[0] = 0;
    for (int32_t e = 0; e < E; e++)
        out_offset[e + 1] = out_offset[e] + (recv_count[e] + align - 1) / align * align;
    if ((int64_t)out_offset[E] > out_rows)
        return -1;
    for (int32_t e = 0; e < E; e++) {
        for (int32_t s = 0; s < recv_count[e]; s++) {
            int64_t src = (int64_t)e * C + s, dst = (int64_t)out_offset[e] + s;
            memcpy((uint8_t *)out_x + dst * rb, (const uint8_t *)x + src * rb, (size_t)rb);
            if (sb > 0)
                memcpy((uint8_t *)out_scale + dst * sb, (const uint8_t *)scale + src * sb, (size_t)sb);
        }
    }
    oracle_row_expert(E, out_offset, recv_count, out_rows, out_row_expert);
    return 0;
}

/* Contiguous expert outputs -> masked slab: y_masked[e*C + s] = y[offset[e] + s]
 * for s < recv_count[e] (bf16 rows of H channels); other slab rows are not
 * written.  `offset` is the out_offset of the masked-to-contiguous repack. */
void oracle_repack_contiguous_to_masked(int32_t E, int32_t C, int32_t H, const int32_t *recv_count,
                                        const int32_t *offset, const uint16_t *y, uint16_t *y_masked)
{
    for (int32_t e = 0; e < E; e++)
        for (int32_t s = 0; s < recv_count[e]; s++)
            memcpy(y_masked + ((int64_t)e * C + s) * H, y + ((int64_t)offset[e] + s) * H,
                   sizeof(uint16_t) * (size_t)H);
}

/* Row-major 32-bit scales [rows, S] -> MN-major [S, ld]: out[j*ld + r] =
 * in[r*S + j] for r < rows and 0 for rows <= r < ld, ld = rows rounded up to a
 * multiple of 4 (16 bytes). */
void oracle_scales_mn_major(int64_t rows, int32_t S, const uint32_t *in, uint32_t *out)
{
    int64_t ld = (rows + 3) / 4 * 4;
    for (int32_t j = 0; j < S; j++)
        for (int64_t r = 0; r < ld; r++)
            out[(int64_t)j * ld + r] = r < rows ? in[r * S + j] : 0u;
}

/* ------------------------------------------------------------------------ */
/* Array forms of the codecs, so the tests can sweep them in bulk           */
/* ------------------------------------------------------------------------ */

/* Threads for the token loops of oracle_dispatch and oracle_combine (OpenMP);
 * the layout is serial.  Results do not depend on the count. */
void oracle_set_threads(int32_t n)
{
    omp_set_num_threads(n < 1 ? 1 : n);
}

int32_t oracle_get_threads(void)
{
    return omp_get_max_threads();
}

void oracle_bf16_rne_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_bf16_rne(in[i]);
}

void oracle_e4m3_encode_array(const float *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_e4m3_encode(in[i]);
}

void oracle_mx_exponent_array(const float *in, int32_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_mx_exponent(in[i]);
}

void oracle_ue8m0_exponent_array(const float *in, int32_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_ue8m0_exponent(in[i]);
}
