/*
 * Drives every exported function of oracle/oracle.c over small seeded inputs
 * (both layouts, every activation format, invalid and unrouted ids, masked
 * overflow, one and four threads).  Built together with oracle.c under
 * AddressSanitizer and UBSan by tests/test_oracle_sanitized.py; the values
 * are checked elsewhere (the oracle pins), this program only has to run
 * clean.  Exit status 0 means every call returned as expected.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_float(uint16_t b);
uint16_t oracle_bf16_rne(float f);
double oracle_e4m3_value(uint8_t code);
uint8_t oracle_e4m3_encode(float v);
int oracle_ue8m0_exponent(float a);
int oracle_mx_exponent(float a);
int oracle_dispatch_layout(int32_t T, int32_t K, int32_t E, int32_t R, int32_t layout, int32_t align,
                           int32_t capacity, int64_t rows_capacity, const int32_t *topk_idx,
                           int32_t *expert_count, int32_t *recv_count, int32_t *expert_offset,
                           int32_t *rank_offset, int32_t *pair_to_row, int32_t *row_to_pair, int32_t *status);
void oracle_dispatch(int32_t T, int32_t K, int32_t H, int32_t quant, const uint16_t *x, const float *topk_w,
                     const int32_t *pair_to_row, void *out_x, void *out_scale, float *out_row_weight);
void oracle_combine(int32_t T, int32_t K, int32_t H, const uint16_t *y, const float *topk_w,
                    const int32_t *pair_to_row, uint16_t *out);
int oracle_rank_layout(int32_t T, int32_t K, int32_t E, int32_t R, int64_t rank_rows_capacity,
                       const int32_t *topk_idx, int32_t *rank_token_count, int32_t *rank_token_offset,
                       int32_t *token_rank_row, int32_t *rank_row_to_token);
void oracle_dispatch_dedup(int32_t T, int32_t R, int32_t H, int32_t quant, const uint16_t *x,
                           const int32_t *token_rank_row, void *send_x, void *send_scale);
void oracle_expand(int32_t T, int32_t K, int32_t E, int32_t R, int32_t H, int32_t quant,
                   const int32_t *topk_idx, const void *send_x, const void *send_scale,
                   const int32_t *token_rank_row, const int32_t *pair_to_row, void *out_x, void *out_scale);
void oracle_combine_partial(int32_t T, int32_t K, int32_t E, int32_t R, int32_t H, const int32_t *topk_idx,
                            const uint16_t *y, const float *topk_w, const int32_t *pair_to_row,
                            const int32_t *token_rank_row, uint16_t *partial);
void oracle_combine_reduce(int32_t T, int32_t R, int32_t H, const uint16_t *partial,
                           const int32_t *token_rank_row, uint16_t *out);
void oracle_row_expert(int32_t E, const int32_t *expert_offset, const int32_t *recv_count, int64_t rows,
                       int32_t *row_expert);
int oracle_repack_masked_to_contiguous(int32_t E, int32_t C, int32_t align, int32_t H, int32_t quant,
                                       const int32_t *recv_count, const void *x, const void *scale,
                                       int64_t out_rows, void *out_x, void *out_scale, int32_t *out_offset,
                                       int32_t *out_row_expert);
void oracle_repack_contiguous_to_masked(int32_t E, int32_t C, int32_t H, const int32_t *recv_count,
                                        const int32_t *offset, const uint16_t *y, uint16_t *y_masked);
void oracle_scales_mn_major(int64_t rows, int32_t S, const uint32_t *in, uint32_t *out);
void oracle_set_threads(int32_t n);
int32_t oracle_get_threads(void);
void oracle_bf16_rne_array(const float *in, uint16_t *out, int64_t n);
void oracle_e4m3_encode_array(const float *in, uint8_t *out, int64_t n);
void oracle_mx_exponent_array(const float *in, int32_t *out, int64_t n);
void oracle_ue8m0_exponent_array(const float *in, int32_t *out, int64_t n);

static uint64_t rng = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void)
{
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(rng >> 32);
}

/* a finite value of magnitude about 2^-8 .. 2^8 with a random sign */
static float next_value(void)
{
    const float u = (float)(next_u32() >> 8) / 16777216.0f;
    const int ex = (int)(next_u32() % 17) - 8;
    const float v = ldexpf(0.5f + u, ex);
    return (next_u32() & 1) ? -v : v;
}

static void *xalloc(size_t n)
{
    void *p = calloc(n ? n : 1, 1);
    if (p == NULL) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void fail(const char *what)
{
    fprintf(stderr, "unexpected result: %s\n", what);
    exit(1);
}

static int64_t row_bytes(int32_t H, int32_t quant) { return quant == 0 ? 2 * (int64_t)H : H; }

static int64_t scale_bytes(int32_t H, int32_t quant)
{
    if (quant == 1)
        return 4 * (int64_t)(H / 128);
    if (quant == 2)
        return 4 * (int64_t)((H / 128 + 3) / 4);
    if (quant == 3)
        return H / 32;
    return 0;
}

/* One layout + dispatch + combine + per-rank chain + adapters pass. */
static void run_case(int32_t T, int32_t K, int32_t E, int32_t R, int32_t H, int32_t layout, int32_t align,
                     int32_t capacity, int32_t quant)
{
    const int64_t P = (int64_t)T * K;
    const int64_t rows = layout == 0 ? P + (int64_t)E * (align - 1) : (int64_t)E * capacity;
    int32_t *idx = xalloc(sizeof(int32_t) * (size_t)P);
    float *w = xalloc(sizeof(float) * (size_t)P);
    for (int64_t p = 0; p < P; p++) {
        const uint32_t r = next_u32() % 100;
        idx[p] = r < 3 ? -1 : (r < 5 ? E + (int32_t)(next_u32() % 5) : (int32_t)(next_u32() % (uint32_t)E));
        if (r == 5)
            idx[p] = -2;  /* invalid, negative */
        w[p] = (float)(next_u32() % 1000) / 1000.0f;
    }
    uint16_t *x = xalloc(sizeof(uint16_t) * (size_t)T * H);
    for (int64_t i = 0; i < (int64_t)T * H; i++)
        x[i] = oracle_bf16_rne(next_value());

    int32_t *cnt = xalloc(sizeof(int32_t) * E), *recv = xalloc(sizeof(int32_t) * E);
    int32_t *eoff = xalloc(sizeof(int32_t) * (E + 1)), *roff = xalloc(sizeof(int32_t) * (R + 1));
    int32_t *p2r = xalloc(sizeof(int32_t) * (size_t)P), *r2p = xalloc(sizeof(int32_t) * (size_t)rows);
    int32_t status[2];
    if (oracle_dispatch_layout(T, K, E, R, layout, align, capacity, rows, idx, cnt, recv, eoff, roff, p2r, r2p,
                               status) != 0)
        fail("layout within capacity");
    if (T > 0 && oracle_dispatch_layout(T, K, E, R, layout, align, capacity, 0, idx, cnt, recv, eoff, roff, p2r,
                                        r2p, status) == 0 && layout == 0 && P > 0)
        fail("layout beyond capacity");
    oracle_dispatch_layout(T, K, E, R, layout, align, capacity, rows, idx, cnt, recv, eoff, roff, p2r, r2p, status);

    const int64_t rb = row_bytes(H, quant), sb = scale_bytes(H, quant);
    uint8_t *ox = xalloc((size_t)(rows * rb));
    uint8_t *osc = xalloc((size_t)(rows * (sb ? sb : 4)));
    float *orw = xalloc(sizeof(float) * (size_t)rows);
    oracle_dispatch(T, K, H, quant, x, w, p2r, ox, sb ? osc : NULL, orw);

    uint16_t *y = xalloc(sizeof(uint16_t) * (size_t)(rows * H));
    for (int64_t i = 0; i < rows * H; i++)
        y[i] = oracle_bf16_rne(next_value());
    uint16_t *out = xalloc(sizeof(uint16_t) * (size_t)T * H);
    oracle_combine(T, K, H, y, w, p2r, out);

    /* per-rank chain */
    const int64_t rrows = (int64_t)T * R;
    int32_t *rcnt = xalloc(sizeof(int32_t) * R), *rtoff = xalloc(sizeof(int32_t) * (R + 1));
    int32_t *trr = xalloc(sizeof(int32_t) * (size_t)rrows), *rr2t = xalloc(sizeof(int32_t) * (size_t)rrows);
    if (oracle_rank_layout(T, K, E, R, rrows, idx, rcnt, rtoff, trr, rr2t) != 0)
        fail("rank layout within capacity");
    uint8_t *sx = xalloc((size_t)(rrows * rb));
    uint8_t *ss = xalloc((size_t)(rrows * (sb ? sb : 4)));
    oracle_dispatch_dedup(T, R, H, quant, x, trr, sx, sb ? ss : NULL);
    uint8_t *ex = xalloc((size_t)(rows * rb));
    uint8_t *es = xalloc((size_t)(rows * (sb ? sb : 4)));
    oracle_expand(T, K, E, R, H, quant, idx, sx, sb ? ss : NULL, trr, p2r, ex, sb ? es : NULL);
    uint16_t *part = xalloc(sizeof(uint16_t) * (size_t)(rrows * H));
    oracle_combine_partial(T, K, E, R, H, idx, y, w, p2r, trr, part);
    uint16_t *out2 = xalloc(sizeof(uint16_t) * (size_t)T * H);
    oracle_combine_reduce(T, R, H, part, trr, out2);

    /* adapters */
    int32_t *rexp = xalloc(sizeof(int32_t) * (size_t)rows);
    oracle_row_expert(E, eoff, recv, rows, rexp);
    if (layout == 1) {
        const int32_t a2 = 4;
        const int64_t crows = (int64_t)E * capacity + (int64_t)E * (a2 - 1);
        uint8_t *cx = xalloc((size_t)(crows * rb));
        uint8_t *cs = xalloc((size_t)(crows * (sb ? sb : 4)));
        int32_t *coff = xalloc(sizeof(int32_t) * (E + 1)), *crexp = xalloc(sizeof(int32_t) * (size_t)crows);
        if (oracle_repack_masked_to_contiguous(E, capacity, a2, H, quant, recv, ox, sb ? osc : NULL, crows, cx,
                                               sb ? cs : NULL, coff, crexp) != 0)
            fail("repack within capacity");
        uint16_t *yc = xalloc(sizeof(uint16_t) * (size_t)(crows * H));
        for (int64_t i = 0; i < crows * H; i++)
            yc[i] = oracle_bf16_rne(next_value());
        uint16_t *ym = xalloc(sizeof(uint16_t) * (size_t)(rows * H));
        oracle_repack_contiguous_to_masked(E, capacity, H, recv, coff, yc, ym);
        free(cx); free(cs); free(coff); free(crexp); free(yc); free(ym);
    }
    if (sb > 0 && quant != 3) {
        const int32_t S = (int32_t)(sb / 4);
        const int64_t ld = (rows + 3) / 4 * 4;
        uint32_t *mn = xalloc(sizeof(uint32_t) * (size_t)(S * ld));
        oracle_scales_mn_major(rows, S, (const uint32_t *)osc, mn);
        free(mn);
    }

    free(idx); free(w); free(x); free(cnt); free(recv); free(eoff); free(roff); free(p2r); free(r2p);
    free(ox); free(osc); free(orw); free(y); free(out); free(rcnt); free(rtoff); free(trr); free(rr2t);
    free(sx); free(ss); free(ex); free(es); free(part); free(out2); free(rexp);
}

int main(void)
{
    /* codecs over their whole domains */
    for (uint32_t b = 0; b < 65536; b++) {
        const float f = oracle_bf16_to_float((uint16_t)b);
        if (isfinite(f)) {  /* the codecs take finite inputs only */
            (void)oracle_bf16_rne(f);
            if (fabsf(f) <= 448.0f)
                (void)oracle_e4m3_encode(f);  /* its callers clamp to the E4M3 range first */
            if (f > 0.0f) {
                (void)oracle_ue8m0_exponent(f);
                (void)oracle_mx_exponent(f);
            }
        }
    }
    for (int c = 0; c <= 0x7E; c++)  /* the finite non-negative codes */
        (void)oracle_e4m3_value((uint8_t)c);
    enum { N = 4096 };
    float *in = xalloc(sizeof(float) * N);
    for (int i = 0; i < N; i++)
        in[i] = fabsf(next_value()) + 1e-10f;
    uint16_t *b16 = xalloc(sizeof(uint16_t) * N);
    uint8_t *e8 = xalloc(N);
    int32_t *ex = xalloc(sizeof(int32_t) * N);
    oracle_bf16_rne_array(in, b16, N);
    oracle_e4m3_encode_array(in, e8, N);
    oracle_mx_exponent_array(in, ex, N);
    oracle_ue8m0_exponent_array(in, ex, N);
    free(in); free(b16); free(e8); free(ex);

    for (int threads = 1; threads <= 4; threads += 3) {
        oracle_set_threads(threads);
        if (oracle_get_threads() != threads)
            fail("thread count");
        for (int32_t quant = 0; quant <= 3; quant++) {
            run_case(37, 3, 10, 2, 256, 0, 4, 1, quant);     /* contiguous, ragged */
            run_case(50, 4, 12, 3, 512, 1, 1, 5, quant);     /* masked with overflow */
            run_case(1, 1, 1, 1, 128, 0, 1, 1, quant);       /* one pair */
            run_case(0, 2, 8, 2, 128, 1, 1, 2, quant);       /* zero tokens */
            run_case(64, 8, 16, 4, 640, 0, 8, 1, quant);     /* H with a partial UE8M0 word */
        }
    }
    oracle_set_threads(1);
    puts("oracle ran clean");
    return 0;
}
