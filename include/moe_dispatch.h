/*
 * moe_dispatch.h -- C ABI of the MI355X (gfx950) MoE token dispatch / combine
 * library (libmoe_dispatch.so).
 *
 * The library computes, on one GPU, the data-parallel part of an
 * expert-parallel MoE layer's token exchange: from router top-k expert ids it
 * builds the dispatch layout, permutes (optionally FP8-quantizes) token rows
 * into that layout, and reduces expert outputs back to token order with the
 * router weights.  Destination ranks are virtual: rank r owns the contiguous
 * row range [rank_offset[r], rank_offset[r+1]) of the device buffers, which is
 * what a real expert-parallel exchange would send to rank r.  There is no
 * transfer between GPUs.
 *
 * Pages cited below by title and section:
 *   [V2-PR]  "moe: add DeepEP V2 ElasticBuffer support to MoE token dispatcher"
 *   [A2A]    "[Feature] Add DeepEPv2 (ElasticBuffer) MoE A2A backend"
 *   [DISC]   "deepep v2 support?"
 *   [VLLM]   vLLM tools/ep_kernels, commit "Add a new deepep_v2 all2all backend"
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers, caller-allocated and
 *     caller-owned; the library never allocates, frees or synchronizes, and
 *     keeps no state between calls (calls are reentrant).
 *   - Arrays are dense and row-major.  Activation / output base pointers must
 *     be 16-byte aligned, int32 / float arrays 4-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns without waiting.
 *   - Argument errors are detected on the host and returned BEFORE anything
 *     is enqueued.  Data errors (invalid expert ids, masked-capacity overflow)
 *     are not errors: they are counted on the device in handle.status.
 *   - A launch failure returns MOE_ERR_HIP (hipGetLastError after launch).
 */
#ifndef MOE_DISPATCH_H
#define MOE_DISPATCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* bad config value, null or misaligned pointer, bad enum */
    MOE_ERR_CAPACITY = 2,    /* num_tokens > max_tokens, or a buffer smaller than required */
    MOE_ERR_UNSUPPORTED = 3, /* a valid but unsupported shape (e.g. too many experts) */
    MOE_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} moe_status_t;

/* Dispatched layout.  Prefill (extend) uses the per-expert-contiguous
 * "expanded" layout, decode the fixed-capacity masked slab, independently of
 * the communication topology ([A2A] Supported scope, layouts paragraph; [A2A]
 * review reply on layout following the inference phase; [VLLM] commit
 * message, do_expand). */
typedef enum {
    MOE_LAYOUT_CONTIGUOUS = 0, /* expert segments back to back, each padded to `align` rows */
    MOE_LAYOUT_MASKED = 1      /* [experts, capacity] rows, slot s of expert e = row e*capacity+s */
} moe_layout_t;

/* Dispatched activation format.  FP8 activations with dynamic per-token
 * 1x128 scales feed 128x128 block-FP8 expert GEMMs; scales are fp32 for
 * Hopper-style consumers or packed UE8M0 powers of two for Blackwell-style
 * consumers ([A2A] Supported scope and Implementation; [DISC] quantization
 * requirement). */
typedef enum {
    MOE_QUANT_NONE = 0,      /* bf16 rows, bit copies of the input */
    MOE_QUANT_FP8_F32 = 1,   /* E4M3 rows + fp32 scale per 128 channels */
    MOE_QUANT_FP8_UE8M0 = 2, /* E4M3 rows + one exponent byte per 128 channels, 4 per uint32 */
    MOE_QUANT_MXFP8 = 3      /* E4M3 rows + one E8M0 byte per 32 channels (OCP MX, 1x32 MXFP8
                                experts with dynamic activation scaling: [A2A] format check) */
} moe_quant_t;

/* Problem shape, fixed for the lifetime of the buffers sized from it.
 * The buffer is sized from the per-rank token cap, hidden size and the real
 * top-k ([V2-PR] Motivation and the num_topk review commit: sizing for a
 * top-k of 32 instead of the model's 8 oversizes memory about 4x); the token
 * cap lives only here, never per call, because a per-call value that silently
 * overrides it is a known pitfall ([V2-PR] Modifications, sizing item). */
typedef struct {
    int32_t max_tokens;  /* per-call token cap (>= 0); num_tokens > max_tokens -> MOE_ERR_CAPACITY */
    int32_t hidden;      /* H: channels per token, multiple of 8 (of 128 with any FP8 format) */
    int32_t num_experts; /* E: routed experts, 1..2048 */
    int32_t num_topk;    /* K: experts per token, 1..32 ([V2-PR] top-k thread: kNumTopk <= 32) */
    int32_t num_ranks;   /* R: virtual destination ranks, E % R == 0; rank r owns experts [r*E/R, (r+1)*E/R) */
    int32_t layout;      /* moe_layout_t */
    int32_t align;       /* contiguous: segment alignment in rows, >= 1 (ignored when masked) */
    int32_t capacity;    /* masked: rows per expert, >= 1 (ignored when contiguous) */
    int32_t quant;       /* moe_quant_t */
    int32_t num_cus;     /* launch-shape override, not a reservation: 0 = automatic plans ([A2A] review:
                            0 = automatic); > 0 = the row and combine grids are sized as if the device had
                            this many compute units (at most 8 * num_cus workgroups of 256 threads) and the
                            one-launch fused dispatch uses num_cus blocks; the layout kernels ignore it */
} moe_config_t;

/* The dispatch handle: caller-allocated int32 device arrays, written by
 * moe_dispatch_layout and read by moe_dispatch and moe_combine.  It carries
 * the per-expert received counts and the source-index map that combine needs
 * ([V2-PR] Motivation: counts live on the handle; combine reuses the dispatch
 * handle).  It is plain data: valid until the caller overwrites it, and
 * combine must be given the handle of the dispatch that produced y's layout
 * ([A2A] Implementation: handles are single-use). */
typedef struct {
    int32_t *expert_count;  /* [E]     routed pairs per expert (before any capacity limit) */
    int32_t *recv_count;    /* [E]     rows written per expert: count (contiguous), min(count, C) (masked) */
    int32_t *expert_offset; /* [E+1]   first row of expert e; [E] = rows used (contiguous) or E*C (masked) */
    int32_t *rank_offset;   /* [R+1]   rank_offset[r] = expert_offset[r*E/R] */
    int32_t *pair_to_row;   /* [max_tokens*K] row of pair p = t*K+k, or -1 (unrouted, invalid, dropped) */
    int32_t *row_to_pair;   /* [moe_rows_capacity] pair held by each row, or -1; written in full */
    int32_t *status;        /* [2]     {pairs dropped by masked capacity, invalid expert ids} */
} moe_handle_t;

/* Rows the dispatched buffers (out_x, out_scale, out_row_weight, y) and
 * handle.row_to_pair must hold: max_tokens*K + E*(align-1) for the contiguous
 * layout (every segment may carry up to align-1 padding rows), E*capacity for
 * the masked layout.  Returns 0 for an invalid config. */
size_t moe_rows_capacity(const moe_config_t *cfg);

/* Bytes of device workspace moe_dispatch_layout needs (block histograms and
 * per-pair slots).
 * Returns 0 for an invalid config. */
size_t moe_workspace_bytes(const moe_config_t *cfg);

/* MOE_OK if the config is valid and supported, else the error code. */
moe_status_t moe_config_check(const moe_config_t *cfg);

/*
 * Layout: infer the dispatch layout from the router's top-k ids ([V2-PR]
 * Motivation and the _dispatch_core commit: V2 derives the layout from
 * topk_idx, with no separate layout pre-pass at the call site).
 *
 *   topk_idx   int32 [num_tokens, K]: expert of pair p = t*K+k.  -1 means
 *              unrouted (skipped); any other id outside [0,E) is invalid
 *              (skipped, counted in status[1]).
 *   handle     every array is written: counts, offsets, both maps, status.
 *   workspace  >= moe_workspace_bytes(cfg) bytes of scratch device memory,
 *              16-byte aligned, clobbered; workspace_bytes is its size.
 *
 * Rows of one expert hold its pairs in ascending pair order (a stable
 * counting sort).  Contiguous: row(p) = expert_offset[e] + slot(p), segments
 * padded to `align`.  Masked: row(p) = e*C + slot(p) if slot(p) < C, else the
 * pair is dropped (pair_to_row = -1) and counted in status[0].  Rows holding
 * no pair get row_to_pair = -1.  num_tokens == 0 is a valid call.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_CAPACITY (num_tokens > max_tokens,
 * workspace too small), MOE_ERR_HIP.
 */
moe_status_t moe_dispatch_layout(const moe_config_t *cfg, int32_t num_tokens,
                                 const int32_t *topk_idx, const moe_handle_t *handle,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_dispatch_layout without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a static device array
 * of the library, 8 MiB on each GPU (held until the process ends, its address
 * looked up once per GPU), so this call allocates nothing: it needs
 * moe_workspace_bytes' table plus 4 bytes per pair, i.e. at most about 1.96M
 * pairs (num_tokens * K) with 2048 experts.  Same arguments (minus the
 * workspace), results and errors as moe_dispatch_layout; larger calls return
 * MOE_ERR_CAPACITY before anything is enqueued.  Every call on a GPU shares
 * its array: calls that overlap on one GPU (other streams, other host
 * threads) race and must not be issued.  The stream's device is used (the
 * current device for a NULL stream).
 */
moe_status_t moe_dispatch_layout_noalloc(const moe_config_t *cfg, int32_t num_tokens,
                                         const int32_t *topk_idx, const moe_handle_t *handle,
                                         void *stream);

/*
 * Dispatch: move token rows into the layout built by moe_dispatch_layout
 * (recv_x of [V2-PR] Motivation), quantizing them to FP8 on the way when
 * cfg.quant asks for it ([A2A] Implementation; [VLLM] commit: FP8
 * block-quantized dispatch).
 *
 *   x               bf16 bits [num_tokens, H].
 *   topk_w          fp32 [num_tokens, K]; read only when out_row_weight != NULL.
 *   out_x           [rows_capacity, H]: bf16 (quant NONE) or E4M3 bytes.
 *   out_scale       quant FP8_F32: fp32 [rows_capacity, H/128];
 *                   quant FP8_UE8M0: uint32 [rows_capacity, ceil(H/512)], byte
 *                   b%4 of word b/4 = k_b + 127 where 2^k_b is block b's scale,
 *                   unused high bytes 0;
 *                   quant MXFP8: uint8 [rows_capacity, H/32], byte b = s_b + 127
 *                   (E8M0) where 2^s_b is 32-channel block b's scale;
 *                   must be NULL for quant NONE.
 *   out_row_weight  optional fp32 [rows_capacity]: router weight of the pair in
 *                   each written row (recv_topk_weights); NULL to skip.
 *
 * Per token t and 128-channel block b: amax = max|x|, a = max(amax, 1e-10);
 * fp32 scales: s = a/448 and q = E4M3(clamp(x/s, -448, 448)); UE8M0: k =
 * smallest integer with a <= 448*2^k and q = E4M3(x*2^-k).  MXFP8 (OCP MX
 * conversion, per 32-channel block): s = floor(log2 a) - 8 and
 * q = E4M3(clamp(x*2^-s, -448, 448)), so values above 448*2^s saturate.  E4M3 is
 * the OCP format (max 448), round to nearest even, sign kept.  Each token is read and
 * quantized once and its bytes stored to all of its kept rows.  Rows that no
 * kept pair maps to (padding, empty masked slots, dropped pairs) are NOT
 * written, in out_x, out_scale and out_row_weight alike.  The row kernel
 * spreads short work items (a token's run of about 1024 channels) over every
 * compute unit.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_CAPACITY, MOE_ERR_HIP.
 */
moe_status_t moe_dispatch(const moe_config_t *cfg, int32_t num_tokens, const uint16_t *x,
                          const float *topk_w, const moe_handle_t *handle, void *out_x,
                          void *out_scale, float *out_row_weight, void *stream);

/*
 * Dispatch with the layout inferred inside the same call, as the V2 dispatch
 * does ([V2-PR] Motivation and the _dispatch_core commit: no separate layout
 * pre-pass; counts come back on the handle).  Same arguments, outputs and
 * errors as moe_dispatch_layout followed by moe_dispatch, and bit-identical
 * results: the handle is written in full and the dispatched rows, scales and
 * row weights are those of moe_dispatch.
 *
 * For batches of at most 65536 pairs and at most 512 experts it is one
 * launch: each block (one per compute unit, or num_cus blocks) owns a run of
 * tokens, issues the loads of its token rows first and builds the layout for
 * its pairs while they are in flight.  Large batches (at least 8 tokens per
 * compute unit) whose token rows x fit in half of the 256 MB Infinity Cache
 * instead run two kernels, unless num_cus > 0: the one-launch layout, with
 * the compute units it leaves idle reading x (the rows of all but the first
 * 3/10 of the tokens) into the Infinity Cache meanwhile, then the row kernel
 * of moe_dispatch over every compute unit.  So a call whose x was evicted
 * from the caches reads most of it from HBM while the layout runs, not behind
 * its own row stores.  Batches beyond the one-launch
 * limits run the two-launch layout and the row kernel; from 8 tokens per
 * compute unit on (num_cus = 0, at most 512 experts) prefetch blocks in the
 * two layout kernels read 100 MB of x (after the first 3/10 of the tokens)
 * into the Infinity Cache meanwhile.
 */
moe_status_t moe_dispatch_fused(const moe_config_t *cfg, int32_t num_tokens, const int32_t *topk_idx,
                                const uint16_t *x, const float *topk_w, const moe_handle_t *handle,
                                void *workspace, size_t workspace_bytes, void *out_x, void *out_scale,
                                float *out_row_weight, void *stream);

/*
 * Combine: reduce expert outputs back to token order with the router weights
 * ([VLLM] commit: weighted reduction in combine; [A2A] review: nothing may
 * reduce again afterwards, an extra post-expert reduction double-counts).
 *
 *   y       bf16 bits [rows_capacity, H]: expert outputs in the dispatched layout.
 *   topk_w  fp32 [num_tokens, K]: the router weights as given (no
 *           renormalisation over kept pairs).
 *   out     bf16 bits [num_tokens, H].
 *
 * out[t,:] = bf16_RNE( sum over k ascending with row = pair_to_row[t*K+k] >= 0
 * of topk_w[t*K+k] * y[row,:] ), accumulated in fp32 from +0 with the product
 * and the sum each rounded to fp32.  A token with no kept pair gives +0.
 * Cache use: reads of at most 64 MiB of y (num_tokens * K rows) use
 * cache-allocating loads, so decode-sized outputs still in the Infinity Cache
 * are found there; larger reads stream with non-temporal loads.  An out larger
 * than 128 MiB is written with non-temporal stores (it cannot stay in the
 * 256 MB Infinity Cache); a smaller one with device-scope stores, which go
 * through L2 to the Infinity Cache and stay there for the kernel that reads it
 * next.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_CAPACITY, MOE_ERR_HIP.
 */
moe_status_t moe_combine(const moe_config_t *cfg, int32_t num_tokens, const uint16_t *y,
                         const float *topk_w, const moe_handle_t *handle, uint16_t *out,
                         void *stream);

/* ------------------------------------------------------------------------
 * Per-rank deduplicated exchange.
 *
 * The V1 dispatch first computed a per-rank layout in a separate pre-pass
 * (get_dispatch_layout, [V2-PR] Motivation) so that a token bound for several
 * experts of one rank crosses the wire once: the sender writes one row per
 * (token, destination rank), the receiver expands it to its experts' rows,
 * and combine returns one partial sum per (token, rank) that the source
 * reduces again (the multiple-reduction option, [VLLM] commit).  On one GPU
 * the calls below compute every local step of that exchange; the transfer
 * itself is not part of the library.  They take num_ranks <= 32 (larger R:
 * MOE_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------ */

/* Per-rank layout: caller-allocated int32 device arrays written by
 * moe_rank_layout.  Expert e belongs to rank e / (E/R); token t is in rank r
 * when one of its valid ids (0 <= id < E) belongs to r (-1 and invalid ids
 * make no rank; masked-capacity drops do not change membership).  Rank r's
 * rows are rank_token_offset[r] .. [r+1], its tokens in ascending order, with
 * no padding. */
typedef struct {
    int32_t *rank_token_count;  /* [R]   tokens in rank r (num_tokens_per_rank) */
    int32_t *rank_token_offset; /* [R+1] exclusive scan of rank_token_count */
    int32_t *token_rank_row;    /* [max_tokens*R] row of (t, r), or -1 when t is not in rank r
                                   (is_token_in_rank = token_rank_row >= 0) */
    int32_t *rank_row_to_token; /* [moe_rank_rows_capacity] token of each row, or -1; written in full */
} moe_rank_handle_t;

/* Rows of the per-rank buffers (send_x, send_scale, partial) and of
 * rank_row_to_token: max_tokens * min(K, R).  Returns 0 for an invalid config
 * or num_ranks > 32. */
size_t moe_rank_rows_capacity(const moe_config_t *cfg);

/*
 * Per-rank layout from the router's top-k ids (the V1 pre-pass, [V2-PR]
 * Motivation).  Every array of rank_handle is written; topk_idx as in
 * moe_dispatch_layout.  No workspace.  num_tokens == 0 is a valid call.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_CAPACITY, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP.
 */
moe_status_t moe_rank_layout(const moe_config_t *cfg, int32_t num_tokens, const int32_t *topk_idx,
                             const moe_rank_handle_t *rank_handle, void *stream);

/*
 * Deduplicated dispatch (sender side): each token row, quantized exactly as
 * moe_dispatch quantizes it (cfg.quant), is written once per rank it is in,
 * to row token_rank_row[t*R + r] of send_x / send_scale, whose layouts are
 * those of out_x / out_scale in moe_dispatch with moe_rank_rows_capacity
 * rows.  Rows holding no (token, rank) are not written.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_CAPACITY, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP.
 */
moe_status_t moe_dispatch_dedup(const moe_config_t *cfg, int32_t num_tokens, const uint16_t *x,
                                const moe_rank_handle_t *rank_handle, void *send_x, void *send_scale,
                                void *stream);

/*
 * Receive-side expansion: each kept pair p = t*K+k of expert e gets the row
 * of its token on rank e / (E/R):
 *   out_x[pair_to_row[p]] = send_x[token_rank_row[t*R + e/(E/R)]]
 * (bytes of the row and of its scales).  With one source rank the result is
 * byte-identical to moe_dispatch of the same tokens.  handle is the
 * per-expert layout of the same topk_idx (moe_dispatch_layout); rows no kept
 * pair maps to are not written.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_CAPACITY, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP.
 */
moe_status_t moe_expand(const moe_config_t *cfg, int32_t num_tokens, const int32_t *topk_idx,
                        const void *send_x, const void *send_scale, const moe_rank_handle_t *rank_handle,
                        const moe_handle_t *handle, void *out_x, void *out_scale, void *stream);

/*
 * Partial combine (receiver side, before the return trip): for every token t
 * and rank r it is in,
 *   partial[token_rank_row[t*R+r], :] = bf16_RNE( sum over k ascending with a
 *       valid id of rank r and row = pair_to_row[t*K+k] >= 0
 *       of topk_w[t*K+k] * y[row, :] )
 * in fp32 from +0, product and sum each rounded; a (token, rank) whose pairs
 * were all dropped gives +0.  partial is bf16 [moe_rank_rows_capacity, H];
 * rows holding no (token, rank) are not written.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_CAPACITY, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP.
 */
moe_status_t moe_combine_partial(const moe_config_t *cfg, int32_t num_tokens, const int32_t *topk_idx,
                                 const uint16_t *y, const float *topk_w, const moe_handle_t *handle,
                                 const moe_rank_handle_t *rank_handle, uint16_t *partial, void *stream);

/*
 * Final reduction on the source, after the return trip:
 *   out[t, :] = bf16_RNE( sum over r ascending with q = token_rank_row[t*R+r]
 *                          >= 0 of partial[q, :] )
 * in fp32 from +0; a token in no rank gives +0.  out is bf16 [num_tokens, H].
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_CAPACITY, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP.
 */
moe_status_t moe_combine_reduce(const moe_config_t *cfg, int32_t num_tokens, const uint16_t *partial,
                                const moe_rank_handle_t *rank_handle, uint16_t *out, void *stream);

/* ------------------------------------------------------------------------
 * Adapters for grouped-GEMM consumers.
 *
 * The dispatched buffers feed grouped expert GEMMs that read either the
 * contiguous layout (prefill) or the masked slab (decode), with fp32 or
 * packed UE8M0 scales ([A2A] Implementation: masked-slab repack kernels and
 * GEMM adapters for contiguous prefill and masked decode).  These calls
 * produce the forms such consumers read; none of them computes a GEMM.
 * ------------------------------------------------------------------------ */

/*
 * Expert index of every dispatched row, the per-row group index a contiguous
 * grouped GEMM reads:  row_expert[r] = e for rows
 * expert_offset[e] .. expert_offset[e] + recv_count[e] - 1, and -1 for every
 * other row (alignment padding, empty masked slots, the tail), over
 * moe_rows_capacity(cfg) rows.  handle is a layout written by
 * moe_dispatch_layout (or the fused call) with this cfg.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_HIP.
 */
moe_status_t moe_row_expert(const moe_config_t *cfg, const moe_handle_t *handle, int32_t *row_expert,
                            void *stream);

/* Rows a masked-to-contiguous repack writes at most:
 * min(max_tokens*K, E*capacity) + E*(align-1).  0 for an invalid config, a
 * contiguous cfg or align < 1. */
size_t moe_repack_rows_capacity(const moe_config_t *cfg, int32_t align);

/*
 * Masked slab -> contiguous segments (cfg.layout must be MASKED; handle is
 * its layout).  out_expert_offset[0] = 0 and out_expert_offset[e+1] =
 * out_expert_offset[e] + recv_count[e] rounded up to `align`; slab row
 * e*capacity + s (s < recv_count[e]) moves to row out_expert_offset[e] + s
 * with its scales.
 *   x, scale         the dispatched slab: out_x / out_scale of moe_dispatch.
 *   out_x, out_scale [moe_repack_rows_capacity(cfg, align)] rows, same row
 *                    formats; padding rows are not written.
 *   out_expert_offset int32 [E+1].
 *   out_row_expert   int32 [moe_repack_rows_capacity(cfg, align)]: as
 *                    moe_row_expert, for the contiguous rows; written in full.
 * Errors: MOE_ERR_INVALID_ARG (also for a contiguous cfg), MOE_ERR_HIP.
 */
moe_status_t moe_repack_masked_to_contiguous(const moe_config_t *cfg, int32_t align, const moe_handle_t *handle,
                                             const void *x, const void *scale, void *out_x, void *out_scale,
                                             int32_t *out_expert_offset, int32_t *out_row_expert,
                                             void *stream);

/*
 * Contiguous expert outputs -> masked slab, so moe_combine can run with the
 * masked handle: y_masked[e*capacity + s] = y[expert_offset[e] + s] for
 * s < recv_count[e] (bf16 rows of H channels); other slab rows are not
 * written.  expert_offset is out_expert_offset of the masked-to-contiguous
 * repack of the same handle.
 * Errors: MOE_ERR_INVALID_ARG (also for a contiguous cfg), MOE_ERR_HIP.
 */
moe_status_t moe_repack_contiguous_to_masked(const moe_config_t *cfg, const moe_handle_t *handle,
                                             const int32_t *expert_offset, const uint16_t *y, uint16_t *y_masked,
                                             void *stream);

/* 32-bit scale words per dispatched row: H/128 (fp32), ceil(H/512) (packed
 * UE8M0), H/128 (MXFP8: four E8M0 bytes per word); 0 for bf16 or an invalid
 * config. */
size_t moe_scale_words(const moe_config_t *cfg);

/*
 * Scales in MN-major order, the layout TMA-fed grouped GEMMs read: the
 * row-major scales [rows, S] (S = moe_scale_words(cfg) 32-bit words per row,
 * as written by the dispatch calls) become [S, ld] with
 * scale_mn[j*ld + r] = scale[r*S + j], ld = rows rounded up to a multiple of 4
 * (16 bytes), and the ld - rows padding entries 0.  Works on the 32-bit words,
 * so packed UE8M0 and MXFP8 scales keep four blocks per word.
 * Errors: MOE_ERR_INVALID_ARG (bf16 cfg, rows < 0, null or misaligned
 * pointers), MOE_ERR_HIP.
 */
moe_status_t moe_scales_mn_major(const moe_config_t *cfg, int32_t rows, const void *scale, void *scale_mn,
                                 void *stream);

/* Static, human-readable name of a status code; any other value (any int)
 * gives "MOE_ERR_UNKNOWN". */
const char *moe_status_str(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DISPATCH_H */
