// Internal declarations shared by the HIP translation units of
// libmoe_dispatch.so.  Not part of the public ABI (include/moe_dispatch.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_dispatch.h"

namespace moe {

constexpr int kWave = 64;             // CDNA wavefront width
constexpr int kBlockThreads = 256;    // 4 waves per workgroup for the row kernels
constexpr int kWavesPerBlock = kBlockThreads / kWave;
constexpr int kMaxBlockWaves = 1024 / kWave;  // waves of the largest (1024-thread) blocks
constexpr int kHistBatch = 8;                 // 16-byte id loads per thread in flight in a layout histogram
constexpr int kQuantGroup = 128;      // 1x128 activation quantization group
constexpr int kMaxTopk = 32;
constexpr int kMaxExperts = 2048;     // layout keeps 7 int32 per expert in LDS
constexpr int kLayoutMaxBlocks = 64;  // cap on layout blocks (columns of the histogram table)
constexpr int64_t kSingleMaxPairs = 65536;  // largest batch the one-launch layout takes
constexpr int kSingleMinBlocks = 16;         // one-launch blocks that share the unused-row fill

// ---- layout ---------------------------------------------------------------

struct LayoutArgs {
    const int32_t *topk_idx;
    int64_t P;          // pairs = num_tokens * K
    int32_t E, R, L;    // experts, ranks, experts per rank
    int32_t layout, align, capacity;
    int32_t rows_cap;   // rows of row_to_pair
    int32_t nbits;      // bits needed to tell experts apart (ballot match)
    int32_t rounds;     // runs of 64 pairs per wave
    int32_t chunk;      // pairs per block = waves * 64 * rounds
    int32_t nblocks;    // blocks = ceil(P / chunk) (one launch: at least kSingleMinBlocks), <= kLayoutMaxBlocks
    int32_t *ws;        // [E + 1][kLayoutMaxBlocks] per-block histograms (row E: invalid ids)
    int32_t *slots;     // [P] slot of each pair among its expert's pairs inside its block
    moe_handle_t h;
    // fused large-batch dispatch: pf_blocks blocks after nblocks prefetch
    // token rows of the dispatch that follows into the Infinity Cache -- in
    // the one-launch layout pf_x [pf_T, pf_H]; in the two-launch layout the
    // rank kernel pf_x [pf_T, pf_H] and the index kernel pf2_x [pf2_T, pf_H]
    const uint16_t *pf_x = nullptr;
    int32_t pf_T = 0, pf_H = 0, pf_blocks = 0;
    const uint16_t *pf2_x = nullptr;
    int32_t pf2_T = 0;
};

struct LayoutPlan {
    int32_t waves, rounds, chunk, nblocks;
    bool single;  // one launch, every block histograms all pairs (small batches)
};
LayoutPlan layout_plan(int64_t P, int32_t E);
size_t layout_table_bytes(int32_t E);
hipError_t launch_layout(const LayoutArgs &a, const LayoutPlan &plan, hipStream_t stream);

// ---- dispatch / combine -----------------------------------------------------

// Work is split into items of (token, run of column iterations); one wave
// processes one item at a time and walks items with a grid stride.
struct RowPlan {
    int32_t width;            // columns per wave iteration
    int32_t n_iters;          // iterations per row = ceil(H / width)
    int32_t items_per_token;
    int32_t iters_per_item;
    int64_t n_items;
    int32_t grid;             // workgroups launched
};

struct DispatchArgs {
    const uint16_t *x;
    const float *topk_w;
    const int32_t *pair_to_row;
    void *out_x;
    void *out_scale;
    float *out_row_weight;
    int32_t T, K, H;
    RowPlan plan;
};

// One launch for layout + dispatch (small batches): block b owns tokens
// [b * tokens_per_block, ...) and the pairs of those tokens.
struct FusedArgs {
    LayoutArgs lay;            // rounds = 1, chunk = tokens_per_block * K, nblocks = blocks
    DispatchArgs d;            // plan: per-token items inside a block (grid/n_items unused)
    int32_t tokens_per_block;
};

struct FusedPlan {
    int32_t blocks, tokens_per_block;
    RowPlan plan;
};

constexpr int kSingleThreads = 1024;   // block of the one-launch layout and of the fused dispatch
constexpr int kFusedWaves = 16;         // waves per fused block (at most one block per compute unit)
static_assert(kFusedWaves * kWave == kSingleThreads, "the fused block runs the one-launch layout");
constexpr int kFusedMaxExperts = 512;   // keeps the fused block's LDS within 44 KiB (80 E + 12 bytes + rows)
constexpr int kPrefetchMinTokensPerCu = 8;  // from this many tokens per compute unit, a fused call prefetches x
constexpr int kPrefetchSegment = 64;        // bytes of x each prefetch load stands for (one per segment)
constexpr int kPrefetchBatch = 16;          // prefetch loads per lane in flight before the wave waits
constexpr int kPrefetchSkipTenths = 3;      // tenths of the tokens, from the first, a fused call does not prefetch
// Token-row bytes the rank and the index kernel of the two-launch layout
// prefetch in a fused call whose rows do not fit the one-launch plan: about
// what HBM streams while each kernel runs (4 and 8 us), 100 MB in all.
constexpr int64_t kRankPrefetchBytes = (int64_t)40 << 20;
constexpr int64_t kIndexPrefetchBytes = (int64_t)60 << 20;

struct CombineArgs {
    const uint16_t *y;
    const float *topk_w;         // NULL: every weight is 1 (the final per-rank reduction)
    const int32_t *pair_to_row;
    uint16_t *out;
    int32_t T, K, H;
    RowPlan plan;
    // partial combine only: sums per (token, rank) into out rows token_rank_row[t*R + r]
    const int32_t *topk_idx;
    const int32_t *token_rank_row;
    int32_t E, R, L;
    int32_t stream_out;          // non-temporal output stores (outputs larger than kCombineStreamOutBytes)
    int32_t stream_in;           // non-temporal loads of y (reads larger than kCombineStreamInBytes)
};

// ---- per-rank (deduplicated) exchange --------------------------------------

constexpr int kMaxDedupRanks = 32;     // one bit of a 32-bit mask per rank; lanes 0..R-1 hold ranks
constexpr int kRankLayoutWaves = 16;
constexpr int kRankLayoutMaxLdsWords = 8192;  // chunk counts [chunks per block][R]
constexpr int kRankLayoutMaxCachedTokens = 4096;  // token masks kept in LDS up to this many per block

struct RankLayoutArgs {
    const int32_t *topk_idx;
    int32_t T, K, E, R, L;
    int32_t tokens_per_block;   // multiple of 64
    int32_t nblocks;
    int32_t rows_cap;           // rows of rank_row_to_token
    int32_t vec4;               // K % 4 == 0 and topk_idx 16-byte aligned: ids load as int4
    uint64_t rank_magic;        // ceil(2^32 / L): e / L = (e * rank_magic) >> 32 for e < 2^21
    int32_t cache_masks;        // the block's token rank masks stay in LDS between passes
    moe_rank_handle_t h;
};

struct ExpandArgs {
    const int32_t *topk_idx;
    const int32_t *pair_to_row;
    const int32_t *token_rank_row;
    const uint8_t *send_x;
    const uint8_t *send_scale;
    uint8_t *out_x;
    uint8_t *out_scale;
    int32_t T, K, E, R, L;
    int32_t row_bytes, scale_words;
    RowPlan plan;               // over row bytes: kExpandWidth bytes per iteration
};

constexpr int kExpandWidth = kWave * 16;  // bytes per wave iteration, 16 per lane
constexpr int kExpandMaxIters = 8;

// ---- adapters for grouped-GEMM consumers ------------------------------------

struct RowExpertArgs {
    const int32_t *expert_offset;  // [E + 1]
    const int32_t *recv_count;     // [E]
    int32_t E;
    int64_t rows;
    int32_t *row_expert;           // [rows]
};

struct RepackArgs {
    const int32_t *recv_count;     // [E] rows received per expert (masked handle)
    const int32_t *in_offset;      // contiguous -> masked: the contiguous segment offsets [E + 1]
    int32_t *out_offset;           // masked -> contiguous: segment offsets written [E + 1]
    int32_t *out_row_expert;       // masked -> contiguous: [out_rows]
    const uint8_t *x;
    const uint8_t *scale;
    uint8_t *out_x;
    uint8_t *out_scale;
    int32_t E, C, align, row_bytes, scale_words;
    int64_t out_rows;              // masked -> contiguous: rows of out_x / out_row_expert
    int32_t to_contiguous;
    RowPlan plan;                  // items over the kept rows (at most min(T*K, E*C)), kAdaptWidth bytes each
};

struct MnMajorArgs {
    const uint32_t *in;
    uint32_t *out;
    int64_t rows, ld;
    int32_t S;
};

constexpr int kAdaptWidth = kWave * 16;  // bytes per wave iteration
constexpr int kAdaptMaxIters = 8;
constexpr int kTransposeTile = 64;

hipError_t launch_row_expert(const RowExpertArgs &a, hipStream_t stream);
hipError_t launch_repack(const RepackArgs &a, hipStream_t stream);
hipError_t launch_scales_mn_major(const MnMajorArgs &a, hipStream_t stream);

int device_cu_count();
RowPlan row_plan(int32_t T, int32_t H, int32_t width, int32_t max_iters_per_item,
                 int32_t num_cus, int32_t min_items_per_token = 1);
hipError_t launch_dispatch(const DispatchArgs &a, int32_t quant, hipStream_t stream);
bool fused_plan(int32_t T, int32_t K, int32_t H, int32_t E, int32_t quant, int32_t num_cus, FusedPlan &fp);
bool fused_prefetch_plan(const DispatchArgs &d, const LayoutPlan &lp, int32_t num_cus, LayoutArgs &la);
bool split_prefetch_plan(const DispatchArgs &d, const LayoutPlan &lp, int32_t num_cus, LayoutArgs &la);
hipError_t launch_dispatch_fused(const FusedArgs &f, int32_t quant, hipStream_t stream);
hipError_t launch_combine(const CombineArgs &a, hipStream_t stream);
hipError_t launch_combine_partial(const CombineArgs &a, hipStream_t stream);
bool rank_layout_plan(int32_t T, int32_t R, RankLayoutArgs &a);
hipError_t launch_rank_layout(const RankLayoutArgs &a, hipStream_t stream);
hipError_t launch_expand(const ExpandArgs &a, hipStream_t stream);

// Columns one wave iteration covers, and how many iterations a wave keeps in
// registers at once, per kernel.
constexpr int kDispatchBf16Width = kWave * 8;    // 8 bf16 = 16 bytes per lane
constexpr int kDispatchBf16MaxIters = 16;
constexpr int kDispatchFp8Width = kWave * 16;    // 16 channels per lane, 8 lanes per block
constexpr int kDispatchFp8MaxIters = 8;
constexpr int kDispatchMinItemsPerToken = 8;     // about 1024 columns per item: many short waves
constexpr int kCombineWidth = kWave * 16;        // two vectors of 8 bf16 per lane
constexpr int kCombineMaxIters = 64;
constexpr int kCombineMinItemsPerToken = 8;      // about 1024 columns per item: many short waves
// Half of MI355X's 256 MB Infinity Cache.  Combine outputs larger than this
// cannot stay in it; they are written non-temporally so that their dirty lines
// do not have to be written back while later kernels stream through the cache.
// Token rows up to this size are prefetched into it by a large fused dispatch.
constexpr int64_t kHalfInfinityCacheBytes = (int64_t)128 << 20;
constexpr int64_t kCombineStreamOutBytes = kHalfInfinityCacheBytes;
// Combines that read at most this many bytes of expert outputs (T * K rows)
// load them with plain, cache-allocating loads: decode-sized outputs are
// served from the Infinity Cache when the kernel that wrote them (or the
// previous step) left them there.  Larger reads stream through with
// non-temporal loads, which do not allocate and are faster for them.
constexpr int64_t kCombineStreamInBytes = (int64_t)64 << 20;

}  // namespace moe
