// Dispatch on gfx950: move each token row into its kept dispatched rows,
// optionally quantizing to OCP E4M3 with dynamic 1x128 scales on the way.
//
// Rows move in the layout of the dispatch handle (recv_x; page "moe: add
// DeepEP V2 ElasticBuffer support to MoE token dispatcher", Motivation).  FP8
// activations carry fp32 or packed UE8M0 scales (page "[Feature] Add DeepEPv2
// (ElasticBuffer) MoE A2A backend", Implementation), one per 128 channels of a
// token, matching 128x128 weight blocks with dynamic activation scaling (page
// "deepep v2 support?", quantization requirement).
//
// The kernel is token-major: a wave reads a token's row once with 16-byte
// loads, quantizes it once, and stores the same bytes to each of the token's
// kept rows (K full-row 16-byte non-temporal store streams), so skewed routing
// only changes where rows land.  FP8 lanes hold 16 channels, so one 128-channel block is 8
// adjacent lanes: the block max is three DPP steps, and one wave iteration
// covers 8 blocks = two packed UE8M0 words.  An MXFP8 block (32 channels, the
// 1x32 MXFP8 expert format named on page "[Feature] Add DeepEPv2
// (ElasticBuffer) MoE A2A backend", format check) is two adjacent lanes.
#include "moe_device.h"

namespace moe {

namespace {

template <int QUANT>
__global__ __launch_bounds__(kBlockThreads) void dispatch_rows(DispatchArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const RowPlan &pl = a.plan;
    for (int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wave; item < pl.n_items;
         item += (int64_t)gridDim.x * kWavesPerBlock) {
        const int t = (int)(item / pl.items_per_token);
        const int c = (int)(item - (int64_t)t * pl.items_per_token);
        // lane k (< K) holds the row of pair t*K+k
        const int32_t myrow = lane < a.K ? a.pair_to_row[(int64_t)t * a.K + lane] : -1;
        const uint64_t kept = __ballot(myrow >= 0);
        if (kept == 0)
            continue;
        if (c == 0 && a.out_row_weight != nullptr && myrow >= 0)
            a.out_row_weight[myrow] = a.topk_w[(int64_t)t * a.K + lane];
        const int it0 = c * pl.iters_per_item;
        const int n = min(pl.iters_per_item, pl.n_iters - it0);
        dev::RowRegs<QUANT> r;
        dev::load_item<QUANT>(r, a.x + (int64_t)t * a.H, it0, n, a.H, lane);
        dev::store_item<QUANT>(r, a, it0, n, lane, kept, myrow);
    }
}

template <int QUANT>
__global__ __launch_bounds__(kSingleThreads) void dispatch_fused(FusedArgs f)
{
    extern __shared__ int32_t lds[];
    __shared__ int32_t red[kMaxBlockWaves];
    const LayoutArgs &la = f.lay;
    const DispatchArgs &a = f.d;
    const RowPlan &pl = a.plan;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    constexpr int nwaves = kFusedWaves;
    int32_t *rows = lds + dev::single_layout_lds_words(la.E, nwaves);  // [tokens_per_block * K]
    const int t0 = blockIdx.x * f.tokens_per_block;
    const int t1 = min(a.T, t0 + f.tokens_per_block);
    const int nitems = (t1 - t0) * pl.items_per_token;

    // the first item's loads are in flight while the layout is built
    dev::RowRegs<QUANT> r;
    int item = wave;
    if (item < nitems) {
        const int t = t0 + item / pl.items_per_token;
        const int it0 = (item % pl.items_per_token) * pl.iters_per_item;
        dev::load_item<QUANT>(r, a.x + (int64_t)t * a.H, it0, min(pl.iters_per_item, pl.n_iters - it0), a.H,
                              lane);
    }
    // items after the first ones are claimed from a block counter: the
    // oldest waves win the memory arbitration and would otherwise finish
    // early, leaving the block's last items to a few waves
    __shared__ int32_t next_item;
    if (threadIdx.x == 0)
        next_item = nwaves;
    // the unused-row fill and the published counts wait until after the rows:
    // nothing here reads them, and waves without items do them meanwhile
    dev::single_layout_block(la, lds, red, rows, false);  // its barriers publish next_item
    __syncthreads();

    bool first = true;
    while (item < nitems) {
        int32_t claim = 0;
        if (lane == 0)
            claim = atomicAdd(&next_item, 1);  // in flight while this item moves
        const int t = t0 + item / pl.items_per_token;
        const int c = item % pl.items_per_token;
        const int it0 = c * pl.iters_per_item;
        const int n = min(pl.iters_per_item, pl.n_iters - it0);
        if (!first)
            dev::load_item<QUANT>(r, a.x + (int64_t)t * a.H, it0, n, a.H, lane);
        first = false;
        const int32_t myrow = lane < a.K ? rows[(t - t0) * a.K + lane] : -1;
        const uint64_t kept = __ballot(myrow >= 0);
        if (c == 0 && a.out_row_weight != nullptr && myrow >= 0)
            a.out_row_weight[myrow] = a.topk_w[(int64_t)t * a.K + lane];
        if (kept)
            dev::store_item<QUANT>(r, a, it0, n, lane, kept, myrow);
        item = __builtin_amdgcn_readfirstlane(claim);
    }
    dev::single_layout_finish(la, lds);
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs &a, int32_t quant, hipStream_t stream)
{
    const dim3 grid(a.plan.grid), block(kBlockThreads);
    switch (quant) {
    case MOE_QUANT_NONE:
        hipLaunchKernelGGL(dispatch_rows<MOE_QUANT_NONE>, grid, block, 0, stream, a);
        break;
    case MOE_QUANT_FP8_F32:
        hipLaunchKernelGGL(dispatch_rows<MOE_QUANT_FP8_F32>, grid, block, 0, stream, a);
        break;
    case MOE_QUANT_MXFP8:
        hipLaunchKernelGGL(dispatch_rows<MOE_QUANT_MXFP8>, grid, block, 0, stream, a);
        break;
    default:
        hipLaunchKernelGGL(dispatch_rows<MOE_QUANT_FP8_UE8M0>, grid, block, 0, stream, a);
        break;
    }
    return hipGetLastError();
}

namespace {

// Items of a fused plan (blocks of kFusedWaves waves, tpb tokens each): short
// items, and enough of them to keep a block's waves busy when it owns few
// tokens.
RowPlan token_run_items(int32_t T, int32_t H, int32_t quant, int32_t tpb, int32_t blocks)
{
    const bool fp8 = quant != MOE_QUANT_NONE;
    RowPlan p;
    p.width = fp8 ? kDispatchFp8Width : kDispatchBf16Width;
    const int max_iters = fp8 ? kDispatchFp8MaxIters : kDispatchBf16MaxIters;
    p.n_iters = (H + p.width - 1) / p.width;
    int per_token = (p.n_iters + max_iters - 1) / max_iters;
    int want = (kFusedWaves + tpb - 1) / tpb;
    if (want < kDispatchMinItemsPerToken)
        want = kDispatchMinItemsPerToken;
    if (per_token < want)
        per_token = want < p.n_iters ? want : p.n_iters;
    p.iters_per_item = (p.n_iters + per_token - 1) / per_token;
    p.items_per_token = (p.n_iters + p.iters_per_item - 1) / p.iters_per_item;
    p.n_items = (int64_t)T * p.items_per_token;
    p.grid = blocks;
    return p;
}

}  // namespace

// The one-launch fused kernel: a block per compute unit (or num_cus blocks),
// each owning a run of tokens and at most one run of 64 pairs per wave.
bool fused_plan(int32_t T, int32_t K, int32_t H, int32_t E, int32_t quant, int32_t num_cus, FusedPlan &fp)
{
    if (T <= 0 || E > kFusedMaxExperts || (int64_t)T * K > kSingleMaxPairs)
        return false;
    int blocks = num_cus > 0 ? num_cus : device_cu_count();
    if (blocks > T)
        blocks = T;
    const int tpb = (T + blocks - 1) / blocks;
    if ((int64_t)tpb * K > (int64_t)kFusedWaves * kWave)
        return false;  // one run of 64 pairs per wave
    fp.tokens_per_block = tpb;
    fp.blocks = (T + tpb - 1) / tpb;
    fp.plan = token_run_items(T, H, quant, tpb, fp.blocks);
    return true;
}

// A fused call on a large batch (at least kPrefetchMinTokensPerCu tokens per
// compute unit) whose token rows fit in half of the Infinity Cache runs as two
// kernels: the one-launch layout, whose blocks leave most compute units idle,
// with prefetch blocks on those units that bring the rows of all but the first
// 3/10 of the tokens into the cache, then the row kernel of the separate
// dispatch over every compute unit (skipping those tokens: 0.7 us less per
// step with x evicted, 1.2 us back to back; skipping half: 2.7 us more).  With x
// evicted beforehand, the row kernel otherwise reads it from HBM behind its
// own row stores (DeepSeek-V3 prefill: a one-launch fused call on a block per
// compute unit 133 us, on 7/16 of them 191 us; this plan 119-120 us).  Sets
// la's prefetch fields; false when the batch does not qualify or num_cus is
// given.
bool fused_prefetch_plan(const DispatchArgs &d, const LayoutPlan &lp, int32_t num_cus, LayoutArgs &la)
{
    const int cus = device_cu_count();
    if (num_cus > 0 || !lp.single || d.T < kPrefetchMinTokensPerCu * cus ||
        (int64_t)d.T * d.H * 2 > kHalfInfinityCacheBytes || la.nblocks >= cus)
        return false;
    const int64_t segs = ((int64_t)2 * d.H + kPrefetchSegment - 1) / kPrefetchSegment;
    if ((int64_t)d.T * ((segs + kWave - 1) / kWave) > INT32_MAX / 2)
        return false;
    // the first tokens are not prefetched: the row kernel's first waves read
    // them from HBM while its own stores are still ramping up
    const int32_t t0 = (int32_t)((int64_t)d.T * kPrefetchSkipTenths / 10);
    la.pf_x = d.x + (int64_t)t0 * d.H;
    la.pf_T = d.T - t0;
    la.pf_H = d.H;
    la.pf_blocks = cus - la.nblocks;
    return true;
}

// A fused call on a large batch that the one-launch layout does not take
// (more than 65,536 pairs, or token rows beyond half of the Infinity Cache)
// runs the two-launch layout and the row kernel; its two layout kernels leave
// most compute units idle for a few microseconds each, and prefetch blocks on
// them read kRankPrefetchBytes and kIndexPrefetchBytes of token rows (from the
// token after the first kPrefetchSkipTenths tenths on) into the Infinity
// Cache meanwhile (16,384-token skewed batches: steps with x evicted 6-23 us
// faster, back to back 1.5-2 us slower).  Sets la's prefetch fields; false
// when the batch does not qualify or num_cus is given.
bool split_prefetch_plan(const DispatchArgs &d, const LayoutPlan &lp, int32_t num_cus, LayoutArgs &la)
{
    const int cus = device_cu_count();
    if (num_cus > 0 || lp.single || lp.waves * kWave != kSingleThreads || d.T < kPrefetchMinTokensPerCu * cus ||
        la.nblocks >= cus)
        return false;
    const int64_t row_bytes = 2 * (int64_t)d.H;
    const int64_t segs = (row_bytes + kPrefetchSegment - 1) / kPrefetchSegment;
    if ((int64_t)d.T * ((segs + kWave - 1) / kWave) > INT32_MAX / 2)
        return false;
    const int32_t t0 = (int32_t)((int64_t)d.T * kPrefetchSkipTenths / 10);
    const int64_t left = (int64_t)d.T - t0;
    const int32_t n_rank = (int32_t)min(left, kRankPrefetchBytes / row_bytes);
    const int32_t n_index = (int32_t)min(left - n_rank, kIndexPrefetchBytes / row_bytes);
    la.pf_x = d.x + (int64_t)t0 * d.H;
    la.pf_T = n_rank;
    la.pf2_x = d.x + (int64_t)(t0 + n_rank) * d.H;
    la.pf2_T = n_index;
    la.pf_H = d.H;
    la.pf_blocks = cus - la.nblocks;
    return true;
}

hipError_t launch_dispatch_fused(const FusedArgs &f, int32_t quant, hipStream_t stream)
{
    const dim3 grid(f.lay.nblocks), block(kFusedWaves * kWave);
    const size_t lds = sizeof(int32_t) * (dev::single_layout_lds_words(f.lay.E, kFusedWaves) +
                                          (size_t)f.tokens_per_block * f.d.K);
    switch (quant) {
    case MOE_QUANT_NONE:
        hipLaunchKernelGGL(dispatch_fused<MOE_QUANT_NONE>, grid, block, lds, stream, f);
        break;
    case MOE_QUANT_FP8_F32:
        hipLaunchKernelGGL(dispatch_fused<MOE_QUANT_FP8_F32>, grid, block, lds, stream, f);
        break;
    case MOE_QUANT_MXFP8:
        hipLaunchKernelGGL(dispatch_fused<MOE_QUANT_MXFP8>, grid, block, lds, stream, f);
        break;
    default:
        hipLaunchKernelGGL(dispatch_fused<MOE_QUANT_FP8_UE8M0>, grid, block, lds, stream, f);
        break;
    }
    return hipGetLastError();
}

}  // namespace moe
