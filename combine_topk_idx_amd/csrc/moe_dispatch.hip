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

// The row phase of dispatch_fused over a layout already on the handle: block
// b owns tokens [b * tokens_per_block, ...) and its waves claim the items of
// those tokens from a block counter.  Large batches with power-of-two scales
// use this on part of the compute units instead of dispatch_rows on all of
// them (the row stores run faster; see runs_plan).
template <int QUANT>
__global__ __launch_bounds__(kSingleThreads) void dispatch_runs(DispatchArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const RowPlan &pl = a.plan;
    const int64_t t0 = (int64_t)blockIdx.x * a.tokens_per_block;
    const int64_t t1 = min((int64_t)a.T, t0 + a.tokens_per_block);
    const int64_t nitems = (t1 - t0) * pl.items_per_token;
    __shared__ int32_t next_item;
    if (threadIdx.x == 0)
        next_item = kFusedWaves;
    __syncthreads();
    int64_t item = wave;
    while (item < nitems) {
        int32_t claim = 0;
        if (lane == 0)
            claim = atomicAdd(&next_item, 1);  // in flight while this item moves
        const int64_t t = t0 + item / pl.items_per_token;
        const int c = (int)(item % pl.items_per_token);
        const int it0 = c * pl.iters_per_item;
        const int n = min(pl.iters_per_item, pl.n_iters - it0);
        // the row loads and the token's rows are in flight together
        dev::RowRegs<QUANT> r;
        dev::load_item<QUANT>(r, a.x + t * a.H, it0, n, a.H, lane);
        const int32_t myrow = lane < a.K ? a.pair_to_row[t * a.K + lane] : -1;
        const uint64_t kept = __ballot(myrow >= 0);
        if (c == 0 && a.out_row_weight != nullptr && myrow >= 0)
            a.out_row_weight[myrow] = a.topk_w[t * a.K + lane];
        if (kept)
            dev::store_item<QUANT>(r, a, it0, n, lane, kept, myrow);
        item = __builtin_amdgcn_readfirstlane(claim);
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
    if (a.tokens_per_block > 0) {
        const dim3 grid(a.plan.grid), block(kSingleThreads);
        if (quant == MOE_QUANT_MXFP8)
            hipLaunchKernelGGL(dispatch_runs<MOE_QUANT_MXFP8>, grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL(dispatch_runs<MOE_QUANT_FP8_UE8M0>, grid, block, 0, stream, a);
        return hipGetLastError();
    }
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

// Blocks for a large batch spread as token runs: 7/16 of the compute units
// for power-of-two scales, half of them otherwise (see fused_plan).
int large_batch_blocks(int32_t quant, int cus)
{
    const bool pow2_scales = quant == MOE_QUANT_FP8_UE8M0 || quant == MOE_QUANT_MXFP8;
    const int b = pow2_scales ? cus * 7 / 16 : cus / 2;
    return b < 1 ? 1 : b;
}

// Items of a token-run plan (blocks of kFusedWaves waves, tpb tokens each):
// short items, and enough of them to keep a block's waves busy when it owns
// few tokens.
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

bool fused_plan(int32_t T, int32_t K, int32_t H, int32_t E, int32_t quant, int32_t num_cus, FusedPlan &fp)
{
    if (T <= 0 || E > kFusedMaxExperts || (int64_t)T * K > kSingleMaxPairs)
        return false;
    int blocks = num_cus;
    if (blocks <= 0) {
        // By default a block per compute unit.  Large batches run their row
        // phase faster on fewer compute units, one full block each over a
        // longer token run, while the token rows are cached: the phase is
        // then bound by the row stores, and at the DeepSeek-V3 prefill shape
        // 7/16 of the compute units (power-of-two scales) or half of them
        // (bf16 rows, fp32 scales, whose division needs more ALU) beat every
        // compute unit by 4-6%.  Rows read from HBM need every compute unit's
        // loads in flight (2x slower on 7/16 of them), so token rows too large
        // to stay cached keep a block per compute unit.
        const int cus = device_cu_count();
        blocks = cus;
        if (T >= kFusedLargeTokensPerCu * cus && (int64_t)T * H * 2 <= kHalfInfinityCacheBytes) {
            blocks = large_batch_blocks(quant, cus);
            const int per_block_max = kFusedWaves * kWave / K;  // one run of 64 pairs per wave
            const int need = (T + per_block_max - 1) / per_block_max;
            if (blocks < need)
                blocks = need;
        }
    }
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

// Separate dispatch of a large batch with power-of-two scales whose token
// rows are likely cached: token runs on 7/16 of the compute units
// (dispatch_runs) move its rows faster than dispatch_rows on all of them
// (DeepSeek-V3 prefill 93.4 -> 88.7 us).  With fp32 scales the same change
// was slower on the skewed batches, bf16 rows showed no gain, and rows read
// from HBM need every compute unit's loads in flight (120 -> 193 us), so
// those keep dispatch_rows, as do smaller batches and an explicit num_cus.
bool runs_plan(int32_t T, int32_t H, int32_t quant, int32_t num_cus, DispatchArgs &a)
{
    if (num_cus > 0 || !(quant == MOE_QUANT_FP8_UE8M0 || quant == MOE_QUANT_MXFP8))
        return false;
    const int cus = device_cu_count();
    if (T < kFusedLargeTokensPerCu * cus || (int64_t)T * H * 2 > kHalfInfinityCacheBytes)
        return false;
    int blocks = large_batch_blocks(quant, cus);
    if (blocks > T)
        blocks = T;
    const int tpb = (T + blocks - 1) / blocks;
    blocks = (T + tpb - 1) / tpb;
    a.plan = token_run_items(T, H, quant, tpb, blocks);
    a.tokens_per_block = tpb;
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
