// Dispatch layout on gfx950: per-expert counts, aligned / masked segment
// offsets, stable slots, and the pair <-> row maps of the dispatch handle.
//
// The layout is inferred from the router's top-k ids (page "moe: add DeepEP V2
// ElasticBuffer support to MoE token dispatcher", Motivation), for the
// per-expert-contiguous prefill layout or the masked decode slab (page
// "[Feature] Add DeepEPv2 (ElasticBuffer) MoE A2A backend", Supported scope,
// layouts paragraph).  Rows of one expert keep ascending pair order, i.e. the
// result is a stable counting sort of the pairs by expert.
//
// Pairs are cut into blocks of `chunk` consecutive pairs; wave w of a block
// owns `rounds` runs of 64 pairs.  A 64-lane ballot match gives each pair its
// rank among equal experts in its run, an LDS scan over the block's waves
// turns that into its slot inside the block, and
//     row = segment_offset[e] + (pairs of e in earlier blocks) + slot.
// No atomic decides an order, so the result is deterministic.  Two schedules
// produce the same result:
//   layout_single  (up to kSingleMaxPairs pairs, E <= 512) one launch, no
//                  workspace: every block histograms ALL pairs itself (32-bit
//                  LDS atomics into two arrays, one for the pairs before the
//                  block and one for the pairs from the block on), so it needs
//                  nothing from other blocks.  The redundant histogram costs about as much as a
//                  second launch would, and no table round trip is needed.
//   layout_rank + layout_index  (larger batches) the rank kernel writes each
//                  pair's slot and its block histogram (one column of an
//                  expert-major table in the workspace); the index kernel
//                  reads the table cooperatively (one 16-byte vector per
//                  thread) and writes the rows.
// Both end with the same steps: segment offsets by a block-wide scan, the
// pair <-> row maps, padding rows filled with -1 (one expert per wave over
// the grid), and the counts and offsets published a slice of experts per
// block (block 0 adds the rank offsets and status).
#include "moe_device.h"

namespace moe {

namespace {

using dev::count_overflow;
using dev::fill_unused_rows;
using dev::lanes_below;
using dev::match_expert;
using dev::publish;
using dev::row_of;
using dev::segment_offsets;

constexpr int kTileRounds = 16;  // runs of 64 pairs a lane keeps in registers

// Pair range [w0, w1) of wave `wave` in block `blk`.
struct WaveRange {
    int64_t w0, w1;
};

__device__ __forceinline__ WaveRange wave_range(const LayoutArgs &a, int blk, int wave)
{
    const int64_t c0 = (int64_t)blk * a.chunk;
    const int64_t c1 = min(a.P, c0 + a.chunk);
    WaveRange r;
    r.w0 = min(c1, c0 + (int64_t)wave * kWave * a.rounds);
    r.w1 = min(c1, r.w0 + (int64_t)kWave * a.rounds);
    return r;
}

// Load runs [base, base + 64*kTileRounds) of a non-empty range ending at w1
// from src; lanes past the end get `fill`.  Runs that start past the end are
// skipped by a wave-uniform test; inside a run the address is clamped into
// the range so the load needs no lane mask.
__device__ __forceinline__ void load_runs(int32_t (&v)[kTileRounds], const int32_t *src, int64_t base,
                                          int64_t w1, int lane, int32_t fill)
{
    int32_t raw[kTileRounds];
#pragma unroll
    for (int r = 0; r < kTileRounds; ++r) {
        const int64_t p = base + (int64_t)r * kWave + lane;
        raw[r] = fill;
        if (base + (int64_t)r * kWave < w1)
            raw[r] = src[p < w1 ? p : w1 - 1];
    }
#pragma unroll
    for (int r = 0; r < kTileRounds; ++r)
        v[r] = base + (int64_t)r * kWave + lane < w1 ? raw[r] : fill;
}

__global__ __launch_bounds__(1024) void layout_rank(LayoutArgs a)
{
    if ((int)blockIdx.x >= a.nblocks) {  // prefetch blocks of a fused call
        dev::prefetch_rows(a.pf_x, a.pf_T, a.pf_H, blockIdx.x - a.nblocks, a.pf_blocks);
        return;
    }
    extern __shared__ int32_t cnt[];  // [WB][E]: per-wave counts, then per-wave slot bases
    __shared__ int32_t red[kMaxBlockWaves];
    const int E = a.E;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int nwaves = blockDim.x / kWave;
    const int blk = blockIdx.x;
    const WaveRange wr = wave_range(a, blk, wave);
    const bool one_tile = wr.w1 - wr.w0 <= (int64_t)kTileRounds * kWave;

    int32_t id[kTileRounds];
    if (wr.w0 < wr.w1)
        load_runs(id, a.topk_idx, wr.w0, wr.w1, lane, -1);
    for (int i = tid; i < nwaves * E; i += blockDim.x)
        cnt[i] = 0;
    if (tid == 0)
        red[0] = 0;  // invalid ids of the block
    __syncthreads();

    // 1. rank of each pair among equal experts earlier in its wave's runs
    int32_t *mycnt = cnt + wave * E;
    int32_t rank[kTileRounds];
    int invalid = 0;
    for (int64_t base = wr.w0; base < wr.w1; base += (int64_t)kTileRounds * kWave) {
        if (base != wr.w0)
            load_runs(id, a.topk_idx, base, wr.w1, lane, -1);
#pragma unroll
        for (int r = 0; r < kTileRounds; ++r) {
            rank[r] = 0;
            if (base + (int64_t)r * kWave >= wr.w1)
                continue;  // wave-uniform
            const int32_t e = id[r];
            const bool in = base + (int64_t)r * kWave + lane < wr.w1;
            const bool routed = e >= 0 && e < E;
            invalid += (in && !routed && e != -1) ? 1 : 0;
            const uint64_t m = match_expert(e, routed, a.nbits);
            if (routed) {
                const int below = lanes_below(m);
                const int32_t first = mycnt[e];     // read by every lane of the match ...
                rank[r] = first + below;
                if (below == 0)
                    mycnt[e] = first + __popcll(m);  // ... before its leader advances it
            }
        }
    }
    if (invalid != 0)
        atomicAdd(&red[0], invalid);  // rare
    __syncthreads();

    // 2. per-wave slot bases inside the block (all of an expert's wave counts
    //    read before any is rewritten); block histogram -> table column
    for (int e = tid; e < E; e += blockDim.x) {
        int32_t c[kMaxBlockWaves];
#pragma unroll
        for (int w = 0; w < kMaxBlockWaves; ++w)
            c[w] = 0;
#pragma unroll
        for (int w = 0; w < kMaxBlockWaves; ++w)
            if (w < nwaves)
                c[w] = cnt[w * E + e];
        int32_t s = 0;
#pragma unroll
        for (int w = 0; w < kMaxBlockWaves; ++w)
            if (w < nwaves) {
                cnt[w * E + e] = s;
                s += c[w];
            }
        a.ws[(int64_t)e * kLayoutMaxBlocks + blk] = s;
    }
    if (tid == 0)
        a.ws[(int64_t)E * kLayoutMaxBlocks + blk] = red[0];
    __syncthreads();

    // 3. slot of each pair inside the block
    for (int64_t base = wr.w0; base < wr.w1; base += (int64_t)kTileRounds * kWave) {
        if (!one_tile)
            load_runs(id, a.topk_idx, base, wr.w1, lane, -1);
#pragma unroll
        for (int r = 0; r < kTileRounds; ++r) {
            if (base + (int64_t)r * kWave >= wr.w1)
                continue;  // wave-uniform
            const int64_t p = base + (int64_t)r * kWave + lane;
            const int32_t e = id[r];
            const bool routed = e >= 0 && e < E;
            int32_t slot = -1;
            if (one_tile) {
                if (routed)
                    slot = mycnt[e] + rank[r];
            } else {
                // several tiles: ranks were not kept, match again from the bases
                const uint64_t m = match_expert(e, routed, a.nbits);
                if (routed) {
                    const int below = lanes_below(m);
                    const int32_t first = mycnt[e];
                    slot = first + below;
                    if (below == 0)
                        mycnt[e] = first + __popcll(m);
                }
            }
            if (p < wr.w1)
                a.slots[p] = slot;
        }
    }
}

// ---- schedule 2: index kernel -------------------------------------------------

__global__ __launch_bounds__(1024) void layout_index(LayoutArgs a)
{
    if ((int)blockIdx.x >= a.nblocks) {  // prefetch blocks of a fused call
        dev::prefetch_rows(a.pf2_x, a.pf2_T, a.pf_H, blockIdx.x - a.nblocks, a.pf_blocks);
        return;
    }
    extern __shared__ int32_t lds[];
    const int E = a.E;
    int32_t *tot = lds;          // [E+1] pairs per expert, all blocks ([E]: invalid ids)
    int32_t *pre = tot + E + 1;  // [E+1] pairs per expert in earlier blocks
    int32_t *off = pre + E + 1;  // [E+1] segment starts
    int32_t *over = off + E + 1; // [1] pairs the masked capacity drops
    __shared__ int32_t red[kMaxBlockWaves];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int blk = blockIdx.x;
    const WaveRange wr = wave_range(a, blk, wave);
    const bool one_tile = wr.w1 - wr.w0 <= (int64_t)kTileRounds * kWave;

    // in flight while the table is read: the wave's ids and slots
    int32_t id[kTileRounds], slot[kTileRounds];
    if (wr.w0 < wr.w1) {
        load_runs(id, a.topk_idx, wr.w0, wr.w1, lane, -1);
        load_runs(slot, a.slots, wr.w0, wr.w1, lane, -1);
    }

    // 1. totals and this block's prefix from the expert-major table (row E:
    //    invalid ids).  Each thread reads one 16-byte vector (4 columns) and
    //    adds its partial sums into LDS; columns >= nblocks are masked (no
    //    pairs: the rank kernel did not run and every column is masked).
    for (int e = tid; e <= E; e += blockDim.x) {
        tot[e] = 0;
        pre[e] = 0;
    }
    if (tid == 0)
        over[0] = 0;
    __syncthreads();
    const int cols = a.P > 0 ? a.nblocks : 0;
    const int nvec = (E + 1) * (kLayoutMaxBlocks / 4);
    for (int vi = tid; vi < nvec; vi += blockDim.x) {
        const int e = vi / (kLayoutMaxBlocks / 4), j = vi % (kLayoutMaxBlocks / 4);
        const int4 v = reinterpret_cast<const int4 *>(a.ws)[vi];
        const int32_t c[4] = {v.x, v.y, v.z, v.w};
        int32_t s = 0, p = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int b = 4 * j + q;
            const int32_t x = b < cols ? c[q] : 0;
            s += x;
            p += b < blk ? x : 0;
        }
        if (s)
            atomicAdd(&tot[e], s);
        if (p)
            atomicAdd(&pre[e], p);
    }
    __syncthreads();
    count_overflow<0>(a, tot, over);  // read after the barriers of step 2

    // 2. segment offsets
    segment_offsets<0>(a, tot, off, red);

    // 3. rows and both maps
    for (int64_t base = wr.w0; base < wr.w1; base += (int64_t)kTileRounds * kWave) {
        if (!one_tile) {
            load_runs(id, a.topk_idx, base, wr.w1, lane, -1);
            load_runs(slot, a.slots, base, wr.w1, lane, -1);
        }
#pragma unroll
        for (int r = 0; r < kTileRounds; ++r) {
            const int64_t p = base + (int64_t)r * kWave + lane;
            if (base + (int64_t)r * kWave >= wr.w1)
                continue;  // wave-uniform
            const int32_t e = id[r];
            const int32_t row = e >= 0 && e < E ? row_of(a, off, e, pre[e] + slot[r]) : -1;
            if (p < wr.w1) {
                a.h.pair_to_row[p] = row;
                if (row >= 0)
                    a.h.row_to_pair[row] = (int32_t)p;
            }
        }
    }

    // 4. rows that hold no pair; 5. counts and offsets, a slice per block
    fill_unused_rows<0>(a, tot, off);
    publish<0>(a, tot, off, over[0], tot[E]);
}

// ---- schedule 1: one launch ---------------------------------------------------

// PREFETCH: blocks after a.nblocks bring the token rows of the dispatch that
// follows into the Infinity Cache instead (the large fused dispatch).
template <bool PREFETCH>
__global__ __launch_bounds__(kSingleThreads) void layout_single(LayoutArgs a)
{
    extern __shared__ int32_t lds[];
    __shared__ int32_t red[kMaxBlockWaves];
    if (PREFETCH && (int)blockIdx.x >= a.nblocks) {
        dev::prefetch_rows(a.pf_x, a.pf_T, a.pf_H, blockIdx.x - a.nblocks, a.pf_blocks);
        return;
    }
    dev::single_layout_block(a, lds, red, nullptr);
}

}  // namespace

// Waves per block: the rank and single kernels keep a [waves][E] int32 table
// in LDS (at most 32 KiB).
static int layout_waves(int32_t E) { return E <= 512 ? 16 : (E <= 1024 ? 8 : 4); }

LayoutPlan layout_plan(int64_t P, int32_t E)
{
    LayoutPlan plan;
    plan.waves = layout_waves(E);
    plan.single = P <= kSingleMaxPairs && E <= 512;
    if (plan.single)
        plan.waves = kSingleThreads / kWave;  // the one-launch kernel is built for this block size
    const int64_t per_round = (int64_t)plan.waves * kWave;  // pairs per block per round
    int64_t rounds = (P + per_round * kLayoutMaxBlocks - 1) / (per_round * kLayoutMaxBlocks);
    if (rounds < 1 || plan.single)
        rounds = 1;
    plan.rounds = (int32_t)rounds;
    plan.chunk = (int32_t)(per_round * rounds);
    int64_t nb = (P + plan.chunk - 1) / plan.chunk;
    if (plan.single && nb < kSingleMinBlocks)
        nb = kSingleMinBlocks;  // blocks past the last pair only fill unused rows and publish
    plan.nblocks = (int32_t)(nb < 1 ? 1 : nb);
    return plan;
}

size_t layout_table_bytes(int32_t E)
{
    const size_t b = sizeof(int32_t) * (size_t)(E + 1) * kLayoutMaxBlocks;
    return (b + 255) / 256 * 256;
}

hipError_t launch_layout(const LayoutArgs &a, const LayoutPlan &plan, hipStream_t stream)
{
    const dim3 grid(a.nblocks), block(plan.waves * kWave);
    if (plan.single) {
        const size_t lds = sizeof(int32_t) * dev::single_layout_lds_words(a.E, plan.waves);
        if (a.pf_blocks > 0)
            hipLaunchKernelGGL(layout_single<true>, dim3(a.nblocks + a.pf_blocks), block, lds, stream, a);
        else
            hipLaunchKernelGGL(layout_single<false>, grid, block, lds, stream, a);
        return hipGetLastError();
    }
    // prefetch blocks (a fused call, split_prefetch_plan) run the same block
    // size as prefetch_rows assumes
    const bool pf = a.pf_blocks > 0 && plan.waves * kWave == kSingleThreads;
    if (a.P > 0) {
        const size_t lds = sizeof(int32_t) * (size_t)plan.waves * a.E;
        const int extra = pf && a.pf_T > 0 ? a.pf_blocks : 0;
        hipLaunchKernelGGL(layout_rank, dim3(a.nblocks + extra), block, lds, stream, a);
    }
    const size_t lds = sizeof(int32_t) * (size_t)(3 * a.E + 4);
    const int extra = pf && a.pf2_T > 0 ? a.pf_blocks : 0;
    hipLaunchKernelGGL(layout_index, dim3(a.nblocks + extra), block, lds, stream, a);
    return hipGetLastError();
}

}  // namespace moe
