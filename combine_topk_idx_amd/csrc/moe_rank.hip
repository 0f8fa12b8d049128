// Per-rank deduplicated exchange on gfx950: the per-rank layout (which ranks
// each token must reach, and its row on each) and the receive-side expansion
// of per-rank rows into per-expert rows.
//
// The V1 dispatch computed this layout in a separate pre-pass
// (get_dispatch_layout; page "moe: add DeepEP V2 ElasticBuffer support to MoE
// token dispatcher", Motivation) so that a token bound for several experts of
// one rank is sent once.  The deduplicated dispatch itself is the row kernel
// of moe_dispatch.hip run over (token, rank) slots, and the two-level combine
// lives in moe_combine.hip.
//
// Layout: one launch.  Every block counts the tokens of every rank over the
// whole batch (wave ballots, one per rank, no atomics), so blocks never
// communicate; then it numbers its own tokens: per-chunk counts in LDS, a scan
// over chunks per rank, and each token's row on rank r = rank offset + tokens
// of r before the block + tokens of r in earlier chunks + lanes below it in
// its chunk.  The order is stable (ascending token) by construction.
#include "moe_device.h"

namespace moe {

namespace {

// Rank of expert e: e / L as a multiply by ceil(2^32 / L), exact for e < 2^21.
__device__ __forceinline__ uint32_t rank_bit(const RankLayoutArgs &a, int32_t e)
{
    const uint32_t r = (uint32_t)(((uint64_t)(uint32_t)e * a.rank_magic) >> 32);
    return (e >= 0 && e < a.E) ? 1u << r : 0u;
}

// Bit r set when one of token t's valid ids belongs to rank r.  The token's
// id loads are issued before any is used (16-byte vectors when rows of ids
// are 16-byte aligned), so one memory latency covers them.
__device__ __forceinline__ uint32_t rank_mask(const RankLayoutArgs &a, int t)
{
    const int32_t *ids = a.topk_idx + (int64_t)t * a.K;
    uint32_t m = 0;
    if (a.vec4) {
        int4 v[kMaxTopk / 4];
#pragma unroll
        for (int i = 0; i < kMaxTopk / 4; ++i)
            if (4 * i < a.K)
                v[i] = *reinterpret_cast<const int4 *>(ids + 4 * i);
#pragma unroll
        for (int i = 0; i < kMaxTopk / 4; ++i)
            if (4 * i < a.K)
                m |= rank_bit(a, v[i].x) | rank_bit(a, v[i].y) | rank_bit(a, v[i].z) | rank_bit(a, v[i].w);
    } else {
        for (int k = 0; k < a.K; ++k)
            m |= rank_bit(a, ids[k]);
    }
    return m;
}

// Rank mask of a token from its KV 16-byte id vectors.
template <int KV>
__device__ __forceinline__ uint32_t rank_mask_of(const RankLayoutArgs &a, const int4 (&v)[KV])
{
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < KV; ++i)
        m |= rank_bit(a, v[i].x) | rank_bit(a, v[i].y) | rank_bit(a, v[i].z) | rank_bit(a, v[i].w);
    return m;
}

// KV > 0: K = 4 * KV ids per token in 16-byte vectors, and phase 1 issues the
// loads of all its chunks before any mask is formed (token indices are
// clamped instead of branched on, so nothing splits the loads into separate
// round trips).  KV = 0: any K, the token-by-token path.
template <int KV>
__global__ __launch_bounds__(kRankLayoutWaves *kWave) void rank_layout_kernel(RankLayoutArgs a)
{
    extern __shared__ int32_t chunk_base[];  // [chunks of this block][R], then the block's token masks
    uint32_t *mask_cache = reinterpret_cast<uint32_t *>(chunk_base) +
                           (size_t)(a.tokens_per_block / kWave) * a.R;  // [tokens_per_block] if a.cache_masks
    __shared__ int32_t wtot[kRankLayoutWaves][kMaxDedupRanks];
    __shared__ int32_t wbef[kRankLayoutWaves][kMaxDedupRanks];
    __shared__ int32_t base[kMaxDedupRanks];
    __shared__ int32_t total_rows;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    constexpr int nwaves = kRankLayoutWaves;  // the launch's block size (blockDim.x would be a load)
    const int R = a.R;
    const int t0 = blockIdx.x * a.tokens_per_block;
    const int t1 = min(a.T, t0 + a.tokens_per_block);

    // 1. tokens per rank over the whole batch, and before this block; lane r
    //    of each wave accumulates rank r
    int32_t tot = 0, bef = 0;
    const int nchunks = (a.T + kWave - 1) / kWave;
    constexpr int kPass = KV == 0 ? 4 : (KV <= 2 ? 4 : 2);  // chunks per wave whose loads are in flight together
    for (int c = wave; c < nchunks; c += kPass * nwaves) {
        uint32_t m[kPass];
        if constexpr (KV > 0) {
            int4 v[kPass][KV];
#pragma unroll
            for (int i = 0; i < kPass; ++i) {
                const int t = min((c + i * nwaves) * kWave + lane, a.T - 1);
                const int4 *p = reinterpret_cast<const int4 *>(a.topk_idx + (int64_t)t * a.K);
#pragma unroll
                for (int j = 0; j < KV; ++j)
                    v[i][j] = p[j];
            }
#pragma unroll
            for (int i = 0; i < kPass; ++i) {
                const int t = (c + i * nwaves) * kWave + lane;
                m[i] = t < a.T ? rank_mask_of<KV>(a, v[i]) : 0u;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kPass; ++i) {
                const int t = (c + i * nwaves) * kWave + lane;
                m[i] = t < a.T ? rank_mask(a, t) : 0u;
            }
        }
        if (a.cache_masks) {
#pragma unroll
            for (int i = 0; i < kPass; ++i) {
                const int t = (c + i * nwaves) * kWave + lane;
                if (t >= t0 && t < t1)
                    mask_cache[t - t0] = m[i];
            }
        }
#pragma unroll
        for (int i = 0; i < kPass; ++i) {
            const int t = (c + i * nwaves) * kWave + lane;
            const uint64_t before = __ballot(t < t0);
            for (int r = 0; r < R; ++r) {
                const uint64_t b = __ballot((m[i] >> r) & 1u);
                if (lane == r) {
                    tot += __popcll(b);
                    bef += __popcll(b & before);
                }
            }
        }
    }
    if (lane < kMaxDedupRanks) {
        wtot[wave][lane] = tot;
        wbef[wave][lane] = bef;
    }
    __syncthreads();

    // 2. rank offsets (exclusive scan over ranks, one wave)
    if (wave == 0) {
        int32_t cnt = 0, before = 0;
        if (lane < R) {
#pragma unroll
            for (int w = 0; w < nwaves; ++w) {  // independent reads, all in flight
                cnt += wtot[w][lane];
                before += wbef[w][lane];
            }
        }
        const int32_t incl = dev::wave_inclusive_sum(cnt);
        const int32_t off = incl - cnt;
        if (lane < R)
            base[lane] = off + before;
        if (blockIdx.x == 0 && lane < R) {
            a.h.rank_token_count[lane] = cnt;
            a.h.rank_token_offset[lane] = off;
        }
        if (lane == R - 1) {
            total_rows = incl;
            if (blockIdx.x == 0)
                a.h.rank_token_offset[R] = incl;
        }
    }

    // 3. this block's tokens: counts per chunk of 64, then a scan over chunks
    __syncthreads();  // mask_cache is complete
    const int nch = t1 > t0 ? (t1 - t0 + kWave - 1) / kWave : 0;
    for (int j = wave; j < nch; j += nwaves) {
        const int t = t0 + j * kWave + lane;
        const uint32_t m = t < t1 ? (a.cache_masks ? mask_cache[t - t0] : rank_mask(a, t)) : 0u;
        for (int r = 0; r < R; ++r) {
            const uint64_t b = __ballot((m >> r) & 1u);
            if (lane == r)
                chunk_base[j * R + r] = __popcll(b);
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < R) {
        // exclusive scan over the block's chunks, kScanBatch counts read before any is rewritten
        constexpr int kScanBatch = 16;
        const int r = threadIdx.x;
        int32_t run = base[r];
        for (int j0 = 0; j0 < nch; j0 += kScanBatch) {
            int32_t c[kScanBatch];
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i)
                c[i] = j0 + i < nch ? chunk_base[(j0 + i) * R + r] : 0;
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i)
                if (j0 + i < nch) {
                    chunk_base[(j0 + i) * R + r] = run;
                    run += c[i];
                }
        }
    }
    __syncthreads();

    // 4. rows of this block's (token, rank) slots and the inverse map
    for (int j = wave; j < nch; j += nwaves) {
        const int t = t0 + j * kWave + lane;
        const bool in = t < t1;
        const uint32_t m = in ? (a.cache_masks ? mask_cache[t - t0] : rank_mask(a, t)) : 0u;
        for (int r = 0; r < R; ++r) {
            const bool bit = (m >> r) & 1u;
            const uint64_t b = __ballot(bit);
            if (in) {
                int32_t row = -1;
                if (bit) {
                    row = chunk_base[j * R + r] + dev::lanes_below(b);
                    a.h.rank_row_to_token[row] = t;
                }
                a.h.token_rank_row[(int64_t)t * R + r] = row;
            }
        }
    }

    // 5. rows past the last rank hold no token
    constexpr int kThreads = kRankLayoutWaves * kWave;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t q = total_rows + (int64_t)blockIdx.x * kThreads + threadIdx.x; q < a.rows_cap; q += stride)
        a.h.rank_row_to_token[q] = -1;
}

// Receive-side expansion.  Work items are (token, run of 1024-byte
// iterations of a row); the wave groups the token's kept pairs by source row
// (one per rank), reads each source row once with non-temporal 16-byte loads
// and stores it to every kept row of that rank.
__global__ __launch_bounds__(kBlockThreads) void expand_kernel(ExpandArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const RowPlan &pl = a.plan;
    for (int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wave; item < pl.n_items;
         item += (int64_t)gridDim.x * kWavesPerBlock) {
        const int t = (int)(item / pl.items_per_token);
        const int c = (int)(item - (int64_t)t * pl.items_per_token);
        const int64_t pbase = (int64_t)t * a.K;
        const int32_t row = lane < a.K ? a.pair_to_row[pbase + lane] : -1;
        const int32_t e = lane < a.K ? a.topk_idx[pbase + lane] : -1;
        const bool keep = row >= 0 && e >= 0 && e < a.E;
        const int32_t src = keep ? a.token_rank_row[(int64_t)t * a.R + e / a.L] : -1;
        const int it0 = c * pl.iters_per_item;
        const int n = min(pl.iters_per_item, pl.n_iters - it0);
        uint64_t todo = __ballot(keep && src >= 0);
        while (todo) {
            const int j = __builtin_ctzll(todo);
            const int32_t s = __builtin_amdgcn_readlane(src, j);
            const uint64_t group = __ballot(keep && src == s);
            todo &= ~group;
            const uint8_t *sp = a.send_x + (int64_t)s * a.row_bytes;
            uint4 v[kExpandMaxIters];
#pragma unroll
            for (int i = 0; i < kExpandMaxIters; ++i) {
                const int off = (it0 + i) * kExpandWidth + lane * 16;
                if (i < n && off < a.row_bytes) {
                    const dev::u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const dev::u32x4 *>(sp + off));
                    v[i] = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
            uint64_t m = group;
            while (m) {
                const int k = __builtin_ctzll(m);
                m &= m - 1;
                const int32_t dst = __builtin_amdgcn_readlane(row, k);
                uint8_t *dp = a.out_x + (int64_t)dst * a.row_bytes;
#pragma unroll
                for (int i = 0; i < kExpandMaxIters; ++i) {
                    const int off = (it0 + i) * kExpandWidth + lane * 16;
                    if (i < n && off < a.row_bytes)
                        dev::store_stream(dp + off, v[i]);
                }
            }
            if (c == 0 && a.scale_words > 0) {
                const uint32_t *ss = reinterpret_cast<const uint32_t *>(a.send_scale) + (int64_t)s * a.scale_words;
                for (int wd = lane; wd < a.scale_words; wd += kWave) {
                    const uint32_t val = ss[wd];
                    uint64_t mm = group;
                    while (mm) {
                        const int k = __builtin_ctzll(mm);
                        mm &= mm - 1;
                        const int32_t dst = __builtin_amdgcn_readlane(row, k);
                        reinterpret_cast<uint32_t *>(a.out_scale)[(int64_t)dst * a.scale_words + wd] = val;
                    }
                }
            }
        }
    }
}

}  // namespace

bool rank_layout_plan(int32_t T, int32_t R, RankLayoutArgs &a)
{
    const int64_t chunks = (T + kWave - 1) / kWave;
    int64_t nblocks = (T + 1023) / 1024;
    if (nblocks > kLayoutMaxBlocks)
        nblocks = kLayoutMaxBlocks;
    // the chunk counts of one block must fit the LDS budget
    const int64_t max_chunks = kRankLayoutMaxLdsWords / (R > 0 ? R : 1);
    const int64_t need = (chunks + max_chunks - 1) / max_chunks;
    if (nblocks < need)
        nblocks = need;
    if (nblocks < 1)
        nblocks = 1;
    const int64_t cpb = (chunks + nblocks - 1) / nblocks;
    a.tokens_per_block = (int32_t)(cpb > 0 ? cpb * kWave : kWave);
    a.nblocks = (int32_t)(T > 0 ? (T + a.tokens_per_block - 1) / a.tokens_per_block : 1);
    a.cache_masks = a.tokens_per_block <= kRankLayoutMaxCachedTokens ? 1 : 0;
    return true;
}

hipError_t launch_rank_layout(const RankLayoutArgs &a, hipStream_t stream)
{
    const size_t lds = sizeof(int32_t) * ((size_t)(a.tokens_per_block / kWave) * (size_t)a.R +
                                          (a.cache_masks ? (size_t)a.tokens_per_block : 0));
    const dim3 grid(a.nblocks), block(kRankLayoutWaves * kWave);
    const int kv = a.vec4 && a.T > 0 ? a.K / 4 : 0;
    if (kv == 2)
        hipLaunchKernelGGL(rank_layout_kernel<2>, grid, block, lds, stream, a);
    else if (kv == 1)
        hipLaunchKernelGGL(rank_layout_kernel<1>, grid, block, lds, stream, a);
    else
        hipLaunchKernelGGL(rank_layout_kernel<0>, grid, block, lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_expand(const ExpandArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL(expand_kernel, dim3(a.plan.grid), dim3(kBlockThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace moe
