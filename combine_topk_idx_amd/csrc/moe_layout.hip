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
// Two launches, no atomics that decide an order:
//   layout_count  one workgroup per chunk of pairs: LDS histogram of its chunk
//                 -> workspace row [block][E], plus its invalid-id count.
//   layout_index  one workgroup per chunk again: every workgroup reads the
//                 whole (small) histogram table, derives the segment offsets
//                 and its own cross-chunk prefix, then ranks its pairs with
//                 64-lane ballot matching (stable inside a wave), writes both
//                 maps, the padding rows of its share of experts, and block 0
//                 writes the counts, offsets and status.
#include "moe_internal.h"

namespace moe {

namespace {

// Lanes of the wave holding the same routed expert as this lane: one ballot
// per expert-id bit.  Returns 0 for lanes that are not routed.
__device__ __forceinline__ uint64_t match_expert(int32_t e, bool routed, int nbits)
{
    uint64_t m = __ballot(routed);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return routed ? m : 0ull;
}

// Number of set bits of m below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ __launch_bounds__(kBlockThreads) void layout_count(LayoutArgs a)
{
    extern __shared__ int32_t hist[];  // [E + 1], hist[E] = invalid ids
    const int tid = threadIdx.x;
    for (int i = tid; i <= a.E; i += kBlockThreads)
        hist[i] = 0;
    __syncthreads();

    const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
    const int64_t c1 = min(a.P, c0 + a.chunk);
    int invalid = 0;
    for (int64_t p = c0 + tid; p < c1; p += kBlockThreads) {
        const int32_t e = a.topk_idx[p];
        if (e >= 0 && e < a.E)
            atomicAdd(&hist[e], 1);
        else if (e != -1)
            ++invalid;
    }
    if (invalid)
        atomicAdd(&hist[a.E], invalid);
    __syncthreads();

    int32_t *row = a.ws + (int64_t)blockIdx.x * (a.E + 1);
    for (int i = tid; i <= a.E; i += kBlockThreads)
        row[i] = hist[i];
}

__global__ __launch_bounds__(kBlockThreads) void layout_index(LayoutArgs a)
{
    extern __shared__ int32_t lds[];
    const int E = a.E;
    int32_t *tot = lds;              // [E]   pairs per expert, all chunks
    int32_t *pre = tot + E;          // [E]   pairs per expert in earlier chunks
    int32_t *off = pre + E;          // [E+1] segment starts
    int32_t *cnt = off + E + 1;      // [4][E] per-wave counts, then per-wave slot bases
    __shared__ int32_t red[kWavesPerBlock * 2];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int blk = blockIdx.x;
    const bool contiguous = a.layout == MOE_LAYOUT_CONTIGUOUS;

    // 1. totals and this chunk's prefix, from the histogram table (no pairs:
    //    the count kernel did not run and the table is not read)
    const int table_rows = a.P > 0 ? a.nblocks : 0;
    for (int e = tid; e < E; e += kBlockThreads) {
        int32_t t = 0, p = 0;
        for (int b = 0; b < table_rows; ++b) {
            const int32_t v = a.ws[(int64_t)b * (E + 1) + e];
            t += v;
            p += b < blk ? v : 0;
        }
        tot[e] = t;
        pre[e] = p;
    }
    for (int i = tid; i < kWavesPerBlock * E; i += kBlockThreads)
        cnt[i] = 0;
    __syncthreads();

    // 2. segment offsets: exclusive scan of padded sizes (contiguous) or e*C
    if (contiguous) {
        const int per = (E + kBlockThreads - 1) / kBlockThreads;
        const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
        int32_t local = 0;
        for (int e = e0; e < e1; ++e)
            local += (tot[e] + a.align - 1) / a.align * a.align;
        // inclusive scan of `local` over the wave
        int32_t incl = local;
        for (int d = 1; d < kWave; d <<= 1) {
            const int32_t v = __shfl_up(incl, d);
            if (lane >= d)
                incl += v;
        }
        if (lane == kWave - 1)
            red[wave] = incl;
        __syncthreads();
        int32_t base = 0;
        for (int w = 0; w < wave; ++w)
            base += red[w];
        int32_t run = base + incl - local;
        for (int e = e0; e < e1; ++e) {
            off[e] = run;
            run += (tot[e] + a.align - 1) / a.align * a.align;
        }
        if (tid == kBlockThreads - 1)
            off[E] = run;
    } else {
        for (int e = tid; e <= E; e += kBlockThreads)
            off[e] = e * a.capacity;
    }

    // 3. each wave counts its quarter of the chunk
    const int64_t c0 = (int64_t)blk * a.chunk;
    const int64_t c1 = min(a.P, c0 + a.chunk);
    const int quarter = a.chunk / kWavesPerBlock;
    const int64_t q0 = min(c1, c0 + (int64_t)wave * quarter);
    const int64_t q1 = min(c1, q0 + quarter);
    int32_t *mycnt = cnt + wave * E;
    for (int64_t base = q0; base < q1; base += kWave) {
        const int64_t p = base + lane;
        const int32_t e = p < q1 ? a.topk_idx[p] : -1;
        const bool routed = p < q1 && e >= 0 && e < E;
        const uint64_t m = match_expert(e, routed, a.nbits);
        if (routed && lanes_below(m) == 0)
            mycnt[e] += __popcll(m);
    }
    __syncthreads();

    // 4. slot base of each wave for each expert
    for (int e = tid; e < E; e += kBlockThreads) {
        int32_t s = pre[e];
        for (int w = 0; w < kWavesPerBlock; ++w) {
            const int32_t c = cnt[w * E + e];
            cnt[w * E + e] = s;
            s += c;
        }
    }
    __syncthreads();

    // 5. stable slots, rows, and both maps
    for (int64_t base = q0; base < q1; base += kWave) {
        const int64_t p = base + lane;
        const bool in = p < q1;
        const int32_t e = in ? a.topk_idx[p] : -1;
        const bool routed = in && e >= 0 && e < E;
        const uint64_t m = match_expert(e, routed, a.nbits);
        int32_t row = -1;
        if (routed) {
            const int rank = lanes_below(m);
            const int32_t first = mycnt[e];     // read by every lane of the match ...
            const int32_t slot = first + rank;
            if (rank == 0)
                mycnt[e] = first + __popcll(m);  // ... before its leader advances it
            if (contiguous)
                row = off[e] + slot;
            else if (slot < a.capacity)
                row = e * a.capacity + slot;
        }
        if (in) {
            a.h.pair_to_row[p] = row;
            if (row >= 0)
                a.h.row_to_pair[row] = (int32_t)p;
        }
    }

    // 6. rows that hold no pair: padding of this block's share of experts and
    //    a slice of the unused tail
    for (int e = blk; e < E; e += a.nblocks) {
        const int32_t used = contiguous ? tot[e] : min(tot[e], a.capacity);
        for (int32_t r = off[e] + used + tid; r < off[e + 1]; r += kBlockThreads)
            a.h.row_to_pair[r] = -1;
    }
    {
        const int64_t tail0 = off[E];
        const int64_t span = (a.rows_cap - tail0 + a.nblocks - 1) / a.nblocks;
        const int64_t r0 = tail0 + (int64_t)blk * span;
        const int64_t r1 = min((int64_t)a.rows_cap, r0 + span);
        for (int64_t r = r0 + tid; r < r1; r += kBlockThreads)
            a.h.row_to_pair[r] = -1;
    }

    // 7. block 0 publishes counts, offsets and status
    if (blk == 0) {
        int32_t overflow = 0;
        for (int e = tid; e < E; e += kBlockThreads) {
            a.h.expert_count[e] = tot[e];
            a.h.recv_count[e] = contiguous ? tot[e] : min(tot[e], a.capacity);
            a.h.expert_offset[e] = off[e];
            if (!contiguous)
                overflow += max(0, tot[e] - a.capacity);
        }
        for (int r = tid; r <= a.R; r += kBlockThreads)
            a.h.rank_offset[r] = off[r * a.L];
        if (tid == 0)
            a.h.expert_offset[E] = off[E];
        int32_t invalid = 0;
        for (int b = tid; b < table_rows; b += kBlockThreads)
            invalid += a.ws[(int64_t)b * (E + 1) + E];
        for (int d = kWave / 2; d > 0; d >>= 1) {
            overflow += __shfl_xor(overflow, d);
            invalid += __shfl_xor(invalid, d);
        }
        __syncthreads();  // `red` is reused
        if (lane == 0) {
            red[wave] = overflow;
            red[kWavesPerBlock + wave] = invalid;
        }
        __syncthreads();
        if (tid == 0) {
            int32_t o = 0, v = 0;
            for (int w = 0; w < kWavesPerBlock; ++w) {
                o += red[w];
                v += red[kWavesPerBlock + w];
            }
            a.h.status[0] = o;
            a.h.status[1] = v;
        }
    }
}

}  // namespace

LayoutPlan layout_plan(int64_t P)
{
    const int64_t unit = kLayoutChunkUnit;
    int64_t per = (P + (int64_t)kLayoutMaxBlocks * unit - 1) / ((int64_t)kLayoutMaxBlocks * unit);
    if (per < 1)
        per = 1;
    LayoutPlan plan;
    plan.chunk = (int32_t)(per * unit);
    int64_t nb = (P + plan.chunk - 1) / plan.chunk;
    plan.nblocks = (int32_t)(nb < 1 ? 1 : nb);
    return plan;
}

hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream)
{
    if (a.P > 0) {
        const size_t lds = sizeof(int32_t) * (size_t)(a.E + 1);
        hipLaunchKernelGGL(layout_count, dim3(a.nblocks), dim3(kBlockThreads), lds, stream, a);
    }
    const size_t lds = sizeof(int32_t) * (size_t)(7 * a.E + 1);
    hipLaunchKernelGGL(layout_index, dim3(a.nblocks), dim3(kBlockThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace moe
