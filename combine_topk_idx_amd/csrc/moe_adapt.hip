// Adapters between the dispatched buffers and grouped-GEMM consumers on
// gfx950: per-row expert indices, masked <-> contiguous repack, and scales in
// MN-major order (page "[Feature] Add DeepEPv2 (ElasticBuffer) MoE A2A
// backend", Implementation: masked-slab repack kernels and GEMM adapters for
// contiguous prefill and masked decode, with fp32 and packed UE8M0 scales).
//
// Row adapters walk the received rows only: every block first scans
// recv_count in LDS (rows before each expert, and the align-padded contiguous
// segment offsets), a wave finds the expert of its row by binary search, and
// the row's bytes move with non-temporal 16-byte loads and stores; one launch
// does the whole repack.  The scale adapter is an LDS-tiled transpose.
#include "moe_device.h"

namespace moe {

namespace {

// Exclusive scan of recv_count rounded up to `align`, into off[0..E] in LDS.
// Block-wide (kBlockThreads threads; red holds kWavesPerBlock words); ends
// with a barrier.
__device__ inline void padded_offsets(const int32_t *recv_count, int32_t E, int32_t align, int32_t *off,
                                      int32_t *red)
{
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int per = (E + kBlockThreads - 1) / kBlockThreads;
    const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
    int32_t local = 0;
    for (int e = e0; e < e1; ++e)
        local += (recv_count[e] + align - 1) / align * align;
    const int32_t incl = dev::wave_inclusive_sum(local);
    if (lane == kWave - 1)
        red[wave] = incl;
    __syncthreads();
    int32_t run = dev::sum_before<kWavesPerBlock>(red, wave) + incl - local;
    for (int e = e0; e < e1; ++e) {
        off[e] = run;
        run += (recv_count[e] + align - 1) / align * align;
    }
    if (tid == kBlockThreads - 1)
        off[E] = run;
    __syncthreads();
}

// Copies `row_bytes` (a multiple of 16) of one row, the iterations
// [it0, it0 + n) of kAdaptWidth bytes each, with non-temporal 16-byte moves.
__device__ __forceinline__ void copy_row_part(const uint8_t *src, uint8_t *dst, int row_bytes, int it0, int n,
                                              int lane)
{
    uint4 v[kAdaptMaxIters];
#pragma unroll
    for (int i = 0; i < kAdaptMaxIters; ++i) {
        const int off = (it0 + i) * kAdaptWidth + lane * 16;
        if (i < n && off < row_bytes) {
            const dev::u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const dev::u32x4 *>(src + off));
            v[i] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
#pragma unroll
    for (int i = 0; i < kAdaptMaxIters; ++i) {
        const int off = (it0 + i) * kAdaptWidth + lane * 16;
        if (i < n && off < row_bytes)
            dev::store_stream(dst + off, v[i]);
    }
}

// row_expert[r] = e over expert e's received rows, -1 over its unused rows
// and over the tail [off[E], rows): one expert per wave over the grid.
__device__ inline void fill_row_expert(const int32_t *off, const int32_t *recv_count, int32_t E, int64_t rows,
                                       int32_t *row_expert)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gwave = (int64_t)blockIdx.x * (kBlockThreads / kWave) + threadIdx.x / kWave;
    const int64_t gwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
    for (int64_t e = gwave; e < E; e += gwaves) {
        const int32_t used = recv_count[e];
        for (int32_t r = off[e] + lane; r < off[e + 1]; r += kWave)
            row_expert[r] = r < off[e] + used ? (int32_t)e : -1;
    }
    const int64_t tail0 = off[E];
    const int64_t span = (rows - tail0 + gwaves - 1) / gwaves;
    const int64_t r0 = tail0 + gwave * span;
    const int64_t r1 = min(rows, r0 + span);
    for (int64_t r = r0 + lane; r < r1; r += kWave)
        row_expert[r] = -1;
}

__global__ __launch_bounds__(kBlockThreads) void row_expert_kernel(RowExpertArgs a)
{
    fill_row_expert(a.expert_offset, a.recv_count, a.E, a.rows, a.row_expert);
}

template <bool TO_CONTIGUOUS>
__global__ __launch_bounds__(kBlockThreads) void repack_kernel(RepackArgs a)
{
    extern __shared__ int32_t lds[];
    int32_t *kept = lds;           // [E + 1] exclusive scan of recv_count: kept rows before expert e
    int32_t *off = lds + a.E + 1;  // [E + 1] contiguous segment offsets
    __shared__ int32_t red[kWavesPerBlock];
    padded_offsets(a.recv_count, a.E, 1, kept, red);
    if (TO_CONTIGUOUS) {
        padded_offsets(a.recv_count, a.E, a.align, off, red);
        if (blockIdx.x == 0)
            for (int e = threadIdx.x; e <= a.E; e += kBlockThreads)
                a.out_offset[e] = off[e];
    } else {
        for (int e = threadIdx.x; e <= a.E; e += kBlockThreads)
            off[e] = a.in_offset[e];
        __syncthreads();
    }
    const int32_t total = kept[a.E];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const RowPlan &pl = a.plan;
    // items walk the kept rows only: item -> (kept row k, part c)
    for (int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wave; item < pl.n_items;
         item += (int64_t)gridDim.x * kWavesPerBlock) {
        const int32_t k = (int32_t)(item / pl.items_per_token);
        if (k >= total)
            break;  // items only grow along the stride
        const int c = (int)(item - (int64_t)k * pl.items_per_token);
        // the expert holding kept row k: the last e with kept[e] <= k
        int lo = 0, hi = a.E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (kept[mid] <= k)
                lo = mid;
            else
                hi = mid;
        }
        const int32_t s = k - kept[lo];
        const int64_t q = (int64_t)lo * a.C + s;   // slab row
        const int64_t crow = (int64_t)off[lo] + s;  // contiguous row
        const int64_t src_row = TO_CONTIGUOUS ? q : crow;
        const int64_t dst_row = TO_CONTIGUOUS ? crow : q;
        const int it0 = c * pl.iters_per_item;
        const int n = min(pl.iters_per_item, pl.n_iters - it0);
        copy_row_part(a.x + src_row * a.row_bytes, a.out_x + dst_row * a.row_bytes, a.row_bytes, it0, n, lane);
        if (c == 0 && a.scale_words > 0) {
            const uint32_t *ss = reinterpret_cast<const uint32_t *>(a.scale) + src_row * a.scale_words;
            uint32_t *ds = reinterpret_cast<uint32_t *>(a.out_scale) + dst_row * a.scale_words;
            for (int w = lane; w < a.scale_words; w += kWave)
                ds[w] = ss[w];
        }
    }
    if (TO_CONTIGUOUS)
        fill_row_expert(off, a.recv_count, a.E, a.out_rows, a.out_row_expert);
}

// 32-bit [rows, S] -> [S, ld]: a 64 x 64 tile per block, read along S and
// written along rows, through an LDS tile padded by one column.
__global__ __launch_bounds__(kBlockThreads) void scales_mn_major_kernel(MnMajorArgs a)
{
    __shared__ uint32_t tile[kTransposeTile][kTransposeTile + 1];
    const int64_t r0 = (int64_t)blockIdx.x * kTransposeTile;
    const int j0 = blockIdx.y * kTransposeTile;
    const int tx = threadIdx.x & (kTransposeTile - 1);
    const int ty = threadIdx.x / kTransposeTile;  // 0..3
    constexpr int kRowsPerPass = kBlockThreads / kTransposeTile;
    for (int i = ty; i < kTransposeTile; i += kRowsPerPass) {
        const int64_t r = r0 + i;
        const int j = j0 + tx;
        tile[i][tx] = (r < a.rows && j < a.S) ? a.in[r * a.S + j] : 0u;
    }
    __syncthreads();
    for (int i = ty; i < kTransposeTile; i += kRowsPerPass) {
        const int j = j0 + i;
        const int64_t r = r0 + tx;
        if (j < a.S && r < a.ld)
            a.out[(int64_t)j * a.ld + r] = tile[tx][i];
    }
}

}  // namespace

hipError_t launch_row_expert(const RowExpertArgs &a, hipStream_t stream)
{
    int64_t grid = (a.E + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t cap = (int64_t)device_cu_count() * 4;
    if (grid > cap)
        grid = cap;
    hipLaunchKernelGGL(row_expert_kernel, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(kBlockThreads), 0, stream,
                       a);
    return hipGetLastError();
}

hipError_t launch_repack(const RepackArgs &a, hipStream_t stream)
{
    // every block starts with the segment offsets of all experts: keep the
    // grid at 8 blocks per compute unit and let waves stride over the items
    int64_t grid = a.plan.grid;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (grid > cap)
        grid = cap;
    const size_t lds = sizeof(int32_t) * 2 * (size_t)(a.E + 1);
    if (a.to_contiguous)
        hipLaunchKernelGGL(repack_kernel<true>, dim3((unsigned)grid), dim3(kBlockThreads), lds, stream, a);
    else
        hipLaunchKernelGGL(repack_kernel<false>, dim3((unsigned)grid), dim3(kBlockThreads), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_scales_mn_major(const MnMajorArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)((a.ld + kTransposeTile - 1) / kTransposeTile),
                    (unsigned)((a.S + kTransposeTile - 1) / kTransposeTile));
    hipLaunchKernelGGL(scales_mn_major_kernel, grid, dim3(kBlockThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace moe
