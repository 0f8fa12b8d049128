// Combine on gfx950: the router-weighted top-k reduction of expert outputs
// back to token order (page vLLM tools/ep_kernels, commit message: weighted
// reduction in combine), with nothing reduced afterwards (page "[Feature] Add
// DeepEPv2 (ElasticBuffer) MoE A2A backend", review: an extra post-expert
// reduction double-counts).
//
// Token-major: a wave owns a token (or a run of its columns).  The token's
// kept rows and weights are compacted once into lanes 0..n-1 (ds_permute),
// then every 1024-column iteration issues two 16-byte loads per kept row (up
// to 16 in flight per lane; non-temporal when the combine reads more than
// 64 MiB), accumulates in ascending k in fp32 with the product
// and the sum each rounded (no FMA), and stores 8 bf16 (round to nearest even,
// v_cvt_pk_bf16_f32) as 16-byte vectors, written through L2 (device-scope
// buffer stores) or, for outputs larger than half the Infinity Cache,
// non-temporally.
//
// The same kernel serves the two levels of the per-rank deduplicated combine
// (the multiple-reduction option on page vLLM tools/ep_kernels, commit
// message).  PARTIAL: the token's pairs are compacted in (rank, k) order and
// the running sum is stored as one bf16 partial row per (token, rank) each
// time the rank changes.  The final reduction is the plain kernel over the
// (token, rank) rows with unit weights.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kBatch = 8;  // kept rows whose loads are in flight together
constexpr int kVecs = kCombineWidth / (kWave * 8);  // 16-byte vectors per lane per row per iteration

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Expert outputs are read exactly once.  Large reads (NT) use non-temporal
// loads, which keep them from displacing useful lines in L2 and the MALL (a
// streaming kernel with the DeepSeek-V3 prefill combine's traffic: 176.5 us,
// against 204 us with plain loads and 204-209 us with any coherence-scope bit
// on the loads).  Small reads use plain loads, which find rows that are still
// in the Infinity Cache and leave them there (DeepSeek-V3 decode: combine 6.9
// -> 6.4 us, a 20-step graph step 14.4-15.1 -> 14.0 us).
template <bool NT>
__device__ __forceinline__ uint4 load_row(const uint16_t *p)
{
    u32x4 v;
    if constexpr (NT)
        v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    else
        v = *reinterpret_cast<const u32x4 *>(p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    const __bf16 ha = (__bf16)a, hb = (__bf16)b;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Word 3 of a raw buffer resource: 32-bit data format, no swizzle or index.
constexpr int kRawBufferWord3 = 0x00020000;
// Cache-policy bit of a buffer store: device (agent) coherence scope, sc1.
constexpr int kStoreDeviceScope = 16;

// Stores the bf16 of the sums of row `row` (H columns) and clears them.
// NT: non-temporal stores (outputs larger than half the Infinity Cache).
// Otherwise the stores carry the device coherence scope: on gfx950 they are
// written through L2 to the memory-side cache instead of staying dirty in L2
// until the write-back at the end of the kernel, which the next kernel waits
// for (DeepSeek-V3 prefill combine, 117 MB out: 182.7 -> 177.3 us; a
// streaming kernel with this mix: 181 us plain, 176.5 us device scope, 188 us
// non-temporal).
template <bool NT>
__device__ __forceinline__ void store_row(uint16_t *row, int32_t H, const int (&col)[kVecs],
                                          const bool (&active)[kVecs], float (&acc)[kVecs][8])
{
    // row is wave-uniform, so the resource lives in scalar registers; the
    // range is the row's 2*H bytes (H < 2^31), offsets 2*col < 2*H
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(row, 0, (int)(2u * (uint32_t)H), kRawBufferWord3);
#pragma unroll
    for (int s = 0; s < kVecs; ++s) {
        if (active[s]) {
            u32x4 o;
            o[0] = pack_bf16(acc[s][0], acc[s][1]);
            o[1] = pack_bf16(acc[s][2], acc[s][3]);
            o[2] = pack_bf16(acc[s][4], acc[s][5]);
            o[3] = pack_bf16(acc[s][6], acc[s][7]);
            if constexpr (NT)
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(row + col[s]));
            else
                __builtin_amdgcn_raw_buffer_store_b128(o, rsrc, (int)(2u * (uint32_t)col[s]), 0, kStoreDeviceScope);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[s][e] = 0.0f;
    }
}

#pragma clang fp contract(off)
__device__ __forceinline__ void accumulate(float (&acc)[8], float w, const uint4 &v)
{
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(u[j] << 16);
        const float hi = __uint_as_float(u[j] & 0xFFFF0000u);
        const float plo = w * lo;
        const float phi = w * hi;
        acc[2 * j] = acc[2 * j] + plo;
        acc[2 * j + 1] = acc[2 * j + 1] + phi;
    }
}

template <bool PARTIAL, bool NT, bool NT_IN>
__global__ __launch_bounds__(kBlockThreads) void combine_kernel(CombineArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const RowPlan &pl = a.plan;
    for (int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wave; item < pl.n_items;
         item += (int64_t)gridDim.x * kWavesPerBlock) {
        const int t = (int)(item / pl.items_per_token);
        const int c = (int)(item - (int64_t)t * pl.items_per_token);

        const int64_t pbase = (int64_t)t * a.K;
        const int32_t r = lane < a.K ? a.pair_to_row[pbase + lane] : -1;
        const float w = lane < a.K ? (a.topk_w != nullptr ? a.topk_w[pbase + lane] : 1.0f) : 0.0f;
        int n, dst;
        int32_t grp = 0, qrow = 0;
        if constexpr (!PARTIAL) {
            // kept rows of the token, compacted in ascending k into lanes 0..n-1
            const uint64_t kept = __ballot(r >= 0);
            n = __popcll(kept);
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(kept >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)kept, 0u));
            // kept lanes go to slot `below`; the others park in lanes 32.. (unused)
            dst = r >= 0 ? below : kMaxTopk + (lane & (kMaxTopk - 1));
        } else {
            // pairs with a valid id (kept or dropped), compacted in (rank, k)
            // order; a dropped pair still opens its rank's partial row
            const int32_t e = lane < a.K ? a.topk_idx[pbase + lane] : -1;
            const bool valid = e >= 0 && e < a.E;
            const int32_t g = valid ? e / a.L : 0;
            const uint64_t vm = __ballot(valid);
            n = __popcll(vm);
            int slot = 0;
            for (int j = 0; j < a.K; ++j) {
                const int32_t gj = __builtin_amdgcn_readlane(g, j);
                slot += (((vm >> j) & 1) && (gj < g || (gj == g && j < lane))) ? 1 : 0;
            }
            dst = valid ? slot : kMaxTopk + (lane & (kMaxTopk - 1));
            const int32_t q = valid ? a.token_rank_row[(int64_t)t * a.R + g] : -1;
            grp = __builtin_amdgcn_ds_permute(dst * 4, g);
            qrow = __builtin_amdgcn_ds_permute(dst * 4, q);
        }
        const int32_t rows = __builtin_amdgcn_ds_permute(dst * 4, r);
        const float wts = __int_as_float(__builtin_amdgcn_ds_permute(dst * 4, __float_as_int(w)));

        const int it0 = c * pl.iters_per_item;
        const int it1 = min(it0 + pl.iters_per_item, pl.n_iters);
        uint16_t *outp = a.out + (int64_t)t * a.H;
        for (int it = it0; it < it1; ++it) {
            // this iteration's columns: 8 at col[0] and 8 at col[1] = col[0] + 512
            int col[kVecs];
            bool active[kVecs];
#pragma unroll
            for (int s = 0; s < kVecs; ++s) {
                col[s] = it * kCombineWidth + s * (kWave * 8) + lane * 8;
                active[s] = col[s] < a.H;
            }
            float acc[kVecs][8];
#pragma unroll
            for (int s = 0; s < kVecs; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[s][e] = 0.0f;
            for (int j0 = 0; j0 < n; j0 += kBatch) {
                uint4 v[kBatch][kVecs];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const int32_t rj = __builtin_amdgcn_readlane(rows, j0 + j);
                    if (j0 + j < n && (!PARTIAL || rj >= 0)) {
                        const uint16_t *src = a.y + (int64_t)rj * a.H;
#pragma unroll
                        for (int s = 0; s < kVecs; ++s)
                            if (active[s])
                                v[j][s] = load_row<NT_IN>(src + col[s]);
                    }
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    if (j0 + j < n) {
                        const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                        __float_as_int(wts), j0 + j));
                        if (!PARTIAL || __builtin_amdgcn_readlane(rows, j0 + j) >= 0) {
#pragma unroll
                            for (int s = 0; s < kVecs; ++s)
                                if (active[s])
                                    accumulate(acc[s], wj, v[j][s]);
                        }
                        if constexpr (PARTIAL) {
                            // the last pair of its rank: store the partial row, restart the sum
                            const int jj = j0 + j;
                            const bool last = jj == n - 1 || __builtin_amdgcn_readlane(grp, jj + 1) !=
                                                                 __builtin_amdgcn_readlane(grp, jj);
                            if (last) {
                                uint16_t *prow = a.out + (int64_t)__builtin_amdgcn_readlane(qrow, jj) * a.H;
                                store_row<NT>(prow, a.H, col, active, acc);
                            }
                        }
                    }
                }
            }
            if constexpr (!PARTIAL)
                store_row<NT>(outp, a.H, col, active, acc);
        }
    }
}

}  // namespace

namespace {

template <bool PARTIAL>
hipError_t launch_combine_kernel(const CombineArgs &a, hipStream_t stream)
{
    const dim3 grid(a.plan.grid), block(kBlockThreads);
    if (a.stream_out && a.stream_in)
        hipLaunchKernelGGL((combine_kernel<PARTIAL, true, true>), grid, block, 0, stream, a);
    else if (a.stream_out)
        hipLaunchKernelGGL((combine_kernel<PARTIAL, true, false>), grid, block, 0, stream, a);
    else if (a.stream_in)
        hipLaunchKernelGGL((combine_kernel<PARTIAL, false, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((combine_kernel<PARTIAL, false, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream)
{
    return launch_combine_kernel<false>(a, stream);
}

hipError_t launch_combine_partial(const CombineArgs &a, hipStream_t stream)
{
    return launch_combine_kernel<true>(a, stream);
}

}  // namespace moe
