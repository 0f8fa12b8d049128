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
// covers 8 blocks = two packed UE8M0 words.
#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// DPP lane exchange within a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// max over the 8 lanes [8j, 8j+8): quad xor 1, quad xor 2, then the mirror
// inside each half-row pairs quad 0 with quad 1.
__device__ __forceinline__ float max8(float v)
{
    v = fmaxf(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp<0x141>(v));  // row_half_mirror
    return v;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Dispatched rows are written once and read by a later kernel (the experts):
// non-temporal stores keep them from filling L2 and the MALL with dirty lines
// that the following kernels would have to evict (measured on the DeepSeek-V3
// prefill shape: dispatch 129 -> 98 us, and the next combine 216 -> 195 us).
__device__ __forceinline__ void store_stream(void *p, const uint4 &v)
{
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

// Four fp32 values -> four E4M3 bytes (byte i = value i), round to nearest
// even; the inputs are within [-448, 448].
__device__ __forceinline__ uint32_t pack_e4m3(float f0, float f1, float f2, float f3)
{
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, r, true);
    return (uint32_t)r;
}

// Lane k (< K) holds the row of pair t*K+k; returns the mask of kept pairs.
__device__ __forceinline__ uint64_t token_rows(const DispatchArgs &a, int t, int lane, int32_t &myrow)
{
    myrow = lane < a.K ? a.pair_to_row[(int64_t)t * a.K + lane] : -1;
    return __ballot(myrow >= 0);
}

__global__ __launch_bounds__(kBlockThreads) void dispatch_bf16(DispatchArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const RowPlan &pl = a.plan;
    for (int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wave; item < pl.n_items;
         item += (int64_t)gridDim.x * kWavesPerBlock) {
        const int t = (int)(item / pl.items_per_token);
        const int c = (int)(item - (int64_t)t * pl.items_per_token);
        int32_t myrow;
        const uint64_t kept = token_rows(a, t, lane, myrow);
        if (kept == 0)
            continue;
        if (c == 0 && a.out_row_weight != nullptr && myrow >= 0)
            a.out_row_weight[myrow] = a.topk_w[(int64_t)t * a.K + lane];

        const int it0 = c * pl.iters_per_item;
        const int n = min(pl.iters_per_item, pl.n_iters - it0);
        const uint16_t *src = a.x + (int64_t)t * a.H;
        uint4 buf[kDispatchBf16MaxIters];
#pragma unroll
        for (int i = 0; i < kDispatchBf16MaxIters; ++i) {
            const int col = (it0 + i) * kDispatchBf16Width + lane * 8;
            if (i < n && col < a.H)
                buf[i] = *reinterpret_cast<const uint4 *>(src + col);
        }
#pragma unroll
        for (int i = 0; i < kDispatchBf16MaxIters; ++i) {
            const int col = (it0 + i) * kDispatchBf16Width + lane * 8;
            if (i < n) {
                const uint4 d = buf[i];
                uint64_t m = kept;
                while (m) {
                    const int k = __builtin_ctzll(m);
                    m &= m - 1;
                    const int32_t row = __builtin_amdgcn_readlane(myrow, k);
                    uint16_t *dst = reinterpret_cast<uint16_t *>(a.out_x) + (int64_t)row * a.H;
                    if (col < a.H)
                        store_stream(dst + col, d);
                }
            }
        }
    }
}

template <int QUANT>
__global__ __launch_bounds__(kBlockThreads) void dispatch_fp8(DispatchArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const RowPlan &pl = a.plan;
    const int NB = a.H / kQuantGroup;
    const int NW = (NB + 3) / 4;
    for (int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wave; item < pl.n_items;
         item += (int64_t)gridDim.x * kWavesPerBlock) {
        const int t = (int)(item / pl.items_per_token);
        const int c = (int)(item - (int64_t)t * pl.items_per_token);
        int32_t myrow;
        const uint64_t kept = token_rows(a, t, lane, myrow);
        if (kept == 0)
            continue;
        if (c == 0 && a.out_row_weight != nullptr && myrow >= 0)
            a.out_row_weight[myrow] = a.topk_w[(int64_t)t * a.K + lane];

        const int it0 = c * pl.iters_per_item;
        const int n = min(pl.iters_per_item, pl.n_iters - it0);
        const uint16_t *src = a.x + (int64_t)t * a.H;

        // load the item's columns: 16 bf16 (two 16-byte vectors) per lane per iteration
        uint4 lo[kDispatchFp8MaxIters], hi[kDispatchFp8MaxIters];
#pragma unroll
        for (int i = 0; i < kDispatchFp8MaxIters; ++i) {
            const int col = (it0 + i) * kDispatchFp8Width + lane * 16;
            if (i < n && col < a.H) {
                lo[i] = *reinterpret_cast<const uint4 *>(src + col);
                hi[i] = *reinterpret_cast<const uint4 *>(src + col + 8);
            }
        }

#pragma unroll
        for (int i = 0; i < kDispatchFp8MaxIters; ++i) {
            if (i >= n)
                break;
            const int col = (it0 + i) * kDispatchFp8Width + lane * 16;
            const bool active = col < a.H;  // whole 8-lane blocks are active together
            float v[16];
            const uint32_t w[8] = {lo[i].x, lo[i].y, lo[i].z, lo[i].w,
                                   hi[i].x, hi[i].y, hi[i].z, hi[i].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[2 * j] = active ? bf16_lo(w[j]) : 0.0f;
                v[2 * j + 1] = active ? bf16_hi(w[j]) : 0.0f;
            }
            float amax = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                amax = fmaxf(amax, fabsf(v[j]));
            amax = max8(amax);
            const float af = fmaxf(amax, 1e-10f);

            uint4 q;
            float scale_f32 = 0.0f;
            uint32_t scale_byte = 0;
            if (QUANT == MOE_QUANT_FP8_UE8M0) {
                // smallest k with af <= 448 * 2^k, from the binary32 fields of af
                // (af >= 1e-10 is normal): af = m * 2^e, 448 = 1.75 * 2^8.
                const uint32_t ab = __float_as_uint(af);
                const int e = (int)(ab >> 23) - 127;
                const int k = e - 8 + ((ab & 0x7FFFFFu) > 0x600000u ? 1 : 0);
                const float inv = __uint_as_float((uint32_t)(127 - k) << 23);  // 2^-k
                scale_byte = (uint32_t)(k + 127);
                q.x = pack_e4m3(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
                q.y = pack_e4m3(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
                q.z = pack_e4m3(v[8] * inv, v[9] * inv, v[10] * inv, v[11] * inv);
                q.w = pack_e4m3(v[12] * inv, v[13] * inv, v[14] * inv, v[15] * inv);
            } else {
                const float s = af / 448.0f;  // correctly rounded binary32 division
                scale_f32 = s;
                float d[16];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    d[j] = fminf(fmaxf(v[j] / s, -448.0f), 448.0f);
                q.x = pack_e4m3(d[0], d[1], d[2], d[3]);
                q.y = pack_e4m3(d[4], d[5], d[6], d[7]);
                q.z = pack_e4m3(d[8], d[9], d[10], d[11]);
                q.w = pack_e4m3(d[12], d[13], d[14], d[15]);
            }

            // packed UE8M0 word: blocks 4w..4w+3 come from lanes 0,8,16,24 of a
            // 32-lane half; unused blocks contribute 0
            const int blk = col / kQuantGroup;
            uint32_t word = 0;
            if (QUANT == MOE_QUANT_FP8_UE8M0) {
                word = active && (lane & 7) == 0 ? scale_byte << (8 * (blk & 3)) : 0u;
                word |= __shfl_xor(word, 8);
                word |= __shfl_xor(word, 16);
            }

            uint64_t m = kept;
            while (m) {
                const int k = __builtin_ctzll(m);
                m &= m - 1;
                const int32_t row = __builtin_amdgcn_readlane(myrow, k);
                uint8_t *dst = reinterpret_cast<uint8_t *>(a.out_x) + (int64_t)row * a.H;
                if (active)
                    store_stream(dst + col, q);
                if (QUANT == MOE_QUANT_FP8_UE8M0) {
                    if (active && (lane & 31) == 0)
                        reinterpret_cast<uint32_t *>(a.out_scale)[(int64_t)row * NW + (blk >> 2)] = word;
                } else {
                    if (active && (lane & 7) == 0)
                        reinterpret_cast<float *>(a.out_scale)[(int64_t)row * NB + blk] = scale_f32;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs &a, int32_t quant, hipStream_t stream)
{
    const dim3 grid(a.plan.grid), block(kBlockThreads);
    switch (quant) {
    case MOE_QUANT_NONE:
        hipLaunchKernelGGL(dispatch_bf16, grid, block, 0, stream, a);
        break;
    case MOE_QUANT_FP8_F32:
        hipLaunchKernelGGL(dispatch_fp8<MOE_QUANT_FP8_F32>, grid, block, 0, stream, a);
        break;
    default:
        hipLaunchKernelGGL(dispatch_fp8<MOE_QUANT_FP8_UE8M0>, grid, block, 0, stream, a);
        break;
    }
    return hipGetLastError();
}

}  // namespace moe
