// Device building blocks shared by the kernels of libmoe_dispatch.so: lane
// helpers, the steps of the dispatch layout, and loading / quantizing /
// storing token rows.  Not part of the public ABI.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace dev {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Lane helpers
// ---------------------------------------------------------------------------

// Number of set bits of m below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

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

// Inclusive prefix sum over the 64 lanes of a wave without LDS: Hillis-Steele
// shifts of 1, 2, 4, 8 inside each row of 16 lanes (row_shr; lanes with no
// source add 0), then the row totals carried across rows (row_bcast:15 into
// rows 1 and 3, row_bcast:31 into rows 2 and 3).
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Sum of red[w] over the waves w before `wave` (red holds N entries); the
// reads are independent, so they are all in flight at once.
template <int N>
__device__ __forceinline__ int32_t sum_before(const int32_t *red, int wave)
{
    int32_t s = 0;
#pragma unroll
    for (int w = 0; w < N; ++w)
        s += w < wave ? red[w] : 0;
    return s;
}

// ---------------------------------------------------------------------------
// Layout steps (a block of NT threads, NT = 0: blockDim.x; a.nblocks blocks).
// A compile-time NT keeps the block size out of memory: reading blockDim.x
// costs a load from the dispatch packet that the first loads wait behind.
// ---------------------------------------------------------------------------

template <int NT>
__device__ __forceinline__ int block_threads()
{
    return NT > 0 ? NT : (int)blockDim.x;
}

// off[0..E] = segment starts: exclusive scan of align-padded totals
// (contiguous) or e * capacity (masked).  Block-wide; ends with a barrier.
// `red` holds kMaxBlockWaves words.
template <int NT>
__device__ inline void segment_offsets(const LayoutArgs &a, const int32_t *tot, int32_t *off, int32_t *red)
{
    const int E = a.E, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nt = block_threads<NT>();
    if (a.layout == MOE_LAYOUT_CONTIGUOUS) {
        const int per = (E + nt - 1) / nt;
        const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
        int32_t local = 0;
        for (int e = e0; e < e1; ++e)
            local += (tot[e] + a.align - 1) / a.align * a.align;
        const int32_t incl = wave_inclusive_sum(local);
        if (lane == kWave - 1)
            red[wave] = incl;
        __syncthreads();
        int32_t run = sum_before<kMaxBlockWaves>(red, wave) + incl - local;
        for (int e = e0; e < e1; ++e) {
            off[e] = run;
            run += (tot[e] + a.align - 1) / a.align * a.align;
        }
        if (tid == nt - 1)
            off[E] = run;
    } else {
        for (int e = tid; e <= E; e += nt)
            off[e] = e * a.capacity;
    }
    __syncthreads();
}

// Row of a routed pair of expert e whose slot among e's pairs is s, or -1
// when the masked capacity drops it.
__device__ __forceinline__ int32_t row_of(const LayoutArgs &a, const int32_t *off, int32_t e, int32_t s)
{
    if (a.layout == MOE_LAYOUT_CONTIGUOUS)
        return off[e] + s;
    return s < a.capacity ? e * a.capacity + s : -1;
}

// row_to_pair = -1 for rows that hold no pair: the padding after each
// expert's rows (one expert per wave over the grid) and a slice of the tail
// past the last segment per wave.
template <int NT>
__device__ inline void fill_unused_rows(const LayoutArgs &a, const int32_t *tot, const int32_t *off)
{
    const int lane = threadIdx.x & (kWave - 1), nwaves = block_threads<NT>() / kWave;
    const int gwave = blockIdx.x * nwaves + (int)(threadIdx.x / kWave);
    const int gwaves = a.nblocks * nwaves;
    const bool contiguous = a.layout == MOE_LAYOUT_CONTIGUOUS;
    for (int e = gwave; e < a.E; e += gwaves) {
        const int32_t used = contiguous ? tot[e] : min(tot[e], a.capacity);
        for (int32_t r = off[e] + used + lane; r < off[e + 1]; r += kWave)
            a.h.row_to_pair[r] = -1;
    }
    const int64_t tail0 = off[a.E];
    const int64_t span = (a.rows_cap - tail0 + gwaves - 1) / gwaves;
    const int64_t r0 = tail0 + (int64_t)gwave * span;
    const int64_t r1 = min((int64_t)a.rows_cap, r0 + span);
    for (int64_t r = r0 + lane; r < r1; r += kWave)
        a.h.row_to_pair[r] = -1;
}

// Counts and offsets of this block's slice of the experts (every block has
// all of them in LDS); block 0 also writes the rank offsets, expert_offset[E]
// and the status.  `overflow` (pairs dropped by the masked capacity) and
// `invalid` (ids outside [-1, E)) are read in thread 0 of block 0 only.
template <int NT>
__device__ inline void publish(const LayoutArgs &a, const int32_t *tot, const int32_t *off, int32_t overflow,
                               int32_t invalid)
{
    const int E = a.E, tid = threadIdx.x, nt = block_threads<NT>();
    const bool contiguous = a.layout == MOE_LAYOUT_CONTIGUOUS;
    const int per = (E + a.nblocks - 1) / a.nblocks;
    const int e0 = min(E, (int)blockIdx.x * per), e1 = min(E, e0 + per);
    for (int e = e0 + tid; e < e1; e += nt) {
        a.h.expert_count[e] = tot[e];
        a.h.recv_count[e] = contiguous ? tot[e] : min(tot[e], a.capacity);
        a.h.expert_offset[e] = off[e];
    }
    if (blockIdx.x != 0)
        return;
    for (int r = tid; r <= a.R; r += nt)
        a.h.rank_offset[r] = off[r * a.L];
    if (tid == 0) {
        a.h.expert_offset[E] = off[E];
        a.h.status[0] = overflow;
        a.h.status[1] = invalid;
    }
}

// Adds the pairs that the masked capacity drops from this thread's experts
// (tot[e] > capacity, rare) into *over with LDS atomics; a later barrier
// orders them before *over is read.
template <int NT>
__device__ __forceinline__ void count_overflow(const LayoutArgs &a, const int32_t *tot, int32_t *over)
{
    if (a.layout == MOE_LAYOUT_CONTIGUOUS)
        return;
    for (int e = threadIdx.x; e < a.E; e += block_threads<NT>())
        if (tot[e] > a.capacity)
            atomicAdd(over, tot[e] - a.capacity);
}

// LDS int32 words the one-launch layout needs.
__host__ __device__ inline size_t single_layout_lds_words(int32_t E, int waves)
{
    return (size_t)2 * E /* pre, post */ + E /* tot */ + (E + 1) /* off */ + (size_t)waves * E /* cnt */ +
           2 /* invalid, overflow */;
}

// The whole layout for one block of kSingleThreads threads that needs nothing
// from other blocks: the block owns pairs [blk*chunk, blk*chunk + chunk)
// (chunk <= 64 * waves, one run of 64 pairs per wave).  It histograms ALL
// pairs itself (32-bit LDS atomics, into `pre` for pairs before the block and
// `post` for the rest), ranks its own pairs with a ballot match per run and
// the counts of earlier waves, derives the segment offsets, writes both maps
// for its pairs, fills its share of unused rows, and publishes its slice of
// the counts and offsets (block 0 also the rank offsets and status).  Invalid ids and dropped pairs
// are rare: lanes that have some add them into LDS counters with atomics.
// `red` holds kMaxBlockWaves words.  When rows_out is given, rows_out[i]
// receives the row of the block's pair i.  With finish = false steps 5 and 6
// are left to single_layout_finish, which the caller runs later (nothing in
// the block reads what they write).
__device__ inline void single_layout_block(const LayoutArgs &a, int32_t *lds, int32_t *red, int32_t *rows_out,
                                           bool finish = true)
{
    constexpr int NT = kSingleThreads;
    const int E = a.E;
    // LDS layout (single_layout_finish derives the same offsets)
    int32_t *pre = lds;          // [E] pairs before the block, then slot bases
    int32_t *post = pre + E;     // [E] pairs from the block on
    int32_t *tot = post + E;     // [E]
    int32_t *off = tot + E;      // [E+1]
    int32_t *cnt = off + E + 1;  // [waves][E] per-wave counts, then per-wave slot bases
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    constexpr int nwaves = NT / kWave;
    int32_t *misc = cnt + nwaves * E;  // [0] invalid ids, [1] dropped pairs
    const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
    const int64_t c1 = min(a.P, c0 + a.chunk);

    // own pair (one run of 64 per wave), in flight while LDS is cleared
    const int64_t p = c0 + (int64_t)wave * kWave + lane;
    const bool own = p < c1;
    const int32_t e_own = own ? a.topk_idx[p] : -1;
    for (int i = tid; i < 2 * E; i += NT)
        pre[i] = 0;  // pre and post
    for (int i = tid; i < nwaves * E; i += NT)
        cnt[i] = 0;
    if (tid < 2)
        misc[tid] = 0;
    __syncthreads();

    // 1. histogram of every pair: whole batches of kHistBatch 16-byte loads
    //    per thread (no bounds tests) are in flight before their atomics;
    //    small batches only take the one-load loop after them
    int32_t invalid = 0;
    const auto count = [&](int32_t e, int64_t q) {
        if (e >= 0 && e < E)
            atomicAdd((q < c0 ? pre : post) + e, 1);
        else if (e != -1)
            ++invalid;
    };
    const auto count4 = [&](const int4 &v, int64_t q) {
        count(v.x, q);
        count(v.y, q + 1);
        count(v.z, q + 2);
        count(v.w, q + 3);
    };
    const bool vec_ok = ((uintptr_t)a.topk_idx & 15) == 0;  // 16-byte loads need 16-byte alignment
    const int64_t nvec = vec_ok ? a.P / 4 : 0;
    const int4 *v4 = reinterpret_cast<const int4 *>(a.topk_idx);
    int64_t i = tid;
    for (; i + (int64_t)(kHistBatch - 1) * NT < nvec; i += (int64_t)kHistBatch * NT) {
        int4 v[kHistBatch];
#pragma unroll
        for (int j = 0; j < kHistBatch; ++j)
            v[j] = v4[i + (int64_t)j * NT];
#pragma unroll
        for (int j = 0; j < kHistBatch; ++j)
            count4(v[j], 4 * (i + (int64_t)j * NT));
    }
    for (; i < nvec; i += NT)
        count4(v4[i], 4 * i);
    for (int64_t q = 4 * nvec + tid; q < a.P; q += NT)
        count(a.topk_idx[q], q);
    if (invalid != 0)
        atomicAdd(&misc[0], invalid);

    // 2. rank of the own pair among equal experts in its run
    const bool routed = e_own >= 0 && e_own < E;
    const uint64_t m = match_expert(e_own, routed, a.nbits);
    const int below = lanes_below(m);
    if (routed && below == 0)
        cnt[wave * E + e_own] = __popcll(m);
    __syncthreads();

    // 3. totals; per-wave slot bases start at the pairs of earlier blocks
    //    (all of an expert's wave counts are read before any is rewritten)
    for (int e = tid; e < E; e += NT) {
        const int32_t before = pre[e];
        tot[e] = before + post[e];
        int32_t c[kMaxBlockWaves];
#pragma unroll
        for (int w = 0; w < kMaxBlockWaves; ++w)
            c[w] = 0;
#pragma unroll
        for (int w = 0; w < kMaxBlockWaves; ++w)
            if (w < nwaves)
                c[w] = cnt[w * E + e];
        int32_t s = before;
#pragma unroll
        for (int w = 0; w < kMaxBlockWaves; ++w)
            if (w < nwaves) {
                cnt[w * E + e] = s;
                s += c[w];
            }
    }
    __syncthreads();
    count_overflow<NT>(a, tot, &misc[1]);  // read after the barriers of step 4

    // 4. segment offsets, then the own pair's row and both maps
    segment_offsets<NT>(a, tot, off, red);
    if (own) {
        const int32_t row = routed ? row_of(a, off, e_own, cnt[wave * E + e_own] + below) : -1;
        a.h.pair_to_row[p] = row;
        if (row >= 0)
            a.h.row_to_pair[row] = (int32_t)p;
        if (rows_out != nullptr)
            rows_out[p - c0] = row;
    }

    // 5. rows that hold no pair; 6. counts and offsets, a slice per block
    if (finish) {
        fill_unused_rows<NT>(a, tot, off);
        publish<NT>(a, tot, off, misc[1], misc[0]);
    }
}

// Steps 5 and 6 of single_layout_block(..., finish = false), from the totals,
// offsets and rare counts it left in LDS.
__device__ inline void single_layout_finish(const LayoutArgs &a, const int32_t *lds)
{
    constexpr int nwaves = kSingleThreads / kWave;
    const int32_t *tot = lds + 2 * a.E;
    const int32_t *off = tot + a.E;
    const int32_t *misc = off + a.E + 1 + nwaves * a.E;
    fill_unused_rows<kSingleThreads>(a, tot, off);
    publish<kSingleThreads>(a, tot, off, misc[1], misc[0]);
}

// ---------------------------------------------------------------------------
// Token rows: prefetch into the Infinity Cache
// ---------------------------------------------------------------------------

// Reads one dword of every kPrefetchSegment bytes of the token rows x [T, H]
// in token order, so that the rows sit in the Infinity Cache -- the
// memory-side cache every XCD reads HBM through -- when the row kernel that
// follows loads them; the loaded values are discarded.  Run by `pf_blocks`
// whole blocks of kSingleThreads threads; `pf_block` is this block's index
// among them.  With the rows evicted, their HBM reads then happen while the
// layout runs, instead of behind the row stores; with them cached, this is a
// pass over them at cache bandwidth.
__device__ inline void prefetch_rows(const uint16_t *x, int32_t T, int32_t H, int32_t pf_block, int32_t pf_blocks)
{
    constexpr int kWaves = kSingleThreads / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int32_t row_bytes = 2 * H;
    const int32_t segs = (row_bytes + kPrefetchSegment - 1) / kPrefetchSegment;
    const int32_t loads_per_row = (segs + kWave - 1) / kWave;
    const int32_t units = T * loads_per_row;  // (token, load of 64 segments), token-major
    const int32_t nw = pf_blocks * kWaves;
    const char *base = reinterpret_cast<const char *>(x);
    for (int32_t u0 = pf_block * kWaves + wave; u0 < units; u0 += nw * kPrefetchBatch) {
        uint32_t v[kPrefetchBatch];
#pragma unroll
        for (int i = 0; i < kPrefetchBatch; ++i) {
            v[i] = 0;
            const int32_t u = u0 + i * nw;
            if (u < units) {
                const int32_t t = u / loads_per_row;
                const int32_t seg = (u - t * loads_per_row) * kWave + lane;
                // seg * 64 < row_bytes and both are multiples of 16: the dword is in the row
                if (seg < segs)
                    v[i] = *reinterpret_cast<const uint32_t *>(base + (int64_t)t * row_bytes +
                                                               (int64_t)seg * kPrefetchSegment);
            }
        }
        // the values are only consumed here, so the batch's loads are all in
        // flight before the one wait for them
#pragma unroll
        for (int i = 0; i < kPrefetchBatch; ++i)
            asm volatile("" ::"v"(v[i]));
    }
}

// ---------------------------------------------------------------------------
// Token rows: load, quantize, store
// ---------------------------------------------------------------------------

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

// Dispatched rows are written once and read by a later kernel (the experts):
// non-temporal stores keep them from filling L2 and the MALL with dirty lines
// that the following kernels would have to evict (measured on the DeepSeek-V3
// prefill shape: dispatch 129 -> 98 us, and the next combine 216 -> 195 us; a
// streaming kernel with dispatch's traffic, back to back: 116.5 us with plain
// stores, 85 us non-temporal).  Adding the device coherence-scope bit to
// these stores changes nothing measurable.
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

// Registers holding the columns of one work item (a run of iterations of one
// token row): bf16 rows move 8 channels (one 16-byte vector) per lane per
// iteration, FP8 rows 16 channels (two vectors: 8 lanes cover one 128-channel
// quantization block).
template <int QUANT>
struct RowRegs {
    static constexpr int kWidth = kDispatchFp8Width;
    static constexpr int kMaxIters = kDispatchFp8MaxIters;
    uint4 lo[kMaxIters], hi[kMaxIters];
};
template <>
struct RowRegs<MOE_QUANT_NONE> {
    static constexpr int kWidth = kDispatchBf16Width;
    static constexpr int kMaxIters = kDispatchBf16MaxIters;
    uint4 v[kMaxIters];
};

// Issue the loads of iterations [it0, it0 + n) of row `src`.
template <int QUANT>
__device__ __forceinline__ void load_item(RowRegs<QUANT> &r, const uint16_t *src, int it0, int n, int H, int lane)
{
    using R = RowRegs<QUANT>;
#pragma unroll
    for (int i = 0; i < R::kMaxIters; ++i) {
        if constexpr (QUANT == MOE_QUANT_NONE) {
            const int col = (it0 + i) * R::kWidth + lane * 8;
            if (i < n && col < H)
                r.v[i] = *reinterpret_cast<const uint4 *>(src + col);
        } else {
            const int col = (it0 + i) * R::kWidth + lane * 16;
            if (i < n && col < H) {
                r.lo[i] = *reinterpret_cast<const uint4 *>(src + col);
                r.hi[i] = *reinterpret_cast<const uint4 *>(src + col + 8);
            }
        }
    }
}

// Store iterations [it0, it0 + n) of a token row held in r to every kept row
// of the token (kept = mask of lanes k whose `myrow` is >= 0), quantizing first
// when QUANT asks for it.  Per 128-channel block b: a = max(|x|, 1e-10);
//   fp32 scales: s = a / 448, q = E4M3(clamp(x / s, +-448))
//   UE8M0:       k = smallest integer with a <= 448 * 2^k, q = E4M3(x * 2^-k),
//                scale byte k + 127, four blocks per little-endian word.
// MXFP8 uses 32-channel blocks (OCP MX conversion): a as above, s = floor(log2 a)
//   - 8, q = E4M3(clamp(x * 2^-s, +-448)), E8M0 byte s + 127, bytes in block order.
template <int QUANT>
__device__ __forceinline__ void store_item(const RowRegs<QUANT> &r, const DispatchArgs &a, int it0, int n,
                                           int lane, uint64_t kept, int32_t myrow)
{
    using R = RowRegs<QUANT>;
    if constexpr (QUANT == MOE_QUANT_NONE) {
#pragma unroll
        for (int i = 0; i < R::kMaxIters; ++i) {
            const int col = (it0 + i) * R::kWidth + lane * 8;
            if (i < n) {
                const uint4 d = r.v[i];
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
    } else {
        const int NB = a.H / kQuantGroup;
        const int NW = (NB + 3) / 4;
#pragma unroll
        for (int i = 0; i < R::kMaxIters; ++i) {
            if (i >= n)
                break;
            const int col = (it0 + i) * R::kWidth + lane * 16;
            const bool active = col < a.H;  // whole 8-lane blocks are active together
            float v[16];
            const uint32_t w[8] = {r.lo[i].x, r.lo[i].y, r.lo[i].z, r.lo[i].w,
                                   r.hi[i].x, r.hi[i].y, r.hi[i].z, r.hi[i].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[2 * j] = active ? bf16_lo(w[j]) : 0.0f;
                v[2 * j + 1] = active ? bf16_hi(w[j]) : 0.0f;
            }
            float amax = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                amax = fmaxf(amax, fabsf(v[j]));
            // block maximum: 8 lanes for 128-channel blocks, 2 for MX blocks
            amax = QUANT == MOE_QUANT_MXFP8 ? fmaxf(amax, dpp<0xB1>(amax)) : max8(amax);
            const float af = fmaxf(amax, 1e-10f);

            uint4 q;
            float scale_f32 = 0.0f;
            uint32_t scale_byte = 0;
            if constexpr (QUANT == MOE_QUANT_MXFP8) {
                // floor(log2 af) - 8 is the exponent field of af (normal) minus 127 + 8
                const int sx = (int)(__float_as_uint(af) >> 23) - 135;
                const float inv = __uint_as_float((uint32_t)(127 - sx) << 23);  // 2^-s, exact
                scale_byte = (uint32_t)(sx + 127);
                float d[16];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    d[j] = fminf(fmaxf(v[j] * inv, -448.0f), 448.0f);
                q.x = pack_e4m3(d[0], d[1], d[2], d[3]);
                q.y = pack_e4m3(d[4], d[5], d[6], d[7]);
                q.z = pack_e4m3(d[8], d[9], d[10], d[11]);
                q.w = pack_e4m3(d[12], d[13], d[14], d[15]);
            } else if constexpr (QUANT == MOE_QUANT_FP8_UE8M0) {
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
            } else if (QUANT == MOE_QUANT_MXFP8) {
                // the 4 MX blocks of a 128-channel group (even lanes 8j..8j+6)
                // form word `blk` of the row's scale bytes
                word = active && (lane & 1) == 0 ? scale_byte << (8 * ((lane >> 1) & 3)) : 0u;
                word |= __shfl_xor(word, 2);
                word |= __shfl_xor(word, 4);
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
                } else if (QUANT == MOE_QUANT_MXFP8) {
                    if (active && (lane & 7) == 0)
                        reinterpret_cast<uint32_t *>(a.out_scale)[(int64_t)row * NB + blk] = word;
                } else {
                    if (active && (lane & 7) == 0)
                        reinterpret_cast<float *>(a.out_scale)[(int64_t)row * NB + blk] = scale_f32;
                }
            }
        }
    }
}

}  // namespace dev
}  // namespace moe
