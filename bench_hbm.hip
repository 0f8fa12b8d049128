// HBM ceilings of the traffic mixes of dispatch and combine on one MI355X:
// plain streaming kernels with the same read:write ratios and store policy
// as the library's row kernels, but contiguous addresses and no other work.
// Each case runs with the caches as a back-to-back repetition leaves them
// ("warm") and after an untimed 512 MiB read of a scratch buffer ("cold").
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       -o /tmp/bench_hbm bench_hbm.hip && /tmp/bench_hbm
//
// Prints one line per case: median of 15 event-timed launches, GB/s of the
// bytes the kernel moves.  Sizes follow the DeepSeek-V3 prefill batch: 117 MB
// of token rows read, 4 x that written (dispatch, E4M3 rows of 8 pairs per
// token: 470 MB); 8 x that read and 117 MB written (combine); 2 x that read
// and 4 x written (the per-rank expansion: about 4 ranks per token).
//
// The last section repeats the two mixes with buffer loads and stores whose
// cache-policy bits (sc0 = 1, nt = 2, sc1 = 16 in the instruction's policy
// operand) are set explicitly, one combination per case.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdio.h>
#include <stdlib.h>
#include <vector>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

constexpr int kThreads = 256;

// n16 16-byte vectors written, plain or non-temporal stores
template <bool NT>
__global__ __launch_bounds__(kThreads) void write_stream(u32x4 *dst, long n16)
{
    const long stride = (long)gridDim.x * kThreads;
    const u32x4 v = {1u, 2u, 3u, 4u};
    for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
        if (NT)
            __builtin_nontemporal_store(v, dst + i);
        else
            dst[i] = v;
    }
}

// n16 16-byte vectors read (four in flight per thread); one vector per
// thread is written to `sink` so that the loads are kept
template <bool NT>
__global__ __launch_bounds__(kThreads) void read_stream(const u32x4 *src, long n16, u32x4 *sink)
{
    const long stride = (long)gridDim.x * kThreads;
    long i = (long)blockIdx.x * kThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        u32x4 a, b, c, d;
        if (NT) {
            a = __builtin_nontemporal_load(src + i);
            b = __builtin_nontemporal_load(src + i + stride);
            c = __builtin_nontemporal_load(src + i + 2 * stride);
            d = __builtin_nontemporal_load(src + i + 3 * stride);
        } else {
            a = src[i];
            b = src[i + stride];
            c = src[i + 2 * stride];
            d = src[i + 3 * stride];
        }
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride)
        acc ^= src[i];
    sink[(long)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// dispatch's mix: each 16-byte vector of src (plain loads) is stored to F
// regions of dst (region f = dst + f * n16) with non-temporal stores
template <int F>
__global__ __launch_bounds__(kThreads) void fan_out(const u32x4 *src, long n16, u32x4 *dst)
{
    const long stride = (long)gridDim.x * kThreads;
    long i = (long)blockIdx.x * kThreads + threadIdx.x;
    for (; i + stride < n16; i += 2 * stride) {
        const u32x4 a = src[i], b = src[i + stride];
#pragma unroll
        for (int f = 0; f < F; ++f) {
            __builtin_nontemporal_store(a, dst + (long)f * n16 + i);
            __builtin_nontemporal_store(b, dst + (long)f * n16 + i + stride);
        }
    }
    for (; i < n16; i += stride) {
        const u32x4 a = src[i];
#pragma unroll
        for (int f = 0; f < F; ++f)
            __builtin_nontemporal_store(a, dst + (long)f * n16 + i);
    }
}

// the per-rank expansion's mix: S source regions (src + s * n16, read with
// non-temporal loads), each stored to D / S destination regions (dst + d *
// n16) with non-temporal stores
template <int S, int D>
__global__ __launch_bounds__(kThreads) void fan_out_sources(const u32x4 *src, long n16, u32x4 *dst)
{
    const long stride = (long)gridDim.x * kThreads;
    for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
        u32x4 v[S];
#pragma unroll
        for (int k = 0; k < S; ++k)
            v[k] = __builtin_nontemporal_load(src + (long)k * n16 + i);
#pragma unroll
        for (int d = 0; d < D; ++d)
            __builtin_nontemporal_store(v[d % S], dst + (long)d * n16 + i);
    }
}

// combine's mix: F regions of src (region f = src + f * n16) read with
// non-temporal loads, their xor stored once to dst with plain stores
template <int F>
__global__ __launch_bounds__(kThreads) void fan_in(const u32x4 *src, long n16, u32x4 *dst)
{
    const long stride = (long)gridDim.x * kThreads;
    for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
        u32x4 v[F];
#pragma unroll
        for (int f = 0; f < F; ++f)
            v[f] = __builtin_nontemporal_load(src + (long)f * n16 + i);
        u32x4 acc = v[0];
#pragma unroll
        for (int f = 1; f < F; ++f)
            acc ^= v[f];
        dst[i] = acc;
    }
}

// Word 3 of a raw buffer resource: 32-bit data format, no swizzle or index.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t resource(const void *p, long bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, kRawBufferWord3);
}

// dispatch's mix with explicit policies: x read with LOAD, 4 regions written with STORE
template <int LOAD, int STORE>
__global__ __launch_bounds__(kThreads) void fan_out_policy(const u32x4 *src, long n16, u32x4 *dst)
{
    const __amdgpu_buffer_rsrc_t rs = resource(src, n16 * 16);
    __amdgpu_buffer_rsrc_t rd[4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
        rd[f] = resource(dst + (long)f * n16, n16 * 16);
    const long stride = (long)gridDim.x * kThreads;
    for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(i * 16), 0, LOAD);
#pragma unroll
        for (int f = 0; f < 4; ++f)
            __builtin_amdgcn_raw_buffer_store_b128(a, rd[f], (int)(i * 16), 0, STORE);
    }
}

// combine's mix with explicit policies: 8 regions read with LOAD, their xor written with STORE
template <int LOAD, int STORE>
__global__ __launch_bounds__(kThreads) void fan_in_policy(const u32x4 *src, long n16, u32x4 *dst)
{
    __amdgpu_buffer_rsrc_t rs[8];
#pragma unroll
    for (int f = 0; f < 8; ++f)
        rs[f] = resource(src + (long)f * n16, n16 * 16);
    const __amdgpu_buffer_rsrc_t rd = resource(dst, n16 * 16);
    const long stride = (long)gridDim.x * kThreads;
    for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
        u32x4 v[8];
#pragma unroll
        for (int f = 0; f < 8; ++f)
            v[f] = __builtin_amdgcn_raw_buffer_load_b128(rs[f], (int)(i * 16), 0, LOAD);
        u32x4 acc = v[0];
#pragma unroll
        for (int f = 1; f < 8; ++f)
            acc ^= v[f];
        __builtin_amdgcn_raw_buffer_store_b128(acc, rd, (int)(i * 16), 0, STORE);
    }
}

int main()
{
    const long xb = 117440512L;  // token rows of the DeepSeek-V3 prefill batch: 8192 x 7168 bf16
    const long n16 = xb / 16;
    const long flush_bytes = 512L << 20;
    const int max_grid = 4096;
    u32x4 *x, *big, *sink, *flush;
    CHECK(hipMalloc(&x, xb));
    CHECK(hipMalloc(&big, 8 * xb));  // dispatched rows, or the expert outputs combine reads
    CHECK(hipMalloc(&sink, (size_t)max_grid * kThreads * 16));
    CHECK(hipMalloc(&flush, flush_bytes));
    CHECK(hipMemset(x, 1, xb));
    CHECK(hipMemset(big, 2, 8 * xb));
    CHECK(hipMemset(flush, 0, flush_bytes));
    CHECK(hipDeviceSynchronize());
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const auto do_flush = [&]() {
        hipLaunchKernelGGL(read_stream<false>, dim3(2048), dim3(kThreads), 0, 0, (const u32x4 *)flush,
                           flush_bytes / 16, sink);
    };
    const auto run = [&](const char *name, long bytes, auto launch) {
        for (int cold = 0; cold < 2; ++cold) {
            std::vector<float> t;
            launch();  // one untimed launch first
            for (int r = 0; r < 15; ++r) {
                if (cold)
                    do_flush();
                CHECK(hipEventRecord(e0, 0));
                launch();
                CHECK(hipEventRecord(e1, 0));
                CHECK(hipEventSynchronize(e1));
                float ms;
                CHECK(hipEventElapsedTime(&ms, e0, e1));
                t.push_back(ms);
            }
            CHECK(hipGetLastError());
            std::sort(t.begin(), t.end());
            const float m = t[t.size() / 2];
            printf("%-48s %-4s %8.1f us %7.0f GB/s\n", name, cold ? "cold" : "warm", m * 1e3, bytes / (m * 1e-3) / 1e9);
            fflush(stdout);
        }
    };
    for (int grid : {1024, 2048, 4096}) {
        printf("grid %d blocks of %d threads\n", grid, kThreads);
        run("write 470 MB, non-temporal", 4 * xb,
            [&] { hipLaunchKernelGGL(write_stream<true>, dim3(grid), dim3(kThreads), 0, 0, big, 4 * n16); });
        run("write 470 MB, plain", 4 * xb,
            [&] { hipLaunchKernelGGL(write_stream<false>, dim3(grid), dim3(kThreads), 0, 0, big, 4 * n16); });
        run("read 470 MB, plain", 4 * xb, [&] {
            hipLaunchKernelGGL(read_stream<false>, dim3(grid), dim3(kThreads), 0, 0, (const u32x4 *)big, 4 * n16, sink);
        });
        run("read 470 MB, non-temporal", 4 * xb, [&] {
            hipLaunchKernelGGL(read_stream<true>, dim3(grid), dim3(kThreads), 0, 0, (const u32x4 *)big, 4 * n16, sink);
        });
        run("dispatch mix: read 117 MB, write 4 x (470 MB)", 5 * xb,
            [&] { hipLaunchKernelGGL(fan_out<4>, dim3(grid), dim3(kThreads), 0, 0, x, n16, big); });
        run("combine mix: read 8 x (940 MB), write 117 MB", 9 * xb,
            [&] { hipLaunchKernelGGL(fan_in<8>, dim3(grid), dim3(kThreads), 0, 0, big, n16, x); });
        // sources in regions 4-5 of big, destinations in regions 0-3
        run("expansion mix: read 235 MB, write 2 x (470 MB)", 6 * xb, [&] {
            hipLaunchKernelGGL((fan_out_sources<2, 4>), dim3(grid), dim3(kThreads), 0, 0, big + 4 * n16, n16, big);
        });
    }
    // cache policies (buffer instructions, grid 2048); every region is 117 MB < 2^31 bytes
    printf("cache policies: load bits / store bits (sc0 = 1, nt = 2, sc1 = 16), grid 2048\n");
    const int grid = 2048;
#define FAN_OUT(L, S)                                                                                   \
    run("dispatch mix, load " #L ", store " #S, 5 * xb,                                               \
        [&] { hipLaunchKernelGGL((fan_out_policy<L, S>), dim3(grid), dim3(kThreads), 0, 0, x, n16, big); })
#define FAN_IN(L, S)                                                                                    \
    run("combine mix, load " #L ", store " #S, 9 * xb,                                                \
        [&] { hipLaunchKernelGGL((fan_in_policy<L, S>), dim3(grid), dim3(kThreads), 0, 0, big, n16, x); })
    FAN_OUT(0, 2);
    FAN_OUT(0, 18);
    FAN_OUT(0, 19);
    FAN_OUT(0, 0);
    FAN_OUT(0, 16);
    FAN_OUT(2, 2);
    FAN_OUT(16, 2);
    FAN_IN(2, 0);
    FAN_IN(2, 2);
    FAN_IN(2, 16);
    FAN_IN(2, 17);
    FAN_IN(2, 18);
    FAN_IN(0, 16);
    FAN_IN(16, 16);
    FAN_IN(18, 16);
    return 0;
}
