// C ABI of libmoe_dispatch.so: host-side validation, launch planning, and
// the extern "C" entry points declared in include/moe_dispatch.h.
//
// Every argument error is found here, before anything is enqueued; the
// library allocates nothing and keeps no state besides a cached compute-unit
// count per device.
#include <limits.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "moe_internal.h"

namespace moe {

// Workspace of moe_dispatch_layout_noalloc: one array per GPU, held until the
// process ends, shared by every call on that GPU (calls that overlap on one
// GPU race).  In host code `scratch` only names the array; its device
// address comes from hipGetSymbolAddress, per device.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Device address of the scratch array on device `dev`, looked up once per
// device with that device current; nullptr if the lookup fails.
void *scratch_address(int dev)
{
    static std::atomic<void *> addr[kMaxDevices];
    static std::mutex mu;
    if (dev < 0 || dev >= kMaxDevices)
        return nullptr;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (p != nullptr)
        return p;
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p != nullptr)
        return p;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess)
        return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess)
        return nullptr;
    void *q = nullptr;
    const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (cur != dev)
        (void)hipSetDevice(cur);
    if (e != hipSuccess || q == nullptr)
        return nullptr;
    addr[dev].store(q, std::memory_order_release);
    return q;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t rows_capacity64(const moe_config_t &c)
{
    if (c.layout == MOE_LAYOUT_CONTIGUOUS)
        return (int64_t)c.max_tokens * c.num_topk + (int64_t)c.num_experts * (c.align - 1);
    return (int64_t)c.num_experts * c.capacity;
}

moe_status_t check_config(const moe_config_t *cfg)
{
    if (cfg == nullptr)
        return MOE_ERR_INVALID_ARG;
    const moe_config_t &c = *cfg;
    if (c.max_tokens < 0 || c.hidden < 8 || c.hidden % 8 != 0)
        return MOE_ERR_INVALID_ARG;
    if (c.num_experts < 1 || c.num_topk < 1 || c.num_topk > kMaxTopk || c.num_ranks < 1)
        return MOE_ERR_INVALID_ARG;
    if (c.num_experts % c.num_ranks != 0)
        return MOE_ERR_INVALID_ARG;
    if (c.layout != MOE_LAYOUT_CONTIGUOUS && c.layout != MOE_LAYOUT_MASKED)
        return MOE_ERR_INVALID_ARG;
    if (c.layout == MOE_LAYOUT_CONTIGUOUS && c.align < 1)
        return MOE_ERR_INVALID_ARG;
    if (c.layout == MOE_LAYOUT_MASKED && c.capacity < 1)
        return MOE_ERR_INVALID_ARG;
    if (c.quant != MOE_QUANT_NONE && c.quant != MOE_QUANT_FP8_F32 && c.quant != MOE_QUANT_FP8_UE8M0 &&
        c.quant != MOE_QUANT_MXFP8)
        return MOE_ERR_INVALID_ARG;
    if (c.quant != MOE_QUANT_NONE && c.hidden % kQuantGroup != 0)
        return MOE_ERR_INVALID_ARG;
    if (c.num_cus < 0)
        return MOE_ERR_INVALID_ARG;
    if (c.num_experts > kMaxExperts)
        return MOE_ERR_UNSUPPORTED;
    if ((int64_t)c.max_tokens * c.num_topk > INT32_MAX || rows_capacity64(c) > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t check_handle(const moe_handle_t *h)
{
    if (h == nullptr)
        return MOE_ERR_INVALID_ARG;
    const int32_t *arr[] = {h->expert_count, h->recv_count, h->expert_offset, h->rank_offset,
                            h->pair_to_row, h->row_to_pair, h->status};
    for (const int32_t *p : arr)
        if (p == nullptr || !aligned(p, 4))
            return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status_t check_rank_handle(const moe_rank_handle_t *h)
{
    if (h == nullptr)
        return MOE_ERR_INVALID_ARG;
    const int32_t *arr[] = {h->rank_token_count, h->rank_token_offset, h->token_rank_row, h->rank_row_to_token};
    for (const int32_t *p : arr)
        if (p == nullptr || !aligned(p, 4))
            return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int32_t scale_words32(const moe_config_t &c)
{
    const int32_t NB = c.hidden / kQuantGroup;
    switch (c.quant) {
    case MOE_QUANT_FP8_F32:
        return NB;
    case MOE_QUANT_FP8_UE8M0:
        return (NB + 3) / 4;
    case MOE_QUANT_MXFP8:
        return NB;  // H/32 E8M0 bytes, four per word
    default:
        return 0;
    }
}

int64_t repack_rows64(const moe_config_t &c, int32_t align)
{
    const int64_t pairs = (int64_t)c.max_tokens * c.num_topk;
    const int64_t slab = (int64_t)c.num_experts * c.capacity;
    return (pairs < slab ? pairs : slab) + (int64_t)c.num_experts * (align - 1);
}

int64_t rank_rows64(const moe_config_t &c)
{
    return (int64_t)c.max_tokens * (c.num_topk < c.num_ranks ? c.num_topk : c.num_ranks);
}

// Config, token count and rank limit shared by the per-rank calls.
moe_status_t check_dedup(const moe_config_t *cfg, int32_t num_tokens, const moe_rank_handle_t *rh)
{
    moe_status_t st = check_config(cfg);
    if (st != MOE_OK)
        return st;
    if (cfg->num_ranks > kMaxDedupRanks)
        return MOE_ERR_UNSUPPORTED;
    if ((st = check_rank_handle(rh)) != MOE_OK)
        return st;
    if (num_tokens < 0)
        return MOE_ERR_INVALID_ARG;
    if (num_tokens > cfg->max_tokens)
        return MOE_ERR_CAPACITY;
    return MOE_OK;
}

moe_status_t check_tokens(const moe_config_t &c, int32_t num_tokens)
{
    if (num_tokens < 0)
        return MOE_ERR_INVALID_ARG;
    if (num_tokens > c.max_tokens)
        return MOE_ERR_CAPACITY;
    return MOE_OK;
}

int bits_for(int32_t E)
{
    int b = 0;
    while ((1 << b) < E)
        ++b;
    return b;
}

moe_status_t from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Validates a layout call and fills its launch arguments.
moe_status_t prepare_layout(const moe_config_t *cfg, int32_t num_tokens, const int32_t *topk_idx,
                            const moe_handle_t *handle, void *workspace, size_t workspace_bytes, LayoutArgs &a,
                            LayoutPlan &lp)
{
    moe_status_t st = check_config(cfg);
    if (st != MOE_OK)
        return st;
    if ((st = check_handle(handle)) != MOE_OK)
        return st;
    if ((st = check_tokens(*cfg, num_tokens)) != MOE_OK)
        return st;
    if ((num_tokens > 0 && (topk_idx == nullptr || !aligned(topk_idx, 4))) || workspace == nullptr ||
        !aligned(workspace, 16))
        return MOE_ERR_INVALID_ARG;
    const int64_t P = (int64_t)num_tokens * cfg->num_topk;
    lp = layout_plan(P, cfg->num_experts);
    const size_t table = layout_table_bytes(cfg->num_experts);
    if (workspace_bytes < table + sizeof(int32_t) * (size_t)P)
        return MOE_ERR_CAPACITY;
    a.topk_idx = topk_idx;
    a.P = P;
    a.E = cfg->num_experts;
    a.R = cfg->num_ranks;
    a.L = cfg->num_experts / cfg->num_ranks;
    a.layout = cfg->layout;
    a.align = cfg->layout == MOE_LAYOUT_CONTIGUOUS ? cfg->align : 1;
    a.capacity = cfg->layout == MOE_LAYOUT_MASKED ? cfg->capacity : 1;
    a.rows_cap = (int32_t)rows_capacity64(*cfg);
    a.nbits = bits_for(cfg->num_experts);
    a.rounds = lp.rounds;
    a.chunk = lp.chunk;
    a.nblocks = lp.nblocks;
    a.ws = static_cast<int32_t *>(workspace);
    a.slots = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + table);
    a.h = *handle;
    return MOE_OK;
}

// Validates a dispatch call and fills its launch arguments (plan included
// when there are tokens).
moe_status_t prepare_dispatch(const moe_config_t *cfg, int32_t num_tokens, const uint16_t *x, const float *topk_w,
                              const moe_handle_t *handle, void *out_x, void *out_scale, float *out_row_weight,
                              DispatchArgs &a)
{
    moe_status_t st = check_config(cfg);
    if (st != MOE_OK)
        return st;
    if ((st = check_handle(handle)) != MOE_OK)
        return st;
    if ((st = check_tokens(*cfg, num_tokens)) != MOE_OK)
        return st;
    const bool fp8 = cfg->quant != MOE_QUANT_NONE;
    if (out_x == nullptr || !aligned(out_x, 16))
        return MOE_ERR_INVALID_ARG;
    if (fp8 ? (out_scale == nullptr || !aligned(out_scale, 4)) : out_scale != nullptr)
        return MOE_ERR_INVALID_ARG;
    if (out_row_weight != nullptr && !aligned(out_row_weight, 4))
        return MOE_ERR_INVALID_ARG;
    if (out_row_weight != nullptr && num_tokens > 0 && (topk_w == nullptr || !aligned(topk_w, 4)))
        return MOE_ERR_INVALID_ARG;
    if (num_tokens > 0 && (x == nullptr || !aligned(x, 16)))
        return MOE_ERR_INVALID_ARG;
    a.x = x;
    a.topk_w = topk_w;
    a.pair_to_row = handle->pair_to_row;
    a.out_x = out_x;
    a.out_scale = out_scale;
    a.out_row_weight = out_row_weight;
    a.T = num_tokens;
    a.K = cfg->num_topk;
    a.H = cfg->hidden;
    if (num_tokens > 0)
        a.plan = fp8 ? row_plan(num_tokens, cfg->hidden, kDispatchFp8Width, kDispatchFp8MaxIters, cfg->num_cus,
                                kDispatchMinItemsPerToken)
                     : row_plan(num_tokens, cfg->hidden, kDispatchBf16Width, kDispatchBf16MaxIters, cfg->num_cus,
                                kDispatchMinItemsPerToken);
    return MOE_OK;
}

}  // namespace

// Compute units of the current device, asked once per device; calls from
// several host threads may race to fill an entry, all with the same value.
int device_cu_count()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Work items: (token, run of iterations).  Each token row has n_iters
// iterations of `width` columns; a wave keeps at most `max_iters` of them in
// flight.  Short batches (decode) split rows further so the launch still has
// several waves per compute unit; num_cus > 0 caps the grid and the waves
// stride over the items.
RowPlan row_plan(int32_t T, int32_t H, int32_t width, int32_t max_iters, int32_t num_cus,
                 int32_t min_items_per_token)
{
    RowPlan p;
    p.width = width;
    p.n_iters = (H + width - 1) / width;
    const int cus = device_cu_count();
    const int64_t target_waves = (int64_t)cus * 8;
    int64_t per_token = (p.n_iters + max_iters - 1) / max_iters;
    if (per_token < min_items_per_token)
        per_token = min_items_per_token < p.n_iters ? min_items_per_token : p.n_iters;
    if ((int64_t)T * per_token < target_waves && T > 0) {
        const int64_t want = (target_waves + T - 1) / T;
        per_token = want < p.n_iters ? want : p.n_iters;
    }
    if (per_token < 1)
        per_token = 1;
    p.iters_per_item = (int32_t)((p.n_iters + per_token - 1) / per_token);
    p.items_per_token = (p.n_iters + p.iters_per_item - 1) / p.iters_per_item;
    p.n_items = (int64_t)T * p.items_per_token;
    int64_t grid = (p.n_items + kWavesPerBlock - 1) / kWavesPerBlock;
    if (num_cus > 0) {
        const int64_t cap = (int64_t)num_cus * 8;  // 8 workgroups (32 waves) per CU
        if (grid > cap)
            grid = cap;
    }
    p.grid = (int32_t)(grid < 1 ? 1 : grid);
    return p;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_rows_capacity(const moe_config_t *cfg)
{
    if (check_config(cfg) != MOE_OK)
        return 0;
    return (size_t)rows_capacity64(*cfg);
}

size_t moe_workspace_bytes(const moe_config_t *cfg)
{
    if (check_config(cfg) != MOE_OK)
        return 0;
    const size_t slots = sizeof(int32_t) * (size_t)cfg->max_tokens * (size_t)cfg->num_topk;
    return layout_table_bytes(cfg->num_experts) + (slots + 255) / 256 * 256;
}

moe_status_t moe_config_check(const moe_config_t *cfg) { return check_config(cfg); }

moe_status_t moe_dispatch_layout(const moe_config_t *cfg, int32_t num_tokens, const int32_t *topk_idx,
                                 const moe_handle_t *handle, void *workspace, size_t workspace_bytes,
                                 void *stream)
{
    LayoutArgs a;
    LayoutPlan lp;
    const moe_status_t st = prepare_layout(cfg, num_tokens, topk_idx, handle, workspace, workspace_bytes, a, lp);
    if (st != MOE_OK)
        return st;
    return from_hip(launch_layout(a, lp, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_dispatch_layout_noalloc(const moe_config_t *cfg, int32_t num_tokens, const int32_t *topk_idx,
                                         const moe_handle_t *handle, void *stream)
{
    // everything that needs no device first: the config, handle and token
    // count, and the size of the workspace this call needs
    moe_status_t st = check_config(cfg);
    if (st != MOE_OK)
        return st;
    if ((st = check_handle(handle)) != MOE_OK)
        return st;
    if ((st = check_tokens(*cfg, num_tokens)) != MOE_OK)
        return st;
    if (num_tokens > 0 && (topk_idx == nullptr || !aligned(topk_idx, 4)))
        return MOE_ERR_INVALID_ARG;
    const size_t need = layout_table_bytes(cfg->num_experts) + sizeof(int32_t) * (size_t)num_tokens * cfg->num_topk;
    if (need > kScratchBytes)
        return MOE_ERR_CAPACITY;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = -1;
    if ((s != nullptr ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess)
        return MOE_ERR_HIP;
    void *ws = scratch_address(dev);
    if (ws == nullptr)
        return MOE_ERR_HIP;
    LayoutArgs a;
    LayoutPlan lp;
    st = prepare_layout(cfg, num_tokens, topk_idx, handle, ws, kScratchBytes, a, lp);
    if (st != MOE_OK)
        return st;
    return from_hip(launch_layout(a, lp, s));
}

moe_status_t moe_dispatch(const moe_config_t *cfg, int32_t num_tokens, const uint16_t *x, const float *topk_w,
                          const moe_handle_t *handle, void *out_x, void *out_scale, float *out_row_weight,
                          void *stream)
{
    DispatchArgs a;
    const moe_status_t st =
        prepare_dispatch(cfg, num_tokens, x, topk_w, handle, out_x, out_scale, out_row_weight, a);
    if (st != MOE_OK || num_tokens == 0)
        return st;
    return from_hip(launch_dispatch(a, cfg->quant, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_dispatch_fused(const moe_config_t *cfg, int32_t num_tokens, const int32_t *topk_idx,
                                const uint16_t *x, const float *topk_w, const moe_handle_t *handle,
                                void *workspace, size_t workspace_bytes, void *out_x, void *out_scale,
                                float *out_row_weight, void *stream)
{
    LayoutArgs la;
    LayoutPlan lp;
    DispatchArgs da;
    moe_status_t st = prepare_layout(cfg, num_tokens, topk_idx, handle, workspace, workspace_bytes, la, lp);
    if (st != MOE_OK)
        return st;
    st = prepare_dispatch(cfg, num_tokens, x, topk_w, handle, out_x, out_scale, out_row_weight, da);
    if (st != MOE_OK)
        return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (num_tokens > 0 && fused_prefetch_plan(da, lp, cfg->num_cus, la)) {
        // large batch: layout with x prefetched on the idle compute units, then the rows
        hipError_t e = launch_layout(la, lp, s);
        if (e == hipSuccess)
            e = launch_dispatch(da, cfg->quant, s);
        return from_hip(e);
    }
    FusedPlan fp;
    if (fused_plan(num_tokens, cfg->num_topk, cfg->hidden, cfg->num_experts, cfg->quant, cfg->num_cus, fp)) {
        FusedArgs f;
        f.lay = la;
        f.lay.rounds = 1;
        f.lay.chunk = fp.tokens_per_block * cfg->num_topk;
        f.lay.nblocks = fp.blocks;
        f.d = da;
        f.d.plan = fp.plan;
        f.tokens_per_block = fp.tokens_per_block;
        return from_hip(launch_dispatch_fused(f, cfg->quant, s));
    }
    // batches the one-launch kernel does not take: the two calls back to back,
    // large ones with part of x prefetched by the layout kernels
    if (num_tokens > 0)
        split_prefetch_plan(da, lp, cfg->num_cus, la);
    hipError_t e = launch_layout(la, lp, s);
    if (e == hipSuccess && num_tokens > 0)
        e = launch_dispatch(da, cfg->quant, s);
    return from_hip(e);
}

moe_status_t moe_combine(const moe_config_t *cfg, int32_t num_tokens, const uint16_t *y, const float *topk_w,
                         const moe_handle_t *handle, uint16_t *out, void *stream)
{
    moe_status_t st = check_config(cfg);
    if (st != MOE_OK)
        return st;
    if ((st = check_handle(handle)) != MOE_OK)
        return st;
    if ((st = check_tokens(*cfg, num_tokens)) != MOE_OK)
        return st;
    if (num_tokens > 0 && (y == nullptr || !aligned(y, 16) || topk_w == nullptr || !aligned(topk_w, 4) ||
                           out == nullptr || !aligned(out, 16)))
        return MOE_ERR_INVALID_ARG;
    if (num_tokens == 0)
        return MOE_OK;

    CombineArgs a;
    a.y = y;
    a.topk_w = topk_w;
    a.pair_to_row = handle->pair_to_row;
    a.out = out;
    a.T = num_tokens;
    a.K = cfg->num_topk;
    a.H = cfg->hidden;
    a.plan = row_plan(num_tokens, cfg->hidden, kCombineWidth, kCombineMaxIters, cfg->num_cus,
                      kCombineMinItemsPerToken);
    a.topk_idx = nullptr;
    a.token_rank_row = nullptr;
    a.E = a.R = a.L = 0;
    a.stream_out = (int64_t)num_tokens * cfg->hidden * 2 > kCombineStreamOutBytes;
    a.stream_in = (int64_t)num_tokens * cfg->num_topk * cfg->hidden * 2 > kCombineStreamInBytes;
    return from_hip(launch_combine(a, static_cast<hipStream_t>(stream)));
}

size_t moe_rank_rows_capacity(const moe_config_t *cfg)
{
    if (check_config(cfg) != MOE_OK || cfg->num_ranks > kMaxDedupRanks)
        return 0;
    return (size_t)rank_rows64(*cfg);
}

moe_status_t moe_rank_layout(const moe_config_t *cfg, int32_t num_tokens, const int32_t *topk_idx,
                             const moe_rank_handle_t *rank_handle, void *stream)
{
    const moe_status_t st = check_dedup(cfg, num_tokens, rank_handle);
    if (st != MOE_OK)
        return st;
    if (num_tokens > 0 && (topk_idx == nullptr || !aligned(topk_idx, 4)))
        return MOE_ERR_INVALID_ARG;
    RankLayoutArgs a;
    a.topk_idx = topk_idx;
    a.T = num_tokens;
    a.K = cfg->num_topk;
    a.E = cfg->num_experts;
    a.R = cfg->num_ranks;
    a.L = cfg->num_experts / cfg->num_ranks;
    a.rows_cap = (int32_t)rank_rows64(*cfg);
    a.vec4 = (a.K % 4 == 0 && aligned(topk_idx, 16)) ? 1 : 0;
    a.rank_magic = ((1ull << 32) + (uint64_t)a.L - 1) / (uint64_t)a.L;
    a.h = *rank_handle;
    rank_layout_plan(num_tokens, a.R, a);
    return from_hip(launch_rank_layout(a, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_dispatch_dedup(const moe_config_t *cfg, int32_t num_tokens, const uint16_t *x,
                                const moe_rank_handle_t *rank_handle, void *send_x, void *send_scale, void *stream)
{
    const moe_status_t st = check_dedup(cfg, num_tokens, rank_handle);
    if (st != MOE_OK)
        return st;
    const bool fp8 = cfg->quant != MOE_QUANT_NONE;
    if (send_x == nullptr || !aligned(send_x, 16))
        return MOE_ERR_INVALID_ARG;
    if (fp8 ? (send_scale == nullptr || !aligned(send_scale, 4)) : send_scale != nullptr)
        return MOE_ERR_INVALID_ARG;
    if (num_tokens > 0 && (x == nullptr || !aligned(x, 16)))
        return MOE_ERR_INVALID_ARG;
    if (num_tokens == 0)
        return MOE_OK;
    // the row kernel of dispatch over (token, rank) slots instead of pairs
    DispatchArgs a;
    a.x = x;
    a.topk_w = nullptr;
    a.pair_to_row = rank_handle->token_rank_row;
    a.out_x = send_x;
    a.out_scale = send_scale;
    a.out_row_weight = nullptr;
    a.T = num_tokens;
    a.K = cfg->num_ranks;
    a.H = cfg->hidden;
    a.plan = fp8 ? row_plan(num_tokens, cfg->hidden, kDispatchFp8Width, kDispatchFp8MaxIters, cfg->num_cus,
                            kDispatchMinItemsPerToken)
                 : row_plan(num_tokens, cfg->hidden, kDispatchBf16Width, kDispatchBf16MaxIters, cfg->num_cus,
                            kDispatchMinItemsPerToken);
    return from_hip(launch_dispatch(a, cfg->quant, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_expand(const moe_config_t *cfg, int32_t num_tokens, const int32_t *topk_idx, const void *send_x,
                        const void *send_scale, const moe_rank_handle_t *rank_handle, const moe_handle_t *handle,
                        void *out_x, void *out_scale, void *stream)
{
    moe_status_t st = check_dedup(cfg, num_tokens, rank_handle);
    if (st != MOE_OK)
        return st;
    if ((st = check_handle(handle)) != MOE_OK)
        return st;
    const bool fp8 = cfg->quant != MOE_QUANT_NONE;
    if (out_x == nullptr || !aligned(out_x, 16))
        return MOE_ERR_INVALID_ARG;
    if (fp8 ? (out_scale == nullptr || !aligned(out_scale, 4)) : out_scale != nullptr)
        return MOE_ERR_INVALID_ARG;
    if (num_tokens > 0 && (topk_idx == nullptr || !aligned(topk_idx, 4) || send_x == nullptr ||
                           !aligned(send_x, 16) || (fp8 && (send_scale == nullptr || !aligned(send_scale, 4)))))
        return MOE_ERR_INVALID_ARG;
    if (num_tokens == 0)
        return MOE_OK;
    const int32_t NB = cfg->hidden / kQuantGroup;
    ExpandArgs a;
    a.topk_idx = topk_idx;
    a.pair_to_row = handle->pair_to_row;
    a.token_rank_row = rank_handle->token_rank_row;
    a.send_x = static_cast<const uint8_t *>(send_x);
    a.send_scale = static_cast<const uint8_t *>(send_scale);
    a.out_x = static_cast<uint8_t *>(out_x);
    a.out_scale = static_cast<uint8_t *>(out_scale);
    a.T = num_tokens;
    a.K = cfg->num_topk;
    a.E = cfg->num_experts;
    a.R = cfg->num_ranks;
    a.L = cfg->num_experts / cfg->num_ranks;
    a.row_bytes = fp8 ? cfg->hidden : 2 * cfg->hidden;
    // words of scales per row: fp32 per 128 channels, UE8M0 4 blocks per word, MX bytes H/32 = NB words
    a.scale_words = cfg->quant == MOE_QUANT_FP8_F32     ? NB
                    : cfg->quant == MOE_QUANT_FP8_UE8M0 ? (NB + 3) / 4
                    : cfg->quant == MOE_QUANT_MXFP8     ? NB
                                                        : 0;
    a.plan = row_plan(num_tokens, a.row_bytes, kExpandWidth, kExpandMaxIters, cfg->num_cus,
                      kDispatchMinItemsPerToken);
    return from_hip(launch_expand(a, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine_partial(const moe_config_t *cfg, int32_t num_tokens, const int32_t *topk_idx,
                                 const uint16_t *y, const float *topk_w, const moe_handle_t *handle,
                                 const moe_rank_handle_t *rank_handle, uint16_t *partial, void *stream)
{
    moe_status_t st = check_dedup(cfg, num_tokens, rank_handle);
    if (st != MOE_OK)
        return st;
    if ((st = check_handle(handle)) != MOE_OK)
        return st;
    if (num_tokens > 0 && (topk_idx == nullptr || !aligned(topk_idx, 4) || y == nullptr || !aligned(y, 16) ||
                           topk_w == nullptr || !aligned(topk_w, 4) || partial == nullptr || !aligned(partial, 16)))
        return MOE_ERR_INVALID_ARG;
    if (num_tokens == 0)
        return MOE_OK;
    CombineArgs a;
    a.y = y;
    a.topk_w = topk_w;
    a.pair_to_row = handle->pair_to_row;
    a.out = partial;
    a.T = num_tokens;
    a.K = cfg->num_topk;
    a.H = cfg->hidden;
    a.plan = row_plan(num_tokens, cfg->hidden, kCombineWidth, kCombineMaxIters, cfg->num_cus,
                      kCombineMinItemsPerToken);
    a.topk_idx = topk_idx;
    a.token_rank_row = rank_handle->token_rank_row;
    a.E = cfg->num_experts;
    a.R = cfg->num_ranks;
    a.L = cfg->num_experts / cfg->num_ranks;
    // device-scope stores that leave the partial rows in the Infinity Cache:
    // the reduction reads them right away (streaming them measured
    // 242 -> 254 us here at the DeepSeek-V3 prefill shape)
    a.stream_out = 0;
    a.stream_in = (int64_t)num_tokens * cfg->num_topk * cfg->hidden * 2 > kCombineStreamInBytes;
    return from_hip(launch_combine_partial(a, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine_reduce(const moe_config_t *cfg, int32_t num_tokens, const uint16_t *partial,
                                const moe_rank_handle_t *rank_handle, uint16_t *out, void *stream)
{
    const moe_status_t st = check_dedup(cfg, num_tokens, rank_handle);
    if (st != MOE_OK)
        return st;
    if (num_tokens > 0 && (partial == nullptr || !aligned(partial, 16) || out == nullptr || !aligned(out, 16)))
        return MOE_ERR_INVALID_ARG;
    if (num_tokens == 0)
        return MOE_OK;
    // the one-level kernel over (token, rank) rows with unit weights
    CombineArgs a;
    a.y = partial;
    a.topk_w = nullptr;
    a.pair_to_row = rank_handle->token_rank_row;
    a.out = out;
    a.T = num_tokens;
    a.K = cfg->num_ranks;
    a.H = cfg->hidden;
    a.plan = row_plan(num_tokens, cfg->hidden, kCombineWidth, kCombineMaxIters, cfg->num_cus,
                      kCombineMinItemsPerToken);
    a.topk_idx = nullptr;
    a.token_rank_row = nullptr;
    a.E = a.R = a.L = 0;
    a.stream_out = (int64_t)num_tokens * cfg->hidden * 2 > kCombineStreamOutBytes;
    a.stream_in = (int64_t)num_tokens * cfg->num_ranks * cfg->hidden * 2 > kCombineStreamInBytes;
    return from_hip(launch_combine(a, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_row_expert(const moe_config_t *cfg, const moe_handle_t *handle, int32_t *row_expert,
                            void *stream)
{
    moe_status_t st = check_config(cfg);
    if (st != MOE_OK)
        return st;
    if ((st = check_handle(handle)) != MOE_OK)
        return st;
    if (row_expert == nullptr || !aligned(row_expert, 4))
        return MOE_ERR_INVALID_ARG;
    RowExpertArgs a;
    a.expert_offset = handle->expert_offset;
    a.recv_count = handle->recv_count;
    a.E = cfg->num_experts;
    a.rows = rows_capacity64(*cfg);
    a.row_expert = row_expert;
    return from_hip(launch_row_expert(a, static_cast<hipStream_t>(stream)));
}

size_t moe_repack_rows_capacity(const moe_config_t *cfg, int32_t align)
{
    if (check_config(cfg) != MOE_OK || cfg->layout != MOE_LAYOUT_MASKED || align < 1)
        return 0;
    const int64_t r = repack_rows64(*cfg, align);
    return r > INT32_MAX ? 0 : (size_t)r;
}

moe_status_t moe_repack_masked_to_contiguous(const moe_config_t *cfg, int32_t align, const moe_handle_t *handle,
                                             const void *x, const void *scale, void *out_x, void *out_scale,
                                             int32_t *out_expert_offset, int32_t *out_row_expert, void *stream)
{
    moe_status_t st = check_config(cfg);
    if (st != MOE_OK)
        return st;
    if (cfg->layout != MOE_LAYOUT_MASKED || align < 1)
        return MOE_ERR_INVALID_ARG;
    if (repack_rows64(*cfg, align) > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    if ((st = check_handle(handle)) != MOE_OK)
        return st;
    const bool fp8 = cfg->quant != MOE_QUANT_NONE;
    if (x == nullptr || !aligned(x, 16) || out_x == nullptr || !aligned(out_x, 16))
        return MOE_ERR_INVALID_ARG;
    if (fp8 ? (scale == nullptr || !aligned(scale, 4) || out_scale == nullptr || !aligned(out_scale, 4))
            : (scale != nullptr || out_scale != nullptr))
        return MOE_ERR_INVALID_ARG;
    if (out_expert_offset == nullptr || !aligned(out_expert_offset, 4) || out_row_expert == nullptr ||
        !aligned(out_row_expert, 4))
        return MOE_ERR_INVALID_ARG;
    RepackArgs a;
    a.recv_count = handle->recv_count;
    a.in_offset = nullptr;
    a.out_offset = out_expert_offset;
    a.out_row_expert = out_row_expert;
    a.x = static_cast<const uint8_t *>(x);
    a.scale = static_cast<const uint8_t *>(scale);
    a.out_x = static_cast<uint8_t *>(out_x);
    a.out_scale = static_cast<uint8_t *>(out_scale);
    a.E = cfg->num_experts;
    a.C = cfg->capacity;
    a.align = align;
    a.row_bytes = fp8 ? cfg->hidden : 2 * cfg->hidden;
    a.scale_words = scale_words32(*cfg);
    a.out_rows = repack_rows64(*cfg, align);
    a.to_contiguous = 1;
    a.plan = row_plan((int32_t)repack_rows64(*cfg, 1), a.row_bytes, kAdaptWidth, kAdaptMaxIters, cfg->num_cus);
    return from_hip(launch_repack(a, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_repack_contiguous_to_masked(const moe_config_t *cfg, const moe_handle_t *handle,
                                             const int32_t *expert_offset, const uint16_t *y, uint16_t *y_masked,
                                             void *stream)
{
    moe_status_t st = check_config(cfg);
    if (st != MOE_OK)
        return st;
    if (cfg->layout != MOE_LAYOUT_MASKED)
        return MOE_ERR_INVALID_ARG;
    if ((st = check_handle(handle)) != MOE_OK)
        return st;
    if (expert_offset == nullptr || !aligned(expert_offset, 4) || y == nullptr || !aligned(y, 16) ||
        y_masked == nullptr || !aligned(y_masked, 16))
        return MOE_ERR_INVALID_ARG;
    RepackArgs a;
    a.recv_count = handle->recv_count;
    a.in_offset = expert_offset;
    a.out_offset = nullptr;
    a.out_row_expert = nullptr;
    a.x = reinterpret_cast<const uint8_t *>(y);
    a.scale = nullptr;
    a.out_x = reinterpret_cast<uint8_t *>(y_masked);
    a.out_scale = nullptr;
    a.E = cfg->num_experts;
    a.C = cfg->capacity;
    a.align = 1;
    a.row_bytes = 2 * cfg->hidden;
    a.scale_words = 0;
    a.out_rows = 0;
    a.to_contiguous = 0;
    a.plan = row_plan((int32_t)repack_rows64(*cfg, 1), a.row_bytes, kAdaptWidth, kAdaptMaxIters, cfg->num_cus);
    return from_hip(launch_repack(a, static_cast<hipStream_t>(stream)));
}

size_t moe_scale_words(const moe_config_t *cfg)
{
    if (check_config(cfg) != MOE_OK)
        return 0;
    return (size_t)scale_words32(*cfg);
}

moe_status_t moe_scales_mn_major(const moe_config_t *cfg, int32_t rows, const void *scale, void *scale_mn,
                                 void *stream)
{
    const moe_status_t st = check_config(cfg);
    if (st != MOE_OK)
        return st;
    const int32_t S = scale_words32(*cfg);
    if (S == 0 || rows < 0)
        return MOE_ERR_INVALID_ARG;
    if (scale == nullptr || !aligned(scale, 4) || scale_mn == nullptr || !aligned(scale_mn, 16))
        return MOE_ERR_INVALID_ARG;
    if (rows == 0)
        return MOE_OK;
    MnMajorArgs a;
    a.in = static_cast<const uint32_t *>(scale);
    a.out = static_cast<uint32_t *>(scale_mn);
    a.rows = rows;
    a.ld = ((int64_t)rows + 3) / 4 * 4;
    a.S = S;
    return from_hip(launch_scales_mn_major(a, static_cast<hipStream_t>(stream)));
}

const char *moe_status_str(moe_status_t status)
{
    // C callers may pass any int: read the bits as an int, since a C++ load of
    // the enum outside its enumerators' range is undefined
    static_assert(sizeof(int32_t) == sizeof(moe_status_t), "moe_status_t is 32 bits");
    int32_t code;
    memcpy(&code, &status, sizeof code);
    switch (code) {
    case MOE_OK:
        return "MOE_OK";
    case MOE_ERR_INVALID_ARG:
        return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_CAPACITY:
        return "MOE_ERR_CAPACITY";
    case MOE_ERR_UNSUPPORTED:
        return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP:
        return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

}  // extern "C"
