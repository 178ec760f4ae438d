// C-ABI entry points of the MoE expert-layer library (declared in include/moe_expert_layer.h).
// Host side only: argument checks, workspace carving, and the launch sequence on the caller's
// stream.  Nothing here allocates device memory or waits for the GPU (except the explicitly
// synchronous status / timing queries).
#include "moe_expert_layer.h"

#include <hip/hip_runtime.h>     // __device__ data: the allocation-free route's scratch
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {


namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

moe_status hip_fail(hipError_t e, const char* what)
{
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t elem_bytes(int dtype) { return dtype == MOE_F32 ? 4 : dtype == MOE_BF16 ? 2 : 1; }
int64_t out_bytes(int dtype) { return dtype == MOE_F32 ? 4 : 2; }

int row_tile(int dtype, int64_t H, int64_t F)
{
    return dtype == MOE_F32 ? kBmF32 : dtype == MOE_BF16 ? bf16_row_tile(H, F) : mx_row_tile(H, F);
}

// Column tiles of the down projection for the chunk counters (tasks per row tile).
int fc2_col_tiles(int dtype, int64_t H, int64_t F)
{
    if (dtype == MOE_F32)
        return static_cast<int>(ceil_div(H, 256));
    if (dtype == MOE_MXFP8_E4M3)
        return static_cast<int>(H / mx_fc2_cols_per_tile(H, F));
    return static_cast<int>(H / bf16_fc2_cols_per_tile(H, F));
}

// ------------------------------------------------------------------------------------- timing

struct TimingRec {
    const char* name;
    hipEvent_t a, b;
};

struct Timing {
    std::mutex mu;
    bool enabled = false;
    std::vector<TimingRec> pending;
    std::vector<hipEvent_t> pool;
    struct Total {
        const char* name;   // a string literal of this file: valid for the life of the library
        double ms;
        int64_t n;
    };
    std::map<std::string, Total> totals;
};

Timing& timing()
{
    static Timing t;
    return t;
}

hipEvent_t take_event(Timing& t)
{
    if (!t.pool.empty()) {
        hipEvent_t e = t.pool.back();
        t.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess)
        return nullptr;
    return e;
}

// Brackets one kernel launch with events when timing is enabled.
class Timed {
public:
    Timed(hipStream_t s, const char* name) : s_(s), name_(name)
    {
        Timing& t = timing();
        std::lock_guard<std::mutex> g(t.mu);
        if (!t.enabled)
            return;
        a_ = take_event(t);
        b_ = take_event(t);
        if (!a_ || !b_ || hipEventRecord(a_, s_) != hipSuccess)
            release(t);                           // timing is best effort: this launch goes untimed
    }
    ~Timed()
    {
        if (!a_ || !b_)
            return;
        const bool ok = hipEventRecord(b_, s_) == hipSuccess;
        Timing& t = timing();
        std::lock_guard<std::mutex> g(t.mu);
        if (ok)
            t.pending.push_back({name_, a_, b_});
        else
            release(t);
    }

private:
    // gives the events back to the pool (t.mu held); the launch is then not timed
    void release(Timing& t)
    {
        if (a_)
            t.pool.push_back(a_);
        if (b_)
            t.pool.push_back(b_);
        a_ = b_ = nullptr;
    }

    hipStream_t s_;
    const char* name_;
    hipEvent_t a_ = nullptr, b_ = nullptr;
};

#define LAUNCH(stream, name, call)                                   \
    do {                                                             \
        hipError_t err_;                                             \
        {                                                            \
            Timed timed_(stream, name);                              \
            err_ = (call);                                           \
        }                                                            \
        if (err_ != hipSuccess)                                      \
            return hip_fail(err_, name);                             \
    } while (0)

// ------------------------------------------------------------------------------------- checks

moe_status check_problem(const moe_problem* p, bool need_tokens, bool gemm = true)
{
    if (p == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "problem is null");
    if ((p->flags & ~static_cast<uint32_t>(MOE_FLAG_SEPARATE_PERMUTE | MOE_FLAG_QUANTIZE_X)) != 0 ||
        p->reserved != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "unknown flags, or reserved not 0");
    if (p->dtype != MOE_F32 && p->dtype != MOE_BF16 && p->dtype != MOE_MXFP8_E4M3)
        return fail(MOE_ERR_UNSUPPORTED, "unknown dtype %d", p->dtype);
    if ((p->flags & MOE_FLAG_QUANTIZE_X) != 0 && p->dtype != MOE_MXFP8_E4M3)
        return fail(MOE_ERR_INVALID_ARGUMENT, "MOE_FLAG_QUANTIZE_X needs dtype MOE_MXFP8_E4M3");
    if (p->H <= 0 || p->F <= 0 || p->E <= 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "H, F and E must be positive");
    if (p->E >= kMaxExperts)
        return fail(MOE_ERR_UNSUPPORTED, "E = %lld exceeds %d", (long long)p->E, kMaxExperts - 1);
    if (need_tokens) {
        if (p->T < 0 || p->k <= 0)
            return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 0 and k >= 1");
        if (p->k > p->E)
            return fail(MOE_ERR_INVALID_ARGUMENT, "k = %lld exceeds E = %lld", (long long)p->k,
                        (long long)p->E);
        if (p->T * p->k > INT32_MAX)
            return fail(MOE_ERR_UNSUPPORTED, "T * k exceeds int32 indexing");
        if (p->dtype == MOE_MXFP8_E4M3 && p->T * p->k * std::max(p->H, p->F) > UINT32_MAX)
            return fail(MOE_ERR_UNSUPPORTED, "MX needs T * k * max(H, F) < 2^32");
    }
    if (p->head_m_size < 0 || p->head_m_size % kChunkAlign != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "head_m_size must be 0 or a multiple of %d",
                    kChunkAlign);
    switch (p->dtype) {
    case MOE_F32:
        if (p->H % 4)
            return fail(MOE_ERR_UNSUPPORTED, "float32 needs H %% 4 == 0");
        break;
    case MOE_BF16:
        if (p->H % 8)
            return fail(MOE_ERR_UNSUPPORTED, "bfloat16 needs H %% 8 == 0");
        if (gemm && !bf16_supported(p->H, p->F))
            return fail(MOE_ERR_UNSUPPORTED, "bfloat16 GEMMs need H %% 128 == 0 and F %% 64 == 0");
        break;
    default:
        if (p->H % 32)
            return fail(MOE_ERR_UNSUPPORTED, "MX needs H %% 32 == 0");
        if (gemm && (p->H % 128 || p->F % 128))
            return fail(MOE_ERR_UNSUPPORTED, "MX GEMMs need H and F multiples of 128");
        break;
    }
    // the GEMMs address a row tile's operands by 32-bit offsets from its first row (at most 256
    // rows of K elements, 32 weight rows of N), which this bound keeps below 2^31 bytes
    if (p->H > MOE_MAX_HIDDEN || p->F > MOE_MAX_HIDDEN)
        return fail(MOE_ERR_UNSUPPORTED, "H and F must be at most %d", MOE_MAX_HIDDEN);
    return MOE_OK;
}

}  // namespace

// ------------------------------------------------------------------------------------- layouts

RouteLayout route_layout(int64_t T, int64_t k, int64_t E, size_t base)
{
    RouteLayout L;
    L.status = 0;
    L.nblocks = ceil_div(T * k, kRouteSlotsPerBlock);
    size_t off = base == 0 ? kAlign : base;
    L.block_counts = off;
    off = align_up(off + sizeof(int32_t) * static_cast<size_t>(L.nblocks * (E + 1)));
    L.total = off;
    return L;
}

FfnLayout ffn_layout(int dtype, int64_t M, int64_t G, int64_t H, int64_t F, int64_t chunk,
                     size_t base)
{
    FfnLayout L;
    L.bm1 = L.bm2 = row_tile(dtype, H, F);
    L.num_chunks = chunk > 0 ? std::max<int64_t>(1, ceil_div(M, chunk)) : 1;
    L.max_tiles1 = max_mtiles(M, G, chunk, L.bm1);
    L.max_tiles2 = max_mtiles(M, G, chunk, L.bm2);
    size_t off = base;
    L.status = 0;
    if (base == 0)
        off = kAlign;
    L.tile_count = off;
    off = align_up(off + 8 * sizeof(int32_t));
    L.task_ctr = off;
    off = align_up(off + 2 * kXcdCount * sizeof(int32_t));
    L.chunk_done = off;
    off = align_up(off + sizeof(int32_t) * static_cast<size_t>(L.num_chunks));
    L.chunk_tiles = off;
    off = align_up(off + sizeof(int32_t) * static_cast<size_t>(L.num_chunks));
    L.tiles1 = off;
    off = align_up(off + sizeof(MTile) * static_cast<size_t>(L.max_tiles1));
    L.tiles2 = L.tiles1;
    if (L.bm2 != L.bm1) {
        L.tiles2 = off;
        off = align_up(off + sizeof(MTile) * static_cast<size_t>(L.max_tiles2));
    }
    L.tiles_run = off;
    off = align_up(off + sizeof(MTile) * static_cast<size_t>(L.max_tiles1));
    L.h = off;
    off = align_up(off + static_cast<size_t>(M * F * elem_bytes(dtype)));
    L.h_scale = off;
    if (dtype == MOE_MXFP8_E4M3)
        off = align_up(off + static_cast<size_t>(M * (F / 32)));
    L.total = off;
    return L;
}

ForwardLayout forward_layout(int dtype, int64_t T, int64_t H, int64_t F, int64_t E, int64_t k,
                             int64_t chunk, bool quantize_x)
{
    const int64_t M = T * k;
    ForwardLayout L;
    L.ffn = ffn_layout(dtype, M, E, H, F, chunk, 0);
    size_t off = L.ffn.total;
    L.route = route_layout(T, k, E, off);
    off = L.route.total;
    L.counts = off;
    off = align_up(off + sizeof(int32_t) * static_cast<size_t>(E));
    L.offsets = off;
    off = align_up(off + sizeof(int32_t) * static_cast<size_t>(E + 1));
    L.perm = off;
    off = align_up(off + sizeof(int32_t) * static_cast<size_t>(M));
    L.pos = off;
    off = align_up(off + sizeof(int32_t) * static_cast<size_t>(M));
    L.x_perm = off;
    off = align_up(off + static_cast<size_t>(M * H * elem_bytes(dtype)));
    L.x_perm_scale = off;
    if (dtype == MOE_MXFP8_E4M3)
        off = align_up(off + static_cast<size_t>(M * (H / 32)));
    L.y_perm = off;
    off = align_up(off + static_cast<size_t>(M * H * out_bytes(dtype)));
    L.x_q = off;
    L.x_q_scale = off;
    if (quantize_x) {
        off = align_up(off + static_cast<size_t>(T * H));
        L.x_q_scale = off;
        off = align_up(off + static_cast<size_t>(T * (H / 32)));
    }
    L.total = off;
    return L;
}

const DeviceInfo& device_info()
{
    static std::mutex mu;
    static std::map<int, DeviceInfo> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        dev = 0;                                  // no current device: the launch itself will fail
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(dev);
    if (it != cache.end())
        return it->second;
    DeviceInfo info{};
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu <= 0)
        cu = 256;
    info.cu_count = (cu + 7) / 8 * 8;   // persistent grids are dealt evenly to the 8 XCDs
    return cache.emplace(dev, info).first->second;
}

namespace {

template <class T>
T* at(void* ws, size_t off)
{
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Route sub-sequence shared by moe_route and the forward.  Writes the status word at ws + 0.
moe_status run_route(const int32_t* ids, int64_t T, int64_t k, int64_t E, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* pos, void* ws,
                     const RouteLayout& L, hipStream_t s)
{
    const int64_t M = T * k;
    int32_t* bc = at<int32_t>(ws, L.block_counts);
    int32_t* status = at<int32_t>(ws, L.status);
    if (M > 0)
        LAUNCH(s, "route_count", launch_route_count(ids, M, E, bc, L.nblocks, s));
    LAUNCH(s, "route_scan", launch_route_scan(bc, L.nblocks, E, M, counts, offsets, perm, status, s));
    if (M > 0)
        LAUNCH(s, "route_scatter", launch_route_scatter(ids, M, E, bc, L.nblocks, perm, pos, s));
    return MOE_OK;
}

// Whether fc1 can read the permuted rows straight from x through perm (the permute step folded
// into its row copies): the 256-row-tile kernels, with x addressable by 32-bit byte offsets.
bool fc1_gathers(int dtype, int64_t T, int64_t H, int64_t F)
{
    if (dtype == MOE_BF16)
        return bf16_row_tile(H, F) == 256 && T * H * 2 < (int64_t{1} << 32);
    if (dtype == MOE_MXFP8_E4M3)
        return mx_row_tile(H, F) == 256 && T * H < (int64_t{1} << 32);
    return false;
}

// fc1 + SwiGLU + fc2 over grouped rows; tiles are built from (offsets, group_expert).  gather
// (may be null, see fc1_gathers): permuted row p is row gather[p] / gather_k of `rows`.
moe_status run_ffn(int dtype, const void* rows, const uint8_t* rows_scale, int64_t M,
                   const int32_t* offsets, const int32_t* group_expert, int64_t G, int64_t E,
                   int64_t H, int64_t F, int64_t head_m_size, const void* wg, const uint8_t* wgs,
                   const void* wu, const uint8_t* wus, const void* wd, const uint8_t* wds,
                   void* y, void* ws, const FfnLayout& L, bool write_status, hipStream_t s,
                   const int32_t* gather = nullptr, int gather_k = 1, uint16_t* save_gu = nullptr)
{
    const int64_t chunk = head_m_size > 0 ? head_m_size : std::max<int64_t>(M, 1);
    int32_t* status = at<int32_t>(ws, L.status);
    int32_t* tcount = at<int32_t>(ws, L.tile_count);
    MTile* tiles = at<MTile>(ws, L.tiles1);
    int32_t* chunk_done = head_m_size > 0 ? at<int32_t>(ws, L.chunk_done) : nullptr;
    int32_t* chunk_tiles = head_m_size > 0 ? at<int32_t>(ws, L.chunk_tiles) : nullptr;
    int32_t* task_ctr = at<int32_t>(ws, L.task_ctr);
    // Unchunked large tiles: fc1 takes a table in which each expert is one run of near-equal tiles, so
    // the tasks of a weight strip run side by side, take equal time and share the strip in the L2;
    // fc2 keeps the tails last (its short ones split into half-width tasks).
    const bool fc1_in_run = head_m_size <= 0 && L.bm1 == 256 && dtype != MOE_F32;
    MTile* tiles_fc1 = fc1_in_run ? at<MTile>(ws, L.tiles_run) : tiles;
    int32_t* tcount_fc1 = fc1_in_run ? tcount + 4 : tcount;
    // The bf16 fc2 takes the same table when groups average at most two row tiles: there the tails
    // are a large share of the tiles, and their weight strips still in the L2 count for more than
    // splitting the short ones into half-width tasks (measured: fine-grained fc2 -10%, while groups
    // of four tiles lose 7-13% without the split).
    const bool fc2_in_run = fc1_in_run && dtype == MOE_BF16 && M <= 2 * int64_t{L.bm2} * G;
    MTile* tiles_fc2 = fc2_in_run ? tiles_fc1 : tiles;
    int32_t* tcount_fc2 = fc2_in_run ? tcount_fc1 : tcount;
    LAUNCH(s, "build_tiles",
           launch_build_tiles(offsets, group_expert, G, E, M, chunk, L.bm1, tiles, L.max_tiles1,
                              tcount, chunk_tiles, chunk_done, L.num_chunks,
                              fc2_col_tiles(dtype, H, F), task_ctr, status, write_status, s,
                              fc1_in_run ? tiles_fc1 : nullptr, fc1_in_run ? tcount_fc1 : nullptr));
    if (dtype == MOE_BF16) {
        uint16_t* h = at<uint16_t>(ws, L.h);
        LAUNCH(s, "fc1_bf16",
               launch_fc1_bf16(static_cast<const uint16_t*>(rows), static_cast<const uint16_t*>(wg),
                               static_cast<const uint16_t*>(wu), h, tiles_fc1, tcount_fc1, H, F,
                               task_ctr, gather, gather_k, save_gu,
                               save_gu != nullptr ? save_gu + M * F : nullptr, s));
        LAUNCH(s, "fc2_bf16",
               launch_fc2_bf16(h, static_cast<const uint16_t*>(wd), static_cast<uint16_t*>(y),
                               tiles_fc2, tcount_fc2, H, F, chunk_done, task_ctr + kXcdCount, s));
    } else if (dtype == MOE_F32) {
        float* h = at<float>(ws, L.h);
        LAUNCH(s, "fc1_f32",
               launch_fc1_f32(static_cast<const float*>(rows), static_cast<const float*>(wg),
                              static_cast<const float*>(wu), h, tiles, tcount, H, F, s));
        LAUNCH(s, "fc2_f32",
               launch_fc2_f32(h, static_cast<const float*>(wd), static_cast<float*>(y), tiles,
                              tcount, H, F, chunk_done, s));
    } else {
        uint8_t* h = at<uint8_t>(ws, L.h);
        uint8_t* hs = at<uint8_t>(ws, L.h_scale);
        LAUNCH(s, "fc1_mx",
               launch_fc1_mx(static_cast<const uint8_t*>(rows), rows_scale,
                             static_cast<const uint8_t*>(wg), wgs, static_cast<const uint8_t*>(wu),
                             wus, h, hs, tiles_fc1, tcount_fc1, H, F, task_ctr, gather, gather_k, s));
        LAUNCH(s, "fc2_mx",
               launch_fc2_mx(h, hs, static_cast<const uint8_t*>(wd), wds, static_cast<uint16_t*>(y),
                             tiles, tcount, H, F, chunk_done, task_ctr + kXcdCount, s));
    }
    return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

// ===================================================================================== C ABI

MOE_API moe_status moe_workspace_size(const moe_problem* p, size_t* bytes)
{
    if (bytes == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is null");
    if (moe_status st = check_problem(p, true); st != MOE_OK)
        return st;
    *bytes = forward_layout(p->dtype, p->T, p->H, p->F, p->E, p->k, p->head_m_size,
                            (p->flags & MOE_FLAG_QUANTIZE_X) != 0).total;
    return MOE_OK;
}

static moe_status forward_common(const moe_problem* p, const void* x, const uint8_t* x_scale,
                                 const void* wg, const uint8_t* wgs, const void* wu,
                                 const uint8_t* wus, const void* wd, const uint8_t* wds,
                                 const int32_t* ids, const float* probs, void* out, void* ws,
                                 size_t ws_bytes, hipStream_t s, void* saved_gu = nullptr)
{
    const bool quantize_x = (p->flags & MOE_FLAG_QUANTIZE_X) != 0;
    const ForwardLayout L = forward_layout(p->dtype, p->T, p->H, p->F, p->E, p->k, p->head_m_size,
                                           quantize_x);
    if (ws == nullptr || ws_bytes < L.total)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", L.total,
                    ws == nullptr ? size_t{0} : ws_bytes);
    const int64_t T = p->T, k = p->k, M = T * k, H = p->H;
    if (T > 0 && (x == nullptr || wg == nullptr || wu == nullptr || wd == nullptr ||
                  ids == nullptr || probs == nullptr || out == nullptr))
        return fail(MOE_ERR_INVALID_ARGUMENT, "null data pointer");
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* perm = at<int32_t>(ws, L.perm);
    int32_t* pos = at<int32_t>(ws, L.pos);
    if (moe_status st = run_route(ids, T, k, p->E, counts, offsets, perm, pos, ws, L.route, s);
        st != MOE_OK)
        return st;
    if (M == 0)
        return MOE_OK;
    const int64_t eb = elem_bytes(p->dtype);
    // The permute step runs inside fc1 (row copies gathered through perm) unless the caller asks
    // for it as a kernel of its own or the small-tile kernels serve these sizes.
    const bool fused = (p->flags & MOE_FLAG_SEPARATE_PERMUTE) == 0 && fc1_gathers(p->dtype, T, H, p->F);
    const void* rows = x;
    const uint8_t* rows_scale = x_scale;
    if (quantize_x) {
        // bfloat16 x is MX-encoded on its way into the gather: once per token, into the workspace,
        // when fc1 gathers the rows itself; otherwise straight into the permuted rows
        const auto* xb = static_cast<const uint16_t*>(x);
        if (fused) {
            LAUNCH(s, "mx_encode_x",
                   launch_mx_encode_bf16_rows(xb, T, H, nullptr, k, M, at<uint8_t>(ws, L.x_q),
                                              at<uint8_t>(ws, L.x_q_scale), s));
            rows = at<void>(ws, L.x_q);
            rows_scale = at<uint8_t>(ws, L.x_q_scale);
        } else {
            LAUNCH(s, "mx_encode_permute",
                   launch_mx_encode_bf16_rows(xb, T, H, pos, k, M, at<uint8_t>(ws, L.x_perm),
                                              at<uint8_t>(ws, L.x_perm_scale), s));
            rows = at<void>(ws, L.x_perm);
            rows_scale = at<uint8_t>(ws, L.x_perm_scale);
        }
    } else if (!fused) {
        LAUNCH(s, "permute", launch_permute(x, pos, at<void>(ws, L.x_perm), T, k, M, H * eb, s));
        if (p->dtype == MOE_MXFP8_E4M3)
            LAUNCH(s, "permute_scale",
                   launch_permute(x_scale, pos, at<void>(ws, L.x_perm_scale), T, k, M, H / 32, s));
        rows = at<void>(ws, L.x_perm);
        rows_scale = at<uint8_t>(ws, L.x_perm_scale);
    }
    if (moe_status st = run_ffn(p->dtype, rows, rows_scale, M, offsets, nullptr, p->E, p->E, H, p->F,
                                p->head_m_size, wg, wgs, wu, wus, wd, wds, at<void>(ws, L.y_perm), ws,
                                L.ffn, false, s, fused ? perm : nullptr, static_cast<int>(k),
                                static_cast<uint16_t*>(saved_gu));
        st != MOE_OK)
        return st;
    LAUNCH(s, "unpermute",
           launch_unpermute(p->dtype == MOE_F32 ? 0 : 1, at<void>(ws, L.y_perm), pos, probs, out,
                            T, k, M, H, s));
    return MOE_OK;
}

MOE_API moe_status moe_expert_forward(const moe_problem* p, const void* x, const void* w_gate,
                                      const void* w_up, const void* w_down,
                                      const int32_t* expert_ids, const float* probs, void* out,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (moe_status st = check_problem(p, true); st != MOE_OK)
        return st;
    if (p->dtype == MOE_MXFP8_E4M3)
        return fail(MOE_ERR_INVALID_ARGUMENT, "MX inputs go through moe_expert_forward_mx");
    return forward_common(p, x, nullptr, w_gate, nullptr, w_up, nullptr, w_down, nullptr,
                          expert_ids, probs, out, workspace, workspace_bytes, stream);
}

MOE_API moe_status moe_expert_forward_train(const moe_problem* p, const void* x, const void* w_gate,
                                            const void* w_up, const void* w_down,
                                            const int32_t* expert_ids, const float* probs, void* out,
                                            void* saved_gu, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream)
{
    if (moe_status st = check_problem(p, true); st != MOE_OK)
        return st;
    if (p->dtype != MOE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "saving g and u for the backward takes bfloat16 only");
    if (p->T > 0 && saved_gu == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "saved_gu is null");
    return forward_common(p, x, nullptr, w_gate, nullptr, w_up, nullptr, w_down, nullptr,
                          expert_ids, probs, out, workspace, workspace_bytes, stream, saved_gu);
}

MOE_API moe_status moe_expert_forward_mx(const moe_problem* p, const uint8_t* x,
                                         const uint8_t* x_scale, const uint8_t* w_gate,
                                         const uint8_t* wg_scale, const uint8_t* w_up,
                                         const uint8_t* wu_scale, const uint8_t* w_down,
                                         const uint8_t* wd_scale, const int32_t* expert_ids,
                                         const float* probs, void* out_bf16, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream)
{
    if (moe_status st = check_problem(p, true); st != MOE_OK)
        return st;
    if (p->dtype != MOE_MXFP8_E4M3)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_expert_forward_mx needs dtype MOE_MXFP8_E4M3");
    const bool quantize_x = (p->flags & MOE_FLAG_QUANTIZE_X) != 0;
    if (quantize_x && x_scale != nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "with MOE_FLAG_QUANTIZE_X, x is bfloat16 and x_scale must be null");
    if (p->T > 0 && ((!quantize_x && x_scale == nullptr) || wg_scale == nullptr ||
                     wu_scale == nullptr || wd_scale == nullptr))
        return fail(MOE_ERR_INVALID_ARGUMENT, "null scale pointer");
    return forward_common(p, x, x_scale, w_gate, wg_scale, w_up, wu_scale, w_down, wd_scale,
                          expert_ids, probs, out_bf16, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------------------------------------- backward

namespace moe {
namespace {

constexpr size_t kWgradZeroBytes = 1024;    // zero rows the weight-gradient copies read past an expert

struct BackwardLayout {
    RouteLayout route;
    size_t counts = 0, offsets = 0, perm = 0, pos = 0, tile_count = 0, task_ctr = 0;
    size_t tiles_r = 0, tiles_d = 0, tiles_run = 0, prow = 0, partial = 0;
    size_t x_perm = 0, dout_perm = 0, g = 0, u = 0, dgu = 0, hp = 0, dx_perm = 0;
    size_t wgrad_ctr = 0, zero = 0, total = 0;   // last: the zero rows sit above every source row
    int64_t max_tiles_r = 0, max_tiles_d = 0;
    int bm_r = 0, bm_d = 0;
};

// g and u are recomputed with the fc1 kernel (h not stored), whose row tiles are bm_r high; the
// backward's own GEMMs use dgrad_row_tile rows.  With 256-row tiles the recompute (and the dgrads,
// when theirs are 256 rows too) take the forward fc1's table: each expert one run of near-equal
// tiles (tiles_run).
BackwardLayout backward_layout(int64_t T, int64_t H, int64_t F, int64_t E, int64_t k)
{
    const int64_t M = T * k;
    BackwardLayout L;
    L.route = route_layout(T, k, E, 0);
    size_t off = L.route.total;
    auto take = [&off](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    const auto n = [](int64_t v) { return static_cast<size_t>(v); };
    L.counts = take(4 * n(E));
    L.offsets = take(4 * n(E + 1));
    L.perm = take(4 * n(M));
    L.pos = take(4 * n(M));
    L.tile_count = take(8 * sizeof(int32_t));      // [0..3] tiles_r ([1..3] tiles_d), [4..7] tiles_run
    L.task_ctr = take(2 * kXcdCount * sizeof(int32_t));
    L.bm_r = bf16_row_tile(H, F);
    L.max_tiles_r = max_mtiles(M, E, 0, L.bm_r);
    L.bm_d = dgrad_row_tile(M, H, F);
    L.max_tiles_d = max_mtiles(M, E, 0, L.bm_d);
    L.tiles_r = take(sizeof(MTile) * n(L.max_tiles_r));
    L.tiles_d = L.bm_r == L.bm_d ? L.tiles_r : take(sizeof(MTile) * n(L.max_tiles_d));
    L.tiles_run = L.bm_r == 256 ? take(sizeof(MTile) * n(L.max_tiles_r)) : 0;
    L.prow = take(4 * n(M));
    L.partial = take(4 * n(M) * n(F / 64));
    L.x_perm = take(2 * n(M) * n(H));
    L.dout_perm = take(2 * n(M) * n(H));
    L.g = take(2 * n(M) * n(F));
    L.u = take(2 * n(M) * n(F));
    L.dgu = take(4 * n(M) * n(F));
    L.hp = take(2 * n(M) * n(F));
    L.dx_perm = take(2 * 4 * n(M) * n(H));   // each slot's dx row: two fp32 parts, or bf16
    L.wgrad_ctr = take(5 * kXcdCount * sizeof(int32_t));     // 3 weight gradients, 2 dgrads
    // a weight-gradient copy source starts at most one row (plus its column offset) past the end
    // of its buffer; the zero rows must lie above every such start
    take(n(std::max(2 * H, 4 * F)));
    L.zero = take(kWgradZeroBytes);
    L.total = off;
    return L;
}

moe_status check_backward(const moe_problem* p)
{
    if (moe_status st = check_problem(p, true); st != MOE_OK)
        return st;
    if (p->dtype != MOE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "the backward takes bfloat16 (dtype MOE_BF16) only");
    if (p->head_m_size != 0)
        return fail(MOE_ERR_UNSUPPORTED, "the backward is unchunked (head_m_size must be 0)");
    if (!bwd_supported(p->H, p->F) || !bf16_supported(p->F, p->H))
        return fail(MOE_ERR_UNSUPPORTED, "the backward needs H and F multiples of 128");
    if (p->T * p->k * 2 * p->F > INT32_MAX)
        return fail(MOE_ERR_UNSUPPORTED, "the backward needs T * k * 2F < 2^31");
    return MOE_OK;
}

}  // namespace
}  // namespace moe

MOE_API moe_status moe_backward_workspace_size(const moe_problem* p, size_t* bytes)
{
    if (bytes == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is null");
    if (moe_status st = check_backward(p); st != MOE_OK)
        return st;
    *bytes = backward_layout(p->T, p->H, p->F, p->E, p->k).total;
    return MOE_OK;
}

MOE_API moe_status moe_expert_backward(const moe_problem* p, const void* x, const void* w_gate,
                                       const void* w_up, const void* w_down,
                                       const int32_t* expert_ids, const float* probs,
                                       const void* dout, const void* saved_gu, void* dx,
                                       float* dw_gate, float* dw_up, float* dw_down, float* dprobs,
                                       void* ws, size_t ws_bytes, hipStream_t s)
{
    if (moe_status st = check_backward(p); st != MOE_OK)
        return st;
    const int64_t T = p->T, H = p->H, F = p->F, E = p->E, k = p->k, M = T * k;
    const BackwardLayout L = backward_layout(T, H, F, E, k);
    if (ws == nullptr || ws_bytes < L.total)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", L.total,
                    ws == nullptr ? size_t{0} : ws_bytes);
    if (w_gate == nullptr || w_up == nullptr || w_down == nullptr || dw_gate == nullptr ||
        dw_up == nullptr || dw_down == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "null weight or weight-gradient pointer");
    if (T > 0 && (x == nullptr || expert_ids == nullptr || probs == nullptr || dout == nullptr ||
                  dx == nullptr || dprobs == nullptr))
        return fail(MOE_ERR_INVALID_ARGUMENT, "null data pointer");
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* perm = at<int32_t>(ws, L.perm);
    int32_t* pos = at<int32_t>(ws, L.pos);
    if (moe_status st = run_route(expert_ids, T, k, E, counts, offsets, perm, pos, ws, L.route, s);
        st != MOE_OK)
        return st;
    // the weight-gradient kernels' task counters and zero rows (one contiguous region)
    LAUNCH(s, "zero_fill",
           launch_zero_i32(at<int32_t>(ws, L.wgrad_ctr),
                           static_cast<int64_t>((L.zero + kWgradZeroBytes - L.wgrad_ctr) / 4), s));
    const bool dma_ok = L.total < (size_t{1} << 32);       // zero rows within 32-bit copy offsets
    const uint16_t* zero = dma_ok ? at<uint16_t>(ws, L.zero) : nullptr;
    int32_t* wctr = at<int32_t>(ws, L.wgrad_ctr);
    const auto* wg = static_cast<const uint16_t*>(w_gate);
    const auto* wu = static_cast<const uint16_t*>(w_up);
    const auto* wd = static_cast<const uint16_t*>(w_down);
    uint16_t* x_perm = at<uint16_t>(ws, L.x_perm);
    uint16_t* dout_perm = at<uint16_t>(ws, L.dout_perm);
    uint16_t* dgu = at<uint16_t>(ws, L.dgu);
    uint16_t* hp = at<uint16_t>(ws, L.hp);
    if (M > 0) {
        int32_t* status = at<int32_t>(ws, L.route.status);
        int32_t* tcount = at<int32_t>(ws, L.tile_count);
        int32_t* task_ctr = at<int32_t>(ws, L.task_ctr);
        MTile* tiles_r = at<MTile>(ws, L.tiles_r);
        MTile* tiles_d = at<MTile>(ws, L.tiles_d);
        // g and u: as the forward saved them (same routing, so the same permuted rows), or recomputed
        const uint16_t* g = saved_gu != nullptr ? static_cast<const uint16_t*>(saved_gu) : at<uint16_t>(ws, L.g);
        const uint16_t* u = saved_gu != nullptr ? g + M * F : at<uint16_t>(ws, L.u);
        void* dx_rows = at<void>(ws, L.dx_perm);
        float* prow = at<float>(ws, L.prow);
        float* partial = at<float>(ws, L.partial);
        LAUNCH(s, "permute", launch_permute(x, pos, x_perm, T, k, M, H * 2, s));
        LAUNCH(s, "permute", launch_permute(dout, pos, dout_perm, T, k, M, H * 2, s));
        MTile* tiles_run = L.tiles_run != 0 ? at<MTile>(ws, L.tiles_run) : nullptr;
        LAUNCH(s, "build_tiles",
               launch_build_tiles(offsets, nullptr, E, E, M, M, L.bm_r, tiles_r, L.max_tiles_r,
                                  tcount, nullptr, nullptr, 1, 0, task_ctr, status, false, s, tiles_run,
                                  tiles_run != nullptr ? tcount + 4 : nullptr));
        if (L.tiles_d != L.tiles_r)
            LAUNCH(s, "build_tiles",
                   launch_build_tiles(offsets, nullptr, E, E, M, M, L.bm_d, tiles_d, L.max_tiles_d,
                                      tcount + 1, nullptr, nullptr, 1, 0, nullptr, status, false, s));
        const int32_t* tcount_d = L.tiles_d != L.tiles_r ? tcount + 1 : tcount;
        // 256-row dgrad tiles take the in-run table too: the tasks that share a weight strip then
        // run side by side and share it in the L2 (measured: Mixtral dgrad_down -3.5%, gate/up -5%)
        if (tiles_run != nullptr && L.tiles_d == L.tiles_r) {
            tiles_d = tiles_run;
            tcount_d = tcount + 4;
        }
        // g = x_perm Wg[e], u = x_perm Wu[e] (K = H, N = F): one launch of fc1's kernel, h not stored
        if (saved_gu == nullptr) {
            // the large-tile kernel reads each row from x through perm, as the forward's fc1 does:
            // a token's row then serves its k slots from the caches (x_perm is k times larger)
            const bool gather = L.bm_r == 256;
            LAUNCH(s, "recompute_gu",
                   launch_recompute_gu_bf16(gather ? static_cast<const uint16_t*>(x) : x_perm,
                                            gather ? perm : nullptr, static_cast<int>(k), wg, wu,
                                            at<uint16_t>(ws, L.g), at<uint16_t>(ws, L.u),
                                            tiles_run != nullptr ? tiles_run : tiles_r,
                                            tiles_run != nullptr ? tcount + 4 : tcount, H, F, task_ctr, s));
        }
        LAUNCH(s, "row_probs", launch_row_probs(perm, probs, prow, M, s));
        LAUNCH(s, "dgrad_down",
               launch_dgrad_down(dout_perm, wd, g, u, prow, dgu, hp, partial, tiles_d, tcount_d,
                                 L.max_tiles_d, M, H, F, wctr + 3 * kXcdCount, s));
        LAUNCH(s, "dprobs", launch_dprobs(partial, pos, dprobs, M, dprobs_partials(M, H, F), s));
        LAUNCH(s, "dgrad_gate_up",
               launch_dgrad_gate_up(dgu, wg, wu, dx_rows, tiles_d, tcount_d, L.max_tiles_d, M, H, F,
                                    wctr + 4 * kXcdCount, s));
        LAUNCH(s, "sum_slots",
               launch_sum_slot_rows(dx_rows, dgrad_gate_up_parts(M, H, F), pos,
                                    static_cast<uint16_t*>(dx), T, k, M, H, s));
    }
    // weight gradients (an expert without rows gets zeros)
    LAUNCH(s, "wgrad_down",
           launch_wgrad(hp, F, dout_perm, H, offsets, E, F, H, dw_down, zero, wctr, s));
    LAUNCH(s, "wgrad_gate",
           launch_wgrad(x_perm, H, dgu, 2 * F, offsets, E, H, F, dw_gate, zero, wctr + kXcdCount, s));
    LAUNCH(s, "wgrad_up",
           launch_wgrad(x_perm, H, dgu + F, 2 * F, offsets, E, H, F, dw_up, zero, wctr + 2 * kXcdCount, s));
    return MOE_OK;
}

MOE_API moe_status moe_route_workspace_size(int64_t T, int64_t k, int64_t E, size_t* bytes)
{
    if (bytes == nullptr || T < 0 || k <= 0 || E <= 0 || k > E)
        return fail(MOE_ERR_INVALID_ARGUMENT, "bad route sizes");
    if (E >= kMaxExperts)
        return fail(MOE_ERR_UNSUPPORTED, "E exceeds %d", kMaxExperts - 1);
    *bytes = route_layout(T, k, E, 0).total;
    return MOE_OK;
}

MOE_API moe_status moe_route(const int32_t* expert_ids, int64_t T, int64_t k, int64_t E,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                             void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    size_t need = 0;
    if (moe_status st = moe_route_workspace_size(T, k, E, &need); st != MOE_OK)
        return st;
    if (T * k > INT32_MAX)
        return fail(MOE_ERR_UNSUPPORTED, "T * k exceeds int32 indexing");
    if (workspace == nullptr || workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes", need);
    if (counts == nullptr || offsets == nullptr ||
        (T > 0 && (expert_ids == nullptr || perm == nullptr || pos == nullptr)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
    return run_route(expert_ids, T, k, E, counts, offsets, perm, pos, workspace,
                     route_layout(T, k, E, 0), stream);
}

MOE_API moe_status moe_permute(const moe_problem* p, const void* x, const uint8_t* x_scale,
                               const int32_t* pos, void* x_perm, uint8_t* x_perm_scale,
                               hipStream_t stream)
{
    if (moe_status st = check_problem(p, true, false); st != MOE_OK)
        return st;
    const int64_t M = p->T * p->k;
    if (M == 0)
        return MOE_OK;
    if (x == nullptr || pos == nullptr || x_perm == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
    const bool mx = p->dtype == MOE_MXFP8_E4M3;
    if (mx && (x_scale == nullptr || x_perm_scale == nullptr))
        return fail(MOE_ERR_INVALID_ARGUMENT, "MX permute needs both scale pointers");
    LAUNCH(stream, "permute",
           launch_permute(x, pos, x_perm, p->T, p->k, M, p->H * elem_bytes(p->dtype), stream));
    if (mx)
        LAUNCH(stream, "permute_scale",
               launch_permute(x_scale, pos, x_perm_scale, p->T, p->k, M, p->H / 32, stream));
    return MOE_OK;
}

MOE_API moe_status moe_unpermute(const moe_problem* p, const void* y_perm, const int32_t* pos,
                                 const float* probs, void* out, hipStream_t stream)
{
    if (moe_status st = check_problem(p, true, false); st != MOE_OK)
        return st;
    const int64_t M = p->T * p->k;
    if (p->T == 0)
        return MOE_OK;
    if (y_perm == nullptr || pos == nullptr || probs == nullptr || out == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
    LAUNCH(stream, "unpermute",
           launch_unpermute(p->dtype == MOE_F32 ? 0 : 1, y_perm, pos, probs, out, p->T, p->k, M,
                            p->H, stream));
    return MOE_OK;
}

MOE_API moe_status moe_grouped_ffn_workspace_size(const moe_problem* p, int64_t M, int64_t G,
                                                  size_t* bytes)
{
    if (bytes == nullptr || M < 0 || G <= 0 || M > INT32_MAX)
        return fail(MOE_ERR_INVALID_ARGUMENT, "bad grouped sizes");
    if (moe_status st = check_problem(p, false); st != MOE_OK)
        return st;
    if (p->dtype == MOE_MXFP8_E4M3 && M * std::max(p->H, p->F) > UINT32_MAX)
        return fail(MOE_ERR_UNSUPPORTED, "MX needs M * max(H, F) < 2^32");
    *bytes = ffn_layout(p->dtype, M, G, p->H, p->F, p->head_m_size, 0).total;
    return MOE_OK;
}

static moe_status grouped_common(const moe_problem* p, const void* rows, const uint8_t* rows_scale,
                                 int64_t M, const int32_t* group_offsets,
                                 const int32_t* group_expert, int64_t G, const void* wg,
                                 const uint8_t* wgs, const void* wu, const uint8_t* wus,
                                 const void* wd, const uint8_t* wds, void* y, void* ws,
                                 size_t ws_bytes, hipStream_t s)
{
    size_t need = 0;
    if (moe_status st = moe_grouped_ffn_workspace_size(p, M, G, &need); st != MOE_OK)
        return st;
    if (ws == nullptr || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes", need);
    if (group_offsets == nullptr || group_expert == nullptr ||
        (M > 0 && (rows == nullptr || wg == nullptr || wu == nullptr || wd == nullptr || y == nullptr)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
    const FfnLayout L = ffn_layout(p->dtype, M, G, p->H, p->F, p->head_m_size, 0);
    return run_ffn(p->dtype, rows, rows_scale, M, group_offsets, group_expert, G, p->E, p->H, p->F,
                   p->head_m_size, wg, wgs, wu, wus, wd, wds, y, ws, L, true, s);
}

MOE_API moe_status moe_grouped_ffn(const moe_problem* p, const void* rows, int64_t M,
                                   const int32_t* group_offsets, const int32_t* group_expert,
                                   int64_t G, const void* w_gate, const void* w_up,
                                   const void* w_down, void* y_rows, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream)
{
    if (p != nullptr && p->dtype == MOE_MXFP8_E4M3)
        return fail(MOE_ERR_INVALID_ARGUMENT, "MX rows go through moe_grouped_ffn_mx");
    return grouped_common(p, rows, nullptr, M, group_offsets, group_expert, G, w_gate, nullptr,
                          w_up, nullptr, w_down, nullptr, y_rows, workspace, workspace_bytes,
                          stream);
}

MOE_API moe_status moe_grouped_ffn_mx(const moe_problem* p, const uint8_t* rows,
                                      const uint8_t* rows_scale, int64_t M,
                                      const int32_t* group_offsets, const int32_t* group_expert,
                                      int64_t G, const uint8_t* w_gate, const uint8_t* wg_scale,
                                      const uint8_t* w_up, const uint8_t* wu_scale,
                                      const uint8_t* w_down, const uint8_t* wd_scale, void* y_rows,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (p == nullptr || p->dtype != MOE_MXFP8_E4M3)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_grouped_ffn_mx needs dtype MOE_MXFP8_E4M3");
    if (M > 0 && (rows_scale == nullptr || wg_scale == nullptr || wu_scale == nullptr ||
                  wd_scale == nullptr))
        return fail(MOE_ERR_INVALID_ARGUMENT, "null scale pointer");
    return grouped_common(p, rows, rows_scale, M, group_offsets, group_expert, G, w_gate, wg_scale,
                          w_up, wu_scale, w_down, wd_scale, y_rows, workspace, workspace_bytes,
                          stream);
}

MOE_API moe_status moe_mx_quantize(const float* v, int64_t rows, int64_t cols, uint8_t* codes,
                                   uint8_t* scales, hipStream_t stream)
{
    if (rows < 0 || cols <= 0 || cols % 32 != 0 || rows * cols > (int64_t{1} << 40))
        return fail(MOE_ERR_INVALID_ARGUMENT, "cols must be a positive multiple of 32");
    if (rows == 0)
        return MOE_OK;
    if (v == nullptr || codes == nullptr || scales == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
    LAUNCH(stream, "mx_quantize", launch_mx_quantize(v, rows, cols, codes, scales, stream));
    return MOE_OK;
}

MOE_API moe_status moe_mx_fc1_epilogue_encode(const float* v, int64_t rows, int64_t cols,
                                              int32_t large_tiles, uint8_t* codes, uint8_t* scales,
                                              hipStream_t stream)
{
    const int64_t bn = large_tiles ? 128 : 64;
    if (rows < 0 || cols <= 0 || cols % bn != 0 || rows * cols > (int64_t{1} << 28))
        return fail(MOE_ERR_INVALID_ARGUMENT,
                    "need rows >= 0, cols a positive multiple of %lld and rows * cols <= 2^28",
                    static_cast<long long>(bn));
    if (rows == 0)
        return MOE_OK;
    if (v == nullptr || codes == nullptr || scales == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
    LAUNCH(stream, "mx_epilogue_probe",
           launch_mx_epilogue_probe(v, rows, cols, large_tiles != 0, codes, scales, stream));
    return MOE_OK;
}

MOE_API moe_status moe_router_topk(const float* logits, int64_t T, int64_t E, int64_t k,
                                   int32_t* expert_ids, float* probs, hipStream_t stream)
{
    if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 64)
        return fail(MOE_ERR_INVALID_ARGUMENT, "need T >= 0, 1 <= E <= 1024, 1 <= k <= min(E, 64)");
    if (T * E > (int64_t{1} << 40))
        return fail(MOE_ERR_INVALID_ARGUMENT, "T * E too large");
    if (T == 0)
        return MOE_OK;
    if (logits == nullptr || expert_ids == nullptr || probs == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
    LAUNCH(stream, "router", launch_router(logits, T, E, k, expert_ids, probs, stream));
    return MOE_OK;
}

MOE_API moe_status moe_query_device_status(const void* workspace, hipStream_t stream,
                                           int32_t* status)
{
    if (workspace == nullptr || status == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return hip_fail(e, "hipStreamSynchronize");
    e = hipMemcpy(status, workspace, sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return hip_fail(e, "hipMemcpy");
    return MOE_OK;
}

MOE_API moe_status moe_chunk_counters(const moe_problem* p, void* workspace,
                                      size_t workspace_bytes, int64_t M,
                                      const int32_t** counters, const int32_t** tiles_per_chunk,
                                      int64_t* num_chunks)
{
    if (p == nullptr || workspace == nullptr || counters == nullptr || tiles_per_chunk == nullptr ||
        num_chunks == nullptr || M < 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
    if (p->head_m_size <= 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "counters exist only in chunked mode");
    // the counters sit at the start of both the forward and the grouped-FFN workspaces
    const FfnLayout L = ffn_layout(p->dtype, M, 1, p->H, p->F, p->head_m_size, 0);
    if (workspace_bytes < L.chunk_tiles + sizeof(int32_t) * static_cast<size_t>(L.num_chunks))
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
    *counters = at<const int32_t>(workspace, L.chunk_done);
    *tiles_per_chunk = at<const int32_t>(workspace, L.chunk_tiles);
    *num_chunks = L.num_chunks;
    return MOE_OK;
}

MOE_API moe_status moe_quantized_x_offsets(const moe_problem* p, size_t* codes_offset,
                                           size_t* scales_offset, int32_t* permuted)
{
    if (codes_offset == nullptr || scales_offset == nullptr || permuted == nullptr)
        return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
    if (moe_status st = check_problem(p, true); st != MOE_OK)
        return st;
    if ((p->flags & MOE_FLAG_QUANTIZE_X) == 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "the problem does not set MOE_FLAG_QUANTIZE_X");
    const ForwardLayout L = forward_layout(p->dtype, p->T, p->H, p->F, p->E, p->k, p->head_m_size, true);
    const bool fused = (p->flags & MOE_FLAG_SEPARATE_PERMUTE) == 0 && fc1_gathers(p->dtype, p->T, p->H, p->F);
    *codes_offset = fused ? L.x_q : L.x_perm;
    *scales_offset = fused ? L.x_q_scale : L.x_perm_scale;
    *permuted = fused ? 0 : 1;
    return MOE_OK;
}

MOE_API moe_status moe_intermediate_offsets(const moe_problem* p, int64_t M, int64_t G,
                                            size_t* h_offset, size_t* h_scale_offset)
{
    if (h_offset == nullptr || h_scale_offset == nullptr || M < 0 || G <= 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "bad arguments");
    if (moe_status st = check_problem(p, false); st != MOE_OK)
        return st;
    // the FFN block (and with it h) starts at the workspace base in both layouts
    const FfnLayout L = ffn_layout(p->dtype, M, G, p->H, p->F, p->head_m_size, 0);
    *h_offset = L.h;
    *h_scale_offset = L.h_scale;
    return MOE_OK;
}

MOE_API const char* moe_status_string(moe_status s)
{
    switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_EXPERT_ID_OUT_OF_RANGE: return "MOE_ERR_EXPERT_ID_OUT_OF_RANGE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "unknown moe_status";
}

MOE_API const char* moe_last_error(void) { return g_last_error.c_str(); }

MOE_API moe_status moe_timing_enable(int enable)
{
    Timing& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    t.enabled = enable != 0;
    return MOE_OK;
}

MOE_API moe_status moe_timing_collect(const char** names, double* total_ms, int64_t* launches,
                                      int capacity, int* count)
{
    Timing& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    for (TimingRec& r : t.pending) {
        float ms = 0.0f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess)
            return hip_fail(e, "timing events");
        auto it = t.totals.find(r.name);
        if (it == t.totals.end())
            it = t.totals.emplace(r.name, Timing::Total{r.name, 0.0, 0}).first;
        it->second.ms += ms;
        it->second.n += 1;
        t.pool.push_back(r.a);
        t.pool.push_back(r.b);
    }
    t.pending.clear();
    int n = 0;
    for (auto& kv : t.totals) {
        if (n < capacity) {
            if (names)
                names[n] = kv.second.name;
            if (total_ms)
                total_ms[n] = kv.second.ms;
            if (launches)
                launches[n] = kv.second.n;
        }
        ++n;
    }
    if (count)
        *count = n;
    return MOE_OK;
}

MOE_API moe_status moe_timing_reset(void)
{
    Timing& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    for (TimingRec& r : t.pending) {
        (void)hipEventSynchronize(r.b);           // the events are recycled either way
        t.pool.push_back(r.a);
        t.pool.push_back(r.b);
    }
    t.pending.clear();
    t.totals.clear();
    return MOE_OK;
}

// ------------------------------------------------------------------- allocation-free routing

namespace moe {
namespace {

// The route's scratch (status word, then per-block expert histograms) for callers that cannot
// allocate: a file-scope device array, one copy per GPU, kept until the process ends.
constexpr size_t kNoAllocScratchBytes = kAlign + (size_t{4} << 20);

}  // namespace
}  // namespace moe

static __device__ __align__(256) unsigned char scratch[moe::kNoAllocScratchBytes];

namespace moe {
namespace {

// Device address of this GPU's copy of `scratch`.  In host code the array's name is a host-side
// stand-in, not a device address, so the address is looked up once per device (with that device
// current) and only the looked-up pointer is ever handed to kernels.
moe_status noalloc_scratch(void** out)
{
    static std::mutex mu;
    static std::map<int, void*> ptrs;
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> g(mu);
    auto it = ptrs.find(dev);
    if (it == ptrs.end()) {
        void* p = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress(scratch)");
        it = ptrs.emplace(dev, p).first;
    }
    *out = it->second;
    return MOE_OK;
}

}  // namespace
}  // namespace moe

MOE_API moe_status moe_route_noalloc(const int32_t* expert_ids, int64_t T, int64_t k, int64_t E,
                                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                                     hipStream_t stream)
{
    size_t need = 0;
    if (moe_status st = moe_route_workspace_size(T, k, E, &need); st != MOE_OK)
        return st;
    if (T * k > INT32_MAX)
        return fail(MOE_ERR_UNSUPPORTED, "T * k exceeds int32 indexing");
    if (need > kNoAllocScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED,
                    "ceil(T*k / %d) * (E + 1) block counts need %zu bytes; the static scratch holds %zu",
                    kRouteSlotsPerBlock, need, kNoAllocScratchBytes);
    if (counts == nullptr || offsets == nullptr ||
        (T > 0 && (expert_ids == nullptr || perm == nullptr || pos == nullptr)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer");
    void* ws = nullptr;
    if (moe_status st = noalloc_scratch(&ws); st != MOE_OK)
        return st;
    // every scratch byte the kernels read is written earlier in the same call (route_count fills
    // each block's histogram row, route_scan the status word): nothing needs clearing
    return run_route(expert_ids, T, k, E, counts, offsets, perm, pos, ws, route_layout(T, k, E, 0),
                     stream);
}

#ifdef MOE_PHASE_PROBE
// ------------------------------------------------------------------------------------ probe build

#include "moe_expert_layer_probe.h"

static_assert(MOE_PROBE_FIELDS == moe::kProbeFields &&
                  MOE_PROBE_KINDS == moe::kProbeKindsBf16 + moe::kProbeKindsBwd + moe::kProbeKindsMx,
              "probe layout");

MOE_API int moe_probe_phases(unsigned long long* out, int reset)
{
    // the launches already enqueued are the ones counted
    if (hipDeviceSynchronize() != hipSuccess)
        return 1;
    if (moe::probe_read_bf16(out, reset) != 0)
        return 1;
    if (moe::probe_read_bwd(out != nullptr ? out + moe::kProbeKindsBf16 * moe::kProbeFields : nullptr,
                            reset) != 0)
        return 1;
    if (moe::probe_read_mx(out != nullptr
                               ? out + (moe::kProbeKindsBf16 + moe::kProbeKindsBwd) * moe::kProbeFields
                               : nullptr,
                           reset) != 0)
        return 1;
    return hipDeviceSynchronize() != hipSuccess;
}
#endif
