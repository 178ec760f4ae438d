// float32 grouped GEMMs for the MoE expert layer (steps 7-9 of "NPU Training Operators - MC2",
// 执行路径).  Plain fused multiply-add with float32 accumulation: this path serves small float32
// problems where launch latency, not arithmetic, sets the time.
//
// Work items are (row tile, 256-column strip): each thread owns one output column of the strip and
// walks the tile's rows, reading B down its column (coalesced across the workgroup) and the A row
// as a broadcast.  Sums run over the contraction index in ascending order.
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <bool kGated>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ B0, const float* __restrict__ B1,
    float* __restrict__ C, const MTile* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    int K, int N, int32_t* __restrict__ chunk_done)
{
    const int n_mt = *tile_count;
    const int n_ct = (N + kThreads - 1) / kThreads;
    for (int task = blockIdx.x; task < n_mt * n_ct; task += gridDim.x) {
        const MTile tile = tiles[task % n_mt];
        const int col = (task / n_mt) * kThreads + threadIdx.x;
        if (col < N) {
            const float* b0 = B0 + static_cast<int64_t>(tile.expert) * K * N + col;
            const float* b1 = kGated ? B1 + static_cast<int64_t>(tile.expert) * K * N + col : nullptr;
            for (int r = tile.row_begin; r < tile.row_end; ++r) {
                const float* a = A + static_cast<int64_t>(r) * K;
                float g = 0.0f, u = 0.0f;
                for (int kk = 0; kk < K; ++kk) {
                    const float av = a[kk];
                    g = fmaf(av, b0[static_cast<int64_t>(kk) * N], g);
                    if (kGated)
                        u = fmaf(av, b1[static_cast<int64_t>(kk) * N], u);
                }
                C[static_cast<int64_t>(r) * N + col] = kGated ? swiglu(g, u) : g;
            }
        }
        if (chunk_done != nullptr) {
            __threadfence();
            __syncthreads();
            // whole first wave (lane 0 adds 1): no lane-divergent region in this barrier loop
            if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0)
                atomicAdd(&chunk_done[tile.chunk], (threadIdx.x & 63) == 0 ? 1 : 0);
        }
    }
}

unsigned grid_for(int64_t max_tasks)
{
    const int64_t cap = static_cast<int64_t>(device_info().cu_count) * 4;
    return static_cast<unsigned>(max_tasks < cap ? (max_tasks > 0 ? max_tasks : 1) : cap);
}

}  // namespace

hipError_t launch_fc1_f32(const float* A, const float* wg, const float* wu, float* h,
                          const MTile* tiles, const int32_t* tile_count, int64_t H, int64_t F,
                          hipStream_t s)
{
    gemm_f32_kernel<true><<<dim3(grid_for(1 << 20)), dim3(kThreads), 0, s>>>(
        A, wg, wu, h, tiles, tile_count, static_cast<int>(H), static_cast<int>(F), nullptr);
    return hipGetLastError();
}

hipError_t launch_fc2_f32(const float* h, const float* wd, float* y, const MTile* tiles,
                          const int32_t* tile_count, int64_t H, int64_t F, int32_t* chunk_done,
                          hipStream_t s)
{
    gemm_f32_kernel<false><<<dim3(grid_for(1 << 20)), dim3(kThreads), 0, s>>>(
        h, wd, nullptr, y, tiles, tile_count, static_cast<int>(F), static_cast<int>(H),
        chunk_done);
    return hipGetLastError();
}

}  // namespace moe
