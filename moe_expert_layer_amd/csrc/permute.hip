// Permute and unpermute for the MoE expert layer on gfx950 (HBM-bound data movement).
//
// permute   ("NPU Training Operators - MC2", 执行路径 step 6): x_perm[pos[s]] = x[s / k].
//           Written as a scatter over tokens: each token row is read once and stored to its k
//           permuted rows, so HBM traffic is exactly (1 + k) row transfers per token.
// unpermute (step 10): out[t] = sum_j probs[t, j] * y_perm[pos[t*k + j]], j ascending, fp32
//           fused multiply-add from 0 and one rounding; a gather, so no atomics and a
//           deterministic result.
// Both move 16-byte vectors.  The flat kernels give every (token, 16-byte column) pair its own
// thread, so a launch keeps as many independent loads in flight as the machine can hold; rows are
// contiguous in the thread index, so every access is coalesced.  Grid-stride versions cover sizes
// whose pair count does not fit 32 bits.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// 16-byte load marked non-temporal: the permute's x rows and the unpermute's y_perm rows are read
// once, and keeping them out of the caches' way took both kernels from 60% / 57% to 64% of the
// HBM bandwidth (100 MB Mixtral-shaped launches, timed back to back).
__device__ __forceinline__ uint4 nt_load(const uint4* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <typename V>
__global__ __launch_bounds__(kThreads) void permute_kernel(const V* __restrict__ x,
                                                           const int32_t* __restrict__ pos,
                                                           V* __restrict__ x_perm, int64_t T,
                                                           int k, int64_t M, int64_t row_vecs)
{
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const V* src = x + t * row_vecs;
        const int32_t* tp = pos + t * k;
        for (int64_t c = threadIdx.x; c < row_vecs; c += kThreads) {
            const V v = src[c];
            for (int j = 0; j < k; ++j) {
                const int64_t p = tp[j];
                if (p >= 0 && p < M)
                    x_perm[p * row_vecs + c] = v;
            }
        }
    }
}

// kVpt consecutive groups of kThreads (token, 16-byte column) pairs per workgroup, each thread one
// pair of each group: total = T * row_vecs < 2^31.  The kVpt rows are loaded before any is stored.
template <typename V, int kVpt>
__global__ __launch_bounds__(kThreads) void permute_flat_kernel(const V* __restrict__ x,
                                                                const int32_t* __restrict__ pos,
                                                                V* __restrict__ x_perm, int k,
                                                                int64_t M, uint32_t row_vecs,
                                                                uint32_t total)
{
    const uint32_t i0 = blockIdx.x * (kThreads * kVpt) + threadIdx.x;
    V v[kVpt];
#pragma unroll
    for (int q = 0; q < kVpt; ++q) {
        const uint32_t i = i0 + q * kThreads;
        if (i < total)
            v[q] = nt_load(x + i);
    }
#pragma unroll
    for (int q = 0; q < kVpt; ++q) {
        const uint32_t i = i0 + q * kThreads;
        if (i >= total)
            break;
        const uint32_t t = i / row_vecs;
        const uint32_t c = i - t * row_vecs;
        const int32_t* tp = pos + static_cast<int64_t>(t) * k;
        for (int j = 0; j < k; ++j) {
            const int64_t p = tp[j];
            if (p >= 0 && p < M)
                x_perm[p * row_vecs + c] = v[q];
        }
    }
}

__device__ __forceinline__ void fma_bf16x8(float (&acc)[8], float w, const uint4& v)
{
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(w, __uint_as_float(d[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(w, __uint_as_float(d[i] & 0xffff0000u), acc[2 * i + 1]);
    }
}

// One thread per (token, 16-byte column) of the output.  The k rows are loaded before any is used
// (k <= 8 in one batch), then summed in j order.
__global__ __launch_bounds__(kThreads) void unpermute_bf16_flat_kernel(
    const uint4* __restrict__ y, const int32_t* __restrict__ pos, const float* __restrict__ probs,
    uint4* __restrict__ out, int k, int64_t M, uint32_t row_vecs, uint32_t total)
{
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= total)
        return;
    const uint32_t t = i / row_vecs;
    const uint32_t c = i - t * row_vecs;
    const int32_t* tp = pos + static_cast<int64_t>(t) * k;
    const float* pp = probs + static_cast<int64_t>(t) * k;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += 8) {
        uint4 v[8];
        float w[8];
        bool ok[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t p = j0 + j < k ? tp[j0 + j] : -1;
            ok[j] = p >= 0 && p < M;
            w[j] = ok[j] ? pp[j0 + j] : 0.0f;
            v[j] = ok[j] ? nt_load(y + p * row_vecs + c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (ok[j])
                fma_bf16x8(acc, w[j], v[j]);
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    out[i] = o;
}

// One workgroup per output row t: the row's k slot rows and weights are the same for every lane
// (scalar loads); each lane takes the 16-byte columns c = lane, lane + kThreads, ... of the row and
// issues the k loads of a column (at most 8 per batch) before using any, then sums them in j order.
__global__ __launch_bounds__(kThreads) void unpermute_bf16_row_kernel(
    const uint4* __restrict__ y, const int32_t* __restrict__ pos, const float* __restrict__ probs,
    uint4* __restrict__ out, int k, int64_t M, int row_vecs)
{
    const int64_t t = blockIdx.x;
    const int32_t* tp = pos + t * k;
    const float* pp = probs + t * k;
    for (int c = threadIdx.x; c < row_vecs; c += kThreads) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += 8) {
            uint4 v[8];
            float w[8];
            bool ok[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t p = j0 + j < k ? tp[j0 + j] : -1;
                ok[j] = p >= 0 && p < M;
                w[j] = ok[j] ? pp[j0 + j] : 0.0f;
                v[j] = ok[j] ? nt_load(y + p * row_vecs + c) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (ok[j])
                    fma_bf16x8(acc, w[j], v[j]);
        }
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        out[t * row_vecs + c] = o;
    }
}

// Grid-stride over output rows, one workgroup per row at a time: the row's k slot indices and weights
// are scalar loads; each lane takes kCols 16-byte columns c, c + kThreads, ... and issues their loads
// (at most 4 slots per batch) before using any, then sums them in j order.
template <int kCols>
__global__ __launch_bounds__(kThreads) void unpermute_bf16_rows_gs_kernel(
    const uint4* __restrict__ y, const int32_t* __restrict__ pos, const float* __restrict__ probs,
    uint4* __restrict__ out, int64_t T, int k, int64_t M, int row_vecs)
{
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const int32_t* tp = pos + t * k;
        const float* pp = probs + t * k;
        for (int c0 = threadIdx.x; c0 < row_vecs; c0 += kThreads * kCols) {
            float acc[kCols][8];
#pragma unroll
            for (int q = 0; q < kCols; ++q)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[q][e] = 0.0f;
            for (int j0 = 0; j0 < k; j0 += 4) {
                uint4 v[4][kCols];
                float w[4];
                bool ok[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t p = j0 + j < k ? tp[j0 + j] : -1;
                    ok[j] = p >= 0 && p < M;
                    w[j] = ok[j] ? pp[j0 + j] : 0.0f;
#pragma unroll
                    for (int q = 0; q < kCols; ++q) {
                        const int c = c0 + q * kThreads;
                        v[j][q] = ok[j] && c < row_vecs ? nt_load(y + p * row_vecs + c) : make_uint4(0, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (ok[j])
#pragma unroll
                        for (int q = 0; q < kCols; ++q)
                            fma_bf16x8(acc[q], w[j], v[j][q]);
            }
#pragma unroll
            for (int q = 0; q < kCols; ++q) {
                const int c = c0 + q * kThreads;
                if (c < row_vecs) {
                    uint4 o;
                    o.x = pack_bf16x2(acc[q][0], acc[q][1]);
                    o.y = pack_bf16x2(acc[q][2], acc[q][3]);
                    o.z = pack_bf16x2(acc[q][4], acc[q][5]);
                    o.w = pack_bf16x2(acc[q][6], acc[q][7]);
                    out[t * row_vecs + c] = o;
                }
            }
        }
    }
}

// bfloat16 rows: 8 values per 16-byte vector.
__global__ __launch_bounds__(kThreads) void unpermute_bf16_kernel(
    const uint4* __restrict__ y, const int32_t* __restrict__ pos, const float* __restrict__ probs,
    uint4* __restrict__ out, int64_t T, int k, int64_t M, int64_t row_vecs)
{
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const int32_t* tp = pos + t * k;
        const float* pp = probs + t * k;
        for (int64_t c = threadIdx.x; c < row_vecs; c += kThreads) {
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = 0.0f;
            for (int j = 0; j < k; ++j) {
                const int64_t p = tp[j];
                if (p < 0 || p >= M)
                    continue;
                const float w = pp[j];
                const uint4 v = y[p * row_vecs + c];
                const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = fmaf(w, __uint_as_float(d[i] << 16), acc[2 * i]);
                    acc[2 * i + 1] = fmaf(w, __uint_as_float(d[i] & 0xffff0000u), acc[2 * i + 1]);
                }
            }
            uint4 o;
            o.x = pack_bf16x2(acc[0], acc[1]);
            o.y = pack_bf16x2(acc[2], acc[3]);
            o.z = pack_bf16x2(acc[4], acc[5]);
            o.w = pack_bf16x2(acc[6], acc[7]);
            out[t * row_vecs + c] = o;
        }
    }
}

// float32 rows: 4 values per 16-byte vector.
__global__ __launch_bounds__(kThreads) void unpermute_f32_kernel(
    const float4* __restrict__ y, const int32_t* __restrict__ pos, const float* __restrict__ probs,
    float4* __restrict__ out, int64_t T, int k, int64_t M, int64_t row_vecs)
{
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        const int32_t* tp = pos + t * k;
        const float* pp = probs + t * k;
        for (int64_t c = threadIdx.x; c < row_vecs; c += kThreads) {
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int j = 0; j < k; ++j) {
                const int64_t p = tp[j];
                if (p < 0 || p >= M)
                    continue;
                const float w = pp[j];
                const float4 v = y[p * row_vecs + c];
                acc.x = fmaf(w, v.x, acc.x);
                acc.y = fmaf(w, v.y, acc.y);
                acc.z = fmaf(w, v.z, acc.z);
                acc.w = fmaf(w, v.w, acc.w);
            }
            out[t * row_vecs + c] = acc;
        }
    }
}

unsigned grid_for_rows(int64_t rows)
{
    const int64_t cap = static_cast<int64_t>(device_info().cu_count) * 16;
    return static_cast<unsigned>(rows < cap ? (rows > 0 ? rows : 1) : cap);
}

}  // namespace

hipError_t launch_permute(const void* x, const int32_t* pos, void* x_perm, int64_t T, int64_t k,
                          int64_t M, int64_t row_bytes, hipStream_t s)
{
    const dim3 block(kThreads);
    if (row_bytes % 16 == 0 && T * (row_bytes / 16) < (int64_t{1} << 31)) {
        const uint32_t total = static_cast<uint32_t>(T * (row_bytes / 16));
        const uint32_t row_vecs = static_cast<uint32_t>(row_bytes / 16);
        // Four rows' worth of loads in flight per thread where a workgroup's 1024 vectors cover
        // whole rows (or a row whole workgroups): Mixtral-shaped rows 64% -> 73% of HBM bandwidth,
        // 4096-byte rows 66% -> 68%; with rows that straddle workgroups (7168-byte MX rows) one
        // vector per thread stays faster (67% against 62%).
        constexpr uint32_t kSpan = kThreads * 4;
        if (row_vecs > 0 && (kSpan % row_vecs == 0 || row_vecs % kSpan == 0))
            permute_flat_kernel<uint4, 4><<<dim3((total + kSpan - 1) / kSpan), block, 0, s>>>(
                static_cast<const uint4*>(x), pos, static_cast<uint4*>(x_perm), static_cast<int>(k), M,
                row_vecs, total);
        else
            permute_flat_kernel<uint4, 1><<<dim3((total + kThreads - 1) / kThreads), block, 0, s>>>(
                static_cast<const uint4*>(x), pos, static_cast<uint4*>(x_perm), static_cast<int>(k), M,
                row_vecs, total);
        return hipGetLastError();
    }
    const dim3 grid(grid_for_rows(T));
    if (row_bytes % 16 == 0)
        permute_kernel<uint4><<<grid, block, 0, s>>>(static_cast<const uint4*>(x), pos,
                                                      static_cast<uint4*>(x_perm), T,
                                                      static_cast<int>(k), M, row_bytes / 16);
    else if (row_bytes % 4 == 0)
        permute_kernel<uint32_t><<<grid, block, 0, s>>>(static_cast<const uint32_t*>(x), pos,
                                                          static_cast<uint32_t*>(x_perm), T,
                                                          static_cast<int>(k), M, row_bytes / 4);
    else
        permute_kernel<uint8_t><<<grid, block, 0, s>>>(static_cast<const uint8_t*>(x), pos,
                                                        static_cast<uint8_t*>(x_perm), T,
                                                        static_cast<int>(k), M, row_bytes);
    return hipGetLastError();
}

// dtype: 0 float32 rows (H % 4 == 0), otherwise bfloat16 rows (H % 8 == 0).
hipError_t launch_unpermute(int dtype, const void* y_perm, const int32_t* pos, const float* probs,
                            void* out, int64_t T, int64_t k, int64_t M, int64_t H, hipStream_t s)
{
    const dim3 grid(grid_for_rows(T)), block(kThreads);
    if (dtype != 0 && T * (H / 8) < (int64_t{1} << 31)) {
        const uint32_t total = static_cast<uint32_t>(T * (H / 8));
        // k >= 8: one workgroup per row, the k slot indices and weights read once per workgroup
        // (fine-grained k = 8: 68% -> 71% of HBM bandwidth); k <= 2: the same over a grid-stride
        // loop of 4 workgroups per CU, two columns per lane (Mixtral-shaped 64% -> 65%, 25 -> 23 us
        // inside the layer); k = 4: the flat kernel (MX-shaped 73% against 67% for either)
        if (k <= 2 && T <= 0x7fffffff)
            unpermute_bf16_rows_gs_kernel<2><<<dim3(static_cast<unsigned>(
                                                    std::min<int64_t>(T, int64_t{device_info().cu_count} * 4))),
                                                block, 0, s>>>(
                static_cast<const uint4*>(y_perm), pos, probs, static_cast<uint4*>(out), T,
                static_cast<int>(k), M, static_cast<int>(H / 8));
        else if (k >= 8 && T <= 0x7fffffff)
            unpermute_bf16_row_kernel<<<dim3(static_cast<unsigned>(T)), block, 0, s>>>(
                static_cast<const uint4*>(y_perm), pos, probs, static_cast<uint4*>(out),
                static_cast<int>(k), M, static_cast<int>(H / 8));
        else
            unpermute_bf16_flat_kernel<<<dim3((total + kThreads - 1) / kThreads), block, 0, s>>>(
                static_cast<const uint4*>(y_perm), pos, probs, static_cast<uint4*>(out),
                static_cast<int>(k), M, static_cast<uint32_t>(H / 8), total);
        return hipGetLastError();
    }
    if (dtype == 0)
        unpermute_f32_kernel<<<grid, block, 0, s>>>(static_cast<const float4*>(y_perm), pos, probs,
                                                     static_cast<float4*>(out), T,
                                                     static_cast<int>(k), M, H / 4);
    else
        unpermute_bf16_kernel<<<grid, block, 0, s>>>(static_cast<const uint4*>(y_perm), pos,
                                                      probs, static_cast<uint4*>(out), T,
                                                      static_cast<int>(k), M, H / 8);
    return hipGetLastError();
}

}  // namespace moe
