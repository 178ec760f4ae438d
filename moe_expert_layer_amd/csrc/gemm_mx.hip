// OCP-MX (E4M3 elements, E8M0 block scales, blocks of 32) pieces of the MoE expert layer on gfx950.
// The MX format is the reference MC2 matmul's ("MC2 通算融合架构总览", §1: AllToAll + MX-FP8
// quantised matmul); the encoder follows OCP Microscaling Formats v1.0.
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// One thread per 32-element block: shared exponent from the block's largest magnitude, then each
// element encoded with it.  Integer arithmetic on the float bits throughout.
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(const float* __restrict__ v,
                                                               int64_t nblocks,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales)
{
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < nblocks;
         b += static_cast<int64_t>(gridDim.x) * kThreads) {
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(v + b * 32);
        f32x4_t x[8];
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = src[i];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                amax = max(amax, __float_as_uint(x[i][j]) & 0x7fffffffu);
        }
        const int e = mx_shared_exponent(amax);
        u32x4_t out[2];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const uint32_t word = e4m3_encode_scaled(x[w][0], e) | (e4m3_encode_scaled(x[w][1], e) << 8) |
                                  (e4m3_encode_scaled(x[w][2], e) << 16) |
                                  (e4m3_encode_scaled(x[w][3], e) << 24);
            out[w / 4][w % 4] = word;
        }
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + b * 32);
        dst[0] = out[0];
        dst[1] = out[1];
        scales[b] = static_cast<uint8_t>(e + 127);
    }
}

}  // namespace

hipError_t launch_mx_quantize(const float* v, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t s)
{
    const int64_t nblocks = rows * (cols / 32);
    const int64_t want = (nblocks + kThreads - 1) / kThreads;
    const int64_t cap = static_cast<int64_t>(device_info().cu_count) * 8;
    mx_quantize_kernel<<<dim3(static_cast<unsigned>(want < cap ? (want > 0 ? want : 1) : cap)),
                         dim3(kThreads), 0, s>>>(v, nblocks, codes, scales);
    return hipGetLastError();
}

}  // namespace moe
