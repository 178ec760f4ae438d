// Router in front of the expert path: the gate's top-k over float32 logits.  The gate is the first
// step of the step breakdown on the page "MC2 通算融合"; the router top-k distribution is one of
// the checks listed on the page "NPU Training Operators - MC2" (验证项).  Reading: the k largest
// logits in descending order, ties to the lower expert id; each selected expert's probability is
// the softmax over the k selected logits (the softmax over all E renormalised over the k).
//
// A group of L lanes (L = 8, 16, 32 or 64, at least E or 64) serves one token, so a wave routes
// 64 / L tokens; lane l of a group holds logits l, l + L, ...  Each candidate is one 64-bit key:
// the logit's bits mapped to an unsigned integer of the same order, above the complement of the
// expert id, so the largest key is the largest logit and, among equal logits, the lowest id.  k
// rounds of a butterfly maximum over the group's untaken keys (lane j keeping round j's winner),
// then exp(l_j - l_max) and their butterfly sum (identical on every lane), and one division.
#include <climits>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Order-preserving map of a non-NaN float to uint32 (negative values reversed below positive).
__device__ __forceinline__ uint32_t ordered(float f)
{
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t key_of(float v, int id)
{
    return (static_cast<uint64_t>(ordered(v)) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(id));
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int off)
{
    const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(static_cast<uint32_t>(v)), off));
    const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(static_cast<uint32_t>(v >> 32)), off));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <int L, int kPer>
__global__ __launch_bounds__(kThreads) void router_kernel(const float* __restrict__ logits, int64_t T,
                                                         int E, int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ probs)
{
    const int lane = threadIdx.x & 63;
    const int g = lane & (L - 1);                             // lane inside the token's group
    const int64_t t = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / L;
    const bool live = t < T;
    const float* row = logits + (live ? t : 0) * E;
    float v[kPer];
    uint64_t key[kPer];                                       // 0: taken, or no expert
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = g + L * i;
        v[i] = (live && e < E ? row[e] : 0.0f) + 0.0f;      // -0 becomes +0: equal logits tie
        key[i] = live && e < E ? key_of(v[i], e) : 0;       // 0: below every real key
    }
    int my_id = 0;
    float my_logit = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            best = key[i] > best ? key[i] : best;
#pragma unroll
        for (int off = L / 2; off >= 1; off >>= 1) {
            const uint64_t o = shfl_xor64(best, off);
            best = o > best ? o : best;
        }
        const int id = static_cast<int>(~static_cast<uint32_t>(best));
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (g + L * i == id)
                key[i] = 0;                                   // taken
        // the winner's logit, from its ordered bits
        const uint32_t ob = static_cast<uint32_t>(best >> 32);
        const float wv = __uint_as_float((ob & 0x80000000u) ? (ob & 0x7fffffffu) : ~ob);
        if (g == j) {
            my_id = id;
            my_logit = wv;
        }
    }
    const float lmax = __shfl(my_logit, lane & ~(L - 1));    // round 0 of this group
    const float ex = g < k ? expf(my_logit - lmax) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1)
        sum += __shfl_xor(sum, off);
    if (live && g < k) {
        ids[t * k + g] = my_id;
        probs[t * k + g] = ex / sum;
    }
}

template <int L, int kPer>
hipError_t launch_router_n(const float* logits, int64_t T, int E, int k, int32_t* ids, float* probs,
                           hipStream_t s)
{
    const int64_t blocks = (T * L + kThreads - 1) / kThreads;
    if (blocks >= (int64_t{1} << 31))
        return hipErrorInvalidValue;
    router_kernel<L, kPer><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s>>>(
        logits, T, E, k, ids, probs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* ids,
                         float* probs, hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    const int e = static_cast<int>(E), kk = static_cast<int>(k);
    if (E <= 8)
        return launch_router_n<8, 1>(logits, T, e, kk, ids, probs, s);
    if (E <= 16)
        return launch_router_n<16, 1>(logits, T, e, kk, ids, probs, s);
    if (E <= 32)
        return launch_router_n<32, 1>(logits, T, e, kk, ids, probs, s);
    if (E <= 64)
        return launch_router_n<64, 1>(logits, T, e, kk, ids, probs, s);
    if (E <= 128)
        return launch_router_n<64, 2>(logits, T, e, kk, ids, probs, s);
    if (E <= 256)
        return launch_router_n<64, 4>(logits, T, e, kk, ids, probs, s);
    if (E <= 512)
        return launch_router_n<64, 8>(logits, T, e, kk, ids, probs, s);
    return launch_router_n<64, 16>(logits, T, e, kk, ids, probs, s);
}

}  // namespace moe
