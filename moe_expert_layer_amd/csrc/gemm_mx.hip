// OCP-MX (E4M3 elements, E8M0 block scales, blocks of 32) grouped GEMMs of the MoE expert layer on
// gfx950.  The MX format is the reference MC2 matmul's ("MC2 通算融合架构总览", §1: AllToAll + MX-FP8
// quantised matmul; §5: per-row scale buffers); the encoder follows OCP Microscaling Formats v1.0.
//
//   fc1:  h = MX-encode(swiglu(A Wg[e], A Wu[e]))   A = permuted x codes [M, H] + scales [M, H/32]
//   fc2:  y = h Wd[e]                               y bfloat16 [M, H]
// Products run on v_mfma_scale_f32_32x32x64_f8f6f4 with fp32 accumulation: each lane supplies one
// E8M0 byte for its (row, 32-element K block), and the hardware applies 2^(s-127) to each operand.
// Operand layout of that instruction (measured): lane l covers row / column l % 32; of its 32 bytes,
// bytes 0-15 are K block 0 and bytes 16-31 K block 1, lane half h = l / 32 holding elements
// 16h .. 16h+15 of each block; lane l's scale byte belongs to K block l / 32 of its row / column.
//
// Structure mirrors the bf16 kernel: persistent workgroups over (row tile, column tile) tasks, A
// rows staged to LDS as loaded, weights ([K, N], N contiguous) transposed byte-wise in registers
// into K-contiguous LDS rows, two LDS stages, XOR-swizzled 16-byte chunks.  The fc1 epilogue stages
// the fp32 SwiGLU tile in LDS so each lane owns one (row, 32-column block), finds its amax, and
// writes 32 E4M3 bytes plus one scale byte with the same integer encoder as the standalone kernel.
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;

// ----------------------------------------------------------------------------------- standalone encoder

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
        for (int w = 0; w < 8; ++w)
            out[w / 4][w % 4] = e4m3_encode_scaled(x[w][0], e) |
                                (e4m3_encode_scaled(x[w][1], e) << 8) |
                                (e4m3_encode_scaled(x[w][2], e) << 16) |
                                (e4m3_encode_scaled(x[w][3], e) << 24);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + b * 32);
        dst[0] = out[0];
        dst[1] = out[1];
        scales[b] = static_cast<uint8_t>(e + 127);
    }
}

// ----------------------------------------------------------------------------------- grouped GEMM

constexpr int BM = kBmMx;          // 128 rows per task
constexpr int BNB = 128;           // weight columns staged per task
constexpr int BK = 128;            // K elements (bytes) per step
constexpr int kWM = 2, kWN = 2;    // 4 waves, each 64 rows x 64 staged columns
constexpr int kTM = 2, kTN = 2;
constexpr int kABytes = BM * BK;
constexpr int kBBytes = BNB * BK;
constexpr int kAScBytes = BM * (BK / 32);        // [BM][4]
constexpr int kBScBytes = (BK / 32) * BNB;       // [4][BNB]
constexpr int kStageBytes = kABytes + kBBytes + kAScBytes + kBScBytes;
constexpr int kStageLd = 36;                      // padded fp32 row stride of the epilogue stage
constexpr int kEpiBytes = 4 * 64 * kStageLd * 4;  // 4 waves x 64 rows
constexpr int kSmemBytes = 2 * kStageBytes > kEpiBytes ? 2 * kStageBytes : kEpiBytes;
static_assert(BM == kWM * kTM * 32 && BNB == kWN * kTN * 32, "tile shape");

// Byte offset of (row, k) in a [rows x 128] byte LDS tile with XOR-swizzled 16-byte chunks.  The
// swizzle mixes row bits 0-2 (fragment reads: 8 consecutive rows) and 4-6 (transposed weight
// writes: lanes 16 rows apart), so neither access pattern piles onto one bank.
__device__ __forceinline__ int lds_off8(int row, int k)
{
    return row * 128 + ((((k >> 4) ^ row ^ (row >> 4)) & 7) << 4) + (k & 15);
}

__device__ __forceinline__ int remap_xcd(int bid, int grid)
{
    return (bid % kXcds) * (grid / kXcds) + bid / kXcds;
}

struct Stage {
    u32x4_t a[4];        // 4 x 16 A bytes
    u32x4_t b[4];        // 4 k rows x 16 weight columns
    uint32_t asc;        // 4 A scale bytes of one row (threads < BM)
    u32x4_t bsc;         // 16 weight scale bytes of one block row (threads < 32)
};

template <bool kGated>
__device__ __forceinline__ void mx_load(Stage& st, const uint8_t* A, const uint32_t (&aoff)[4],
                                        const uint8_t* bsrc, const uint8_t* ascsrc,
                                        const uint8_t* bscsrc, int k0, int64_t N_w, int tid)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        st.a[i] = *reinterpret_cast<const u32x4_t*>(A + aoff[i] + k0);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        st.b[r] = *reinterpret_cast<const u32x4_t*>(bsrc + static_cast<int64_t>(k0 + r) * N_w);
    if (tid < BM)
        st.asc = *reinterpret_cast<const uint32_t*>(ascsrc + k0 / 32);
    if (tid < 32)
        st.bsc = *reinterpret_cast<const u32x4_t*>(bscsrc + static_cast<int64_t>(k0 / 32) * N_w);
}

__device__ __forceinline__ void mx_store(unsigned char* smem, int buf, const Stage& st,
                                         int a_row0, int a_k, int b0, int kg, int tid)
{
    unsigned char* As = smem + buf * kStageBytes;
    unsigned char* Bs = As + kABytes;
    unsigned char* Asc = Bs + kBBytes;
    unsigned char* Bsc = Asc + kAScBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4_t*>(As + lds_off8(a_row0 + 32 * i, a_k)) = st.a[i];   // rows tid/8 + 32 i
    // 4 (k) x 16 (n) bytes -> 16 columns of 4 consecutive k bytes: a 4x4 byte transpose per dword
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t x0 = st.b[0][d], x1 = st.b[1][d], x2 = st.b[2][d], x3 = st.b[3][d];
        const uint32_t t0 = __builtin_amdgcn_perm(x1, x0, 0x05010400u);
        const uint32_t t1 = __builtin_amdgcn_perm(x1, x0, 0x07030602u);
        const uint32_t t2 = __builtin_amdgcn_perm(x3, x2, 0x05010400u);
        const uint32_t t3 = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
        const uint32_t c[4] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u),
                               __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                               __builtin_amdgcn_perm(t3, t1, 0x05040100u),
                               __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<uint32_t*>(Bs + lds_off8(b0 + 4 * d + j, kg * 4)) = c[j];
    }
    if (tid < BM)
        *reinterpret_cast<uint32_t*>(Asc + tid * 4) = st.asc;
    if (tid < 32)
        *reinterpret_cast<u32x4_t*>(Bsc + (tid / 8) * BNB + (tid % 8) * 16) = st.bsc;
}

template <bool kGated>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_mx(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ A_sc,
    const uint8_t* __restrict__ B0, const uint8_t* __restrict__ B0_sc,
    const uint8_t* __restrict__ B1, const uint8_t* __restrict__ B1_sc,
    uint8_t* __restrict__ Cq, uint8_t* __restrict__ Cq_sc, uint16_t* __restrict__ Cy,
    const MTile* __restrict__ tiles, const int32_t* __restrict__ tile_count, int K, int N_out,
    int32_t* __restrict__ chunk_done)
{
    constexpr int BN = kGated ? BNB / 2 : BNB;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    const int h = lane >> 5;
    const int n_mt = *tile_count;
    const int n_nt = N_out / BN;
    const int total = n_mt * n_nt;
    const int KT = K / BK;
    const int64_t N_w = N_out;
    const int KS = K / 32;                      // scale bytes per A row

    const int cb = tid % (BNB / 16);            // 16-column chunk staged by this thread
    const int kg = tid / (BNB / 16);            // group of 4 k rows
    const int b0 = cb * 16;

    for (int t = remap_xcd(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
        const MTile tile = tiles[t % n_mt];
        const int n0 = (t / n_mt) * BN;
        const int64_t eoff = static_cast<int64_t>(tile.expert) * K * N_w;
        const int64_t esoff = static_cast<int64_t>(tile.expert) * (K / 32) * N_w;

        // staged weight column of this thread, and (threads < 32) of its scale chunk
        auto col_of = [&](int b) -> int {
            return kGated ? n0 + 32 * (b / 64) + (b % 32) : n0 + b;
        };
        const bool up_half = kGated && ((b0 / 32) & 1);
        const uint8_t* bsrc = (up_half ? B1 : B0) + eoff + col_of(b0) +
                              static_cast<int64_t>(kg * 4) * N_w;
        const int sb0 = (tid % 8) * 16;
        const bool sc_up = kGated && ((sb0 / 32) & 1);
        const uint8_t* bscsrc = (sc_up ? B1_sc : B0_sc) + esoff + col_of(sb0) +
                                static_cast<int64_t>(tid / 8) * N_w;
        const int arow = min(tile.row_begin + (tid < BM ? tid : 0), tile.row_end - 1);
        const uint8_t* ascsrc = A_sc + static_cast<int64_t>(arow) * KS;

        // A rows tid/8 + 32 i (clamped into the tile; rows past row_end are never stored), as
        // 32-bit byte offsets (the host bounds M * K below 2^32)
        uint32_t aoff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int grow = min(tile.row_begin + tid / 8 + 32 * i, tile.row_end - 1);
            aoff[i] = static_cast<uint32_t>(grow) * static_cast<uint32_t>(K) + (tid % 8) * 16;
        }
        const int a_row0 = tid / 8, a_k = (tid % 8) * 16;

        f32x16_t acc[kTM][kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;

        Stage st;
        mx_load<kGated>(st, A, aoff, bsrc, ascsrc, bscsrc, 0, N_w, tid);
        mx_store(smem, 0, st, a_row0, a_k, b0, kg, tid);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < KT)
                mx_load<kGated>(st, A, aoff, bsrc, ascsrc, bscsrc, (kt + 1) * BK, N_w, tid);
            const unsigned char* As = smem + cur * kStageBytes;
            const unsigned char* Bs = As + kABytes;
            const unsigned char* Asc = Bs + kBBytes;
            const unsigned char* Bsc = Asc + kAScBytes;
#pragma unroll 1
            for (int s = 0; s < BK / 64; ++s) {
                i32x8_t af[kTM], bfr[kTN];
                int sa[kTM], sbv[kTN];
#pragma unroll
                for (int i = 0; i < kTM; ++i) {
                    const int row = wm * kTM * 32 + 32 * i + (lane & 31);
                    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(As + lds_off8(row, 64 * s + 16 * h));
                    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(As + lds_off8(row, 64 * s + 32 + 16 * h));
                    af[i] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    sa[i] = Asc[row * 4 + 2 * s + h];
                }
#pragma unroll
                for (int j = 0; j < kTN; ++j) {
                    const int col = wn * kTN * 32 + 32 * j + (lane & 31);
                    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(Bs + lds_off8(col, 64 * s + 16 * h));
                    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(Bs + lds_off8(col, 64 * s + 32 + 16 * h));
                    bfr[j] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    sbv[j] = Bsc[(2 * s + h) * BNB + col];
                }
#pragma unroll
                for (int i = 0; i < kTM; ++i)
#pragma unroll
                    for (int j = 0; j < kTN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            af[i], bfr[j], acc[i][j], 0, 0, 0, sa[i], 0, sbv[j]);
            }
            if (kt + 1 < KT)
                mx_store(smem, cur ^ 1, st, a_row0, a_k, b0, kg, tid);
            __syncthreads();
        }

        if constexpr (kGated) {
            // SwiGLU in fp32 into this wave's LDS stage [64 rows][32 columns] (padded rows), then
            // one lane per row encodes its 32-column block.
            float* stage = reinterpret_cast<float*>(smem) + wave * 64 * kStageLd;
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    stage[row * kStageLd + (lane & 31)] = swiglu(acc[i][0][r], acc[i][1][r]);
                }
            __syncthreads();
            const int grow = tile.row_begin + wm * kTM * 32 + lane;
            if (grow < tile.row_end) {
                const f32x4_t* src = reinterpret_cast<const f32x4_t*>(stage + lane * kStageLd);
                f32x4_t x[8];
                uint32_t amax = 0;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    x[q] = src[q];
#pragma unroll
                    for (int z = 0; z < 4; ++z)
                        amax = max(amax, __float_as_uint(x[q][z]) & 0x7fffffffu);
                }
                const int e = mx_shared_exponent(amax);
                u32x4_t out[2];
#pragma unroll
                for (int w = 0; w < 8; ++w)
                    out[w / 4][w % 4] = e4m3_encode_scaled(x[w][0], e) |
                                        (e4m3_encode_scaled(x[w][1], e) << 8) |
                                        (e4m3_encode_scaled(x[w][2], e) << 16) |
                                        (e4m3_encode_scaled(x[w][3], e) << 24);
                const int hcol = n0 + 32 * wn;         // this wave's 32 output columns
                u32x4_t* dst = reinterpret_cast<u32x4_t*>(Cq + static_cast<int64_t>(grow) * N_out + hcol);
                dst[0] = out[0];
                dst[1] = out[1];
                Cq_sc[static_cast<int64_t>(grow) * (N_out / 32) + hcol / 32] =
                    static_cast<uint8_t>(e + 127);
            }
            __syncthreads();
        } else {
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = tile.row_begin + wm * kTM * 32 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (row >= tile.row_end)
                        continue;
                    uint16_t* crow = Cy + static_cast<int64_t>(row) * N_out;
#pragma unroll
                    for (int j = 0; j < kTN; ++j)
                        crow[n0 + wn * kTN * 32 + 32 * j + (lane & 31)] = f32_to_bf16(acc[i][j][r]);
                }
            if (chunk_done != nullptr) {
                __threadfence();
                __syncthreads();
                if (wave == 0)   // whole wave (lane 0 adds 1): no lane-divergent region in the loop
                    atomicAdd(&chunk_done[tile.chunk], lane == 0 ? 1 : 0);
            }
        }
    }
}

unsigned persistent_grid() { return static_cast<unsigned>(device_info().cu_count * 2); }

hipError_t ensure_smem_limits()
{
    static bool done[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 64 && done[dev])
        return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_mx<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_mx<false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
    if (e == hipSuccess && dev < 64)
        done[dev] = true;
    return e;
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

int mx_fc2_cols_per_tile() { return BNB; }

hipError_t launch_fc1_mx(const uint8_t* A, const uint8_t* a_scale, const uint8_t* wg,
                         const uint8_t* wg_scale, const uint8_t* wu, const uint8_t* wu_scale,
                         uint8_t* h, uint8_t* h_scale, const MTile* tiles,
                         const int32_t* tile_count, int64_t H, int64_t F, hipStream_t s)
{
    if (hipError_t e = ensure_smem_limits(); e != hipSuccess)
        return e;
    grouped_gemm_mx<true><<<dim3(persistent_grid()), dim3(kThreads), kSmemBytes, s>>>(
        A, a_scale, wg, wg_scale, wu, wu_scale, h, h_scale, nullptr, tiles, tile_count,
        static_cast<int>(H), static_cast<int>(F), nullptr);
    return hipGetLastError();
}

hipError_t launch_fc2_mx(const uint8_t* h, const uint8_t* h_scale, const uint8_t* wd,
                         const uint8_t* wd_scale, uint16_t* y, const MTile* tiles,
                         const int32_t* tile_count, int64_t H, int64_t F, int32_t* chunk_done,
                         hipStream_t s)
{
    if (hipError_t e = ensure_smem_limits(); e != hipSuccess)
        return e;
    grouped_gemm_mx<false><<<dim3(persistent_grid()), dim3(kThreads), kSmemBytes, s>>>(
        h, h_scale, wd, wd_scale, nullptr, nullptr, nullptr, nullptr, y, tiles, tile_count,
        static_cast<int>(F), static_cast<int>(H), chunk_done);
    return hipGetLastError();
}

}  // namespace moe
