// bfloat16 grouped GEMMs for the MoE expert layer on gfx950 MFMA ("NPU Training Operators - MC2",
// 执行路径 steps 7-9; grouped matmul over expert groups as in 底层 API 对照's npu_grouped_matmul).
//
//   fc1:  h[r, :] = swiglu(A[r, :] Wg[e], A[r, :] Wu[e])     A = permuted x [M, H], h [M, F]
//   fc2:  y[r, :] = h[r, :] Wd[e]                             y [M, H]
// where e is the expert of the row tile holding r.  Accumulation is fp32 on
// v_mfma_f32_32x32x16_bf16; each output element sums its whole contraction in one workgroup, in
// the same K order whatever tile or chunk the row falls in (no split-K), so results do not depend
// on the tiling of M.
//
// Structure (one persistent workgroup per CU slot, looping over (row tile, column tile) tasks):
//   - A tile [BM x 64] is read as 16-byte row segments and stored to LDS unchanged (K contiguous).
//   - The weights are N-contiguous ([K, N]); MFMA wants K-contiguous fragments, so each thread
//     loads a (rows of k) x 8-column block, transposes it in registers with v_perm_b32, and
//     stores K-contiguous columns to LDS.  For fc1 the staged columns interleave 32 gate columns
//     with the matching 32 up columns, so one wave holds both halves of every SwiGLU pair.
//   - LDS rows are 128 bytes; their 16-byte chunks are XOR-swizzled by (row mod 8) so the
//     fragment reads (8 consecutive rows, same chunk) hit distinct banks.
//   - Two LDS stages: the global loads for step k+1 are in flight while step k's MFMAs run.
//   - Task order puts the row tiles of one column strip next to each other, and consecutive task
//     ids go to workgroups of one XCD (workgroups are dealt to the 8 XCDs round-robin), so the
//     weight strip a group of tiles shares is fetched into that XCD's L2 once.
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kXcds = 8;

template <bool kGated, int kWM, int kWN, int kTM, int kTN>
struct Cfg {
    static constexpr int kWaves = kWM * kWN;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int BM = kWM * kTM * 32;
    static constexpr int BNB = kWN * kTN * 32;            // weight columns staged per task
    static constexpr int BN = kGated ? BNB / 2 : BNB;      // output columns per task
    static constexpr int BK = 64;
    static constexpr int kAChunks = BM * BK / 8 / kThreads;  // 16-byte A chunks per thread
    static constexpr int kBRows = BK * BNB / 8 / kThreads;   // k rows (of 8 columns) per thread
    static constexpr int kABytes = BM * BK * 2;
    static constexpr int kBBytes = BNB * BK * 2;
    static constexpr int kStageBytes = kABytes + kBBytes;
    static_assert(kAChunks * kThreads * 8 == BM * BK, "A tile split");
    static_assert(kBRows * kThreads * 8 == BK * BNB, "B tile split");
    static_assert(kBRows == 4 || kBRows == 8, "B transpose handles 4 or 8 rows");
    static_assert(!kGated || kTN % 2 == 0, "gated tiles pair gate/up subtiles");
};

// Byte offset of element (row, k) in a [rows x 64] bf16 LDS tile with XOR-swizzled 16-byte chunks.
__device__ __forceinline__ int lds_off(int row, int k)
{
    return row * 128 + ((((k >> 3) ^ row) & 7) << 4) + ((k & 7) << 1);
}

__device__ __forceinline__ int remap_xcd(int bid, int grid)
{
    // grid is a multiple of kXcds: workgroup bid runs on XCD bid % kXcds; give each XCD a
    // contiguous range of logical ids.
    return (bid % kXcds) * (grid / kXcds) + bid / kXcds;
}

// Global -> register staging of one K step (k0) of the A and B tiles.
template <class G>
__device__ __forceinline__ void load_tiles(u32x4_t (&ra)[G::kAChunks], u32x4_t (&rb)[G::kBRows],
                                           const uint16_t* const (&asrc)[G::kAChunks],
                                           const uint16_t* bsrc, int k0, int64_t N_w)
{
#pragma unroll
    for (int i = 0; i < G::kAChunks; ++i)
        ra[i] = *reinterpret_cast<const u32x4_t*>(asrc[i] + k0);
#pragma unroll
    for (int r = 0; r < G::kBRows; ++r)
        rb[r] = *reinterpret_cast<const u32x4_t*>(bsrc + static_cast<int64_t>(k0 + r) * N_w);
}

// Register -> LDS: A chunks as loaded; B transposed from kBRows x 8 (k x n) into 8 columns of
// kBRows consecutive k values.
template <class G>
__device__ __forceinline__ void store_tiles(unsigned char* smem, int buf,
                                            const u32x4_t (&ra)[G::kAChunks],
                                            const u32x4_t (&rb)[G::kBRows],
                                            const int (&a_lds)[G::kAChunks], int b0, int kg)
{
    unsigned char* As = smem + buf * G::kStageBytes;
    unsigned char* Bs = As + G::kABytes;
#pragma unroll
    for (int i = 0; i < G::kAChunks; ++i)
        *reinterpret_cast<u32x4_t*>(As + a_lds[i]) = ra[i];
#pragma unroll
    for (int col = 0; col < 8; ++col) {
        const int d = col >> 1;
        const uint32_t sel = (col & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[G::kBRows / 2];
#pragma unroll
        for (int c = 0; c < G::kBRows / 2; ++c)
            w[c] = __builtin_amdgcn_perm(rb[2 * c + 1][d], rb[2 * c][d], sel);
        unsigned char* dst = Bs + lds_off(b0 + col, kg * G::kBRows);
        if constexpr (G::kBRows == 4)
            *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{w[0], w[1]};
        else
            *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{w[0], w[1], w[2], w[3]};
    }
}

template <bool kGated, int kWM, int kWN, int kTM, int kTN>
__global__ __launch_bounds__(kWM * kWN * 64, 2) void grouped_gemm_bf16(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, uint16_t* __restrict__ C, const MTile* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, int K, int N_out, int32_t* __restrict__ chunk_done)
{
    using G = Cfg<kGated, kWM, kWN, kTM, kTN>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / kWN;
    const int wn = wave % kWN;
    const int n_mt = *tile_count;
    const int n_nt = N_out / G::BN;
    const int total = n_mt * n_nt;
    const int KT = K / G::BK;
    const int64_t N_w = N_out;        // row stride of the weight matrices

    // B staging position of this thread
    const int cb = tid % (G::BNB / 8);          // 8-column chunk of the staged columns
    const int kg = tid / (G::BNB / 8);          // group of kBRows k rows
    const int b0 = cb * 8;

    for (int t = remap_xcd(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
        const MTile tile = tiles[t % n_mt];
        const int nt = t / n_mt;
        const int n0 = nt * G::BN;

        // global column and matrix this thread stages
        const uint16_t* bsrc;
        if (kGated) {
            const int q = b0 / 64, which = (b0 / 32) & 1, c = b0 % 32;
            const uint16_t* Bm = which ? B1 : B0;
            bsrc = Bm + static_cast<int64_t>(tile.expert) * K * N_w + n0 + 32 * q + c;
        } else {
            bsrc = B0 + static_cast<int64_t>(tile.expert) * K * N_w + n0 + b0;
        }
        bsrc += static_cast<int64_t>(kg * G::kBRows) * N_w;

        // A rows this thread stages (clamped into the tile; rows past row_end are never stored)
        const uint16_t* asrc[G::kAChunks];
        int a_lds[G::kAChunks];
#pragma unroll
        for (int i = 0; i < G::kAChunks; ++i) {
            const int idx = tid + i * G::kThreads;
            const int row = idx / 8, ch = idx % 8;
            const int grow = min(tile.row_begin + row, tile.row_end - 1);
            asrc[i] = A + static_cast<int64_t>(grow) * K + ch * 8;
            a_lds[i] = lds_off(row, ch * 8);
        }

        u32x4_t ra[G::kAChunks];
        u32x4_t rb[G::kBRows];

        f32x16_t acc[kTM][kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;

        load_tiles<G>(ra, rb, asrc, bsrc, 0, N_w);
        store_tiles<G>(smem, 0, ra, rb, a_lds, b0, kg);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < KT)
                load_tiles<G>(ra, rb, asrc, bsrc, (kt + 1) * G::BK, N_w);
            const unsigned char* As = smem + cur * G::kStageBytes;
            const unsigned char* Bs = As + G::kABytes;
#pragma unroll
            for (int ks = 0; ks < G::BK / 16; ++ks) {
                const int kk = ks * 16 + 8 * (lane >> 5);
                bf16x8_t af[kTM], bfr[kTN];
#pragma unroll
                for (int i = 0; i < kTM; ++i)
                    af[i] = *reinterpret_cast<const bf16x8_t*>(
                        As + lds_off(wm * kTM * 32 + 32 * i + (lane & 31), kk));
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    bfr[j] = *reinterpret_cast<const bf16x8_t*>(
                        Bs + lds_off(wn * kTN * 32 + 32 * j + (lane & 31), kk));
#pragma unroll
                for (int i = 0; i < kTM; ++i)
#pragma unroll
                    for (int j = 0; j < kTN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j],
                                                                           acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < KT)
                store_tiles<G>(smem, cur ^ 1, ra, rb, a_lds, b0, kg);
            __syncthreads();
        }

        // epilogue: lane holds column (lane % 32) of each 32x32 block, rows
        // 8 * (r / 4) + 4 * (lane / 32) + r % 4 for r = 0..15
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = tile.row_begin + wm * kTM * 32 + 32 * i + 8 * (r >> 2) +
                                4 * (lane >> 5) + (r & 3);
                if (row >= tile.row_end)
                    continue;
                uint16_t* crow = C + static_cast<int64_t>(row) * N_out;
                if (kGated) {
#pragma unroll
                    for (int j = 0; j < kTN; j += 2) {
                        const int q = (wn * kTN + j) / 2;
                        crow[n0 + 32 * q + (lane & 31)] =
                            f32_to_bf16(swiglu(acc[i][j][r], acc[i][j + 1][r]));
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < kTN; ++j)
                        crow[n0 + wn * kTN * 32 + 32 * j + (lane & 31)] = f32_to_bf16(acc[i][j][r]);
                }
            }
        }
        if (chunk_done != nullptr) {
            __threadfence();
            __syncthreads();
            if (tid == 0)
                atomicAdd(&chunk_done[tile.chunk], 1);
        }
    }
}

// Tile configuration: 4 waves (2 x 2), each 64 rows x 64 staged columns.
constexpr int kWM = 2, kWN = 2, kTM = 2, kTN = 2;
using Fc1Cfg = Cfg<true, kWM, kWN, kTM, kTN>;
using Fc2Cfg = Cfg<false, kWM, kWN, kTM, kTN>;
static_assert(Fc1Cfg::BM == kBmBf16 && Fc2Cfg::BM == kBmBf16, "row tile height");

unsigned persistent_grid()
{
    return static_cast<unsigned>(device_info().cu_count * 2);
}

}  // namespace

int bf16_fc1_cols_per_tile() { return Fc1Cfg::BN; }
int bf16_fc2_cols_per_tile() { return Fc2Cfg::BN; }

hipError_t launch_fc1_bf16(const uint16_t* A, const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                           const MTile* tiles, const int32_t* tile_count, int64_t H, int64_t F,
                           hipStream_t s)
{
    grouped_gemm_bf16<true, kWM, kWN, kTM, kTN>
        <<<dim3(persistent_grid()), dim3(Fc1Cfg::kThreads), 2 * Fc1Cfg::kStageBytes, s>>>(
            A, wg, wu, h, tiles, tile_count, static_cast<int>(H), static_cast<int>(F), nullptr);
    return hipGetLastError();
}

hipError_t launch_fc2_bf16(const uint16_t* h, const uint16_t* wd, uint16_t* y, const MTile* tiles,
                           const int32_t* tile_count, int64_t H, int64_t F, int32_t* chunk_done,
                           hipStream_t s)
{
    grouped_gemm_bf16<false, kWM, kWN, kTM, kTN>
        <<<dim3(persistent_grid()), dim3(Fc2Cfg::kThreads), 2 * Fc2Cfg::kStageBytes, s>>>(
            h, wd, nullptr, y, tiles, tile_count, static_cast<int>(F), static_cast<int>(H),
            chunk_done);
    return hipGetLastError();
}

}  // namespace moe
