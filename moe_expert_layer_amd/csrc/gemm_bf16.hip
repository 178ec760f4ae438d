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
//   - Tasks are enumerated run by run (a run is the consecutive row tiles of one expert in one
//     chunk), column-tile-major inside a run, and consecutive task ids go to workgroups of one XCD
//     (workgroups are dealt to the 8 XCDs round-robin): the workgroups of an XCD then share the
//     run's A rows and a handful of weight strips in their L2.
//   - In a partial row tile, 32-row MFMA blocks that lie wholly past the tile's last row are
//     skipped (the condition is uniform per wave).
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

template <bool kGated, int kWM, int kWN, int kTM, int kTN, int kMinBlocks>
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
    static constexpr int kSmemBytes = 2 * kStageBytes;
};

// Byte offset of element (row, k) in a [rows x 64] bf16 LDS tile with XOR-swizzled 16-byte chunks.
__device__ __forceinline__ int lds_off(int row, int k)
{
    return row * 128 + ((((k >> 3) ^ row) & 7) << 4) + ((k & 7) << 1);
}

// Global -> register staging of one K step (k0) of the A and B tiles.
template <class G>
__device__ __forceinline__ void load_tiles(u32x4_t (&ra)[G::kAChunks], u32x4_t (&rb)[G::kBRows],
                                           const uint16_t* A, const uint32_t (&aoff)[G::kAChunks],
                                           const uint16_t* bsrc, int k0, int64_t N_w)
{
#pragma unroll
    for (int i = 0; i < G::kAChunks; ++i)
        ra[i] = *reinterpret_cast<const u32x4_t*>(A + aoff[i] + k0);
#pragma unroll
    for (int r = 0; r < G::kBRows; ++r)
        rb[r] = *reinterpret_cast<const u32x4_t*>(bsrc + static_cast<int64_t>(k0 + r) * N_w);
}

// Register -> LDS: A chunks as loaded; B transposed from kBRows x 8 (k x n) into 8 columns of
// kBRows consecutive k values.
template <class G>
__device__ __forceinline__ void store_tiles(unsigned char* smem, int buf,
                                            const u32x4_t (&ra)[G::kAChunks],
                                            const u32x4_t (&rb)[G::kBRows], int a_lds0, int b0,
                                            int kg)
{
    unsigned char* As = smem + buf * G::kStageBytes;
    unsigned char* Bs = As + G::kABytes;
    // A chunk i of this thread is row tid / 8 + (kThreads / 8) * i: same swizzle phase
#pragma unroll
    for (int i = 0; i < G::kAChunks; ++i)
        *reinterpret_cast<u32x4_t*>(As + a_lds0 + i * (G::kThreads / 8) * 128) = ra[i];
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

// Row block i of wave row wm covers tile rows 32 * (kWM * i + wm) .. + 31 (wave rows interleave, so
// a partial tile splits its row blocks evenly between them).
template <int kWM>
__device__ __forceinline__ int row_block(int i, int wm)
{
    return 32 * (kWM * i + wm);
}

// MFMA fragments of k sub-step ks (16 values of K): the first NB row blocks and all kTN column blocks.
template <int kWM, int kTM, int kTN, int NB>
__device__ __forceinline__ void load_frags(bf16x8_t (&af)[kTM], bf16x8_t (&bfr)[kTN],
                                           const unsigned char* As, const unsigned char* Bs, int wm,
                                           int wn, int lane, int ks)
{
    const int kk = ks * 16 + 8 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < kTN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(
            Bs + lds_off(wn * kTN * 32 + 32 * j + (lane & 31), kk));
#pragma unroll
    for (int i = 0; i < NB; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(
            As + lds_off(row_block<kWM>(i, wm) + (lane & 31), kk));
}

template <int kTM, int kTN, int NB>
__device__ __forceinline__ void mfma_block(f32x16_t (&acc)[kTM][kTN], const bf16x8_t (&af)[kTM],
                                           const bf16x8_t (&bfr)[kTN])
{
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
}

// The K loop of one task with NB active row blocks in this wave (NB = 0: the wave only helps stage
// tiles and keeps the barriers).  Two LDS stages; global loads of step kt + 1 and LDS fragment reads
// of sub-step ks + 1 are in flight while the MFMAs of kt / ks run.
template <class G, int kWM, int kTM, int kTN, int NB>
__device__ __forceinline__ void k_loop(f32x16_t (&acc)[kTM][kTN], unsigned char* smem,
                                       const uint16_t* A, const uint32_t (&aoff)[G::kAChunks],
                                       const uint16_t* bsrc, int64_t N_w, int a_lds0, int b0,
                                       int kg, int KT, int wm, int wn, int lane)
{
    u32x4_t ra[G::kAChunks];
    u32x4_t rb[G::kBRows];
    load_tiles<G>(ra, rb, A, aoff, bsrc, 0, N_w);
    store_tiles<G>(smem, 0, ra, rb, a_lds0, b0, kg);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT)
            load_tiles<G>(ra, rb, A, aoff, bsrc, (kt + 1) * G::BK, N_w);
        const unsigned char* As = smem + cur * G::kStageBytes;
        const unsigned char* Bs = As + G::kABytes;
        if constexpr (NB > 0) {
            bf16x8_t af[2][kTM], bfr[2][kTN];
            load_frags<kWM, kTM, kTN, NB>(af[0], bfr[0], As, Bs, wm, wn, lane, 0);
#pragma unroll 1
            for (int ks = 0; ks < G::BK / 16; ks += 2) {
                load_frags<kWM, kTM, kTN, NB>(af[1], bfr[1], As, Bs, wm, wn, lane, ks + 1);
                mfma_block<kTM, kTN, NB>(acc, af[0], bfr[0]);
                if (ks + 2 < G::BK / 16)
                    load_frags<kWM, kTM, kTN, NB>(af[0], bfr[0], As, Bs, wm, wn, lane, ks + 2);
                mfma_block<kTM, kTN, NB>(acc, af[1], bfr[1]);
            }
        }
        if (kt + 1 < KT)
            store_tiles<G>(smem, cur ^ 1, ra, rb, a_lds0, b0, kg);
        __syncthreads();
    }
}

template <bool kGated, int kWM, int kWN, int kTM, int kTN, int kMinBlocks>
__global__ __launch_bounds__(kWM * kWN * 64, kMinBlocks) void grouped_gemm_bf16(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, uint16_t* __restrict__ C, const MTile* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, int K, int N_out, int32_t* __restrict__ chunk_done,
    int32_t* __restrict__ task_ctr)
{
    using G = Cfg<kGated, kWM, kWN, kTM, kTN, kMinBlocks>;
    __shared__ int claimed;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave: keep scalar
    const int wm = wave / kWN;
    const int wn = wave % kWN;
    const int n_mt = *tile_count;
    const int n_nt = N_out / G::BN;
    const int total = n_mt * n_nt;
    const int KT = K / G::BK;
    const int64_t N_w = N_out;        // row stride of the weight matrices

    // B staging position of this thread.  The k group varies fastest across lanes, so the 8 lanes
    // writing one transposed column chunk fill the 8 (swizzled) 16-byte chunks of one LDS row and
    // never collide on a bank; each global load still covers whole 128-byte row segments.
    constexpr int kKGroups = G::BK / G::kBRows;
    const int kg = tid % kKGroups;              // group of kBRows k rows
    const int cb = tid / kKGroups;              // 8-column chunk of the staged columns
    const int b0 = cb * 8;

    // Tasks are dealt in blocks of `blk` (the workgroups of one XCD): block j belongs to XCD j % 8,
    // and each XCD's workgroups claim that XCD's tasks in order from its own counter.  Whatever the
    // workgroups' relative speeds, an XCD works on about `blk` consecutive tasks at a time (shared
    // A rows and weight strips in its L2), and overall progress follows task order.
    const int xcd = blockIdx.x % kXcdCount;
    const int blk = gridDim.x / kXcdCount;
    for (;;) {
        // Wave 0 claims the next task: every lane takes part (lane 0 adds 1, the others 0) so no
        // lane-divergent branch sits in this barrier loop; lane-divergent regions here let the
        // compiler's loop restructuring split one wave's lanes across different barrier paths.
        if (wave == 0) {
            const int v = atomicAdd(&task_ctr[xcd], lane == 0 ? 1 : 0);
            claimed = __builtin_amdgcn_readfirstlane(v);
        }
        __syncthreads();
        const int i = __builtin_amdgcn_readfirstlane(claimed);   // one value per workgroup
        const int t = ((i / blk) * kXcdCount + xcd) * blk + i % blk;
        if (t >= total)
            break;
        // task t belongs to the run holding row tile t / n_nt; inside the run, row tiles vary fastest
        const MTile head = tiles[t / n_nt];
        const int local = t - n_nt * head.run_begin;
        const MTile tile = tiles[head.run_begin + local % head.run_len];
        const int nt = local / head.run_len;
        const int n0 = nt * G::BN;
        // 32-row MFMA blocks of this wave that hold at least one row of the tile
        const int tile_blocks = (tile.row_end - tile.row_begin + 31) / 32;
        const int nb = __builtin_amdgcn_readfirstlane(
            min(kTM, max(0, (tile_blocks - wm + kWM - 1) / kWM)));

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

        // A rows this thread stages (clamped into the tile; rows past row_end are never stored), as
        // element offsets from A (the host bounds M * K below 2^31)
        uint32_t aoff[G::kAChunks];
#pragma unroll
        for (int i = 0; i < G::kAChunks; ++i) {
            const int grow = min(tile.row_begin + tid / 8 + (G::kThreads / 8) * i, tile.row_end - 1);
            aoff[i] = static_cast<uint32_t>(grow) * static_cast<uint32_t>(K) + (tid % 8) * 8;
        }
        const int a_lds0 = lds_off(tid / 8, (tid % 8) * 8);

        f32x16_t acc[kTM][kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;

        switch (nb) {
#define MOE_KLOOP(NB)                                                                               \
    case NB:                                                                                        \
        k_loop<G, kWM, kTM, kTN, (NB < kTM ? NB : kTM)>(acc, smem, A, aoff, bsrc, N_w, a_lds0, b0, \
                                                         kg, KT, wm, wn, lane);                     \
        break;
            MOE_KLOOP(0) MOE_KLOOP(1) MOE_KLOOP(2) MOE_KLOOP(3)
            default:
                k_loop<G, kWM, kTM, kTN, kTM>(acc, smem, A, aoff, bsrc, N_w, a_lds0, b0, kg, KT,
                                              wm, wn, lane);
                break;
#undef MOE_KLOOP
        }

        // epilogue: lane holds column (lane % 32) of each 32x32 block, rows
        // 8 * (r / 4) + 4 * (lane / 32) + r % 4 for r = 0..15
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            // keep the scheduler from pulling every accumulator into VGPRs at once
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = tile.row_begin + row_block<kWM>(i, wm) + 8 * (r >> 2) +
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
            if (wave == 0)
                atomicAdd(&chunk_done[tile.chunk], lane == 0 ? 1 : 0);
        }
    }
}

// Tile configurations.  Large: 4 waves (2 x 2), each 128 rows x 128 staged columns (16 accumulator
// blocks of 32 x 32 per wave), one workgroup per CU, 128 KiB of LDS for the two stages; used when
// H % 256 == 0 and F % 128 == 0.  Small: 4 waves of 64 x 64, two workgroups per CU, for other sizes
// (H % 128 == 0, F % 64 == 0).
using Fc1Big = Cfg<true, 2, 2, 4, 4, 1>;
using Fc2Big = Cfg<false, 2, 2, 4, 4, 1>;
using Fc1Small = Cfg<true, 2, 2, 2, 2, 2>;
using Fc2Small = Cfg<false, 2, 2, 2, 2, 2>;
#define FC1_BIG grouped_gemm_bf16<true, 2, 2, 4, 4, 1>
#define FC2_BIG grouped_gemm_bf16<false, 2, 2, 4, 4, 1>
#define FC1_SMALL grouped_gemm_bf16<true, 2, 2, 2, 2, 2>
#define FC2_SMALL grouped_gemm_bf16<false, 2, 2, 2, 2, 2>

bool use_big(int64_t H, int64_t F) { return H % Fc2Big::BN == 0 && F % Fc1Big::BN == 0; }

hipError_t ensure_smem_limits()
{
    static bool done[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 64 && done[dev])
        return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&FC1_BIG),
                            hipFuncAttributeMaxDynamicSharedMemorySize, Fc1Big::kSmemBytes);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&FC2_BIG),
                                hipFuncAttributeMaxDynamicSharedMemorySize, Fc2Big::kSmemBytes);
    if (e == hipSuccess && dev < 64)
        done[dev] = true;
    return e;
}

}  // namespace

int bf16_row_tile(int64_t H, int64_t F) { return use_big(H, F) ? Fc1Big::BM : Fc1Small::BM; }
int bf16_fc2_cols_per_tile(int64_t H, int64_t F) { return use_big(H, F) ? Fc2Big::BN : Fc2Small::BN; }
bool bf16_supported(int64_t H, int64_t F) { return H % Fc2Small::BN == 0 && F % Fc1Small::BN == 0; }

hipError_t launch_fc1_bf16(const uint16_t* A, const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                           const MTile* tiles, const int32_t* tile_count, int64_t H, int64_t F,
                           int32_t* task_ctr, hipStream_t s)
{
    const int cu = device_info().cu_count;
    if (use_big(H, F)) {
        if (hipError_t e = ensure_smem_limits(); e != hipSuccess)
            return e;
        FC1_BIG<<<dim3(cu), dim3(Fc1Big::kThreads), Fc1Big::kSmemBytes, s>>>(
            A, wg, wu, h, tiles, tile_count, static_cast<int>(H), static_cast<int>(F), nullptr,
            task_ctr);
    } else {
        FC1_SMALL<<<dim3(2 * cu), dim3(Fc1Small::kThreads), Fc1Small::kSmemBytes, s>>>(
            A, wg, wu, h, tiles, tile_count, static_cast<int>(H), static_cast<int>(F), nullptr,
            task_ctr);
    }
    return hipGetLastError();
}

hipError_t launch_fc2_bf16(const uint16_t* h, const uint16_t* wd, uint16_t* y, const MTile* tiles,
                           const int32_t* tile_count, int64_t H, int64_t F, int32_t* chunk_done,
                           int32_t* task_ctr, hipStream_t s)
{
    const int cu = device_info().cu_count;
    if (use_big(H, F)) {
        if (hipError_t e = ensure_smem_limits(); e != hipSuccess)
            return e;
        FC2_BIG<<<dim3(cu), dim3(Fc2Big::kThreads), Fc2Big::kSmemBytes, s>>>(
            h, wd, nullptr, y, tiles, tile_count, static_cast<int>(F), static_cast<int>(H),
            chunk_done, task_ctr);
    } else {
        FC2_SMALL<<<dim3(2 * cu), dim3(Fc2Small::kThreads), Fc2Small::kSmemBytes, s>>>(
            h, wd, nullptr, y, tiles, tile_count, static_cast<int>(F), static_cast<int>(H),
            chunk_done, task_ctr);
    }
    return hipGetLastError();
}

}  // namespace moe
