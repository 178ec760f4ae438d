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
// Both kernels are persistent (one or two workgroups per CU slot) and loop over (row tile, column
// tile) tasks.  Tasks are enumerated run by run (a run is the consecutive row tiles of one expert in
// one chunk), column-tile-major inside a run, and consecutive task ids go to workgroups of one XCD
// (workgroups are dealt to the 8 XCDs round-robin): the workgroups of an XCD then share the run's A
// rows and a handful of weight strips in their L2.  In a partial row tile, 32-row MFMA blocks that
// lie wholly past the tile's last row are skipped (the condition is uniform per wave).
//
// Large tiles (256 rows x 256 weight columns, 8 waves of 64 x 128, two per SIMD; H % 256 == 0,
// F % 128 == 0):
//   - global -> LDS copies bypass registers (global_load_lds_dwordx4: each lane moves 16 bytes to
//     LDS at the wave's base + 16 * lane); four LDS stages of 32 values of K, so the copies of three
//     K steps are in flight while one is multiplied;
//   - A sits in LDS as [256 rows][32 k] and is read as K-contiguous fragments (ds_read_b128);
//   - the weights stay N-contiguous in LDS ([32 k][columns], one region per matrix) and are read
//     with the transposing ds_read_b64_tr_b16, which hands every lane 4 consecutive k of one column;
//   - 16-byte chunks are XOR-swizzled inside each LDS row (the copy lanes pick their global source
//     to match), so fragment reads hit distinct banks;
//   - inside a k sub-step every MFMA is followed by its share of the next sub-step's fragment reads
//     and of the copies, and the barrier that opens K step kt + 1 sits between the two sub-steps of
//     step kt, so neither barrier nor LDS latency idles the matrix cores;
//   - the workgroup claims its tasks two ahead (the atomic's round trip overlaps a K loop) and
//     issues the next task's first copies before the current epilogue, which writes through a
//     per-wave LDS staging area as 16-byte stores.
// Small tiles (128 x 128, two workgroups per CU, other sizes): register-staged copies, the weights
// transposed in registers with v_perm_b32 and stored K-contiguous, two LDS stages.
#include <atomic>
#include <utility>

#include "common.h"
#include "gemm_common.h"
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

// Writes the wave's accumulators.  Lane holds column (lane % 32) of each 32 x 32 block, rows
// 8 * (r / 4) + 4 * (lane / 32) + r % 4 for r = 0..15.  Gated: blocks j and j + 1 are the gate and
// up halves of output columns 32 * ((wn * kTN + j) / 2) ..
template <bool kGated, int kWM, int kTM, int kTN>
__device__ __forceinline__ void store_output(const f32x16_t (&acc)[kTM][kTN], uint16_t* __restrict__ C,
                                             const MTile& tile, int n0, int N_out, int wm, int wn,
                                             int lane, uint16_t* __restrict__ save_g,
                                             uint16_t* __restrict__ save_u)
{
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        // keep the scheduler from pulling every accumulator into VGPRs at once
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = tile.row_begin + row_block<kWM>(i, wm) + 8 * (r >> 2) + 4 * (lane >> 5) +
                            (r & 3);
            if (row >= tile.row_end)
                continue;
            if (kGated) {
#pragma unroll
                for (int j = 0; j < kTN; j += 2) {
                    const int q = (wn * kTN + j) / 2;
                    const int64_t at = static_cast<int64_t>(row) * N_out + n0 + 32 * q + (lane & 31);
                    if (C != nullptr)           // null: only g and u are wanted
                        C[at] = f32_to_bf16(swiglu(acc[i][j][r], acc[i][j + 1][r]));
                    if (save_g != nullptr) {
                        save_g[at] = f32_to_bf16(acc[i][j][r]);
                        save_u[at] = f32_to_bf16(acc[i][j + 1][r]);
                    }
                }
            } else {
                uint16_t* crow = C + static_cast<int64_t>(row) * N_out;
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    crow[n0 + wn * kTN * 32 + 32 * j + (lane & 31)] = f32_to_bf16(acc[i][j][r]);
            }
        }
    }
}

template <bool kGated, int kWM, int kWN, int kTM, int kTN, int kMinBlocks>
__global__ __launch_bounds__(kWM * kWN * 64, kMinBlocks) void grouped_gemm_bf16(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, uint16_t* __restrict__ C, const MTile* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, int K, int N_out, int32_t* __restrict__ chunk_done,
    int32_t* __restrict__ task_ctr, uint16_t* __restrict__ save_g, uint16_t* __restrict__ save_u)
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

    const int xcd = blockIdx.x % kXcdCount;
    const int blk = gridDim.x / kXcdCount;
    for (;;) {
        const int t = claim_task(&claimed, task_ctr, xcd, blk, wave, lane);
        if (t >= total)
            break;
        int nt;
        const MTile tile = decode_task(t, n_nt, tiles, nt);
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
        // element offsets from the tile's first row: below BM * K, which the host keeps under 2^31
        // (K <= 2^22), whatever the number of rows M
        const uint16_t* A_tile = A + static_cast<int64_t>(tile.row_begin) * K;
        uint32_t aoff[G::kAChunks];
#pragma unroll
        for (int i = 0; i < G::kAChunks; ++i) {
            const int trow = min(tid / 8 + (G::kThreads / 8) * i, tile.row_end - 1 - tile.row_begin);
            aoff[i] = static_cast<uint32_t>(trow) * static_cast<uint32_t>(K) + (tid % 8) * 8;
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
        case 0: k_loop<G, kWM, kTM, kTN, 0>(acc, smem, A_tile, aoff, bsrc, N_w, a_lds0, b0, kg, KT, wm, wn, lane); break;
        case 1: k_loop<G, kWM, kTM, kTN, 1>(acc, smem, A_tile, aoff, bsrc, N_w, a_lds0, b0, kg, KT, wm, wn, lane); break;
        default: k_loop<G, kWM, kTM, kTN, kTM>(acc, smem, A_tile, aoff, bsrc, N_w, a_lds0, b0, kg, KT, wm, wn, lane); break;
        }
        store_output<kGated, kWM, kTM, kTN>(acc, C, tile, n0, N_out, wm, wn, lane, save_g, save_u);
        if (chunk_done != nullptr)
            count_done(chunk_done, tile.chunk, wave, lane);
    }
}

// ------------------------------------------------------------------------------------------------
// Large tiles with LDS DMA

#ifdef MOE_PHASE_PROBE
// Per-task phase timing, compiled only into the probe library (timestamps only; every kernel does
// the same work as in the product library).  Wave 0 of each workgroup reads the cycle counter at
// the points of its task loop marked MOE_PROBE and keeps per-workgroup sums in scalar registers;
// after its last task lane 0 adds them to g_phase[kind] (kind 0 fc2, 1 fc1, 2 the backward's
// recompute), outside the task loop and its barriers.
__device__ unsigned long long g_phase[kProbeKindsBf16][kProbeFields];
#define MOE_PROBE(...) __VA_ARGS__
#else
#define MOE_PROBE(...)
#endif

namespace big {
constexpr int kWM = 4, kWN = 2, kTM = 2, kTN = 4;     // 8 waves (2 per SIMD), 64 x 128 each
constexpr int kWaves = kWM * kWN;
constexpr int kThreads = kWaves * 64;
constexpr int BM = kWM * kTM * 32;                     // 256 rows
constexpr int BNB = kWN * kTN * 32;                    // 256 weight columns
constexpr int BK = 32;
constexpr int kStages = 4;
constexpr int kABytes = BM * BK * 2;                   // [256 rows][32 k], 64-byte rows
constexpr int kBBytes = BK * BNB * 2;                  // [32 k][256 columns] over 1 or 2 matrices
constexpr int kBRing = kStages * kABytes;             // the A parts of all stages, then the B parts
constexpr int kRingBytes = kStages * (kABytes + kBBytes);   // 128 KiB
constexpr int kOutRows = 32;                           // epilogue staging: 32 rows x 64 columns
constexpr int kOutWaveBytes = kOutRows * 128;          //   of bf16 per wave (4 KiB)
constexpr int kSmemBytes = kRingBytes + kWaves * kOutWaveBytes;   // 160 KiB, the whole LDS of a CU
// A moves in pairs of K steps (rows of 128 bytes, whole cache lines): two pair stages of 32 KiB
// fill the A half of the ring.  The weights move per K step through the four B stages.
constexpr int kAPairBytes = 2 * kABytes;               // [256 rows][64 k]
constexpr int kACopies = kAPairBytes / 1024 / kWaves;  // 1 KiB copies per wave per pair (4)
constexpr int kBCopies = kBBytes / 1024 / kWaves;      // per wave per K step (2)
constexpr int kAHalf = kACopies / 2;                   // A copies per half pair
static_assert(kACopies % 2 == 0 && kACopies * kWaves * 1024 == kAPairBytes, "whole copies");

template <bool kGated>
struct BLayout {
    static constexpr int kMats = kGated ? 2 : 1;
    static constexpr int kRowBytes = BNB / kMats * 2;   // one k row of one matrix: 256 or 512 bytes
    static constexpr int kChunks = kRowBytes / 16;      // 16-byte chunks per row
    static constexpr int kRowsPerCopy = 64 / kChunks;
    static constexpr int kMatBytes = BK * kRowBytes;
    static_assert(kChunks >= 16, "the k-row swizzle uses chunk bits 2..3");
};

// Waits until at most N of this wave's copies are still in flight, and for this wave's LDS reads,
// then joins the workgroup barrier.  One statement with a memory clobber: no memory operation
// moves across it.
template <int N>
__device__ __forceinline__ void step_barrier()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// A: LDS row r of a pair stage (128 bytes = 8 chunks of 8 k) keeps logical chunk c at position
// c ^ ((r >> 1) & 7): the 16 rows one read instruction serves per chunk cover all 16 bank groups
// of 16 bytes.  B: k row kr keeps 16-byte chunk c at c ^ (4 * (kr & 3)): the four k rows of one
// transposing read group land 64 bytes apart within each 256-byte bank window.
//
// A copy j of wave w moves pair rows 32 w + 8 j .. + 7 (8 lanes per 128-byte row); B copy j moves
// slot bi0 + j (kRowsPerCopy k rows of one matrix).  The per-lane global offsets (a_voff, b_voff:
// the lane's row and swizzled 16-byte chunk) stay fixed for a task; rows past the tile's last row
// re-read its last row (their results are never stored).  Sources advance by 64 elements of A per
// pair and BK weight rows per K step.
struct CopyCtx {
    const uint16_t* a;     // A at the first k of the next pair to fetch
    const uint16_t* b;     // this wave's weight matrix at the next step's first k row
    uint32_t a_lds;        // LDS destination of the wave's first A copy in pair stage 0
    uint32_t b_lds;        // LDS destination of the wave's first B copy in B stage 0
    bool b_on;             // half-width task: this lane's weight chunk lies in the task's columns
};

// What a sub-step copies: nothing, the weights of one step, the second half of a pair's A, or the
// weights of one step and then the first half of a pair's A.  kHalfW marks the weight copies of a
// half-width task (only the lanes with b_on copy).
enum CopySet { kNone = 0, kB = 1, kA2 = 2, kBA1 = 3, kHalfW = 4 };
template <int CS>
constexpr int set_size()
{
    return (CS & 3) == kNone ? 0 : (CS & 3) == kBA1 ? kBCopies + kAHalf : (CS & 3) == kB ? kBCopies : kAHalf;
}

// Copy C of copy set CS: weights into B stage SB, A into pair stage QA.
template <int CS, int SB, int QA, int C>
__device__ __forceinline__ void copy_one(const CopyCtx& s, const uint32_t (&a_voff)[kACopies],
                                         const uint32_t (&b_voff)[kBCopies])
{
    if constexpr ((CS & 3) == kA2) {
        lds_copy16(s.a, a_voff[kAHalf + C], s.a_lds + QA * kAPairBytes + (kAHalf + C) * 1024);
    } else if constexpr (C < kBCopies) {
        if constexpr ((CS & kHalfW) != 0) {
            if (s.b_on)
                lds_copy16(s.b, b_voff[C], s.b_lds + SB * kBBytes + C * 1024);
        } else {
            lds_copy16(s.b, b_voff[C], s.b_lds + SB * kBBytes + C * 1024);
        }
    } else {
        lds_copy16(s.a, a_voff[C - kBCopies], s.a_lds + QA * kAPairBytes + (C - kBCopies) * 1024);
    }
}

template <int CS, int SB, int QA, int C0, int... Is>
__device__ __forceinline__ void copies_impl(std::integer_sequence<int, Is...>, const CopyCtx& s,
                                            const uint32_t (&a_voff)[kACopies],
                                            const uint32_t (&b_voff)[kBCopies])
{
    (copy_one<CS, SB, QA, C0 + Is>(s, a_voff, b_voff), ...);
}

// Copies C0 .. C1 - 1 of copy set CS.
template <int CS, int SB, int QA, int C0, int C1>
__device__ __forceinline__ void copies(const CopyCtx& s, const uint32_t (&a_voff)[kACopies],
                                       const uint32_t (&b_voff)[kBCopies])
{
    copies_impl<CS, SB, QA, C0>(std::make_integer_sequence<int, C1 - C0>{}, s, a_voff, b_voff);
}

// All four A copies of a pair into pair stage QA (task prologue).
template <int QA>
__device__ __forceinline__ void issue_pair(const CopyCtx& s, const uint32_t (&a_voff)[kACopies])
{
#pragma unroll
    for (int j = 0; j < kACopies; ++j)
        lds_copy16(s.a, a_voff[j], s.a_lds + QA * kAPairBytes + j * 1024);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// MFMA operands of one k sub-step (16 k): A row blocks and weight column blocks.
struct Frags {
    bf16x8_t a[kTM];
    bf16x8_t b[kTN];
    i16x4_t lo[kTN];       // first half of b[j] until its second half arrives
};

// Fragment read Q of sub-step KS of K step position S (B stage S, pair stage S / 2, pair half
// S % 2), in the order the next sub-step's MFMAs consume them: Q = 0 is A row block 0, Q = 1 + 2 j,
// 2 + 2 j the two transposing reads (k 0..3, 4..7 of the lane's 8) of weight block j, Q = 2 kTN + i
// (i >= 1) A row block i.  a_base[h][ks] / b_base[j] are the lane's addresses in stage 0; the stage,
// sub-step and block parts are constants below 64 KiB, immediate offsets of the LDS instructions.
template <bool kGated, int S, int KS, int Q>
__device__ __forceinline__ void read_one(Frags& f, const uint32_t (&a_base)[2][2], const uint32_t (&b_base)[kTN])
{
    using L = BLayout<kGated>;
    if constexpr (Q >= 1 && Q <= 2 * kTN) {
        constexpr int j = (Q - 1) / 2, h = (Q - 1) % 2;
        const uint32_t p = b_base[j] + S * kBBytes + (16 * KS + 4 * h) * L::kRowBytes;
        const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4_t*>(p));
        if constexpr (h == 0)
            f.lo[j] = v;
        else
            f.b[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(f.lo[j], v, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
        constexpr int i = Q == 0 ? 0 : Q - 2 * kTN;
        f.a[i] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
            a_base[S % 2][KS] + (S / 2) * kAPairBytes + kWM * 32 * 128 * i);
    }
}

template <bool kGated, int S, int KS, int Q0, int... Is>
__device__ __forceinline__ void reads_impl(std::integer_sequence<int, Is...>, Frags& f,
                                           const uint32_t (&a_base)[2][2], const uint32_t (&b_base)[kTN])
{
    (read_one<kGated, S, KS, Q0 + Is>(f, a_base, b_base), ...);
}

template <bool kGated, int S, int KS, int Q0, int Q1>
__device__ __forceinline__ void reads(Frags& f, const uint32_t (&a_base)[2][2], const uint32_t (&b_base)[kTN])
{
    reads_impl<kGated, S, KS, Q0>(std::make_integer_sequence<int, Q1 - Q0>{}, f, a_base, b_base);
}

// Operands shared by the sub-steps of a K loop.
struct LoopArgs {
    const uint32_t (&a_base)[2][2];
    const uint32_t (&b_base)[kTN];
    const uint32_t (&a_voff)[kACopies];
    const uint32_t (&b_voff)[kBCopies];
};

// Slot M of a sub-step: MFMA M (row block M / kTN, column block M % kTN), then this slot's share of
// the next sub-step's fragment reads (sub-step KS of step position SR) and of the sub-step's copies
// (copy set CS into B stage SB / pair stage QA).  The reads go out over the first half of the
// MFMAs, so they have landed well before a barrier's lgkmcnt(0) (spread over all of them, the last
// read's latency was exposed at every barrier: 2% of the GEMM); the copies are spread over all.
template <bool kGated, int NB, int CS, int SB, int QA, int SR, int KS, int M>
__device__ __forceinline__ void slot(f32x16_t (&acc)[kTM][kTN], const Frags& use, Frags& load,
                                     const CopyCtx& cp, const LoopArgs& g)
{
    constexpr int NM = NB * kTN, NR = 2 * kTN + NB, NC = set_size<CS>();
    // weights as the first operand: the accumulator block is the transposed 32 x 32 output block,
    // so a lane holds one output row (lane % 32) and four runs of four adjacent columns, 8 (r / 4) +
    // 4 (lane / 32) + r % 4 (the two operands' registers have the same layout)
    acc[M / kTN][M % kTN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(use.b[M % kTN], use.a[M / kTN],
                                                                    acc[M / kTN][M % kTN], 0, 0, 0);
    constexpr int RF = NM / 2 > 0 ? NM / 2 : 1;                    // slots that carry the reads
    if constexpr (M < RF)
        reads<kGated, SR, KS, M * NR / RF, (M + 1) * NR / RF>(load, g.a_base, g.b_base);
    copies<CS, SB, QA, M * NC / NM, (M + 1) * NC / NM>(cp, g.a_voff, g.b_voff);
    __builtin_amdgcn_sched_barrier(0);
}

template <bool kGated, int NB, int CS, int SB, int QA, int SR, int KS, int... Ms>
__device__ __forceinline__ void slots(std::integer_sequence<int, Ms...>, f32x16_t (&acc)[kTM][kTN],
                                      const Frags& use, Frags& load, const CopyCtx& cp,
                                      const LoopArgs& g)
{
    (slot<kGated, NB, CS, SB, QA, SR, KS, Ms>(acc, use, load, cp, g), ...);
}

// One k sub-step: the NB * kTN MFMAs on `use`, the fragment reads of sub-step KS of step position
// SR into `load`, and the copies of set CS.  A wave without MFMAs (NB = 0) only issues the copies.
template <bool kGated, int NB, int CS, int SB, int QA, int SR, int KS>
__device__ __forceinline__ void substep(f32x16_t (&acc)[kTM][kTN], const Frags& use, Frags& load,
                                        const CopyCtx& cp, const LoopArgs& g)
{
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NB == 0)
        copies<CS, SB, QA, 0, set_size<CS>()>(cp, g.a_voff, g.b_voff);
    else
        slots<kGated, NB, CS, SB, QA, SR, KS>(std::make_integer_sequence<int, NB * kTN>{}, acc, use,
                                              load, cp, g);
    __builtin_amdgcn_sched_barrier(0);
}

// Copy schedule.  The weights of K step s go out during the second sub-step of step s - 4 (into
// the B stage step s - 4 has just freed).  The A of pair p (steps 2p, 2p + 1) goes out in two
// halves, during the second sub-step of step 2p - 3 and the first sub-step of step 2p - 2 (into the
// pair stage pair p - 2 has just freed).  Copies are issued in a fixed order, so "what step t + 1
// needs has landed" is "at most N copies are in flight", N counted from that order: 8 at the
// barrier of an even step, 2 at that of an odd one (fewer near the end of the task).
//
// A wave whose 32 A rows all lie past the tile's last row (a partial tile) copies no A at all: its
// copies are the weights alone, and the step t + 1 weights have landed once at most the weights of
// steps t + 2 and t + 3 are in flight, at every barrier.
template <bool kA>
constexpr int wait_even() { return kA ? 2 * kBCopies + kACopies : 2 * kBCopies; }
template <bool kA>
constexpr int wait_odd() { return kA ? kBCopies : 2 * kBCopies; }

// K step t (t % 4 = S): sub-step 1 of step t on the fragments of sub-step 0, with the second A half
// of pair t / 2 + 1 when t is even and kCopyA2; the barrier after which step t + 1 has landed (at
// most W copies in flight; none for W < 0) and step t's stages are free; sub-step 0 of step t + 1
// on the fragments of sub-step 1, with the weights of step t + 4 (and, t odd, the first A half of
// pair (t + 3) / 2) when kCopyB.  kA = false: the wave copies no A.
template <bool kGated, int NB, bool kA, bool kHalf, int S, bool kCopyA2, bool kCopyB, int W>
__device__ __forceinline__ void k_step(f32x16_t (&acc)[kTM][kTN], Frags& f0, Frags& f1, CopyCtx& cp,
                                       const LoopArgs& g, int64_t N_w)
{
    constexpr int CS1 = kA && S % 2 == 0 && kCopyA2 ? kA2 : kNone;
    constexpr int CS2 = !kCopyB ? kNone : (S % 2 == 0 || !kA ? kB : kBA1) | (kHalf ? kHalfW : 0);
    constexpr int Qnext = (S / 2 + 1) % 2;                    // pair stage of pair t / 2 + 1
    substep<kGated, NB, CS1, 0, Qnext, S, 1>(acc, f0, f1, cp, g);
    if constexpr (CS1 == kA2)
        cp.a += 64;                                           // the next pair's A
    if constexpr (W >= 0)
        step_barrier<W>();
    // after the last step this reads a stale stage whose fragments are never used
    substep<kGated, NB, CS2, S, S / 2, (S + 1) % kStages, 0>(acc, f1, f0, cp, g);
    if constexpr (kCopyB)
        cp.b += BK * N_w;
}

// The K loop of one task.  KT is a multiple of kStages (at least kStages); the caller issued A
// pair 0, the weights of steps 0 .. 3 and the first A half of pair 1, in that order (kA = false:
// the weights alone), cp points at pair 1 and at step 4's weights, and the caller has waited for
// step 0 (step_barrier<top_wait<kA>()>).  The body is unrolled over the four B stages (two pair
// stages), so every LDS address is a lane base plus a constant.
template <bool kA>
constexpr int top_wait() { return kA ? 3 * kBCopies + kAHalf : 3 * kBCopies; }   // steps 1 .. 3 (+ A)

template <bool kGated, int NB, bool kA, bool kHalf>
__device__ __forceinline__ void k_loop(f32x16_t (&acc)[kTM][kTN], CopyCtx cp, const LoopArgs& g,
                                       int64_t N_w, int KT)
{
    static_assert(kStages == 4, "the unrolled body below covers four stages");
    constexpr int WE = wait_even<kA>(), WO = wait_odd<kA>();
    Frags f0, f1;
    if constexpr (NB > 0)
        reads<kGated, 0, 0, 0, 2 * kTN + NB>(f0, g.a_base, g.b_base);
    for (int kt = 0; kt < KT - kStages; kt += kStages) {
        k_step<kGated, NB, kA, kHalf, 0, true, true, WE>(acc, f0, f1, cp, g, N_w);
        k_step<kGated, NB, kA, kHalf, 1, true, true, WO>(acc, f0, f1, cp, g, N_w);
        k_step<kGated, NB, kA, kHalf, 2, true, true, WE>(acc, f0, f1, cp, g, N_w);
        k_step<kGated, NB, kA, kHalf, 3, true, true, WO>(acc, f0, f1, cp, g, N_w);
    }
    // the last four steps: only the second A half of the last pair is still to be copied
    k_step<kGated, NB, kA, kHalf, 0, true, false, WE>(acc, f0, f1, cp, g, N_w);
    k_step<kGated, NB, kA, kHalf, 1, false, false, 0>(acc, f0, f1, cp, g, N_w);
    k_step<kGated, NB, kA, kHalf, 2, false, false, 0>(acc, f0, f1, cp, g, N_w);
    k_step<kGated, NB, kA, kHalf, 3, false, false, -1>(acc, f0, f1, cp, g, N_w);
}

// Epilogue through LDS.  The wave's output (64 rows x 64 columns for fc1, 64 x 128 for fc2) goes
// out in 32 x 64 pieces: the accumulators (transposed blocks: a lane holds one row and runs of four
// adjacent columns) are written to the wave's staging area as bf16, four columns per 8-byte LDS
// write (rows of 128 bytes with 16-byte chunks XOR-swizzled by row), then read back as 16-byte row
// chunks and stored to global memory 16 bytes per lane.  Only this wave touches its
// area, and LDS operations of one wave complete in order, so no barrier is needed.
// kVal (fc1): 0 the SwiGLU output h, 1 the gate values g, 2 the up values u (the last two saved for
// the backward, same layout as h).
template <bool kGated, int kVal = 0>
__device__ __forceinline__ void store_output_staged(const f32x16_t (&acc)[kTM][kTN], uint16_t* __restrict__ C,
                                                    const MTile& tile, int n0, int N_out, uint32_t stage,
                                                    int wm, int wn, int lane, bool through)
{
    constexpr int kOutCols = kGated ? 16 * kTN : 32 * kTN;       // the wave's output columns
    constexpr int PC = kOutCols < 64 ? kOutCols : 64;           // piece columns
    constexpr int PR = kOutWaveBytes / (2 * PC);                // piece rows (a multiple of 32)
    constexpr int CPR = PC / 8;                                 // 16-byte chunks per staged row
    constexpr int kSwz = CPR == 8 ? 0 : 2;                      // rows sharing a 256-byte bank window
    static_assert(PR % 32 == 0 && (32 * kTM) % PR == 0, "pieces cover whole row blocks");
#pragma unroll
    for (int rp = 0; rp < 32 * kTM / PR; ++rp) {
#pragma unroll
        for (int cp = 0; cp < kOutCols / PC; ++cp) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ii = 0; ii < PR / 32; ++ii) {
                const int i = rp * (PR / 32) + ii;
#pragma unroll
                for (int jj = 0; jj < PC / 32; ++jj) {
                    const int ob = cp * (PC / 32) + jj;               // 32-column output block
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 4 * q + e;
                            if constexpr (kGated && kVal == 0)
                                v[e] = swiglu(acc[i][2 * ob][r], acc[i][2 * ob + 1][r]);   // gate, up blocks
                            else if constexpr (kGated)
                                v[e] = acc[i][2 * ob + kVal - 1][r];
                            else
                                v[e] = acc[i][ob][r];
                        }
                        const int row = 32 * ii + (lane & 31);
                        const int col = 32 * jj + 8 * q + 4 * (lane >> 5);          // 4 adjacent columns
                        const uint32_t a = stage + row * (2 * PC) +
                                           ((((col >> 3) ^ (row >> kSwz)) & (CPR - 1)) << 4) + 2 * (col & 7);
                        *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(a) =
                            u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                    }
                }
            }
            // PR rows x CPR chunks of 16 bytes: lane reads chunk (lane % CPR) of rows lane / CPR + ..
            const int chunk = lane % CPR;
            const int col0 = n0 + kOutCols * wn + PC * cp + 8 * chunk;
#pragma unroll
            for (int m = 0; m < PR * CPR / 64; ++m) {
                const int row = lane / CPR + (64 / CPR) * m;
                const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
                    stage + row * (2 * PC) + (((chunk ^ (row >> kSwz)) & (CPR - 1)) << 4));
                const int grow = tile.row_begin + row_block<kWM>(rp * (PR / 32) + row / 32, wm) + row % 32;
                if (grow < tile.row_end) {
                    uint16_t* dst = C + static_cast<int64_t>(grow) * N_out + col0;
                    if (through)
                        store16_through(dst, v);
                    else
                        *reinterpret_cast<u32x4_t*>(dst) = v;
                }
            }
        }
    }
}

// gather (fc1 only, may be null): permuted row p of A is row gather[p] / gather_k of the matrix
// A points at (the permute step folded into the row copies); null: row p of A.
// C (gated) may be null when save_g / save_u are set: then h is not stored.
// kRole only separates launches in profiles: 0 for the forward, 1 for the backward's recompute of g
// and u (the same code).
template <bool kGated, int kRole = 0>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16_dma(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, uint16_t* __restrict__ C, const MTile* __restrict__ tiles,
    const int32_t* __restrict__ tile_count, int K, int N_out, int32_t* __restrict__ chunk_done,
    int32_t* __restrict__ task_ctr, const int32_t* __restrict__ gather, int gather_k,
    uint16_t* __restrict__ save_g, uint16_t* __restrict__ save_u)
{
    using L = BLayout<kGated>;
    constexpr int BN = kGated ? BNB / 2 : BNB;
    // dynamic LDS: the kStages-stage ring, then each wave's epilogue staging area.  The claimed-task
    // word sits at the start of wave 0's area: wave 0 writes it after its epilogue, every wave reads
    // it after the next task's first barrier, and wave 0's next epilogue (which overwrites it) starts
    // only after the barrier that ends that task's K loop.
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    int* const claimed = reinterpret_cast<int*>(smem + kRingBytes);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char*)(smem)));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN;
    const int wn = wave % kWN;
    const int n_mt = *tile_count;
    const int n_nt = N_out / BN;
    // Half-width tasks (non-gated, unchunked tables): the table ends in its short partial tiles (at
    // most 64 rows, each its own run), whose tasks stream the whole weight strip for a few rows; each
    // of their column tiles becomes two tasks of BN / 2 columns, so the launch's last tasks spread
    // over twice as many CUs.  tile_count[2] holds the number of tiles before that suffix.
    const int n_full = !kGated && chunk_done == nullptr ? min(max(tile_count[2], 0), n_mt) : n_mt;
    const int t_full = n_full * n_nt;
    const int total = t_full + 2 * (n_mt - n_full) * n_nt;
    const int KT = K / BK;
    const int64_t N_w = N_out;

    // copy sources, lane parts (bytes from the step's first weight row): B copy j covers k rows
    // kRowsPerCopy * (bi0 + j) .. + kRowsPerCopy - 1, lane / kChunks within them
    const int bi0 = kGated ? kBCopies * (wave % (kWaves / 2)) : kBCopies * wave;
    uint32_t b_voff[kBCopies];
#pragma unroll
    for (int j = 0; j < kBCopies; ++j) {
        const int kr = (bi0 + j) * L::kRowsPerCopy + lane / L::kChunks;
        const int c = (lane % L::kChunks) ^ (4 * (kr & 3));
        b_voff[j] = static_cast<uint32_t>(kr) * static_cast<uint32_t>(N_out) * 2u + 16u * c;
    }
    CopyCtx cp;
    cp.a_lds = lds0 + kACopies * wave * 1024;
    cp.b_lds = lds0 + kBRing + (kGated ? (wave / (kWaves / 2)) * L::kMatBytes : 0) + bi0 * 1024;
    // fragment reads: the lane's LDS addresses in stage 0 (A: row block 0 of this wave, sub-step ks;
    // B: weight block j, sub-step 0).  Each is hidden from the optimiser so that it stays one
    // register and the constant parts of every read go into the instruction's offset field.
    uint32_t a_base[2][2];                                    // [pair half][sub-step]
#pragma unroll
    for (int hp = 0; hp < 2; ++hp)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int r = lane & 31;
            a_base[hp][ks] = lds0 + row_block<kWM>(0, wm) * 128 + r * 128 +
                             16 * ((4 * hp + 2 * ks + (lane >> 5)) ^ ((r >> 1) & 7));
            asm volatile("" : "+v"(a_base[hp][ks]));
        }
    uint32_t b_base[kTN];
    {
        const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
        const int kr = 8 * (g >> 1) + e;                       // + 16 ks + 4 for the upper half
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int m = kGated ? (j & 1) : 0;
            const int col = (kGated ? 16 * kTN * wn + 32 * (j >> 1) : 32 * kTN * wn + 32 * j) + 16 * (g & 1) + 4 * q;
            b_base[j] = lds0 + kBRing + m * L::kMatBytes + kr * L::kRowBytes + 16 * ((col >> 3) ^ (4 * e)) +
                        2 * (col & 7);
            asm volatile("" : "+v"(b_base[j]));
        }
    }

    const int xcd = blockIdx.x % kXcdCount;
    const int blk = gridDim.x / kXcdCount;

    // Task state.  The copies of a task's first K steps are issued before the previous task's
    // epilogue, so the epilogue hides their latency.
    MTile tile{};
    int n0 = 0;
    bool half = false;                                        // a half-width task (see n_full)
    // task t: its row tile, first output column and width
    auto decode = [&](int t, int& col0, bool& is_half) -> MTile {
        if (t < t_full) {
            int nt;
            const MTile tl = decode_task(t, n_nt, tiles, nt);
            col0 = nt * BN;
            is_half = false;
            return tl;
        }
        const int r = (t - t_full) % (2 * n_nt);
        col0 = (r >> 1) * BN + (r & 1) * (BN / 2);
        is_half = true;
        return tiles[n_full + (t - t_full) / (2 * n_nt)];
    };
    uint32_t a_voff[kACopies];
    // Gathered fc1 rows: the slot-list entries of this lane's A copy rows for the next task, loaded
    // one task ahead (during the previous task's K loop) and first used in setup, so that nothing
    // waits for them.
    int gsrc[kACopies] = {};
    auto fetch_rows = [&](int t) {
        if (gather == nullptr)
            return;
        int c0;
        bool hf;
        const MTile tl = decode(t, c0, hf);
#pragma unroll
        for (int j = 0; j < kACopies; ++j) {
            const int r = 8 * (kACopies * wave + j) + lane / 8;
            gsrc[j] = gather[tl.row_begin + min(r, tl.row_end - tl.row_begin - 1)];   // used in setup
        }
    };
    // setup_from: the task whose tile, first column and width decode() gave
    auto setup_from = [&](const MTile& tl, int col0, bool hf) {
        tile = tl;
        n0 = col0;
        half = hf;
        // the weight chunks of the task's columns: chunk c of a 512-byte row holds columns 8c ..
        // 8c + 7, and copy lanes 0 .. 15 (32 .. 47) take chunks 0 .. 15 whatever the swizzle
        cp.b_on = !half || (lane & 16) == 0;
        const int rows = tile.row_end - tile.row_begin;
#pragma unroll
        for (int j = 0; j < kACopies; ++j) {
            const int r = 8 * (kACopies * wave + j) + lane / 8;
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            const int src = gather != nullptr ? gsrc[j] / gather_k : min(r, rows - 1);
            a_voff[j] = static_cast<uint32_t>(src) * static_cast<uint32_t>(K) * 2u + 16u * c;
        }
        cp.a = gather != nullptr ? A : A + static_cast<int64_t>(tile.row_begin) * K;
        cp.b = (kGated && wave >= kWaves / 2 ? B1 : B0) + static_cast<int64_t>(tile.expert) * K * N_w + n0;
        // A pair 0, the weights of steps 0 .. 3, the first half of A pair 1 (k_loop's order); a wave
        // whose A rows all lie past the tile's end copies the weights alone
        const bool a_on = 32 * wave < rows;
        if (a_on)
            issue_pair<0>(cp, a_voff);
        cp.a += 64;
        if (!kGated && half) {
            copies<kB | kHalfW, 0, 0, 0, kBCopies>(cp, a_voff, b_voff);
            cp.b += BK * N_w;
            copies<kB | kHalfW, 1, 0, 0, kBCopies>(cp, a_voff, b_voff);
            cp.b += BK * N_w;
            copies<kB | kHalfW, 2, 0, 0, kBCopies>(cp, a_voff, b_voff);
            cp.b += BK * N_w;
            copies<kB | kHalfW, 3, 0, 0, kBCopies>(cp, a_voff, b_voff);
            cp.b += BK * N_w;
        } else {
            copies<kB, 0, 0, 0, kBCopies>(cp, a_voff, b_voff);
            cp.b += BK * N_w;
            copies<kB, 1, 0, 0, kBCopies>(cp, a_voff, b_voff);
            cp.b += BK * N_w;
            copies<kB, 2, 0, 0, kBCopies>(cp, a_voff, b_voff);
            cp.b += BK * N_w;
            copies<kB, 3, 0, 0, kBCopies>(cp, a_voff, b_voff);
            cp.b += BK * N_w;
        }
        if (a_on)
            copies<kBA1, 0, 1, kBCopies, kBCopies + kAHalf>(cp, a_voff, b_voff);
    };
    auto setup = [&](int t) {
        int col0;
        bool hf;
        const MTile tl = decode(t, col0, hf);
        setup_from(tl, col0, hf);
    };

    // Claims (claim_issue: the atomic's round trip overlaps a K loop).  Launches that gather fc1 rows
    // or run at least four tasks per workgroup claim two ahead: t's successor is in the claim word
    // at every top barrier, the atomic issued there claims the task after it, and the successor's
    // tile (and gathered rows) are loaded during t's K loop.  The others claim one ahead, late: the
    // atomic issued at the top barrier claims t's successor and is read after the K loop, so with
    // few tasks per workgroup the short tasks at a table's end still go to the workgroups that free
    // up first.
    const bool ahead2 = gather != nullptr || total >= 4 * static_cast<int>(gridDim.x);
    MOE_PROBE(unsigned long long pr[kProbeFields] = {};
              const unsigned long long pr_k0 = __builtin_readcyclecounter();
              const unsigned long long pr_r0 = __builtin_amdgcn_s_memrealtime();
              unsigned long long pr_t = pr_k0, pr_b = 0, pr_k = 0, pr_s = 0, pr_u = 0;)
    int t = claim_task(claimed, task_ctr, xcd, blk, wave, lane);
    if (ahead2)
        claim_task(claimed, task_ctr, xcd, blk, wave, lane);  // t's successor, left in the claim word
    if (t < total) {
        fetch_rows(t);
        setup(t);
    }
    while (t < total) {
        const int rows = tile.row_end - tile.row_begin;
        // a half-width task leaves the second column half (wave column 1) without work
        const bool half_task = __builtin_amdgcn_readfirstlane(half ? 1 : 0) != 0;
        const int nb = __builtin_amdgcn_readfirstlane(
            half_task && wn == 1 ? 0 : min(kTM, max(0, ((rows + 31) / 32 - wm + kWM - 1) / kWM)));
        // the wave copies A rows 32 wave .. + 31, row block `wave`; row block v is used by wave row
        // v % kWM, so a wave that copies no A has at most one row block (nb <= 1) and a wave without
        // row blocks copies no A
        const int a_on = __builtin_amdgcn_readfirstlane(32 * wave < rows ? 1 : 0);

        f32x16_t acc[kTM][kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;

        // step 0 has landed; past this barrier every wave sees the claim of the following task
        // (two ahead), whose gathered source rows are loaded now and used after this task's K loop
        if (a_on)
            step_barrier<top_wait<true>()>();
        else
            step_barrier<top_wait<false>()>();
        MOE_PROBE(pr_b = __builtin_readcyclecounter(); pr[kProbeWait] += pr_b - pr_t;)
        int t_next = total;
        MTile tile_next{};
        int n0_next = 0;
        bool half_next = false;
        if (ahead2) {
            const int i = __builtin_amdgcn_readfirstlane(*claimed);
            t_next = ((i / blk) * kXcdCount + xcd) * blk + i % blk;
            if (t_next < total)
                tile_next = decode(t_next, n0_next, half_next);
        }
        const int claim_ret = claim_issue(task_ctr, xcd, wave, lane);
        if (t_next < total)
            fetch_rows(t_next);
        const LoopArgs g{a_base, b_base, a_voff, b_voff};
        bool ran = false;
        if constexpr (!kGated) {
            if (half_task) {
                // the waves of column half 1 copy A rows for the others but compute nothing
                if (nb == 0 && !a_on)
                    k_loop<kGated, 0, false, true>(acc, cp, g, N_w, KT);
                else if (nb == 0)
                    k_loop<kGated, 0, true, true>(acc, cp, g, N_w, KT);
                else if (nb == 1 && !a_on)
                    k_loop<kGated, 1, false, true>(acc, cp, g, N_w, KT);
                else if (nb == 1)
                    k_loop<kGated, 1, true, true>(acc, cp, g, N_w, KT);
                else
                    k_loop<kGated, kTM, true, true>(acc, cp, g, N_w, KT);
                ran = true;
            }
        }
        if (!ran) {
            if (nb == 0)
                k_loop<kGated, 0, false, false>(acc, cp, g, N_w, KT);
            else if (nb == 1 && !a_on)
                k_loop<kGated, 1, false, false>(acc, cp, g, N_w, KT);
            else if (nb == 1)
                k_loop<kGated, 1, true, false>(acc, cp, g, N_w, KT);
            else
                k_loop<kGated, kTM, true, false>(acc, cp, g, N_w, KT);
        }
        MOE_PROBE(pr_k = __builtin_readcyclecounter(); pr[kProbeLoop] += pr_k - pr_b; ++pr[kProbeTasks];
                  pr[kProbeSteps] += KT;
                  if (rows == BM && !half_task) { pr[kProbeLoopFull] += pr_k - pr_b; ++pr[kProbeTasksFull]; })
        const int claim_after = claim_value(claim_ret, wave);
        if (!ahead2) {
            // one ahead: the claim word (in wave 0's staging area, idle between its epilogues)
            // carries t's successor across one barrier
            if (wave == 0)
                *claimed = claim_after;
            __syncthreads();
            const int i = __builtin_amdgcn_readfirstlane(*claimed);
            t_next = ((i / blk) * kXcdCount + xcd) * blk + i % blk;
        }
        const MTile done = tile;
        const int done_n0 = n0;
        const bool done_skip = half_task && wn == 1;          // columns of the other half task
        t = t_next;
        // every wave is past its last read of this task's stages (and of the claim word)
        __syncthreads();
        MOE_PROBE(pr_s = __builtin_readcyclecounter(); pr[kProbeSync] += pr_s - pr_k;)
        if (t < total) {
            if (ahead2)
                setup_from(tile_next, n0_next, half_next);
            else
                setup(t);
        }
        MOE_PROBE(pr_u = __builtin_readcyclecounter(); pr[kProbeSetup] += pr_u - pr_s;)
        if (!done_skip && C != nullptr)
            store_output_staged<kGated>(acc, C, done, done_n0, N_out, lds0 + kRingBytes + wave * kOutWaveBytes,
                                         wm, wn, lane, chunk_done != nullptr);
        if constexpr (kGated) {
            if (save_g != nullptr) {
                store_output_staged<kGated, 1>(acc, save_g, done, done_n0, N_out,
                                               lds0 + kRingBytes + wave * kOutWaveBytes, wm, wn, lane,
                                               chunk_done != nullptr);
                store_output_staged<kGated, 2>(acc, save_u, done, done_n0, N_out,
                                               lds0 + kRingBytes + wave * kOutWaveBytes, wm, wn, lane,
                                               chunk_done != nullptr);
            }
        }
        if (chunk_done != nullptr)
            count_done_through(chunk_done, done.chunk, wave, lane);
        // two ahead: publish the claim after wave 0's last read of its staging area (which holds
        // the word)
        if (ahead2 && wave == 0)
            *claimed = claim_after;
        MOE_PROBE(pr_t = __builtin_readcyclecounter(); pr[kProbeEpilogue] += pr_t - pr_u;)
    }
#ifdef MOE_PHASE_PROBE
    if (wave == 0 && lane == 0) {
        pr[kProbeTotal] = __builtin_readcyclecounter() - pr_k0;
        pr[kProbeRealtime] = __builtin_amdgcn_s_memrealtime() - pr_r0;
        pr[kProbeWorkgroups] = 1;
        const int kind = kRole == 1 ? 2 : (kGated ? 1 : 0);
#pragma unroll
        for (int q = 0; q < kProbeFields; ++q)
            atomicAdd(&g_phase[kind][q], pr[q]);
    }
#endif
}
}  // namespace big

// Tile configurations.  Large (LDS DMA, above): one workgroup per CU, used when H % 256 == 0 and
// F % 128 == 0.  Small: 4 waves of 64 x 64, two workgroups per CU, two register-staged LDS stages,
// for other sizes (H % 128 == 0, F % 64 == 0).
using Fc1Small = Cfg<true, 2, 2, 2, 2, 2>;
using Fc2Small = Cfg<false, 2, 2, 2, 2, 2>;
#define FC1_SMALL grouped_gemm_bf16<true, 2, 2, 2, 2, 2>
#define FC2_SMALL grouped_gemm_bf16<false, 2, 2, 2, 2, 2>
constexpr int kBigFc1Cols = big::BNB / 2;    // output columns per fc1 task
constexpr int kBigFc2Cols = big::BNB;        // output columns per fc2 task
constexpr int kBigSmem = big::kSmemBytes;

// The large kernels run K loops of whole multiples of four steps (H / 32, F / 32).
bool use_big(int64_t H, int64_t F) { return H % kBigFc2Cols == 0 && F % kBigFc1Cols == 0; }

hipError_t ensure_smem_limits()
{
    static std::atomic<bool> done[64];    // per device: the attribute is set
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 64 && done[dev])
        return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&big::grouped_gemm_bf16_dma<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kBigSmem);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&big::grouped_gemm_bf16_dma<false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kBigSmem);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&big::grouped_gemm_bf16_dma<true, 1>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kBigSmem);
    if (e == hipSuccess && dev < 64)
        done[dev] = true;
    return e;
}

}  // namespace

int bf16_row_tile(int64_t H, int64_t F) { return use_big(H, F) ? big::BM : Fc1Small::BM; }
int bf16_fc2_cols_per_tile(int64_t H, int64_t F) { return use_big(H, F) ? kBigFc2Cols : Fc2Small::BN; }
bool bf16_supported(int64_t H, int64_t F) { return H % Fc2Small::BN == 0 && F % Fc1Small::BN == 0; }

hipError_t launch_fc1_bf16(const uint16_t* A, const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                           const MTile* tiles, const int32_t* tile_count, int64_t H, int64_t F,
                           int32_t* task_ctr, const int32_t* gather, int gather_k, uint16_t* save_g,
                           uint16_t* save_u, hipStream_t s)
{
    const int cu = device_info().cu_count;
    if (gather != nullptr && !use_big(H, F))
        return hipErrorInvalidValue;              // only the large-tile kernel gathers rows
    if (use_big(H, F)) {
        if (hipError_t e = ensure_smem_limits(); e != hipSuccess)
            return e;
        big::grouped_gemm_bf16_dma<true><<<dim3(cu), dim3(big::kThreads), kBigSmem, s>>>(
            A, wg, wu, h, tiles, tile_count, static_cast<int>(H), static_cast<int>(F), nullptr,
            task_ctr, gather, gather_k, save_g, save_u);
    } else {
        FC1_SMALL<<<dim3(2 * cu), dim3(Fc1Small::kThreads), Fc1Small::kSmemBytes, s>>>(
            A, wg, wu, h, tiles, tile_count, static_cast<int>(H), static_cast<int>(F), nullptr,
            task_ctr, save_g, save_u);
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
        big::grouped_gemm_bf16_dma<false><<<dim3(cu), dim3(big::kThreads), kBigSmem, s>>>(
            h, wd, nullptr, y, tiles, tile_count, static_cast<int>(F), static_cast<int>(H),
            chunk_done, task_ctr, nullptr, 1, nullptr, nullptr);
    } else {
        FC2_SMALL<<<dim3(2 * cu), dim3(Fc2Small::kThreads), Fc2Small::kSmemBytes, s>>>(
            h, wd, nullptr, y, tiles, tile_count, static_cast<int>(F), static_cast<int>(H),
            chunk_done, task_ctr, nullptr, nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_recompute_gu_bf16(const uint16_t* A, const int32_t* gather, int gather_k,
                                    const uint16_t* wg, const uint16_t* wu, uint16_t* g, uint16_t* u,
                                    const MTile* tiles, const int32_t* tile_count, int64_t H, int64_t F,
                                    int32_t* task_ctr, hipStream_t s)
{
    const int cu = device_info().cu_count;
    if (gather != nullptr && !use_big(H, F))
        return hipErrorInvalidValue;              // only the large-tile kernel gathers rows
    if (use_big(H, F)) {
        if (hipError_t e = ensure_smem_limits(); e != hipSuccess)
            return e;
        big::grouped_gemm_bf16_dma<true, 1><<<dim3(cu), dim3(big::kThreads), kBigSmem, s>>>(
            A, wg, wu, nullptr, tiles, tile_count, static_cast<int>(H), static_cast<int>(F), nullptr,
            task_ctr, gather, gather_k, g, u);
    } else {
        FC1_SMALL<<<dim3(2 * cu), dim3(Fc1Small::kThreads), Fc1Small::kSmemBytes, s>>>(
            A, wg, wu, nullptr, tiles, tile_count, static_cast<int>(H), static_cast<int>(F), nullptr,
            task_ctr, g, u);
    }
    return hipGetLastError();
}

}  // namespace moe

#ifdef MOE_PHASE_PROBE
int moe::probe_read_bf16(unsigned long long* out, int reset)
{
    if (out != nullptr &&
        hipMemcpyFromSymbol(out, HIP_SYMBOL(g_phase), sizeof(g_phase)) != hipSuccess)
        return 1;
    if (reset) {
        const unsigned long long zero[kProbeKindsBf16 * kProbeFields] = {};
        if (hipMemcpyToSymbol(HIP_SYMBOL(g_phase), zero, sizeof(zero)) != hipSuccess)
            return 1;
    }
    return 0;
}
#endif
