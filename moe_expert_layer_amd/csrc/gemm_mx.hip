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
// writes 32 E4M3 bytes plus one scale byte with the same encoder as the standalone kernel.
#include <atomic>

#include "common.h"
#include "gemm_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;

// ----------------------------------------------------------------------------------- standalone encoder

// One thread per 32-element block: shared exponent from the block's largest magnitude (integer
// arithmetic on the float bits), then each element encoded with it (e4m3_encode4_scaled).
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
            out[w / 4][w % 4] = e4m3_encode4_scaled(x[w][0], x[w][1], x[w][2], x[w][3], e);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + b * 32);
        dst[0] = out[0];
        dst[1] = out[1];
        scales[b] = static_cast<uint8_t>(e + 127);
    }
}

// bfloat16 activation rows -> OCP-MX, on the way into the gather.  One thread per (token, block of
// 32 along H): the block's 64 bytes are widened exactly to float32, the shared exponent comes from
// the largest magnitude, every element is encoded with it (the encoder above), and the 32
// code bytes and the scale byte go to the token's own row (pos null: token order, rows [T, H]) or
// to each of its k permuted rows pos[t k + j] (the permute step with the encoding on its gather;
// slots whose row lies outside [0, M) are skipped).
__global__ __launch_bounds__(kThreads) void mx_encode_bf16_rows_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t blocks_per_row, const int32_t* __restrict__ pos,
    int k, int64_t M, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales)
{
    const int64_t total = T * blocks_per_row;
    const int64_t H = blocks_per_row * 32;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
        const int64_t t = i / blocks_per_row;
        const int64_t b = i - t * blocks_per_row;
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + t * H + 32 * b);
        u32x4_t raw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            raw[q] = src[q];
        uint32_t amax = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int w = 0; w < 4; ++w)
                amax = max(amax, max((raw[q][w] << 16) & 0x7fffffffu, raw[q][w] & 0x7fff0000u));
        const int e = mx_shared_exponent(amax);
        u32x4_t out[2];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const uint32_t lo = raw[q][2 * w], hi = raw[q][2 * w + 1];
                out[q / 2][2 * (q % 2) + w] =
                    e4m3_encode4_scaled(__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u),
                                        __uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u), e);
            }
        const uint8_t sc = static_cast<uint8_t>(e + 127);
        if (pos == nullptr) {
            u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + t * H + 32 * b);
            dst[0] = out[0];
            dst[1] = out[1];
            scales[t * blocks_per_row + b] = sc;
        } else {
            for (int j = 0; j < k; ++j) {
                const int64_t p = pos[t * k + j];
                if (p < 0 || p >= M)
                    continue;
                u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + p * H + 32 * b);
                dst[0] = out[0];
                dst[1] = out[1];
                scales[p * blocks_per_row + b] = sc;
            }
        }
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

// fc1 epilogue of the 128-row tiles: the wave's 64 rows x 32 output columns go in fp32 into its LDS
// stage [64 rows][32 columns] (padded rows), then one lane per row encodes its 32-column block.
// kSwiGLU: the value of output (row, column) is swiglu(gate accumulator, up accumulator) (the GEMM);
// otherwise the gate accumulator itself (the encoder probe, which loads caller values there).  All
// threads of the workgroup call it (two workgroup barriers).
template <bool kSwiGLU>
__device__ __forceinline__ void store_h_small(const f32x16_t (&acc)[kTM][kTN], unsigned char* smem,
                                              uint8_t* __restrict__ Cq, uint8_t* __restrict__ Cq_sc,
                                              const MTile& tile, int n0, int N_out, int wave, int lane)
{
    const int wm = wave / kWN, wn = wave % kWN;
    const int h = lane >> 5;
    float* stage = reinterpret_cast<float*>(smem) + wave * 64 * kStageLd;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
            stage[row * kStageLd + (lane & 31)] = kSwiGLU ? swiglu(acc[i][0][r], acc[i][1][r]) : acc[i][0][r];
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
            out[w / 4][w % 4] = e4m3_encode4_scaled(x[w][0], x[w][1], x[w][2], x[w][3], e);
        const int hcol = n0 + 32 * wn;         // this wave's 32 output columns
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(Cq + static_cast<int64_t>(grow) * N_out + hcol);
        dst[0] = out[0];
        dst[1] = out[1];
        Cq_sc[static_cast<int64_t>(grow) * (N_out / 32) + hcol / 32] = static_cast<uint8_t>(e + 127);
    }
    __syncthreads();
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
            store_h_small<true>(acc, smem, Cq, Cq_sc, tile, n0, N_out, wave, lane);
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

// ----------------------------------------------------------------------------------- large tiles
//
// 256 rows x 256 weight columns per task (8 waves of 64 x 128, two per SIMD), for H and F multiples
// of 512.  The structure is the bfloat16 large-tile kernel's: global -> LDS copies
// (global_load_lds_dwordx4) into a four-stage ring, three K steps in flight, tasks claimed per XCD,
// the next task's first copies issued before the current epilogue.  A K step is 64 values (one
// scaled MFMA): A [256 rows][64 bytes], weights [64 k][columns] N-contiguous.  Weight fragments come
// from ds_read_b64_tr_b8 (measured: lane i of a 16-lane group receives byte e from source lane
// 2e + i / 8, byte i % 8, so 16 source lanes reading 8 rows x 16 columns hand every lane 8
// consecutive k of one column).  Block scales ride in their own two-slot LDS ring, one slot per 8
// K steps (16 scale blocks): A scales [256 rows][16] and weight scales [16][columns].
#ifdef MOE_PHASE_PROBE
// Per-task phase timing of the large-tile kernel below, compiled only into the probe library (the
// kernel does the same work): wave 0 of each workgroup sums cycle-counter differences at the
// points marked MOE_PROBE in scalar registers, and lane 0 adds them to g_phase_mx[kind] (0 fc2,
// 1 fc1) after the workgroup's last task, outside the task loop and its barriers.
__device__ unsigned long long g_phase_mx[kProbeKindsMx][kProbeFields];
#define MOE_PROBE(...) __VA_ARGS__
#else
#define MOE_PROBE(...)
#endif

namespace big {

constexpr int kWM = 4, kWN = 2, kTM = 2, kTN = 4;
constexpr int kWaves = kWM * kWN;
constexpr int kThreads = kWaves * 64;
constexpr int BM = kWM * kTM * 32;                    // 256
constexpr int BNB = kWN * kTN * 32;                   // 256
constexpr int BK = 64;
constexpr int kStages = 4;
constexpr int kABytes = BM * BK;
constexpr int kBBytes = BK * BNB;
constexpr int kBRing = kStages * kABytes;            // the A parts of all stages, then the B parts
constexpr int kRingBytes = kStages * (kABytes + kBBytes);   // 128 KiB
constexpr int kScaleSteps = 8;                        // K steps per scale slot (16 blocks of 32)
constexpr int kAScBytes = BM * 16;                    // [256 rows][16 blocks]
constexpr int kBScBytes = 16 * BNB;                   // [16 blocks][256 columns]
constexpr int kScSlotBytes = kAScBytes + kBScBytes;
constexpr int kScRing = kRingBytes;
constexpr int kOutBase = kScRing + 2 * kScSlotBytes;  // 144 KiB
constexpr int kOutWaveBytes = 2048;                   // epilogue staging per wave
constexpr int kSmemBytes = kOutBase + kWaves * kOutWaveBytes;   // 160 KiB
// A moves in pairs of K steps (rows of 128 bytes, whole cache lines): two pair stages of 32 KiB
// fill the A half of the ring.  The weights move per K step through the four B stages.
constexpr int kAPairBytes = 2 * kABytes;              // [256 rows][128 k]
constexpr int kACopies = kAPairBytes / 1024 / kWaves; // per wave per pair (4)
constexpr int kBCopies = kBBytes / 1024 / kWaves;     // 2
static_assert(kSmemBytes <= 160 * 1024, "LDS");

template <bool kGated>
struct BLayout {
    static constexpr int kMats = kGated ? 2 : 1;
    static constexpr int kRowBytes = BNB / kMats;       // one k row of one matrix: 128 or 256 bytes
    static constexpr int kChunks = kRowBytes / 16;
    static constexpr int kRowsPerCopy = 64 / kChunks;
    static constexpr int kMatBytes = BK * kRowBytes;
};

// 16-byte chunk position of logical chunk c in weight k row kr.  The transposing reads take 8
// consecutive k rows x 2 neighbouring chunks per 32 lanes; the XOR keeps those 16 pieces in
// distinct bank groups (rows of 256 bytes fill a bank window, rows of 128 bytes share one).
template <bool kGated>
__device__ __forceinline__ int bswz(int c, int kr)
{
    return BLayout<kGated>::kChunks == 16 ? c ^ ((kr & 7) << 1) : c ^ (((kr >> 1) & 3) << 1);
}


// Waits until at most N copies of this wave are in flight and for its LDS reads, then joins the
// workgroup barrier (one statement with a memory clobber).
template <int N>
__device__ __forceinline__ void step_barrier()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// Copy sources (uniform) and the LDS destinations of this wave's copies in stage 0 / pair stage 0
// / scale slot 0: A at the next pair to fetch (a pair advances it by 2 BK bytes), the weights at
// the next step (BK rows per step), the scales at the next block (sc_step bytes per block).
struct MxCopy {
    const uint8_t* a;
    const uint8_t* b;
    const uint8_t* sc;
    int64_t sc_step;
    uint32_t a_lds, b_lds, sc_lds;
};

// The copies of one K step: the scales of the block it opens into slot Q when kScale, its weights
// into B stage SB, and the A of a pair into pair stage QA when QA >= 0 (in that order); each
// source then moves on.
template <bool kScale, int Q, int SB, int QA>
__device__ __forceinline__ void mx_issue(MxCopy& c, const uint32_t (&a_voff)[kACopies],
                                         const uint32_t (&b_voff)[kBCopies], uint32_t sc_voff, int64_t N_w)
{
    if constexpr (kScale) {
        lds_copy16(c.sc, sc_voff, c.sc_lds + Q * kScSlotBytes);
        c.sc += c.sc_step;
    }
    if constexpr (SB >= 0) {
#pragma unroll
        for (int j = 0; j < kBCopies; ++j)
            lds_copy16(c.b, b_voff[j], c.b_lds + SB * kBBytes + j * 1024);
        c.b += BK * N_w;
    }
    if constexpr (QA >= 0) {
#pragma unroll
        for (int j = 0; j < kACopies; ++j)
            lds_copy16(c.a, a_voff[j], c.a_lds + QA * kAPairBytes + j * 1024);
        c.a += 2 * BK;
    }
}

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

__device__ __forceinline__ i32x8_t read_a(uint32_t p0, uint32_t p1)
{
    const u32x4_t lo = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(p0);
    const u32x4_t hi = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(p1);
    return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <int kRowBytes>
__device__ __forceinline__ i32x8_t read_b(uint32_t p)
{
    const i32x2_t r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_i32x2_t*>(p));
    const i32x2_t r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_i32x2_t*>(p + 8 * kRowBytes));
    const i32x2_t r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_i32x2_t*>(p + 32 * kRowBytes));
    const i32x2_t r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_i32x2_t*>(p + 40 * kRowBytes));
    return i32x8_t{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

__device__ __forceinline__ int read_u8(uint32_t p)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) uint8_t*>(p);
}

// Lane parts of the fragment and scale addresses.
// The lane's LDS addresses in stage 0 / scale slot 0 (row block 0 of this wave, k step 0 of the
// scale block).  Each is one register hidden from the optimiser, so the stage, slot, step and
// block parts below are immediate offsets of the LDS instructions.
struct LaneAddr {
    uint32_t a[2][2];         // A, pair half hp: chunks 4 hp + h and 4 hp + 2 + h of the lane's row
    uint32_t b[kTN];          // first transposing read of weight block j
    uint32_t asc;             // A scale byte: row * 16 + h
    uint32_t bsc;             // weight scale byte of block 0: column + h * row bytes (block j at
                              // the constant bsc_off<kGated>(j) from it)
};

// Offset of weight block j's scale bytes from block 0's (the lane's column moves by the block's
// column base, and for the up matrix of fc1 by half a scale slot).
template <bool kGated>
constexpr int bsc_off(int j)
{
    return kGated ? (j & 1) * (kBScBytes / 2) + 32 * (j >> 1) : 32 * j;
}

struct MxFrags {
    i32x8_t a[kTM];
    int sa[kTM];
};

// Fragments of K step position p (stage p % 4, scale slot P): A row blocks and their scales.
template <int NB, int P, int p>
__device__ __forceinline__ void read_a_frags(MxFrags& A, const LaneAddr& la)
{
    constexpr int S = p % kStages;                // pair stage S / 2, pair half S % 2
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        constexpr int kRowBlock = kWM * 32 * 128;
        A.a[i] = read_a(la.a[S % 2][0] + (S / 2) * kAPairBytes + i * kRowBlock,
                        la.a[S % 2][1] + (S / 2) * kAPairBytes + i * kRowBlock);
        A.sa[i] = read_u8(la.asc + P * kScSlotBytes + row_block<kWM>(i, 0) * 16 + 2 * p);
    }
}

// Weight blocks J0, J0 + 1 of K step position p and their scales.
template <bool kGated, int P, int p, int J0>
__device__ __forceinline__ void read_b_frags(i32x8_t (&b)[2], int (&sb)[2], const LaneAddr& la)
{
    using L = BLayout<kGated>;
    constexpr int S = p % kStages;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        b[jj] = read_b<L::kRowBytes>(la.b[J0 + jj] + S * kBBytes);
        sb[jj] = read_u8(la.bsc + bsc_off<kGated>(J0 + jj) + P * kScSlotBytes + 2 * p * L::kRowBytes);
    }
}

// Copy schedule.  After the barrier of step t: the scales of the block step t + 4 opens (when it
// opens one), the weights of step t + 4 (into the B stage step t has just freed) and, t odd, the A
// of pair (t + 3) / 2 (into the pair stage pair (t - 1) / 2 has just freed), in that order.  Copies
// are issued in a fixed order, so "what step t + 1 needs has landed" is "at most N copies are in
// flight", counted from that order: at an odd step, the weights of step t + 3 and any scales
// issued with them (none near the end of the task); at an even step, what step t + 1 needs was
// already complete at the previous barrier except for a task's first step, where 8 is exact.
constexpr bool scale_at(int u) { return u % kScaleSteps == 4; }   // step u issues scales
template <int p, bool kLast>
constexpr int mx_wait()
{
    if (p % 2 == 0)
        return 2 * kBCopies + kACopies;
    const bool w = !kLast || p + 3 < 2 * kScaleSteps;             // step t + 3 exists
    const bool sc = scale_at(p - 1) && (!kLast || p + 3 < 2 * kScaleSteps);
    return (w ? kBCopies : 0) + (sc ? 1 : 0);
}
// A wave whose A rows all lie past the tile's last row copies no A: step t + 1 has landed once at
// most the weights of steps t + 2 and t + 3 are in flight (scales issued among them are not
// counted, which only makes the wait longer).
template <int p, bool kLast>
constexpr int mx_wait_no_a()
{
    constexpr int kUnitSteps = 2 * kScaleSteps;
    return (!kLast || p + 2 < kUnitSteps ? kBCopies : 0) + (!kLast || p + 3 < kUnitSteps ? kBCopies : 0);
}

// Copy C of one K step's copy list (the scales of the block it opens into slot Q when kScale, its
// weights into B stage SB when SB >= 0, the A of a pair into pair stage QA when QA >= 0, in that
// order; the copy waits count on that order).  The sources move on in mx_advance, after the list.
template <bool kScale, int Q, int SB, int QA>
constexpr int mx_copy_count()
{
    return (kScale ? 1 : 0) + (SB >= 0 ? kBCopies : 0) + (QA >= 0 ? kACopies : 0);
}
template <bool kScale, int Q, int SB, int QA, int C>
__device__ __forceinline__ void mx_copy_one(const MxCopy& c, const uint32_t (&a_voff)[kACopies],
                                            const uint32_t (&b_voff)[kBCopies], uint32_t sc_voff)
{
    constexpr int c0 = kScale ? 1 : 0, c1 = c0 + (SB >= 0 ? kBCopies : 0);
    if constexpr (C < c0)
        lds_copy16(c.sc, sc_voff, c.sc_lds + Q * kScSlotBytes);
    else if constexpr (C < c1)
        lds_copy16(c.b, b_voff[C - c0], c.b_lds + SB * kBBytes + (C - c0) * 1024);
    else
        lds_copy16(c.a, a_voff[C - c1], c.a_lds + QA * kAPairBytes + (C - c1) * 1024);
}
template <bool kScale, int Q, int SB, int QA, int C0, int... Is>
__device__ __forceinline__ void mx_copies_impl(std::integer_sequence<int, Is...>, const MxCopy& c,
                                               const uint32_t (&a_voff)[kACopies],
                                               const uint32_t (&b_voff)[kBCopies], uint32_t sc_voff)
{
    (mx_copy_one<kScale, Q, SB, QA, C0 + Is>(c, a_voff, b_voff, sc_voff), ...);
}
// Copies C0 .. C1 - 1 of the list.
template <bool kScale, int Q, int SB, int QA, int C0, int C1>
__device__ __forceinline__ void mx_copies(const MxCopy& c, const uint32_t (&a_voff)[kACopies],
                                          const uint32_t (&b_voff)[kBCopies], uint32_t sc_voff)
{
    mx_copies_impl<kScale, Q, SB, QA, C0>(std::make_integer_sequence<int, C1 - C0>{}, c, a_voff, b_voff,
                                          sc_voff);
}
template <bool kScale, int SB, int QA>
__device__ __forceinline__ void mx_advance(MxCopy& c, int64_t N_w)
{
    if constexpr (kScale)
        c.sc += c.sc_step;
    if constexpr (SB >= 0)
        c.b += BK * N_w;
    if constexpr (QA >= 0)
        c.a += 2 * BK;
}

// Fragment read R of the next step (K step position p, scale slot P), in the order its first MFMAs
// consume them: R = 0 A row block 0, R = 1, 2 weight blocks 0, 1, R = 2 + i (i >= 1) A row block i.
template <bool kGated, int NB, int P, int p, int R>
__device__ __forceinline__ void mx_read_next(MxFrags& A, i32x8_t (&b01)[2], int (&sb01)[2], const LaneAddr& la)
{
    using L = BLayout<kGated>;
    constexpr int S = p % kStages;
    if constexpr (R == 1 || R == 2) {
        constexpr int jj = R - 1;
        b01[jj] = read_b<L::kRowBytes>(la.b[jj] + S * kBBytes);
        sb01[jj] = read_u8(la.bsc + bsc_off<kGated>(jj) + P * kScSlotBytes + 2 * p * L::kRowBytes);
    } else {
        constexpr int i = R == 0 ? 0 : R - 2;
        constexpr int kRowBlock = kWM * 32 * 128;
        A.a[i] = read_a(la.a[S % 2][0] + (S / 2) * kAPairBytes + i * kRowBlock,
                        la.a[S % 2][1] + (S / 2) * kAPairBytes + i * kRowBlock);
        A.sa[i] = read_u8(la.asc + P * kScSlotBytes + row_block<kWM>(i, 0) * 16 + 2 * p);
    }
}
template <bool kGated, int NB, int P, int p, int R0, int... Is>
__device__ __forceinline__ void mx_reads_impl(std::integer_sequence<int, Is...>, MxFrags& A, i32x8_t (&b01)[2],
                                              int (&sb01)[2], const LaneAddr& la)
{
    (mx_read_next<kGated, NB, P, p, R0 + Is>(A, b01, sb01, la), ...);
}

// Weight block 2 + jj of the current step (position p, slot P).
template <bool kGated, int P, int p, int jj>
__device__ __forceinline__ void mx_read_b23(i32x8_t (&b23)[2], int (&sb23)[2], const LaneAddr& la)
{
    using L = BLayout<kGated>;
    constexpr int S = p % kStages;
    b23[jj] = read_b<L::kRowBytes>(la.b[2 + jj] + S * kBBytes);
    sb23[jj] = read_u8(la.bsc + bsc_off<kGated>(2 + jj) + P * kScSlotBytes + 2 * p * L::kRowBytes);
}

// Weights as the first operand: the accumulator block is the transposed 32 x 32 output block, so a
// lane holds one output row (lane % 32) and four runs of four adjacent columns, 8 (r / 4) +
// 4 (lane / 32) + r % 4 (both operands have the same register layout, scale bytes included).
__device__ __forceinline__ void mx_mfma(f32x16_t& acc, const i32x8_t& a, int sa, const i32x8_t& b, int sb)
{
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc, 0, 0, 0, sb, 0, sa);
}

// Slot m before the barrier: MFMA m on weight blocks 0-1 (row block m / 2, block m % 2), then, in
// the first two slots, the read of weight block 2 + m of the current step.
template <bool kGated, int NB, int P, int q, int m>
__device__ __forceinline__ void mx_pre_slot(f32x16_t (&acc)[kTM][kTN], const MxFrags& Acur,
                                            const i32x8_t (&b01)[2], const int (&sb01)[2], i32x8_t (&b23)[2],
                                            int (&sb23)[2], const LaneAddr& la)
{
    mx_mfma(acc[m / 2][m % 2], Acur.a[m / 2], Acur.sa[m / 2], b01[m % 2], sb01[m % 2]);
    if constexpr (m < 2)
        mx_read_b23<kGated, P, q, m>(b23, sb23, la);
    __builtin_amdgcn_sched_barrier(0);
}
template <bool kGated, int NB, int P, int q, int... Ms>
__device__ __forceinline__ void mx_pre_slots(std::integer_sequence<int, Ms...>, f32x16_t (&acc)[kTM][kTN],
                                             const MxFrags& Acur, const i32x8_t (&b01)[2], const int (&sb01)[2],
                                             i32x8_t (&b23)[2], int (&sb23)[2], const LaneAddr& la)
{
    (mx_pre_slot<kGated, NB, P, q, Ms>(acc, Acur, b01, sb01, b23, sb23, la), ...);
}

// Slot m after the barrier: MFMA m on weight blocks 2-3, then this slot's share of the step's
// copies and of the next step's fragment reads (both spread over the first half of the slots, so
// the reads land well before the next step's first MFMAs).
template <bool kGated, int NB, int P, int q, int Pn, int qn, bool kScale, int Q, int SB, int QA, int m>
__device__ __forceinline__ void mx_post_slot(f32x16_t (&acc)[kTM][kTN], const MxFrags& Acur, MxFrags& Anext,
                                             const i32x8_t (&b23)[2], const int (&sb23)[2], i32x8_t (&b01)[2],
                                             int (&sb01)[2], const LaneAddr& la, const MxCopy& cp,
                                             const uint32_t (&a_voff)[kACopies],
                                             const uint32_t (&b_voff)[kBCopies], uint32_t sc_voff)
{
    constexpr int M = 2 * NB, RF = M / 2 > 0 ? M / 2 : 1;
    constexpr int NC = mx_copy_count<kScale, Q, SB, QA>(), NR = NB + 2;
    mx_mfma(acc[m / 2][2 + m % 2], Acur.a[m / 2], Acur.sa[m / 2], b23[m % 2], sb23[m % 2]);
    if constexpr (m < RF) {
        mx_copies<kScale, Q, SB, QA, m * NC / RF, (m + 1) * NC / RF>(cp, a_voff, b_voff, sc_voff);
        mx_reads_impl<kGated, NB, Pn, qn, m * NR / RF>(
            std::make_integer_sequence<int, (m + 1) * NR / RF - m * NR / RF>{}, Anext, b01, sb01, la);
    }
    __builtin_amdgcn_sched_barrier(0);
}
template <bool kGated, int NB, int P, int q, int Pn, int qn, bool kScale, int Q, int SB, int QA, int... Ms>
__device__ __forceinline__ void mx_post_slots(std::integer_sequence<int, Ms...>, f32x16_t (&acc)[kTM][kTN],
                                              const MxFrags& Acur, MxFrags& Anext, const i32x8_t (&b23)[2],
                                              const int (&sb23)[2], i32x8_t (&b01)[2], int (&sb01)[2],
                                              const LaneAddr& la, const MxCopy& cp,
                                              const uint32_t (&a_voff)[kACopies],
                                              const uint32_t (&b_voff)[kBCopies], uint32_t sc_voff)
{
    (mx_post_slot<kGated, NB, P, q, Pn, qn, kScale, Q, SB, QA, Ms>(acc, Acur, Anext, b23, sb23, b01, sb01, la,
                                                                  cp, a_voff, b_voff, sc_voff),
     ...);
}

// K step kt at position p of a 16-step unit (stage p % 4, pair stage p % 4 / 2; scales of the
// 8-step block in slot p / 8): the MFMAs of weight blocks 0-1 (fragments loaded during the
// previous step), each followed by a share of the reads of blocks 2-3; the barrier after which
// step kt + 1 has landed (W copies may stay in flight; none when W < 0); the MFMAs of blocks 2-3,
// each followed by a share of the copies (scales and weights of step kt + 4 when kCopyB, A of pair
// (kt + 3) / 2 when kCopyA) and of the next step's A and blocks 0-1 fragments.  Interleaving keeps
// the matrix pipe fed while a step's copies and reads issue.
template <bool kGated, int NB, int p, bool kCopyB, bool kCopyA, int W>
__device__ __forceinline__ void mx_step(f32x16_t (&acc)[kTM][kTN], const MxFrags& Acur, MxFrags& Anext,
                                        i32x8_t (&b01)[2], int (&sb01)[2], i32x8_t (&b23)[2],
                                        int (&sb23)[2], const LaneAddr& la, MxCopy& cp,
                                        const uint32_t (&a_voff)[kACopies],
                                        const uint32_t (&b_voff)[kBCopies], uint32_t sc_voff, int64_t N_w)
{
    constexpr int P = p / kScaleSteps, q = p % kScaleSteps;                  // slot, step in block
    constexpr int pn = (p + 1) % (2 * kScaleSteps);                          // the next step
    constexpr int Pn = pn / kScaleSteps, qn = pn % kScaleSteps;
    constexpr bool kScale = kCopyB && q == 4;
    constexpr int Q = 1 - P, SB = kCopyB ? p % kStages : -1, QA = kCopyA ? ((p + 3) / 2) % 2 : -1;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NB > 0)
        mx_pre_slots<kGated, NB, P, q>(std::make_integer_sequence<int, 2 * NB>{}, acc, Acur, b01, sb01, b23,
                                       sb23, la);
    if constexpr (W >= 0)
        step_barrier<W>();
    __builtin_amdgcn_sched_barrier(0);
    // after the last step the reads below read a stale stage whose fragments are never used
    if constexpr (NB > 0)
        mx_post_slots<kGated, NB, P, q, Pn, qn, kScale, Q, SB, QA>(std::make_integer_sequence<int, 2 * NB>{},
                                                                   acc, Acur, Anext, b23, sb23, b01, sb01, la,
                                                                   cp, a_voff, b_voff, sc_voff);
    else
        mx_copies<kScale, Q, SB, QA, 0, mx_copy_count<kScale, Q, SB, QA>()>(cp, a_voff, b_voff, sc_voff);
    mx_advance<kScale, SB, QA>(cp, N_w);
    __builtin_amdgcn_sched_barrier(0);
}

constexpr int kUnit = 2 * kScaleSteps;    // steps per unrolled unit: four stages, two scale slots

// One unit of 16 K steps; in the last unit of a task, the weight copies stop after position 11,
// the A copies after position 11, and the last step has no barrier.  kA = false: no A copies.
template <bool kGated, int NB, bool kLast, bool kA, int... Ps>
__device__ __forceinline__ void mx_unit_impl(std::integer_sequence<int, Ps...>, f32x16_t (&acc)[kTM][kTN],
                                             MxFrags& A0, MxFrags& A1, i32x8_t (&b01)[2], int (&sb01)[2],
                                             i32x8_t (&b23)[2], int (&sb23)[2], const LaneAddr& la,
                                             MxCopy& cp, const uint32_t (&a_voff)[kACopies],
                                             const uint32_t (&b_voff)[kBCopies], uint32_t sc_voff,
                                             int64_t N_w)
{
    ((Ps % 2 == 0
          ? mx_step<kGated, NB, Ps, !kLast || Ps + 4 < kUnit,
                    kA && Ps % 2 == 1 && (!kLast || Ps + 3 < kUnit),
                    kLast && Ps == kUnit - 1 ? -1 : kA ? mx_wait<Ps, kLast>() : mx_wait_no_a<Ps, kLast>()>(
                acc, A0, A1, b01, sb01, b23, sb23, la, cp, a_voff, b_voff, sc_voff, N_w)
          : mx_step<kGated, NB, Ps, !kLast || Ps + 4 < kUnit,
                    kA && Ps % 2 == 1 && (!kLast || Ps + 3 < kUnit),
                    kLast && Ps == kUnit - 1 ? -1 : kA ? mx_wait<Ps, kLast>() : mx_wait_no_a<Ps, kLast>()>(
                acc, A1, A0, b01, sb01, b23, sb23, la, cp, a_voff, b_voff, sc_voff, N_w)),
     ...);
}

template <bool kGated, int NB, bool kLast, bool kA>
__device__ __forceinline__ void mx_unit(f32x16_t (&acc)[kTM][kTN], MxFrags& A0, MxFrags& A1,
                                        i32x8_t (&b01)[2], int (&sb01)[2], i32x8_t (&b23)[2],
                                        int (&sb23)[2], const LaneAddr& la, MxCopy& cp,
                                        const uint32_t (&a_voff)[kACopies],
                                        const uint32_t (&b_voff)[kBCopies], uint32_t sc_voff, int64_t N_w)
{
    mx_unit_impl<kGated, NB, kLast, kA>(std::make_integer_sequence<int, kUnit>{}, acc, A0, A1, b01, sb01,
                                        b23, sb23, la, cp, a_voff, b_voff, sc_voff, N_w);
}

// Copies a task's setup leaves in flight once its step 0 has landed: the weights of steps 1 .. 3
// and A pair 1 (kA = false: the weights alone).
template <bool kA>
constexpr int top_wait() { return kA ? 3 * kBCopies + kACopies : 3 * kBCopies; }

// The K loop of one task.  KT is a multiple of 16; the caller issued the scales of block 0, A pair
// 0, the weights of steps 0 .. 3 and A pair 1 (in that order), cp points at pair 2, step 4 and
// block 1, and the caller has waited for step 0 (step_barrier<top_wait<kA>()>).  kA = false: the
// wave copies no A (its rows all lie past the tile's end).  Every LDS address is a lane base plus a
// constant.
template <bool kGated, int NB, bool kA>
__device__ __forceinline__ void mx_k_loop(f32x16_t (&acc)[kTM][kTN], const LaneAddr& la, MxCopy cp,
                                          const uint32_t (&a_voff)[kACopies],
                                          const uint32_t (&b_voff)[kBCopies], uint32_t sc_voff, int KT,
                                          int64_t N_w)
{
    static_assert(kStages == 4 && kUnit % kStages == 0, "the unrolled unit below");
    MxFrags A0, A1;
    i32x8_t b01[2], b23[2];
    int sb01[2], sb23[2];
    if constexpr (NB > 0) {
        read_a_frags<NB, 0, 0>(A0, la);
        read_b_frags<kGated, 0, 0, 0>(b01, sb01, la);
    }
    for (int kt = 0; kt < KT - kUnit; kt += kUnit)
        mx_unit<kGated, NB, false, kA>(acc, A0, A1, b01, sb01, b23, sb23, la, cp, a_voff, b_voff, sc_voff, N_w);
    mx_unit<kGated, NB, true, kA>(acc, A0, A1, b01, sb01, b23, sb23, la, cp, a_voff, b_voff, sc_voff, N_w);
}

// fc2 epilogue: bf16 rows through the wave's 2 KiB staging area, one 32 x 32 output block at a time
// (transposed accumulator blocks: a lane holds one row and four runs of four adjacent columns, each
// written as one 8-byte LDS store; rows of 64 bytes with 16-byte chunks XOR-swizzled by row / 4),
// read back as 16-byte row chunks and stored 16 bytes per lane.
__device__ __forceinline__ void store_y(const f32x16_t (&acc)[kTM][kTN], uint16_t* __restrict__ C,
                                        const MTile& tile, int n0, int N_out, uint32_t stage, int wm,
                                        int wn, int lane, bool through)
{
    const int lrow = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = g;                                    // 16-byte chunk of columns 8g .. 8g + 7
                const uint32_t a = stage + lrow * 64 + (((c ^ (lrow >> 2)) & 3) << 4) + 8 * lh;
                *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(a) =
                    u32x2_t{pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                            pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
            }
            const int chunk = lane & 3;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int row = (lane >> 2) + 16 * m;
                const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
                    stage + row * 64 + (((chunk ^ (row >> 2)) & 3) << 4));
                const int grow = tile.row_begin + row_block<kWM>(i, wm) + row;
                if (grow < tile.row_end) {
                    uint16_t* dst = C + static_cast<int64_t>(grow) * N_out + n0 + 128 * wn + 32 * j + 8 * chunk;
                    if (through)
                        store16_through(dst, v);
                    else
                        *reinterpret_cast<u32x4_t*>(dst) = v;
                }
            }
        }
}

// fc1 epilogue, in registers (transposed accumulator blocks): for output block ob of row block i a
// lane holds 16 of the 32 values of one row's MX block (runs of four columns 8 g + 4 (lane / 32) ..
// + 3), lane l + 32 the other 16.  The block's largest magnitude comes from the lane's 16 and one
// exchange with lane l ^ 32; each lane encodes its 16 values (OCP-MX, e4m3_encode4_scaled) into
// four words, the two halves swap two words so that each holds 16 consecutive code bytes (lane l
// columns 0 .. 15, lane l + 32 columns 16 .. 31), and lane l stores the scale byte.
//
// kSwiGLU: the value of output (row, column) is swiglu(gate accumulator, up accumulator) (the GEMM);
// otherwise the gate accumulator itself (the encoder probe, which loads caller values there).
template <bool kSwiGLU>
__device__ __forceinline__ void store_h(const f32x16_t (&acc)[kTM][kTN], uint8_t* __restrict__ Cq,
                                        uint8_t* __restrict__ Cq_sc, const MTile& tile, int n0,
                                        int N_out, int wm, int wn, int lane)
{
    const int lrow = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int ob = 0; ob < 2; ++ob) {          // output block: gate block 2 ob, up block 2 ob + 1
            __builtin_amdgcn_sched_barrier(0);
            float v[16];
            uint32_t amax = 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                v[r] = kSwiGLU ? swiglu(acc[i][2 * ob][r], acc[i][2 * ob + 1][r]) : acc[i][2 * ob][r];
                amax = max(amax, __float_as_uint(v[r]) & 0x7fffffffu);
            }
            amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 32)));
            const int e = mx_shared_exponent(amax);
            uint32_t w[4];
#pragma unroll
            for (int g = 0; g < 4; ++g)
                w[g] = e4m3_encode4_scaled(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3], e);
            // lane l keeps words 0, 1 (columns 0-3, 8-11) and takes lane l + 32's (4-7, 12-15);
            // lane l + 32 keeps words 2, 3 (20-23, 28-31) and takes lane l's (16-19, 24-27)
            const uint32_t x = static_cast<uint32_t>(__shfl_xor(static_cast<int>(lh ? w[0] : w[2]), 32));
            const uint32_t y = static_cast<uint32_t>(__shfl_xor(static_cast<int>(lh ? w[1] : w[3]), 32));
            const u32x4_t out = lh ? u32x4_t{x, w[2], y, w[3]} : u32x4_t{w[0], x, w[1], y};
            const int grow = tile.row_begin + row_block<kWM>(i, wm) + lrow;
            const int hcol = n0 + 64 * wn + 32 * ob;
            if (grow < tile.row_end) {
                *reinterpret_cast<u32x4_t*>(Cq + static_cast<int64_t>(grow) * N_out + hcol + 16 * lh) = out;
                if (lh == 0)
                    Cq_sc[static_cast<int64_t>(grow) * (N_out / 32) + hcol / 32] = static_cast<uint8_t>(e + 127);
            }
        }
}

template <bool kGated>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_mx_dma(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ A_sc,
    const uint8_t* __restrict__ B0, const uint8_t* __restrict__ B0_sc,
    const uint8_t* __restrict__ B1, const uint8_t* __restrict__ B1_sc,
    uint8_t* __restrict__ Cq, uint8_t* __restrict__ Cq_sc, uint16_t* __restrict__ Cy,
    const MTile* __restrict__ tiles, const int32_t* __restrict__ tile_count, int K, int N_out,
    int32_t* __restrict__ chunk_done, int32_t* __restrict__ task_ctr, const int32_t* __restrict__ gather,
    int gather_k)
{
    // gather (fc1 only, may be null): permuted row p of A (and of its scales) is row
    // gather[p] / gather_k of the matrices A and A_sc point at; null: row p.
    using L = BLayout<kGated>;
    constexpr int BN = kGated ? BNB / 2 : BNB;
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    int* const claimed = reinterpret_cast<int*>(smem + kOutBase);   // start of wave 0's staging
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char*)(smem)));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN;
    const int wn = wave % kWN;
    const int h = lane >> 5;
    const int n_mt = *tile_count;
    const int n_nt = N_out / BN;
    const int total = n_mt * n_nt;
    const int KT = K / BK;
    const int64_t N_w = N_out;
    const int KS = K / 32;

    // weight copy offsets (bytes from the step's first weight row): copy j covers k rows
    // kRowsPerCopy * (bi0 + j) .. + kRowsPerCopy - 1, lane / kChunks within them
    const int bi0 = kGated ? kBCopies * (wave % (kWaves / 2)) : kBCopies * wave;
    uint32_t b_voff[kBCopies];
#pragma unroll
    for (int j = 0; j < kBCopies; ++j) {
        const int kr = (bi0 + j) * L::kRowsPerCopy + lane / L::kChunks;
        const int c = bswz<kGated>(lane % L::kChunks, kr);
        b_voff[j] = static_cast<uint32_t>(kr) * static_cast<uint32_t>(N_out) + 16u * c;
    }
    MxCopy cp{};
    cp.a_lds = lds0 + kACopies * wave * 1024;
    cp.b_lds = lds0 + kBRing + (kGated ? (wave / (kWaves / 2)) * L::kMatBytes : 0) + bi0 * 1024;
    cp.sc_lds = lds0 + kScRing + (wave < 4 ? wave * 1024 : kAScBytes + (wave - 4) * 1024);
    // fragment and scale addresses (see LaneAddr)
    LaneAddr la;
    {
        const int r = lane & 31;
        const uint32_t rb = row_block<kWM>(0, wm);
        // A pair rows of 128 bytes keep logical chunk c at c ^ ((r >> 1) & 7)
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
            la.a[hp][0] = lds0 + rb * 128 + r * 128 + 16 * ((4 * hp + h) ^ ((r >> 1) & 7));
            la.a[hp][1] = lds0 + rb * 128 + r * 128 + 16 * ((4 * hp + 2 + h) ^ ((r >> 1) & 7));
        }
        la.asc = lds0 + kScRing + rb * 16 + r * 16 + h;
        const int g = lane >> 4, sl = lane & 15;
        const int hh = g >> 1;
        const int kr = 16 * hh + (sl >> 1);                     // first read; + 8, + 32, + 40
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int m = kGated ? (j & 1) : 0;
            const int cb = kGated ? 16 * kTN * wn + 32 * (j >> 1) : 32 * kTN * wn + 32 * j;
            const int col = cb + 16 * (g & 1) + 8 * (sl & 1);
            la.b[j] = lds0 + kBRing + m * L::kMatBytes + kr * L::kRowBytes + 16 * bswz<kGated>(col >> 4, kr) + (col & 15);
        }
        // block 0's scale column: the wave's first output column plus the lane's
        la.bsc = lds0 + kScRing + kAScBytes + h * L::kRowBytes + (kGated ? 16 * kTN * wn : 32 * kTN * wn) + (lane & 31);
        asm volatile("" : "+v"(la.a[0][0]), "+v"(la.a[0][1]), "+v"(la.a[1][0]), "+v"(la.a[1][1]),
                          "+v"(la.asc), "+v"(la.bsc));
#pragma unroll
        for (int j = 0; j < kTN; ++j)
            asm volatile("" : "+v"(la.b[j]));
    }

    const int xcd = blockIdx.x % kXcdCount;
    const int blk = gridDim.x / kXcdCount;
    MTile tile{};
    int n0 = 0;
    uint32_t a_voff[kACopies];
    uint32_t sc_voff = 0;
    // Gathered fc1 rows: the slot-list entries of this lane's A copy rows and A scale row for the
    // next task, loaded one task ahead (during the previous task's K loop) and first used in setup.
    int gsrc[kACopies + 1] = {};
    auto fetch_rows = [&](int tk) {
        if (gather == nullptr)
            return;
        int nt;
        const MTile tl = decode_task(tk, n_nt, tiles, nt);
        const int last = tl.row_end - tl.row_begin - 1;
#pragma unroll
        for (int j = 0; j < kACopies; ++j)
            gsrc[j] = gather[tl.row_begin + min(32 * wave + 8 * j + lane / 8, last)];
        if (wave < 4)
            gsrc[kACopies] = gather[tl.row_begin + min(64 * wave + lane, last)];
    };
    // setup_from: the task whose tile and column tile decode_task gave
    auto setup_from = [&](const MTile& tl, int nt) {
        tile = tl;
        n0 = nt * BN;
        const int rows = tile.row_end - tile.row_begin;
#pragma unroll
        for (int j = 0; j < kACopies; ++j) {
            const int r = 32 * wave + 8 * j + lane / 8;           // 8 lanes per 128-byte pair row
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            const int src = gather != nullptr ? gsrc[j] / gather_k : min(r, rows - 1);
            a_voff[j] = static_cast<uint32_t>(src) * static_cast<uint32_t>(K) + 16u * c;
        }
        const int64_t eoff = static_cast<int64_t>(tile.expert) * K * N_w;
        const int64_t esoff = static_cast<int64_t>(tile.expert) * KS * N_w;
        cp.a = gather != nullptr ? A : A + static_cast<int64_t>(tile.row_begin) * K;
        cp.b = (kGated && wave >= kWaves / 2 ? B1 : B0) + eoff + n0;
        if (wave < 4) {
            // A scale rows 64 wave .. + 63, 16 blocks (one scale block) per lane
            const int src = gather != nullptr ? gsrc[kACopies] / gather_k : min(64 * wave + lane, rows - 1);
            cp.sc = gather != nullptr ? A_sc : A_sc + static_cast<int64_t>(tile.row_begin) * KS;
            cp.sc_step = 16;
            sc_voff = static_cast<uint32_t>(src) * static_cast<uint32_t>(KS);
        } else {
            const int c = wave - 4;
            cp.sc_step = int64_t{16} * N_w;
            if (kGated) {
                // scale copy c: matrix c / 2, block rows 8 (c % 2) .. + 7, 8 lanes per 128-byte row
                cp.sc = (c >= 2 ? B1_sc : B0_sc) + esoff + n0 + int64_t{8} * (c & 1) * N_w;
                sc_voff = static_cast<uint32_t>(lane >> 3) * static_cast<uint32_t>(N_out) + 16u * (lane & 7);
            } else {
                // scale copy c: block rows 4 c .. + 3, 16 lanes per 256-byte row
                cp.sc = B0_sc + esoff + n0 + int64_t{4} * c * N_w;
                sc_voff = static_cast<uint32_t>(lane >> 4) * static_cast<uint32_t>(N_out) + 16u * (lane & 15);
            }
        }
        // scales of block 0 and A pair 0, the weights of steps 0 .. 3, A pair 1 (mx_k_loop's order);
        // a wave whose A rows all lie past the tile's end copies the scales and the weights alone
        // (the A source still moves on by the two pairs)
        if (32 * wave < rows)
            mx_issue<true, 0, -1, 0>(cp, a_voff, b_voff, sc_voff, N_w);
        else
            mx_issue<true, 0, -1, -1>(cp, a_voff, b_voff, sc_voff, N_w);
        mx_issue<false, 0, 0, -1>(cp, a_voff, b_voff, sc_voff, N_w);
        mx_issue<false, 0, 1, -1>(cp, a_voff, b_voff, sc_voff, N_w);
        mx_issue<false, 0, 2, -1>(cp, a_voff, b_voff, sc_voff, N_w);
        mx_issue<false, 0, 3, -1>(cp, a_voff, b_voff, sc_voff, N_w);
        if (32 * wave < rows)
            mx_issue<false, 0, -1, 1>(cp, a_voff, b_voff, sc_voff, N_w);
        else
            cp.a += 4 * BK;
    };
    auto setup = [&](int tk) {
        int nt;
        const MTile tl = decode_task(tk, n_nt, tiles, nt);
        setup_from(tl, nt);
    };

    // claims as in the bf16 kernel: two ahead when gathering fc1 rows or running at least four tasks
    // per workgroup (t's successor is in the claim word at every top barrier, and its tile entry is
    // loaded during t's K loop), else one ahead, read after the K loop
    const bool ahead2 = gather != nullptr || total >= 4 * static_cast<int>(gridDim.x);
    MOE_PROBE(unsigned long long pr[kProbeFields] = {};
              const unsigned long long pr_k0 = __builtin_readcyclecounter();
              const unsigned long long pr_r0 = __builtin_amdgcn_s_memrealtime();
              unsigned long long pr_t = pr_k0, pr_b = 0, pr_k = 0, pr_s = 0, pr_u = 0;)
    int t = claim_task(claimed, task_ctr, xcd, blk, wave, lane);
    if (ahead2)
        claim_task(claimed, task_ctr, xcd, blk, wave, lane);
    if (t < total) {
        fetch_rows(t);
        setup(t);
    }
    while (t < total) {
        const int rows = tile.row_end - tile.row_begin;
        const int nb = __builtin_amdgcn_readfirstlane(
            min(kTM, max(0, ((rows + 31) / 32 - wm + kWM - 1) / kWM)));
        // the wave copies A rows 32 wave .. + 31 (row block `wave`, used by wave row wave % kWM):
        // a wave that copies no A has at most one row block, a wave without row blocks copies none
        const int a_on = __builtin_amdgcn_readfirstlane(32 * wave < rows ? 1 : 0);
        f32x16_t acc[kTM][kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;
        // step 0 has landed; past this barrier every wave sees the claim of the following task,
        // whose gathered source rows are loaded now and used after this task's K loop
        if (a_on)
            step_barrier<top_wait<true>()>();
        else
            step_barrier<top_wait<false>()>();
        MOE_PROBE(pr_b = __builtin_readcyclecounter(); pr[kProbeWait] += pr_b - pr_t;)
        int t_next = total;
        MTile tile_next{};
        int nt_next = 0;
        if (ahead2) {
            const int ci = __builtin_amdgcn_readfirstlane(*claimed);
            t_next = ((ci / blk) * kXcdCount + xcd) * blk + ci % blk;
            if (t_next < total)
                tile_next = decode_task(t_next, n_nt, tiles, nt_next);
        }
        const int claim_ret = claim_issue(task_ctr, xcd, wave, lane);
        if (t_next < total)
            fetch_rows(t_next);
        if (nb == 0)
            mx_k_loop<kGated, 0, false>(acc, la, cp, a_voff, b_voff, sc_voff, KT, N_w);
        else if (nb == 1 && !a_on)
            mx_k_loop<kGated, 1, false>(acc, la, cp, a_voff, b_voff, sc_voff, KT, N_w);
        else if (nb == 1)
            mx_k_loop<kGated, 1, true>(acc, la, cp, a_voff, b_voff, sc_voff, KT, N_w);
        else
            mx_k_loop<kGated, 2, true>(acc, la, cp, a_voff, b_voff, sc_voff, KT, N_w);
        MOE_PROBE(pr_k = __builtin_readcyclecounter(); pr[kProbeLoop] += pr_k - pr_b; ++pr[kProbeTasks];
                  pr[kProbeSteps] += KT;
                  if (rows == BM) { pr[kProbeLoopFull] += pr_k - pr_b; ++pr[kProbeTasksFull]; })
        const int claim_after = claim_value(claim_ret, wave);
        if (!ahead2) {
            if (wave == 0)
                *claimed = claim_after;
            __syncthreads();
            const int ci = __builtin_amdgcn_readfirstlane(*claimed);
            t_next = ((ci / blk) * kXcdCount + xcd) * blk + ci % blk;
        }
        const MTile done = tile;
        const int done_n0 = n0;
        t = t_next;
        __syncthreads();
        MOE_PROBE(pr_s = __builtin_readcyclecounter(); pr[kProbeSync] += pr_s - pr_k;)
        if (t < total) {
            if (ahead2)
                setup_from(tile_next, nt_next);
            else
                setup(t);
        }
        MOE_PROBE(pr_u = __builtin_readcyclecounter(); pr[kProbeSetup] += pr_u - pr_s;)
        const uint32_t stg = lds0 + kOutBase + wave * kOutWaveBytes;
        if constexpr (kGated)
            store_h<true>(acc, Cq, Cq_sc, done, done_n0, N_out, wm, wn, lane);
        else
            store_y(acc, Cy, done, done_n0, N_out, stg, wm, wn, lane, chunk_done != nullptr);
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
#pragma unroll
        for (int q = 0; q < kProbeFields; ++q)
            atomicAdd(&g_phase_mx[kGated ? 1 : 0][q], pr[q]);
    }
#endif
}

// The fc1 epilogue's encoder on caller values: workgroup (x, y) takes output columns [128 x, 128 x +
// 128) and rows [256 y, 256 y + 256) of v [rows, cols], puts each value in the gate accumulator
// register that holds that output in the GEMM (transposed 32 x 32 blocks: lane row lane % 32,
// columns 8 (r / 4) + 4 (lane / 32) + r % 4), and runs store_h on them without the SwiGLU.
__global__ __launch_bounds__(kThreads, 1) void mx_epilogue_probe(const float* __restrict__ v, int rows,
                                                                 int cols, uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    MTile tile{};
    tile.row_begin = static_cast<int>(blockIdx.y) * BM;
    tile.row_end = min(rows, tile.row_begin + BM);
    const int n0 = static_cast<int>(blockIdx.x) * (BNB / 2);
    f32x16_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = tile.row_begin + row_block<kWM>(i, wm) + (lane & 31);
                const int col = n0 + 64 * wn + 32 * ob + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                acc[i][2 * ob][r] = row < tile.row_end ? v[static_cast<int64_t>(row) * cols + col] : 0.0f;
            }
    store_h<false>(acc, codes, scales, tile, n0, cols, wm, wn, lane);
}

}  // namespace big

// The 128-row-tile fc1 epilogue's encoder on caller values (see big::mx_epilogue_probe): workgroup
// (x, y) takes output columns [64 x, 64 x + 64) and rows [128 y, 128 y + 128).
__global__ __launch_bounds__(kThreads) void mx_epilogue_probe_small(const float* __restrict__ v, int rows,
                                                                    int cols, uint8_t* __restrict__ codes,
                                                                    uint8_t* __restrict__ scales)
{
    __shared__ __attribute__((aligned(16))) unsigned char smem[kEpiBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    MTile tile{};
    tile.row_begin = static_cast<int>(blockIdx.y) * BM;
    tile.row_end = min(rows, tile.row_begin + BM);
    const int n0 = static_cast<int>(blockIdx.x) * (BNB / 2);
    f32x16_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = tile.row_begin + wm * kTM * 32 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int col = n0 + 32 * wn + (lane & 31);
            acc[i][0][r] = row < tile.row_end ? v[static_cast<int64_t>(row) * cols + col] : 0.0f;
        }
    store_h_small<false>(acc, smem, codes, scales, tile, n0, cols, wave, lane);
}

// The large kernels run K loops of whole 16-step units (H / 64, F / 64 multiples of 16).
bool mx_use_big(int64_t H, int64_t F) { return H % 1024 == 0 && F % 1024 == 0; }

unsigned persistent_grid() { return static_cast<unsigned>(device_info().cu_count * 2); }

hipError_t ensure_smem_limits()
{
    static std::atomic<bool> done[64];    // per device: the attribute is set
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
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&big::grouped_gemm_mx_dma<true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, big::kSmemBytes);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&big::grouped_gemm_mx_dma<false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, big::kSmemBytes);
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

hipError_t launch_mx_encode_bf16_rows(const uint16_t* x, int64_t T, int64_t H, const int32_t* pos,
                                     int64_t k, int64_t M, uint8_t* codes, uint8_t* scales, hipStream_t s)
{
    const int64_t total = T * (H / 32);
    if (total <= 0)
        return hipSuccess;
    const int64_t want = (total + kThreads - 1) / kThreads;
    const int64_t cap = static_cast<int64_t>(device_info().cu_count) * 16;
    mx_encode_bf16_rows_kernel<<<dim3(static_cast<unsigned>(want < cap ? want : cap)), dim3(kThreads), 0, s>>>(
        x, T, H / 32, pos, static_cast<int>(k), M, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx_epilogue_probe(const float* v, int64_t rows, int64_t cols, bool large_tiles,
                                   uint8_t* codes, uint8_t* scales, hipStream_t s)
{
    const int bn = large_tiles ? big::BNB / 2 : BNB / 2;
    const int bm = large_tiles ? big::BM : BM;
    if (rows <= 0)
        return hipSuccess;
    if (cols % bn != 0 || rows * cols > (int64_t{1} << 28))
        return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(cols / bn), static_cast<unsigned>(ceil_div(rows, bm)));
    if (large_tiles)
        big::mx_epilogue_probe<<<grid, dim3(big::kThreads), 0, s>>>(v, static_cast<int>(rows),
                                                                    static_cast<int>(cols), codes, scales);
    else
        mx_epilogue_probe_small<<<grid, dim3(kThreads), 0, s>>>(v, static_cast<int>(rows),
                                                                static_cast<int>(cols), codes, scales);
    return hipGetLastError();
}

int mx_fc2_cols_per_tile(int64_t H, int64_t F) { return mx_use_big(H, F) ? big::BNB : BNB; }
int mx_row_tile(int64_t H, int64_t F) { return mx_use_big(H, F) ? big::BM : BM; }

hipError_t launch_fc1_mx(const uint8_t* A, const uint8_t* a_scale, const uint8_t* wg,
                         const uint8_t* wg_scale, const uint8_t* wu, const uint8_t* wu_scale,
                         uint8_t* h, uint8_t* h_scale, const MTile* tiles,
                         const int32_t* tile_count, int64_t H, int64_t F, int32_t* task_ctr,
                         const int32_t* gather, int gather_k, hipStream_t s)
{
    if (hipError_t e = ensure_smem_limits(); e != hipSuccess)
        return e;
    if (gather != nullptr && !mx_use_big(H, F))
        return hipErrorInvalidValue;              // only the large-tile kernel gathers rows
    if (mx_use_big(H, F)) {
        big::grouped_gemm_mx_dma<true><<<dim3(device_info().cu_count), dim3(big::kThreads), big::kSmemBytes, s>>>(
            A, a_scale, wg, wg_scale, wu, wu_scale, h, h_scale, nullptr, tiles, tile_count,
            static_cast<int>(H), static_cast<int>(F), nullptr, task_ctr, gather, gather_k);
        return hipGetLastError();
    }
    grouped_gemm_mx<true><<<dim3(persistent_grid()), dim3(kThreads), kSmemBytes, s>>>(
        A, a_scale, wg, wg_scale, wu, wu_scale, h, h_scale, nullptr, tiles, tile_count,
        static_cast<int>(H), static_cast<int>(F), nullptr);
    return hipGetLastError();
}

hipError_t launch_fc2_mx(const uint8_t* h, const uint8_t* h_scale, const uint8_t* wd,
                         const uint8_t* wd_scale, uint16_t* y, const MTile* tiles,
                         const int32_t* tile_count, int64_t H, int64_t F, int32_t* chunk_done,
                         int32_t* task_ctr, hipStream_t s)
{
    if (hipError_t e = ensure_smem_limits(); e != hipSuccess)
        return e;
    if (mx_use_big(H, F)) {
        big::grouped_gemm_mx_dma<false><<<dim3(device_info().cu_count), dim3(big::kThreads), big::kSmemBytes, s>>>(
            h, h_scale, wd, wd_scale, nullptr, nullptr, nullptr, nullptr, y, tiles, tile_count,
            static_cast<int>(F), static_cast<int>(H), chunk_done, task_ctr, nullptr, 1);
        return hipGetLastError();
    }
    grouped_gemm_mx<false><<<dim3(persistent_grid()), dim3(kThreads), kSmemBytes, s>>>(
        h, h_scale, wd, wd_scale, nullptr, nullptr, nullptr, nullptr, y, tiles, tile_count,
        static_cast<int>(F), static_cast<int>(H), chunk_done);
    return hipGetLastError();
}

}  // namespace moe

#ifdef MOE_PHASE_PROBE
int moe::probe_read_mx(unsigned long long* out, int reset)
{
    if (out != nullptr &&
        hipMemcpyFromSymbol(out, HIP_SYMBOL(g_phase_mx), sizeof(g_phase_mx)) != hipSuccess)
        return 1;
    if (reset) {
        const unsigned long long zero[kProbeKindsMx * kProbeFields] = {};
        if (hipMemcpyToSymbol(HIP_SYMBOL(g_phase_mx), zero, sizeof(zero)) != hipSuccess)
            return 1;
    }
    return 0;
}
#endif
