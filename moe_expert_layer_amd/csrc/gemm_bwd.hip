// Grouped GEMMs of the expert layer's backward on gfx950 MFMA (bf16 operands, fp32 accumulation
// on v_mfma_f32_32x32x16_bf16).  The page "NPU Training Operators - MC2" wraps forward and backward
// of every step of 执行路径 in its fused ops; its 验证项 list the fc1 / fc2 gradients among the
// checks.  With the permuted rows p (expert e(p)), the forward's g = x Wg, u = x Wu and the routing
// probability w(p) of the slot behind row p:
//
//   down dgrad (N = F):  d[p, f] = sum_h dout_perm[p, h] Wd[e][f, h]          (dout Wd^T)
//       epilogue: sg = sigmoid(g), h = g sg u, dh = w d,
//                 dg = dh u sg (1 + g (1 - sg)), du = dh g sg   -> dgu [M, 2F] = [dg | du]
//                 hp = w h                                      -> hp [M, F]
//                 sum over the wave's 64 columns of h d          -> dprobs partial [M, F / 64]
//   gate/up dgrad (N = H): dx_perm[p, h] = sum_f dg[p, f] Wg[e][h, f] + du[p, f] Wu[e][h, f]
//   weight gradients (per expert, K = the expert's rows, in ascending p):
//       dWd[e][f, h] = sum_p hp[p, f] dout_perm[p, h]
//       dWg[e][h, f] = sum_p x_perm[p, h] dg[p, f],   dWu likewise with du
//
// Tiles of 128 x 128 outputs, 4 waves of 64 x 64 (2 x 2 MFMA blocks of 32 x 32), K steps of 64,
// two LDS stages filled through registers, two workgroups per CU.  In LDS both operands are
// K-contiguous rows of 64 values with XOR-swizzled 16-byte chunks, read as 16-byte fragments.
//   - dgrad: both operands are K-contiguous in memory (activation rows; weight rows of Wd[e] as
//     [F][H], of Wg[e] / Wu[e] as [H][F]) and are copied as they are;
//   - weight gradients: both operands are rows over K (activations [M][cols]); each thread loads 4
//     consecutive rows of 8 columns and transposes them in registers (v_perm_b32) into 8 columns of
//     4 consecutive k; rows past the expert's last row load as zero.
// Every output element sums its whole contraction in one workgroup in a fixed order, so results
// are deterministic.  Tasks: dgrad over (row tile, column tile) of the row-tile table, weight
// gradients over (expert, column tile of the gradient's rows, column tile of its columns) in groups
// of 8 row tiles; consecutive tasks go to one XCD (workgroup b runs on XCD b % 8), so the
// workgroups of an XCD share operand strips in its L2.
#include <atomic>
#include <utility>

#include "common.h"
#include "gemm_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWM = 2, kWN = 2, kTM = 2, kTN = 2;
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kTileBytes = BM * BK * 2;        // one operand, one stage: 16 KiB
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kSmemBytes = 2 * kStageBytes;    // 64 KiB

enum Epi { kEpiDown = 0, kEpiGateUp = 1, kEpiWgrad = 2 };

#ifdef MOE_PHASE_PROBE
// Per-task phase timing of the LDS-DMA kernels below, compiled only into the probe library (the
// kernels do the same work): wave 0 of each workgroup sums cycle-counter differences in scalar
// registers and lane 0 adds them to g_phase_bwd[kind] (0 weight gradients, 1 down dgrad, 2 gate/up
// dgrad) after the workgroup's last task, outside the task loop and its barriers.
__device__ unsigned long long g_phase_bwd[kProbeKindsBwd][kProbeFields];
#define MOE_PROBE(...) __VA_ARGS__
#else
#define MOE_PROBE(...)
#endif

// Byte offset of element (row, k) in a [128 rows][64 k] bf16 tile, 16-byte chunks XOR-swizzled by row.
__device__ __forceinline__ int tile_off(int row, int k)
{
    return row * 128 + ((((k >> 3) ^ row) & 7) << 4) + ((k & 7) << 1);
}

__device__ __forceinline__ float sigmoid_f(float z)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

struct BwdArgs {
    // A: dgrad, K-contiguous rows (row stride lda); weight gradients, rows over K (stride lda)
    const uint16_t* a;
    int64_t lda;
    // B: dgrad, weight rows of expert e at b0 + e * b_estride + n * ldb (k < kseg) and
    // b1 + e * b_estride + n * ldb (k >= kseg); weight gradients, rows over K at b0 (stride ldb)
    const uint16_t* b0;
    const uint16_t* b1;
    int64_t ldb;
    int64_t b_estride;
    int kseg;
    int K;                        // dgrad contraction length
    int N;                        // output columns
    int Mo;                       // weight gradients: output rows
    const MTile* tiles;           // dgrad row tiles (128 rows)
    const int32_t* tile_count;
    const int32_t* offsets;       // weight gradients: expert e owns rows [offsets[e], offsets[e+1])
    int E;
    void* c;                      // dgu (down dgrad), dx_perm (gate/up dgrad), dW (fp32)
    const uint16_t* g;            // down dgrad: recomputed g, u [M, F]; row weights w(p)
    const uint16_t* u;
    const float* prow;
    uint16_t* hp;                 // down dgrad: w h [M, F]
    float* partial;               // down dgrad: [M, F / 64]
};

// Register staging of one K step.  K-contiguous operand: 4 chunks of 16 bytes, rows tid / 8 + 32 i,
// k chunk tid % 8.  Rows over K: 4 rows (4 (tid % 16) + r) of the 8 columns 8 (tid / 16) ...
struct Stage {
    u32x4_t a[4];
    u32x4_t b[4];
};

template <int kEpi>
struct Src {
    // dgrad: per chunk row pointers (k = 0 of segment 0 and of segment 1)
    const uint16_t* a_row[4];
    const uint16_t* b_row0[4];
    const uint16_t* b_row1[4];
    // weight gradients: column chunk pointers at the expert's first row, rows available
    const uint16_t* a_col;
    const uint16_t* b_col;
    int kend;
};

template <int kEpi>
__device__ __forceinline__ void load_step(Stage& st, const Src<kEpi>& s, const BwdArgs& g, int k0,
                                          int tid)
{
    if constexpr (kEpi != kEpiWgrad) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            st.a[i] = *reinterpret_cast<const u32x4_t*>(s.a_row[i] + k0);
            const uint16_t* bp = k0 < g.kseg ? s.b_row0[i] + k0 : s.b_row1[i] + (k0 - g.kseg);
            st.b[i] = *reinterpret_cast<const u32x4_t*>(bp);
        }
    } else {
        const int kk = k0 + 4 * (tid % 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool ok = kk + r < s.kend;
            const u32x4_t z = {0u, 0u, 0u, 0u};
            st.a[r] = ok ? *reinterpret_cast<const u32x4_t*>(s.a_col + static_cast<int64_t>(kk + r) * g.lda) : z;
            st.b[r] = ok ? *reinterpret_cast<const u32x4_t*>(s.b_col + static_cast<int64_t>(kk + r) * g.ldb) : z;
        }
    }
}

// 4 rows x 8 columns (r[row] holds the row's 8 values) -> 8 columns of 4 consecutive k
__device__ __forceinline__ void store_transposed(unsigned char* T, const u32x4_t (&r)[4], int c0, int k0)
{
#pragma unroll
    for (int col = 0; col < 8; ++col) {
        const int d = col >> 1;
        const uint32_t sel = (col & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t w0 = __builtin_amdgcn_perm(r[1][d], r[0][d], sel);
        const uint32_t w1 = __builtin_amdgcn_perm(r[3][d], r[2][d], sel);
        *reinterpret_cast<u32x2_t*>(T + tile_off(c0 + col, k0)) = u32x2_t{w0, w1};
    }
}

template <int kEpi>
__device__ __forceinline__ void store_step(unsigned char* smem, int buf, const Stage& st, int tid)
{
    unsigned char* As = smem + buf * kStageBytes;
    unsigned char* Bs = As + kTileBytes;
    if constexpr (kEpi != kEpiWgrad) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = tile_off(tid / 8 + 32 * i, 8 * (tid % 8));
            *reinterpret_cast<u32x4_t*>(As + off) = st.a[i];
            *reinterpret_cast<u32x4_t*>(Bs + off) = st.b[i];
        }
    } else {
        store_transposed(As, st.a, 8 * (tid / 16), 4 * (tid % 16));
        store_transposed(Bs, st.b, 8 * (tid / 16), 4 * (tid % 16));
    }
}

__device__ __forceinline__ void load_frags(bf16x8_t (&af)[kTM], bf16x8_t (&bf)[kTN],
                                           const unsigned char* As, const unsigned char* Bs, int wm,
                                           int wn, int lane, int ks)
{
    const int kk = ks * 16 + 8 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + tile_off(32 * (kWM * i + wm) + (lane & 31), kk));
#pragma unroll
    for (int j = 0; j < kTN; ++j)
        bf[j] = *reinterpret_cast<const bf16x8_t*>(Bs + tile_off(64 * wn + 32 * j + (lane & 31), kk));
}

__device__ __forceinline__ void mfmas(f32x16_t (&acc)[kTM][kTN], const bf16x8_t (&af)[kTM],
                                      const bf16x8_t (&bf)[kTN])
{
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
}

// The K loop: KT steps of 64; the global loads of step kt + 1 and the fragment reads of sub-step
// ks + 1 are in flight while the MFMAs of kt / ks run.
template <int kEpi>
__device__ __forceinline__ void k_loop(f32x16_t (&acc)[kTM][kTN], unsigned char* smem,
                                       const Src<kEpi>& s, const BwdArgs& g, int KT, int tid,
                                       int wm, int wn, int lane)
{
    if (KT <= 0)
        return;
    Stage st;
    load_step<kEpi>(st, s, g, 0, tid);
    store_step<kEpi>(smem, 0, st, tid);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT)
            load_step<kEpi>(st, s, g, (kt + 1) * BK, tid);
        const unsigned char* As = smem + cur * kStageBytes;
        const unsigned char* Bs = As + kTileBytes;
        bf16x8_t af[2][kTM], bf[2][kTN];
        load_frags(af[0], bf[0], As, Bs, wm, wn, lane, 0);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ks += 2) {
            load_frags(af[1], bf[1], As, Bs, wm, wn, lane, ks + 1);
            mfmas(acc, af[0], bf[0]);
            if (ks + 2 < BK / 16)
                load_frags(af[0], bf[0], As, Bs, wm, wn, lane, ks + 2);
            mfmas(acc, af[1], bf[1]);
        }
        if (kt + 1 < KT)
            store_step<kEpi>(smem, cur ^ 1, st, tid);
        __syncthreads();
    }
}

// Task t of this workgroup (consecutive tasks on one XCD), or -1.
__device__ __forceinline__ int task_of_block(int total)
{
    const int per = (total + kXcdCount - 1) / kXcdCount;
    const int b = blockIdx.x;
    const int local = b / kXcdCount;
    const int t = (b % kXcdCount) * per + local;
    return local < per && t < total ? t : -1;
}

template <int kEpi>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_bwd(BwdArgs g)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN;
    const int wn = wave % kWN;
    const int n_nt = g.N / BN;

    Src<kEpi> s{};
    MTile tile{};
    int n0 = 0, m0 = 0, e = 0, KT = 0;
    if constexpr (kEpi != kEpiWgrad) {
        const int total = *g.tile_count * n_nt;
        const int t = task_of_block(total);
        if (t < 0)
            return;
        int nt;
        tile = decode_task(t, n_nt, g.tiles, nt);
        n0 = nt * BN;
        e = tile.expert;
        KT = g.K / BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = tid / 8 + 32 * i;
            const int row = min(tile.row_begin + r, tile.row_end - 1);   // rows past the end: never stored
            const int c = 8 * (tid % 8);
            s.a_row[i] = g.a + static_cast<int64_t>(row) * g.lda + c;
            const int64_t boff = static_cast<int64_t>(e) * g.b_estride + static_cast<int64_t>(n0 + r) * g.ldb + c;
            s.b_row0[i] = g.b0 + boff;
            s.b_row1[i] = g.b1 + boff;
        }
    } else {
        const int n_mt = g.Mo / BM;
        const int per_e = n_mt * n_nt;
        const int t = task_of_block(per_e * g.E);
        if (t < 0)
            return;
        e = t / per_e;
        const int tl = t - e * per_e;
        constexpr int kGroup = 8;                                   // row tiles per group
        const int grp = tl / (kGroup * n_nt);
        const int first = grp * kGroup;
        const int gsz = min(kGroup, n_mt - first);
        const int idx = tl - grp * kGroup * n_nt;
        m0 = (first + idx % gsz) * BM;
        n0 = (idx / gsz) * BN;
        const int k_begin = g.offsets[e];
        s.kend = g.offsets[e + 1] - k_begin;
        KT = (s.kend + BK - 1) / BK;
        const int c = 8 * (tid / 16);
        s.a_col = g.a + static_cast<int64_t>(k_begin) * g.lda + m0 + c;
        s.b_col = g.b0 + static_cast<int64_t>(k_begin) * g.ldb + n0 + c;
    }

    f32x16_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;
    k_loop<kEpi>(acc, smem, s, g, KT, tid, wm, wn, lane);

    // Lane holds column lane % 32 of each 32 x 32 block, rows 8 (r / 4) + 4 (lane / 32) + r % 4.
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int lrow = 32 * (kWM * i + wm) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if constexpr (kEpi == kEpiWgrad) {
                float* C = static_cast<float*>(g.c) + (static_cast<int64_t>(e) * g.Mo + m0 + lrow) * g.N;
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    C[n0 + 64 * wn + 32 * j + (lane & 31)] = acc[i][j][r];
            } else if constexpr (kEpi == kEpiGateUp) {
                const int p = tile.row_begin + lrow;
                if (p < tile.row_end) {
                    uint16_t* C = static_cast<uint16_t*>(g.c) + static_cast<int64_t>(p) * g.N;
#pragma unroll
                    for (int j = 0; j < kTN; ++j)
                        C[n0 + 64 * wn + 32 * j + (lane & 31)] = f32_to_bf16(acc[i][j][r]);
                }
            } else {
                const int p = tile.row_begin + lrow;
                const bool live = p < tile.row_end;
                const int F = g.N;
                float part = 0.0f;
                if (live) {
                    const float w = g.prow[p];
                    const int64_t rowF = static_cast<int64_t>(p) * F;
                    uint16_t* dgu = static_cast<uint16_t*>(g.c) + 2 * rowF;
#pragma unroll
                    for (int j = 0; j < kTN; ++j) {
                        const int f = n0 + 64 * wn + 32 * j + (lane & 31);
                        const float gv = bf16_to_f32(g.g[rowF + f]);
                        const float uv = bf16_to_f32(g.u[rowF + f]);
                        const float d = acc[i][j][r];
                        const float sg = sigmoid_f(gv);
                        const float hv = gv * sg * uv;
                        part += hv * d;
                        const float dh = w * d;
                        dgu[f] = f32_to_bf16(dh * uv * sg * (1.0f + gv * (1.0f - sg)));
                        dgu[F + f] = f32_to_bf16(dh * gv * sg);
                        g.hp[rowF + f] = f32_to_bf16(w * hv);
                    }
                }
                // sum over the 32 lanes that share this row (every lane takes part)
#pragma unroll
                for (int off = 16; off >= 1; off >>= 1)
                    part += __shfl_xor(part, off);
                if (live && (lane & 31) == 0)
                    g.partial[static_cast<int64_t>(p) * (F / 64) + n0 / 64 + wn] = part;
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Weight gradients with LDS DMA (gradient tiles of 256 x 256; Mo and No multiples of 256).
//
// Both operands are activation rows over K (the expert's rows), so both take the path the forward's
// large-tile kernel uses for its weights: four LDS stages of 32 k rows each ([32][256] bf16, 512-byte
// rows, 16-byte chunks XOR-swizzled by c ^ 4 (kr & 3)), filled by global_load_lds_dwordx4 (no
// staging registers) and read with the transposing ds_read_b64_tr_b16, which hands each lane 4
// consecutive k of one column: an MFMA operand fragment from two reads.  Each K step every wave
// issues 2 copies of A rows and 2 of B rows for step t + 4 right after the barrier of step t, so at
// every barrier "step t + 1 has landed" is "at most 8 copies in flight".  A copy lane whose row lies
// past the expert's last row reads a zeroed buffer instead (its offset from the copy's base is the
// buffer's distance), and the K loop runs whole groups of four steps, so no row is masked in the
// arithmetic.  8 waves of 64 x 128 (2 x 4 blocks of 32 x 32), one persistent workgroup per CU,
// tasks (expert, gradient row tile, column tile) claimed per XCD; the next task's first copies go
// out before the current task's fp32 stores.
namespace tn {

constexpr int kWM = 4, kWN = 2, kTM = 2, kTN = 4;
constexpr int kWaves = kWM * kWN;
constexpr int kThreads = kWaves * 64;
constexpr int BM = kWM * kTM * 32;                 // 256 gradient rows
constexpr int BN = kWN * kTN * 32;                 // 256 gradient columns
constexpr int BK = 32;
constexpr int kStages = 4;
constexpr int kRowBytes = BM * 2;                  // one k row of a stage
constexpr int kStageBytes = BK * kRowBytes;        // 16 KiB
constexpr int kBRing = kStages * kStageBytes;      // A stages in the first 64 KiB, B in the next
constexpr int kSmemBytes = 2 * kBRing + 256;       // + the claimed-task word
constexpr int kCopies = kStageBytes / 1024 / kWaves;   // 1 KiB copies per operand, wave and step (2)
constexpr int kStepCopies = 2 * kCopies;
static_assert(BM == BN, "one stage layout serves both operands");

// Gradient row tiles per task group (tasks run group by group, row tiles fastest within one).
// Measured on the Mixtral weight gradients: groups of 4 when a gradient has at least 16 row tiles
// (dWg, dWu: 16, 6% faster than groups of 8; dWd: 56, the same); the fine-grained ones (8 and 3
// row tiles) were not faster with 4.
inline int wgrad_group(int64_t Mo) { return Mo / BM >= 16 ? 4 : 8; }

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

template <int N>
__device__ __forceinline__ void step_barrier()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

struct Frags {
    bf16x8_t a[kTM];
    bf16x8_t b[kTN];
    i16x4_t alo[kTM];
    i16x4_t blo[kTN];
};

// Running copy state: sources at the next step's first row (columns m0 / n0), rows of the expert
// left from there, and the zero buffer's byte distance from each source.
struct Copy {
    const uint16_t* a;
    const uint16_t* b;
    int rem;
    uint32_t za, zb;
    uint32_t a_lds, b_lds;
};

// Fixed per lane: copy j moves stage rows 2 (kCopies wave + j) + lane / 32, chunk position lane % 32.
struct Lane {
    uint32_t a_voff[kCopies], b_voff[kCopies], c16[kCopies];
    int krl[kCopies];
    uint32_t a_base[kTM], b_base[kTN];        // fragment-read addresses in stage 0
};

template <int C>
__device__ __forceinline__ void copy_one(const Copy& cp, const Lane& ln, int SB)
{
    constexpr int j = C % kCopies;
    if constexpr (C < kCopies) {
        const uint32_t v = ln.krl[j] < cp.rem ? ln.a_voff[j] : cp.za + ln.c16[j];
        lds_copy16(cp.a, v, cp.a_lds + SB * kStageBytes + j * 1024);
    } else {
        const uint32_t v = ln.krl[j] < cp.rem ? ln.b_voff[j] : cp.zb + ln.c16[j];
        lds_copy16(cp.b, v, cp.b_lds + SB * kStageBytes + j * 1024);
    }
}

// The sources move on by one step while rows of the expert remain; after its last row they stay
// (every copy then reads the zero rows), so a source never passes the zero rows above it.
__device__ __forceinline__ void advance(Copy& cp, int64_t lda, int64_t ldb)
{
    cp.rem -= BK;
    if (cp.rem > 0) {
        cp.a += BK * lda;
        cp.b += BK * ldb;
        cp.za -= static_cast<uint32_t>(BK * lda * 2);
        cp.zb -= static_cast<uint32_t>(BK * ldb * 2);
    }
}

// Fragment read Q of sub-step KS of stage S, in the order the MFMAs consume them: Q 0-1 the two
// halves of A block 0, then two per weight block j, then two per A block i >= 1.
template <int S, int KS, int Q>
__device__ __forceinline__ void read_one(Frags& f, const Lane& ln)
{
    constexpr int kB0 = 2, kB1 = 2 + 2 * kTN;
    constexpr bool isB = Q >= kB0 && Q < kB1;
    constexpr int h = Q % 2;
    constexpr int idx = isB ? (Q - kB0) / 2 : (Q < kB0 ? 0 : 1 + (Q - kB1) / 2);
    uint32_t base;
    if constexpr (isB)
        base = ln.b_base[idx];
    else
        base = ln.a_base[idx];
    const uint32_t p = base + S * kStageBytes + (16 * KS + 4 * h) * kRowBytes;
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4_t*>(p));
    if constexpr (isB) {
        if constexpr (h == 0)
            f.blo[idx] = v;
        else
            f.b[idx] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(f.blo[idx], v, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
        if constexpr (h == 0)
            f.alo[idx] = v;
        else
            f.a[idx] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(f.alo[idx], v, 0, 1, 2, 3, 4, 5, 6, 7));
    }
}

template <int S, int KS, int Q0, int... Is>
__device__ __forceinline__ void reads_impl(std::integer_sequence<int, Is...>, Frags& f, const Lane& ln)
{
    (read_one<S, KS, Q0 + Is>(f, ln), ...);
}

template <int S, int KS, int Q0, int Q1>
__device__ __forceinline__ void reads(Frags& f, const Lane& ln)
{
    reads_impl<S, KS, Q0>(std::make_integer_sequence<int, Q1 - Q0>{}, f, ln);
}

template <int C0, int... Is>
__device__ __forceinline__ void copies_impl(std::integer_sequence<int, Is...>, const Copy& cp,
                                            const Lane& ln, int SB)
{
    (copy_one<C0 + Is>(cp, ln, SB), ...);
}

template <int C0, int C1>
__device__ __forceinline__ void copies(const Copy& cp, const Lane& ln, int SB)
{
    copies_impl<C0>(std::make_integer_sequence<int, C1 - C0>{}, cp, ln, SB);
}

// Slot M of a sub-step: MFMA M, then its share of the next fragment reads (issued over the first
// half of the MFMAs, so that they have landed before a barrier waits for them) and of the copies.
template <int NC, int SB, int SR, int KS, int M>
__device__ __forceinline__ void slot(f32x16_t (&acc)[kTM][kTN], const Frags& use, Frags& load,
                                     const Copy& cp, const Lane& ln)
{
    constexpr int NM = kTM * kTN, NR = 2 * (kTM + kTN);
    acc[M / kTN][M % kTN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(use.a[M / kTN], use.b[M % kTN],
                                                                    acc[M / kTN][M % kTN], 0, 0, 0);
    constexpr int RF = NM / 2;                                      // slots that carry the reads
    if constexpr (M < RF)
        reads<SR, KS, M * NR / RF, (M + 1) * NR / RF>(load, ln);
    copies<M * NC / NM, (M + 1) * NC / NM>(cp, ln, SB);
    __builtin_amdgcn_sched_barrier(0);
}

template <int NC, int SB, int SR, int KS, int... Ms>
__device__ __forceinline__ void slots(std::integer_sequence<int, Ms...>, f32x16_t (&acc)[kTM][kTN],
                                      const Frags& use, Frags& load, const Copy& cp, const Lane& ln)
{
    (slot<NC, SB, SR, KS, Ms>(acc, use, load, cp, ln), ...);
}

// K step t (stage S): the MFMAs of sub-step 0 while sub-step 1's fragments are read; the barrier
// after which step t + 1 has landed (at most W copies in flight; none for W < 0); the MFMAs of
// sub-step 1 while step t + 1's first fragments are read and (kCopy) step t + 4's copies go into
// the stage step t has freed.
template <int S, bool kCopy, int W>
__device__ __forceinline__ void k_step(f32x16_t (&acc)[kTM][kTN], Frags& f0, Frags& f1, Copy& cp,
                                       const Lane& ln, int64_t lda, int64_t ldb)
{
    __builtin_amdgcn_sched_barrier(0);
    slots<0, 0, S, 1>(std::make_integer_sequence<int, kTM * kTN>{}, acc, f0, f1, cp, ln);
    if constexpr (W >= 0)
        step_barrier<W>();
    __builtin_amdgcn_sched_barrier(0);
    slots<kCopy ? kStepCopies : 0, S, (S + 1) % kStages, 0>(std::make_integer_sequence<int, kTM * kTN>{},
                                                             acc, f1, f0, cp, ln);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kCopy)
        advance(cp, lda, ldb);
}

constexpr int kTopWait = 3 * kStepCopies;       // steps 1 .. 3 may still be in flight

// The K loop of one task: KT a multiple of 4 (at least 4); the caller issued steps 0 .. 3 and
// waited for step 0 (step_barrier<kTopWait>); cp is at step 4.
__device__ __forceinline__ void k_loop(f32x16_t (&acc)[kTM][kTN], Copy cp, const Lane& ln, int KT,
                                       int64_t lda, int64_t ldb)
{
    constexpr int W = 2 * kStepCopies;
    Frags f0, f1;
    reads<0, 0, 0, 2 * (kTM + kTN)>(f0, ln);
    for (int kt = 0; kt < KT - kStages; kt += kStages) {
        k_step<0, true, W>(acc, f0, f1, cp, ln, lda, ldb);
        k_step<1, true, W>(acc, f0, f1, cp, ln, lda, ldb);
        k_step<2, true, W>(acc, f0, f1, cp, ln, lda, ldb);
        k_step<3, true, W>(acc, f0, f1, cp, ln, lda, ldb);
    }
    k_step<0, false, W>(acc, f0, f1, cp, ln, lda, ldb);
    k_step<1, false, kStepCopies>(acc, f0, f1, cp, ln, lda, ldb);
    k_step<2, false, 0>(acc, f0, f1, cp, ln, lda, ldb);
    k_step<3, false, -1>(acc, f0, f1, cp, ln, lda, ldb);
}

struct WgradArgs {
    const uint16_t* a;       // rows over K: [rows][>= Mo], row stride lda
    const uint16_t* b;       // [rows][>= No], row stride ldb
    int64_t lda, ldb;
    const int32_t* offsets;  // expert e owns rows [offsets[e], offsets[e + 1])
    const uint16_t* zero;    // >= 512 zero bytes at or above (source end + one source row)
    float* c;                // [E][Mo][No]
    int E, Mo, No;
    int32_t* task_ctr;       // kXcdCount zeroed counters
    int group;               // gradient row tiles per task group (wgrad_group)
};

__global__ __launch_bounds__(kThreads, 1) void wgrad_dma(WgradArgs g)
{
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    int* const claimed = reinterpret_cast<int*>(smem + 2 * kBRing);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char*)(smem)));
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN;
    const int wn = wave % kWN;
    const int n_mt = g.Mo / BM, n_nt = g.No / BN;
    const int per_e = n_mt * n_nt;
    const int total = per_e * g.E;

    Lane ln;
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
        const int kr = 2 * (kCopies * wave + j) + lane / 32;
        const int c = (lane & 31) ^ (4 * (kr & 3));
        ln.krl[j] = kr;
        ln.c16[j] = 16u * c;
        ln.a_voff[j] = static_cast<uint32_t>(kr) * static_cast<uint32_t>(g.lda) * 2u + 16u * c;
        ln.b_voff[j] = static_cast<uint32_t>(kr) * static_cast<uint32_t>(g.ldb) * 2u + 16u * c;
    }
    {
        const int gq = lane >> 4, e4 = (lane >> 2) & 3, q = lane & 3;
        const int kr = 8 * (gq >> 1) + e4;
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            const int col = 32 * (kWM * i + wm) + 16 * (gq & 1) + 4 * q;
            ln.a_base[i] = lds0 + kr * kRowBytes + 16 * ((col >> 3) ^ (4 * e4)) + 2 * (col & 7);
            asm volatile("" : "+v"(ln.a_base[i]));
        }
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int col = 32 * kTN * wn + 32 * j + 16 * (gq & 1) + 4 * q;
            ln.b_base[j] = lds0 + kBRing + kr * kRowBytes + 16 * ((col >> 3) ^ (4 * e4)) + 2 * (col & 7);
            asm volatile("" : "+v"(ln.b_base[j]));
        }
    }
    Copy cp;
    cp.a_lds = lds0 + kCopies * wave * 1024;
    cp.b_lds = lds0 + kBRing + kCopies * wave * 1024;

    const int xcd = blockIdx.x % kXcdCount;
    const int blk = gridDim.x / kXcdCount;
    int e = 0, m0 = 0, n0 = 0, KT = 0;
    auto setup = [&](int t) {
        e = t / per_e;
        const int tl = t - e * per_e;
        const int grp = tl / (g.group * n_nt);
        const int first = grp * g.group;
        const int gsz = min(g.group, n_mt - first);
        const int idx = tl - grp * g.group * n_nt;
        m0 = (first + idx % gsz) * BM;
        n0 = (idx / gsz) * BN;
        const int k_begin = g.offsets[e];
        const int cnt = g.offsets[e + 1] - k_begin;
        KT = max(kStages, (cnt + kStages * BK - 1) / (kStages * BK) * kStages);
        cp.a = g.a + static_cast<int64_t>(k_begin) * g.lda + m0;
        cp.b = g.b + static_cast<int64_t>(k_begin) * g.ldb + n0;
        cp.rem = cnt;
        cp.za = static_cast<uint32_t>(reinterpret_cast<const char*>(g.zero) - reinterpret_cast<const char*>(cp.a));
        cp.zb = static_cast<uint32_t>(reinterpret_cast<const char*>(g.zero) - reinterpret_cast<const char*>(cp.b));
#pragma unroll
        for (int S = 0; S < kStages; ++S) {
            copies<0, kStepCopies>(cp, ln, S);
            advance(cp, g.lda, g.ldb);
        }
    };

    // tasks claimed two ahead (claim_issue): t's successor is in the claim word at every top barrier
    MOE_PROBE(unsigned long long pr[kProbeFields] = {};
              const unsigned long long pr_k0 = __builtin_readcyclecounter();
              const unsigned long long pr_r0 = __builtin_amdgcn_s_memrealtime();
              unsigned long long pr_t = pr_k0, pr_b = 0, pr_k = 0, pr_s = 0, pr_u = 0;)
    int t = claim_task(claimed, g.task_ctr, xcd, blk, wave, lane);
    claim_task(claimed, g.task_ctr, xcd, blk, wave, lane);
    if (t < total)
        setup(t);
    while (t < total) {
        f32x16_t acc[kTM][kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;
        step_barrier<kTopWait>();
        const int ci = __builtin_amdgcn_readfirstlane(*claimed);
        const int t_next = ((ci / blk) * kXcdCount + xcd) * blk + ci % blk;
        const int claim_ret = claim_issue(g.task_ctr, xcd, wave, lane);    // the task after t_next
        MOE_PROBE(pr_b = __builtin_readcyclecounter(); pr[kProbeWait] += pr_b - pr_t;)
        k_loop(acc, cp, ln, KT, g.lda, g.ldb);
        MOE_PROBE(pr_k = __builtin_readcyclecounter(); pr[kProbeLoop] += pr_k - pr_b;
                  pr[kProbeLoopFull] += pr_k - pr_b; ++pr[kProbeTasks]; ++pr[kProbeTasksFull];
                  pr[kProbeSteps] += KT;)
        const int claim_after = claim_value(claim_ret, wave);
        const int de = e, dm0 = m0, dn0 = n0;
        t = t_next;
        // every wave is past its last read of this task's stages (and of the claim word)
        __syncthreads();
        MOE_PROBE(pr_s = __builtin_readcyclecounter(); pr[kProbeSync] += pr_s - pr_k;)
        if (t < total)
            setup(t);
        MOE_PROBE(pr_u = __builtin_readcyclecounter(); pr[kProbeSetup] += pr_u - pr_s;)
        float* C = g.c + static_cast<int64_t>(de) * g.Mo * g.No;
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = dm0 + 32 * (kWM * i + wm) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                float* crow = C + static_cast<int64_t>(row) * g.No + dn0 + 32 * kTN * wn + (lane & 31);
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    crow[32 * j] = acc[i][j][r];
            }
        }
        if (wave == 0)
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
            atomicAdd(&g_phase_bwd[0][q], pr[q]);
    }
#endif
}

}  // namespace tn

// ------------------------------------------------------------------------------------------------
// dgrads with LDS DMA (256 x 256 tiles over the 256-row tile table; N a multiple of 256, K of 128).
//
// Both operands are K-contiguous rows (activation rows of the tile, weight rows of the expert).
// They move in pairs of K steps: two pair stages per operand of [256 rows][64 k], rows of 128 bytes
// (whole cache lines; with one K step per stage every line was fetched in two halves), 16-byte chunk
// c of row r at position c ^ ((r >> 1) & 7), so the 16 rows one fragment read serves per chunk
// cover all 16 bank groups; fragments are single ds_read_b128.  Pair p (steps 2p, 2p + 1) goes out
// in two halves: the first after the barrier of step 2p - 3 (which frees the stage of pair p - 2),
// the second before the barrier of step 2p - 2; the barrier of step 2p - 1 waits for it whole.
// Task claiming and the overlap of the next task's first copies with the epilogue are those of
// the weight-gradient kernel above.  Rows past a partial tile's end re-read its last row and are
// never stored.  The gate/up dgrad's weight source switches from Wg[e] to Wu[e] at k = F.
namespace nt {

constexpr int kWM = 4, kWN = 2, kTM = 2, kTN = 4;
constexpr int kWaves = kWM * kWN;
constexpr int kThreads = kWaves * 64;
constexpr int BM = kWM * kTM * 32;                 // 256 rows (the tile table's height)
constexpr int BN = kWN * kTN * 32;                 // 256 output columns
constexpr int BK = 32;                             // one K step (two MFMA sub-steps)
constexpr int kStages = 4;                         // K steps per unrolled loop body: two pairs
constexpr int kRowBytes = 2 * BK * 2;              // 128: a pair stage row holds two K steps
constexpr int kPairBytes = BM * kRowBytes;         // 32 KiB per operand
constexpr int kBRing = 2 * kPairBytes;             // A pair stages in the first 64 KiB, B in the next
constexpr int kSmemBytes = 2 * kBRing + 256;
constexpr int kCopies = kPairBytes / 1024 / kWaves;   // 4 per operand and pair: rows 8 (4 wave + j) .. + 7
constexpr int kHalfCopies = kCopies;               // a half pair: two copies of A, then two of B
static_assert(BM == BN, "one stage layout serves both operands");

using tn::step_barrier;

struct Frags {
    bf16x8_t a[kTM];
    bf16x8_t b[kTN];
};

struct Copy {
    const uint16_t* a;       // A at the first k of the pair being copied (row offsets in a_voff)
    const uint16_t* b;       // the expert's weights at the same k
    const uint16_t* b1;      // segment 1's weights at k = kseg
    int pair, kseg_pairs;    // the pair being copied; the pair at which the weights switch to b1
    uint32_t a_lds, b_lds;   // this wave's first copy in pair stage 0
};

struct Lane {
    uint32_t a_voff[kCopies], b_voff[kCopies];
    uint32_t a_base[2][2], b_base[2][2];   // fragment reads in pair stage 0: [pair half][sub-step]
};

// Copy C (0 .. 3) of half H of a pair into pair stage QA: C = 0, 1 move A copies 2H + C, C = 2, 3
// weight copies 2H + C - 2.
template <int H, int C>
__device__ __forceinline__ void copy_one(const Copy& cp, const Lane& ln, int QA)
{
    constexpr int j = 2 * H + C % 2;
    if constexpr (C < 2)
        lds_copy16(cp.a, ln.a_voff[j], cp.a_lds + QA * kPairBytes + j * 1024);
    else
        lds_copy16(cp.b, ln.b_voff[j], cp.b_lds + QA * kPairBytes + j * 1024);
}

// After a pair's second half: the sources move on to the next pair.
__device__ __forceinline__ void advance(Copy& cp)
{
    cp.a += 2 * BK;
    ++cp.pair;
    cp.b = cp.pair == cp.kseg_pairs ? cp.b1 : cp.b + 2 * BK;
}

// Read Q of sub-step KS of step position S (pair stage S / 2, pair half S % 2): A block 0, weight
// blocks 0 .. kTN - 1, then A blocks 1 ...
template <int S, int KS, int Q>
__device__ __forceinline__ void read_one(Frags& f, const Lane& ln)
{
    using LdsV = const __attribute__((address_space(3))) bf16x8_t;
    constexpr int q = S / 2, h = S % 2;
    if constexpr (Q >= 1 && Q <= kTN) {
        constexpr int j = Q - 1;
        f.b[j] = *reinterpret_cast<LdsV*>(ln.b_base[h][KS] + q * kPairBytes + j * 32 * kRowBytes);
    } else {
        constexpr int i = Q == 0 ? 0 : Q - kTN;
        f.a[i] = *reinterpret_cast<LdsV*>(ln.a_base[h][KS] + q * kPairBytes + i * kWM * 32 * kRowBytes);
    }
}

template <int S, int KS, int Q0, int... Is>
__device__ __forceinline__ void reads_impl(std::integer_sequence<int, Is...>, Frags& f, const Lane& ln)
{
    (read_one<S, KS, Q0 + Is>(f, ln), ...);
}

template <int S, int KS, int Q0, int Q1>
__device__ __forceinline__ void reads(Frags& f, const Lane& ln)
{
    reads_impl<S, KS, Q0>(std::make_integer_sequence<int, Q1 - Q0>{}, f, ln);
}

template <int H, int C0, int... Is>
__device__ __forceinline__ void copies_impl(std::integer_sequence<int, Is...>, const Copy& cp,
                                            const Lane& ln, int QA)
{
    (copy_one<H, C0 + Is>(cp, ln, QA), ...);
}

// Copies C0 .. C1 - 1 of half H into pair stage QA.
template <int H, int C0, int C1>
__device__ __forceinline__ void copies(const Copy& cp, const Lane& ln, int QA)
{
    copies_impl<H, C0>(std::make_integer_sequence<int, C1 - C0>{}, cp, ln, QA);
}

template <int NC, int H, int QA, int SR, int KS, int M>
__device__ __forceinline__ void slot(f32x16_t (&acc)[kTM][kTN], const Frags& use, Frags& load,
                                     const Copy& cp, const Lane& ln)
{
    constexpr int NM = kTM * kTN, NR = kTM + kTN;
    acc[M / kTN][M % kTN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(use.a[M / kTN], use.b[M % kTN],
                                                                    acc[M / kTN][M % kTN], 0, 0, 0);
    constexpr int RF = NM / 2;                                      // slots that carry the reads
    if constexpr (M < RF)
        reads<SR, KS, M * NR / RF, (M + 1) * NR / RF>(load, ln);
    copies<H, M * NC / NM, (M + 1) * NC / NM>(cp, ln, QA);
    __builtin_amdgcn_sched_barrier(0);
}

template <int NC, int H, int QA, int SR, int KS, int... Ms>
__device__ __forceinline__ void slots(std::integer_sequence<int, Ms...>, f32x16_t (&acc)[kTM][kTN],
                                      const Frags& use, Frags& load, const Copy& cp, const Lane& ln)
{
    (slot<NC, H, QA, SR, KS, Ms>(acc, use, load, cp, ln), ...);
}

// K step t at position S = t % 4: sub-step 1 of step t on f0 (reading step t's second sub-step into
// f1), with the second half of pair t / 2 + 1 when S is even and kPre; the barrier (at most W copies
// in flight; none when W < 0); sub-step 0 of step t + 1 on f1 (reading step t + 1's first sub-step
// into f0), with the first half of pair (t + 3) / 2 when S is odd and kPost.
template <int S, bool kPre, bool kPost, int W>
__device__ __forceinline__ void k_step(f32x16_t (&acc)[kTM][kTN], Frags& f0, Frags& f1, Copy& cp,
                                       const Lane& ln)
{
    static_assert(!(kPre && S % 2 == 1) && !(kPost && S % 2 == 0), "copy points");
    __builtin_amdgcn_sched_barrier(0);
    slots<kPre ? kHalfCopies : 0, 1, (S / 2 + 1) % 2, S, 1>(std::make_integer_sequence<int, kTM * kTN>{},
                                                            acc, f0, f1, cp, ln);
    if constexpr (kPre)
        advance(cp);
    if constexpr (W >= 0)
        step_barrier<W>();
    __builtin_amdgcn_sched_barrier(0);
    slots<kPost ? kHalfCopies : 0, 0, ((S + 3) / 2) % 2, (S + 1) % kStages, 0>(
        std::make_integer_sequence<int, kTM * kTN>{}, acc, f1, f0, cp, ln);
    __builtin_amdgcn_sched_barrier(0);
}

// Copies a task's setup leaves in flight once pair 0 has landed: the first half of pair 1.
constexpr int kTopWait = kHalfCopies;

// The K loop of one task.  KT is a multiple of 4; the caller issued pair 0 and the first half of
// pair 1, cp points at pair 1, and the caller has waited for pair 0 (step_barrier<kTopWait>).  At
// an even step's barrier the halves of the next pair may be in flight (the step after it lies in
// the current pair); at an odd step's barrier the next pair must have landed.
__device__ __forceinline__ void k_loop(f32x16_t (&acc)[kTM][kTN], Copy cp, const Lane& ln, int KT)
{
    constexpr int WE = 2 * kHalfCopies;
    Frags f0, f1;
    reads<0, 0, 0, kTM + kTN>(f0, ln);
    for (int kt = 0; kt < KT - kStages; kt += kStages) {
        k_step<0, true, false, WE>(acc, f0, f1, cp, ln);
        k_step<1, false, true, 0>(acc, f0, f1, cp, ln);
        k_step<2, true, false, WE>(acc, f0, f1, cp, ln);
        k_step<3, false, true, 0>(acc, f0, f1, cp, ln);
    }
    // the last four steps: only the second half of the last pair is still to be copied
    k_step<0, true, false, WE>(acc, f0, f1, cp, ln);
    k_step<1, false, false, 0>(acc, f0, f1, cp, ln);
    k_step<2, false, false, 0>(acc, f0, f1, cp, ln);
    k_step<3, false, false, -1>(acc, f0, f1, cp, ln);
}

// kParts (gate/up only): 1, one pass over k < 2F storing bf16 rows; 2, tasks [0, T0) take dg Wg^T
// and tasks [T0, 2 T0) du Wu^T, each storing an fp32 part (twice the tasks, for problems with
// too few 256 x 256 tiles to keep every CU busy to the end).
template <int kEpi, int kParts>
__global__ __launch_bounds__(kThreads, 1) void dgrad_dma(BwdArgs g, int32_t* __restrict__ task_ctr)
{
    extern __shared__ __attribute__((aligned(256))) unsigned char smem[];
    int* const claimed = reinterpret_cast<int*>(smem + 2 * kBRing);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char*)(smem)));
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN;
    const int wn = wave % kWN;
    const int n_nt = g.N / BN;
    const int T0 = *g.tile_count * n_nt;
    const int total = kParts * T0;
    const int KT = (kParts == 2 ? g.kseg : g.K) / BK;

    Lane ln;
    {
        const int r = lane & 31;
        const int swz = (r >> 1) & 7;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int pos = (4 * h + 2 * ks + (lane >> 5)) ^ swz;
                ln.a_base[h][ks] = lds0 + (32 * wm + r) * kRowBytes + 16 * pos;
                ln.b_base[h][ks] = lds0 + kBRing + (32 * kTN * wn + r) * kRowBytes + 16 * pos;
                asm volatile("" : "+v"(ln.a_base[h][ks]));
                asm volatile("" : "+v"(ln.b_base[h][ks]));
            }
    }
    // copy j of this wave moves stage rows 8 (kCopies wave + j) .. + 7, eight lanes per row; the
    // lane at position p of its row fetches logical chunk p ^ ((row >> 1) & 7)
    uint32_t c16[kCopies];
    int crow[kCopies];
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
        crow[j] = 8 * (kCopies * wave + j) + lane / 8;
        c16[j] = 16u * static_cast<uint32_t>((lane & 7) ^ ((crow[j] >> 1) & 7));
    }
    Copy cp;
    cp.a_lds = lds0 + kCopies * wave * 1024;
    cp.b_lds = lds0 + kBRing + kCopies * wave * 1024;
    cp.kseg_pairs = kParts == 2 ? KT / 2 : g.kseg / (2 * BK);   // parts: one weight matrix per task

    const int xcd = blockIdx.x % kXcdCount;
    const int blk = gridDim.x / kXcdCount;
    MTile tile{};
    int n0 = 0, part = 0;
    auto setup = [&](int t) {
        int nt;
        part = t >= T0 ? 1 : 0;
        tile = decode_task(t - part * T0, n_nt, g.tiles, nt);
        n0 = nt * BN;
        const int last = tile.row_end - 1;
#pragma unroll
        for (int j = 0; j < kCopies; ++j) {
            const int row = min(tile.row_begin + crow[j], last);
            ln.a_voff[j] = static_cast<uint32_t>(row) * static_cast<uint32_t>(g.lda) * 2u + c16[j];
            ln.b_voff[j] = static_cast<uint32_t>(n0 + crow[j]) * static_cast<uint32_t>(g.ldb) * 2u + c16[j];
        }
        const int64_t eoff = static_cast<int64_t>(tile.expert) * g.b_estride;
        cp.a = g.a + part * g.kseg;
        cp.b = (part ? g.b1 : g.b0) + eoff;
        cp.b1 = g.b1 + eoff;
        cp.pair = 0;
        // pair 0 whole, then the first half of pair 1 (k_loop's order)
        copies<0, 0, kHalfCopies>(cp, ln, 0);
        copies<1, 0, kHalfCopies>(cp, ln, 0);
        advance(cp);
        copies<0, 0, kHalfCopies>(cp, ln, 1);
    };

    // tasks claimed two ahead (claim_issue): t's successor is in the claim word at every top barrier
    MOE_PROBE(unsigned long long pr[kProbeFields] = {};
              const unsigned long long pr_k0 = __builtin_readcyclecounter();
              const unsigned long long pr_r0 = __builtin_amdgcn_s_memrealtime();
              unsigned long long pr_t = pr_k0, pr_b = 0, pr_k = 0, pr_s = 0, pr_u = 0;)
    int t = claim_task(claimed, task_ctr, xcd, blk, wave, lane);
    claim_task(claimed, task_ctr, xcd, blk, wave, lane);
    if (t < total)
        setup(t);
    while (t < total) {
        f32x16_t acc[kTM][kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] = 0.0f;
        step_barrier<kTopWait>();
        const int ci = __builtin_amdgcn_readfirstlane(*claimed);
        const int t_next = ((ci / blk) * kXcdCount + xcd) * blk + ci % blk;
        const int claim_ret = claim_issue(task_ctr, xcd, wave, lane);    // the task after t_next
        MOE_PROBE(pr_b = __builtin_readcyclecounter(); pr[kProbeWait] += pr_b - pr_t;)
        k_loop(acc, cp, ln, KT);
        MOE_PROBE(pr_k = __builtin_readcyclecounter(); pr[kProbeLoop] += pr_k - pr_b; ++pr[kProbeTasks];
                  pr[kProbeSteps] += KT;
                  if (tile.row_end - tile.row_begin == BM) { pr[kProbeLoopFull] += pr_k - pr_b; ++pr[kProbeTasksFull]; })
        const int claim_after = claim_value(claim_ret, wave);
        const MTile done = tile;
        const int dn0 = n0, dpart = part;
        t = t_next;
        __syncthreads();
        MOE_PROBE(pr_s = __builtin_readcyclecounter(); pr[kProbeSync] += pr_s - pr_k;)
        if (t < total)
            setup(t);
        MOE_PROBE(pr_u = __builtin_readcyclecounter(); pr[kProbeSetup] += pr_u - pr_s;)
        // Lane holds column lane % 32 of each 32 x 32 block, rows 8 (r / 4) + 4 (lane / 32) + r % 4.
        const int col0 = dn0 + 32 * kTN * wn + (lane & 31);
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            const int pbase = done.row_begin + 32 * (kWM * i + wm) + 4 * (lane >> 5);
            if constexpr (kEpi == kEpiGateUp) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int p = pbase + 8 * (r >> 2) + (r & 3);
                    if (p < done.row_end) {
                        if constexpr (kParts == 2) {
                            float* C = static_cast<float*>(g.c) + (static_cast<int64_t>(dpart) * g.Mo + p) * g.N + col0;
#pragma unroll
                            for (int j = 0; j < kTN; ++j)
                                C[32 * j] = acc[i][j][r];
                        } else {
                            uint16_t* C = static_cast<uint16_t*>(g.c) + static_cast<int64_t>(p) * g.N + col0;
#pragma unroll
                            for (int j = 0; j < kTN; ++j)
                                C[32 * j] = f32_to_bf16(acc[i][j][r]);
                        }
                    }
                }
            } else {
                const int F = g.N;
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    float part[4];
                    // rows 8 rb + .. + 3 of the lane: every g, u and weight they need is loaded before
                    // any is used (rows past the tile's end read its last row and store nothing)
                    uint16_t gq[4][kTN], uq[4][kTN];
                    float wq[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int pc = min(pbase + 8 * rb + rr, done.row_end - 1);
                        const int64_t rowF = static_cast<int64_t>(pc) * F;
                        wq[rr] = g.prow[pc];
#pragma unroll
                        for (int j = 0; j < kTN; ++j) {
                            gq[rr][j] = g.g[rowF + col0 + 32 * j];
                            uq[rr][j] = g.u[rowF + col0 + 32 * j];
                        }
                    }
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int r = 4 * rb + rr;
                        const int p = pbase + 8 * rb + rr;
                        const bool live = p < done.row_end;   // r = 4 rb + rr: row 8 rb + rr
                        const int64_t rowF = static_cast<int64_t>(p) * F;
                        uint16_t* dgu = static_cast<uint16_t*>(g.c) + 2 * rowF;
                        float pt = 0.0f;
#pragma unroll
                        for (int j = 0; j < kTN; ++j) {
                            const int f = col0 + 32 * j;
                            const float gv = bf16_to_f32(gq[rr][j]);
                            const float uv = bf16_to_f32(uq[rr][j]);
                            const float d = acc[i][j][r];
                            const float sg = sigmoid_f(gv);
                            const float hv = gv * sg * uv;
                            pt += hv * d;
                            const float dh = wq[rr] * d;
                            if (live) {
                                dgu[f] = f32_to_bf16(dh * uv * sg * (1.0f + gv * (1.0f - sg)));
                                dgu[F + f] = f32_to_bf16(dh * gv * sg);
                                g.hp[rowF + f] = f32_to_bf16(wq[rr] * hv);
                            }
                        }
                        part[rr] = pt;
                    }
                    // each row's sum over the wave's 128 columns (32 lanes hold one row each)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                        for (int off = 16; off >= 1; off >>= 1)
                            part[rr] += __shfl_xor(part[rr], off);
                    if ((lane & 31) == 0) {
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const int p = pbase + 8 * rb + rr;
                            if (p < done.row_end)
                                g.partial[static_cast<int64_t>(p) * (F / 128) + dn0 / 128 + wn] = part[rr];
                        }
                    }
                }
            }
        }
        if (wave == 0)
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
            atomicAdd(&g_phase_bwd[kEpi == kEpiDown ? 1 : 2][q], pr[q]);
    }
#endif
}

template <int kEpi, int kParts>
hipError_t launch(const BwdArgs& a, int32_t* task_ctr, hipStream_t s)
{
    static std::atomic<bool> done[64];    // per device: the attribute is set
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
        return e;
    if (dev >= 64 || !done[dev]) {
        if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dgrad_dma<kEpi, kParts>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
            e != hipSuccess)
            return e;
        if (dev < 64)
            done[dev] = true;
    }
    dgrad_dma<kEpi, kParts><<<dim3(device_info().cu_count), dim3(kThreads), kSmemBytes, s>>>(a, task_ctr);
    return hipGetLastError();
}

}  // namespace nt

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        p[i] = 0;
}

constexpr int kSmallThreads = 256;

// dx[t] = sum over j (in order) of row pos[t k + j]: fp32 rows as part 0 + part 1 (kParts 2) or
// bf16 rows (kParts 0).  One thread per (token, 16 bytes of each source row: 8 bf16 or 4 fp32
// columns); bf16 rows are loaded 8 at a time before any is added.
template <int kParts>
__global__ __launch_bounds__(kSmallThreads) void sum_slot_rows_kernel(
    const void* __restrict__ rows, const int32_t* __restrict__ pos, uint16_t* __restrict__ dx, int k,
    int64_t M, uint32_t row_vecs, uint32_t total)
{
    constexpr int kCols = kParts == 0 ? 8 : 4;
    const uint32_t i = blockIdx.x * kSmallThreads + threadIdx.x;
    if (i >= total)
        return;
    const uint32_t t = i / row_vecs;
    const uint32_t c = i - t * row_vecs;
    float acc[kCols];
#pragma unroll
    for (int e = 0; e < kCols; ++e)
        acc[e] = 0.0f;
    if constexpr (kParts == 2) {
        // few slots per token where the parts are used: one row at a time
        for (int j = 0; j < k; ++j) {
            const int64_t p = pos[static_cast<int64_t>(t) * k + j];
            if (p < 0 || p >= M)
                continue;
            // each part row is read once: non-temporal loads
            const f32x4_t a = __builtin_nontemporal_load(static_cast<const f32x4_t*>(rows) + p * row_vecs + c);
            const f32x4_t b = __builtin_nontemporal_load(static_cast<const f32x4_t*>(rows) + (M + p) * row_vecs + c);
            acc[0] += a[0] + b[0];
            acc[1] += a[1] + b[1];
            acc[2] += a[2] + b[2];
            acc[3] += a[3] + b[3];
        }
    }
    for (int j0 = 0; kParts == 0 && j0 < k; j0 += 8) {
        float v[8][kCols];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t p = j0 + j < k ? pos[static_cast<int64_t>(t) * k + j0 + j] : -1;
            const bool ok = p >= 0 && p < M;
            const int64_t at = (ok ? p : 0) * row_vecs + c;
            if constexpr (kParts == 0) {
                const u32x4_t b = ok ? __builtin_nontemporal_load(static_cast<const u32x4_t*>(rows) + at)
                                     : u32x4_t{0u, 0u, 0u, 0u};
                const uint32_t d[4] = {b[0], b[1], b[2], b[3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[j][2 * e] = __uint_as_float(d[e] << 16);
                    v[j][2 * e + 1] = __uint_as_float(d[e] & 0xffff0000u);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < kCols; ++e)
                acc[e] += v[j][e];                // skipped slots add 0 exactly
    }
    if constexpr (kCols == 8)
        reinterpret_cast<uint4*>(dx)[i] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    else
        reinterpret_cast<uint2*>(dx)[i] = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
}

// w(p) = probs of the slot behind permuted row p (0 for rows past the valid ones).
__global__ __launch_bounds__(kSmallThreads) void row_probs_kernel(const int32_t* __restrict__ perm,
                                                                  const float* __restrict__ probs,
                                                                  float* __restrict__ prow, int64_t M)
{
    const int64_t p = static_cast<int64_t>(blockIdx.x) * kSmallThreads + threadIdx.x;
    if (p < M) {
        const int32_t slot = perm[p];          // -1 past the valid rows (out-of-range ids)
        prow[p] = slot >= 0 ? probs[slot] : 0.0f;
    }
}

// dprobs[s] = sum over q ascending of partial[pos[s]][q] (0 for a slot with pos < 0).
__global__ __launch_bounds__(kSmallThreads) void dprobs_kernel(const float* __restrict__ partial,
                                                               const int32_t* __restrict__ pos,
                                                               float* __restrict__ dprobs, int64_t M, int nq)
{
    const int64_t s = static_cast<int64_t>(blockIdx.x) * kSmallThreads + threadIdx.x;
    if (s >= M)
        return;
    const int32_t p = pos[s];
    if (p < 0 || p >= M) {                     // slot with an out-of-range id: skipped
        dprobs[s] = 0.0f;
        return;
    }
    const float* row = partial + static_cast<int64_t>(p) * nq;
    float acc = 0.0f;
    for (int q = 0; q < nq; ++q)
        acc += row[q];
    dprobs[s] = acc;
}

template <int kEpi>
hipError_t launch_bwd(const BwdArgs& a, int64_t total_bound, hipStream_t s)
{
    static std::atomic<bool> done[64];    // per device: the attribute is set
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
        return e;
    if (dev >= 64 || !done[dev]) {
        if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_bwd<kEpi>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
            e != hipSuccess)
            return e;
        if (dev < 64)
            done[dev] = true;
    }
    if (total_bound <= 0)
        return hipSuccess;
    const int64_t blocks = (total_bound + kXcdCount - 1) / kXcdCount * kXcdCount;
    if (blocks >= (int64_t{1} << 31))
        return hipErrorInvalidValue;
    grouped_gemm_bwd<kEpi><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), kSmemBytes, s>>>(a);
    return hipGetLastError();
}

}  // namespace

bool bwd_supported(int64_t H, int64_t F) { return H % BN == 0 && F % BN == 0; }

hipError_t launch_row_probs(const int32_t* perm, const float* probs, float* prow, int64_t M, hipStream_t s)
{
    if (M <= 0)
        return hipSuccess;
    row_probs_kernel<<<dim3(static_cast<unsigned>((M + kSmallThreads - 1) / kSmallThreads)),
                       dim3(kSmallThreads), 0, s>>>(perm, probs, prow, M);
    return hipGetLastError();
}

bool dgrad_dma_fits(int64_t M, int64_t H, int64_t F)
{
    const int64_t row_elems = H > 2 * F ? H : 2 * F;          // the wider activation row (dout or dgu)
    return H % nt::BN == 0 && F % nt::BN == 0 && H % (nt::kStages * nt::BK) == 0 &&
           M * row_elems * 2 < (int64_t{1} << 32) && F * H * 2 < (int64_t{1} << 32);
}

int dgrad_row_tile(int64_t M, int64_t H, int64_t F) { return dgrad_dma_fits(M, H, F) ? nt::BM : BM; }

int dprobs_partials(int64_t M, int64_t H, int64_t F) { return static_cast<int>(F / (dgrad_dma_fits(M, H, F) ? 128 : 64)); }

hipError_t launch_dgrad_down(const uint16_t* dout_perm, const uint16_t* wd, const uint16_t* g,
                             const uint16_t* u, const float* prow, uint16_t* dgu, uint16_t* hp,
                             float* partial, const MTile* tiles, const int32_t* tile_count,
                             int64_t max_tiles, int64_t M, int64_t H, int64_t F, int32_t* task_ctr,
                             hipStream_t s)
{
    BwdArgs a{};
    a.a = dout_perm;
    a.lda = H;
    a.b0 = a.b1 = wd;
    a.ldb = H;
    a.b_estride = F * H;
    a.K = a.kseg = static_cast<int>(H);
    a.N = static_cast<int>(F);
    a.tiles = tiles;
    a.tile_count = tile_count;
    a.c = dgu;
    a.g = g;
    a.u = u;
    a.prow = prow;
    a.hp = hp;
    a.partial = partial;
    if (dgrad_dma_fits(M, H, F))
        return nt::launch<kEpiDown, 1>(a, task_ctr, s);
    return launch_bwd<kEpiDown>(a, max_tiles * (F / BN), s);
}

hipError_t launch_dprobs(const float* partial, const int32_t* pos, float* dprobs, int64_t M, int nq,
                         hipStream_t s)
{
    if (M <= 0)
        return hipSuccess;
    dprobs_kernel<<<dim3(static_cast<unsigned>((M + kSmallThreads - 1) / kSmallThreads)),
                    dim3(kSmallThreads), 0, s>>>(partial, pos, dprobs, M, nq);
    return hipGetLastError();
}

// Split into two parts when one pass has fewer than 3 tasks per CU (the last round of equal tasks
// would leave most CUs idle); the fp32 parts cost their extra traffic only then.
int dgrad_gate_up_parts(int64_t M, int64_t H, int64_t F)
{
    if (!dgrad_dma_fits(M, H, F))
        return 1;
    const int64_t tasks = ceil_div(M, nt::BM) * (H / nt::BN);
    return tasks < 3 * int64_t{device_info().cu_count} ? 2 : 1;
}

hipError_t launch_dgrad_gate_up(const uint16_t* dgu, const uint16_t* wg, const uint16_t* wu,
                                void* dx_rows, const MTile* tiles, const int32_t* tile_count,
                                int64_t max_tiles, int64_t M, int64_t H, int64_t F, int32_t* task_ctr,
                                hipStream_t s)
{
    BwdArgs a{};
    a.a = dgu;
    a.lda = 2 * F;
    a.b0 = wg;
    a.b1 = wu;
    a.ldb = F;
    a.b_estride = H * F;
    a.kseg = static_cast<int>(F);
    a.K = static_cast<int>(2 * F);
    a.N = static_cast<int>(H);
    a.Mo = static_cast<int>(M);
    a.tiles = tiles;
    a.tile_count = tile_count;
    a.c = dx_rows;
    if (dgrad_gate_up_parts(M, H, F) == 2)
        return nt::launch<kEpiGateUp, 2>(a, task_ctr, s);
    if (dgrad_dma_fits(M, H, F))
        return nt::launch<kEpiGateUp, 1>(a, task_ctr, s);
    return launch_bwd<kEpiGateUp>(a, max_tiles * (H / BN), s);
}

hipError_t launch_sum_slot_rows(const void* rows, int parts, const int32_t* pos, uint16_t* dx,
                                int64_t T, int64_t k, int64_t M, int64_t H, hipStream_t s)
{
    const int64_t cols = parts == 2 ? 4 : 8;                 // columns per thread
    const int64_t total = T * (H / cols);
    if (total <= 0)
        return hipSuccess;
    if (total >= (int64_t{1} << 31))
        return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>((total + kSmallThreads - 1) / kSmallThreads)), block(kSmallThreads);
    const int kk = static_cast<int>(k);
    const uint32_t rv = static_cast<uint32_t>(H / cols), tt = static_cast<uint32_t>(total);
    if (parts == 2)
        sum_slot_rows_kernel<2><<<grid, block, 0, s>>>(rows, pos, dx, kk, M, rv, tt);
    else
        sum_slot_rows_kernel<0><<<grid, block, 0, s>>>(rows, pos, dx, kk, M, rv, tt);
    return hipGetLastError();
}

bool wgrad_dma_fits(int64_t Mo, int64_t No) { return Mo % tn::BM == 0 && No % tn::BN == 0; }

hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    zero_i32_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(p, static_cast<int>(n));
    return hipGetLastError();
}

hipError_t launch_wgrad(const uint16_t* a_rows, int64_t lda, const uint16_t* b_rows, int64_t ldb,
                        const int32_t* offsets, int64_t E, int64_t Mo, int64_t No, float* dw,
                        const uint16_t* zero, int32_t* task_ctr, hipStream_t s)
{
    if (zero != nullptr && task_ctr != nullptr && wgrad_dma_fits(Mo, No)) {
        static std::atomic<bool> done[64];    // per device: the attribute is set
        int dev = 0;
        if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
            return e;
        if (dev >= 64 || !done[dev]) {
            if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&tn::wgrad_dma),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   tn::kSmemBytes);
                e != hipSuccess)
                return e;
            if (dev < 64)
                done[dev] = true;
        }
        tn::WgradArgs a{a_rows, b_rows, lda, ldb, offsets, zero, dw, static_cast<int>(E),
                        static_cast<int>(Mo), static_cast<int>(No), task_ctr, tn::wgrad_group(Mo)};
        tn::wgrad_dma<<<dim3(device_info().cu_count), dim3(tn::kThreads), tn::kSmemBytes, s>>>(a);
        return hipGetLastError();
    }
    BwdArgs a{};
    a.a = a_rows;
    a.lda = lda;
    a.b0 = a.b1 = b_rows;
    a.ldb = ldb;
    a.Mo = static_cast<int>(Mo);
    a.N = static_cast<int>(No);
    a.offsets = offsets;
    a.E = static_cast<int>(E);
    a.c = dw;
    return launch_bwd<kEpiWgrad>(a, E * (Mo / BM) * (No / BN), s);
}

}  // namespace moe

#ifdef MOE_PHASE_PROBE
int moe::probe_read_bwd(unsigned long long* out, int reset)
{
    if (out != nullptr &&
        hipMemcpyFromSymbol(out, HIP_SYMBOL(g_phase_bwd), sizeof(g_phase_bwd)) != hipSuccess)
        return 1;
    if (reset) {
        const unsigned long long zero[kProbeKindsBwd * kProbeFields] = {};
        if (hipMemcpyToSymbol(HIP_SYMBOL(g_phase_bwd), zero, sizeof(zero)) != hipSuccess)
            return 1;
    }
    return 0;
}
#endif
