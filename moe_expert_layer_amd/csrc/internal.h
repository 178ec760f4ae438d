// Host-side internals shared by the C-ABI layer (api.cpp) and the kernel launchers (*.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// A tile of work for the grouped GEMMs: rows [row_begin, row_end) of the grouped activations all
// use weights of `expert`; `chunk` is the M-axis chunk the rows belong to (0 when unchunked).
// Consecutive tiles of one expert inside one chunk form a run [run_begin, run_begin + run_len) of
// the table; the GEMMs enumerate a run's (row tile, column tile) tasks column-tile-major so that
// the workgroups working at the same time share the run's A rows and a few weight strips.
struct MTile {
    int expert;
    int row_begin;
    int row_end;
    int chunk;
    int run_begin;
    int run_len;
    int pad0, pad1;
};

// ---------------------------------------------------------------------------------------------
// Kernel configuration constants the host needs (tile shapes decide workspace sizes).
// ---------------------------------------------------------------------------------------------
constexpr int kRouteSlotsPerBlock = 2048;  // slots handled by one routing workgroup
constexpr int kMaxExperts = 1024;          // routing LDS histograms are sized for this
constexpr int kChunkAlign = 256;           // head_m_size must be a multiple of this
constexpr size_t kAlign = 256;
constexpr int kXcdCount = 8;               // MI355X: workgroup b runs on XCD b % 8 (measured)

// Row-tile heights of the grouped GEMMs (the tile tables are built per height); the bf16 height
// depends on the problem (bf16_row_tile).
constexpr int kBmF32 = 32;
constexpr int kBmMx = 128;
// Chunked mode: consecutive chunks whose tiles of one expert form one run of tasks.
constexpr int kChunkWindow = 4;

inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Upper bound on the number of row tiles for M rows in G groups, chunks of `chunk` rows
// (chunk == 0: one chunk) and tile height bm: each group adds at most one partial tile and each
// chunk boundary splits at most one more tile.
inline int64_t max_mtiles(int64_t M, int64_t G, int64_t chunk, int bm)
{
    int64_t chunks = chunk > 0 ? ceil_div(M, chunk) : 1;
    return ceil_div(M, bm) + G + chunks + 1;
}

// ---------------------------------------------------------------------------------------------
// Workspace layout.  Byte offsets from the workspace base; the status word is always at 0.
// ---------------------------------------------------------------------------------------------
struct RouteLayout {
    size_t status = 0;        // int32 status word (+ padding)
    size_t block_counts = 0;  // int32 [nblocks, E + 1]: per-block expert counts, last = invalid ids
    size_t total = 0;
    int64_t nblocks = 0;
};

struct FfnLayout {
    size_t status = 0;
    size_t tiles1 = 0, tiles2 = 0;     // MTile tables for fc1 / fc2 row-tile heights
    size_t tiles_run = 0;              // unchunked large tiles: fc1's table, each group one run of balanced tiles
    size_t tile_count = 0;             // int32 [8]: [0] tiles in the table, [2] tiles before its short tails;
                                       // [4], [6] the same for tiles_run
    size_t task_ctr = 0;               // int32 [2][kXcdCount]: per-XCD task counters of fc1 / fc2
    size_t chunk_done = 0;             // int32 [num_chunks]: fc2 tiles finished per chunk
    size_t chunk_tiles = 0;            // int32 [num_chunks]: fc2 tiles per chunk
    size_t h = 0, h_scale = 0;         // SwiGLU output [M, F] (+ MX scales [M, F/32])
    size_t total = 0;
    int64_t max_tiles1 = 0, max_tiles2 = 0, num_chunks = 0;
    int bm1 = 0, bm2 = 0;
};

struct ForwardLayout {
    RouteLayout route;                 // offsets relative to the workspace base
    FfnLayout ffn;                     // offsets relative to the workspace base
    size_t counts = 0, offsets = 0, perm = 0, pos = 0;
    size_t x_perm = 0, x_perm_scale = 0, y_perm = 0;
    size_t x_q = 0, x_q_scale = 0;     // MX-encoded x in token order [T, H] + [T, H/32] (bf16 input)
    size_t total = 0;
};

RouteLayout route_layout(int64_t T, int64_t k, int64_t E, size_t base);
FfnLayout ffn_layout(int dtype, int64_t M, int64_t G, int64_t H, int64_t F, int64_t chunk,
                     size_t base);
ForwardLayout forward_layout(int dtype, int64_t T, int64_t H, int64_t F, int64_t E, int64_t k,
                             int64_t chunk, bool quantize_x = false);

// ---------------------------------------------------------------------------------------------
// Launchers (defined in the .hip files).  Each returns the hipError_t of its launch.
// ---------------------------------------------------------------------------------------------
struct DeviceInfo {
    int cu_count;
};
const DeviceInfo& device_info();       // for the current device (cached)

// route.hip
hipError_t launch_route_count(const int32_t* ids, int64_t M, int64_t E, int32_t* block_counts,
                              int64_t nblocks, hipStream_t s);
hipError_t launch_route_scan(int32_t* block_counts, int64_t nblocks, int64_t E, int64_t M,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* status,
                             hipStream_t s);
hipError_t launch_route_scatter(const int32_t* ids, int64_t M, int64_t E,
                                const int32_t* block_counts, int64_t nblocks, int32_t* perm,
                                int32_t* pos, hipStream_t s);
// Builds the row-tile table: groups are rows [offsets[g], offsets[g+1]) (clamped into [0, M]) with expert
// group_expert[g] (identity when null).  Writes tiles, tile_count[0] (their number) and tile_count[2]
// (how many precede the suffix of short partial tiles, at most 64 rows, that an unchunked table with
// sorted tails ends in; all of them otherwise); when chunk_tiles is not
// null also the expected (row tile x column tile) tasks per chunk (row tiles * col_tiles) and
// zeroes chunk_done; zeroes the 2 * kXcdCount task counters at task_ctr.  A non-empty group with an expert outside [0, E) is skipped and sets
// *status; with write_status the status word is written either way.  tiles_in_run (may be null;
// unchunked tables only): also a table in which each group is one run of R = ceil(rows / bm) tiles
// of near-equal height in row order (their 32-row blocks differ by at most one; the last tile ends
// the group), its number in count_in_run[0] and [2] (laid out as tile_count, so either table can be
// handed to a GEMM with its counts).
hipError_t launch_build_tiles(const int32_t* offsets, const int32_t* group_expert, int64_t G,
                              int64_t E, int64_t M, int64_t chunk, int bm, MTile* tiles, int64_t max_tiles,
                              int32_t* tile_count, int32_t* chunk_tiles, int32_t* chunk_done,
                              int64_t num_chunks, int col_tiles, int32_t* task_ctr,
                              int32_t* status, bool write_status, hipStream_t s,
                              MTile* tiles_in_run = nullptr, int32_t* count_in_run = nullptr);

// permute.hip
// Slots whose pos is outside [0, M) are skipped.
hipError_t launch_permute(const void* x, const int32_t* pos, void* x_perm, int64_t T, int64_t k,
                          int64_t M, int64_t row_bytes, hipStream_t s);
hipError_t launch_unpermute(int dtype, const void* y_perm, const int32_t* pos, const float* probs,
                            void* out, int64_t T, int64_t k, int64_t M, int64_t H, hipStream_t s);

// gemm_bf16.hip: grouped GEMMs on bf16 MFMA.  fc1: h = swiglu(A Wg, A Wu); fc2: y = h Wd.
bool bf16_supported(int64_t H, int64_t F);
int bf16_row_tile(int64_t H, int64_t F);
int bf16_fc2_cols_per_tile(int64_t H, int64_t F);
// task_ctr: kXcdCount zeroed counters for this launch (workspace).  gather (may be null; only
// with 256-row tiles): permuted row p of A is row gather[p] / gather_k of A.  save_g / save_u (both
// null or both set): also store the gate and up values g, u as bf16 [M, F], the layout of h.
hipError_t launch_fc1_bf16(const uint16_t* A, const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                           const MTile* tiles, const int32_t* tile_count, int64_t H, int64_t F,
                           int32_t* task_ctr, const int32_t* gather, int gather_k, uint16_t* save_g,
                           uint16_t* save_u, hipStream_t s);
hipError_t launch_fc2_bf16(const uint16_t* h, const uint16_t* wd, uint16_t* y, const MTile* tiles,
                           const int32_t* tile_count, int64_t H, int64_t F, int32_t* chunk_done,
                           int32_t* task_ctr, hipStream_t s);

// g = A Wg[e], u = A Wu[e] as bf16 [M, F]: the fc1 kernels with h not stored (the backward's
// recompute of g and u, launched under its own kernel name).  Row tiles of bf16_row_tile(H, F) rows.
// gather (large tiles only, may be null) as for launch_fc1_bf16: permuted row p of A is row
// gather[p] / gather_k of A.
hipError_t launch_recompute_gu_bf16(const uint16_t* A, const int32_t* gather, int gather_k,
                                    const uint16_t* wg, const uint16_t* wu, uint16_t* g, uint16_t* u,
                                    const MTile* tiles, const int32_t* tile_count, int64_t H, int64_t F,
                                    int32_t* task_ctr, hipStream_t s);

// gemm_f32.hip: float32 grouped GEMMs (plain FMA).
hipError_t launch_fc1_f32(const float* A, const float* wg, const float* wu, float* h,
                          const MTile* tiles, const int32_t* tile_count, int64_t H, int64_t F,
                          hipStream_t s);
hipError_t launch_fc2_f32(const float* h, const float* wd, float* y, const MTile* tiles,
                          const int32_t* tile_count, int64_t H, int64_t F, int32_t* chunk_done,
                          hipStream_t s);

// gemm_mx.hip: OCP-MX grouped GEMMs on scaled fp8 MFMA.
// task_ctr: kXcdCount zeroed counters for this launch (used by the large-tile kernels).
hipError_t launch_fc1_mx(const uint8_t* A, const uint8_t* a_scale, const uint8_t* wg,
                         const uint8_t* wg_scale, const uint8_t* wu, const uint8_t* wu_scale,
                         uint8_t* h, uint8_t* h_scale, const MTile* tiles,
                         const int32_t* tile_count, int64_t H, int64_t F, int32_t* task_ctr,
                         const int32_t* gather, int gather_k, hipStream_t s);
hipError_t launch_fc2_mx(const uint8_t* h, const uint8_t* h_scale, const uint8_t* wd,
                         const uint8_t* wd_scale, uint16_t* y, const MTile* tiles,
                         const int32_t* tile_count, int64_t H, int64_t F, int32_t* chunk_done,
                         int32_t* task_ctr, hipStream_t s);
// MX tile shapes: 256 x 256 when H and F are multiples of 1024, else 128 x 128.
int mx_row_tile(int64_t H, int64_t F);
int mx_fc2_cols_per_tile(int64_t H, int64_t F);
// gemm_bwd.hip: the backward's grouped GEMMs (bf16, 128-row tiles; H and F multiples of 128).
bool bwd_supported(int64_t H, int64_t F);
// prow[p] = probs[perm[p]]
hipError_t launch_row_probs(const int32_t* perm, const float* probs, float* prow, int64_t M,
                            hipStream_t s);
// The dgrads run on LDS DMA with 256-row tiles when dgrad_dma_fits (H, F multiples of 256, 32-bit
// row offsets), else register-staged with 128-row tiles; dgrad_row_tile gives the tile table's
// height they need and dprobs_partials the partial sums per row (F / 128 or F / 64).
bool dgrad_dma_fits(int64_t M, int64_t H, int64_t F);
int dgrad_row_tile(int64_t M, int64_t H, int64_t F);
int dprobs_partials(int64_t M, int64_t H, int64_t F);
// d = dout_perm Wd^T with the SwiGLU backward in the epilogue: dgu [M, 2F] = [dg | du], hp [M, F]
// = w h, partial [M, dprobs_partials] (sums of h d over consecutive column groups).  task_ctr:
// kXcdCount zeroed counters (used by the DMA kernel).
hipError_t launch_dgrad_down(const uint16_t* dout_perm, const uint16_t* wd, const uint16_t* g,
                             const uint16_t* u, const float* prow, uint16_t* dgu, uint16_t* hp,
                             float* partial, const MTile* tiles, const int32_t* tile_count,
                             int64_t max_tiles, int64_t M, int64_t H, int64_t F, int32_t* task_ctr,
                             hipStream_t s);
// dprobs[s] = sum of partial[pos[s]][0 .. nq)
hipError_t launch_dprobs(const float* partial, const int32_t* pos, float* dprobs, int64_t M, int nq,
                         hipStream_t s);
// Each slot's dx row dg Wg^T + du Wu^T: with dgrad_gate_up_parts(M, H, F) == 2, as two fp32 parts
// [M, H] at dx_rows (dg Wg^T) and dx_rows + M H floats (du Wu^T), computed as separate tasks for an
// even spread over the CUs when one pass has few tasks; otherwise as bf16 rows [M, H].
int dgrad_gate_up_parts(int64_t M, int64_t H, int64_t F);
hipError_t launch_dgrad_gate_up(const uint16_t* dgu, const uint16_t* wg, const uint16_t* wu,
                                void* dx_rows, const MTile* tiles, const int32_t* tile_count,
                                int64_t max_tiles, int64_t M, int64_t H, int64_t F, int32_t* task_ctr,
                                hipStream_t s);
// dx[t] = bf16(sum over j in order of row pos[t k + j]), the rows as launch_dgrad_gate_up left them
// (parts 2: fp32 part 0 + part 1 per slot; otherwise bf16); slots with pos outside [0, M) skipped.
hipError_t launch_sum_slot_rows(const void* rows, int parts, const int32_t* pos, uint16_t* dx,
                                int64_t T, int64_t k, int64_t M, int64_t H, hipStream_t s);
// dw[e] [Mo, No] (fp32) = sum over the rows p of expert e of a_rows[p, :Mo]^T b_rows[p, :No].
// With zero (>= 512 zero bytes at least one source row above the end of both sources, less than
// 4 GiB above their starts) and task_ctr
// (kXcdCount zeroed counters), Mo and No multiples of 256: the LDS-DMA kernel; otherwise the
// register-staged one.
bool wgrad_dma_fits(int64_t Mo, int64_t No);
hipError_t launch_wgrad(const uint16_t* a_rows, int64_t lda, const uint16_t* b_rows, int64_t ldb,
                        const int32_t* offsets, int64_t E, int64_t Mo, int64_t No, float* dw,
                        const uint16_t* zero, int32_t* task_ctr, hipStream_t s);
hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t s);
// router.hip: top-k gate over float32 logits [T, E] (E <= 1024, k <= min(E, 64)).
hipError_t launch_router(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* ids,
                         float* probs, hipStream_t s);
hipError_t launch_mx_quantize(const float* v, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);
// bfloat16 rows x [T, H] -> OCP-MX codes and scales (H a multiple of 32): in token order (pos null;
// codes [T, H], scales [T, H/32]) or written to each token's k permuted rows pos[t k + j] (codes
// [M, H], scales [M, H/32]; rows outside [0, M) skipped).
hipError_t launch_mx_encode_bf16_rows(const uint16_t* x, int64_t T, int64_t H, const int32_t* pos,
                                     int64_t k, int64_t M, uint8_t* codes, uint8_t* scales, hipStream_t s);
// The MX fc1 epilogue's encoder (large_tiles: the 256-row kernel's, else the 128-row kernel's) on
// float32 values v [rows, cols] in place of the SwiGLU output; cols a multiple of 128 (64), rows * cols
// <= 2^28.
hipError_t launch_mx_epilogue_probe(const float* v, int64_t rows, int64_t cols, bool large_tiles,
                                   uint8_t* codes, uint8_t* scales, hipStream_t s);

#ifdef MOE_PHASE_PROBE
// The probe build's per-task cycle sums (one row of kProbeFields per kernel kind; the layout of
// moe_probe_phases).  Kinds 0 fc2, 1 fc1, 2 the backward's recompute (gemm_bf16.hip); 3 weight
// gradients, 4 down dgrad, 5 gate/up dgrad (gemm_bwd.hip); 6 MX fc2, 7 MX fc1 (gemm_mx.hip).
enum ProbeField {
    kProbeWait,           // from the previous epilogue's end (or the kernel's start) past the top barrier
    kProbeLoop,           // K loops
    kProbeLoopFull,       // K loops of full-height, full-width tasks
    kProbeSync,           // after the K loop: the claim's result and the barrier that ends the loop
    kProbeSetup,          // the next task's setup (its first copies)
    kProbeEpilogue,       // the epilogue
    kProbeTasks,
    kProbeTasksFull,
    kProbeTotal,          // cycles from the kernel's start to the workgroup's end
    kProbeRealtime,       // the same span on the 100 MHz real-time counter
    kProbeWorkgroups,
    kProbeSteps,          // K steps of 32 over all tasks
    kProbeFields
};
constexpr int kProbeKindsBf16 = 3, kProbeKindsBwd = 3, kProbeKindsMx = 2;
// Copy one file's sums into out (unless null), then zero them when reset is set.
int probe_read_bf16(unsigned long long* out, int reset);
int probe_read_bwd(unsigned long long* out, int reset);
int probe_read_mx(unsigned long long* out, int reset);
#endif

}  // namespace moe
