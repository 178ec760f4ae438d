// Routing for the MoE expert layer on gfx950: per-expert counts, offsets, and the stable slot
// permutation, plus the row-tile table the grouped GEMMs consume.
//
// The counting step is histc over the flattened expert ids with E bins on [0, E) ("NPU Training
// Operators - MC2", 执行路径 step 2); ids outside [0, E) are left out of every bin, as histc does,
// and flagged in the status word (section 迁移检查 requires ids in [0, E)).  The permutation orders
// slots s = t*k + j by expert and, inside an expert, by s: the row layout permute (step 6) writes
// and unpermute (step 10) reads back.
//
// Three launches, all integer and deterministic:
//   count   one workgroup per 2048 slots: LDS histogram -> block_counts[b][e]
//   scan    one workgroup: per expert, prefix over blocks; exclusive scan over experts -> offsets;
//           block_counts becomes each block's first row per expert
//   scatter one workgroup per 2048 slots, in rounds of 256 slots: a slot's rank among same-expert
//           slots of its wave comes from ballots over the id bits; waves are ordered through LDS.
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kStatusOk = 0;
constexpr int kStatusBadId = 4;   // MOE_ERR_EXPERT_ID_OUT_OF_RANGE
// Partial tiles of at most this many rows are the ones the non-gated GEMM runs as two half-width
// tasks: their time is the weight stream, which halves; for taller tiles the A rows that both halves
// copy cost more than the split gains.
constexpr int kHalfWidthMaxRows = 64;

__global__ __launch_bounds__(kThreads) void route_count_kernel(const int32_t* __restrict__ ids,
                                                               int64_t M, int E,
                                                               int32_t* __restrict__ block_counts)
{
    __shared__ int hist[kMaxExperts + 1];
    for (int i = threadIdx.x; i <= E; i += kThreads)
        hist[i] = 0;
    __syncthreads();
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kRouteSlotsPerBlock;
    for (int i = threadIdx.x; i < kRouteSlotsPerBlock; i += kThreads) {
        const int64_t s = base + i;
        if (s < M) {
            const int id = ids[s];
            atomicAdd(&hist[(id >= 0 && id < E) ? id : E], 1);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i <= E; i += kThreads)
        block_counts[static_cast<int64_t>(blockIdx.x) * (E + 1) + i] = hist[i];
}

// Inclusive scan of one value per thread over a 1024-thread workgroup: a scan inside each wave by
// shuffles, the 16 wave totals scanned by wave 0, then each wave adds the totals of the waves before
// it.  Two barriers; buf needs 32 ints, and a following call only writes entries this one has
// finished reading.
__device__ int block_inclusive_scan(int v, int* buf)
{
    constexpr int kWaves = kScanThreads / 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(v, off);
        if (lane >= off)
            v += y;
    }
    if (lane == 63)
        buf[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int w = lane < kWaves ? buf[lane] : 0;
#pragma unroll
        for (int off = 1; off < kWaves; off <<= 1) {
            const int y = __shfl_up(w, off);
            if (lane >= off)
                w += y;
        }
        if (lane < kWaves)
            buf[kWaves + lane] = w;
    }
    __syncthreads();
    return wave > 0 ? v + buf[kWaves + wave - 1] : v;
}

__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(
    int32_t* __restrict__ block_counts, int nblocks, int E, int64_t M, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ status)
{
    __shared__ int buf[2 * (kScanThreads / 64)];
    __shared__ int total_valid;
    const int e = threadIdx.x;           // E <= kMaxExperts == kScanThreads
    constexpr int kBatch = 8;            // block counts loaded per batch, all before any is used
    int tot = 0;
    if (e <= E) {
        for (int b0 = 0; b0 < nblocks; b0 += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                v[j] = b0 + j < nblocks ? block_counts[static_cast<int64_t>(b0 + j) * (E + 1) + e] : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                tot += v[j];
        }
    }
    const int v = e < E ? tot : 0;
    const int incl = block_inclusive_scan(v, buf);
    const int excl = incl - v;
    if (e < E) {
        counts[e] = tot;
        offsets[e] = excl;
        // each block's count becomes the block's first row for the expert
        int run = excl;
        for (int b0 = 0; b0 < nblocks; b0 += kBatch) {
            int c[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                c[j] = b0 + j < nblocks ? block_counts[static_cast<int64_t>(b0 + j) * (E + 1) + e] : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (b0 + j < nblocks) {
                    block_counts[static_cast<int64_t>(b0 + j) * (E + 1) + e] = run;
                    run += c[j];
                }
        }
    }
    if (e == E - 1) {
        offsets[E] = incl;
        total_valid = incl;
    }
    if (e == E)
        *status = tot > 0 ? kStatusBadId : kStatusOk;
    __syncthreads();
    // rows that no valid slot fills (only when some ids were out of range)
    for (int64_t p = total_valid + threadIdx.x; p < M; p += kScanThreads)
        perm[p] = -1;
}

__global__ __launch_bounds__(kThreads) void route_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t M, int E, int id_bits,
    const int32_t* __restrict__ block_base, int32_t* __restrict__ perm, int32_t* __restrict__ pos)
{
    constexpr int kWaves = kThreads / 64;
    __shared__ int running[kMaxExperts];
    __shared__ int wave_cnt[kWaves][kMaxExperts];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int e = threadIdx.x; e < E; e += kThreads) {
        running[e] = block_base[static_cast<int64_t>(blockIdx.x) * (E + 1) + e];
        for (int w = 0; w < kWaves; ++w)
            wave_cnt[w][e] = 0;
    }
    __syncthreads();
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kRouteSlotsPerBlock;
    for (int round = 0; round < kRouteSlotsPerBlock / kThreads; ++round) {
        const int64_t s = base + round * kThreads + threadIdx.x;
        const bool in_range = s < M;
        const int id = in_range ? ids[s] : -1;
        const bool ok = in_range && id >= 0 && id < E;
        // peers: the lanes of this wave holding a valid slot with the same expert id
        uint64_t peers = __ballot(ok);
        for (int bit = 0; bit < id_bits; ++bit) {
            const bool b = (id >> bit) & 1;
            const uint64_t m = __ballot(b);
            peers &= b ? m : ~m;
        }
        const int rank = __popcll(peers & lt_mask);
        const int cnt = __popcll(peers);
        if (ok && rank == cnt - 1)
            wave_cnt[wave][id] = cnt;
        __syncthreads();
        if (ok) {
            int p = running[id] + rank;
            for (int w = 0; w < wave; ++w)
                p += wave_cnt[w][id];
            perm[p] = static_cast<int32_t>(s);
            pos[s] = p;
        } else if (in_range) {
            pos[s] = -1;
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += kThreads) {
            int add = 0;
            for (int w = 0; w < kWaves; ++w) {
                add += wave_cnt[w][e];
                wave_cnt[w][e] = 0;
            }
            running[e] += add;
        }
        __syncthreads();
    }
}

// Row-tile table.  Group g covers rows [offsets[g], offsets[g+1]) with expert group_expert[g]
// (g itself when group_expert is null).  Each group is cut at chunk boundaries (multiples of
// `chunk` rows) and each piece into tiles of at most bm rows; a run is the tiles of one piece.
// Chunked (num_chunks > 1): tiles in row order (chunk-major); a run spans a group's tiles within a
// window of kChunkWindow chunks, so the tasks sharing a weight strip stay together across the
// window's chunks, and chunks complete in order window by window; each group's piece inside one
// chunk is cut into balanced tiles (as below).  Unchunked: first every group's
// full tiles (row order), then the partial tail tiles, each its own run, so that the short tasks
// come last and even out the workgroups' finishing times.  The second table (tiles_in_run,
// unchunked calls only) keeps each group as one run of R = ceil(rows / bm) tiles of near-equal
// height (their 32-row blocks differ by at most one): the tasks that share a weight strip then
// take equal time, so the workgroups of an XCD stay in step and share the strip in its L2.
// One workgroup per table (two when the in-run table is asked for); groups are handled 1024 at a time.
__global__ __launch_bounds__(kScanThreads) void build_tiles_kernel(
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ group_expert, int G, int E,
    int64_t M, int64_t chunk, int bm, MTile* __restrict__ tiles_main, int max_tiles, int32_t* __restrict__ tile_count,
    int32_t* __restrict__ chunk_tiles, int32_t* __restrict__ chunk_done, int num_chunks,
    int col_tiles, int32_t* __restrict__ task_ctr, int32_t* __restrict__ status, int write_status,
    MTile* __restrict__ tiles_in_run, int32_t* __restrict__ count_in_run)
{
    // one workgroup per layout: 0 the table (unchunked: partial tails last, sorted; chunked: row
    // order), 1 (unchunked, when asked for; the launch's second workgroup) every group as one run
    // of balanced tiles.  Workgroup 0 alone clears the counters and writes the status.
    const int layout = blockIdx.x;
    if (layout == 0 && task_ctr != nullptr && threadIdx.x < 2 * kXcdCount)
        task_ctr[threadIdx.x] = 0;
    __shared__ int buf[2 * (kScanThreads / 64)];
    __shared__ int carry;
    __shared__ int bad;
    __shared__ int full_tiles;
    __shared__ int tall_tails;        // partial tiles above kHalfWidthMaxRows rows (sorted tables)
    if (threadIdx.x == 0) {
        carry = 0;
        bad = 0;
        full_tiles = 0;
        tall_tails = 0;
    }
    if (layout == 0 && chunk_tiles != nullptr)
        for (int c = threadIdx.x; c < num_chunks; c += kScanThreads) {
            chunk_tiles[c] = 0;
            chunk_done[c] = 0;
        }
    __syncthreads();
    {
        MTile* const tiles = layout == 0 ? tiles_main : tiles_in_run;
        const bool tails_last = layout == 0 && num_chunks <= 1;
        for (int pass = 0; pass < (tails_last ? 2 : 1); ++pass) {
            if (pass == 1 && threadIdx.x == 0)
                full_tiles = carry;                   // read by thread 0 only, after the last barrier
            for (int g0 = 0; g0 < G; g0 += kScanThreads) {
                const int g = g0 + threadIdx.x;
                int64_t rb = 0, re = 0;
                int ex = 0, n = 0;
                if (g < G) {
                    // clamp into [0, M] so that malformed offsets can never address rows outside the buffers
                    rb = min(max(static_cast<int64_t>(offsets[g]), int64_t{0}), M);
                    re = min(max(static_cast<int64_t>(offsets[g + 1]), rb), M);
                    ex = group_expert ? group_expert[g] : g;
                    if (ex < 0 || ex >= E) {
                        if (re > rb)
                            atomicOr(&bad, 1);
                        re = rb;   // skipped
                    }
                    if (!tails_last) {
                        for (int64_t r = rb; r < re;) {
                            const int64_t cend = min(re, (r / chunk + 1) * chunk);
                            n += static_cast<int>((cend - r + bm - 1) / bm);
                            r = cend;
                        }
                    } else if (pass == 0) {
                        n = static_cast<int>(re - rb) / bm;
                    } else {
                        n = static_cast<int>(re - rb) % bm != 0 ? 1 : 0;
                    }
                }
                int incl = block_inclusive_scan(n, buf);
                int t = carry + incl - n;
                if (tails_last && pass == 1 && G <= kScanThreads) {
                    // longest partial tiles first (all groups fit one pass): the rank of this group's
                    // tail among all tails, larger first, ties by group index
                    __shared__ int tail_rows[kScanThreads];
                    const int mine = n != 0 ? static_cast<int>(re - rb) % bm : -1;
                    tail_rows[threadIdx.x] = mine;
                    if (mine > kHalfWidthMaxRows)
                        atomicAdd(&tall_tails, 1);
                    __syncthreads();
                    int rank = 0;
                    if (n != 0) {                     // groups without a tail skip the count
    #pragma unroll 8
                        for (int q = 0; q < G; ++q) {
                            const int other = tail_rows[q];
                            rank += (other > mine || (other == mine && q < g)) ? 1 : 0;
                        }
                    }
                    __syncthreads();
                    if (n != 0)
                        t = carry + rank;
                }
                // c: the tile's chunk (0 unchunked), computed once per chunk piece by the caller, since a
                // 64-bit division is a long software sequence
                auto emit = [&](int64_t r0, int64_t r1, int run_begin, int run_len, int c) {
                    if (t < max_tiles) {
                        MTile mt;
                        mt.expert = ex;
                        mt.row_begin = static_cast<int>(r0);
                        mt.row_end = static_cast<int>(r1);
                        mt.chunk = c;
                        mt.run_begin = run_begin;
                        mt.run_len = run_len;
                        mt.pad0 = mt.pad1 = 0;
                        tiles[t] = mt;
                    }
                    if (layout == 0 && chunk_tiles != nullptr && c < num_chunks)
                        atomicAdd(&chunk_tiles[c], col_tiles);
                    ++t;
                };
                if (!tails_last) {
                    // a run: the group's tiles inside one window of kChunkWindow chunks
                    const int64_t win = chunk * kChunkWindow;
                    for (int64_t r = rb; r < re;) {
                        const int64_t wend = min(re, (r / win + 1) * win);
                        int run_len = 0;
                        for (int64_t q = r; q < wend;) {
                            const int64_t cend = min(wend, (q / chunk + 1) * chunk);
                            run_len += static_cast<int>((cend - q + bm - 1) / bm);
                            q = cend;
                        }
                        const int run_begin = t;
                        for (int64_t q = r; q < wend;) {
                            const int64_t c = q / chunk;
                            const int64_t cend = min(wend, (c + 1) * chunk);
                            if ((layout == 1 || num_chunks > 1) && bm % 32 == 0) {
                                // balanced (the in-run table, and the chunked table's pieces): the
                                // piece's 32-row blocks spread over its R tiles as evenly as possible
                                // (at most one block apart; the last tile ends the piece)
                                const int len = static_cast<int>(cend - q);
                                const int nblk = (len + 31) / 32, R = (len + bm - 1) / bm;
                                int64_t r0 = q;
                                for (int i = 0; i < R; ++i) {
                                    const int64_t r1 = i == R - 1 ? cend : r0 + 32 * (nblk / R + (i < nblk % R ? 1 : 0));
                                    emit(r0, r1, run_begin, run_len, static_cast<int>(c));
                                    r0 = r1;
                                }
                                q = cend;
                                continue;
                            }
                            for (int64_t r0 = q; r0 < cend; r0 += bm)
                                emit(r0, min(cend, r0 + bm), run_begin, run_len, static_cast<int>(c));
                            q = cend;
                        }
                        r = wend;
                    }
                } else if (pass == 0) {
                    const int run_begin = t;
                    for (int i = 0; i < n; ++i)
                        emit(rb + int64_t{i} * bm, rb + int64_t{i + 1} * bm, run_begin, n, 0);
                } else if (n != 0) {
                    emit(rb + static_cast<int>(re - rb) / bm * bm, re, t, 1, 0);
                }
                __syncthreads();
                if (threadIdx.x == kScanThreads - 1)
                    carry += incl;
                __syncthreads();
            }
        }
        if (layout == 1 && threadIdx.x == 0) {
            count_in_run[0] = min(carry, max_tiles);
            count_in_run[2] = count_in_run[0];    // no suffix of short tails: no half-width tasks
        }
        if (layout == 0 && threadIdx.x == 0) {
            tile_count[0] = min(carry, max_tiles);
            // tile_count[2]: how many tiles lead the table before the short partial tiles (rows <=
            // kHalfWidthMaxRows) that the non-gated GEMM splits into half-width tasks.  Only an unchunked
            // table whose tails were sorted (longest first, one pass over the groups) has such a suffix.
            const bool sorted_tails = tails_last && G <= kScanThreads;
            tile_count[2] = sorted_tails ? min(full_tiles + tall_tails, max_tiles) : min(carry, max_tiles);
            if (write_status)
                *status = bad ? kStatusBadId : kStatusOk;
            else if (bad)
                *status = kStatusBadId;
        }
    }
}

}  // namespace

hipError_t launch_route_count(const int32_t* ids, int64_t M, int64_t E, int32_t* block_counts,
                              int64_t nblocks, hipStream_t s)
{
    route_count_kernel<<<dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s>>>(
        ids, M, static_cast<int>(E), block_counts);
    return hipGetLastError();
}

hipError_t launch_route_scan(int32_t* block_counts, int64_t nblocks, int64_t E, int64_t M,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* status,
                             hipStream_t s)
{
    route_scan_kernel<<<dim3(1), dim3(kScanThreads), 0, s>>>(
        block_counts, static_cast<int>(nblocks), static_cast<int>(E), M, counts, offsets, perm,
        status);
    return hipGetLastError();
}

hipError_t launch_route_scatter(const int32_t* ids, int64_t M, int64_t E,
                                const int32_t* block_counts, int64_t nblocks, int32_t* perm,
                                int32_t* pos, hipStream_t s)
{
    int bits = 0;
    while ((int64_t{1} << bits) < E)
        ++bits;
    route_scatter_kernel<<<dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, s>>>(
        ids, M, static_cast<int>(E), bits, block_counts, perm, pos);
    return hipGetLastError();
}

hipError_t launch_build_tiles(const int32_t* offsets, const int32_t* group_expert, int64_t G,
                              int64_t E, int64_t M, int64_t chunk, int bm, MTile* tiles, int64_t max_tiles,
                              int32_t* tile_count, int32_t* chunk_tiles, int32_t* chunk_done,
                              int64_t num_chunks, int col_tiles, int32_t* task_ctr,
                              int32_t* status, bool write_status, hipStream_t s,
                              MTile* tiles_in_run, int32_t* count_in_run)
{
    const unsigned layouts = tiles_in_run != nullptr && num_chunks <= 1 ? 2 : 1;
    build_tiles_kernel<<<dim3(layouts), dim3(kScanThreads), 0, s>>>(
        offsets, group_expert, static_cast<int>(G), static_cast<int>(E), M, chunk, bm, tiles,
        static_cast<int>(max_tiles), tile_count, chunk_tiles, chunk_done,
        static_cast<int>(num_chunks), col_tiles, task_ctr, status, write_status ? 1 : 0,
        tiles_in_run, count_in_run);
    return hipGetLastError();
}

}  // namespace moe
