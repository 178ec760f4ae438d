// Pieces shared by the grouped-GEMM kernels: the persistent task scheduler, row-block placement,
// the chunk-completion counter and the global->LDS copy.
#pragma once

#include "common.h"
#include "internal.h"

namespace moe {

// Row block i of wave row wm covers tile rows 32 * (kWM * i + wm) .. + 31 (wave rows interleave, so
// a partial tile splits its row blocks evenly between them).
template <int kWM>
__device__ __forceinline__ int row_block(int i, int wm)
{
    return 32 * (kWM * i + wm);
}

// The workgroup's next task: wave 0 claims it (every lane takes part, lane 0 adds 1, the others 0,
// so no lane-divergent branch sits in the barrier loop: lane-divergent regions there let the
// compiler's loop restructuring split one wave's lanes across different barrier paths).  Tasks are
// dealt in blocks of `blk` (the workgroups of one XCD): block j belongs to XCD j % 8, and each XCD's
// workgroups claim that XCD's tasks in order from its own counter.  Whatever the workgroups'
// relative speeds, an XCD works on about `blk` consecutive tasks at a time (shared A rows and
// weight strips in its L2), and overall progress follows task order.
__device__ __forceinline__ int claim_task(int* claimed, int32_t* task_ctr, int xcd, int blk, int wave,
                                          int lane)
{
    if (wave == 0) {
        const int v = atomicAdd(&task_ctr[xcd], lane == 0 ? 1 : 0);
        *claimed = __builtin_amdgcn_readfirstlane(v);
    }
    __syncthreads();
    const int i = __builtin_amdgcn_readfirstlane(*claimed);   // one value per workgroup
    __syncthreads();                                          // read by all before wave 0 reuses it
    return ((i / blk) * kXcdCount + xcd) * blk + i % blk;
}

// Claims issued early and read late in the persistent kernels.  claim_issue: every wave runs the
// same instruction sequence, so no lane-divergent region sits in the kernels' barrier loops (such a
// region once let the compiler split a wave across barrier paths); inside it EXEC is narrowed to
// lane 0 of wave 0 (none elsewhere) for one returning atomic add on the XCD's counter.  Written as
// assembly because the compiler's atomic either becomes a scan that waits for the result at once
// (uniform address) or, as a wave-wide operation, 64 serialised same-address atomics.  The result
// register is written when the atomic returns: it is read only by claim_value, after the K loop,
// whose barriers have waited for every load of the wave, and claim_value waits once more itself.
__device__ __forceinline__ int claim_issue(int32_t* task_ctr, int xcd, int wave, int lane)
{
    (void)lane;
    int v;
    uint64_t saved;
    const int mask = __builtin_amdgcn_readfirstlane(wave == 0 ? 1 : 0);
    int32_t* const addr = task_ctr + xcd;
    const int one = 1;
    asm volatile("s_mov_b64 %1, exec\n\t"
                 "s_mov_b32 exec_lo, %4\n\t"
                 "s_mov_b32 exec_hi, 0\n\t"
                 "global_atomic_add %0, %2, %3, off sc0\n\t"
                 "s_mov_b64 exec, %1"
                 : "=&v"(v), "=&s"(saved)
                 : "v"(addr), "v"(one), "s"(mask)
                 : "memory");
    return v;
}

// The claim of claim_issue (wave 0's lane 0; other waves get 0).
__device__ __forceinline__ int claim_value(int v, int wave)
{
    int c;
    asm volatile("s_waitcnt vmcnt(0)\n\tv_readlane_b32 %0, %1, 0" : "=s"(c) : "v"(v) : "memory");
    return wave == 0 ? c : 0;
}

// Task t belongs to the run holding row tile t / n_nt; inside the run, row tiles vary fastest.
__device__ __forceinline__ MTile decode_task(int t, int n_nt, const MTile* __restrict__ tiles, int& nt)
{
    const MTile head = tiles[t / n_nt];
    const int local = t - n_nt * head.run_begin;
    nt = local / head.run_len;
    return tiles[head.run_begin + local % head.run_len];
}

// Counts a finished fc2 tile for its chunk (the whole first wave takes part; see claim_task).
__device__ __forceinline__ void count_done(int32_t* chunk_done, int chunk, int wave, int lane)
{
    __threadfence();
    __syncthreads();
    if (wave == 0)
        atomicAdd(&chunk_done[chunk], lane == 0 ? 1 : 0);
}

// LDS DMA of 16 bytes per lane (global_load_lds_dwordx4): lane i reads base + voff (bytes) and
// writes LDS byte address lds + 16 * i.  `base` and `lds` must be wave-uniform.  M0 carries the
// LDS address; no compiled code keeps a live value in M0 across this statement (LDS instructions on
// this target do not use it).  The copies count in vmcnt like any other vector-memory load, and
// the waits for them are explicit (step_barrier).  Written as inline assembly: the compiler's own
// form of this instruction makes every later LDS read wait for all copies in flight.
__device__ __forceinline__ void lds_copy16(const void* base, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory");
}

// 16-byte store that writes through the L2 (sc0 sc1), for outputs whose completion other XCDs may
// watch through the chunk counters.
__device__ __forceinline__ void store16_through(void* p, u32x4_t v)
{
    asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" :: "v"(p), "v"(v) : "memory");
}

// Counts a finished tile whose outputs all went out with store16_through: every store of the
// workgroup has completed (vmcnt), then one relaxed device-scope increment.  Unlike a device-scope
// fence this writes back and invalidates nothing in the L2.
__device__ __forceinline__ void count_done_through(int32_t* chunk_done, int chunk, int wave, int lane)
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (wave == 0)
        atomicAdd(&chunk_done[chunk], lane == 0 ? 1 : 0);
}

}  // namespace moe
