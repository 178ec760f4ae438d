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

// Claims two tasks ahead in the persistent kernels: while task t runs, wave 0 claims the task after
// t's successor.  claim_issue issues the atomic on lane 0 of wave 0, its address hidden from the
// compiler so that it stays a single-lane operation whose result is waited for only where it is
// first used (a wave-wide form is rewritten into a scan that waits for the result at once);
// claim_value reads that result, after the K loop, whose last barrier has waited for every load of
// the wave.  Wave 0 then publishes the value in the claim word, and every wave reads it after the
// next task's first barrier.
__device__ __forceinline__ int claim_issue(int32_t* task_ctr, int xcd, int wave, int lane)
{
    int v = 0;
    if (wave == 0 && lane == 0) {
        int off = 0;
        asm volatile("" : "+v"(off));
        v = atomicAdd(task_ctr + xcd + off, 1);
    }
    return v;
}

__device__ __forceinline__ int claim_value(int v, int wave)
{
    int c = 0;
    if (wave == 0) {
        c = __builtin_amdgcn_readlane(v, 0);
        asm volatile("" : "+s"(c));
    }
    return c;
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
