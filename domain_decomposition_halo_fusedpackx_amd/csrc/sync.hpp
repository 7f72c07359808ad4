// sync.hpp -- device-side dependency signals of the fused exchange kernels.
//
// "Redesigning GROMACS Halo Exchange" (paper review), Algorithm 4 (a leader
// acquire-waits on the signal of each pulse it depends on, then a scope
// barrier releases the rest of the block) and Algorithm 5 (block barrier, then
// one GPU-scope atomic per block on a per-pulse completion counter), s.4
// "Memory ordering semantics".
//
// On one MI355X every domain lives in the same HBM, so the pages' system-scope
// signals become agent-scope ones. gfx950 has one L2 per XCD and the L2s are
// not coherent with one another. An agent-scope release or acquire fence is
// implemented by writing back or invalidating the whole L2 of the XCD, which
// costs far more than the data it protects. The kernels therefore keep every
// slot that one work item writes and another reads in the same launch out of
// the non-coherent caches: such slots are written and read with agent-scope
// (sc1) buffer accesses, which go to the device-coherent level. What is left
// to order is completion, not visibility:
//   producer: its (sc1) stores are complete (s_waitcnt vmcnt(0)) in every wave
//             -> workgroup barrier -> one relaxed agent-scope atomic add;
//   consumer: relaxed agent-scope loads of the counter until it is reached ->
//             s_waitcnt vmcnt(0) -> workgroup barrier -> (sc1) loads.
// This is the same discipline AMD's rocPRIM uses for its decoupled look-back
// on gfx942/gfx950.
//
// Counters are monotone: segment s (one pulse of one sending domain) is cut
// into m_s work items, each adds 1 when it is done, so after exchange number
// e (the epoch) the counter holds e * m_s (mod 2^32). A waiter compares with
// wrap-around arithmetic; nothing is reset between exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace halo {

constexpr int kCounterStride = 32;  // uint32 words: one 128-byte line per counter

// A counter block holds n_seg counters of the coordinate direction, then
// n_seg of the force direction. The plan keeps one block per kernel family,
// each with its own epochs, so that the families never mix their counts.
__device__ __forceinline__ uint32_t *counter_x(uint32_t *state, int32_t seg)
{
    return state + (size_t)seg * kCounterStride;
}

__device__ __forceinline__ uint32_t *counter_f(uint32_t *state, int32_t n_seg, int32_t seg)
{
    return state + ((size_t)n_seg + seg) * kCounterStride;
}

// s_waitcnt with vmcnt(0) only (gfx9 encoding: expcnt and lgkmcnt left at max).
__device__ __forceinline__ void wait_vmem()
{
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
}

// Wave 0 polls the counters of the listed segments (lane i the i-th) until
// every one shows this epoch's completion; the workgroup then meets at a
// barrier. A wait longer than spin_limit polls sets the error word and gives
// up, so that the kernel always drains.
__device__ __forceinline__ void wait_segments(const int32_t *list, int32_t n, const uint32_t *seg_items,
                                              uint32_t *state, int32_t n_seg, bool force_dir,
                                              uint32_t epoch, uint32_t spin_limit,
                                              uint32_t *err_word)
{
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        for (int32_t base = 0; base < n; base += 64) {
            const bool mine = base + lane < n;
            uint32_t *ctr = nullptr;
            uint32_t target = 0;
            if (mine) {
                const int32_t s = list[base + lane];
                ctr = force_dir ? counter_f(state, n_seg, s) : counter_x(state, s);
                target = epoch * seg_items[s];
            }
            uint32_t polls = 0;
            while (true) {
                bool ok = true;
                if (mine) {
                    uint32_t c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ok = (int32_t)(c - target) >= 0;
                }
                if (__all(ok)) break;
                if (++polls > spin_limit) {
                    if (lane == 0)
                        __hip_atomic_store(err_word, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_SYSTEM);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        wait_vmem();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    __syncthreads();
}

// The same wait for one segment, polled by lane 0 of wave 0.
__device__ __forceinline__ void wait_one(int32_t s, const uint32_t *seg_items, uint32_t *state,
                                         int32_t n_seg, bool force_dir, uint32_t epoch,
                                         uint32_t spin_limit, uint32_t *err_word)
{
    if (threadIdx.x == 0) {
        uint32_t *ctr = force_dir ? counter_f(state, n_seg, s) : counter_x(state, s);
        const uint32_t target = epoch * seg_items[s];
        uint32_t polls = 0;
        while ((int32_t)(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                         target) < 0) {
            if (++polls > spin_limit) {
                __hip_atomic_store(err_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        wait_vmem();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    __syncthreads();
}

// Wave 0 waits until the counter that each of its lanes names (ctr; nullptr:
// none) reaches that lane's target; the workgroup then meets at a barrier.
// One round of polls covers up to 64 counters.
__device__ __forceinline__ void wait_lanes(uint32_t *ctr, uint32_t target, uint32_t spin_limit,
                                           uint32_t *err_word)
{
    if (threadIdx.x < 64) {
        uint32_t polls = 0;
        while (true) {
            bool ok = true;
            if (ctr) {
                const uint32_t c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = (int32_t)(c - target) >= 0;
            }
            if (__all(ok)) break;
            if (++polls > spin_limit) {
                if (threadIdx.x == 0)
                    __hip_atomic_store(err_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        wait_vmem();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    __syncthreads();
}

// Completion of one work item: every wave waits until its stores are
// complete, the workgroup meets at a barrier, and one thread adds 1 to the
// segment's counter.
__device__ __forceinline__ void signal_done(uint32_t *ctr, bool withhold)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0 && !withhold)
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace halo
