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
//
// A captured HIP graph replays its kernel arguments unchanged, so a replayed
// launch cannot be handed its epoch; it infers it from launch counts on the
// device (eager calls pass the epoch the host counted, and keep the counts
// up to date for later replays). Work unit u of a launch (an item or a
// chunk) belongs to group u mod kLaunchGroups; the units that wait are the
// group's members, and each adds 1 to the group's 64-bit count once per
// launch. With m_g members, the count holds k * m_g + j while launch k + 1
// runs, j < m_g being the members of this launch that have added. A launch
// that infers its epoch adds as each member's last action, after the member
// read the count (with its first poll), so k = count / m_g and the epoch is
// k + 1, the same for every unit of the launch. A launch that was handed
// its epoch reads no count and adds early. 64 bits never wrap.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "plan.hpp"

namespace halo {

constexpr int kCounterStride = 32;  // uint32 words: one 128-byte line per counter

// Values of the plan's error word (0: no error): a dependency wait exceeded
// its spin limit; a flag came from another XCD than the waiting unit's.
constexpr uint32_t kErrWordTimeout = 1;
constexpr uint32_t kErrWordPlacement = 2;

// Device state of a plan with n_seg segments, in uint32 words: segment
// counters of the work-item kernels (X, then F), of the chunk kernels (X,
// then F), of the atomic force kernel (F only), the launch counts of the
// kernel families (kLaunchGroups each), one spare line.
inline size_t state_words_for(size_t n_seg)
{
    return (5 * n_seg + (size_t)kFamilies * kLaunchGroups + 1) * kCounterStride;
}

// Base for counter_f() of the atomic force kernel's own block.
inline size_t atomic_state_offset(size_t n_seg) { return 3 * n_seg * kCounterStride; }

// First launch count of a family.
inline size_t launch_groups_offset(size_t n_seg, int family)
{
    return (5 * n_seg + (size_t)family * kLaunchGroups) * kCounterStride;
}

// A counter block holds n_seg counters of the coordinate direction, then
// n_seg of the force direction. The plan keeps one block per kernel form
// (work items, chunks), each with its own launch counts, so that the forms
// never mix their counts.
__device__ __forceinline__ uint32_t *counter_x(uint32_t *state, int32_t seg)
{
    return state + (size_t)seg * kCounterStride;
}

__device__ __forceinline__ uint32_t *counter_f(uint32_t *state, int32_t n_seg, int32_t seg)
{
    return state + ((size_t)n_seg + seg) * kCounterStride;
}

// A unit's launch-count group: its count and its number of members.
struct LaunchGroup {
    uint64_t *count;
    const uint32_t *members;
};

__device__ __forceinline__ LaunchGroup launch_group(uint32_t *groups, const uint32_t *members,
                                                   uint32_t unit)
{
    const uint32_t g = unit % kLaunchGroups;
    return LaunchGroup{reinterpret_cast<uint64_t *>(groups + (size_t)g * kCounterStride),
                       members + g};
}

// Start of a member's first wait when the epoch is not known yet (0): read
// its group's count and size, completed by finish_epoch after the first poll
// has been issued.
struct EpochRead {
    uint64_t count;
    uint32_t members;
};

__device__ __forceinline__ EpochRead start_epoch(const LaunchGroup &lg, uint32_t epoch)
{
    if (epoch != 0) return EpochRead{0, 1};
    return EpochRead{__hip_atomic_load(lg.count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                     *lg.members};
}

__device__ __forceinline__ void finish_epoch(const EpochRead &r, uint32_t &epoch)
{
    if (epoch == 0) epoch = (uint32_t)(r.count / r.members) + 1u;
}

// A unit's launch-count bookkeeping: its group, its epoch (the host's, or 0
// until a wait infers it), and whether its add has been made.
struct LaunchState {
    LaunchGroup lg;
    uint32_t epoch;
    bool eager;    // the host passed the epoch: this launch reads no count
    bool counted;
};

__device__ __forceinline__ LaunchState launch_state(uint32_t *groups, const uint32_t *members,
                                                    uint32_t unit, uint32_t host_epoch)
{
    return LaunchState{launch_group(groups, members, unit), host_epoch, host_epoch != 0, false};
}

__device__ __forceinline__ void count_unit(LaunchState &ls)
{
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(ls.lg.count, (uint64_t)1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    ls.counted = true;
}

// A member's add, as early as possible when nothing in the launch reads the
// counts (its latency then overlaps the unit's work)...
__device__ __forceinline__ void count_early(LaunchState &ls, bool member)
{
    if (ls.eager && member && !ls.counted) count_unit(ls);
}

// ... else as the unit's last action, after its read of the count (same
// address, same thread or an earlier instruction of its wave), where the adds
// do not compete with the reads of the units still starting.
__device__ __forceinline__ void count_late(LaunchState &ls, bool member)
{
    if (member && !ls.counted) count_unit(ls);
}

// s_waitcnt with vmcnt(0) only (gfx9 encoding: expcnt and lgkmcnt left at max).
__device__ __forceinline__ void wait_vmem()
{
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
}

// The waits below take the unit's launch-count group and an epoch cache (0:
// not known yet). On the first wait of a unit the polling lanes read the
// launch count together with their first poll and fill the cache.

// Wave 0 polls the counters of the listed segments (lane i the i-th) until
// every one shows this epoch's completion; the workgroup then meets at a
// barrier. A wait longer than spin_limit polls sets the error word and gives
// up, so that the kernel always drains.
__device__ __forceinline__ void wait_segments(const int32_t *list, int32_t n, const uint32_t *seg_items,
                                              uint32_t *state, int32_t n_seg, bool force_dir,
                                              const LaunchGroup &lg, uint32_t &epoch,
                                              uint32_t spin_limit, uint32_t *err_word)
{
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        for (int32_t base = 0; base < n; base += 64) {
            const bool mine = base + lane < n;
            uint32_t *ctr = nullptr;
            uint32_t mult = 0;
            if (mine) {
                const int32_t s = list[base + lane];
                ctr = force_dir ? counter_f(state, n_seg, s) : counter_x(state, s);
                mult = seg_items[s];
            }
            const EpochRead er = start_epoch(lg, epoch);
            uint32_t c = mine ? __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                              : 0u;
            finish_epoch(er, epoch);
            const uint32_t target = epoch * mult;
            uint32_t polls = 0;
            while (true) {
                const bool ok = !mine || (int32_t)(c - target) >= 0;
                if (__all(ok)) break;
                if (++polls > spin_limit) {
                    if (lane == 0)
                        __hip_atomic_store(err_word, kErrWordTimeout, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_SYSTEM);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                if (mine) c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        wait_vmem();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    __syncthreads();
}

// The same wait for one segment, polled by lane 0 of wave 0.
__device__ __forceinline__ void wait_one(int32_t s, const uint32_t *seg_items, uint32_t *state,
                                         int32_t n_seg, bool force_dir, const LaunchGroup &lg,
                                         uint32_t &epoch, uint32_t spin_limit, uint32_t *err_word)
{
    if (threadIdx.x == 0) {
        uint32_t *ctr = force_dir ? counter_f(state, n_seg, s) : counter_x(state, s);
        const EpochRead er = start_epoch(lg, epoch);
        uint32_t c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        finish_epoch(er, epoch);
        const uint32_t target = epoch * seg_items[s];
        uint32_t polls = 0;
        while ((int32_t)(c - target) < 0) {
            if (++polls > spin_limit) {
                __hip_atomic_store(err_word, kErrWordTimeout, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_SYSTEM);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        wait_vmem();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    __syncthreads();
}

// Wave 0 waits until the counter that each of its lanes names (ctr; nullptr:
// none) reaches mult times this launch's epoch; the workgroup then meets at a
// barrier. One round of polls covers up to 64 counters.
__device__ __forceinline__ void wait_lanes(uint32_t *ctr, uint32_t mult, const LaunchGroup &lg,
                                           uint32_t &epoch, uint32_t spin_limit,
                                           uint32_t *err_word)
{
    if (threadIdx.x < 64) {
        const EpochRead er = start_epoch(lg, epoch);
        uint32_t c = ctr ? __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
        finish_epoch(er, epoch);
        const uint32_t target = epoch * mult;
        uint32_t polls = 0;
        while (true) {
            const bool ok = !ctr || (int32_t)(c - target) >= 0;
            if (__all(ok)) break;
            if (++polls > spin_limit) {
                if (threadIdx.x == 0)
                    __hip_atomic_store(err_word, kErrWordTimeout, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_SYSTEM);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            if (ctr) c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        wait_vmem();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    __syncthreads();
}

// ---- XCD-local flags (the index-list kernels on plans built on the host) ----
// The units of one origin run on one XCD (plan.hpp, LocalUnit), so a unit's
// stores reach the consumer through that XCD's L2: the producer writes its
// data with plain stores, waits for them (s_waitcnt vmcnt(0): the L2 has
// acknowledged them), meets its workgroup at a barrier and then stores its
// flag word, also plainly: {epoch, 0x100 | its XCC}. The consumer polls the
// flag words with loads that bypass the CU cache and are served by the L2
// (agent-scope relaxed loads), waits for them (s_waitcnt), meets at a
// barrier, and reads the data with the same kind of load. A flag from
// another XCD (the grid's workgroups did not go to the XCDs round-robin)
// would not be seen there in time, or, if seen, is reported: the error word
// becomes kErrWordPlacement.
__device__ __forceinline__ uint32_t xcc_id()
{
    return (uint32_t)__builtin_amdgcn_s_getreg(20 | (31 << 11)) & 0xfu;  // HW_REG_XCC_ID
}

// Flag word of unit position b: class-major, kp words per class (a multiple
// of 16, so that no 128-byte line holds flags of two classes).
__device__ __forceinline__ uint64_t *local_flag(uint64_t *flags, int32_t kp, int32_t b)
{
    return flags + (size_t)(b % kXcdClasses) * (size_t)kp + (size_t)(b / kXcdClasses);
}

// Wave 0 polls the flags of the listed unit positions (lane i the i-th)
// until every one shows this epoch; the workgroup then meets at a barrier.
// The epoch, if not known yet (0), is inferred with the first poll.
__device__ __forceinline__ void wait_flags(const int32_t *list, int32_t n, uint64_t *flags,
                                           int32_t kp, const LaunchGroup &lg, uint32_t &epoch,
                                           uint32_t spin_limit, uint32_t *err_word)
{
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const uint32_t mine_xcc = xcc_id() | 0x100u;
        for (int32_t base = 0; base < n; base += 64) {
            const bool mine = base + lane < n;
            uint64_t *fp = mine ? local_flag(flags, kp, list[base + lane]) : nullptr;
            const EpochRead er = start_epoch(lg, epoch);
            uint64_t f = mine ? __hip_atomic_load(fp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                              : 0u;
            finish_epoch(er, epoch);
            uint32_t polls = 0;
            while (true) {
                const bool ok = !mine || (int32_t)((uint32_t)f - epoch) >= 0;
                if (__all(ok)) break;
                if (++polls > spin_limit) {
                    if (lane == 0)
                        __hip_atomic_store(err_word, kErrWordTimeout, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_SYSTEM);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                if (mine) f = __hip_atomic_load(fp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            // a flag of this epoch written on another XCD (a flag never
            // written, after a timeout, is not a placement error)
            const bool seen = mine && (int32_t)((uint32_t)f - epoch) >= 0;
            if (__any(seen && (uint32_t)(f >> 32) != mine_xcc) && lane == 0)
                __hip_atomic_store(err_word, kErrWordPlacement, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_SYSTEM);
        }
        wait_vmem();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    __syncthreads();
}

// The unit's stores are complete in every wave (they reached the XCD's L2),
// the workgroup meets at a barrier, and thread 0 stores the flag word
// (plain store: it stays in the L2, where the consumers on this XCD poll).
__device__ __forceinline__ void set_local_flag(uint64_t *flags, int32_t kp, int32_t b,
                                               uint32_t epoch, bool withhold)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0 && !withhold)
        __hip_atomic_store(local_flag(flags, kp, b),
                           (uint64_t)epoch | ((uint64_t)(xcc_id() | 0x100u) << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// The epoch of a unit that writes a flag without waiting first, in a launch
// that was not handed its epoch (thread 0, which stores the flag).
__device__ __forceinline__ void learn_epoch(const LaunchGroup &lg, uint32_t &epoch)
{
    if (threadIdx.x == 0 && epoch == 0) {
        const EpochRead er = start_epoch(lg, epoch);
        finish_epoch(er, epoch);
    }
}

// One poll, without waiting, of two counters (lanes 0 and 1 of wave 0):
// whether both already show this epoch's completion (targets m0 and m1
// times the epoch; an epoch not known yet is read with the poll, as in the
// waits below). The workgroup then meets at a barrier, so that loads issued
// after a true answer are ordered after the poll.
__device__ __forceinline__ bool poll_both(uint32_t *c0, uint32_t m0, uint32_t *c1, uint32_t m1,
                                          const LaunchGroup &lg, uint32_t &epoch)
{
    __shared__ uint32_t ready;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        bool ok = true;
        if (lane < 2) {
            uint32_t *c = lane == 0 ? c0 : c1;
            const EpochRead er = start_epoch(lg, epoch);
            const uint32_t now = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            finish_epoch(er, epoch);
            ok = (int32_t)(now - epoch * (lane == 0 ? m0 : m1)) >= 0;
        }
        const bool all = __all(ok);
        wait_vmem();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        if (lane == 0) ready = all ? 1u : 0u;
    }
    __syncthreads();
    return ready != 0;
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
