// exchange_kernels.hpp -- the exchange kernels for gfx950 (device code only;
// the host side and the C-ABI are in halo_api.hip, which includes this file
// inside its anonymous namespace).
//
// Method: "Redesigning GROMACS Halo Exchange" (paper review):
//   Algorithm 3 FusedPackCommX  -> k_pack_fused: every pulse in one launch;
//     workgroups take work items (a run of one pulse's indexMap for one
//     sending domain) and store x[indexMap[i]] + coordShift straight into the
//     receiver's region (the pages' NVLink zero-copy store: here the receiver
//     is another region of the same HBM buffer);
//   Algorithm 4 packWithDeps    -> an item's entries below depOffset are
//     stored at once; the rest wait for the regions they forward;
//   Algorithm 5 syncAndCommWithDeps -> block barrier + one atomic per item on
//     the (pulse, sender) completion counter;
//   Algorithm 6 FusedCommUnpackF -> k_unpack_fused: pulses in reverse; the
//     forces of the receiver's region are added onto the sender's indexMap
//     targets (k_unpack_atomic: the same with atomicAdd, all pulses in flight).
// The transposed form (k_push_x, k_pull_f) runs the same exchanges from
// per-slot pulse masks. "GPU-Initiated Halo Exchange Cuts CPU Bottlenecks in
// GROMACS", "Fusing pack, put, and wait into one kernel": the per-pulse first
// design is kept as k_pack_pulse / k_unpack_pulse, one launch per pulse in
// stream order, and the staged design as k_stage_*. k_gather_x is the
// one-GPU direct coordinate form (every halo slot from its atom's home slot).
// The fused kernels take the epoch (the pages' sigVal) from the host, or
// infer it from launch counts on the device when replayed from a graph
// (sync.hpp).
//
// Everything is float32 and every add is a single IEEE add (no FMA, no flush
// of subnormals: the build passes -ffp-contract=off and keeps denormals).
//
// No #include here: halo_api.hip includes this file inside its anonymous
// namespace, after <hip/hip_runtime.h>, plan.hpp and sync.hpp.
#pragma once

constexpr int kThreads = 256;  // 4 waves of 64 per workgroup

// Debugging modes of the fused kernels, both off in normal runs:
//  - stress (halo_plan_debug_stress): workgroup b takes work unit order[b]
//    instead of its usual one (the host reverses the order inside every group
//    of mutually independent units), and every unit first sleeps a
//    pseudo-random while. Results must not change. order == nullptr and
//    seed == 0 when off.
//  - timing (halo_plan_debug_timing): wave 0 of every unit records the
//    device's constant-rate clock at the steps of the unit (start, first
//    wait, end of the last wait, first completion signal, end) and where it
//    ran, kStampWords words per unit. stamps == nullptr when off.
struct Debug {
    const int32_t *order;
    uint32_t seed;
    uint64_t *stamps;
};

constexpr int kStampWords = 8;
enum : int {
    kStampStart = 0,      // the unit's first instruction
    kStampWaitBegin = 1,  // its first dependency wait begins (0: it never waits)
    kStampWaitEnd = 2,    // its last dependency wait has ended
    kStampSignal = 3,     // its first completion signal is sent (stores complete)
    kStampEnd = 4,        // its last instruction
    kStampBlock = 5,      // workgroup index
    kStampHwId = 6,       // HW_ID register (wave, SIMD, CU, shader array, engine)
    kStampXcc = 7         // XCC_ID register (the XCD the unit ran on)
};

__device__ __forceinline__ void stress_delay(uint32_t seed, uint32_t unit)
{
    uint32_t h = (unit + 1u) * 0x9E3779B1u ^ seed;
    h ^= h >> 15;
    h *= 0x85EBCA77u;
    h ^= h >> 13;
    for (uint32_t i = 0; i < (h & 31u); ++i) __builtin_amdgcn_s_sleep(127);
}

// s_getreg_b32 operands: register id, bit offset 0, 32 bits.
constexpr int kHwRegHwId = 4 | (31 << 11);
constexpr int kHwRegXccId = 20 | (31 << 11);

// The unit's first stamp: its start, where it runs, and zeros for the steps
// it may not reach.
__device__ __forceinline__ void stamp_start(const Debug &d, uint32_t unit)
{
    if (d.stamps && threadIdx.x == 0) {
        uint64_t *s = d.stamps + (size_t)unit * kStampWords;
        s[kStampStart] = __builtin_amdgcn_s_memrealtime();
        s[kStampWaitBegin] = 0;
        s[kStampWaitEnd] = 0;
        s[kStampSignal] = 0;
        s[kStampEnd] = 0;
        s[kStampBlock] = blockIdx.x;
        s[kStampHwId] = (uint32_t)__builtin_amdgcn_s_getreg(kHwRegHwId);
        s[kStampXcc] = (uint32_t)__builtin_amdgcn_s_getreg(kHwRegXccId) & 0xfu;
    }
}

// Stamp k of the unit; with first_only, only if it is still 0.
__device__ __forceinline__ void stamp(const Debug &d, uint32_t unit, int k, bool first_only = false)
{
    if (d.stamps && threadIdx.x == 0) {
        uint64_t *s = d.stamps + (size_t)unit * kStampWords + k;
        if (!first_only || *s == 0) *s = __builtin_amdgcn_s_memrealtime();
    }
}

// ---- buffer addressing ----------------------------------------------------
// x, f and the indexMap are read and written through buffer descriptors: one
// 12-byte float triple per buffer_load/store_dwordx3, 32-bit byte offsets, and
// hardware range checking (an offset past the end returns zeros on a load and
// drops a store). kInvalid is such an offset; the plan keeps every buffer
// below 2 GiB so that it is never in range.
typedef float f3v __attribute__((ext_vector_type(3)));
constexpr uint32_t kInvalid = 0x80000000u;
constexpr int kPlain = 0;      // cached: data another access of this XCD may reuse
constexpr int kStream = 2;     // nt: touched once in this launch, streamed past the caches
constexpr int kShared = 16;    // sc1: agent-coherent access, bypasses the XCD-private caches
constexpr int32_t kRsrcWord3 = 0x00020000;  // raw buffer, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, kRsrcWord3);
}

template <int AUX>
__device__ __forceinline__ f3v load3(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    return __builtin_amdgcn_raw_buffer_load_b96(r, byte_off, 0, AUX);
}

template <int AUX>
__device__ __forceinline__ void store3(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f3v v)
{
    __builtin_amdgcn_raw_buffer_store_b96(v, r, byte_off, 0, AUX);
}

// indexMap entry e, or 0 when !ok (the load is issued either way, so that no
// branch separates the loads of one thread).
__device__ __forceinline__ uint32_t load_index(__amdgpu_buffer_rsrc_t r, int32_t e, bool ok)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, ok ? (uint32_t)e * 4u : kInvalid, 0, kStream);
}

// Gather x[idx[map_begin + e]] + shift and store it at slot region_begin + e,
// for e in [lo, hi), hi - lo <= EPT * kThreads. Branch-free: lanes past hi
// load slot 0 and store to kInvalid. All index loads are issued first, then
// all gathers, then all stores.
template <int EPT, int LD, int ST>
__device__ __forceinline__ void pack_span(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t ridx,
                                          int32_t map_begin, int32_t region_begin, int32_t lo,
                                          int32_t hi, f3v shift)
{
    uint32_t src[EPT], dst[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = lo + (int32_t)threadIdx.x + j * kThreads;
        const bool ok = e < hi;
        src[j] = load_index(ridx, map_begin + e, ok) * 12u;
        dst[j] = ok ? (uint32_t)(region_begin + e) * 12u : kInvalid;
    }
    f3v v[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) v[j] = load3<LD>(rx, src[j]);
#pragma unroll
    for (int j = 0; j < EPT; ++j) store3<ST>(rx, dst[j], v[j] + shift);
}

// ---- work items ------------------------------------------------------------

// One coordinate-direction item of the fused exchange (Algorithms 3 and 4).
// Thread t owns entries t, t+256, ... of the item. All index loads are
// issued first (the indexMap is read-only), then the entries below depOffset
// are gathered and stored at once; the rest wait for the regions they
// forward. Lanes outside a phase use kInvalid offsets, so the code has no
// branches between the loads of one thread. Home slots are never written
// during the launch and are read through the caches; forwarded regions are
// stored and read with sc1 accesses.
template <int EPT, int ST>
__device__ __forceinline__ void pack_item_fused_st(const WorkItem *it, __amdgpu_buffer_rsrc_t rx,
                                                   __amdgpu_buffer_rsrc_t ridx,
                                                   const int32_t *recv_from,
                                                   const uint32_t *seg_items, uint32_t *state,
                                                   int32_t n_dom, const halo::LaunchGroup &lg,
                                                   uint32_t &epoch, uint32_t spin_limit,
                                                   uint32_t *err_word, const Debug &dbg,
                                                   uint32_t unit)
{
    const int32_t n_indep = it->n_indep;
    const int32_t n_total = it->n_total;
    const int32_t region_begin = it->region_begin;
    const f3v shift = {it->shift[0], it->shift[1], it->shift[2]};
    uint32_t src[EPT], dst[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        const bool ok = e < n_total;
        src[j] = load_index(ridx, it->map_begin + e, ok) * 12u;
        dst[j] = ok ? (uint32_t)(region_begin + e) * 12u : kInvalid;
    }
    f3v v[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const bool ind = (int32_t)threadIdx.x + j * kThreads < n_indep;
        v[j] = load3<kPlain>(rx, ind ? src[j] : kInvalid);
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const bool ind = (int32_t)threadIdx.x + j * kThreads < n_indep;
        store3<ST>(rx, ind ? dst[j] : kInvalid, v[j] + shift);
    }
    if (n_total > n_indep) {
        // lane r of wave 0 polls the arrival of the region the sender
        // received in pulse r, if the dependent entries read it
        const uint32_t lane = threadIdx.x, wmask = it->xwait_mask;
        uint32_t *ctr = nullptr;
        uint32_t mult = 0;
        if (lane < 32u && ((wmask >> lane) & 1u)) {
            const int32_t s = (int32_t)lane * n_dom + recv_from[(int32_t)lane * n_dom + it->domain];
            ctr = halo::counter_x(state, s);
            mult = seg_items[s];
        }
        stamp(dbg, unit, kStampWaitBegin);
        halo::wait_lanes(ctr, mult, lg, epoch, spin_limit, err_word);
        stamp(dbg, unit, kStampWaitEnd);
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const bool dep = (int32_t)threadIdx.x + j * kThreads >= n_indep;
            v[j] = load3<kShared>(rx, dep ? src[j] : kInvalid);
        }
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const bool dep = (int32_t)threadIdx.x + j * kThreads >= n_indep;
            store3<ST>(rx, dep ? dst[j] : kInvalid, v[j] + shift);
        }
    }
}

template <int EPT>
__device__ __forceinline__ void pack_item_fused(const WorkItem *it, __amdgpu_buffer_rsrc_t rx,
                                                __amdgpu_buffer_rsrc_t ridx,
                                                const int32_t *recv_from,
                                                const uint32_t *seg_items, uint32_t *state,
                                                int32_t n_dom, const halo::LaunchGroup &lg,
                                                uint32_t &epoch, uint32_t spin_limit,
                                                uint32_t *err_word, int32_t withhold,
                                                const Debug &dbg, uint32_t unit)
{
    if (it->flags & halo::kItemXStoreShared) {
        pack_item_fused_st<EPT, kShared>(it, rx, ridx, recv_from, seg_items, state, n_dom, lg,
                                         epoch, spin_limit, err_word, dbg, unit);
        halo::signal_done(halo::counter_x(state, it->seg), it->seg == withhold);
        stamp(dbg, unit, kStampSignal);
    } else {
        // last pulse: no later pulse forwards its region, nobody waits on it
        pack_item_fused_st<EPT, kStream>(it, rx, ridx, recv_from, seg_items, state, n_dom, lg,
                                        epoch, spin_limit, err_word, dbg, unit);
    }
}

// f[idx[map_begin + e]] += f[region_begin + e] for e < n; the index loads were
// issued before the dependency wait.
template <int EPT, int LD, int ST>
__device__ __forceinline__ void unpack_span(__amdgpu_buffer_rsrc_t rf, const uint32_t *tgt,
                                            int32_t region_begin, int32_t n)
{
    f3v add[EPT], cur[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        add[j] = load3<LD>(rf, e < n ? (uint32_t)(region_begin + e) * 12u : kInvalid);
        cur[j] = load3<LD>(rf, tgt[j]);  // kInvalid reads zeros
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) store3<ST>(rf, tgt[j], cur[j] + add[j]);
}

template <int EPT>
__device__ __forceinline__ void load_targets(__amdgpu_buffer_rsrc_t ridx, int32_t map_begin,
                                             int32_t n_total, uint32_t *tgt)
{
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        const bool ok = e < n_total;
        const uint32_t t = load_index(ridx, map_begin + e, ok) * 12u;
        tgt[j] = ok ? t : kInvalid;
    }
}

// One force-direction item of the fused exchange (Algorithm 6): wait until
// pulse p+1 is finished for the sender and its receiver, then add.
template <int EPT>
__device__ __forceinline__ void unpack_item_fused(const WorkItem *it, __amdgpu_buffer_rsrc_t rf,
                                                  __amdgpu_buffer_rsrc_t ridx,
                                                  const uint32_t *seg_items, uint32_t *state,
                                                  int32_t n_seg, const halo::LaunchGroup &lg,
                                                  uint32_t &epoch, uint32_t spin_limit,
                                                  uint32_t *err_word, int32_t withhold,
                                                  const Debug &dbg, uint32_t unit)
{
    const int32_t n_total = it->n_total;
    const int32_t region_begin = it->region_begin;
    // The indexMap is read-only during the exchange: load it before waiting.
    uint32_t tgt[EPT];
    load_targets<EPT>(ridx, it->map_begin, n_total, tgt);
    if (it->fwait[0] >= 0) {
        const int32_t nw = it->fwait[1] >= 0 && it->fwait[1] != it->fwait[0] ? 2 : 1;
        stamp(dbg, unit, kStampWaitBegin);
        halo::wait_segments(it->fwait, nw, seg_items, state, n_seg, true, lg, epoch, spin_limit,
                            err_word);
        stamp(dbg, unit, kStampWaitEnd);
    }
    const int32_t fl = it->flags;
    if (fl & halo::kItemFLoadShared) {
        if (fl & halo::kItemFStoreShared)
            unpack_span<EPT, kShared, kShared>(rf, tgt, region_begin, n_total);
        else
            unpack_span<EPT, kShared, kStream>(rf, tgt, region_begin, n_total);
    } else {
        if (fl & halo::kItemFStoreShared)
            unpack_span<EPT, kStream, kShared>(rf, tgt, region_begin, n_total);
        else
            unpack_span<EPT, kStream, kStream>(rf, tgt, region_begin, n_total);
    }
    // pulse 0 runs last: nobody waits on its completion
    if (fl & halo::kItemFStoreShared) {
        halo::signal_done(halo::counter_f(state, n_seg, it->seg), it->seg == withhold);
        stamp(dbg, unit, kStampSignal);
    }
}

// One force-direction item with atomic accumulation: Algorithm 6 as the
// pages print it, with the items of every pulse in flight together and the
// adds done by atomicAdd. The item waits only until the slots it reads (the
// receiver's region of its pulse) hold their final sums, i.e. for the
// later-pulse segments that add into them; its own targets may take adds of
// other pulses at the same time. The order of the adds onto one slot is not
// fixed, so the result equals the ordered exchange up to rounding, and
// exactly whenever every partial sum is exact (small integers, for example).
template <int EPT>
__device__ __forceinline__ void unpack_item_atomic(const WorkItem *it, float *f,
                                                   __amdgpu_buffer_rsrc_t rf,
                                                   __amdgpu_buffer_rsrc_t ridx,
                                                   const uint32_t *seg_items, uint32_t *state,
                                                   int32_t n_seg, int32_t n_dom,
                                                   const halo::LaunchGroup &lg, uint32_t &epoch,
                                                   uint32_t spin_limit, uint32_t *err_word,
                                                   int32_t withhold)
{
    const int32_t n_total = it->n_total;
    const int32_t region_begin = it->region_begin;
    uint32_t tgt[EPT], src[EPT];
    load_targets<EPT>(ridx, it->map_begin, n_total, tgt);
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        src[j] = e < n_total ? (uint32_t)(region_begin + e) * 12u : kInvalid;
    }
    f3v add[EPT];
    const uint32_t amask = it->await_mask;
    if (amask) {
        // lane q of wave 0 polls segment (q, receiver)
        const uint32_t lane = threadIdx.x;
        uint32_t *ctr = nullptr;
        uint32_t mult = 0;
        if (lane < 32u && ((amask >> lane) & 1u)) {
            const int32_t s = (int32_t)lane * n_dom + it->receiver;
            ctr = halo::counter_f(state, n_seg, s);
            mult = seg_items[s];
        }
        halo::wait_lanes(ctr, mult, lg, epoch, spin_limit, err_word);
#pragma unroll
        for (int j = 0; j < EPT; ++j) add[j] = load3<kShared>(rf, src[j]);
    } else {
#pragma unroll
        for (int j = 0; j < EPT; ++j) add[j] = load3<kStream>(rf, src[j]);
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (tgt[j] == kInvalid) continue;
        float *t = f + tgt[j] / 4u;
        __hip_atomic_fetch_add(t + 0, add[j].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(t + 1, add[j].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(t + 2, add[j].z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the targets of a pulse p > 0 may be the sources of an earlier pulse
    if (it->flags & halo::kItemFStoreShared)
        halo::signal_done(halo::counter_f(state, n_seg, it->seg), it->seg == withhold);
}

// ---- kernels -----------------------------------------------------------------

// Fused coordinate exchange: ONE launch for all pulses, one item per
// workgroup, items in pulse-major order of the workgroup index. An item only
// waits on items of earlier pulses, i.e. on workgroups with smaller indices.
// The hardware hands workgroups of a grid to the XCDs round-robin and each
// XCD dispatches its share in increasing index order, so the smallest
// unfinished item is always resident or next in line: every wait ends. The
// spin limit turns a violation of that order into HALO_ERR_TIMEOUT, not a
// hang. (No atomic ticket: 2560 same-address device atomics serialise for
// about 20 us on MI355X; and no cooperative launch, which idles the GPU for
// about 20 us before each launch.)
template <int EPT>
__global__ __launch_bounds__(kThreads) void k_pack_fused(
    float *x, uint32_t x_bytes, const int32_t *__restrict__ idx, uint32_t idx_bytes,
    const WorkItem *__restrict__ items, const int32_t *__restrict__ recv_from,
    const uint32_t *__restrict__ seg_items, uint32_t *state, int32_t n_dom, uint32_t *groups,
    const uint32_t *__restrict__ members, uint32_t host_epoch, uint32_t spin_limit,
    uint32_t *err_word, int32_t withhold, Debug dbg)
{
    const uint32_t u = dbg.order ? (uint32_t)dbg.order[blockIdx.x] : blockIdx.x;
    stamp_start(dbg, u);
    if (dbg.seed) stress_delay(dbg.seed, u);
    halo::LaunchState ls = halo::launch_state(groups, members, u, host_epoch);
    const WorkItem *it = items + u;
    const bool member = it->n_total > it->n_indep;  // the item waits
    halo::count_early(ls, member);
    pack_item_fused<EPT>(it, make_rsrc(x, x_bytes), make_rsrc(idx, idx_bytes), recv_from,
                         seg_items, state, n_dom, ls.lg, ls.epoch, spin_limit, err_word, withhold,
                         dbg, u);
    halo::count_late(ls, member);
    stamp(dbg, u, kStampEnd);
}

// Fused force exchange: ONE launch, workgroup b takes item n_items-1-b, so
// the last pulse comes first; same progress argument.
template <int EPT>
__global__ __launch_bounds__(kThreads) void k_unpack_fused(
    float *f, uint32_t f_bytes, const int32_t *__restrict__ idx, uint32_t idx_bytes,
    const WorkItem *__restrict__ items, const uint32_t *__restrict__ seg_items, uint32_t *state,
    int32_t n_seg, uint32_t n_items, uint32_t *groups, const uint32_t *__restrict__ members,
    uint32_t host_epoch, uint32_t spin_limit, uint32_t *err_word, int32_t withhold, Debug dbg)
{
    const uint32_t u = dbg.order ? (uint32_t)dbg.order[blockIdx.x] : n_items - 1u - blockIdx.x;
    stamp_start(dbg, u);
    if (dbg.seed) stress_delay(dbg.seed, u);
    halo::LaunchState ls = halo::launch_state(groups, members, u, host_epoch);
    const WorkItem *it = items + u;
    const bool member = it->fwait[0] >= 0;  // the item waits
    halo::count_early(ls, member);
    unpack_item_fused<EPT>(it, make_rsrc(f, f_bytes), make_rsrc(idx, idx_bytes), seg_items,
                           state, n_seg, ls.lg, ls.epoch, spin_limit, err_word, withhold, dbg, u);
    halo::count_late(ls, member);
    stamp(dbg, u, kStampEnd);
}

// Fused force exchange with atomic adds: ONE launch, last pulse first; an item
// waits only on segments of later pulses, i.e. on smaller workgroup indices.
template <int EPT>
__global__ __launch_bounds__(kThreads) void k_unpack_atomic(
    float *f, uint32_t f_bytes, const int32_t *__restrict__ idx, uint32_t idx_bytes,
    const WorkItem *__restrict__ items, const uint32_t *__restrict__ seg_items, uint32_t *state,
    int32_t n_seg, int32_t n_dom, uint32_t n_items, uint32_t *groups,
    const uint32_t *__restrict__ members, uint32_t host_epoch, uint32_t spin_limit,
    uint32_t *err_word, int32_t withhold, Debug dbg)
{
    const uint32_t u = dbg.order ? (uint32_t)dbg.order[blockIdx.x] : n_items - 1u - blockIdx.x;
    stamp_start(dbg, u);
    if (dbg.seed) stress_delay(dbg.seed, u);
    halo::LaunchState ls = halo::launch_state(groups, members, u, host_epoch);
    // every item is a member here (which items wait is known on the device only)
    halo::count_early(ls, true);
    unpack_item_atomic<EPT>(items + u, f, make_rsrc(f, f_bytes), make_rsrc(idx, idx_bytes),
                            seg_items, state, n_seg, n_dom, ls.lg, ls.epoch, spin_limit, err_word,
                            withhold);
    halo::count_late(ls, true);
    stamp(dbg, u, kStampEnd);
}

// ---- index-list form, XCD-local units (plans built on the host) -------------
// The same exchanges as k_pack_fused / k_unpack_fused, with the units of
// plan.hpp's LocalUnit: runs of one origin, placed so that every dependency
// stays on one XCD. Data written in the launch and read by another unit
// stays in that XCD's L2 (plain stores, reads past the CU cache); the
// signals are per-unit flag words (sync.hpp, wait_flags / set_local_flag).
// Unit position b is workgroup b of the coordinate kernel and workgroup
// n - 1 - b of the force kernel; empty positions exit at once.

// Store a unit's n consecutive float triples (v[j] of thread t is entry
// t + j * kThreads) at slots region_begin, region_begin + 1, ... through LDS:
// the triples are written to LDS, then the run's bytes go out as 16-byte
// stores on 16-byte boundaries (a head and a tail of up to three 4-byte
// stores). The form the pages' design names for float3 coordinates; kept as
// an ablation beside the 12-byte stores.
template <int EPT, int ST>
__device__ __forceinline__ void store_run_lds4(__amdgpu_buffer_rsrc_t rx, int32_t region_begin,
                                               int32_t n, const f3v *v, float *lds)
{
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        if (e < n) {
            lds[3 * e] = v[j].x;
            lds[3 * e + 1] = v[j].y;
            lds[3 * e + 2] = v[j].z;
        }
    }
    __syncthreads();
    // words k < words of the run sit at byte b0 + 4k; the body [a0, a1) is
    // 16-byte aligned, the head (before a0) and the tail (from the body's
    // end) have at most three words each
    const uint32_t words = (uint32_t)n * 3u;
    const uint32_t b0 = (uint32_t)region_begin * 12u, b1 = b0 + words * 4u;
    const uint32_t a0 = (b0 + 15u) & ~15u, a1 = b1 & ~15u;
    const uint32_t head = min(words, (a0 - b0) / 4u);
    const uint32_t body_end = a1 > a0 ? (a1 - b0) / 4u : head;
    // (the 4-byte store takes the word's bits, not a converted value)
    if (threadIdx.x < head)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lds[threadIdx.x]), rx,
                                              b0 + 4u * threadIdx.x, 0, ST);
    if (threadIdx.x < words - body_end) {
        const uint32_t w = body_end + threadIdx.x;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lds[w]), rx, b0 + 4u * w, 0, ST);
    }
    if (a1 > a0) {
        typedef float f4v __attribute__((ext_vector_type(4)));
        for (uint32_t q = threadIdx.x; q < (a1 - a0) / 16u; q += kThreads) {
            const uint32_t w = head + 4u * q;
            const f4v d = {lds[w], lds[w + 1], lds[w + 2], lds[w + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(d, rx, a0 + 16u * q, 0, ST);
        }
    }
}

// Coordinates (Algorithms 3 and 4): x[region_begin + e] = x[idx[map_begin +
// e]] + shift; a unit that reads a region first waits for its writers.
// LDS4: the stores go through LDS as 16-byte stores (store_run_lds4).
template <int EPT, bool LDS4 = false>
__global__ __launch_bounds__(kThreads) void k_pack_local(
    float *x, uint32_t x_bytes, const int32_t *__restrict__ idx, uint32_t idx_bytes,
    const halo::LocalUnit *__restrict__ units, const int32_t *__restrict__ waits,
    uint64_t *flags, int32_t kp, uint32_t *groups, const uint32_t *__restrict__ members,
    uint32_t host_epoch, uint32_t spin_limit, uint32_t *err_word, int32_t withhold, Debug dbg)
{
    const int32_t b = dbg.order ? dbg.order[blockIdx.x] : (int32_t)blockIdx.x;
    stamp_start(dbg, (uint32_t)b);
    const halo::LocalUnit *un = units + b;
    const int32_t n = un->n_total;
    if (n == 0) {  // an empty position
        stamp(dbg, (uint32_t)b, kStampEnd);
        return;
    }
    if (dbg.seed) stress_delay(dbg.seed, (uint32_t)b);
    halo::LaunchState ls = halo::launch_state(groups, members, (uint32_t)b, host_epoch);
    const int32_t nw = un->wx_n;
    const bool flagged = (un->flags & halo::kLocalXWaited) != 0;
    const bool member = nw > 0 || flagged;
    halo::count_early(ls, member);
    const auto rx = make_rsrc(x, x_bytes), ridx = make_rsrc(idx, idx_bytes);
    const f3v shift = {un->shift[0], un->shift[1], un->shift[2]};
    const int32_t map_begin = un->map_begin, region_begin = un->region_begin;
    uint32_t src[EPT], dst[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        const bool ok = e < n;
        src[j] = load_index(ridx, map_begin + e, ok) * 12u;
        dst[j] = ok ? (uint32_t)(region_begin + e) * 12u : kInvalid;
    }
    f3v v[EPT];
    if (nw == 0) {
        // home slots: final before the launch
        if (flagged) halo::learn_epoch(ls.lg, ls.epoch);
#pragma unroll
        for (int j = 0; j < EPT; ++j) v[j] = load3<kPlain>(rx, src[j]);
    } else {
        stamp(dbg, (uint32_t)b, kStampWaitBegin);
        halo::wait_flags(waits + un->wx_off, nw, flags, kp, ls.lg, ls.epoch, spin_limit,
                         err_word);
        stamp(dbg, (uint32_t)b, kStampWaitEnd);
#pragma unroll
        for (int j = 0; j < EPT; ++j) v[j] = load3<kShared>(rx, src[j]);
    }
    if constexpr (LDS4) {
        __shared__ float lds[3 * EPT * kThreads];
#pragma unroll
        for (int j = 0; j < EPT; ++j) v[j] = v[j] + shift;
        if (flagged) {
            store_run_lds4<EPT, kPlain>(rx, region_begin, n, v, lds);
            halo::set_local_flag(flags, kp, b, ls.epoch, un->seg == withhold);
            stamp(dbg, (uint32_t)b, kStampSignal);
        } else {
            store_run_lds4<EPT, kStream>(rx, region_begin, n, v, lds);
        }
    } else if (flagged) {
        // a later unit of this XCD forwards these slots
#pragma unroll
        for (int j = 0; j < EPT; ++j) store3<kPlain>(rx, dst[j], v[j] + shift);
        halo::set_local_flag(flags, kp, b, ls.epoch, un->seg == withhold);
        stamp(dbg, (uint32_t)b, kStampSignal);
    } else {
#pragma unroll
        for (int j = 0; j < EPT; ++j) store3<kStream>(rx, dst[j], v[j] + shift);
    }
    halo::count_late(ls, member);
    stamp(dbg, (uint32_t)b, kStampEnd);
}

// Forces (Algorithm 6, pulses in reverse): f[idx[map_begin + e]] +=
// f[region_begin + e], after every later unit that adds into either slot.
template <int EPT>
__global__ __launch_bounds__(kThreads) void k_unpack_local(
    float *f, uint32_t f_bytes, const int32_t *__restrict__ idx, uint32_t idx_bytes,
    const halo::LocalUnit *__restrict__ units, int32_t n_units,
    const int32_t *__restrict__ waits, uint64_t *flags, int32_t kp, uint32_t *groups,
    const uint32_t *__restrict__ members, uint32_t host_epoch, uint32_t spin_limit,
    uint32_t *err_word, int32_t withhold, Debug dbg)
{
    // Every scalar argument in SGPRs from the start: their loads go out
    // together here instead of one by one on the way to the first wait
    // (0.2-0.3 us per exchange on the 4x4x4 and 4x4x8 workloads).
    asm volatile("" ::"s"(groups), "s"(members), "s"(host_epoch), "s"(spin_limit), "s"(err_word),
                 "s"(withhold), "s"(dbg.seed), "s"(dbg.stamps), "s"(flags), "s"(kp), "s"(waits));
    const int32_t b = dbg.order ? dbg.order[blockIdx.x] : n_units - 1 - (int32_t)blockIdx.x;
    stamp_start(dbg, (uint32_t)b);
    const halo::LocalUnit *un = units + b;
    const int32_t n = un->n_total;
    if (n == 0) {  // an empty position
        stamp(dbg, (uint32_t)b, kStampEnd);
        return;
    }
    if (dbg.seed) stress_delay(dbg.seed, (uint32_t)b);
    halo::LaunchState ls = halo::launch_state(groups, members, (uint32_t)b, host_epoch);
    const int32_t nw = un->wf_n;
    const bool flagged = (un->flags & halo::kLocalFWaited) != 0;
    const bool member = nw > 0 || flagged;
    halo::count_early(ls, member);
    const auto rf = make_rsrc(f, f_bytes), ridx = make_rsrc(idx, idx_bytes);
    const int32_t map_begin = un->map_begin, region_begin = un->region_begin;
    // the indexMap is read-only in the launch: its loads go out before the wait
    uint32_t tgt[EPT], src[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        const bool ok = e < n;
        const uint32_t t = load_index(ridx, map_begin + e, ok) * 12u;
        tgt[j] = ok ? t : kInvalid;
        src[j] = ok ? (uint32_t)(region_begin + e) * 12u : kInvalid;
    }
    f3v add[EPT], cur[EPT];
    if (nw == 0) {
        // no unit of this launch has touched these slots yet
        if (flagged) halo::learn_epoch(ls.lg, ls.epoch);
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            add[j] = load3<kStream>(rf, src[j]);
            cur[j] = load3<kStream>(rf, tgt[j]);
        }
    } else {
        stamp(dbg, (uint32_t)b, kStampWaitBegin);
        halo::wait_flags(waits + un->wf_off, nw, flags, kp, ls.lg, ls.epoch, spin_limit,
                         err_word);
        stamp(dbg, (uint32_t)b, kStampWaitEnd);
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            add[j] = load3<kShared>(rf, src[j]);
            cur[j] = load3<kShared>(rf, tgt[j]);
        }
    }
    if (flagged) {
        // an earlier pulse reads or adds into these targets in this launch
#pragma unroll
        for (int j = 0; j < EPT; ++j) store3<kPlain>(rf, tgt[j], cur[j] + add[j]);
        halo::set_local_flag(flags, kp, b, ls.epoch, un->seg == withhold);
        stamp(dbg, (uint32_t)b, kStampSignal);
    } else {
#pragma unroll
        for (int j = 0; j < EPT; ++j) store3<kStream>(rf, tgt[j], cur[j] + add[j]);
    }
    halo::count_late(ls, member);
    stamp(dbg, (uint32_t)b, kStampEnd);
}

// ---- transposed form: per-slot pulse masks --------------------------------

// Pulse ranks of one chunk. Thread t owns slots first + t + j*256 (j < EPT),
// i.e. slot order is row-major over rows (j, wave) of 64 slots. For pulse p
// the slot's entry of indexMap_p is chunk.rank[p], plus the chunk's bit-p
// slots in earlier rows, plus those earlier in its own row (a wave ballot).
// The middle term depends on the masks only; the plan keeps it in a table
// built once by k_chunk_rows (uint16, since a chunk holds at most 2048
// slots): rows[((chunk * 4 + wave) * n_pulse + p) * EPT + j].
__device__ __forceinline__ size_t chunk_rows_at(int32_t chunk, int wave, int32_t n_pulse, int ept)
{
    return ((size_t)chunk * 4 + (size_t)wave) * (size_t)n_pulse * (size_t)ept;
}

// Builds the row table of every chunk: per pulse and row, the count of the
// row's bit-p slots (ballots), then exclusive prefixes over the rows.
template <int EPT>
__global__ __launch_bounds__(kThreads) void k_chunk_rows(const uint8_t *__restrict__ slot_mask,
                                                         const halo::Chunk *__restrict__ chunks,
                                                         int32_t n_pulse,
                                                         uint16_t *__restrict__ rows)
{
    constexpr int kRow = EPT * 4;
    __shared__ uint32_t cnt[halo::kMaxMaskPulses][kRow];
    const halo::Chunk *c = chunks + blockIdx.x;
    const int32_t first = c->first, count = c->count;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint32_t m[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        m[j] = e < count ? (uint32_t)slot_mask[first + e] : 0u;
    }
    for (int32_t p = 0; p < n_pulse; ++p) {
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const uint64_t b = __ballot((m[j] >> p) & 1u);
            if (lane == 0) cnt[p][j * 4 + wave] = (uint32_t)__popcll(b);
        }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < n_pulse * kRow; k += kThreads) {
        const int p = k / kRow, q = k % kRow;
        uint32_t acc = 0;
        for (int r = 0; r < q; ++r) acc += cnt[p][r];
        rows[chunk_rows_at((int32_t)blockIdx.x, q % 4, n_pulse, EPT) + (size_t)p * EPT + q / 4] =
            (uint16_t)acc;
    }
}

// The row table entries of this thread's wave, one per lane (lane p*EPT + j
// holds pulse p, row j), loaded with the chunk's masks.
template <int EPT>
__device__ __forceinline__ uint32_t load_wave_rows(const uint16_t *rows, int32_t chunk,
                                                   int32_t n_pulse)
{
    const int lane = threadIdx.x & 63;
    const size_t at = chunk_rows_at(chunk, threadIdx.x >> 6, n_pulse, EPT);
    return lane < n_pulse * EPT ? (uint32_t)rows[at + lane] : 0u;
}

// Position among the chunk's bit-p slots of this thread's row-j slot.
template <int EPT>
__device__ __forceinline__ uint32_t rank_in_chunk(uint32_t wave_rows, int32_t p, int j, bool bit)
{
    const uint64_t b = __ballot(bit);
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_rows, p * EPT + j) +
           __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}

// Fused coordinate exchange, transposed form (Algorithms 3 and 4): one
// workgroup per chunk, chunks in zone order (home slots of every domain,
// then the region of pulse 0, pulse 1, ...). A home chunk never waits (its
// entries are the independent ones below depOffset); a region chunk waits for
// the arrival of its region, then forwards it. Each slot is read once and
// stored, plus coordShift, to every pulse whose bit it carries.
template <int EPT>
__global__ __launch_bounds__(kThreads) void k_push_x(
    float *x, uint32_t x_bytes, const uint8_t *__restrict__ slot_mask,
    const halo::Chunk *__restrict__ chunks, const uint16_t *__restrict__ rows,
    const int32_t *__restrict__ dest_start, const float4 *__restrict__ shift4,
    const uint32_t *__restrict__ x_arrivals, uint32_t *state, int32_t n_dom, int32_t n_pulse,
    uint32_t *groups, const uint32_t *__restrict__ members, uint32_t host_epoch,
    uint32_t spin_limit, uint32_t *err_word, int32_t withhold, Debug dbg)
{
    const uint32_t u = dbg.order ? (uint32_t)dbg.order[blockIdx.x] : blockIdx.x;
    stamp_start(dbg, u);
    if (dbg.seed) stress_delay(dbg.seed, u);
    halo::LaunchState ls = halo::launch_state(groups, members, u, host_epoch);
    const halo::Chunk *c = chunks + u;
    halo::count_early(ls, c->zone >= 0);  // region chunks wait
    const int32_t first = c->first, count = c->count, D = c->domain;
    const uint32_t umask = c->mask;
    const auto rx = make_rsrc(x, x_bytes);

    uint32_t m[EPT], off[EPT];
    f3v v[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        m[j] = e < count ? (uint32_t)slot_mask[first + e] : 0u;
        off[j] = e < count ? (uint32_t)(first + e) * 12u : kInvalid;
    }
    const uint32_t wrows = load_wave_rows<EPT>(rows, (int32_t)u, n_pulse);
    if (c->zone < 0) {
        // home slots are final before the launch: load them with the masks
#pragma unroll
        for (int j = 0; j < EPT; ++j) v[j] = load3<kStream>(rx, off[j]);
    }
    if (c->zone >= 0) {
        // region slots are filled by another domain in this launch; every
        // slot is loaded, sent or not, so that the loads cover whole lines
        stamp(dbg, u, kStampWaitBegin);
        halo::wait_one(c->xwait, x_arrivals, state, n_dom * n_pulse, false, ls.lg, ls.epoch,
                       spin_limit, err_word);
        stamp(dbg, u, kStampWaitEnd);
#pragma unroll
        for (int j = 0; j < EPT; ++j) v[j] = load3<kShared>(rx, off[j]);
    }
    for (int32_t p = 0; p < n_pulse; ++p) {
        if (!((umask >> p) & 1u)) continue;
        const int32_t base = dest_start[p * n_dom + D] + c->rank[p];
        const float4 sh4 = shift4[p * n_dom + D];
        const f3v s3 = {sh4.x, sh4.y, sh4.z};
        uint32_t dst[EPT];
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const bool bit = (m[j] >> p) & 1u;
            const uint32_t r = rank_in_chunk<EPT>(wrows, p, j, bit);
            dst[j] = bit ? (uint32_t)(base + (int32_t)r) * 12u : kInvalid;
        }
        if (p + 1 < n_pulse) {
            // the region may be forwarded by a later pulse of this launch:
            // store coherently and signal its arrival as soon as it is
            // complete, before the stores of later pulses
#pragma unroll
            for (int j = 0; j < EPT; ++j) store3<kShared>(rx, dst[j], v[j] + s3);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            halo::wait_vmem();
            __syncthreads();
            const int32_t seg = p * n_dom + D;
            if (threadIdx.x == 0 && seg != withhold)
                __hip_atomic_fetch_add(halo::counter_x(state, seg), 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            stamp(dbg, u, kStampSignal, true);
        } else {
            // last pulse: nobody forwards this region, nobody waits on it
#pragma unroll
            for (int j = 0; j < EPT; ++j) store3<kStream>(rx, dst[j], v[j] + s3);
        }
    }
    halo::count_late(ls, c->zone >= 0);
    stamp(dbg, u, kStampEnd);
}

// Fused force exchange, transposed form (Algorithm 6): one workgroup per
// chunk, regions of later pulses first, home slots last. Every thread keeps
// the running sum of its target slot in registers and adds the sources of
// its pulses in strict reverse order; before pulse p it waits until the
// sources (the receiver's region of pulse p) hold their final sums. Every
// slot of the chunk is read once and written once, the ones no pulse sends
// with the value they were read with: no other work unit writes them, and
// whole-line stores cost less than the byte-masked stores that leaving them
// out would make.
template <int EPT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void k_pull_f(
    float *f, uint32_t f_bytes, const uint8_t *__restrict__ slot_mask,
    const halo::Chunk *__restrict__ chunks, const int32_t *__restrict__ forder,
    const uint16_t *__restrict__ rows, const int32_t *__restrict__ dest_start,
    const int32_t *__restrict__ send_to, const uint32_t *__restrict__ zone_chunks,
    uint32_t *state, int32_t n_dom, int32_t n_pulse, uint32_t *groups,
    const uint32_t *__restrict__ members, uint32_t host_epoch, uint32_t spin_limit,
    uint32_t *err_word, int32_t withhold, Debug dbg)
{
    const int32_t u = dbg.order ? dbg.order[blockIdx.x] : forder[blockIdx.x];
    stamp_start(dbg, (uint32_t)u);
    if (dbg.seed) stress_delay(dbg.seed, (uint32_t)u);
    halo::LaunchState ls = halo::launch_state(groups, members, (uint32_t)u, host_epoch);
    const halo::Chunk *c = chunks + u;
    const int32_t first = c->first, count = c->count, D = c->domain, zone = c->zone;
    const uint32_t umask = c->mask;
    const auto rf = make_rsrc(f, f_bytes);
    const int32_t n_seg = n_dom * n_pulse;

    // The last pulse's regions are summed by nobody in this launch, so its
    // sources need no wait: they are the dense run of the receiver's region
    // from this chunk's rank on. They are loaded at once, with the masks,
    // straight into LDS (buffer-to-LDS loads: lane l of a load writes its
    // 12 bytes at 16 * l from the wave's base), and read there by rank.
    __shared__ float top_src[4 * EPT * kThreads];
    const int32_t top = n_pulse - 1;
    const bool has_top = (umask >> top) & 1u;
    const int32_t top_n = has_top ? c->top_sends : 0;
    if (has_top) {
        const int32_t tbase = dest_start[top * n_dom + D] + c->rank[top];
        const int32_t wave = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int32_t e = (int32_t)threadIdx.x + j * kThreads;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rf, (__attribute__((address_space(3))) void *)(top_src + 4 * (j * kThreads + wave * 64)),
                12, e < top_n ? (uint32_t)(tbase + e) * 12u : kInvalid, 0, 0, kStream);
        }
    }
    uint32_t m[EPT], off[EPT];
    f3v v[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        m[j] = e < count ? (uint32_t)slot_mask[first + e] : 0u;
        off[j] = e < count ? (uint32_t)(first + e) * 12u : kInvalid;
    }
    const uint32_t wrows = load_wave_rows<EPT>(rows, (int32_t)u, n_pulse);
    // Only this workgroup writes these slots, and nobody before it in this
    // launch: plain loads (streamed, read once), issued together with the
    // masks.
#pragma unroll
    for (int j = 0; j < EPT; ++j) v[j] = load3<kStream>(rf, off[j]);
    if (has_top) {
        halo::wait_vmem();  // this wave's loads into LDS are done
        __syncthreads();    // and every other wave's
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const bool bit = (m[j] >> top) & 1u;
            const uint32_t r = rank_in_chunk<EPT>(wrows, top, j, bit);
            if (bit) {
                const f3v a = {top_src[4 * r], top_src[4 * r + 1], top_src[4 * r + 2]};
                v[j] = v[j] + a;
            }
        }
    }
    bool waited = false;
    int32_t p_next = n_pulse - 2;
    // The two pulses below the last one: when the regions both read already
    // hold their final sums (one poll of both), their loads go out together;
    // otherwise each waits in turn in the loop below.
    if (n_pulse >= 3 && ((umask >> (n_pulse - 3)) & 3u) == 3u) {
        const int32_t hi = n_pulse - 2, lo = n_pulse - 3;
        const int32_t zh = hi * n_dom + send_to[hi * n_dom + D];
        const int32_t zl = lo * n_dom + send_to[lo * n_dom + D];
        if (zone_chunks[zh] > 0 && zone_chunks[zl] > 0) {
            halo::count_early(ls, true);  // the chunk waits
            stamp(dbg, (uint32_t)u, kStampWaitBegin);
            const bool both = halo::poll_both(halo::counter_f(state, n_seg, zh), zone_chunks[zh],
                                              halo::counter_f(state, n_seg, zl), zone_chunks[zl],
                                              ls.lg, ls.epoch);
            stamp(dbg, (uint32_t)u, kStampWaitEnd);
            if (both) {
                waited = true;
                p_next = lo - 1;
                const int32_t bh = dest_start[hi * n_dom + D] + c->rank[hi];
                const int32_t bl = dest_start[lo * n_dom + D] + c->rank[lo];
                uint32_t sh[EPT], sl[EPT];
#pragma unroll
                for (int j = 0; j < EPT; ++j) {
                    const bool bit_h = (m[j] >> hi) & 1u;
                    const uint32_t rh = rank_in_chunk<EPT>(wrows, hi, j, bit_h);
                    sh[j] = bit_h ? (uint32_t)(bh + (int32_t)rh) * 12u : kInvalid;
                    const bool bit_l = (m[j] >> lo) & 1u;
                    const uint32_t rl = rank_in_chunk<EPT>(wrows, lo, j, bit_l);
                    sl[j] = bit_l ? (uint32_t)(bl + (int32_t)rl) * 12u : kInvalid;
                }
                f3v ah[EPT], al[EPT];
#pragma unroll
                for (int j = 0; j < EPT; ++j) ah[j] = load3<kShared>(rf, sh[j]);
#pragma unroll
                for (int j = 0; j < EPT; ++j) al[j] = load3<kShared>(rf, sl[j]);
#pragma unroll
                for (int j = 0; j < EPT; ++j) {
                    if (sh[j] != kInvalid) v[j] = v[j] + ah[j];
                    if (sl[j] != kInvalid) v[j] = v[j] + al[j];
                }
            }
        }
    }
    for (int32_t p = p_next; p >= 0; --p) {
        if (!((umask >> p) & 1u)) continue;
        const int32_t R = send_to[p * n_dom + D];
        const int32_t zseg = p * n_dom + R;
        if (zone_chunks[zseg] > 0) {
            halo::count_early(ls, true);  // the chunk waits
            stamp(dbg, (uint32_t)u, kStampWaitBegin, true);
            halo::wait_one(zseg, zone_chunks, state, n_seg, true, ls.lg, ls.epoch, spin_limit,
                           err_word);
            stamp(dbg, (uint32_t)u, kStampWaitEnd);
            waited = true;
        }
        const int32_t base = dest_start[p * n_dom + D] + c->rank[p];
        uint32_t src[EPT];
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const bool bit = (m[j] >> p) & 1u;
            const uint32_t r = rank_in_chunk<EPT>(wrows, p, j, bit);
            src[j] = bit ? (uint32_t)(base + (int32_t)r) * 12u : kInvalid;
        }
        f3v add[EPT];
        if (zone_chunks[zseg] > 0) {
#pragma unroll
            for (int j = 0; j < EPT; ++j) add[j] = load3<kShared>(rf, src[j]);
        } else {
#pragma unroll
            for (int j = 0; j < EPT; ++j) add[j] = load3<kStream>(rf, src[j]);
        }
#pragma unroll
        for (int j = 0; j < EPT; ++j)
            if (src[j] != kInvalid) v[j] = v[j] + add[j];
    }
    if (zone >= 0) {
        // region sums are read by another domain in this launch
#pragma unroll
        for (int j = 0; j < EPT; ++j) store3<kShared>(rf, off[j], v[j]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        halo::wait_vmem();
        __syncthreads();
        const int32_t seg = zone * n_dom + D;
        if (threadIdx.x == 0 && seg != withhold)
            __hip_atomic_fetch_add(halo::counter_f(state, n_seg, seg), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        stamp(dbg, (uint32_t)u, kStampSignal);
    } else {
#pragma unroll
        for (int j = 0; j < EPT; ++j) store3<kStream>(rf, off[j], v[j]);
    }
    halo::count_late(ls, waited);
    stamp(dbg, (uint32_t)u, kStampEnd);
}

// Per-pulse baseline: one launch per pulse, one item per workgroup, no
// counters; the kernel boundary orders the pulses, so every access is cached.
template <int EPT>
__global__ __launch_bounds__(kThreads) void k_pack_pulse(float *x, uint32_t x_bytes,
                                                         const int32_t *__restrict__ idx,
                                                         uint32_t idx_bytes,
                                                         const WorkItem *__restrict__ items,
                                                         int32_t item_base)
{
    const WorkItem *it = items + item_base + blockIdx.x;
    const f3v shift = {it->shift[0], it->shift[1], it->shift[2]};
    pack_span<EPT, kPlain, kPlain>(make_rsrc(x, x_bytes), make_rsrc(idx, idx_bytes),
                                   it->map_begin, it->region_begin, 0, it->n_total, shift);
}

template <int EPT>
__global__ __launch_bounds__(kThreads) void k_unpack_pulse(float *f, uint32_t f_bytes,
                                                           const int32_t *__restrict__ idx,
                                                           uint32_t idx_bytes,
                                                           const WorkItem *__restrict__ items,
                                                           int32_t item_base)
{
    const WorkItem *it = items + item_base + blockIdx.x;
    uint32_t tgt[EPT];
    load_targets<EPT>(make_rsrc(idx, idx_bytes), it->map_begin, it->n_total, tgt);
    unpack_span<EPT, kPlain, kPlain>(make_rsrc(f, f_bytes), tgt, it->region_begin, it->n_total);
}

// Staged baseline (the message-passing design the pages compare against): a
// pulse first packs into a staging buffer, entry e of the concatenated
// indexMap at stage[e], and a second launch moves the staged run into the
// receiver's region; forces go the other way round (region -> stage, then
// the scatter-add from stage). Two launches per pulse and 24 bytes more per
// entry than the zero-copy store.
template <int EPT>
__global__ __launch_bounds__(kThreads) void k_stage_pack(
    float *x, uint32_t x_bytes, float *stage, uint32_t stage_bytes,
    const int32_t *__restrict__ idx, uint32_t idx_bytes, const WorkItem *__restrict__ items,
    int32_t item_base)
{
    const WorkItem *it = items + item_base + blockIdx.x;
    const f3v shift = {it->shift[0], it->shift[1], it->shift[2]};
    const auto rx = make_rsrc(x, x_bytes), rs = make_rsrc(stage, stage_bytes);
    const auto ridx = make_rsrc(idx, idx_bytes);
    uint32_t src[EPT], dst[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        const bool ok = e < it->n_total;
        src[j] = load_index(ridx, it->map_begin + e, ok) * 12u;
        dst[j] = ok ? (uint32_t)(it->map_begin + e) * 12u : kInvalid;
    }
    f3v v[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) v[j] = load3<kPlain>(rx, src[j]);
#pragma unroll
    for (int j = 0; j < EPT; ++j) store3<kPlain>(rs, dst[j], v[j] + shift);
}

// to_region != 0: buf[region_begin + e] = stage[map_begin + e] (coordinates);
// to_region == 0: stage[map_begin + e] = buf[region_begin + e] (forces).
template <int EPT>
__global__ __launch_bounds__(kThreads) void k_stage_move(float *buf, uint32_t buf_bytes,
                                                         float *stage, uint32_t stage_bytes,
                                                         const WorkItem *__restrict__ items,
                                                         int32_t item_base, int32_t to_region)
{
    const WorkItem *it = items + item_base + blockIdx.x;
    const auto rb = make_rsrc(buf, buf_bytes), rs = make_rsrc(stage, stage_bytes);
    const auto rsrc = to_region ? rs : rb, rdst = to_region ? rb : rs;
    uint32_t src[EPT], dst[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        const bool ok = e < it->n_total;
        const uint32_t so = ok ? (uint32_t)(it->map_begin + e) * 12u : kInvalid;
        const uint32_t ro = ok ? (uint32_t)(it->region_begin + e) * 12u : kInvalid;
        src[j] = to_region ? so : ro;
        dst[j] = to_region ? ro : so;
    }
    f3v v[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) v[j] = load3<kPlain>(rsrc, src[j]);
#pragma unroll
    for (int j = 0; j < EPT; ++j) store3<kPlain>(rdst, dst[j], v[j]);
}

template <int EPT>
__global__ __launch_bounds__(kThreads) void k_stage_unpack(
    float *f, uint32_t f_bytes, float *stage, uint32_t stage_bytes,
    const int32_t *__restrict__ idx, uint32_t idx_bytes, const WorkItem *__restrict__ items,
    int32_t item_base)
{
    const WorkItem *it = items + item_base + blockIdx.x;
    const auto rf = make_rsrc(f, f_bytes), rs = make_rsrc(stage, stage_bytes);
    uint32_t tgt[EPT];
    load_targets<EPT>(make_rsrc(idx, idx_bytes), it->map_begin, it->n_total, tgt);
    f3v add[EPT], cur[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        add[j] = load3<kPlain>(rs, e < it->n_total ? (uint32_t)(it->map_begin + e) * 12u
                                                   : kInvalid);
        cur[j] = load3<kPlain>(rf, tgt[j]);
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) store3<kPlain>(rf, tgt[j], cur[j] + add[j]);
}


// ---- direct coordinate form (halo_exchange_x_direct) -----------------------
// With every domain in one buffer, the value the forwarding chain delivers to
// a halo slot can be gathered straight from its atom's home slot: it is the
// home value plus the coordShift of every pulse on the atom's path. An atom
// wraps at most once per dimension (a dimension has at most n_d - 1 pulses,
// which start from distinct cells), so each component receives at most one
// non-zero shift and one IEEE add per component gives the chain's bits (the
// zero adds change nothing but -0 into +0, which both forms do on their first
// add). origin[e] = home slot of entry e's atom | wrap bits << kOriginShift
// (bit d: +L_d); slots stay below 2^28.
constexpr uint32_t kOriginShift = 28;
constexpr uint32_t kOriginSlot = (1u << kOriginShift) - 1u;

// slot_origin[s] = s for every slot (home slots are their own origin; halo
// slots are overwritten pulse by pulse before anything reads them).
__global__ __launch_bounds__(kThreads) void k_origin_init(uint32_t *__restrict__ slot_origin,
                                                          int32_t n_slots)
{
    const int32_t s = (int32_t)(blockIdx.x * kThreads + threadIdx.x);
    if (s < n_slots) slot_origin[s] = (uint32_t)s;
}

// One pulse's items: each entry takes the origin of the slot it reads plus
// the segment's wrap bit and passes it on to the slot it fills. A pulse reads
// only slots filled before it, so one launch per pulse in stream order is
// race-free.
template <int EPT>
__global__ __launch_bounds__(kThreads) void k_origin_pulse(const int32_t *__restrict__ idx,
                                                           const WorkItem *__restrict__ items,
                                                           int32_t item_base,
                                                           uint32_t *__restrict__ slot_origin,
                                                           uint32_t *__restrict__ origin)
{
    const WorkItem *it = items + item_base + blockIdx.x;
    const uint32_t bits = (it->shift[0] != 0.f ? 1u : 0u) | (it->shift[1] != 0.f ? 2u : 0u) |
                          (it->shift[2] != 0.f ? 4u : 0u);
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        if (e < it->n_total) {
            const uint32_t o = slot_origin[idx[it->map_begin + e]] | (bits << kOriginShift);
            origin[it->map_begin + e] = o;
            slot_origin[it->region_begin + e] = o;
        }
    }
}

// x[region_begin + e] = x[origin slot] + (L_d where the wrap bit d is set,
// else 0), every item independently: no waits, no counters, one launch.
template <int EPT>
__global__ __launch_bounds__(kThreads) void k_gather_x(float *x, uint32_t x_bytes,
                                                       const uint32_t *origin,
                                                       uint32_t origin_bytes,
                                                       const WorkItem *__restrict__ items,
                                                       float lx, float ly, float lz, Debug dbg)
{
    stamp_start(dbg, blockIdx.x);
    const WorkItem *it = items + blockIdx.x;
    const auto rx = make_rsrc(x, x_bytes), ro = make_rsrc(origin, origin_bytes);
    const int32_t n = it->n_total;
    uint32_t o[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        o[j] = __builtin_amdgcn_raw_buffer_load_b32(
            ro, e < n ? (uint32_t)(it->map_begin + e) * 4u : kInvalid, 0, kStream);
    }
    f3v v[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        v[j] = load3<kPlain>(rx, e < n ? (o[j] & kOriginSlot) * 12u : kInvalid);
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int32_t e = (int32_t)threadIdx.x + j * kThreads;
        const uint32_t b = o[j] >> kOriginShift;
        const f3v s = {(b & 1u) ? lx : 0.f, (b & 2u) ? ly : 0.f, (b & 4u) ? lz : 0.f};
        store3<kStream>(rx, e < n ? (uint32_t)(it->region_begin + e) * 12u : kInvalid, v[j] + s);
    }
    stamp(dbg, blockIdx.x, kStampEnd);
}

// ---- home slots and per-atom arrays (halo_scatter_home, halo_gather_home) ----
// Atom a's values live at slot home_slot[a]: scatter copies a per-atom array
// of float triples into the home slots, gather copies them back out.
__global__ __launch_bounds__(kThreads) void k_scatter_home(const float *values, uint32_t value_bytes,
                                                           float *slots, uint32_t slot_bytes,
                                                           const int64_t *__restrict__ home_slot,
                                                           int64_t n_atoms)
{
    const int64_t a = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const bool ok = a < n_atoms;
    const uint32_t hs = (uint32_t)home_slot[ok ? a : 0];  // n_atoms >= 1
    const uint32_t s = ok ? hs * 12u : kInvalid;
    const f3v v = load3<kStream>(make_rsrc(values, value_bytes), ok ? (uint32_t)a * 12u : kInvalid);
    store3<kPlain>(make_rsrc(slots, slot_bytes), s, v);
}

__global__ __launch_bounds__(kThreads) void k_gather_home(const float *slots, uint32_t slot_bytes,
                                                          float *values, uint32_t value_bytes,
                                                          const int64_t *__restrict__ home_slot,
                                                          int64_t n_atoms)
{
    const int64_t a = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const bool ok = a < n_atoms;
    const uint32_t hs = (uint32_t)home_slot[ok ? a : 0];  // n_atoms >= 1
    const uint32_t s = ok ? hs * 12u : kInvalid;
    const f3v v = load3<kPlain>(make_rsrc(slots, slot_bytes), s);
    store3<kStream>(make_rsrc(values, value_bytes), ok ? (uint32_t)a * 12u : kInvalid, v);
}
