// halo_api.hip -- the C-ABI of include/halo.h: plans, uploads, launches.
//
// The kernels are in exchange_kernels.hpp (included below); the host plan
// builder in plan.cpp, the device plan builder in plan_device.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "../../include/halo.h"
#include "plan.hpp"
#include "plan_state.hpp"
#include "sync.hpp"

static_assert(HALO_SELECT_SLAB == halo::kSelectSlab && HALO_SELECT_CORNER == halo::kSelectCorner,
              "selection codes");

using halo::WorkItem;

namespace {

constexpr int32_t kDefaultItemEntries = 1024;

thread_local std::string g_last_error;

halo_status fail(halo_status st, const std::string &msg)
{
    g_last_error = msg;
    return st;
}

// Device code; included here, inside this anonymous namespace, after the
// HIP runtime, plan.hpp and sync.hpp.
#include "exchange_kernels.hpp"

}  // namespace

namespace {

halo_status hip_fail(hipError_t e, const char *what)
{
    return fail(HALO_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

void free_device(halo_plan *p)
{
    halo::free_device_build(p);  // arenas first: the pointers into them become null
    for (void *q : {(void *)p->d_idx, (void *)p->d_items, (void *)p->d_recv_from,
                    (void *)p->d_send_to, (void *)p->d_stage, (void *)p->d_seg_items,
                    (void *)p->d_state, (void *)p->d_mask, (void *)p->d_chunks,
                    (void *)p->d_forder, (void *)p->d_dest_start, (void *)p->d_shift4,
                    (void *)p->d_x_arrivals, (void *)p->d_zone_chunks, (void *)p->d_local_map,
                    (void *)p->d_home_slot, (void *)p->d_stress, (void *)p->d_origin,
                    (void *)p->d_members, (void *)p->d_rows, (void *)p->d_stamps,
                    (void *)p->d_lunits, (void *)p->d_lwaits, (void *)p->d_lflags})
        if (q) (void)hipFree(q);
    if (p->h_err) (void)hipHostFree(p->h_err);
    p->d_idx = p->d_recv_from = p->d_send_to = p->d_forder = p->d_dest_start = nullptr;
    p->d_stress = nullptr;
    p->stress_seed = 0;
    p->d_stamps = nullptr;
    p->stamp_units = 0;
    p->d_lunits = nullptr;
    p->d_lwaits = nullptr;
    p->d_lflags = nullptr;
    p->lflag_words = 0;
    p->d_local_map = nullptr;
    p->d_home_slot = nullptr;
    p->d_items = nullptr;
    p->d_stage = p->d_shift4 = nullptr;
    p->d_origin = nullptr;
    p->d_members = nullptr;
    p->d_rows = nullptr;
    p->rows_cap = 0;
    p->d_seg_items = p->d_state = p->d_x_arrivals = p->d_zone_chunks = nullptr;
    p->d_mask = nullptr;
    p->d_chunks = nullptr;
    p->h_err = p->d_err = nullptr;
    p->uploaded = false;
}

// Copy v to a new device array at *dst, unless *dst already exists (arrays a
// device-side build produced in place).
template <class T>
hipError_t upload_vec(T **dst, const std::vector<T> &v)
{
    if (*dst) return hipSuccess;
    size_t bytes = std::max<size_t>(v.size() * sizeof(T), 16);
    hipError_t e = hipMalloc((void **)dst, bytes);
    if (e != hipSuccess) return e;
    if (!v.empty()) e = hipMemcpy(*dst, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice);
    return e;
}

int ept_for(int32_t item_entries)
{
    const int e = (item_entries + kThreads - 1) / kThreads;
    return e <= 1 ? 1 : e <= 2 ? 2 : e <= 4 ? 4 : 8;
}

// Kernel entry points for the plan's items-per-thread.
struct Kernels {
    const void *pack_fused, *unpack_fused, *pack_pulse, *unpack_pulse, *push_x, *pull_f,
        *unpack_atomic, *stage_pack, *stage_move, *stage_unpack, *origin_pulse, *gather_x,
        *chunk_rows, *pack_local, *unpack_local, *pack_local_lds4;
};

template <int EPT>
Kernels kernels_for()
{
    return {(const void *)&k_pack_fused<EPT>,    (const void *)&k_unpack_fused<EPT>,
            (const void *)&k_pack_pulse<EPT>,    (const void *)&k_unpack_pulse<EPT>,
            (const void *)&k_push_x<EPT>,        (const void *)&k_pull_f<EPT>,
            (const void *)&k_unpack_atomic<EPT>, (const void *)&k_stage_pack<EPT>,
            (const void *)&k_stage_move<EPT>,    (const void *)&k_stage_unpack<EPT>,
            (const void *)&k_origin_pulse<EPT>,  (const void *)&k_gather_x<EPT>,
            (const void *)&k_chunk_rows<EPT>,    (const void *)&k_pack_local<EPT>,
            (const void *)&k_unpack_local<EPT>,  (const void *)&k_pack_local<EPT, true>};
}

Kernels kernels(int32_t item_entries)
{
    switch (ept_for(item_entries)) {
    case 1: return kernels_for<1>();
    case 2: return kernels_for<2>();
    case 4: return kernels_for<4>();
    default: return kernels_for<8>();
    }
}

// Debugging modes of a kernel family: the stress-mode order (see
// halo_plan_debug_stress; [items X | items F | chunks X | chunks F | local
// units X | local units F] in p->d_stress) and the timing stamps
// (halo_plan_debug_timing).
enum StressOrder {
    kOrderItemsX = 0,
    kOrderItemsF = 1,
    kOrderChunksX = 2,
    kOrderChunksF = 3,
    kOrderLocalX = 4,
    kOrderLocalF = 5
};

Debug debug_of(const halo_plan *p, StressOrder which)
{
    Debug d{nullptr, 0u, p->d_stamps};
    if (!p->stress_seed || !p->d_stress) return d;
    const size_t ni = p->h.items.size(), nc = p->h.chunks.size(), nl = p->h.lunits.size();
    const size_t off[6] = {0, ni, 2 * ni, 2 * ni + nc, 2 * ni + 2 * nc, 2 * ni + 2 * nc + nl};
    d.order = p->d_stress + off[which];
    d.seed = p->stress_seed;
    return d;
}

// Launch counts of a kernel family and their group sizes (the fused kernels
// infer their epoch from them).
uint32_t *launch_groups(halo_plan *p, int family)
{
    return p->d_state + halo::launch_groups_offset(p->h.seg.size(), family);
}

const uint32_t *launch_members(halo_plan *p, int family)
{
    return p->d_members + (size_t)family * halo::kLaunchGroups;
}

// The epoch argument of a fused launch: the host's count for eager calls; 0
// (inferred on the device) for calls being captured and for every call after
// the first capture, since replays then advance the counts unseen. The count
// moves only when the launch is enqueued (epoch_launched).
uint32_t launch_epoch_arg(halo_plan *p, int family, hipStream_t s)
{
    bool capturing = false;
    if (!p->epochs.on_device) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        capturing = hipStreamIsCapturing(s, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
    }
    return p->epochs.next(family, capturing);
}

hipError_t epoch_launched(halo_plan *p, int family, hipError_t e)
{
    p->epochs.launched(family, e == hipSuccess);
    return e;
}

hipError_t launch_fused(halo_plan *p, bool force_dir, float *buf, hipStream_t s)
{
    const halo::HostPlan &h = p->h;
    int32_t n_seg = (int32_t)h.seg.size();
    uint32_t n_items = (uint32_t)h.items.size();
    uint32_t bytes = (uint32_t)(h.total_slots * 12);
    uint32_t idx_bytes = (uint32_t)(h.n_entries * 4);
    const Kernels k = kernels(h.item_entries);
    if (force_dir) {
        Debug st = debug_of(p, kOrderItemsF);
        uint32_t *groups = launch_groups(p, halo::kFamItemsF);
        const uint32_t *members = launch_members(p, halo::kFamItemsF);
        uint32_t epoch = launch_epoch_arg(p, halo::kFamItemsF, s);
        void *args[] = {&buf, &bytes, &p->d_idx, &idx_bytes, &p->d_items, &p->d_seg_items,
                        &p->d_state, &n_seg, &n_items, &groups, &members, &epoch,
                        &p->spin_limit, &p->d_err, &p->withhold, &st};
        return epoch_launched(p, halo::kFamItemsF,
                              hipLaunchKernel(k.unpack_fused, dim3(n_items), dim3(kThreads), args,
                                              0, s));
    }
    int32_t n_dom = h.n_dom;
    Debug st = debug_of(p, kOrderItemsX);
    uint32_t *groups = launch_groups(p, halo::kFamItemsX);
    const uint32_t *members = launch_members(p, halo::kFamItemsX);
    uint32_t epoch = launch_epoch_arg(p, halo::kFamItemsX, s);
    void *args[] = {&buf, &bytes, &p->d_idx, &idx_bytes, &p->d_items, &p->d_recv_from,
                    &p->d_seg_items, &p->d_state, &n_dom, &groups, &members, &epoch,
                    &p->spin_limit, &p->d_err, &p->withhold, &st};
    return epoch_launched(p, halo::kFamItemsX,
                          hipLaunchKernel(k.pack_fused, dim3(n_items), dim3(kThreads), args, 0, s));
}

// Transposed-form kernels: counters in the second block of state.
hipError_t launch_chunks(halo_plan *p, bool force_dir, float *buf, hipStream_t s)
{
    const halo::HostPlan &h = p->h;
    int32_t n_dom = h.n_dom, n_pulse = h.n_pulse;
    uint32_t bytes = (uint32_t)(h.total_slots * 12);
    uint32_t *state = p->d_state + 2 * h.seg.size() * halo::kCounterStride;
    const uint32_t n = (uint32_t)h.chunks.size();
    const Kernels k = kernels(h.chunk_slots);
    if (force_dir) {
        uint32_t *groups = launch_groups(p, halo::kFamChunksF);
        const uint32_t *members = launch_members(p, halo::kFamChunksF);
        uint32_t epoch = launch_epoch_arg(p, halo::kFamChunksF, s);
        Debug st = debug_of(p, kOrderChunksF);
        void *args[] = {&buf, &bytes, &p->d_mask, &p->d_chunks, &p->d_forder, &p->d_rows,
                        &p->d_dest_start, &p->d_send_to, &p->d_zone_chunks, &state, &n_dom,
                        &n_pulse, &groups, &members, &epoch, &p->spin_limit, &p->d_err,
                        &p->withhold, &st};
        return epoch_launched(p, halo::kFamChunksF,
                              hipLaunchKernel(k.pull_f, dim3(n), dim3(kThreads), args, 0, s));
    }
    uint32_t *groups = launch_groups(p, halo::kFamChunksX);
    const uint32_t *members = launch_members(p, halo::kFamChunksX);
    uint32_t epoch = launch_epoch_arg(p, halo::kFamChunksX, s);
    Debug st = debug_of(p, kOrderChunksX);
    void *args[] = {&buf, &bytes, &p->d_mask, &p->d_chunks, &p->d_rows, &p->d_dest_start,
                    &p->d_shift4, &p->d_x_arrivals, &state, &n_dom, &n_pulse, &groups,
                    &members, &epoch, &p->spin_limit, &p->d_err, &p->withhold, &st};
    return epoch_launched(p, halo::kFamChunksX,
                          hipLaunchKernel(k.push_x, dim3(n), dim3(kThreads), args, 0, s));
}

hipError_t launch_pulse(halo_plan *p, bool force_dir, float *buf, hipStream_t s, int32_t q)
{
    const halo::HostPlan &h = p->h;
    uint32_t bytes = (uint32_t)(h.total_slots * 12);
    uint32_t idx_bytes = (uint32_t)(h.n_entries * 4);
    int32_t base = h.pulse_item_off[q];
    const uint32_t n = (uint32_t)(h.pulse_item_off[q + 1] - base);
    const Kernels k = kernels(h.item_entries);
    void *args[] = {&buf, &bytes, &p->d_idx, &idx_bytes, &p->d_items, &base};
    return hipLaunchKernel(force_dir ? k.unpack_pulse : k.pack_pulse, dim3(n), dim3(kThreads),
                           args, 0, s);
}

hipError_t launch_atomic(halo_plan *p, float *buf, hipStream_t s)
{
    const halo::HostPlan &h = p->h;
    int32_t n_seg = (int32_t)h.seg.size();
    uint32_t n_items = (uint32_t)h.items.size();
    uint32_t bytes = (uint32_t)(h.total_slots * 12);
    uint32_t idx_bytes = (uint32_t)(h.n_entries * 4);
    const Kernels k = kernels(h.item_entries);
    int32_t n_dom = h.n_dom;
    Debug st = debug_of(p, kOrderItemsF);
    // its own counters and launch counts: which items wait differs from the
    // ordered force kernel
    uint32_t *state = p->d_state + halo::atomic_state_offset(h.seg.size());
    uint32_t *groups = launch_groups(p, halo::kFamAtomicF);
    const uint32_t *members = launch_members(p, halo::kFamAtomicF);
    uint32_t epoch = launch_epoch_arg(p, halo::kFamAtomicF, s);
    void *args[] = {&buf, &bytes, &p->d_idx, &idx_bytes, &p->d_items, &p->d_seg_items,
                    &state, &n_seg, &n_dom, &n_items, &groups, &members, &epoch,
                    &p->spin_limit, &p->d_err, &p->withhold, &st};
    return epoch_launched(p, halo::kFamAtomicF,
                          hipLaunchKernel(k.unpack_atomic, dim3(n_items), dim3(kThreads), args, 0,
                                          s));
}

// XCD-local index-list kernels (plans built on the host): one launch, one
// unit position per workgroup; the flags of the coordinate direction, then
// of the force direction.
hipError_t launch_local(halo_plan *p, bool force_dir, float *buf, hipStream_t s,
                        bool lds4 = false)
{
    const halo::HostPlan &h = p->h;
    uint32_t bytes = (uint32_t)(h.total_slots * 12);
    uint32_t idx_bytes = (uint32_t)(h.n_entries * 4);
    int32_t n_units = (int32_t)h.lunits.size();
    int32_t kp = halo::local_flag_stride(h.local_k);
    const Kernels k = kernels(h.local_entries);
    const int fam = force_dir ? halo::kFamLocalF : halo::kFamLocalX;
    uint32_t *groups = launch_groups(p, fam);
    const uint32_t *members = launch_members(p, fam);
    uint32_t epoch = launch_epoch_arg(p, fam, s);
    Debug dbg = debug_of(p, force_dir ? kOrderLocalF : kOrderLocalX);
    uint64_t *flags = p->d_lflags + (force_dir ? (size_t)kp * halo::kXcdClasses : 0);
    hipError_t e;
    if (force_dir) {
        void *args[] = {&buf,  &bytes,  &p->d_idx, &idx_bytes, &p->d_lunits, &n_units,
                        &p->d_lwaits, &flags, &kp, &groups, &members, &epoch,
                        &p->spin_limit, &p->d_err, &p->withhold, &dbg};
        e = hipLaunchKernel(k.unpack_local, dim3((uint32_t)n_units), dim3(kThreads), args, 0, s);
    } else {
        void *args[] = {&buf,   &bytes, &p->d_idx, &idx_bytes, &p->d_lunits, &p->d_lwaits,
                        &flags, &kp,    &groups,   &members,   &epoch,       &p->spin_limit,
                        &p->d_err, &p->withhold, &dbg};
        e = hipLaunchKernel(lds4 ? k.pack_local_lds4 : k.pack_local, dim3((uint32_t)n_units),
                            dim3(kThreads), args, 0, s);
    }
    return epoch_launched(p, fam, e);
}

// One pulse of the staged baseline: two launches.
hipError_t launch_staged(halo_plan *p, bool force_dir, float *buf, float *stage, hipStream_t s,
                         int32_t q)
{
    const halo::HostPlan &h = p->h;
    uint32_t bytes = (uint32_t)(h.total_slots * 12);
    uint32_t idx_bytes = (uint32_t)(h.n_entries * 4);
    uint32_t stage_bytes = (uint32_t)(h.n_entries * 12);
    int32_t base = h.pulse_item_off[q];
    const uint32_t n = (uint32_t)(h.pulse_item_off[q + 1] - base);
    const Kernels k = kernels(h.item_entries);
    int32_t to_region = force_dir ? 0 : 1;
    void *args_io[] = {&buf, &bytes, &stage, &stage_bytes, &p->d_idx, &idx_bytes, &p->d_items,
                       &base};
    void *args_mv[] = {&buf, &bytes, &stage, &stage_bytes, &p->d_items, &base, &to_region};
    hipError_t e;
    if (!force_dir) {
        e = hipLaunchKernel(k.stage_pack, dim3(n), dim3(kThreads), args_io, 0, s);
        if (e == hipSuccess) e = hipLaunchKernel(k.stage_move, dim3(n), dim3(kThreads), args_mv, 0, s);
    } else {
        e = hipLaunchKernel(k.stage_move, dim3(n), dim3(kThreads), args_mv, 0, s);
        if (e == hipSuccess) e = hipLaunchKernel(k.stage_unpack, dim3(n), dim3(kThreads), args_io, 0, s);
    }
    return e;
}

halo_status ensure_uploaded(halo_plan *p)
{
    if (p->uploaded) return HALO_OK;
    hipError_t e;
    if ((e = hipGetDevice(&p->device)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (p->built_on_device && !p->d_idx)
        return fail(HALO_ERR_STATE, "halo_plan_upload: device-built plan lost its device arrays");
    const halo::HostPlan &h = p->h;
    if ((e = upload_vec(&p->d_idx, h.abs_map)) != hipSuccess ||
        (e = upload_vec(&p->d_items, h.items)) != hipSuccess ||
        (e = upload_vec(&p->d_recv_from, h.recv_from)) != hipSuccess ||
        (e = upload_vec(&p->d_send_to, h.send_to)) != hipSuccess ||
        (e = upload_vec(&p->d_seg_items, h.seg_items)) != hipSuccess ||
        (e = upload_vec(&p->d_members, h.launch_members)) != hipSuccess) {
        free_device(p);
        return hip_fail(e, "halo_plan_upload");
    }
    if (h.has_chunks &&
        ((e = upload_vec(&p->d_mask, h.slot_mask)) != hipSuccess ||
         (e = upload_vec(&p->d_chunks, h.chunks)) != hipSuccess ||
         (e = upload_vec(&p->d_forder, h.chunk_forder)) != hipSuccess ||
         (e = upload_vec(&p->d_dest_start, h.dest_start)) != hipSuccess ||
         (e = upload_vec(&p->d_shift4, h.shift4)) != hipSuccess ||
         (e = upload_vec(&p->d_x_arrivals, h.x_arrivals)) != hipSuccess ||
         (e = upload_vec(&p->d_zone_chunks, h.zone_chunks)) != hipSuccess)) {
        free_device(p);
        return hip_fail(e, "halo_plan_upload");
    }
    if (h.has_chunks && !h.chunks.empty() &&
        (e = halo::plan_chunk_rows(p, p->d_mask, p->d_chunks, nullptr)) != hipSuccess) {
        free_device(p);
        return hip_fail(e, "halo_plan_upload");
    }
    if (h.has_local) {
        p->lflag_words = 2 * (size_t)halo::kXcdClasses * halo::local_flag_stride(h.local_k);
        if ((e = upload_vec(&p->d_lunits, h.lunits)) != hipSuccess ||
            (e = upload_vec(&p->d_lwaits, h.lwaits)) != hipSuccess ||
            (e = hipMalloc((void **)&p->d_lflags, p->lflag_words * 8)) != hipSuccess ||
            (e = hipMemset(p->d_lflags, 0, p->lflag_words * 8)) != hipSuccess) {
            free_device(p);
            return hip_fail(e, "halo_plan_upload");
        }
    }
    // two counter blocks (work items, chunks), each X then F, and the launch
    // counts; 128 B per counter
    p->state_words = halo::state_words_for(h.seg.size());
    if ((e = hipMalloc((void **)&p->d_state, p->state_words * 4)) != hipSuccess ||
        (e = hipMemset(p->d_state, 0, p->state_words * 4)) != hipSuccess ||
        (e = hipHostMalloc((void **)&p->h_err, 64, hipHostMallocMapped)) != hipSuccess ||
        (e = hipHostGetDevicePointer((void **)&p->d_err, p->h_err, 0)) != hipSuccess ||
        (e = hipDeviceSynchronize()) != hipSuccess) {
        free_device(p);
        return hip_fail(e, "halo_plan_upload");
    }
    std::memset(p->h_err, 0, 64);
    p->epochs.reset();
    p->uploaded = true;
    return HALO_OK;
}

}  // namespace

int halo::plan_upload(halo_plan *p) { return ensure_uploaded(p); }

hipError_t halo::plan_chunk_rows(halo_plan *p, const uint8_t *mask, const Chunk *chunks,
                                 hipStream_t s)
{
    const HostPlan &h = p->h;
    const int ept = ept_for(h.chunk_slots);
    const size_t need = h.chunks.size() * 4 * (size_t)h.n_pulse * (size_t)ept;
    if (need == 0) return hipSuccess;
    hipError_t e;
    if (p->rows_cap < need) {
        if (p->d_rows) (void)hipFree(p->d_rows);
        p->d_rows = nullptr;
        p->rows_cap = 0;
        if ((e = hipMalloc((void **)&p->d_rows, need * sizeof(uint16_t))) != hipSuccess) {
            p->d_rows = nullptr;
            return e;
        }
        p->rows_cap = need;
    }
    int32_t n_pulse = h.n_pulse;
    void *args[] = {&mask, &chunks, &n_pulse, &p->d_rows};
    return hipLaunchKernel(kernels(h.chunk_slots).chunk_rows, dim3((uint32_t)h.chunks.size()),
                           dim3(kThreads), args, 0, s);
}

namespace {

// Calls whose first use allocates or synchronises (the upload, staging
// buffers, origin maps) refuse a stream that is being captured, and so do the
// device plan builds, which queue clears and copies and then wait. The check
// comes before anything is queued or freed.
halo_status refuse_capture(hipStream_t stream, const char *what,
                           const char *why = "its first call on a plan allocates and "
                                             "synchronises, so it cannot be captured; call it "
                                             "(or halo_plan_upload) once before capturing")
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
        return fail(HALO_ERR_ARG, std::string(what) + ": " + why);
    return HALO_OK;
}

constexpr const char *kBuildUncapturable =
    "a plan build allocates, queues copies and waits for them, so it cannot be captured";

halo_status check_exchange(halo_plan *p, float *buf, const char *what, void *stream)
{
    if (!p) return fail(HALO_ERR_ARG, std::string(what) + ": NULL plan");
    if (p->invalid)
        return fail(HALO_ERR_STATE, std::string(what) +
                                        ": the plan's last rebuild failed; rebuild it again");
    if (!buf && p->h.total_slots > 0) return fail(HALO_ERR_ARG, std::string(what) + ": NULL buffer");
    if (p->uploaded && p->h_err && __atomic_load_n(p->h_err, __ATOMIC_ACQUIRE) != 0)
        p->poisoned = true;
    if (p->poisoned)
        return fail(HALO_ERR_STATE, std::string(what) +
                                        ": plan poisoned by an in-kernel wait timeout or "
                                        "placement error; call halo_plan_reset");
    halo_status st;
    if (!p->uploaded && (st = refuse_capture((hipStream_t)stream, what)) != HALO_OK) return st;
    st = ensure_uploaded(p);
    if (st != HALO_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != p->device)
        return fail(HALO_ERR_ARG, std::string(what) + ": current device differs from the plan's");
    return HALO_OK;
}

int32_t item_entries_from_env()
{
    const char *v = std::getenv("HALO_ITEM_ENTRIES");
    if (!v) return kDefaultItemEntries;
    long n = std::strtol(v, nullptr, 10);
    if (n < 1) n = 1;
    if (n > 8 * kThreads) n = 8 * kThreads;
    return (int32_t)n;
}

}  // namespace

extern "C" {

const char *halo_last_error(void) { return g_last_error.c_str(); }

halo_status halo_plan_create(const float *positions, int64_t n_atoms, const float *box,
                             const int32_t *grid, float cutoff, halo_plan **out)
{
    return halo_plan_create_ex(positions, n_atoms, box, grid, cutoff, HALO_SELECT_SLAB, out);
}

halo_status halo_plan_create_ex(const float *positions, int64_t n_atoms, const float *box,
                                const int32_t *grid, float cutoff, int32_t selection,
                                halo_plan **out)
{
    if (!out) return fail(HALO_ERR_ARG, "halo_plan_create: NULL output pointer");
    *out = nullptr;
    halo_plan *p = new (std::nothrow) halo_plan();
    if (!p) return fail(HALO_ERR_NOMEM, "halo_plan_create: out of host memory");
    std::string msg;
    int rc;
    try {
        rc = halo::build_plan(positions, n_atoms, box, grid, cutoff, selection,
                              item_entries_from_env(), p->h, msg);
    } catch (const std::bad_alloc &) {
        rc = halo::kErrNoMem;
        msg = "halo_plan_create: out of host memory";
    } catch (const std::exception &ex) {
        rc = halo::kErrArg;
        msg = std::string("halo_plan_create: internal error: ") + ex.what();
    }
    if (rc != halo::kOk) {
        delete p;
        return fail((halo_status)rc, msg);
    }
    *out = p;
    return HALO_OK;
}

halo_status halo_plan_create_device(const float *positions, int64_t n_atoms, const float *box,
                                    const int32_t *grid, float cutoff, void *stream,
                                    halo_plan **out)
{
    return halo_plan_create_device_ex(positions, n_atoms, box, grid, cutoff, HALO_SELECT_SLAB,
                                      stream, out);
}

halo_status halo_plan_create_device_ex(const float *positions, int64_t n_atoms, const float *box,
                                       const int32_t *grid, float cutoff, int32_t selection,
                                       void *stream, halo_plan **out)
{
    if (!out) return fail(HALO_ERR_ARG, "halo_plan_create_device: NULL output pointer");
    *out = nullptr;
    if (halo_status st = refuse_capture((hipStream_t)stream, "halo_plan_create_device",
                                        kBuildUncapturable);
        st != HALO_OK)
        return st;
    halo_plan *p = new (std::nothrow) halo_plan();
    if (!p) return fail(HALO_ERR_NOMEM, "halo_plan_create_device: out of host memory");
    std::string msg;
    int rc;
    g_last_error.clear();
    try {
        rc = halo::build_plan_device(p, positions, n_atoms, box, grid, cutoff, selection,
                                     item_entries_from_env(), (hipStream_t)stream, msg);
    } catch (const std::bad_alloc &) {
        rc = halo::kErrNoMem;
        msg = "halo_plan_create_device: out of host memory";
    } catch (const std::exception &ex) {
        rc = halo::kErrArg;
        msg = std::string("halo_plan_create_device: internal error: ") + ex.what();
    }
    if (rc != halo::kOk) {
        free_device(p);
        delete p;
        // an upload failure has already set the message
        return msg.empty() ? (halo_status)rc : fail((halo_status)rc, msg);
    }
    *out = p;
    return HALO_OK;
}

halo_status halo_plan_rebuild_device(halo_plan *p, const float *positions, int64_t n_atoms,
                                     const float *box, void *stream)
{
    if (!p || !box) return fail(HALO_ERR_ARG, "halo_plan_rebuild_device: NULL argument");
    // before anything is freed or queued: a refused rebuild leaves the plan as it was
    if (halo_status st = refuse_capture((hipStream_t)stream, "halo_plan_rebuild_device",
                                        kBuildUncapturable);
        st != HALO_OK)
        return st;
    const int32_t grid[3] = {p->h.grid[0], p->h.grid[1], p->h.grid[2]};
    const float cutoff = p->h.cutoff;
    const int32_t selection = p->h.selection;
    {
        // argument and geometry errors leave the plan as it was
        halo::HostPlan probe;
        std::string msg;
        if (n_atoms < 0 || (n_atoms > 0 && !positions))
            return fail(HALO_ERR_ARG, "halo_plan_rebuild_device: NULL pointer or negative count");
        const int rc = halo::plan_geometry(n_atoms, box, grid, cutoff, selection, probe, msg);
        if (rc != halo::kOk) return fail((halo_status)rc, msg);
    }
    if (!p->built_on_device) {
        free_device(p);  // the host-built device copy is replaced
    } else {
        // derived arrays sized for the old plan: staging, origin map and the
        // stress orders (the stress mode ends with the plan it was set for)
        if (p->d_stage) (void)hipFree(p->d_stage);
        if (p->d_origin) (void)hipFree(p->d_origin);
        if (p->d_stress) (void)hipFree(p->d_stress);
        if (p->d_stamps) (void)hipFree(p->d_stamps);
        p->d_stage = nullptr;
        p->d_origin = nullptr;
        p->d_stress = nullptr;
        p->stress_seed = 0;
        p->d_stamps = nullptr;
        p->stamp_units = 0;
    }
    p->uploaded = false;
    std::string msg;
    int rc;
    g_last_error.clear();
    try {
        rc = halo::build_plan_device(p, positions, n_atoms, box, grid, cutoff, selection,
                                     item_entries_from_env(), (hipStream_t)stream, msg);
    } catch (const std::bad_alloc &) {
        rc = halo::kErrNoMem;
        msg = "halo_plan_rebuild_device: out of host memory";
    } catch (const std::exception &ex) {
        rc = halo::kErrArg;
        msg = std::string("halo_plan_rebuild_device: internal error: ") + ex.what();
    }
    if (rc != halo::kOk) {
        free_device(p);
        p->h = halo::HostPlan();
        p->h.grid[0] = grid[0];
        p->h.grid[1] = grid[1];
        p->h.grid[2] = grid[2];
        p->h.cutoff = cutoff;
        p->h.selection = selection;
        p->built_on_device = false;
        p->invalid = true;
        return msg.empty() ? (halo_status)rc : fail((halo_status)rc, msg);
    }
    p->invalid = false;
    return HALO_OK;
}

void halo_plan_destroy(halo_plan *plan)
{
    if (!plan) return;
    free_device(plan);
    delete plan;
}

int64_t halo_plan_total_slots(const halo_plan *p) { return p ? p->h.total_slots : -1; }
int32_t halo_plan_num_domains(const halo_plan *p) { return p ? p->h.n_dom : -1; }
int32_t halo_plan_num_pulses(const halo_plan *p) { return p ? p->h.n_pulse : -1; }
int64_t halo_plan_num_entries(const halo_plan *p) { return p ? (int64_t)p->h.n_entries : -1; }
int32_t halo_plan_num_items(const halo_plan *p) { return p ? (int32_t)p->h.items.size() : -1; }
int32_t halo_plan_selection(const halo_plan *p) { return p ? p->h.selection : -1; }

halo_status halo_plan_pulse_dim(const halo_plan *p, int32_t pulse, int32_t *dim, int32_t *k)
{
    if (!p || pulse < 0 || pulse >= p->h.n_pulse)
        return fail(HALO_ERR_ARG, "halo_plan_pulse_dim: no such pulse");
    if (dim) *dim = p->h.pulse_dim[pulse];
    if (k) *k = p->h.pulse_k[pulse];
    return HALO_OK;
}

halo_status halo_plan_domain(const halo_plan *p, int32_t d, int64_t *base, int32_t *n_home,
                             int32_t *n_halo)
{
    if (!p || d < 0 || d >= p->h.n_dom) return fail(HALO_ERR_ARG, "halo_plan_domain: no such domain");
    if (base) *base = p->h.base[d];
    if (n_home) *n_home = p->h.n_home[d];
    if (n_halo) *n_halo = p->h.n_halo[d];
    return HALO_OK;
}

// Host copies of a device-built plan's indexMap and home slots, fetched on
// first use (a blocking copy).
static halo_status ensure_host_maps(const halo_plan *cp)
{
    halo_plan *p = const_cast<halo_plan *>(cp);
    halo::HostPlan &h = p->h;
    if (!p->built_on_device) return HALO_OK;
    hipError_t e;
    if ((int64_t)h.local_map.size() != h.n_entries) {
        std::vector<int32_t> m((size_t)h.n_entries);
        if (h.n_entries > 0 &&
            (e = hipMemcpy(m.data(), p->d_local_map, m.size() * 4, hipMemcpyDeviceToHost)) !=
                hipSuccess)
            return hip_fail(e, "fetching the indexMap");
        h.local_map.swap(m);
    }
    if ((int64_t)h.home_slot.size() != h.n_atoms) {
        std::vector<int64_t> hs((size_t)h.n_atoms);
        if (h.n_atoms > 0 &&
            (e = hipMemcpy(hs.data(), p->d_home_slot, hs.size() * 8, hipMemcpyDeviceToHost)) !=
                hipSuccess)
            return hip_fail(e, "fetching the home slots");
        h.home_slot.swap(hs);
    }
    return HALO_OK;
}

halo_status halo_plan_home_slots(const halo_plan *p, int64_t *slot_of_atom)
{
    if (!p || (!slot_of_atom && p->h.n_atoms > 0))
        return fail(HALO_ERR_ARG, "halo_plan_home_slots: NULL argument");
    if (halo_status st = ensure_host_maps(p); st != HALO_OK) return st;
    if (p->h.n_atoms > 0)
        std::memcpy(slot_of_atom, p->h.home_slot.data(), (size_t)p->h.n_atoms * sizeof(int64_t));
    return HALO_OK;
}

halo_status halo_plan_pulse(const halo_plan *p, int32_t pulse, int32_t d, int32_t *send_to,
                            int32_t *send_size, int32_t *recv_from, int32_t *recv_size,
                            int32_t *atom_offset, int32_t *dep_start, int32_t *items, float *shift,
                            int32_t *index_map)
{
    if (!p || pulse < 0 || pulse >= p->h.n_pulse || d < 0 || d >= p->h.n_dom)
        return fail(HALO_ERR_ARG, "halo_plan_pulse: no such pulse or domain");
    const halo::Segment &s = p->h.at(pulse, d);
    if (send_to) *send_to = s.send_to;
    if (send_size) *send_size = s.send_size;
    if (recv_from) *recv_from = s.recv_from;
    if (recv_size) *recv_size = s.recv_size;
    if (atom_offset) *atom_offset = s.atom_offset;
    if (dep_start) *dep_start = s.dep_start;
    if (items) *items = s.n_items;
    if (shift)
        for (int c = 0; c < 3; ++c) shift[c] = s.shift[c];
    if (index_map && s.send_size > 0) {
        if (halo_status st = ensure_host_maps(p); st != HALO_OK) return st;
        std::memcpy(index_map, p->h.local_map.data() + s.map_off, (size_t)s.send_size * 4);
    }
    return HALO_OK;
}

halo_status halo_plan_item_waits(const halo_plan *p, int32_t item, int32_t *segment,
                                 uint32_t *xwait_mask, uint32_t *await_mask)
{
    if (!p || item < 0 || item >= (int32_t)p->h.items.size())
        return fail(HALO_ERR_ARG, "halo_plan_item_waits: no such work item");
    halo::WorkItem it = p->h.items[item];
    if (p->built_on_device) {
        // the wait masks were computed on the device
        hipError_t e = hipMemcpy(&it, p->d_items + item, sizeof(it), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "halo_plan_item_waits");
    }
    if (segment) *segment = it.seg;
    if (xwait_mask) *xwait_mask = it.xwait_mask;
    if (await_mask) *await_mask = it.await_mask;
    return HALO_OK;
}

int32_t halo_plan_num_chunks(const halo_plan *p) { return p ? (int32_t)p->h.chunks.size() : -1; }

int32_t halo_plan_num_local_units(const halo_plan *p)
{
    return p ? (int32_t)p->h.lunits.size() : -1;
}

halo_status halo_plan_local_unit(const halo_plan *p, int32_t position, int32_t *segment,
                                 int32_t *origin, int32_t *entries, int32_t *x_waits,
                                 int32_t *f_waits)
{
    if (!p || position < 0 || position >= (int32_t)p->h.lunits.size())
        return fail(HALO_ERR_ARG, "halo_plan_local_unit: no such unit position");
    const halo::LocalUnit &u = p->h.lunits[(size_t)position];
    if (segment) *segment = u.n_total > 0 ? u.seg : -1;
    if (origin) *origin = u.n_total > 0 ? u.origin : -1;
    if (entries) *entries = u.n_total;
    if (x_waits) *x_waits = u.wx_n;
    if (f_waits) *f_waits = u.wf_n;
    return HALO_OK;
}

halo_status halo_plan_chunk(const halo_plan *p, int32_t chunk, int32_t *domain, int32_t *zone,
                            int64_t *first, int32_t *count, uint32_t *mask)
{
    if (!p || chunk < 0 || chunk >= (int32_t)p->h.chunks.size())
        return fail(HALO_ERR_ARG, "halo_plan_chunk: no such chunk");
    const halo::Chunk &c = p->h.chunks[chunk];
    if (domain) *domain = c.domain;
    if (zone) *zone = c.zone;
    if (first) *first = c.first;
    if (count) *count = c.count;
    if (mask) *mask = c.mask;
    return HALO_OK;
}

halo_status halo_plan_upload(halo_plan *p)
{
    if (!p) return fail(HALO_ERR_ARG, "halo_plan_upload: NULL plan");
    return ensure_uploaded(p);
}

// The fused defaults take, per direction, the form that measured fastest.
// Both directions: the transposed kernel from 2^20 entries up (the 8x8x8
// box; forces only for plans of at most 3 pulses), the index-list kernel on
// XCD-local units below, where the exchanges are latency-bound and the units
// keep each forwarding stage in one XCD's L2, and for more pulses, each of
// which adds a dependent stage to the transposed kernel's work units.
constexpr int64_t kTransposedCoordMinEntries = 1 << 20;
constexpr int64_t kTransposedForceMinEntries = 1 << 20;
constexpr int32_t kTransposedForceMaxPulses = 3;

halo_status halo_exchange_x(halo_plan *p, float *x, void *stream)
{
    if (p && (!p->h.has_chunks || (int64_t)p->h.n_entries < kTransposedCoordMinEntries))
        return halo_exchange_x_indexmap(p, x, stream);
    return halo_exchange_x_transposed(p, x, stream);
}

halo_status halo_exchange_f(halo_plan *p, float *f, void *stream)
{
    if (p && (!p->h.has_chunks || (int64_t)p->h.n_entries < kTransposedForceMinEntries ||
              p->h.n_pulse > kTransposedForceMaxPulses))
        return halo_exchange_f_indexmap(p, f, stream);
    return halo_exchange_f_transposed(p, f, stream);
}

halo_status halo_exchange_x_transposed(halo_plan *p, float *x, void *stream)
{
    halo_status st = check_exchange(p, x, "halo_exchange_x_transposed", stream);
    if (st != HALO_OK) return st;
    if (p->h.items.empty() || p->h.total_slots == 0) return HALO_OK;
    if (!p->h.has_chunks)
        return fail(HALO_ERR_ARG, "halo_exchange_x_transposed: plan has more than 8 pulses");
    if (p->h.chunks.empty()) return HALO_OK;
    hipError_t e = launch_chunks(p, false, x, (hipStream_t)stream);
    return e == hipSuccess ? HALO_OK : hip_fail(e, "halo_exchange_x_transposed launch");
}

halo_status halo_exchange_f_transposed(halo_plan *p, float *f, void *stream)
{
    halo_status st = check_exchange(p, f, "halo_exchange_f_transposed", stream);
    if (st != HALO_OK) return st;
    if (p->h.items.empty() || p->h.total_slots == 0) return HALO_OK;
    if (!p->h.has_chunks)
        return fail(HALO_ERR_ARG, "halo_exchange_f_transposed: plan has more than 8 pulses");
    if (p->h.chunks.empty()) return HALO_OK;
    hipError_t e = launch_chunks(p, true, f, (hipStream_t)stream);
    return e == hipSuccess ? HALO_OK : hip_fail(e, "halo_exchange_f_transposed launch");
}

halo_status halo_exchange_x_indexmap(halo_plan *p, float *x, void *stream)
{
    halo_status st = check_exchange(p, x, "halo_exchange_x_indexmap", stream);
    if (st != HALO_OK) return st;
    if (p->h.items.empty() || p->h.total_slots == 0) return HALO_OK;
    hipError_t e = p->h.has_local ? launch_local(p, false, x, (hipStream_t)stream)
                                  : launch_fused(p, false, x, (hipStream_t)stream);
    return e == hipSuccess ? HALO_OK : hip_fail(e, "halo_exchange_x_indexmap launch");
}

halo_status halo_exchange_x_items(halo_plan *p, float *x, void *stream)
{
    halo_status st = check_exchange(p, x, "halo_exchange_x_items", stream);
    if (st != HALO_OK) return st;
    if (p->h.items.empty() || p->h.total_slots == 0) return HALO_OK;
    hipError_t e = launch_fused(p, false, x, (hipStream_t)stream);
    return e == hipSuccess ? HALO_OK : hip_fail(e, "halo_exchange_x_items launch");
}

halo_status halo_exchange_f_items(halo_plan *p, float *f, void *stream)
{
    halo_status st = check_exchange(p, f, "halo_exchange_f_items", stream);
    if (st != HALO_OK) return st;
    if (p->h.items.empty() || p->h.total_slots == 0) return HALO_OK;
    hipError_t e = launch_fused(p, true, f, (hipStream_t)stream);
    return e == hipSuccess ? HALO_OK : hip_fail(e, "halo_exchange_f_items launch");
}

halo_status halo_exchange_x_indexmap_lds(halo_plan *p, float *x, void *stream)
{
    const char *what = "halo_exchange_x_indexmap_lds";
    halo_status st = check_exchange(p, x, what, stream);
    if (st != HALO_OK) return st;
    if (p->h.items.empty() || p->h.total_slots == 0) return HALO_OK;
    if (!p->h.has_local)
        return fail(HALO_ERR_ARG, std::string(what) + ": the plan has no XCD-local units");
    hipError_t e = launch_local(p, false, x, (hipStream_t)stream, true);
    return e == hipSuccess ? HALO_OK : hip_fail(e, what);
}

halo_status halo_exchange_f_indexmap(halo_plan *p, float *f, void *stream)
{
    halo_status st = check_exchange(p, f, "halo_exchange_f_indexmap", stream);
    if (st != HALO_OK) return st;
    if (p->h.items.empty() || p->h.total_slots == 0) return HALO_OK;
    hipError_t e = p->h.has_local ? launch_local(p, true, f, (hipStream_t)stream)
                                  : launch_fused(p, true, f, (hipStream_t)stream);
    return e == hipSuccess ? HALO_OK : hip_fail(e, "halo_exchange_f_indexmap launch");
}

halo_status halo_exchange_x_pulsewise(halo_plan *p, float *x, void *stream)
{
    halo_status st = check_exchange(p, x, "halo_exchange_x_pulsewise", stream);
    if (st != HALO_OK) return st;
    const halo::HostPlan &h = p->h;
    if (h.total_slots == 0) return HALO_OK;
    for (int32_t q = 0; q < h.n_pulse; ++q) {
        hipError_t e = launch_pulse(p, false, x, (hipStream_t)stream, q);
        if (e != hipSuccess) return hip_fail(e, "halo_exchange_x_pulsewise launch");
    }
    return HALO_OK;
}

halo_status halo_exchange_f_pulsewise(halo_plan *p, float *f, void *stream)
{
    halo_status st = check_exchange(p, f, "halo_exchange_f_pulsewise", stream);
    if (st != HALO_OK) return st;
    const halo::HostPlan &h = p->h;
    if (h.total_slots == 0) return HALO_OK;
    for (int32_t q = h.n_pulse - 1; q >= 0; --q) {
        hipError_t e = launch_pulse(p, true, f, (hipStream_t)stream, q);
        if (e != hipSuccess) return hip_fail(e, "halo_exchange_f_pulsewise launch");
    }
    return HALO_OK;
}

halo_status halo_exchange_f_atomic(halo_plan *p, float *f, void *stream)
{
    halo_status st = check_exchange(p, f, "halo_exchange_f_atomic", stream);
    if (st != HALO_OK) return st;
    if (p->h.items.empty() || p->h.total_slots == 0) return HALO_OK;
    hipError_t e = launch_atomic(p, f, (hipStream_t)stream);
    return e == hipSuccess ? HALO_OK : hip_fail(e, "halo_exchange_f_atomic launch");
}

static halo_status exchange_staged(halo_plan *p, bool force_dir, float *buf, void *stream,
                                   const char *what)
{
    halo_status st = check_exchange(p, buf, what, stream);
    if (st != HALO_OK) return st;
    const halo::HostPlan &h = p->h;
    if (h.total_slots == 0 || h.n_entries == 0) return HALO_OK;
    if (!p->d_stage) {
        if ((st = refuse_capture((hipStream_t)stream, what)) != HALO_OK) return st;
        hipError_t e = hipMalloc((void **)&p->d_stage, h.n_entries * 12);
        if (e != hipSuccess) {
            p->d_stage = nullptr;
            return hip_fail(e, what);
        }
    }
    for (int32_t i = 0; i < h.n_pulse; ++i) {
        const int32_t q = force_dir ? h.n_pulse - 1 - i : i;
        hipError_t e = launch_staged(p, force_dir, buf, p->d_stage, (hipStream_t)stream, q);
        if (e != hipSuccess) return hip_fail(e, what);
    }
    return HALO_OK;
}

static_assert(halo::kMaxSlots <= (int64_t)kOriginSlot, "origin slots need 28 bits");

halo_status halo_exchange_x_direct(halo_plan *p, float *x, void *stream)
{
    const char *what = "halo_exchange_x_direct";
    halo_status st = check_exchange(p, x, what, stream);
    if (st != HALO_OK) return st;
    const halo::HostPlan &h = p->h;
    if (h.total_slots == 0 || h.n_entries == 0) return HALO_OK;
    const hipStream_t s = (hipStream_t)stream;
    const Kernels k = kernels(h.item_entries);
    hipError_t e;
    if (!p->d_origin) {
        // first call: derive the origin map from the indexMaps, pulse by pulse
        if ((st = refuse_capture(s, what)) != HALO_OK) return st;
        uint32_t *slot_origin = nullptr;
        if ((e = hipMalloc((void **)&p->d_origin, h.n_entries * 4)) != hipSuccess) {
            p->d_origin = nullptr;
            return hip_fail(e, what);
        }
        if ((e = hipMalloc((void **)&slot_origin, h.total_slots * 4)) != hipSuccess) {
            (void)hipFree(p->d_origin);
            p->d_origin = nullptr;
            return hip_fail(e, what);
        }
        int32_t n_slots = (int32_t)h.total_slots;
        void *a0[] = {&slot_origin, &n_slots};
        e = hipLaunchKernel((const void *)&k_origin_init,
                            dim3((uint32_t)((h.total_slots + kThreads - 1) / kThreads)),
                            dim3(kThreads), a0, 0, s);
        for (int32_t q = 0; q < h.n_pulse && e == hipSuccess; ++q) {
            int32_t base = h.pulse_item_off[q];
            const uint32_t n = (uint32_t)(h.pulse_item_off[q + 1] - base);
            if (n == 0) continue;
            void *a1[] = {&p->d_idx, &p->d_items, &base, &slot_origin, &p->d_origin};
            e = hipLaunchKernel(k.origin_pulse, dim3(n), dim3(kThreads), a1, 0, s);
        }
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        (void)hipFree(slot_origin);
        if (e != hipSuccess) {
            (void)hipFree(p->d_origin);
            p->d_origin = nullptr;
            return hip_fail(e, what);
        }
    }
    uint32_t bytes = (uint32_t)(h.total_slots * 12);
    uint32_t obytes = (uint32_t)(h.n_entries * 4);
    float lx = h.box[0], ly = h.box[1], lz = h.box[2];
    Debug dbg{nullptr, 0u, p->d_stamps};
    void *args[] = {&x, &bytes, &p->d_origin, &obytes, &p->d_items, &lx, &ly, &lz, &dbg};
    e = hipLaunchKernel(k.gather_x, dim3((uint32_t)h.items.size()), dim3(kThreads), args, 0, s);
    return e == hipSuccess ? HALO_OK : hip_fail(e, what);
}

// Device copy of the home slots (built on the device already for device-built
// plans; uploaded on the first call for host-built ones).
static halo_status ensure_home_slots(halo_plan *p, hipStream_t s, const char *what)
{
    if (p->d_home_slot || p->h.n_atoms == 0) return HALO_OK;
    halo_status st = refuse_capture(s, what);
    if (st != HALO_OK) return st;
    if ((st = ensure_host_maps(p)) != HALO_OK) return st;
    hipError_t e = hipMalloc((void **)&p->d_home_slot, (size_t)p->h.n_atoms * 8);
    if (e == hipSuccess)
        e = hipMemcpy(p->d_home_slot, p->h.home_slot.data(), (size_t)p->h.n_atoms * 8,
                      hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        if (p->d_home_slot) (void)hipFree(p->d_home_slot);
        p->d_home_slot = nullptr;
        return hip_fail(e, what);
    }
    return HALO_OK;
}

static halo_status home_copy(halo_plan *p, const float *src, float *dst, void *stream,
                             bool scatter, const char *what)
{
    halo_status st = check_exchange(p, scatter ? dst : const_cast<float *>(src), what, stream);
    if (st != HALO_OK) return st;
    const int64_t n = p->h.n_atoms;
    if (n == 0) return HALO_OK;
    if (!src || !dst) return fail(HALO_ERR_ARG, std::string(what) + ": NULL buffer");
    const hipStream_t s = (hipStream_t)stream;
    if ((st = ensure_home_slots(p, s, what)) != HALO_OK) return st;
    uint32_t slot_bytes = (uint32_t)(p->h.total_slots * 12);
    uint32_t value_bytes = (uint32_t)(n * 12);
    const void *kernel = scatter ? (const void *)&k_scatter_home : (const void *)&k_gather_home;
    uint32_t b0 = scatter ? value_bytes : slot_bytes, b1 = scatter ? slot_bytes : value_bytes;
    void *args[] = {&src, &b0, &dst, &b1, &p->d_home_slot, (void *)&n};
    hipError_t e = hipLaunchKernel(kernel, dim3((uint32_t)((n + kThreads - 1) / kThreads)),
                                   dim3(kThreads), args, 0, s);
    return e == hipSuccess ? HALO_OK : hip_fail(e, what);
}

halo_status halo_scatter_home(halo_plan *p, const float *values, float *slots, void *stream)
{
    return home_copy(p, values, slots, stream, true, "halo_scatter_home");
}

halo_status halo_gather_home(halo_plan *p, const float *slots, float *values, void *stream)
{
    return home_copy(p, slots, values, stream, false, "halo_gather_home");
}

halo_status halo_exchange_x_staged(halo_plan *p, float *x, void *stream)
{
    return exchange_staged(p, false, x, stream, "halo_exchange_x_staged");
}

}  // extern "C"

// ---- the staged coordinate exchange without allocation ---------------------
// For callers that cannot allocate (graph capture, tight loops, harnesses
// that forbid it): the staging area is a static device array, one per GPU
// the library runs on, held until the process ends. Its device address is
// looked up once per device (with that device current) and used from then
// on; the array's name itself is a host-side stand-in.
constexpr size_t kScratchBytes = (size_t)32 << 20;  // 12 bytes per indexMap entry
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
float *g_scratch_ptr[kMaxScratchDevices] = {};

halo_status scratch_of_device(int dev, float **out, const char *what)
{
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(HALO_ERR_ARG, std::string(what) + ": device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return hip_fail(e, what);
        g_scratch_ptr[dev] = static_cast<float *>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return HALO_OK;
}

}  // namespace

extern "C" {

halo_status halo_exchange_x_staged_noalloc(halo_plan *p, float *x, void *stream)
{
    const char *what = "halo_exchange_x_staged_noalloc";
    if (!p) return fail(HALO_ERR_ARG, std::string(what) + ": NULL plan");
    if (!p->uploaded && !p->invalid)
        return fail(HALO_ERR_STATE, std::string(what) +
                                        ": the plan is not on the device yet; call "
                                        "halo_plan_upload (or any exchange) first");
    halo_status st = check_exchange(p, x, what, stream);  // uploaded: allocates nothing
    if (st != HALO_OK) return st;
    const halo::HostPlan &h = p->h;
    if (h.total_slots == 0 || h.n_entries == 0) return HALO_OK;
    if ((size_t)h.n_entries * 12 > kScratchBytes)
        return fail(HALO_ERR_ARG, std::string(what) + ": the plan has " +
                                      std::to_string((long long)h.n_entries) +
                                      " indexMap entries; the static staging area holds " +
                                      std::to_string((long long)(kScratchBytes / 12)));
    float *stage = nullptr;
    if ((st = scratch_of_device(p->device, &stage, what)) != HALO_OK) return st;
    for (int32_t q = 0; q < h.n_pulse; ++q) {
        const hipError_t e = launch_staged(p, false, x, stage, (hipStream_t)stream, q);
        if (e != hipSuccess) return hip_fail(e, what);
    }
    return HALO_OK;
}

halo_status halo_exchange_f_staged(halo_plan *p, float *f, void *stream)
{
    return exchange_staged(p, true, f, stream, "halo_exchange_f_staged");
}

halo_status halo_plan_sync(halo_plan *p, void *stream)
{
    if (!p) return fail(HALO_ERR_ARG, "halo_plan_sync: NULL plan");
    if (!p->uploaded) return HALO_OK;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "halo_plan_sync");
    const uint32_t word = __atomic_load_n(p->h_err, __ATOMIC_ACQUIRE);
    if (word == halo::kErrWordPlacement) {
        p->poisoned = true;
        return fail(HALO_ERR_PLACEMENT,
                    "halo_plan_sync: a work unit ran on another XCD than the units it waits "
                    "for (the grid's workgroups did not go to the XCDs round-robin); the "
                    "results of that exchange are not valid");
    }
    if (word != 0) {
        p->poisoned = true;
        return fail(HALO_ERR_TIMEOUT, "halo_plan_sync: an in-kernel dependency wait timed out");
    }
    return HALO_OK;
}

halo_status halo_plan_reset(halo_plan *p)
{
    if (!p) return fail(HALO_ERR_ARG, "halo_plan_reset: NULL plan");
    if (!p->uploaded) {
        p->poisoned = false;
        return HALO_OK;
    }
    hipError_t e;
    if ((e = hipDeviceSynchronize()) != hipSuccess ||
        (e = hipMemset(p->d_state, 0, p->state_words * 4)) != hipSuccess ||
        (p->d_lflags && (e = hipMemset(p->d_lflags, 0, p->lflag_words * 8)) != hipSuccess) ||
        (e = hipDeviceSynchronize()) != hipSuccess)
        return hip_fail(e, "halo_plan_reset");
    std::memset(p->h_err, 0, 64);
    p->epochs.reset();
    p->poisoned = false;
    return HALO_OK;
}

halo_status halo_plan_set_spin_limit(halo_plan *p, uint32_t polls)
{
    if (!p || polls == 0) return fail(HALO_ERR_ARG, "halo_plan_set_spin_limit: bad argument");
    p->spin_limit = polls;
    return HALO_OK;
}

halo_status halo_plan_debug_stress(halo_plan *p, uint32_t seed)
{
    if (!p) return fail(HALO_ERR_ARG, "halo_plan_debug_stress: NULL plan");
    if (p->invalid) return fail(HALO_ERR_STATE, "halo_plan_debug_stress: invalid plan");
    halo_status st = ensure_uploaded(p);
    if (st != HALO_OK) return st;
    if (p->d_stress) {
        hipError_t e = hipDeviceSynchronize();  // no launch still reads the old orders
        if (e != hipSuccess) return hip_fail(e, "halo_plan_debug_stress");
        (void)hipFree(p->d_stress);
        p->d_stress = nullptr;
    }
    p->stress_seed = 0;
    if (seed == 0) return HALO_OK;
    const halo::HostPlan &h = p->h;
    const int32_t ni = (int32_t)h.items.size(), nc = (int32_t)h.chunks.size();
    const int32_t nl = (int32_t)h.lunits.size();
    // Work units that never wait on each other, in launch order: the items of
    // one pulse; the chunks of one zone; the XCD-local units of one class and
    // one pulse (reversed among the positions of their class, so that every
    // unit stays on its XCD). Each such group runs reversed.
    std::vector<int32_t> order((size_t)2 * ni + 2 * nc + 2 * nl);
    auto reverse_groups = [](int32_t *dst, const std::vector<int32_t> &seq,
                             const std::vector<int32_t> &key) {
        const int32_t n = (int32_t)seq.size();
        for (int32_t lo = 0; lo < n;) {
            int32_t hi = lo;
            while (hi < n && key[hi] == key[lo]) ++hi;
            for (int32_t i = lo; i < hi; ++i) dst[i] = seq[lo + hi - 1 - i];
            lo = hi;
        }
    };
    std::vector<int32_t> seq(ni), key(ni);
    for (int32_t i = 0; i < ni; ++i) {
        seq[i] = i;
        key[i] = h.items[i].seg / h.n_dom;  // pulse
    }
    reverse_groups(order.data(), seq, key);
    for (int32_t b = 0; b < ni; ++b) {  // force direction: last pulse first
        seq[b] = ni - 1 - b;
        key[b] = h.items[ni - 1 - b].seg / h.n_dom;
    }
    reverse_groups(order.data() + ni, seq, key);
    seq.resize(nc);
    key.resize(nc);
    for (int32_t i = 0; i < nc; ++i) {
        seq[i] = i;
        key[i] = h.chunks[i].zone;
    }
    reverse_groups(order.data() + 2 * ni, seq, key);
    for (int32_t b = 0; b < nc; ++b) {
        seq[b] = h.chunk_forder[b];
        key[b] = h.chunks[h.chunk_forder[b]].zone;
    }
    reverse_groups(order.data() + 2 * ni + nc, seq, key);
    if (nl > 0) {
        // class c holds positions c, c + 8, ...; its units in launch order
        int32_t *ox = order.data() + 2 * ni + 2 * nc, *of = ox + nl;
        for (int32_t b = 0; b < nl; ++b) {
            ox[b] = b;
            of[b] = nl - 1 - b;
        }
        const int32_t K = h.local_k;
        for (int c = 0; c < halo::kXcdClasses; ++c) {
            int32_t lo = 0;
            while (lo < K) {
                const halo::LocalUnit &u0 = h.lunits[(size_t)lo * halo::kXcdClasses + c];
                if (u0.n_total == 0) break;  // the class's empty tail
                const int32_t pulse = u0.seg / h.n_dom;
                int32_t hi = lo;
                while (hi < K) {
                    const halo::LocalUnit &u = h.lunits[(size_t)hi * halo::kXcdClasses + c];
                    if (u.n_total == 0 || u.seg / h.n_dom != pulse) break;
                    ++hi;
                }
                for (int32_t k = lo; k < hi; ++k) {
                    const int32_t pos = k * halo::kXcdClasses + c;
                    const int32_t partner = (lo + hi - 1 - k) * halo::kXcdClasses + c;
                    ox[pos] = partner;
                    of[nl - 1 - pos] = partner;
                }
                lo = hi;
            }
        }
    }
    hipError_t e = hipMalloc((void **)&p->d_stress, std::max<size_t>(order.size(), 1) * 4);
    if (e == hipSuccess && !order.empty())
        e = hipMemcpy(p->d_stress, order.data(), order.size() * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        if (p->d_stress) (void)hipFree(p->d_stress);
        p->d_stress = nullptr;
        return hip_fail(e, "halo_plan_debug_stress");
    }
    p->stress_seed = seed;
    return HALO_OK;
}

halo_status halo_plan_debug_timing(halo_plan *p, int32_t enable)
{
    if (!p) return fail(HALO_ERR_ARG, "halo_plan_debug_timing: NULL plan");
    if (p->invalid) return fail(HALO_ERR_STATE, "halo_plan_debug_timing: invalid plan");
    halo_status st = ensure_uploaded(p);
    if (st != HALO_OK) return st;
    if (p->d_stamps) {
        hipError_t e = hipDeviceSynchronize();  // no launch still writes the old buffer
        if (e != hipSuccess) return hip_fail(e, "halo_plan_debug_timing");
        (void)hipFree(p->d_stamps);
        p->d_stamps = nullptr;
        p->stamp_units = 0;
    }
    if (!enable) return HALO_OK;
    const size_t units =
        std::max<size_t>({p->h.items.size(), p->h.chunks.size(), p->h.lunits.size(), 1});
    const size_t bytes = units * kStampWords * sizeof(uint64_t);
    hipError_t e = hipMalloc((void **)&p->d_stamps, bytes);
    if (e == hipSuccess) e = hipMemset(p->d_stamps, 0, bytes);
    if (e != hipSuccess) {
        if (p->d_stamps) (void)hipFree(p->d_stamps);
        p->d_stamps = nullptr;
        return hip_fail(e, "halo_plan_debug_timing");
    }
    p->stamp_units = units;
    return HALO_OK;
}

halo_status halo_plan_debug_timing_read(halo_plan *p, uint64_t *stamps, int64_t max_units,
                                        int64_t *units, int32_t *clock_khz)
{
    if (!p || !p->d_stamps)
        return fail(HALO_ERR_ARG, "halo_plan_debug_timing_read: timing is not enabled");
    const int64_t n = (int64_t)p->stamp_units;
    if (units) *units = n;
    if (clock_khz) {
        int rate = 0;
        hipError_t e = hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, p->device);
        if (e != hipSuccess) return hip_fail(e, "halo_plan_debug_timing_read");
        *clock_khz = rate;
    }
    if (!stamps) return HALO_OK;
    if (max_units < n)
        return fail(HALO_ERR_ARG, "halo_plan_debug_timing_read: the buffer holds fewer units "
                                  "than the plan's");
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess)
        e = hipMemcpy(stamps, p->d_stamps, (size_t)n * kStampWords * sizeof(uint64_t),
                      hipMemcpyDeviceToHost);
    return e == hipSuccess ? HALO_OK : hip_fail(e, "halo_plan_debug_timing_read");
}

halo_status halo_plan_debug_withhold(halo_plan *p, int32_t segment)
{
    if (!p || segment < -1 || segment >= (int32_t)p->h.seg.size())
        return fail(HALO_ERR_ARG, "halo_plan_debug_withhold: no such segment");
    p->withhold = segment;
    return HALO_OK;
}

}  // extern "C"
