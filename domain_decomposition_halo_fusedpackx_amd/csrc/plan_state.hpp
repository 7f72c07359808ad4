// plan_state.hpp -- what a halo_plan holds: the host-side plan and its device
// copy (shared by the C-ABI and the device-side plan builder).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "epochs.hpp"
#include "plan.hpp"

namespace halo {

// One device allocation carved into 256-byte aligned arrays.
struct Arena {
    char *base = nullptr;
    size_t cap = 0;
    size_t used = 0;
};

// Device memory of a plan built on the GPU, kept across rebuilds and grown
// only when a rebuild needs more.
struct DeviceBuild {
    Arena work;               // build temporaries
    Arena entries;            // local-slot indexMap and sent atom ids
    size_t entry_cap = 0;     // entries each array of `entries` holds
    Arena maps;               // absolute indexMap, home slots, pulse masks; build
                              // temporaries of the XCD-local units
    Arena pieces;             // chunk candidates and their statistics
    Arena tables;             // work items, segment tables, chunks, XCD-local units
    Arena units_more;         // XCD-local unit pieces, when more than the first copy held
    char *pinned = nullptr;   // host staging for the small copies
    size_t pinned_cap = 0;
    hipEvent_t done = nullptr;        // polled for the build's waits
    hipEvent_t units_back = nullptr;  // the XCD-local units' pieces are on the host
    hipEvent_t stats_back = nullptr;  // the chunk statistics are on the host
};

}  // namespace halo

struct halo_plan {
    halo::HostPlan h;
    int device = -1;
    bool uploaded = false;
    bool poisoned = false;
    bool built_on_device = false;  // host copies of the maps are fetched on first use
    bool invalid = false;          // a rebuild failed: empty until rebuilt
    halo::DeviceBuild *dev = nullptr;  // arenas of a device-built plan
    int32_t *d_idx = nullptr;      // concatenated indexMap, absolute slots
    halo::WorkItem *d_items = nullptr;
    int32_t *d_recv_from = nullptr;
    int32_t *d_send_to = nullptr;
    uint32_t *d_seg_items = nullptr;
    uint32_t *d_state = nullptr;
    size_t state_words = 0;
    uint32_t *h_err = nullptr;  // pinned host word, written by kernels on a timeout
    uint32_t *d_err = nullptr;  // its device address
    // transposed form
    uint8_t *d_mask = nullptr;
    halo::Chunk *d_chunks = nullptr;
    int32_t *d_forder = nullptr;
    uint16_t *d_rows = nullptr;  // per chunk, wave, pulse and row: bit-p slots in earlier rows
    size_t rows_cap = 0;         // entries d_rows holds
    int32_t *d_dest_start = nullptr;
    float *d_shift4 = nullptr;
    uint32_t *d_x_arrivals = nullptr;
    uint32_t *d_zone_chunks = nullptr;
    // staged baseline: one float triple per indexMap entry, allocated on first use
    float *d_stage = nullptr;
    uint32_t *d_origin = nullptr;  // direct form: home slot | wrap bits per entry (lazy)
    uint32_t *d_members = nullptr;  // launch-count group sizes [family][group]
    // epochs of the fused kernel families as the host counts them; passed to
    // eager launches (0 once a fused exchange of the plan has been captured)
    halo::EpochBook<halo::kFamilies> epochs;
    // device-built plans: local-slot indexMap and home slot of every atom
    int32_t *d_local_map = nullptr;
    int64_t *d_home_slot = nullptr;
    uint32_t spin_limit = 1u << 20;
    int32_t withhold = -1;
    // testing: stress mode (seed 0 = off) and its launch orders
    uint32_t stress_seed = 0;
    int32_t *d_stress = nullptr;
    // XCD-local index-list kernels: units, wait lists, and per-unit flags
    // (coordinates, then forces; 8 bytes each, class-major)
    halo::LocalUnit *d_lunits = nullptr;
    int32_t *d_lwaits = nullptr;
    uint64_t *d_lflags = nullptr;
    size_t lflag_words = 0;
    // tuning: per-unit clock stamps of the fused kernels (nullptr = off)
    uint64_t *d_stamps = nullptr;
    size_t stamp_units = 0;
};

namespace halo {

// Allocate and fill whatever device copy of the plan is still missing (arrays
// already on the device are kept), the counters and the error word.
// Returns a halo_status code; the message goes to halo_last_error.
int plan_upload(halo_plan *p);

// (Re)builds the row table of the transposed kernels (d_rows) from the
// plan's device masks and chunks, on stream s; allocates when it must grow.
hipError_t plan_chunk_rows(halo_plan *p, const uint8_t *mask, const Chunk *chunks,
                           hipStream_t s);

// Free the arenas of a device-built plan and clear the pointers into them.
void free_device_build(halo_plan *p);

// Build p->h and its device arrays on the GPU from device-resident positions
// (plan_device.hip), reusing p's arenas from an earlier device build.
// Returns a status code and a message on failure.
int build_plan_device(halo_plan *p, const float *pos, int64_t n_atoms, const float *box,
                      const int32_t *grid, float cutoff, int32_t selection, int32_t item_entries,
                      hipStream_t stream, std::string &msg);

}  // namespace halo
