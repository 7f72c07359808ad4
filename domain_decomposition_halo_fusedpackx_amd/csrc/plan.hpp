// plan.hpp -- host-side exchange plan: PulseData per (pulse, domain) and the
// work items the fused kernels run.
//
// "Redesigning GROMACS Halo Exchange" (paper review), Algorithm 1 (PulseData:
// sendSize, recvSize, atomOffset, coordShift, indexMap, blocksForPulse) and
// Algorithm 4 (depOffset split). The plan is rebuilt whenever the atoms are
// redistributed (the pages' domain decomposition / neighbour search step).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace halo {

// Work-item flags: which accesses of the item touch slots that another item
// of the same launch writes or reads, and so must be coherent across XCDs.
enum : int32_t {
    kItemXStoreShared = 1,  // X: the region stored is forwarded by a later pulse
    kItemFLoadShared = 2,   // F: the slots read were updated by a later pulse
    kItemFStoreShared = 4,  // F: the slots written are read by an earlier pulse
};

// One work item = one workgroup of the fused kernels: a contiguous run of the
// indexMap of one (pulse, sending domain) segment. 64 bytes, read with scalar
// loads.
struct alignas(16) WorkItem {
    int32_t map_begin;     // first entry (index into the concatenated indexMap)
    int32_t n_indep;       // leading entries below depOffset: no wait needed
    int32_t n_total;       // entries in this item
    int32_t region_begin;  // receiver-region slot of the first entry (X: store, F: load)
    float shift[3];        // coordShift of the segment
    int32_t seg;           // segment id = pulse * n_domains + sending domain
    uint32_t xwait_mask;   // coordinate direction: bit r = the dependent entries read
                           //   the region the sender received in pulse r
    int32_t domain;        // sending domain
    int32_t fwait[2];      // force direction: (p+1, D) and (p+1, receiver); -1 = none
    int32_t flags;         // kItem* bits
    uint32_t await_mask;   // atomic force direction: bit q = segment (q, receiver) adds
                           //   into the region this item reads
    int32_t receiver;      // receiving domain
    int32_t pad;
};
static_assert(sizeof(WorkItem) == 64, "WorkItem layout");

// Transposed form of the indexMaps: one chunk = a run of consecutive local
// slots of one domain inside one zone (the home slots, or the region received
// in one pulse). For every pulse p the chunk's slots whose mask has bit p are
// exactly the entries rank[p], rank[p]+1, ... of indexMap_p(domain), in order.
constexpr int kMaxMaskPulses = 8;

struct alignas(16) Chunk {
    int32_t first;        // absolute first slot
    int32_t count;        // slots in the chunk
    int32_t domain;
    int32_t zone;         // -1: home slots; r >= 0: region received in pulse r
    uint32_t mask;        // union of the pulse masks of the chunk's slots
    int32_t xwait;        // X: segment (r * n_dom + sender) that fills this region; -1 for home
    int32_t top_sends;    // slots of the chunk sent in the last pulse
    int32_t pad;
    int32_t rank[kMaxMaskPulses];  // entries of indexMap_p(domain) before the chunk
};
static_assert(sizeof(Chunk) == 64, "Chunk layout");

// XCD-local units of the index-list kernels (plans built on the host). The
// entries of every indexMap are cut into runs whose atoms share one home
// domain (their "origin"); a run reads either home slots or a stretch of one
// region written by the runs of the same origin in earlier pulses. Every
// dependency of both exchanges therefore stays among the runs of one origin,
// and the units of an origin all run on one XCD: unit position b (the
// workgroup index of the coordinate kernel) belongs to class b mod
// kXcdClasses, and a grid's workgroups go to the XCDs round-robin. Data that
// one unit writes and another reads then stays in that XCD's L2: written
// with plain stores, read past the CU cache, and signalled by a per-unit flag
// word instead of a device-wide counter.
constexpr int kXcdClasses = 8;

struct alignas(16) LocalUnit {
    int32_t map_begin;     // first entry (index into the concatenated indexMap)
    int32_t n_total;       // entries (0: an empty position)
    int32_t region_begin;  // receiver-region slot of the first entry
    int32_t seg;           // pulse * n_domains + sending domain
    float shift[3];        // coordShift of the segment
    int32_t origin;        // home domain of the run's atoms
    int32_t wx_off, wx_n;  // coordinates: the units (positions) whose stores it reads
    int32_t wf_off, wf_n;  // forces: the units (positions) that must add before it
    int32_t flags;         // kLocal* bits
    int32_t pad[3];
};
static_assert(sizeof(LocalUnit) == 64, "LocalUnit layout");

// Flag words per class of the XCD-local kernels: positions per class rounded
// up to whole 128-byte lines of 8-byte flags.
inline int32_t local_flag_stride(int32_t local_k) { return (local_k + 15) / 16 * 16 + 16; }

enum : int32_t {
    kLocalXWaited = 1,  // coordinates: a later unit reads what this one stores
    kLocalFWaited = 2,  // forces: a unit waits until this one has added
};

struct Segment {
    int32_t send_to = 0;
    int32_t send_size = 0;
    int32_t recv_from = 0;
    int32_t recv_size = 0;
    int32_t atom_offset = 0;  // local slot where this domain's region of the pulse starts
    int32_t dep_start = 0;
    float shift[3] = {0.f, 0.f, 0.f};
    int64_t map_off = 0;      // first entry in the concatenated indexMap
    int32_t item_off = 0;     // first work item (pulse-major item order)
    int32_t n_items = 0;
};

struct HostPlan {
    // inputs
    int64_t n_atoms = 0;
    float box[3] = {0, 0, 0};
    int32_t grid[3] = {1, 1, 1};
    float cutoff = 0;
    int32_t selection = 0;        // kSelectSlab or kSelectCorner
    // geometry
    double width[3] = {0, 0, 0};
    double reach[3] = {0, 0, 0};  // cutoff / width
    int32_t pulses_in[3] = {0, 0, 0};
    int32_t n_dom = 0;
    int32_t n_pulse = 0;
    std::vector<int32_t> pulse_dim, pulse_k;
    // layout
    std::vector<int64_t> base;
    std::vector<int32_t> n_home, n_halo;
    int64_t total_slots = 0;
    std::vector<int64_t> home_slot;        // per atom
    // pulses
    std::vector<Segment> seg;              // [n_pulse * n_dom]
    int64_t n_entries = 0;                 // entries of all indexMaps
    std::vector<int32_t> local_map;        // concatenated indexMap, local slots
    std::vector<int32_t> abs_map;          // same entries as absolute slots
    std::vector<int32_t> send_to;          // [p][D]: receiver of D in pulse p
    std::vector<int32_t> recv_from;        // [p][D]: sender to D in pulse p
    // work items
    int32_t item_entries = 0;
    std::vector<WorkItem> items;
    std::vector<uint32_t> seg_items;       // items per segment
    std::vector<int32_t> pulse_item_off;   // [n_pulse + 1]
    // transposed form (only when n_pulse <= kMaxMaskPulses)
    bool has_chunks = false;
    int32_t chunk_slots = 0;
    std::vector<uint8_t> slot_mask;        // per slot: pulses that send it
    std::vector<Chunk> chunks;             // zone-major: home, region 0, region 1, ...
    std::vector<int32_t> chunk_forder;     // force-direction order: last region first, home last
    std::vector<int32_t> dest_start;       // [p][D]: first slot of the receiver's region of pulse p
    std::vector<float> shift4;             // [p][D][4]: coordShift of (p, D)
    std::vector<uint32_t> x_arrivals;      // [p][D]: chunks of D that send in pulse p
    std::vector<uint32_t> zone_chunks;     // [r][D]: chunks in region zone r of D
    // XCD-local units of the index-list kernels (host-built plans only)
    bool has_local = false;
    int32_t local_k = 0;                   // positions per class
    int32_t local_entries = 0;             // most entries of a unit (sets the kernels' width)
    std::vector<LocalUnit> lunits;         // [kXcdClasses * local_k]; position b: class b % 8
    std::vector<int32_t> lwaits;           // wait lists (positions)
    // launch counts: members of each group of each kernel family
    std::vector<uint32_t> launch_members;  // [family][kLaunchGroups]

    const Segment &at(int32_t p, int32_t d) const { return seg[(size_t)p * n_dom + d]; }
};

// Most pulses of one plan: the work items keep per-pulse wait sets as 32-bit
// masks.
constexpr int32_t kMaxPulses = 32;

// Largest slot count of one plan: byte offsets of float triples stay below
// 2^31, so the kernels address x and f with 32-bit buffer offsets and use
// 0x80000000 as an always-out-of-range offset.
constexpr int64_t kMaxSlots = ((int64_t)1 << 31) / 12 - 1;

// Halo selection tests, shared with halo.h: the slab test alone, or the slab
// test and the atom's Euclidean distance to the receiver's box below the
// cutoff.
enum : int32_t { kSelectSlab = 0, kSelectCorner = 1 };

// Status codes shared with halo.h.
enum : int { kOk = 0, kErrArg = -1, kErrGeometry = -2, kErrRange = -3, kErrHip = -4, kErrNoMem = -7 };

// Launch counts, from which the fused kernels infer the epoch of a launch
// (the number of this family's launches so far, plus one) without a kernel
// argument: the work units of a launch (work items, chunks) fall into
// kLaunchGroups groups by unit index, and per kernel family the units that
// wait on a counter are the members of their group. Each member adds 1 to its
// group's count once per launch.
constexpr int kLaunchGroups = 512;
enum : int {
    kFamItemsX = 0,   // k_pack_fused: items with dependent entries
    kFamItemsF = 1,   // k_unpack_fused: items of every pulse but the last
    kFamChunksX = 2,  // k_push_x: region chunks
    kFamChunksF = 3,  // k_pull_f: chunks that pull a region summed in the launch
    kFamAtomicF = 4,  // k_unpack_atomic: every item
    kFamLocalX = 5,   // k_pack_local: units that wait or are waited for
    kFamLocalF = 6,   // k_unpack_local: the same in the force direction
    kFamilies = 7
};

// Fill plan.launch_members from the items, the XCD-local units and the
// chunks; the two halves may also run apart (the first zeroes the counts),
// once the items and units exist and once the chunks do.
void make_launch_members(HostPlan &plan);
void launch_members_items_units(HostPlan &plan);
void launch_members_chunks(HostPlan &plan);

// Whether make_items places the items of one domain on one XCD.
bool xcd_ordering_enabled();

// Build the XCD-local units (runs of one origin, at most unit_entries
// entries each), their placement and their wait lists.
void make_local_units(HostPlan &plan, int32_t unit_entries);

// One piece of a run of entries of segment (pulse, sender) whose sources lie
// in one zone of the sender and hold atoms of one origin; entries e0 .. e0+n-1
// of the segment. The input of the placement below, from the host build
// (make_local_units) or the device build.
struct LocalRun {
    int32_t pulse, sender, e0, n, zone, origin;
    int32_t src_lo, src_hi;  // absolute slots of the first and last source
};
static_assert(sizeof(LocalRun) == 32, "LocalRun layout");

// Classes, positions, wait lists and flags of the XCD-local units from their
// pieces, given in segment order (pulse-major, then sender, then entry).
void place_local_units(HostPlan &plan, const std::vector<LocalRun> &runs);

// The size bound of the XCD-local units: the largest power of two from 128 to
// 1024 entries (and at most item_entries) at which the plan still has about
// two units per compute unit of the chip (512 units' worth of entries).
int32_t local_unit_entries(int64_t n_entries, int32_t item_entries);

// Build the transposed form (masks and chunks of at most chunk_slots slots).
void make_chunks(HostPlan &plan, int32_t chunk_slots);

// The transposed form exists for plans with 1..kMaxMaskPulses pulses.
bool plan_has_chunks(const HostPlan &plan);

// Chunk candidates: every zone of every domain cut into balanced pieces of
// at most chunk_slots slots, per domain in slot order.
struct Piece {
    int32_t first;   // absolute first slot
    int32_t count;
    int32_t domain;
    int32_t zone;    // -1 home, r >= 0 region of pulse r
};
struct PieceStats {
    uint32_t mask;                   // union of the slots' pulse masks
    int32_t count[kMaxMaskPulses];   // slots with bit q
};
std::vector<Piece> chunk_pieces(const HostPlan &plan, int32_t chunk_slots);

// Chunks, ranks, per-zone counts and the force-direction order from the
// pieces and their statistics (pieces with an empty mask are dropped).
void finish_chunks(HostPlan &plan, int32_t chunk_slots, const std::vector<Piece> &pieces,
                   const std::vector<PieceStats> &stats);

// Geometry of a plan: validates box, grid and cutoff and fills widths,
// reaches, the pulse list and the send/receive tables.
int plan_geometry(int64_t n_atoms, const float *box, const int32_t *grid, float cutoff,
                  int32_t selection, HostPlan &plan, std::string &msg);

// Build the plan; returns a status code and a message on failure.
int build_plan(const float *pos, int64_t n_atoms, const float *box, const int32_t *grid,
               float cutoff, int32_t selection, int32_t item_entries, HostPlan &out,
               std::string &msg);

// Cut every segment into work items of at most item_entries entries and,
// with with_masks, compute their wait masks from the indexMaps (without, the
// masks are left 0 for the caller to fill).
void make_items(HostPlan &plan, int32_t item_entries, bool with_masks = true);

}  // namespace halo
