/*
 * halo.h -- eighth-shell halo exchange over virtual domains on one MI355X.
 *
 * The method is the GPU-resident GROMACS domain-decomposition halo exchange:
 *   "Redesigning GROMACS Halo Exchange: Improving Strong Scaling with
 *    GPU-initiated NVSHMEM" (paper review), s.3 "GROMACS domain decomposition
 *    halo exchange", Algorithms 1-6, s.4 "Core formulas";
 *   "GPU-Initiated Halo Exchange Cuts CPU Bottlenecks in GROMACS", "Fusing
 *    pack, put, and wait into one kernel".
 *
 * A periodic rectangular box is cut into nx*ny*nz domains. Every domain holds
 * its home atoms and, after a coordinate exchange, a halo: the atoms within the
 * cutoff above its upper faces (the eighth shell), delivered by forwarding
 * pulses in z, then y, then x. All domains live in one device buffer, so the
 * pages' remote store into a peer's coordinate array is a store into another
 * domain's region of the same allocation.
 *
 * Conventions fixed by this library where the pages leave them open:
 *  - pulses per dimension: ceil(cutoff / w_d) for a decomposed dimension
 *    (n_d > 1), none otherwise; it may not exceed n_d - 1;
 *  - a domain sends to its lower neighbour (periodic); a send from cell 0 of
 *    the pulse's dimension wraps and adds +L_d (coordShift);
 *  - an atom is sent in pulse (d, k) iff, measured from its original position
 *    in double precision in units of w_d, it lies less than cutoff/w_d above
 *    the receiver's upper face; candidates are all local slots for k = 0 and
 *    the region received in pulse (d, k-1) for k >= 1;
 *  - domain id = cx + nx*(cy + ny*cz); home atoms in ascending atom id; indexMap
 *    ascending; a domain's slots are [home | region of pulse 0 | pulse 1 | ...]
 *    and domains follow one another in id order ("slots" below);
 *  - force exchange: pulses strictly in reverse order, one fp32 add per
 *    component, so results are bitwise deterministic.
 *
 * Coordinates and forces are float32 triples (x, y, z), 12 bytes per slot,
 * packed without padding.
 *
 * Errors: every call returns a halo_status; halo_last_error() gives a message
 * for the calling thread's last failure. Argument and geometry errors return
 * synchronously with no side effect. A wait inside a kernel that exceeds its
 * spin limit sets the plan's device error word; halo_plan_sync() or the next
 * exchange reports HALO_ERR_TIMEOUT, and the plan refuses exchanges until
 * halo_plan_reset().
 */
#ifndef HALO_H
#define HALO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct halo_plan halo_plan; /* opaque; created and freed by the library */

typedef enum {
    HALO_OK = 0,
    HALO_ERR_ARG = -1,      /* NULL pointer, negative count, index out of range   */
    HALO_ERR_GEOMETRY = -2, /* box/grid/cutoff not positive and finite, more
                               pulses in a dimension than n_d - 1, or more than
                               32 pulses in all (the work items keep their
                               per-pulse wait sets as 32-bit masks)              */
    HALO_ERR_RANGE = -3,    /* a position not finite or outside [0, L); more
                               slots than fit a 32-bit index                      */
    HALO_ERR_HIP = -4,      /* a HIP runtime call failed                          */
    HALO_ERR_TIMEOUT = -5,  /* an in-kernel dependency wait exceeded its limit    */
    HALO_ERR_STATE = -6,    /* plan poisoned by an earlier timeout                */
    HALO_ERR_NOMEM = -7,    /* host allocation failed                             */
    HALO_ERR_PLACEMENT = -8 /* a work unit of the XCD-local index-list kernels ran
                               on another XCD than the units it waits for; the
                               exchange's results are not valid (plan poisoned)   */
} halo_status;

/* Build the exchange plan (the pages' PulseData per pulse and domain,
 * Algorithm 1) from the atom positions. Host only: no HIP call is made; device
 * metadata is uploaded by halo_plan_upload() or by the first exchange.
 *   positions : host, n_atoms*3 float32 (x,y,z per atom), each in [0, L_d)
 *   n_atoms   : >= 0 (positions may be NULL when 0)
 *   box       : host, 3 float32, periodic box lengths Lx, Ly, Lz > 0
 *   grid      : host, 3 int32, domains per dimension nx, ny, nz >= 1
 *   cutoff    : > 0, in the units of box
 *   out       : receives the plan; set to NULL on error
 * The caller keeps ownership of every input; the plan copies what it needs.
 * Work units: work items and transposed runs of at most 1024 entries (the
 * environment variable HALO_ITEM_ENTRIES, read at plan creation, sets another
 * bound from 1 to 2048, for tuning); XCD-local units of the largest power of
 * two from 128 to 1024 entries (never above that bound) at which the plan
 * keeps at least 512 units' worth of entries. */
halo_status halo_plan_create(const float *positions, int64_t n_atoms, const float *box,
                             const int32_t *grid, float cutoff, halo_plan **out);

/* Halo selection tests. The pages define the halo as the atoms within the
 * cutoff of a domain ("Redesigning GROMACS Halo Exchange", s.3), without
 * spelling out the per-pulse test; this library offers two readings:
 *   HALO_SELECT_SLAB   : the per-dimension slab test above (the default of
 *                        halo_plan_create); edge and corner zones of the
 *                        eighth shell are full boxes;
 *   HALO_SELECT_CORNER : the slab test and, in addition, the atom's Euclidean
 *                        distance to the receiver's box below the cutoff:
 *                        sum_d (delta_d * w_d)^2 < cutoff^2 in double over
 *                        d = x, y, z in this order, delta_d = 0 where the
 *                        atom's cell equals the receiver's along d (d other
 *                        than the pulse's dimension), else its distance in
 *                        units of w_d above the receiver's upper face as in
 *                        the slab test. It trims the edge and corner zones to
 *                        their rounded shape (about 5% fewer halo slots on an
 *                        8x8x8 grid at cutoff/w = 0.66). Distances only grow
 *                        along a forwarding path, so the set equals the
 *                        direct definition for the final receiver. */
typedef enum { HALO_SELECT_SLAB = 0, HALO_SELECT_CORNER = 1 } halo_selection;

/* halo_plan_create with a selection test (a halo_selection value; anything
 * else gives HALO_ERR_ARG). halo_plan_create is this call with
 * HALO_SELECT_SLAB. */
halo_status halo_plan_create_ex(const float *positions, int64_t n_atoms, const float *box,
                                const int32_t *grid, float cutoff, int32_t selection,
                                halo_plan **out);

/* Build the same plan on the GPU from device-resident positions, for
 * repartitioning steps of a GPU-resident simulation (the pages rebuild the
 * halo metadata at every domain-decomposition / neighbour-search step; see
 * "Redesigning GROMACS Halo Exchange", s.3 and Algorithms 1 and 4). The
 * result is identical to halo_plan_create on the same positions: layout,
 * home slots, every PulseData field, the work items, the XCD-local units and
 * the exchanges' results. (The units' pieces come back in one copy of an
 * estimated size and, when there are more, in a second one; the environment
 * variable HALO_UNIT_PIECES_CAP, read at the build, caps the first copy, for
 * testing that path.)
 *   positions : DEVICE, n_atoms*3 float32 on the current device, read on
 *               `stream` (so work queued there before the call is seen)
 *   stream    : a hipStream_t; the call synchronises it a few times (it reads
 *               back per-pulse sizes) and returns with the plan uploaded. A
 *               stream that is being captured into a HIP graph gives
 *               HALO_ERR_ARG before anything is queued.
 *   others    : as halo_plan_create.
 * Limits: at most 8192 domains (HALO_ERR_GEOMETRY beyond). A position not
 * finite or outside [0, L) gives HALO_ERR_RANGE naming the first such atom.
 * The host copies of the indexMaps and home slots (halo_plan_pulse's
 * index_map, halo_plan_home_slots) are fetched from the device on first use. */
halo_status halo_plan_create_device(const float *positions, int64_t n_atoms, const float *box,
                                    const int32_t *grid, float cutoff, void *stream,
                                    halo_plan **out);

/* halo_plan_create_device with a selection test, as halo_plan_create_ex. */
halo_status halo_plan_create_device_ex(const float *positions, int64_t n_atoms, const float *box,
                                       const int32_t *grid, float cutoff, int32_t selection,
                                       void *stream, halo_plan **out);

/* Rebuild an existing plan on the GPU for new positions (a repartitioning
 * step), keeping its domain grid, cutoff and selection test; `box` may change (pressure
 * coupling). The result is the plan halo_plan_create_device would build, and
 * a plan built on the device keeps its device memory (grown only when the new
 * plan needs more), so a rebuild allocates nothing in the steady state.
 *   positions, n_atoms, stream : as halo_plan_create_device
 *   box : host, 3 float32
 * The counters restart (no exchange of this plan may be in flight on any
 * stream); total_slots, the layout and the home slots change, so x and f must
 * be re-laid out by the caller. Argument and geometry errors, and a stream
 * that is being captured (HALO_ERR_ARG, checked before anything is freed or
 * queued), leave the plan unchanged; any other error (HALO_ERR_RANGE for a position out of range, a
 * HIP failure) leaves it empty, and exchanges return HALO_ERR_STATE until a
 * rebuild succeeds. */
halo_status halo_plan_rebuild_device(halo_plan *plan, const float *positions, int64_t n_atoms,
                                     const float *box, void *stream);

/* Free the plan and its device metadata (NULL is accepted). Waits for nothing:
 * the caller must make sure no exchange on the plan is still running. */
void halo_plan_destroy(halo_plan *plan);

/* Message describing the calling thread's most recent error ("" if none). */
const char *halo_last_error(void);

/* ---- plan read-out ----------------------------------------------------------------- */

int64_t halo_plan_total_slots(const halo_plan *plan);  /* slots in x and f; -1 on NULL */
int32_t halo_plan_num_domains(const halo_plan *plan);  /* nx*ny*nz; -1 on NULL        */
int32_t halo_plan_num_pulses(const halo_plan *plan);   /* np(x)+np(y)+np(z); -1 on NULL */
int64_t halo_plan_num_entries(const halo_plan *plan);  /* indexMap entries, all pulses */
int32_t halo_plan_num_items(const halo_plan *plan);    /* work items (workgroups) per exchange */
int32_t halo_plan_selection(const halo_plan *plan);    /* a halo_selection value; -1 on NULL */

/* Dimension (0 = x, 1 = y, 2 = z) and number within that dimension of pulse p. */
halo_status halo_plan_pulse_dim(const halo_plan *plan, int32_t p, int32_t *dim, int32_t *k);

/* Layout of domain d: first slot, home count, halo count (outputs may be NULL). */
halo_status halo_plan_domain(const halo_plan *plan, int32_t d, int64_t *base, int32_t *n_home,
                             int32_t *n_halo);

/* Home slot of every atom: slot_of_atom is host memory of n_atoms int64. */
halo_status halo_plan_home_slots(const halo_plan *plan, int64_t *slot_of_atom);

/* PulseData of pulse p for sending domain d (Algorithm 1); outputs may be NULL.
 *   send_to     : the receiving domain
 *   send_size   : indexMap length
 *   recv_from   : the domain that sends to d in this pulse
 *   recv_size   : entries d receives in this pulse
 *   atom_offset : first local slot of d's region for this pulse
 *   dep_start   : entries of indexMap below depOffset (= d's home count): the
 *                 independent prefix of Algorithm 4
 *   items       : work items the plan cut this (pulse, domain) into
 *   shift       : 3 float32, coordShift
 *   index_map   : host, send_size int32 local slots of d, ascending */
halo_status halo_plan_pulse(const halo_plan *plan, int32_t p, int32_t d, int32_t *send_to,
                            int32_t *send_size, int32_t *recv_from, int32_t *recv_size,
                            int32_t *atom_offset, int32_t *dep_start, int32_t *items, float *shift,
                            int32_t *index_map);

/* ---- device side ------------------------------------------------------------------- */

/* Work item `item` (0 <= item < halo_plan_num_items) of the index-list
 * kernels, in launch order: its segment (pulse * num_domains + sending
 * domain); the pulses whose regions its dependent entries read (bit r: the
 * region the sender received in pulse r; the coordinate exchange waits for
 * their arrival, Algorithm 4); and, for halo_exchange_f_atomic, the later
 * pulses q whose segment (q, receiver) adds into the region the item reads.
 * Any output may be NULL. A read-out for tests and tools. */
halo_status halo_plan_item_waits(const halo_plan *plan, int32_t item, int32_t *segment,
                                 uint32_t *xwait_mask, uint32_t *await_mask);

/* Chunks of the transposed form (0 for plans of more than 8 pulses), in
 * launch order of its coordinate kernel: the home slots of every domain, then
 * the region received in pulse 0, pulse 1, ... Chunk c is a run of `count`
 * consecutive slots from absolute slot `first` of `domain`, inside its home
 * slots (zone -1) or its region of pulse `zone`; bit p of `mask` is set when
 * one of its slots is sent in pulse p. Outputs may be NULL. A read-out for
 * tests and tools. */
int32_t halo_plan_num_chunks(const halo_plan *plan);  /* -1 on NULL */
halo_status halo_plan_chunk(const halo_plan *plan, int32_t chunk, int32_t *domain, int32_t *zone,
                            int64_t *first, int32_t *count, uint32_t *mask);

/* XCD-local units of the index-list kernels (both builds make the same
 * units). A unit is a run of one indexMap whose
 * atoms share one home domain (their origin); it sits at a position of the
 * coordinate kernel's grid whose index mod 8 is its origin mod 8, so that all
 * units of an origin, and with them every dependency of both exchanges, run
 * on one XCD. Unit `position`: its segment (pulse * num_domains + sending
 * domain; -1 for an empty position), origin (-1 if empty), entries, and the
 * number of units it waits for in the coordinate and in the force exchange.
 * Outputs may be NULL. A read-out for tests and tools. */
int32_t halo_plan_num_local_units(const halo_plan *plan);  /* -1 on NULL */
halo_status halo_plan_local_unit(const halo_plan *plan, int32_t position, int32_t *segment,
                                 int32_t *origin, int32_t *entries, int32_t *x_waits,
                                 int32_t *f_waits);

/* Allocate and upload the device metadata on the current HIP device (blocking:
 * it synchronises the device). The first exchange on a plan built by
 * halo_plan_create calls it implicitly, and is then the only exchange call
 * that synchronises; call it up front to keep every exchange asynchronous.
 * Plans built on the device are uploaded when they are built. */
halo_status halo_plan_upload(halo_plan *plan);

/* Coordinate exchange, Algorithms 3-5 fused into ONE kernel launch on
 * `stream` (a hipStream_t; NULL = default stream). All pulses run at once:
 * the entries of each indexMap below depOffset (home slots) are packed
 * immediately; entries that forward atoms received in earlier pulses wait,
 * inside the kernel, on the arrival counters of exactly the regions they
 * read. Runs the transposed form (halo_exchange_x_transposed) for plans of
 * at least 2^20 indexMap entries, the index-list form
 * (halo_exchange_x_indexmap) for smaller plans and for plans with more than
 * 8 pulses.
 *   x : device, total_slots*3 float32, 4-byte aligned. Home slots are read;
 *       every halo slot is overwritten with x[indexMap[i]] + coordShift.
 * Asynchronous; exchanges of one plan must be ordered on one stream. Fused
 * exchanges of different plans may run at once on different streams; their
 * in-kernel waits then compete for the same compute units, and an
 * interleaving that starves a producer ends in HALO_ERR_TIMEOUT, not a hang.
 * HIP graphs: every exchange form can be captured once the plan is uploaded
 * (halo_plan_upload, or any earlier exchange). The fused kernels take no
 * per-call argument: each launch infers its epoch (Algorithm 5's signal
 * value) from launch counters in the plan's device memory, so replays of
 * captured exchanges and eager calls of the same plan may follow one another
 * in any order, as long as they are ordered on one stream. Before the upload,
 * a call on a capturing stream returns HALO_ERR_ARG (the upload allocates and
 * synchronises). A graph holds the plan's device addresses: after
 * halo_plan_rebuild_device or halo_plan_debug_stress, capture it again
 * (halo_plan_reset keeps them). */
halo_status halo_exchange_x(halo_plan *plan, float *x, void *stream);

/* Force exchange, Algorithm 6 in ONE kernel launch: pulses from last to
 * first; for every sender d of pulse p, f[indexMap[i]] += f[receiver's region
 * of pulse p][i], with the per-slot order of additions of the serial
 * reverse-pulse loop, so results are bitwise deterministic. Runs the
 * transposed form (halo_exchange_f_transposed) for plans of at most 3 pulses
 * and at least 2^20 indexMap entries, the index-list form
 * (halo_exchange_f_indexmap) for the others.
 *   f : device, total_slots*3 float32, updated in place. On return home slots
 *       hold the accumulated forces; forwarding halo slots hold partial sums.
 * Asynchronous; exchanges of one plan must be ordered on one stream. */
halo_status halo_exchange_f(halo_plan *plan, float *f, void *stream);

/* Index-list form of the fused exchanges (Algorithms 3-6): one work unit
 * (workgroup) per run of an indexMap, in pulse-major order (reverse for
 * forces); entries below depOffset go at once, the others after a wait on
 * the units that wrote the region stretch they read; forces added with one
 * read-modify-write per entry, after every later pulse that adds into the
 * same slots. The units are XCD-local (halo_plan_local_unit): runs of one
 * origin, placed so that each forwarding stage stays in one XCD's L2, with
 * per-unit flags; an exchange whose units find their producers on another
 * XCD reports HALO_ERR_PLACEMENT from halo_plan_sync. */
halo_status halo_exchange_x_indexmap(halo_plan *plan, float *x, void *stream);
halo_status halo_exchange_f_indexmap(halo_plan *plan, float *f, void *stream);

/* The index-list form on the plan's work items (halo_plan_item_waits) with
 * one completion counter per (pulse, sender) segment at the device-coherent
 * level instead of the XCD-local units and their flags: the same results,
 * kept as an ablation of the XCD-local placement. */
halo_status halo_exchange_x_items(halo_plan *plan, float *x, void *stream);
halo_status halo_exchange_f_items(halo_plan *plan, float *f, void *stream);

/* Ablation of the coordinate store ("Redesigning GROMACS Halo Exchange",
 * s.4 on the coalescing of float3 coordinates into aligned stores): the
 * index-list coordinate exchange on XCD-local units with each unit's
 * contiguous run of destination slots staged in LDS and written as 16-byte
 * stores on 16-byte boundaries, instead of one 12-byte store per slot. Same
 * results. */
halo_status halo_exchange_x_indexmap_lds(halo_plan *plan, float *x, void *stream);

/* Transposed form of the fused exchanges: the indexMaps stored as one pulse
 * mask per slot; a workgroup takes a run of slots of one domain inside one
 * zone (home slots, or the region of one pulse). Coordinates: each slot is
 * read once and stored, plus coordShift, to every pulse it carries, at its
 * rank among the run's slots of that pulse (a per-row count the plan keeps,
 * plus a wave ballot); region runs wait for their region to arrive. Forces: each target slot keeps its running sum in a
 * register and adds its pulses' sources in strict reverse order, waiting
 * until each source holds its final sum; every target is read and written
 * once. HALO_ERR_ARG for plans with more than 8 pulses. */
halo_status halo_exchange_x_transposed(halo_plan *plan, float *x, void *stream);
halo_status halo_exchange_f_transposed(halo_plan *plan, float *f, void *stream);

/* The same two exchanges as one kernel launch per pulse, with no in-kernel
 * waits: stream order between the launches carries the dependencies (the
 * per-pulse "first design" of the NVIDIA guide, "Fusing pack, put, and wait
 * into one kernel"). Results are bitwise identical to the fused calls. */
halo_status halo_exchange_x_pulsewise(halo_plan *plan, float *x, void *stream);
halo_status halo_exchange_f_pulsewise(halo_plan *plan, float *f, void *stream);

/* Force exchange with atomic accumulation, as "Redesigning GROMACS Halo
 * Exchange" (paper review), Algorithm 6, prints it: one launch, the items of
 * every pulse in flight together, each adding its received forces onto its
 * indexMap targets with atomicAdd. An item waits only until the slots it
 * reads (the receiver's region of its pulse) hold their final sums. The order
 * of the adds onto one slot is not fixed, so the result matches
 * halo_exchange_f only up to fp32 rounding: per slot, at most
 * 2 * (n - 1) * 2^-24 * (sum of |terms|) apart, n being the number of values
 * summed into the slot; it is bitwise equal whenever every partial sum is
 * exact (small integers, for example). Same arguments, ownership and errors
 * as halo_exchange_f. Like every exchange of one plan, order it on one
 * stream with the plan's other exchanges. */
halo_status halo_exchange_f_atomic(halo_plan *plan, float *f, void *stream);

/* Staged baseline (the message-passing design that the pages measure the
 * zero-copy exchange against, "GPU-Initiated Halo Exchange Cuts CPU
 * Bottlenecks in GROMACS"): per pulse, one launch packs x[indexMap] +
 * coordShift into a staging buffer owned by the plan, and a second launch
 * moves the staged entries into the receiver's region; for forces the region
 * is first copied out to the staging buffer and then scatter-added onto the
 * targets. 2 * num_pulses launches per exchange, bitwise identical results.
 * The first staged call on a plan allocates the staging buffer
 * (num_entries * 12 bytes; HALO_ERR_HIP if that fails). */
halo_status halo_exchange_x_staged(halo_plan *plan, float *x, void *stream);
halo_status halo_exchange_f_staged(halo_plan *plan, float *f, void *stream);

/* halo_exchange_x_staged for callers that cannot allocate device memory
 * (code under HIP graph capture, tight loops, harnesses that forbid it): the
 * same launches and results, staging in a static device array of 32 MiB per
 * GPU (held until the process ends) instead of a buffer the plan allocates.
 * The plan must already be on the device (halo_plan_upload or any earlier
 * exchange; HALO_ERR_STATE otherwise); plans of more than 2,796,202 indexMap
 * entries (12 bytes each) get HALO_ERR_ARG. Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (other streams, other plans)
 * race and must be ordered by the caller. Asynchronous on `stream`. */
halo_status halo_exchange_x_staged_noalloc(halo_plan *plan, float *x, void *stream);

/* Direct coordinate exchange, a one-GPU form of the same result: every halo
 * slot is gathered straight from its atom's home slot, adding +L_d for each
 * dimension in which the atom's forwarding path wraps, in one launch with no
 * waits and no counters. Because an atom wraps at most once per dimension,
 * one add per component gives the bits of the pulse-by-pulse chain
 * (x[indexMap[i]] + coordShift per pulse), so results are bitwise identical to
 * halo_exchange_x. The forwarding of the pages ("Redesigning GROMACS Halo
 * Exchange", Algorithm 4) is what a decomposition over several GPUs needs;
 * on one GPU it is a choice, and this form measures what it costs.
 * The first call on a plan derives the origin map (num_entries * 4 bytes,
 * plus total_slots * 4 bytes of temporary memory) from the indexMaps and
 * synchronises `stream`; it refuses a capturing stream (HALO_ERR_ARG) and
 * reports HALO_ERR_HIP if an allocation fails. Later calls are one
 * asynchronous launch and can be captured into a HIP graph. A rebuild
 * discards the map. Same arguments as halo_exchange_x. */
halo_status halo_exchange_x_direct(halo_plan *plan, float *x, void *stream);

/* Copy a per-atom array of float triples into the home slots of a slot
 * buffer (slots[home_slot[a]] = values[a]), or back out of them
 * (values[a] = slots[home_slot[a]]), home_slot being halo_plan_home_slots.
 * Fills x before halo_exchange_x, or collects the forces after
 * halo_exchange_f, from or into the caller's atom order.
 *   values : device, n_atoms*3 float32 (the positions' order at creation)
 *   slots  : device, total_slots*3 float32; only home slots are touched
 * One asynchronous launch on `stream`. For a plan built on the host, the
 * first call uploads the home slots (n_atoms*8 bytes), synchronises and
 * refuses a capturing stream; later calls can be captured. HALO_ERR_ARG for
 * NULL buffers. */
halo_status halo_scatter_home(halo_plan *plan, const float *values, float *slots, void *stream);
halo_status halo_gather_home(halo_plan *plan, const float *slots, float *values, void *stream);

/* Wait for the plan's work on `stream` and report a timeout raised inside a
 * kernel (HALO_ERR_TIMEOUT); poisons the plan in that case. */
halo_status halo_plan_sync(halo_plan *plan, void *stream);

/* Clear a poisoned plan: zero the device counters and the error word (blocking,
 * device-wide synchronisation). */
halo_status halo_plan_reset(halo_plan *plan);

/* Bound on the polls of one in-kernel dependency wait (default 1<<20, each
 * separated by a short sleep). A debugging and testing knob. */
halo_status halo_plan_set_spin_limit(halo_plan *plan, uint32_t polls);

/* Testing hook: when `segment` >= 0, the fused kernels skip the completion
 * signal of that (pulse * num_domains + domain) segment, so that its
 * dependents run into their spin limit and the timeout path is exercised.
 * -1 (the default) disables it. */
halo_status halo_plan_debug_withhold(halo_plan *plan, int32_t segment);

/* Testing hook: with seed != 0 the fused kernels (index-list, transposed and
 * atomic forms) run every group of mutually independent work units (the
 * items of one pulse, the chunks of one zone, the XCD-local units of one class
 * and one pulse) in reversed order, and every
 * unit first sleeps a pseudo-random while (up to about 100 us) derived from
 * the seed. Results must not change: this exposes missing waits or orderings.
 * seed = 0 (the default) turns it off. Synchronises the device when it
 * changes an existing setting. A rebuild turns it off. */
halo_status halo_plan_debug_stress(halo_plan *plan, uint32_t seed);

/* Tuning aid (where an exchange's time goes along the forwarding chain of
 * "Redesigning GROMACS Halo Exchange", Algorithms 4-6): with enable != 0, the
 * fused kernels of every form and halo_exchange_x_direct record, for every
 * work unit (work item or chunk) they run, the device's constant-rate clock
 * at the unit's start, when its first dependency wait begins, when its last
 * wait ends, when its first completion signal is sent (its stores complete)
 * and at its end, plus where it ran. Each launch overwrites the records of
 * the units it runs. enable == 0 frees the record buffer. The call allocates
 * and synchronises the device (not under graph capture); a rebuild turns the
 * recording off. Results of the exchanges do not change. */
halo_status halo_plan_debug_timing(halo_plan *plan, int32_t enable);

/* Copy the records of halo_plan_debug_timing (blocking: synchronises the
 * device). Unit u (a work item of the index-list and direct forms, a chunk of
 * the transposed form, in the plan's unit numbering) occupies words
 * [8u, 8u + 8) of `stamps` (host memory of max_units * 8 uint64):
 *   0 start, 1 first wait begins, 2 last wait ends, 3 first signal sent,
 *   4 end (clock ticks; 0 = the unit did not reach that step),
 *   5 workgroup index, 6 HW_ID register, 7 XCC_ID register.
 *   units     : receives the number of units recorded (may be NULL)
 *   clock_khz : receives the clock's rate in kHz (may be NULL)
 * stamps may be NULL to query units and clock_khz only; HALO_ERR_ARG if the
 * recording is off or max_units is below the unit count. */
halo_status halo_plan_debug_timing_read(halo_plan *plan, uint64_t *stamps, int64_t max_units,
                                        int64_t *units, int32_t *clock_khz);

#ifdef __cplusplus
}
#endif

#endif /* HALO_H */
