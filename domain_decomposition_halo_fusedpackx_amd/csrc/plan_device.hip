// plan_device.hip -- build the exchange plan on the GPU from device-resident
// positions, for repartitioning steps.
//
// Same plan as plan.cpp, and the same readings of "Redesigning GROMACS Halo
// Exchange" (paper review), s.3 and Algorithms 1 and 4: the domain of an atom
// is floor(min(x / w, nextafter(n, 0))) per dimension in double precision;
// home atoms in ascending id; pulses z, then y, then x; an atom is sent when
// its original position lies less than cutoff / w above the receiver's upper
// face (periodically); candidates are all slots on the first pulse of a
// dimension and the previous pulse's region otherwise; indexMap ascending;
// slots of a domain = [home | region per pulse], domains in id order.
//
// The work that grows with the atoms and the entries runs in kernels:
//   k_owner          domain of every atom, range check, per-tile histogram
//   k_tile_scan      per domain, exclusive scan of the tile histogram
//   k_home_start     first home slot of every domain; slot cursors
//   k_home_scatter   stable counting sort: home atoms of every domain in
//                    ascending id (wave-level radix sort by domain, waves in order)
//   k_select<false>  per (pulse, domain): how many candidates are sent, and
//                    how many of them are home slots (depOffset split)
//   k_pulse_scan     the pulse's map offsets and the receivers' regions
//   k_select<true>   the same selection writing the indexMap (local slots)
//                    and the id of every sent atom, by stable compaction
//   k_abs_map        indexMap entries as absolute slots; the origin (home
//                    domain) of every home slot
//   k_home_slot      slot of every atom
//   k_origin_pulse   per pulse, the origins of the regions received
//   k_unit_runs      per segment, the runs of entries whose sources share
//   k_unit_scan        origin and zone, cut into pieces (the XCD-local
//   k_unit_write       units' pieces), with their offsets
//   k_mask           per-slot pulse masks of the transposed form
//   k_item_masks     wait masks of the work items
//   k_piece_stats    union mask and per-pulse counts of every chunk candidate
// and the host keeps the O(domains x pulses + items + chunks + units)
// bookkeeping that needs the sizes: the layout, the work items, the chunk
// order and the placement of the units. The host synchronises three times:
// after the pulses (sizes), after the chunk statistics, and at the end.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <string>
#include <vector>

#include "plan.hpp"
#include "plan_state.hpp"
#include "sync.hpp"

namespace halo {
namespace {

constexpr int kBT = 256;                 // threads per block
// Atoms per histogram tile: 512 (two per thread), or 2048 for systems that
// still give every compute unit a 2048-atom tile and whenever the 512-atom
// tiles' histogram (domains x tiles) would pass 16 M counters.
constexpr int kTileSmall = 512, kTileLarge = 2048;
constexpr int64_t kMaxTileCounters = (int64_t)1 << 24;
constexpr int64_t kComputeUnits = 256;  // MI355X
constexpr int32_t kMaxDeviceDomains = 8192;  // LDS histogram of 32 KiB

struct Geom {
    double width[3];
    double top[3];  // nextafter(n_d, 0): scaled positions are clamped below n_d
    double rc2;     // cutoff^2, for the corner selection
    float box[3];
    int32_t grid[3];
    int32_t corner; // 1: corner selection, 0: slab selection
};

__device__ __forceinline__ double scaled(float v, double width, double top)
{
    double s = (double)v / width;
    return s > top ? top : s;
}

// Exclusive prefix of v over the block's threads (in thread order); total
// receives the block sum. Every thread of the block must call it.
__device__ uint32_t block_scan_excl(uint32_t v, uint32_t &total)
{
    __shared__ uint32_t ws[kBT / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) ws[w] = x;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kBT / 64; ++i) {
        if (i < w) off += ws[i];
        tot += ws[i];
    }
    __syncthreads();
    total = tot;
    return off + x - v;
}

__device__ __forceinline__ uint64_t lanes_below(int lane)
{
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Position of the thread among the block's NT threads with flag set (thread
// order); total receives their number.
template <int NT>
__device__ uint32_t block_rank(bool flag, uint32_t &total)
{
    __shared__ uint32_t wc[NT / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t b = __ballot(flag);
    if (lane == 0) wc[w] = (uint32_t)__popcll(b);
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        if (i < w) off += wc[i];
        tot += wc[i];
    }
    __syncthreads();
    total = tot;
    return off + (uint32_t)__popcll(b & lanes_below(lane));
}

// Domain of every atom (0 for an atom out of range, whose smallest index goes
// to *bad) and the tile's histogram over domains, stored domain-major.
template <int kTile>
__global__ __launch_bounds__(kBT) void k_owner(const float *__restrict__ pos, int64_t n_atoms,
                                               Geom g, int32_t n_dom, int32_t n_tiles,
                                               int32_t *__restrict__ owner,
                                               uint32_t *__restrict__ tile_hist,
                                               unsigned long long *bad)
{
    extern __shared__ uint32_t hist[];
    for (int32_t d = threadIdx.x; d < n_dom; d += kBT) hist[d] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * kTile;
    for (int j = 0; j < kTile / kBT; ++j) {
        const int64_t a = t0 + j * kBT + threadIdx.x;
        if (a < n_atoms) {
            bool ok = true;
            int32_t c[3];
#pragma unroll
            for (int d = 0; d < 3; ++d) {
                const float v = pos[3 * a + d];
                if (!(__builtin_isfinite(v) && v >= 0.f && v < g.box[d])) ok = false;
                c[d] = ok ? (int32_t)floor(scaled(v, g.width[d], g.top[d])) : 0;
            }
            const int32_t dom = ok ? c[0] + g.grid[0] * (c[1] + g.grid[1] * c[2]) : 0;
            if (!ok) atomicMin(bad, (unsigned long long)a);
            owner[a] = dom;
            atomicAdd(&hist[dom], 1u);
        }
    }
    __syncthreads();
    for (int32_t d = threadIdx.x; d < n_dom; d += kBT)
        tile_hist[(size_t)d * n_tiles + blockIdx.x] = hist[d];
}

// Block d: exclusive scan over the tiles of domain d's histogram row (in
// place); n_home[d] = the row total.
__global__ __launch_bounds__(kBT) void k_tile_scan(uint32_t *__restrict__ tile_hist,
                                                   int32_t n_tiles, int32_t *__restrict__ n_home)
{
    uint32_t *row = tile_hist + (size_t)blockIdx.x * n_tiles;
    uint32_t carry = 0;
    for (int32_t b = 0; b < n_tiles; b += kBT) {
        const int32_t t = b + threadIdx.x;
        const uint32_t v = t < n_tiles ? row[t] : 0u;
        uint32_t tot;
        const uint32_t ex = block_scan_excl(v, tot);
        if (t < n_tiles) row[t] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) n_home[blockIdx.x] = (int32_t)carry;
}

// Stable sort of the wave's 64 values by their key bits (value = key << 6 |
// lane): LSD radix, one key bit per pass, each lane pushing its value to its
// new position. Every lane of the wave must take part.
__device__ __forceinline__ uint32_t wave_sort_by_key(uint32_t v, int key_bits)
{
    const int lane = threadIdx.x & 63;
    const uint64_t below = lanes_below(lane);
    for (int b = 0; b < key_bits; ++b) {
        const bool one = (v >> (6 + b)) & 1u;
        const uint64_t ones = __ballot(one);
        const uint32_t zeros_total = 64u - (uint32_t)__popcll(ones);
        const uint32_t pos = one ? zeros_total + (uint32_t)__popcll(ones & below)
                                 : (uint32_t)__popcll(~ones & below);
        v = (uint32_t)__builtin_amdgcn_ds_permute((int)(pos * 4u), (int)v);
    }
    return v;
}

// Stable counting sort of the atoms by domain, carrying their coordinates
// (x, y, z interleaved per home slot: one 12-byte store per atom, where
// three scattered 4-byte stores cost twice the kernel's time). Block = tile;
// LDS counters start at the tile's offsets within each domain. In each round of 256 atoms
// a wave sorts its lanes by domain (stable), so that lanes with one domain
// form a run in id order; the waves then add their run lengths to the
// counters one after the other, so that lower ids get lower ranks.
template <int kTile>
__global__ __launch_bounds__(kBT) void k_home_scatter(const int32_t *__restrict__ owner,
                                                      int64_t n_atoms, int32_t n_dom,
                                                      int32_t n_tiles,
                                                      const uint32_t *__restrict__ tile_off,
                                                      const int32_t *__restrict__ home_start,
                                                      const float *__restrict__ pos,
                                                      float *__restrict__ home_c,
                                                      int32_t *__restrict__ home_rank)
{
    extern __shared__ uint32_t cnt[];
    for (int32_t d = threadIdx.x; d < n_dom; d += kBT)
        cnt[d] = tile_off[(size_t)d * n_tiles + blockIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    // keys of up to n_dom (n_dom marks lanes past the last atom)
    int key_bits = 1;
    while ((1 << key_bits) <= n_dom) ++key_bits;
    // all of the tile's domain ids are loaded up front
    int32_t keys[kTile / kBT];
#pragma unroll
    for (int j = 0; j < kTile / kBT; ++j) {
        const int64_t a = (int64_t)blockIdx.x * kTile + j * kBT + threadIdx.x;
        keys[j] = a < n_atoms ? owner[a] : n_dom;
    }
    const uint64_t le = lane == 63 ? ~0ull : ((2ull << lane) - 1ull);  // lanes <= this one
#pragma unroll
    for (int j = 0; j < kTile / kBT; ++j) {
        const int64_t a = (int64_t)blockIdx.x * kTile + j * kBT + threadIdx.x;
        const bool valid = a < n_atoms;
        // after the sort, sorted lane i holds (key, original lane) of the
        // i-th value in (key, lane) order
        const uint32_t sv = wave_sort_by_key(((uint32_t)keys[j] << 6) | (uint32_t)lane, key_bits);
        const int32_t skey = (int32_t)(sv >> 6);
        const int32_t prev = __shfl_up((int)skey, 1, 64);
        const bool head = lane == 0 || prev != skey;
        const uint64_t heads = __ballot(head);
        const int run_start = 63 - __clzll((long long)(heads & le));
        const uint64_t after = heads & ~le;
        const int run_end = after ? __ffsll((long long)after) - 1 : 64;
        uint32_t base = 0;
        for (int t = 0; t < kBT / 64; ++t) {
            if (w == t && head && skey < n_dom) {
                base = cnt[skey];
                cnt[skey] = base + (uint32_t)(run_end - lane);
            }
            __syncthreads();
        }
        base = (uint32_t)__shfl((int)base, run_start, 64);
        const uint32_t r_sorted = base + (uint32_t)(lane - run_start);
        // back to the lane that holds the atom
        const uint32_t r = (uint32_t)__builtin_amdgcn_ds_permute((int)((sv & 63u) * 4u),
                                                                 (int)r_sorted);
        if (valid) {
            const int32_t key = keys[j];
            const int64_t h = home_start[key] + (int64_t)r;
#pragma unroll
            for (int d = 0; d < 3; ++d) home_c[3 * h + d] = pos[3 * a + d];
            home_rank[a] = (int32_t)r;
        }
    }
}

// Device copy of the segment table: per pulse, five rows of n_dom int32
// (sendSize, send count from home slots, recvSize, atomOffset, map offset),
// so that a pulse's counts come back, and its offsets go out, in one copy.
enum { kSendSize = 0, kDepStart = 1, kRecvSize = 2, kAtomOffset = 3, kMapOff = 4, kSegRows = 5 };
struct SegTable {
    int32_t *t;
    int32_t nd;
    __host__ __device__ int32_t *row(int32_t p, int f) const
    {
        return t + ((size_t)p * kSegRows + f) * nd;
    }
};

// Corner selection: the squared distance from the atom at src (coordinates
// `stride` apart) to the box of the receiver in cell cr, summed over x, y, z
// in this order in double, is below cutoff^2. A dimension where the atom lies
// in the receiver's slab (other than the pulse's own) adds nothing.
__device__ __forceinline__ bool corner_test(const float *src, int64_t stride, int32_t dim,
                                         const int32_t cr[3], const Geom &g)
{
    double dist2 = 0.0;
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const double t = scaled(src[d * stride], g.width[d], g.top[d]);
        double delta = 0.0;
        if (d == dim || (int32_t)floor(t) != cr[d]) {
            delta = t - (double)(cr[d] + 1);
            if (delta < 0.0) delta += (double)g.grid[d];
        }
        const double dist = delta * g.width[d];
        dist2 += dist * dist;
    }
    return dist2 < g.rc2;
}

// Selection of pulse p for domain D = blockIdx.x. Candidates in ascending
// local slot: the home slots and every region received so far (k == 0), or
// the region of the previous pulse (k > 0). A candidate is sent when its
// atom's original position lies less than reach above the receiver's upper
// face and, with the corner selection, its Euclidean distance to the
// receiver's box is below the cutoff. WRITE == false: store the send count and how many candidates were
// home slots; WRITE == true: store the indexMap (local slots) and the sent
// atoms' coordinates (entry_c, one row of `cap` per dimension) from map_off
// on, in candidate order.
constexpr int kSelectThreads = 512;  // one block per domain: 8 waves (1024 measured slower)

template <bool WRITE>
__global__ __launch_bounds__(kSelectThreads) void k_select(
    int32_t p, int32_t dim, int32_t k, int32_t n_dom, Geom g,
    double reach, const int32_t *__restrict__ send_to, const int32_t *__restrict__ recv_from,
    const int32_t *__restrict__ n_home, const int32_t *__restrict__ home_start,
    const float *__restrict__ home_c, int64_t n_atoms, SegTable seg, float *entry_c,
    int32_t *__restrict__ local_map, int32_t cap)
{
    constexpr int NT = kSelectThreads;
    constexpr int kRows = 1;  // rows of NT candidates per step (2, 4 or 8 measured slower)
    // The candidate zones in slot order ([home,] regions), laid end to end:
    // candidate i of the domain is entry i - zbeg[z] of zone z.
    __shared__ int32_t zbeg[kMaxPulses + 2], zslot[kMaxPulses + 1], zoff[kMaxPulses + 1],
        zlen[kMaxPulses + 1];
    __shared__ uint32_t dep_lds;
    const int32_t D = blockIdx.x;
    const int32_t zfirst = k == 0 ? -1 : p - 1;
    const int32_t nz = p - zfirst;
    // thread j reads zone j's sizes (one round of loads for all zones)
    if ((int32_t)threadIdx.x < nz) {
        const int32_t j = threadIdx.x, z = zfirst + j;
        int32_t len;
        if (z < 0) {
            len = n_home[D];
            zslot[j] = 0;
            zoff[j] = home_start[D];
        } else {
            const int32_t S = recv_from[z * n_dom + D];
            len = seg.row(z, kRecvSize)[D];
            zslot[j] = seg.row(z, kAtomOffset)[D];
            const int32_t off = seg.row(z, kMapOff)[S];
            zoff[j] = off;
            // an earlier pulse overflowed the entry arrays: the host
            // rebuilds with more room; read nothing past them meanwhile
            if (off > cap - len) len = 0;
        }
        zlen[j] = len;
    }
    if (threadIdx.x == 0) dep_lds = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t acc = 0;
        for (int32_t j = 0; j < nz; ++j) {
            zbeg[j] = acc;
            acc += zlen[j];
        }
        zbeg[nz] = acc;
    }
    __syncthreads();
    const int32_t total = zbeg[nz];
    const int32_t R = send_to[p * n_dom + D];
    const int32_t cr[3] = {R % g.grid[0], (R / g.grid[0]) % g.grid[1],
                           R / (g.grid[0] * g.grid[1])};  // receiver's cell
    const double face = (double)(cr[dim] + 1);
    const double ncell = (double)g.grid[dim];
    const int32_t out0 = WRITE ? seg.row(p, kMapOff)[D] : 0;
    const int32_t limit = WRITE ? seg.row(p, kSendSize)[D] : 0;
    const bool home_first = zfirst < 0;
    uint32_t count = 0;
    for (int32_t b = 0; b < total; b += kRows * NT) {
        // candidate coordinates in slot order: the home slots' interleaved
        // (x, y, z), the entries' one row per dimension (the order they were
        // sent in); contiguous either way
        const float *src[kRows];
        int32_t slot[kRows];
        int64_t stride[kRows];
        float v[kRows];
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            const int32_t i = b + j * NT + (int32_t)threadIdx.x;
            src[j] = nullptr;
            slot[j] = 0;
            stride[j] = 0;
            if (i < total) {
                int32_t z = 0;
                while (i >= zbeg[z + 1]) ++z;
                const int32_t e = i - zbeg[z];
                const bool from_home = home_first && z == 0;
                src[j] = from_home ? home_c + 3 * ((int64_t)zoff[z] + e) : entry_c + zoff[z] + e;
                stride[j] = from_home ? 1 : (int64_t)cap;
                slot[j] = zslot[z] + e;
            }
        }
#pragma unroll
        for (int j = 0; j < kRows; ++j) v[j] = src[j] ? src[j][dim * stride[j]] : 0.f;
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            bool flag = false;
            if (src[j]) {
                double above = scaled(v[j], g.width[dim], g.top[dim]) - face;
                if (above < 0.0) above += ncell;
                flag = above < reach;
                if (flag && g.corner) flag = corner_test(src[j], stride[j], dim, cr, g);
            }
            if (!WRITE) {
                // sends from home slots (the depOffset split)
                const bool home = home_first && b + j * NT + (int32_t)threadIdx.x < zbeg[1];
                const uint64_t hb = __ballot(flag && home);
                if ((threadIdx.x & 63) == 0 && hb) atomicAdd(&dep_lds, (uint32_t)__popcll(hb));
            }
            uint32_t tot;
            const uint32_t r = block_rank<NT>(flag, tot);
            if (WRITE && flag && (int32_t)(count + r) < limit &&
                out0 + (int32_t)(count + r) < cap) {
                const int32_t o = out0 + (int32_t)(count + r);
                local_map[o] = slot[j];
#pragma unroll
                for (int d = 0; d < 3; ++d) entry_c[d * (int64_t)cap + o] = src[j][d * stride[j]];
            }
            count += tot;
        }
    }
    if (!WRITE) {
        __syncthreads();
        if (threadIdx.x == 0) {
            seg.row(p, kSendSize)[D] = (int32_t)count;
            seg.row(p, kDepStart)[D] = (int32_t)dep_lds;
        }
    }
}

// One block: home_start = exclusive scan of the home counts; every domain's
// slot cursor starts at its home count; no entries yet.
__global__ __launch_bounds__(kBT) void k_home_start(const int32_t *__restrict__ n_home,
                                                    int32_t nd, int32_t *__restrict__ home_start,
                                                    int32_t *__restrict__ cur,
                                                    int32_t *__restrict__ count)
{
    uint32_t carry = 0;
    for (int32_t b = 0; b < nd; b += kBT) {
        const int32_t d = b + (int32_t)threadIdx.x;
        const uint32_t v = d < nd ? (uint32_t)n_home[d] : 0u;
        uint32_t tot;
        const uint32_t ex = block_scan_excl(v, tot);
        if (d < nd) {
            home_start[d] = (int32_t)(carry + ex);
            cur[d] = (int32_t)v;
        }
        carry += tot;
    }
    if (threadIdx.x == 0) count[0] = 0;
}

// One block, between the two selection passes of pulse p: the map offsets of
// the pulse's segments (pulse-major, then domain, after all earlier entries),
// and every receiver's region: recvSize = its sender's count, atomOffset =
// the receiver's slot count so far (each domain receives from exactly one
// sender per pulse, so the cursor updates do not collide).
__global__ __launch_bounds__(kBT) void k_pulse_scan(SegTable seg, int32_t p, int32_t nd,
                                                    const int32_t *__restrict__ send_to,
                                                    int32_t *__restrict__ cur,
                                                    int32_t *__restrict__ count)
{
    const int32_t base = count[0];
    uint32_t carry = 0;
    for (int32_t b = 0; b < nd; b += kBT) {
        const int32_t D = b + (int32_t)threadIdx.x;
        const uint32_t v = D < nd ? (uint32_t)seg.row(p, kSendSize)[D] : 0u;
        uint32_t tot;
        const uint32_t ex = block_scan_excl(v, tot);
        if (D < nd) {
            seg.row(p, kMapOff)[D] = base + (int32_t)(carry + ex);
            const int32_t R = send_to[p * nd + D];
            seg.row(p, kRecvSize)[R] = (int32_t)v;
            seg.row(p, kAtomOffset)[R] = cur[R];
            cur[R] += (int32_t)v;
        }
        carry += tot;
    }
    __syncthreads();  // every thread has read count[0]
    if (threadIdx.x == 0) count[0] = base + (int32_t)carry;
}

// Block = segment (pulse-major): absolute slots of its indexMap entries. The
// blocks of pulse 0 also give the home slots of their domain its id as their
// origin (home domain), when `origin` is not null.
__global__ __launch_bounds__(kBT) void k_abs_map(const int32_t *__restrict__ local_map,
                                                 SegTable seg, int32_t n_dom,
                                                 const int64_t *__restrict__ base,
                                                 int32_t *__restrict__ abs_map,
                                                 const int32_t *__restrict__ n_home,
                                                 int32_t *__restrict__ origin)
{
    const int32_t s = blockIdx.x;
    const int32_t p = s / n_dom, D = s % n_dom;
    const int32_t m0 = seg.row(p, kMapOff)[D], n = seg.row(p, kSendSize)[D];
    const int64_t b = base[D];
    for (int32_t i = threadIdx.x; i < n; i += kBT) abs_map[m0 + i] = (int32_t)(b + local_map[m0 + i]);
    if (origin && p == 0)
        for (int32_t i = threadIdx.x; i < n_home[D]; i += kBT) origin[b + i] = D;
}

__global__ __launch_bounds__(kBT) void k_home_slot(const int32_t *__restrict__ owner,
                                                   const int32_t *__restrict__ home_rank,
                                                   const int64_t *__restrict__ base,
                                                   int64_t n_atoms, int64_t *__restrict__ slot)
{
    const int64_t a = (int64_t)blockIdx.x * kBT + threadIdx.x;
    if (a < n_atoms) slot[a] = base[owner[a]] + home_rank[a];
}

// Bit p on the slots sent in pulse p (entries [e0, e1)). A slot appears at
// most once per pulse, and pulses run as separate launches.
__global__ __launch_bounds__(kBT) void k_mask(const int32_t *__restrict__ abs_map, int32_t e0,
                                              int32_t e1, int32_t p, uint8_t *__restrict__ mask)
{
    const int32_t e = e0 + (int32_t)(blockIdx.x * kBT + threadIdx.x);
    if (e < e1) {
        const int32_t s = abs_map[e];
        mask[s] = (uint8_t)(mask[s] | (1u << p));
    }
}

// Block = work item: the pulses whose regions its dependent entries read
// (coordinate direction) and, for the atomic force exchange, the later pulses
// q whose segment (q, receiver) has targets in the region the item reads.
__global__ __launch_bounds__(kBT) void k_item_masks(WorkItem *__restrict__ items,
                                                    const int32_t *__restrict__ local_map,
                                                    SegTable seg, int32_t n_dom,
                                                    int32_t n_pulse)
{
    __shared__ uint32_t xm;
    WorkItem *it = items + blockIdx.x;
    const int32_t s = it->seg, p = s / n_dom, D = s % n_dom, R = it->receiver;
    if (threadIdx.x == 0) xm = 0;
    __syncthreads();
    uint32_t mine = 0;
    for (int32_t i = it->n_indep + (int32_t)threadIdx.x; i < it->n_total; i += kBT) {
        const int32_t slot = local_map[it->map_begin + i];
        for (int32_t r = 0; r < p; ++r) {
            const int32_t lo = seg.row(r, kAtomOffset)[D];
            if (slot >= lo && slot < lo + seg.row(r, kRecvSize)[D]) {
                mine |= 1u << r;
                break;
            }
        }
    }
    if (mine) atomicOr(&xm, mine);
    // the item's sources: R's region of pulse p
    const int32_t lo = seg.row(p, kAtomOffset)[R];
    const int32_t hi = lo + seg.row(p, kRecvSize)[R];
    uint32_t am = 0;
    const int32_t q = p + 1 + (int32_t)threadIdx.x;
    if (q < n_pulse && lo < hi) {
        const int32_t *m = local_map + seg.row(q, kMapOff)[R];
        int32_t a = 0, b = seg.row(q, kSendSize)[R];
        while (a < b) {  // first entry >= lo
            const int32_t mid = a + (b - a) / 2;
            if (m[mid] < lo)
                a = mid + 1;
            else
                b = mid;
        }
        if (a < seg.row(q, kSendSize)[R] && m[a] < hi) am = 1u << q;
    }
    __shared__ uint32_t amask;
    if (threadIdx.x == 0) amask = 0;
    __syncthreads();
    if (am) atomicOr(&amask, am);
    __syncthreads();
    if (threadIdx.x == 0) {
        it->xwait_mask = xm;
        it->await_mask = amask;
    }
}

// Block = chunk candidate: union of its slots' masks and the number of slots
// with each pulse bit.
__global__ __launch_bounds__(kBT) void k_piece_stats(const Piece *__restrict__ pieces,
                                                     const uint8_t *__restrict__ mask,
                                                     int32_t n_pulse,
                                                     PieceStats *__restrict__ stats)
{
    constexpr int kRows = 8;  // slots per thread and round (a piece holds at most 8 * kBT)
    __shared__ uint32_t um;
    __shared__ int32_t cnt[kMaxMaskPulses];
    if (threadIdx.x == 0) um = 0;
    if (threadIdx.x < kMaxMaskPulses) cnt[threadIdx.x] = 0;
    __syncthreads();
    const Piece pc = pieces[blockIdx.x];
    // per wave: the union and the per-pulse counts, from ballots
    uint32_t u = 0;
    int32_t c[kMaxMaskPulses] = {0};
    for (int32_t i0 = 0; i0 < pc.count; i0 += kRows * kBT) {
        uint32_t m[kRows];
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            const int32_t i = i0 + j * kBT + (int32_t)threadIdx.x;
            m[j] = i < pc.count ? (uint32_t)mask[pc.first + i] : 0u;
        }
#pragma unroll
        for (int q = 0; q < kMaxMaskPulses; ++q) {
            if (q >= n_pulse) break;
#pragma unroll
            for (int j = 0; j < kRows; ++j) {
                const uint64_t bq = __ballot((m[j] >> q) & 1u);
                c[q] += __popcll(bq);
                if (bq) u |= 1u << q;
            }
        }
    }
    if ((threadIdx.x & 63) == 0) {
        if (u) atomicOr(&um, u);
#pragma unroll
        for (int q = 0; q < kMaxMaskPulses; ++q)
            if (c[q]) atomicAdd(&cnt[q], c[q]);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        stats[blockIdx.x].mask = um;
        for (int q = 0; q < kMaxMaskPulses; ++q) stats[blockIdx.x].count[q] = cnt[q];
    }
}

// ---- XCD-local units (plan.cpp, make_local_units, does the same on the host) ----

// Block = sender D of pulse p: the origins of the receiver's region of pulse p
// are those of the slots D sends (home slots or regions of earlier pulses,
// set by earlier launches).
__global__ __launch_bounds__(kBT) void k_origin_pulse(SegTable seg, int32_t p, int32_t n_dom,
                                                      const int32_t *__restrict__ send_to,
                                                      const int64_t *__restrict__ base,
                                                      const int32_t *__restrict__ abs_map,
                                                      int32_t *__restrict__ origin)
{
    const int32_t D = blockIdx.x;
    const int32_t m0 = seg.row(p, kMapOff)[D], n = seg.row(p, kSendSize)[D];
    const int32_t R = send_to[(size_t)p * n_dom + D];
    const int64_t dst = base[R] + seg.row(p, kAtomOffset)[R];
    for (int32_t i = threadIdx.x; i < n; i += kBT) origin[dst + i] = origin[abs_map[m0 + i]];
}

// Origin and zone (-1: home slots; q: the region of pulse q) of the source of
// entry i of segment (p, D), packed as origin * 64 + zone + 1.
__device__ __forceinline__ int32_t unit_key(SegTable seg, int32_t p, int32_t D, int32_t m0,
                                            int32_t i, const int32_t *__restrict__ local_map,
                                            const int32_t *__restrict__ abs_map,
                                            const int32_t *__restrict__ origin,
                                            const int32_t *__restrict__ n_home)
{
    const int32_t l = local_map[m0 + i];
    int32_t z = -1;
    if (l >= n_home[D])
        for (int32_t q = 0; q < p; ++q) {
            const int32_t lo = seg.row(q, kAtomOffset)[D];
            if (l >= lo && l < lo + seg.row(q, kRecvSize)[D]) z = q;
        }
    return origin[abs_map[m0 + i]] * 64 + z + 1;
}

// Block = segment (pulse-major): the first entry of every run of entries
// whose sources share origin and zone (in runs[m0 ...]), the run count, and
// the number of pieces of at most unit_entries entries the runs are cut into.
__global__ __launch_bounds__(kBT) void k_unit_runs(SegTable seg, int32_t n_dom,
                                                   const int32_t *__restrict__ local_map,
                                                   const int32_t *__restrict__ abs_map,
                                                   const int32_t *__restrict__ origin,
                                                   const int32_t *__restrict__ n_home,
                                                   int32_t unit_entries, int32_t *__restrict__ runs,
                                                   int32_t *__restrict__ seg_runs,
                                                   int32_t *__restrict__ seg_pieces)
{
    constexpr int kWaves = kBT / 64;
    __shared__ int32_t wave_n[kWaves];
    __shared__ int32_t carry;
    __shared__ int32_t keys[kBT + 1];  // keys[0]: the previous round's last key
    const int32_t s = blockIdx.x, p = s / n_dom, D = s % n_dom;
    const int32_t m0 = seg.row(p, kMapOff)[D], n = seg.row(p, kSendSize)[D];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (threadIdx.x == 0) {
        carry = 0;
        keys[0] = -1;  // no key is negative
    }
    __syncthreads();
    for (int32_t t0 = 0; t0 < n; t0 += kBT) {
        const int32_t i = t0 + (int32_t)threadIdx.x;
        // every entry's key once; a run starts where it differs from the one before
        const int32_t key =
            i < n ? unit_key(seg, p, D, m0, i, local_map, abs_map, origin, n_home) : -1;
        keys[threadIdx.x + 1] = key;
        __syncthreads();
        const bool brk = i < n && key != keys[threadIdx.x];
        const uint64_t b = __ballot(brk);
        if (lane == 0) wave_n[w] = __popcll(b);
        __syncthreads();
        int32_t at = carry;
        for (int k = 0; k < w; ++k) at += wave_n[k];
        at += (int32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        if (brk) runs[m0 + at] = i;  // at < n: one run start per entry at most
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int k = 0; k < kWaves; ++k) carry += wave_n[k];
            keys[0] = keys[kBT];
        }
        __syncthreads();
    }
    const int32_t n_runs = carry;
    int32_t pieces = 0;
    for (int32_t k = threadIdx.x; k < n_runs; k += kBT) {
        const int32_t a = runs[m0 + k], e = k + 1 < n_runs ? runs[m0 + k + 1] : n;
        pieces += (e - a + unit_entries - 1) / unit_entries;
    }
    __shared__ int32_t total;
    if (threadIdx.x == 0) total = 0;
    __syncthreads();
    if (pieces) atomicAdd(&total, pieces);
    __syncthreads();
    if (threadIdx.x == 0) {
        seg_runs[s] = n_runs;
        seg_pieces[s] = total;
    }
}

// One block: exclusive prefix of the segments' piece counts; the total at
// out[n_seg].
__global__ __launch_bounds__(kBT) void k_unit_scan(const int32_t *__restrict__ seg_pieces,
                                                   int32_t n_seg, int32_t *__restrict__ out)
{
    constexpr int kWaves = kBT / 64;
    __shared__ int32_t wave_sum[kWaves];
    __shared__ int32_t carry;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int32_t t0 = 0; t0 < n_seg; t0 += kBT) {
        const int32_t i = t0 + (int32_t)threadIdx.x;
        const int32_t v = i < n_seg ? seg_pieces[i] : 0;
        int32_t x = v;  // inclusive scan within the wave
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) wave_sum[w] = x;
        __syncthreads();
        int32_t at = carry;
        for (int k = 0; k < w; ++k) at += wave_sum[k];
        if (i < n_seg) out[i] = at + x - v;
        __syncthreads();
        if (threadIdx.x == 0)
            for (int k = 0; k < kWaves; ++k) carry += wave_sum[k];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[n_seg] = carry;
}

// Block = segment: its runs cut into near-equal pieces of at most
// unit_entries entries, written from out[piece_off[s]] on (pieces at or past
// `cap` are counted but not written).
__global__ __launch_bounds__(kBT) void k_unit_write(SegTable seg, int32_t n_dom,
                                                    const int32_t *__restrict__ local_map,
                                                    const int32_t *__restrict__ abs_map,
                                                    const int32_t *__restrict__ origin,
                                                    const int32_t *__restrict__ n_home,
                                                    int32_t unit_entries,
                                                    const int32_t *__restrict__ runs,
                                                    const int32_t *__restrict__ seg_runs,
                                                    const int32_t *__restrict__ piece_off,
                                                    int64_t cap, LocalRun *__restrict__ out)
{
    constexpr int kWaves = kBT / 64;
    __shared__ int32_t wave_sum[kWaves];
    __shared__ int32_t carry;
    const int32_t s = blockIdx.x, p = s / n_dom, D = s % n_dom;
    const int32_t m0 = seg.row(p, kMapOff)[D], n = seg.row(p, kSendSize)[D];
    const int32_t n_runs = seg_runs[s];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int32_t t0 = 0; t0 < n_runs; t0 += kBT) {
        const int32_t k = t0 + (int32_t)threadIdx.x;
        int32_t a = 0, len = 0, np_ = 0;
        if (k < n_runs) {
            a = runs[m0 + k];
            len = (k + 1 < n_runs ? runs[m0 + k + 1] : n) - a;
            np_ = (len + unit_entries - 1) / unit_entries;
        }
        int32_t x = np_;
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) wave_sum[w] = x;
        __syncthreads();
        int32_t at = carry;
        for (int c = 0; c < w; ++c) at += wave_sum[c];
        at += x - np_;
        if (np_ > 0) {
            const int32_t key = unit_key(seg, p, D, m0, a, local_map, abs_map, origin, n_home);
            for (int32_t j = 0; j < np_; ++j) {
                const int64_t o = (int64_t)piece_off[s] + at + j;
                if (o >= cap) break;
                const int32_t e0 = a + (int32_t)((int64_t)len * j / np_);
                const int32_t e1 = a + (int32_t)((int64_t)len * (j + 1) / np_);
                out[o] = LocalRun{p, D, e0, e1 - e0, (key & 63) - 1, key >> 6,
                                  abs_map[m0 + e0], abs_map[m0 + e1 - 1]};
            }
        }
        __syncthreads();
        if (threadIdx.x == 0)
            for (int c = 0; c < kWaves; ++c) carry += wave_sum[c];
        __syncthreads();
    }
}

unsigned grid_for(int64_t n, int per_block) { return (unsigned)((n + per_block - 1) / per_block); }

constexpr size_t kAlign = 256;

size_t aligned(size_t bytes) { return (bytes + kAlign - 1) & ~(kAlign - 1); }

// Make the arena hold at least `bytes` (contents are not kept; 1/8 slack so
// that rebuilds of a slightly larger system reuse it) and start carving from
// its beginning.
hipError_t arena_reserve(Arena &a, size_t bytes)
{
    a.used = 0;
    if (bytes <= a.cap && a.base) return hipSuccess;
    if (a.base) (void)hipFree(a.base);
    a.base = nullptr;
    a.cap = 0;
    const size_t want = std::max<size_t>(aligned(bytes + bytes / 8), kAlign);
    hipError_t e = hipMalloc((void **)&a.base, want);
    if (e == hipSuccess) a.cap = want;
    return e;
}

template <class T>
T *arena_take(Arena &a, size_t n)
{
    T *p = (T *)(a.base + a.used);
    a.used += aligned(std::max<size_t>(n, 1) * sizeof(T));
    return p;
}

void arena_free(Arena &a)
{
    if (a.base) (void)hipFree(a.base);
    a = Arena();
}

hipError_t pinned_reserve(DeviceBuild &B, size_t bytes)
{
    if (bytes <= B.pinned_cap && B.pinned) return hipSuccess;
    if (B.pinned) (void)hipHostFree(B.pinned);
    B.pinned = nullptr;
    B.pinned_cap = 0;
    const size_t want = std::max<size_t>(aligned(bytes + bytes / 8), kAlign);
    hipError_t e = hipHostMalloc((void **)&B.pinned, want, hipHostMallocDefault);
    if (e == hipSuccess) B.pinned_cap = want;
    return e;
}

// The entries arena holds the local-slot indexMap and the sent atoms'
// coordinates (three rows), `cap` entries each; its contents are not kept
// when it grows (the pulses then run again).
hipError_t entries_reserve(DeviceBuild &B, size_t need)
{
    if (need <= B.entry_cap && B.entries.base) return hipSuccess;
    const size_t cap = std::max<size_t>(need, B.entry_cap * 2);
    B.entry_cap = 0;
    hipError_t e = arena_reserve(B.entries, aligned(cap * 4) + 3 * cap * 4);
    if (e == hipSuccess) B.entry_cap = cap;
    return e;
}

// Wait for the work queued on `st` so far. The runtime's stream wait can
// sleep and take far longer to return than the GPU takes to finish short
// work; the build waits often for little, so it records an event and polls
// it instead.
// Bytes of the tables copy: items; seg_items, send_to, recv_from, dest_start,
// x_arrivals, zone_chunks; shift4; chunks; chunk order; launch members; the
// XCD-local units, their wait lists and their flags.
size_t tables_bytes(size_t n_items, size_t nseg, size_t npc, size_t n_lunits, size_t n_lwaits,
                    size_t lflag_words)
{
    return aligned(std::max<size_t>(n_items, 1) * sizeof(WorkItem)) +
           6 * aligned(std::max<size_t>(nseg, 1) * 4) + aligned(std::max<size_t>(nseg, 1) * 16) +
           aligned(std::max<size_t>(npc, 1) * sizeof(Chunk)) +
           aligned(std::max<size_t>(npc, 1) * 4) + aligned((size_t)kFamilies * kLaunchGroups * 4) +
           aligned(std::max<size_t>(n_lunits, 1) * sizeof(LocalUnit)) +
           aligned(std::max<size_t>(n_lwaits, 1) * 4) + aligned(std::max<size_t>(lflag_words, 1) * 8);
}

// Records ev (created on first use) at the stream's current end.
hipError_t record_event(hipEvent_t &ev, hipStream_t st)
{
    if (!ev) {
        const hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) {
            ev = nullptr;
            return e;
        }
    }
    return hipEventRecord(ev, st);
}

// Waits for a recorded event by polling it: the runtime's own wait could
// sleep far longer than the GPU needs.
hipError_t poll_event(hipEvent_t ev)
{
    hipError_t e;
    while ((e = hipEventQuery(ev)) == hipErrorNotReady) {
    }
    return e;
}

hipError_t wait_stream(DeviceBuild &B, hipStream_t st)
{
    const hipError_t e = record_event(B.done, st);
    return e != hipSuccess ? e : poll_event(B.done);
}

}  // namespace

void free_device_build(halo_plan *pl)
{
    if (!pl->dev) return;
    DeviceBuild &B = *pl->dev;
    for (Arena *a : {&B.work, &B.entries, &B.maps, &B.pieces, &B.tables, &B.units_more})
        arena_free(*a);
    if (B.pinned) (void)hipHostFree(B.pinned);
    if (B.done) (void)hipEventDestroy(B.done);
    if (B.units_back) (void)hipEventDestroy(B.units_back);
    if (B.stats_back) (void)hipEventDestroy(B.stats_back);
    delete pl->dev;
    pl->dev = nullptr;
    // these pointed into the arenas
    pl->d_idx = pl->d_local_map = pl->d_recv_from = pl->d_send_to = nullptr;
    pl->d_forder = pl->d_dest_start = nullptr;
    pl->d_home_slot = nullptr;
    pl->d_mask = nullptr;
    pl->d_items = nullptr;
    pl->d_seg_items = pl->d_x_arrivals = pl->d_zone_chunks = nullptr;
    pl->d_members = nullptr;
    pl->d_chunks = nullptr;
    pl->d_shift4 = nullptr;
    pl->d_lunits = nullptr;
    pl->d_lwaits = nullptr;
    pl->d_lflags = nullptr;
    pl->lflag_words = 0;
}

int build_plan_device(halo_plan *pl, const float *pos, int64_t n_atoms, const float *box,
                      const int32_t *grid, float cutoff, int32_t selection, int32_t item_entries,
                      hipStream_t st, std::string &msg)
{
    if (n_atoms < 0 || !box || !grid || (n_atoms > 0 && !pos)) {
        msg = "halo_plan_create_device: NULL pointer or negative atom count";
        return kErrArg;
    }
    HostPlan &P = pl->h;
    int rc = plan_geometry(n_atoms, box, grid, cutoff, selection, P, msg);
    if (rc != kOk) return rc;
    // the XCD-local units are made after the pulses
    P.has_local = false;
    P.local_k = 0;
    P.local_entries = 0;
    P.lunits.clear();
    P.lwaits.clear();
    if (P.n_dom > kMaxDeviceDomains) {
        msg = "halo_plan_create_device: at most " + std::to_string(kMaxDeviceDomains) +
              " domains (use halo_plan_create)";
        return kErrGeometry;
    }
    if (n_atoms > kMaxSlots) {
        msg = "halo_plan_create_device: too many atoms for one plan";
        return kErrRange;
    }
    if (!pl->dev) pl->dev = new DeviceBuild();
    DeviceBuild &B = *pl->dev;
    const int32_t nd = P.n_dom, np = P.n_pulse;
    const size_t nseg = (size_t)np * nd;
    Geom g;
    for (int d = 0; d < 3; ++d) {
        g.width[d] = P.width[d];
        g.top[d] = std::nextafter((double)grid[d], 0.0);
        g.box[d] = box[d];
        g.grid[d] = grid[d];
    }
    g.rc2 = (double)cutoff * (double)cutoff;
    g.corner = selection == kSelectCorner ? 1 : 0;
    hipError_t e = hipSuccess;
    auto hip_err = [&](const char *what) {
        msg = std::string("halo_plan_create_device: ") + what + ": " + hipGetErrorString(e);
        return kErrHip;
    };
#define HALO_TRY(call, what)            \
    do {                                \
        if ((e = (call)) != hipSuccess) \
            return hip_err(what);       \
    } while (0)

    // -- build temporaries in one arena ------------------------------------------
    // 2048-atom tiles once they still give every compute unit a tile (their
    // histogram is a quarter of the size: 8 us less on a million atoms), or
    // when the 512-atom tiles' histogram would pass kMaxTileCounters
    const bool small_tiles =
        (n_atoms + kTileLarge - 1) / kTileLarge < kComputeUnits &&
        (int64_t)nd * ((n_atoms + kTileSmall - 1) / kTileSmall) <= kMaxTileCounters;
    const int kTile = small_tiles ? kTileSmall : kTileLarge;
    const int32_t n_tiles = (int32_t)std::max<int64_t>(1, (n_atoms + kTile - 1) / kTile);
    const size_t N = (size_t)n_atoms;
    // summary read back once: first bad atom, entry count, home counts, cursors
    const size_t xfer_bytes = 16 + 8 * (size_t)nd;
    HALO_TRY(arena_reserve(B.work, 2 * aligned(std::max<size_t>(N, 1) * 4) +
                                       aligned(std::max<size_t>(N, 1) * 12) +
                                       aligned((size_t)nd * n_tiles * 4) + aligned(xfer_bytes) +
                                       aligned(4 * nd) + aligned(std::max<size_t>(nseg, 1) * 20) +
                                       aligned(std::max<size_t>(nseg, 1) * 8) + aligned(8 * nd)),
             "device memory");
    int32_t *owner = arena_take<int32_t>(B.work, N);
    int32_t *home_rank = arena_take<int32_t>(B.work, N);
    float *home_c = arena_take<float>(B.work, 3 * N);  // home coordinates, (x, y, z) per slot
    uint32_t *tile_hist = arena_take<uint32_t>(B.work, (size_t)nd * n_tiles);
    char *xfer = arena_take<char>(B.work, xfer_bytes);
    unsigned long long *bad = (unsigned long long *)xfer;
    int32_t *d_count = (int32_t *)(xfer + 8);
    int32_t *d_n_home = (int32_t *)(xfer + 16);
    int32_t *d_cur = d_n_home + nd;
    int32_t *d_home_start = arena_take<int32_t>(B.work, nd);
    SegTable sg{arena_take<int32_t>(B.work, nseg * kSegRows), nd};
    int32_t *w_send_to = arena_take<int32_t>(B.work, 2 * nseg);
    int32_t *w_recv_from = w_send_to + nseg;
    int64_t *d_base = arena_take<int64_t>(B.work, nd);

    // host staging: fixed part of the build
    const size_t h_sum = 0, h_seg = aligned(xfer_bytes),
                 h_tab = h_seg + aligned(std::max<size_t>(nseg, 1) * 20),
                 h_base = h_tab + aligned(8 * std::max<size_t>(nseg, 1)),
                 h_fixed = h_base + aligned(8 * (size_t)nd);
    HALO_TRY(pinned_reserve(B, h_fixed), "pinned host memory");
    char *hp = B.pinned;
    std::memcpy(hp + h_tab, P.send_to.data(), nseg * 4);
    std::memcpy(hp + h_tab + nseg * 4, P.recv_from.data(), nseg * 4);
    if (nseg > 0)
        HALO_TRY(hipMemcpyAsync(w_send_to, hp + h_tab, 2 * nseg * 4, hipMemcpyHostToDevice, st),
                 "hipMemcpyAsync");

    // -- domains and home order ------------------------------------------------
    HALO_TRY(hipMemsetAsync(bad, 0xff, 8, st), "hipMemsetAsync");
    const size_t lds = (size_t)nd * sizeof(uint32_t);
    if (n_atoms > 0 && small_tiles)
        k_owner<kTileSmall>
            <<<n_tiles, kBT, lds, st>>>(pos, n_atoms, g, nd, n_tiles, owner, tile_hist, bad);
    else if (n_atoms > 0)
        k_owner<kTileLarge>
            <<<n_tiles, kBT, lds, st>>>(pos, n_atoms, g, nd, n_tiles, owner, tile_hist, bad);
    else
        HALO_TRY(hipMemsetAsync(tile_hist, 0, (size_t)nd * n_tiles * 4, st), "hipMemsetAsync");
    k_tile_scan<<<nd, kBT, 0, st>>>(tile_hist, n_tiles, d_n_home);
    k_home_start<<<1, kBT, 0, st>>>(d_n_home, nd, d_home_start, d_cur, d_count);
    if (n_atoms > 0 && small_tiles)
        k_home_scatter<kTileSmall><<<n_tiles, kBT, lds, st>>>(owner, n_atoms, nd, n_tiles,
                                                              tile_hist, d_home_start, pos,
                                                              home_c, home_rank);
    else if (n_atoms > 0)
        k_home_scatter<kTileLarge><<<n_tiles, kBT, lds, st>>>(owner, n_atoms, nd, n_tiles,
                                                              tile_hist, d_home_start, pos,
                                                              home_c, home_rank);
    HALO_TRY(hipGetLastError(), "launch");

    // -- pulses, all on the device; one read-back at the end -------------------------
    // Room for the entries: what the previous build used, else the halo
    // volume expected at uniform density, with a margin. If a pulse does not
    // fit, the pulses run again with the count that came back.
    size_t want = std::max<size_t>(1024, 2 * N);
    {
        double vol = 1.0;
        for (int d = 0; d < 3; ++d)
            if (grid[d] > 1) vol *= 1.0 + P.reach[d];
        want = std::max(want, (size_t)((vol - 1.0) * 1.25 * (double)N) + 1024);
    }
    HALO_TRY(entries_reserve(B, want), "device memory");
    int64_t entries = 0;
    for (int attempt = 0;; ++attempt) {
        const int32_t cap = (int32_t)std::min<size_t>(B.entry_cap, (size_t)INT32_MAX);
        int32_t *lmap = (int32_t *)B.entries.base;
        float *ecoord = (float *)(B.entries.base + aligned(B.entry_cap * 4));
        if (attempt > 0) k_home_start<<<1, kBT, 0, st>>>(d_n_home, nd, d_home_start, d_cur, d_count);
        for (int32_t p = 0; p < np; ++p) {
            const int dim = P.pulse_dim[p];
            const int32_t k = P.pulse_k[p];
            k_select<false><<<nd, kSelectThreads, 0, st>>>(p, dim, k, nd, g, P.reach[dim], w_send_to,
                                                w_recv_from, d_n_home, d_home_start, home_c,
                                                n_atoms, sg, ecoord, lmap, cap);
            k_pulse_scan<<<1, kBT, 0, st>>>(sg, p, nd, w_send_to, d_cur, d_count);
            k_select<true><<<nd, kSelectThreads, 0, st>>>(p, dim, k, nd, g, P.reach[dim], w_send_to,
                                               w_recv_from, d_n_home, d_home_start, home_c,
                                               n_atoms, sg, ecoord, lmap, cap);
        }
        HALO_TRY(hipGetLastError(), "launch");
        HALO_TRY(hipMemcpyAsync(hp + h_sum, xfer, xfer_bytes, hipMemcpyDeviceToHost, st),
                 "hipMemcpyAsync");
        if (nseg > 0)
            HALO_TRY(hipMemcpyAsync(hp + h_seg, sg.t, nseg * kSegRows * 4, hipMemcpyDeviceToHost,
                                    st), "hipMemcpyAsync");
        HALO_TRY(wait_stream(B, st), "waiting for the stream");
        unsigned long long first_bad;
        std::memcpy(&first_bad, hp + h_sum, 8);
        if (first_bad != ~0ull) {
            msg = "halo_plan_create: atom " + std::to_string(first_bad) +
                  " lies outside [0, L) or is not finite";
            return kErrRange;
        }
        int32_t count;
        std::memcpy(&count, hp + h_sum + 8, 4);
        entries = (uint32_t)count;
        if (entries > kMaxSlots) {
            msg = "halo_plan_create_device: too many halo entries for one plan";
            return kErrRange;
        }
        if ((size_t)entries <= B.entry_cap) break;
        if (attempt > 0) {
            msg = "halo_plan_create_device: internal error: entry count not stable";
            return kErrArg;
        }
        HALO_TRY(entries_reserve(B, (size_t)entries), "device memory");
    }
    P.n_home.assign(nd, 0);
    std::memcpy(P.n_home.data(), hp + h_sum + 16, 4 * (size_t)nd);
    std::vector<int32_t> cur(nd);
    std::memcpy(cur.data(), hp + h_sum + 16 + 4 * (size_t)nd, 4 * (size_t)nd);
    {
        int64_t acc = 0;
        for (int32_t d = 0; d < nd; ++d) acc += P.n_home[d];
        if (acc != n_atoms) {
            msg = "halo_plan_create_device: internal error: home counts do not add up";
            return kErrArg;
        }
    }
    P.seg.assign(nseg, Segment());
    {
        const int32_t *t = (const int32_t *)(hp + h_seg);
        for (int32_t p = 0; p < np; ++p) {
            const int dim = P.pulse_dim[p];
            const int32_t *row = t + (size_t)p * kSegRows * nd;
            for (int32_t D = 0; D < nd; ++D) {
                Segment &s = P.seg[(size_t)p * nd + D];
                s.send_to = P.send_to[(size_t)p * nd + D];
                s.recv_from = P.recv_from[(size_t)p * nd + D];
                s.send_size = row[kSendSize * nd + D];
                s.dep_start = row[kDepStart * nd + D];
                s.recv_size = row[kRecvSize * nd + D];
                s.atom_offset = row[kAtomOffset * nd + D];
                s.map_off = row[kMapOff * nd + D];
                const int32_t cd = dim == 0   ? D % grid[0]
                                   : dim == 1 ? (D / grid[0]) % grid[1]
                                              : D / (grid[0] * grid[1]);
                s.shift[0] = s.shift[1] = s.shift[2] = 0.f;
                if (cd == 0) s.shift[dim] = box[dim];
            }
        }
    }
    int32_t *local_map = (int32_t *)B.entries.base;

    // -- layout, then everything the host derives from the sizes -----------------------
    P.base.assign(nd, 0);
    P.n_halo.assign(nd, 0);
    int64_t acc = 0;
    for (int32_t d = 0; d < nd; ++d) {
        P.base[d] = acc;
        P.n_halo[d] = cur[d] - P.n_home[d];
        acc += cur[d];
    }
    P.total_slots = acc;
    if (acc > kMaxSlots) {
        msg = "halo_plan_create: more than " + std::to_string((long long)kMaxSlots) +
              " slots (2 GiB of float triples) in one plan";
        return kErrRange;
    }
    P.n_entries = entries;
    P.has_chunks = plan_has_chunks(P);
    if (!P.has_chunks) {  // a rebuild may have left those of the previous plan
        P.chunks.clear();
        P.chunk_forder.clear();
        P.slot_mask.clear();
    }
    P.chunk_slots = item_entries;
    const int32_t unit_entries = local_unit_entries(P.n_entries, item_entries);
    const std::vector<Piece> pieces =
        P.has_chunks ? chunk_pieces(P, item_entries) : std::vector<Piece>();
    const size_t npc = pieces.size();
    // the work items are cut while the GPU runs; until then, a bound on
    // their count (a segment's two spans give at most ceil(n / U) items each,
    // an empty segment one)
    const size_t items_bound = (size_t)(entries / unit_entries) + 3 * nseg + 1;
    // host staging for the rest: base, pieces, their statistics, the pieces
    // of the XCD-local units (their count, then at most lr_cap of them; a
    // plan with more fetches them again), then the tables
    int64_t lr_cap = std::max<int64_t>(
        1, std::min<int64_t>(entries, entries / unit_entries + 4 * (int64_t)nseg + 1024));
    if (const char *v = std::getenv("HALO_UNIT_PIECES_CAP")) {
        // testing: a smaller first copy, so that the second fetch runs
        const long c = std::strtol(v, nullptr, 10);
        if (c >= 1) lr_cap = std::min<int64_t>(lr_cap, c);
    }
    // the tables are staged from the buffer's start once the rest has been
    // read: room for them too, with an estimate of the units' part (about
    // one unit position per piece)
    const size_t tab_est = tables_bytes(items_bound, nseg, npc, (size_t)lr_cap, (size_t)lr_cap * 4,
                                        2 * (size_t)kXcdClasses *
                                            local_flag_stride((int32_t)(lr_cap / 8 + 1)));
    const size_t h_pieces = h_fixed, h_stats = h_pieces + aligned(std::max<size_t>(npc, 1) * 16),
                 h_lruns = h_stats + aligned(std::max<size_t>(npc, 1) * sizeof(PieceStats)),
                 h_total = std::max(h_lruns + aligned(16 + (size_t)lr_cap * sizeof(LocalRun)),
                                    tab_est);
    if (h_total > B.pinned_cap) {
        HALO_TRY(wait_stream(B, st), "waiting for the stream");  // no copy from it in flight
        char *keep = (char *)std::malloc(h_fixed);
        if (!keep) {
            msg = "halo_plan_create_device: out of host memory";
            return kErrNoMem;
        }
        std::memcpy(keep, B.pinned, h_fixed);
        e = pinned_reserve(B, h_total);
        if (e == hipSuccess) std::memcpy(B.pinned, keep, h_fixed);
        std::free(keep);
        if (e != hipSuccess) return hip_err("pinned host memory");
        hp = B.pinned;
    }
    std::memcpy(hp + h_base, P.base.data(), 8 * (size_t)nd);
    HALO_TRY(hipMemcpyAsync(d_base, hp + h_base, 8 * (size_t)nd, hipMemcpyHostToDevice, st),
             "hipMemcpyAsync");

    // -- maps: absolute indexMap, home slots, pulse masks ------------------------------
    const size_t S = (size_t)P.total_slots;
    // (then the XCD-local units' temporaries: slot origins, runs, pieces)
    const size_t units_tmp = entries > 0 ? aligned(S * 4) + aligned((size_t)entries * 4) +
                                               3 * aligned(nseg * 4 + 4) +
                                               aligned((size_t)lr_cap * sizeof(LocalRun))
                                         : 0;
    HALO_TRY(arena_reserve(B.maps, aligned(std::max<int64_t>(entries, 1) * 4) +
                                       aligned(std::max<size_t>(N, 1) * 8) +
                                       (P.has_chunks ? aligned(S) : 0) + units_tmp),
             "device memory");
    int32_t *abs_map = arena_take<int32_t>(B.maps, (size_t)entries);
    int64_t *home_slot = arena_take<int64_t>(B.maps, N);
    uint8_t *mask = P.has_chunks ? arena_take<uint8_t>(B.maps, S) : nullptr;
    // XCD-local units: the origin of every slot (home slots with the absolute
    // indexMap, then pulse by pulse); per segment the runs of one origin and
    // zone and their pieces; the pieces come back while the host works
    int32_t *origin = entries > 0 ? arena_take<int32_t>(B.maps, S) : nullptr;
    if (nseg > 0)
        k_abs_map<<<(unsigned)nseg, kBT, 0, st>>>(local_map, sg, nd, d_base, abs_map, d_n_home,
                                                  origin);
    if (n_atoms > 0)
        k_home_slot<<<grid_for(n_atoms, kBT), kBT, 0, st>>>(owner, home_rank, d_base, n_atoms,
                                                            home_slot);
    HALO_TRY(hipGetLastError(), "launch");
    int32_t *u_origin = nullptr, *u_runs = nullptr, *u_seg_runs = nullptr, *u_piece_off = nullptr;
    if (entries > 0) {
        int32_t *runs = arena_take<int32_t>(B.maps, (size_t)entries);
        int32_t *seg_runs = arena_take<int32_t>(B.maps, nseg + 1);
        int32_t *seg_pieces = arena_take<int32_t>(B.maps, nseg + 1);
        int32_t *piece_off = arena_take<int32_t>(B.maps, nseg + 1);
        LocalRun *lruns = arena_take<LocalRun>(B.maps, (size_t)lr_cap);
        u_origin = origin;
        u_runs = runs;
        u_seg_runs = seg_runs;
        u_piece_off = piece_off;
        for (int32_t p = 0; p < np; ++p)
            k_origin_pulse<<<(unsigned)nd, kBT, 0, st>>>(sg, p, nd, w_send_to, d_base, abs_map,
                                                         origin);
        k_unit_runs<<<(unsigned)nseg, kBT, 0, st>>>(sg, nd, local_map, abs_map, origin, d_n_home,
                                                    unit_entries, runs, seg_runs, seg_pieces);
        k_unit_scan<<<1, kBT, 0, st>>>(seg_pieces, (int32_t)nseg, piece_off);
        k_unit_write<<<(unsigned)nseg, kBT, 0, st>>>(sg, nd, local_map, abs_map, origin,
                                                     d_n_home, unit_entries, runs, seg_runs,
                                                     piece_off, lr_cap, lruns);
        HALO_TRY(hipGetLastError(), "launch");
        HALO_TRY(hipMemcpyAsync(hp + h_lruns, piece_off + nseg, 4, hipMemcpyDeviceToHost, st),
                 "hipMemcpyAsync");
        HALO_TRY(hipMemcpyAsync(hp + h_lruns + 16, lruns, (size_t)lr_cap * sizeof(LocalRun),
                                hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
        HALO_TRY(record_event(B.units_back, st), "hipEventRecord");
    }
    std::vector<PieceStats> stats(npc);
    if (P.has_chunks) {
        HALO_TRY(hipMemsetAsync(mask, 0, S, st), "hipMemsetAsync");
        for (int32_t p = 0; p < np; ++p) {
            const int32_t e0 = (int32_t)P.at(p, 0).map_off;
            const int32_t e1 = p + 1 < np ? (int32_t)P.at(p + 1, 0).map_off : (int32_t)entries;
            if (e1 > e0) k_mask<<<grid_for(e1 - e0, kBT), kBT, 0, st>>>(abs_map, e0, e1, p, mask);
        }
        if (npc > 0) {
            HALO_TRY(arena_reserve(B.pieces, aligned(npc * sizeof(Piece)) +
                                                 aligned(npc * sizeof(PieceStats))),
                     "device memory");
            Piece *d_pieces = arena_take<Piece>(B.pieces, npc);
            PieceStats *d_stats = arena_take<PieceStats>(B.pieces, npc);
            std::memcpy(hp + h_pieces, pieces.data(), npc * sizeof(Piece));
            HALO_TRY(hipMemcpyAsync(d_pieces, hp + h_pieces, npc * sizeof(Piece),
                                    hipMemcpyHostToDevice, st), "hipMemcpyAsync");
            k_piece_stats<<<(unsigned)npc, kBT, 0, st>>>(d_pieces, mask, np, d_stats);
            HALO_TRY(hipGetLastError(), "launch");
            HALO_TRY(hipMemcpyAsync(hp + h_stats, d_stats, npc * sizeof(PieceStats),
                                    hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
            // the last work queued before the host's wait: recorded now, so
            // that a wait on a stream that has long finished costs no new marker
            HALO_TRY(record_event(B.stats_back, st), "hipEventRecord");
        }
    }

    // Host work while the GPU runs: the work items, then the XCD-local
    // units, placed as soon as their pieces are back (unless the first copy
    // was too short; the second fetch comes after the chunk statistics)
    make_items(P, unit_entries, false);
    const size_t n_items = P.items.size();
    int32_t n_lr = 0;
    bool units_placed = false;
    if (entries > 0) {
        HALO_TRY(poll_event(B.units_back), "waiting for the stream");
        std::memcpy(&n_lr, hp + h_lruns, 4);
        if (n_lr < 1 || n_lr > entries) {
            (void)wait_stream(B, st);  // no copy into the staging buffer left in flight
            msg = "halo_plan_create_device: internal error: unit count";
            return kErrArg;
        }
        if (n_lr <= lr_cap) {
            std::vector<LocalRun> lr((size_t)n_lr);
            std::memcpy(lr.data(), hp + h_lruns + 16, (size_t)n_lr * sizeof(LocalRun));
            place_local_units(P, lr);
            units_placed = true;
        }
    }
    // the launch-count members of the items and units, still before the wait
    if (units_placed || entries == 0) launch_members_items_units(P);
    if (P.has_chunks) {
        HALO_TRY(npc > 0 ? poll_event(B.stats_back) : wait_stream(B, st), "waiting for the stream");
        std::memcpy(stats.data(), hp + h_stats, npc * sizeof(PieceStats));
        try {
            finish_chunks(P, item_entries, pieces, stats);
        } catch (const std::exception &ex) {
            msg = std::string("halo_plan_create_device: internal error: ") + ex.what();
            return kErrArg;
        }
    }
    if (entries > 0 && !units_placed) {
        // more pieces than the first copy held: write them again, all of
        // them, into an arena of their own, and fetch them
        std::vector<LocalRun> lr((size_t)n_lr);
        HALO_TRY(arena_reserve(B.units_more, (size_t)n_lr * sizeof(LocalRun)), "device memory");
        LocalRun *more = arena_take<LocalRun>(B.units_more, (size_t)n_lr);
        k_unit_write<<<(unsigned)nseg, kBT, 0, st>>>(sg, nd, local_map, abs_map, u_origin, d_n_home,
                                                     unit_entries, u_runs, u_seg_runs, u_piece_off,
                                                     n_lr, more);
        HALO_TRY(hipGetLastError(), "launch");
        // no copy into the staging buffer is in flight here: it may be regrown
        HALO_TRY(pinned_reserve(B, (size_t)n_lr * sizeof(LocalRun)), "pinned host memory");
        hp = B.pinned;
        HALO_TRY(hipMemcpyAsync(hp, more, (size_t)n_lr * sizeof(LocalRun), hipMemcpyDeviceToHost,
                                st), "hipMemcpyAsync");
        HALO_TRY(wait_stream(B, st), "waiting for the stream");
        std::memcpy(lr.data(), hp, (size_t)n_lr * sizeof(LocalRun));
        place_local_units(P, lr);
        launch_members_items_units(P);
    }
    launch_members_chunks(P);

    // -- tables: items, segment tables, chunks, XCD-local units and their
    // (cleared) flags; one copy -------------------------------------------------------
    // items; seg_items, send_to, recv_from, dest_start, x_arrivals, zone_chunks;
    // shift4; chunks; chunk order; launch members; units, wait lists, flags
    const size_t n_lunits = P.lunits.size(), n_lwaits = P.lwaits.size();
    const size_t lflag_words =
        P.has_local ? 2 * (size_t)kXcdClasses * local_flag_stride(P.local_k) : 0;
    const size_t tab_bytes = tables_bytes(n_items, nseg, npc, n_lunits, n_lwaits, lflag_words);
    // nothing is in flight from the staging buffer here: it may be regrown
    HALO_TRY(pinned_reserve(B, tab_bytes), "pinned host memory");
    hp = B.pinned;
    HALO_TRY(arena_reserve(B.tables, tab_bytes), "device memory");
    char *tp = hp;
    size_t off = 0;
    auto put = [&](const void *src, size_t bytes, size_t reserve_bytes) {
        if (bytes) std::memcpy(tp + off, src, bytes);
        void *dst = B.tables.base + off;
        off += aligned(std::max<size_t>(reserve_bytes, 1));
        return dst;
    };
    const size_t ns4 = std::max<size_t>(nseg, 1) * 4;
    WorkItem *items = (WorkItem *)put(P.items.data(), n_items * sizeof(WorkItem),
                                      n_items * sizeof(WorkItem));
    uint32_t *seg_items = (uint32_t *)put(P.seg_items.data(), nseg * 4, ns4);
    int32_t *send_to = (int32_t *)put(P.send_to.data(), nseg * 4, ns4);
    int32_t *recv_from = (int32_t *)put(P.recv_from.data(), nseg * 4, ns4);
    uint32_t *members = (uint32_t *)put(P.launch_members.data(), P.launch_members.size() * 4,
                                        P.launch_members.size() * 4);
    Chunk *chunks = nullptr;
    int32_t *forder = nullptr, *dest_start = nullptr;
    float *shift4 = nullptr;
    uint32_t *x_arrivals = nullptr, *zone_chunks = nullptr;
    if (P.has_chunks) {
        const size_t nc = P.chunks.size();
        chunks = (Chunk *)put(P.chunks.data(), nc * sizeof(Chunk), npc * sizeof(Chunk));
        forder = (int32_t *)put(P.chunk_forder.data(), nc * 4, npc * 4);
        dest_start = (int32_t *)put(P.dest_start.data(), nseg * 4, ns4);
        shift4 = (float *)put(P.shift4.data(), nseg * 16, std::max<size_t>(nseg, 1) * 16);
        x_arrivals = (uint32_t *)put(P.x_arrivals.data(), nseg * 4, ns4);
        zone_chunks = (uint32_t *)put(P.zone_chunks.data(), nseg * 4, ns4);
    }
    LocalUnit *lunits = nullptr;
    int32_t *lwaits = nullptr;
    uint64_t *lflags = nullptr;
    if (P.has_local) {
        lunits = (LocalUnit *)put(P.lunits.data(), n_lunits * sizeof(LocalUnit),
                                  n_lunits * sizeof(LocalUnit));
        lwaits = (int32_t *)put(P.lwaits.data(), n_lwaits * 4, n_lwaits * 4);
        std::memset(tp + off, 0, lflag_words * 8);
        lflags = (uint64_t *)put(nullptr, 0, lflag_words * 8);
    }
    if (off > tab_bytes) {
        msg = "halo_plan_create_device: internal error: table layout";
        return kErrArg;
    }
    HALO_TRY(hipMemcpyAsync(B.tables.base, tp, off, hipMemcpyHostToDevice, st), "hipMemcpyAsync");
    if (n_items > 0) {
        k_item_masks<<<(unsigned)n_items, kBT, 0, st>>>(items, local_map, sg, nd, np);
        HALO_TRY(hipGetLastError(), "launch");
    }
    if (P.has_chunks && !P.chunks.empty())
        HALO_TRY(plan_chunk_rows(pl, mask, chunks, st), "the chunks' row table");

    // -- counters and the error word --------------------------------------------------------
    const size_t words = state_words_for(nseg);
    if (pl->d_state && pl->state_words != words) {
        (void)hipFree(pl->d_state);
        pl->d_state = nullptr;
    }
    if (!pl->d_state) HALO_TRY(hipMalloc((void **)&pl->d_state, words * 4), "device memory");
    pl->state_words = words;
    HALO_TRY(hipMemsetAsync(pl->d_state, 0, words * 4, st), "hipMemsetAsync");
    if (!pl->h_err) {
        HALO_TRY(hipHostMalloc((void **)&pl->h_err, 64, hipHostMallocMapped), "pinned memory");
        HALO_TRY(hipHostGetDevicePointer((void **)&pl->d_err, pl->h_err, 0), "pinned memory");
    }
    HALO_TRY(wait_stream(B, st), "waiting for the stream");
    std::memset(pl->h_err, 0, 64);
    HALO_TRY(hipGetDevice(&pl->device), "hipGetDevice");

    pl->d_idx = abs_map;
    pl->d_local_map = local_map;
    pl->d_home_slot = home_slot;
    pl->d_mask = mask;
    pl->d_items = items;
    pl->d_seg_items = seg_items;
    pl->d_send_to = send_to;
    pl->d_recv_from = recv_from;
    pl->d_chunks = chunks;
    pl->d_forder = forder;
    pl->d_dest_start = dest_start;
    pl->d_shift4 = shift4;
    pl->d_x_arrivals = x_arrivals;
    pl->d_zone_chunks = zone_chunks;
    pl->d_members = members;
    pl->d_lunits = lunits;
    pl->d_lwaits = lwaits;
    pl->d_lflags = lflags;
    pl->lflag_words = lflag_words;
    pl->epochs.reset();
    pl->poisoned = false;
    pl->built_on_device = true;
    pl->uploaded = true;
#undef HALO_TRY
    return kOk;
}

}  // namespace halo
