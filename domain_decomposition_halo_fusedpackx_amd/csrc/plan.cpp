// plan.cpp -- build the exchange plan on the host.
//
// Method: "Redesigning GROMACS Halo Exchange" (paper review), s.3 "GROMACS
// domain decomposition halo exchange" (domains own home atoms; atoms within
// the cutoff are forwarded through intermediate domains in pulses along z,
// then y, then x), Algorithm 1 (PulseData) and Algorithm 4 (depOffset).
//
// Choices where the pages are silent (also stated in include/halo.h):
// pulses per dimension ceil(cutoff / w); data flows to the lower neighbour
// with +L on a periodic wrap; an atom is sent when its original position,
// in units of w and in double precision, lies less than cutoff / w above the
// receiver's upper face (with the corner selection also when its Euclidean
// distance to the receiver's box is below the cutoff); home atoms in
// ascending id; indexMap ascending;
// slots of a domain = [home | region per pulse], domains in id order.
//
// The build runs the pulses on index lists only (no coordinates are moved):
// every pulse first lets each domain pick its sends from its slots as they
// were before the pulse, then appends each pick to the receiver. Domains are
// independent within each phase, so both phases run in parallel.
#include "plan.hpp"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <limits>
#include <cstdlib>
#include <stdexcept>
#include <thread>

namespace halo {
namespace {

template <class F>
void parallel_for(int32_t n, F &&fn)
{
    unsigned hw = std::thread::hardware_concurrency();
    int32_t workers = (int32_t)std::min<unsigned>(hw ? hw : 1, 16);
    workers = std::min(workers, std::max<int32_t>(1, n / 4));
    if (workers <= 1) {
        for (int32_t i = 0; i < n; ++i) fn(i);
        return;
    }
    std::atomic<int32_t> next{0};
    std::vector<std::thread> pool;
    pool.reserve(workers);
    for (int32_t w = 0; w < workers; ++w)
        pool.emplace_back([&] {
            for (int32_t i = next.fetch_add(1); i < n; i = next.fetch_add(1)) fn(i);
        });
    for (auto &t : pool) t.join();
}

}  // namespace

// XCD-aware item order (on by default; HALO_XCD_ORDER=0 turns it off for
// comparisons).
bool xcd_ordering_enabled()
{
    const char *v = std::getenv("HALO_XCD_ORDER");
    return !(v && v[0] == '0');
}

namespace {

struct Cell3 {
    int32_t c[3];
};

inline Cell3 cell_of_domain(const int32_t *grid, int32_t id)
{
    Cell3 r;
    r.c[0] = id % grid[0];
    r.c[1] = (id / grid[0]) % grid[1];
    r.c[2] = id / (grid[0] * grid[1]);
    return r;
}

inline int32_t domain_of_cell(const int32_t *grid, const int32_t *c)
{
    return c[0] + grid[0] * (c[1] + grid[1] * c[2]);
}

}  // namespace

int plan_geometry(int64_t n_atoms, const float *box, const int32_t *grid, float cutoff,
                  int32_t selection, HostPlan &P, std::string &msg)
{
    P = HostPlan();
    P.n_atoms = n_atoms;
    P.cutoff = cutoff;
    if (selection != kSelectSlab && selection != kSelectCorner) {
        msg = "halo_plan_create: selection must be HALO_SELECT_SLAB or HALO_SELECT_CORNER";
        return kErrArg;
    }
    P.selection = selection;
    for (int d = 0; d < 3; ++d) {
        P.box[d] = box[d];
        P.grid[d] = grid[d];
        if (!(box[d] > 0.f) || !std::isfinite(box[d]) || grid[d] < 1) {
            msg = "halo_plan_create: box lengths must be finite and > 0, grid counts >= 1";
            return kErrGeometry;
        }
    }
    if (!(cutoff > 0.f) || !std::isfinite(cutoff)) {
        msg = "halo_plan_create: cutoff must be finite and > 0";
        return kErrGeometry;
    }
    for (int d = 0; d < 3; ++d) {
        P.width[d] = (double)box[d] / (double)grid[d];
        P.reach[d] = (double)cutoff / P.width[d];
        P.pulses_in[d] = 0;
        if (grid[d] > 1) {
            double np = std::ceil(P.reach[d]);
            if (np > (double)(grid[d] - 1)) {
                msg = "halo_plan_create: cutoff needs " + std::to_string((long long)np) +
                      " pulses in dimension " + std::to_string(d) + " but the grid allows only " +
                      std::to_string(grid[d] - 1);
                return kErrGeometry;
            }
            P.pulses_in[d] = (int32_t)np;
        }
    }
    int64_t nd = (int64_t)grid[0] * grid[1] * grid[2];
    if (nd > std::numeric_limits<int32_t>::max() / 64) {
        msg = "halo_plan_create: too many domains";
        return kErrGeometry;
    }
    P.n_dom = (int32_t)nd;
    for (int dim = 2; dim >= 0; --dim)
        for (int32_t k = 0; k < P.pulses_in[dim]; ++k) {
            P.pulse_dim.push_back(dim);
            P.pulse_k.push_back(k);
        }
    P.n_pulse = (int32_t)P.pulse_dim.size();
    if (P.n_pulse > kMaxPulses) {
        msg = "halo_plan_create: the cutoff needs " + std::to_string(P.n_pulse) +
              " pulses; at most " + std::to_string(kMaxPulses) + " are supported";
        return kErrGeometry;
    }
    // Receiver and sender of every (pulse, domain): data flows to the lower
    // neighbour along the pulse's dimension, periodically.
    P.send_to.assign((size_t)P.n_pulse * P.n_dom, 0);
    P.recv_from.assign((size_t)P.n_pulse * P.n_dom, 0);
    for (int32_t p = 0; p < P.n_pulse; ++p) {
        const int dim = P.pulse_dim[p];
        for (int32_t D = 0; D < P.n_dom; ++D) {
            Cell3 cd = cell_of_domain(grid, D);
            int32_t cr[3] = {cd.c[0], cd.c[1], cd.c[2]};
            cr[dim] = cd.c[dim] == 0 ? grid[dim] - 1 : cd.c[dim] - 1;
            const int32_t R = domain_of_cell(grid, cr);
            P.send_to[(size_t)p * P.n_dom + D] = R;
            P.recv_from[(size_t)p * P.n_dom + R] = D;
        }
    }
    return kOk;
}

int build_plan(const float *pos, int64_t n_atoms, const float *box, const int32_t *grid,
               float cutoff, int32_t selection, int32_t item_entries, HostPlan &P,
               std::string &msg)
{
    if (n_atoms < 0 || !box || !grid || (n_atoms > 0 && !pos)) {
        msg = "halo_plan_create: NULL pointer or negative atom count";
        return kErrArg;
    }
    int rc = plan_geometry(n_atoms, box, grid, cutoff, selection, P, msg);
    if (rc != kOk) return rc;

    // Atoms in blocks of kBlock, processed in parallel. Per block: the range
    // check (the first bad atom of the lowest block is reported, as a serial
    // scan would), the owner, and the block's count per domain.
    constexpr int64_t kBlock = 1 << 15;
    const int32_t n_blocks = (int32_t)((n_atoms + kBlock - 1) / kBlock);
    std::vector<int32_t> owner((size_t)n_atoms);
    std::vector<int64_t> bad(n_blocks, -1);
    std::vector<int32_t> block_count((size_t)n_blocks * P.n_dom, 0);
    // Position in units of the domain width; a rounding up to n is pulled
    // back below n so that the cell index stays in range.
    double top[3];
    for (int d = 0; d < 3; ++d) top[d] = std::nextafter((double)grid[d], 0.0);
    auto scaled = [&](float v, int d) {
        const double t = (double)v / P.width[d];
        return t > top[d] ? top[d] : t;
    };
    {
        parallel_for(n_blocks, [&](int32_t b) {
            const int64_t a0 = (int64_t)b * kBlock, a1 = std::min(n_atoms, a0 + kBlock);
            int32_t *cnt = &block_count[(size_t)b * P.n_dom];
            for (int64_t a = a0; a < a1; ++a) {
                int32_t c[3];
                for (int d = 0; d < 3; ++d) {
                    const float v = pos[3 * a + d];
                    if (!std::isfinite(v) || !(v >= 0.f) || !(v < box[d])) {
                        bad[b] = a;
                        return;
                    }
                    c[d] = (int32_t)std::floor(scaled(v, d));
                }
                owner[a] = domain_of_cell(grid, c);
                cnt[owner[a]] += 1;
            }
        });
    }
    for (int32_t b = 0; b < n_blocks; ++b)
        if (bad[b] >= 0) {
            msg = "halo_plan_create: atom " + std::to_string((long long)bad[b]) +
                  " lies outside [0, L) or is not finite";
            return kErrRange;
        }
    const bool corner = selection == kSelectCorner;
    const double rc2 = (double)cutoff * (double)cutoff;

    // Home atoms by stable counting sort: ascending id within each domain.
    // Every slot also carries its atom's position (slot_pos), so that the
    // pulses read their candidates' positions in slot order.
    std::vector<std::vector<int64_t>> slot_atom(P.n_dom);
    std::vector<std::vector<float>> slot_pos(P.n_dom);
    P.n_home.assign(P.n_dom, 0);
    for (int32_t b = 0; b < n_blocks; ++b)
        for (int32_t d = 0; d < P.n_dom; ++d) {
            int32_t &c = block_count[(size_t)b * P.n_dom + d];
            const int32_t start = P.n_home[d];
            P.n_home[d] += c;
            c = start;  // now the block's first slot in domain d
        }
    for (int32_t d = 0; d < P.n_dom; ++d) {
        slot_atom[d].reserve((size_t)P.n_home[d] * 2 + 8);
        slot_atom[d].resize((size_t)P.n_home[d]);
        slot_pos[d].reserve(((size_t)P.n_home[d] * 2 + 8) * 3);
        slot_pos[d].resize((size_t)P.n_home[d] * 3);
    }
    parallel_for(n_blocks, [&](int32_t b) {
        const int64_t a0 = (int64_t)b * kBlock, a1 = std::min(n_atoms, a0 + kBlock);
        int32_t *next = &block_count[(size_t)b * P.n_dom];
        for (int64_t a = a0; a < a1; ++a) {
            const int32_t d = owner[a];
            const int32_t sl = next[d]++;
            slot_atom[d][sl] = a;
            for (int k = 0; k < 3; ++k) slot_pos[d][3 * (size_t)sl + k] = pos[3 * a + k];
        }
    });

    // Pulses.
    P.seg.assign((size_t)P.n_pulse * P.n_dom, Segment());
    std::vector<std::vector<int32_t>> picks((size_t)P.n_pulse * P.n_dom);
    std::vector<std::vector<int64_t>> moving(P.n_dom);
    std::vector<std::vector<float>> moving_pos(P.n_dom);
    for (int32_t p = 0; p < P.n_pulse; ++p) {
        const int dim = P.pulse_dim[p];
        const int32_t k = P.pulse_k[p];
        const int32_t n = grid[dim];
        const double reach = P.reach[dim];
        Segment *row = &P.seg[(size_t)p * P.n_dom];
        std::vector<int32_t> *prow = &picks[(size_t)p * P.n_dom];

        // Phase 1 reads only the sender's own slots.
        parallel_for(P.n_dom, [&](int32_t D) {
            Cell3 cd = cell_of_domain(grid, D);
            Segment &s = row[D];
            s.send_to = P.send_to[(size_t)p * P.n_dom + D];
            const Cell3 cr = cell_of_domain(grid, s.send_to);
            const int32_t c_recv = cr.c[dim];
            s.shift[0] = s.shift[1] = s.shift[2] = 0.f;
            if (cd.c[dim] == 0) s.shift[dim] = box[dim];
            // Candidate slots: all of them on the first pulse of a dimension,
            // otherwise only what arrived in the previous pulse.
            int32_t first = 0, last = (int32_t)slot_atom[D].size();
            if (k > 0) {
                const Segment &prev = P.seg[(size_t)(p - 1) * P.n_dom + D];
                first = prev.atom_offset;
                last = prev.atom_offset + prev.recv_size;
            }
            const double face = (double)(c_recv + 1);
            // Appends go to local vectors, handed over at the end: the
            // shared arrays of vectors would have neighbouring domains'
            // headers, written by other threads, in one cache line.
            std::vector<int32_t> out;
            std::vector<int64_t> mv;
            std::vector<float> mp;
            out.reserve((size_t)(last - first));
            mv.reserve((size_t)(last - first));
            mp.reserve((size_t)(last - first) * 3);
            const std::vector<int64_t> &sa = slot_atom[D];
            const float *sp = slot_pos[D].data();
            for (int32_t slot = first; slot < last; ++slot) {
                const float *ps = sp + 3 * (size_t)slot;
                double above = scaled(ps[dim], dim) - face;
                if (above < 0.0) above += (double)n;
                bool send = above < reach;
                if (send && corner) {
                    const double t[3] = {scaled(ps[0], 0), scaled(ps[1], 1), scaled(ps[2], 2)};
                    // squared distance to the receiver's box, x + y + z in
                    // this order; dimensions where the atom lies in the
                    // receiver's slab add nothing
                    double dist2 = 0.0;
                    for (int d = 0; d < 3; ++d) {
                        double delta = 0.0;
                        if (d == dim || (int32_t)std::floor(t[d]) != cr.c[d]) {
                            delta = t[d] - (double)(cr.c[d] + 1);
                            if (delta < 0.0) delta += (double)grid[d];
                        }
                        const double dist = delta * P.width[d];
                        dist2 += dist * dist;
                    }
                    send = dist2 < rc2;
                }
                if (send) {
                    out.push_back(slot);
                    mv.push_back(sa[slot]);
                    mp.insert(mp.end(), ps, ps + 3);
                }
            }
            s.send_size = (int32_t)out.size();
            s.dep_start = (int32_t)(std::lower_bound(out.begin(), out.end(), P.n_home[D]) -
                                    out.begin());
            prow[D] = std::move(out);
            moving[D] = std::move(mv);
            moving_pos[D] = std::move(mp);
        });

        // Phase 2 writes only the receiver's slots; each receiver has exactly
        // one sender per pulse.
        parallel_for(P.n_dom, [&](int32_t D) {
            const Segment &s = row[D];
            Segment &r = row[s.send_to];
            std::vector<int64_t> &dst = slot_atom[s.send_to];
            r.recv_from = D;
            r.recv_size = s.send_size;
            r.atom_offset = (int32_t)dst.size();
            dst.insert(dst.end(), moving[D].begin(), moving[D].end());
            std::vector<float> &dst_p = slot_pos[s.send_to];
            dst_p.insert(dst_p.end(), moving_pos[D].begin(), moving_pos[D].end());
        });
    }

    // Layout.
    P.base.assign(P.n_dom, 0);
    P.n_halo.assign(P.n_dom, 0);
    int64_t acc = 0;
    for (int32_t d = 0; d < P.n_dom; ++d) {
        P.base[d] = acc;
        P.n_halo[d] = (int32_t)slot_atom[d].size() - P.n_home[d];
        acc += (int64_t)slot_atom[d].size();
    }
    P.total_slots = acc;
    if (acc > kMaxSlots) {
        msg = "halo_plan_create: more than " + std::to_string((long long)kMaxSlots) +
              " slots (2 GiB of float triples) in one plan";
        return kErrRange;
    }
    P.home_slot.assign((size_t)n_atoms, 0);
    parallel_for(P.n_dom, [&](int32_t d) {  // each atom is a home atom of one domain
        for (int32_t s = 0; s < P.n_home[d]; ++s) P.home_slot[slot_atom[d][s]] = P.base[d] + s;
    });

    // Concatenated indexMap, pulse-major then domain.
    int64_t entries = 0;
    for (auto &s : P.seg) {
        s.map_off = entries;
        entries += s.send_size;
    }
    P.n_entries = entries;
    P.local_map.resize((size_t)entries);
    P.abs_map.resize((size_t)entries);

    parallel_for(P.n_pulse * P.n_dom, [&](int32_t sg) {
        const Segment &s = P.seg[(size_t)sg];
        const int32_t D = sg % P.n_dom;
        const std::vector<int32_t> &pk = picks[(size_t)sg];
        for (int32_t i = 0; i < s.send_size; ++i) {
            P.local_map[s.map_off + i] = pk[i];
            P.abs_map[s.map_off + i] = (int32_t)(P.base[D] + pk[i]);
        }
    });
    // work items and XCD-local units take the plan-sized bound; the
    // transposed runs keep item_entries
    const int32_t unit_entries = local_unit_entries(P.n_entries, item_entries);
    make_items(P, unit_entries);
    make_chunks(P, item_entries);
    make_local_units(P, unit_entries);
    make_launch_members(P);
    return kOk;
}

// The members of each launch-count group: exactly the units for which the
// kernel of the family executes a wait (the conditions below mirror the
// kernels').
static inline void add_member(HostPlan &P, int family, size_t unit)
{
    P.launch_members[(size_t)family * kLaunchGroups + unit % kLaunchGroups] += 1u;
}

void make_launch_members(HostPlan &P)
{
    launch_members_items_units(P);
    launch_members_chunks(P);
}

void launch_members_items_units(HostPlan &P)
{
    P.launch_members.assign((size_t)kFamilies * kLaunchGroups, 0u);
    auto add = [&](int family, size_t unit) { add_member(P, family, unit); };
    for (size_t u = 0; u < P.items.size(); ++u) {
        const WorkItem &it = P.items[u];
        if (it.n_total > it.n_indep) add(kFamItemsX, u);
        if (it.fwait[0] >= 0) add(kFamItemsF, u);
        add(kFamAtomicF, u);
    }
    // The XCD-local index-list kernels: a unit that waits, or that writes a
    // flag another unit waits for, takes part (in a replayed graph it reads
    // the count to learn the epoch).
    for (size_t b = 0; b < P.lunits.size(); ++b) {
        const LocalUnit &un = P.lunits[b];
        if (un.wx_n > 0 || (un.flags & kLocalXWaited)) add(kFamLocalX, b);
        if (un.wf_n > 0 || (un.flags & kLocalFWaited)) add(kFamLocalF, b);
    }
}

void launch_members_chunks(HostPlan &P)
{
    if (!P.has_chunks) return;
    auto add = [&](int family, size_t unit) { add_member(P, family, unit); };
    for (size_t u = 0; u < P.chunks.size(); ++u) {
        const Chunk &c = P.chunks[u];
        if (c.zone >= 0) add(kFamChunksX, u);
        bool waits = false;
        for (int32_t p = 0; p < P.n_pulse; ++p) {
            if (!((c.mask >> p) & 1u)) continue;
            const int32_t R = P.send_to[(size_t)p * P.n_dom + c.domain];
            if (P.zone_chunks[(size_t)p * P.n_dom + R] > 0) waits = true;
        }
        if (waits) add(kFamChunksF, u);
    }
}

// Reorder the items of one pulse so that the items of domain D sit at
// positions whose index is D mod 8 (mod 8) where possible. Workgroups of a
// grid go to the 8 XCDs of an MI355X round-robin, so all pulses of a domain
// then run on one XCD and re-read its home slots from that XCD's L2. Items of
// one pulse never wait on each other, so any order within a pulse is valid.
static void xcd_order(std::vector<WorkItem> &items, size_t begin, int32_t n_dom)
{
    constexpr int kXcds = 8;
    const size_t n = items.size() - begin;
    if (n == 0) return;
    // stable buckets by XCD (domain mod 8), as index lists over a copy
    thread_local std::vector<WorkItem> copy;
    thread_local std::vector<uint32_t> order;
    copy.assign(items.begin() + (std::ptrdiff_t)begin, items.end());
    order.resize(n);
    size_t off[kXcds + 1] = {0}, head[kXcds], end[kXcds];
    for (const WorkItem &it : copy) ++off[(it.seg % n_dom) % kXcds + 1];
    for (int c = 0; c < kXcds; ++c) {
        off[c + 1] += off[c];
        head[c] = off[c];
        end[c] = off[c];
    }
    for (size_t i = 0; i < n; ++i) order[end[(copy[i].seg % n_dom) % kXcds]++] = (uint32_t)i;
    for (size_t k = 0; k < n; ++k) {
        int want = (int)((begin + k) % kXcds);
        if (head[want] == end[want]) {  // that XCD's bucket is empty: the fullest one
            size_t best = 0;
            for (int c = 0; c < kXcds; ++c)
                if (end[c] - head[c] > best) {
                    best = end[c] - head[c];
                    want = c;
                }
        }
        items[begin + k] = copy[order[head[want]++]];
    }
}

// Work items of the index-list kernels. Every segment (pulse p, sender D) is
// cut into items of at most item_entries entries, separately for its
// independent span (entries below depOffset) and its dependent span, and
// every segment has at least one item (its counter must advance). Launch
// order, which is also the dependency order: for every pulse the independent
// items, then the dependent ones; for the last pulse, whose completion nobody
// waits for, the dependent items come first and its independent bulk last,
// so that the forwarding chain meets less memory traffic.
// Force direction with atomic adds: the later pulses q whose segment (q, R)
// has targets in the region that segment (p, D) reads (R's region of pulse
// p, R the receiver). Only those write the item's sources during the launch.
static uint32_t atomic_force_waits(const HostPlan &P, int32_t p, int32_t D)
{
    uint32_t out = 0;
    const int32_t R = P.at(p, D).send_to;
    const Segment &rs = P.at(p, R);
    const int32_t lo = rs.atom_offset, hi = rs.atom_offset + rs.recv_size;
    if (lo == hi) return out;
    for (int32_t q = p + 1; q < P.n_pulse; ++q) {
        const Segment &w = P.at(q, R);
        const int32_t *m = P.local_map.data() + w.map_off;
        const int32_t *it = std::lower_bound(m, m + w.send_size, lo);
        if (it != m + w.send_size && *it < hi) out |= 1u << q;
    }
    return out;
}

static void cut_span(HostPlan &P, int32_t p, int32_t D, int32_t lo, int32_t hi,
                     int32_t item_entries, bool keep_empty, bool with_masks)
{
    Segment &s = P.seg[(size_t)p * P.n_dom + D];
    const Segment &rs = P.at(p, s.send_to);
    const int32_t len = hi - lo;
    int32_t n = (len + item_entries - 1) / item_entries;
    if (n == 0 && keep_empty) n = 1;
    const uint32_t aw = n > 0 && with_masks ? atomic_force_waits(P, p, D) : 0u;
    for (int32_t j = 0; j < n; ++j) {
        const int32_t b = lo + (int32_t)((int64_t)len * j / n);
        const int32_t e = lo + (int32_t)((int64_t)len * (j + 1) / n);
        WorkItem it{};
        it.map_begin = (int32_t)(s.map_off + b);
        it.n_total = e - b;
        it.n_indep = std::min(std::max(s.dep_start - b, 0), it.n_total);
        it.region_begin = (int32_t)(P.base[s.send_to] + rs.atom_offset + b);
        for (int c = 0; c < 3; ++c) it.shift[c] = s.shift[c];
        it.seg = p * P.n_dom + D;
        // Coordinate direction: wait for exactly the regions that the
        // dependent entries read (each was filled by one sender in an
        // earlier pulse).
        it.xwait_mask = 0;
        int32_t r = 0;
        for (int32_t i = b + it.n_indep; with_masks && i < e; ++i) {
            const int32_t slot = P.local_map[s.map_off + i];
            while (r < p && !(slot >= P.at(r, D).atom_offset &&
                              slot < P.at(r, D).atom_offset + P.at(r, D).recv_size))
                ++r;
            if (r < p) it.xwait_mask |= 1u << r;
        }
        it.domain = D;
        it.receiver = s.send_to;
        // Force direction: pulse p+1 finished for D and for its receiver.
        it.fwait[0] = it.fwait[1] = -1;
        if (p + 1 < P.n_pulse) {
            it.fwait[0] = (p + 1) * P.n_dom + D;
            it.fwait[1] = (p + 1) * P.n_dom + s.send_to;
        }
        it.await_mask = aw;
        // Regions of every pulse but the last are candidates of a later
        // pulse; in the force direction the last pulse runs first (reads
        // untouched slots) and pulse 0 runs last (its sums are read by nobody
        // in the same launch).
        it.flags = 0;
        if (p + 1 < P.n_pulse) it.flags |= kItemXStoreShared | kItemFLoadShared;
        if (p > 0) it.flags |= kItemFStoreShared;
        P.items.push_back(it);
        s.n_items += 1;
        P.seg_items[(size_t)p * P.n_dom + D] += 1;
    }
}

void make_items(HostPlan &P, int32_t item_entries, bool with_masks)
{
    P.item_entries = item_entries;
    P.items.clear();
    {
        size_t est = 0;
        for (const Segment &sg : P.seg)
            est += 2 + (size_t)(sg.send_size / std::max<int32_t>(item_entries, 1));
        P.items.reserve(est);
    }
    P.seg_items.assign(P.seg.size(), 0);
    P.pulse_item_off.assign(P.n_pulse + 1, 0);
    for (auto &s : P.seg) {
        s.n_items = 0;
        s.item_off = 0;
    }
    for (int32_t p = 0; p < P.n_pulse; ++p) {
        P.pulse_item_off[p] = (int32_t)P.items.size();
        const bool last = p + 1 == P.n_pulse;
        for (int pass = 0; pass < 2; ++pass) {
            const bool indep = (pass == 0) != last;
            const size_t group = P.items.size();
            for (int32_t D = 0; D < P.n_dom; ++D) {
                const Segment &s = P.seg[(size_t)p * P.n_dom + D];
                // an empty segment keeps one (empty) item in its first group
                const bool keep_empty = s.send_size == 0 && pass == 0;
                if (indep)
                    cut_span(P, p, D, 0, s.dep_start, item_entries, keep_empty, with_masks);
                else
                    cut_span(P, p, D, s.dep_start, s.send_size, item_entries, keep_empty,
                             with_masks);
            }
            if (xcd_ordering_enabled()) xcd_order(P.items, group, P.n_dom);
        }
    }
    P.pulse_item_off[P.n_pulse] = (int32_t)P.items.size();
}

// A unit's entries are one stage of the forwarding chain for that stretch:
// smaller units start their dependants sooner and run fewer entries per
// thread, larger ones cost fewer waits and workgroups. Measured over the five
// workloads, about two units per compute unit is where the two balance (the
// chip has 256 compute units).
int32_t local_unit_entries(int64_t n_entries, int32_t item_entries)
{
    int32_t u = 1024;
    while (u > 128 && (int64_t)u * 512 > n_entries) u /= 2;
    return std::max<int32_t>(1, std::min(u, item_entries));
}

// XCD-local units. A unit is a run of consecutive entries of one indexMap
// (pulse p, sender D) whose source slots lie in one zone of D (its home
// slots or the region it received in one pulse) and hold atoms of one home
// domain, the run's origin; runs longer than unit_entries are cut into
// near-equal pieces. All images of an atom in one domain arrive by the same
// path, so each origin occupies one contiguous stretch of one zone.
//
// Dependencies, all among units of one origin:
//  - coordinates (Algorithm 4): a unit reading region q of D waits for the
//    units of segment (q, sender to D) that wrote the stretch it reads;
//  - forces (Algorithm 6, pulses in reverse): a unit of pulse p adds its
//    receiver's region slots onto its source slots, so it waits for every
//    unit of a later pulse that adds into those region slots (they must be
//    final) or into its own source slots (their adds come first).
// Placement: the units of origin o form class o mod kXcdClasses; a class
// lists its units pulse by pulse (roots, which read home slots, before the
// others; in the last pulse the others first, as the index-list items),
// and the k-th unit of class c sits at position 8k + c. Unused positions
// hold empty units. A unit then waits only for units of its own class at
// smaller positions (coordinates) or larger positions (forces, launched in
// reverse).
void make_local_units(HostPlan &P, int32_t unit_entries)
{
    P.has_local = false;
    P.local_k = 0;
    P.local_entries = 0;
    P.lunits.clear();
    P.lwaits.clear();
    if (P.n_pulse == 0 || P.n_entries == 0 || P.total_slots == 0) return;
    const int32_t nd = P.n_dom, np = P.n_pulse;
    unit_entries = std::max<int32_t>(unit_entries, 1);

    // origin of every slot, pulse by pulse (the senders of one pulse write
    // disjoint regions)
    std::vector<int32_t> origin((size_t)P.total_slots, -1);
    parallel_for(nd, [&](int32_t D) {
        for (int32_t l = 0; l < P.n_home[D]; ++l) origin[(size_t)(P.base[D] + l)] = D;
    });
    for (int32_t p = 0; p < np; ++p)
        parallel_for(nd, [&](int32_t D) {
            const Segment &g = P.at(p, D);
            const int64_t dst = P.base[g.send_to] + P.at(p, g.send_to).atom_offset;
            for (int32_t i = 0; i < g.send_size; ++i)
                origin[(size_t)(dst + i)] = origin[(size_t)P.abs_map[(size_t)g.map_off + i]];
        });

    // per segment: runs of one origin and zone, cut into pieces
    std::vector<std::vector<LocalRun>> per_seg((size_t)np * nd);
    parallel_for(np * nd, [&](int32_t sg) {
        const int32_t p = sg / nd, D = sg % nd;
        const Segment &g = P.at(p, D);
        auto zone_of = [&](int32_t l) {
            if (l < P.n_home[D]) return -1;
            for (int32_t q = 0; q < np; ++q) {
                const Segment &r = P.at(q, D);
                if (l >= r.atom_offset && l < r.atom_offset + r.recv_size) return q;
            }
            return np;  // not reached: every local slot is home or in a region
        };
        std::vector<LocalRun> &out = per_seg[(size_t)sg];
        int32_t i = 0;
        while (i < g.send_size) {
            const int32_t l0 = P.local_map[(size_t)g.map_off + i];
            const int32_t z = zone_of(l0);
            const int32_t o = origin[(size_t)(P.base[D] + l0)];
            int32_t j = i + 1;
            while (j < g.send_size) {
                const int32_t l = P.local_map[(size_t)g.map_off + j];
                if (origin[(size_t)(P.base[D] + l)] != o || zone_of(l) != z) break;
                ++j;
            }
            const int32_t len = j - i, pieces = (len + unit_entries - 1) / unit_entries;
            for (int32_t k = 0; k < pieces; ++k) {
                const int32_t a = i + (int32_t)((int64_t)len * k / pieces);
                const int32_t b = i + (int32_t)((int64_t)len * (k + 1) / pieces);
                out.push_back(LocalRun{p, D, a, b - a, z, o, P.abs_map[(size_t)g.map_off + a],
                                       P.abs_map[(size_t)g.map_off + b - 1]});
            }
            i = j;
        }
    });
    std::vector<LocalRun> raw;
    for (const auto &v : per_seg) raw.insert(raw.end(), v.begin(), v.end());
    place_local_units(P, raw);
}

void place_local_units(HostPlan &P, const std::vector<LocalRun> &raw)
{
    P.has_local = false;
    P.local_k = 0;
    P.local_entries = 0;
    P.lunits.clear();
    P.lwaits.clear();
    const int32_t nd = P.n_dom, np = P.n_pulse;
    // the pieces by (sending domain, pulse), each bucket in piece order
    const size_t n_raw = raw.size();
    std::vector<int32_t> bucket_off((size_t)nd * np + 1, 0), by_bucket(n_raw);
    for (const LocalRun &u : raw) ++bucket_off[(size_t)u.sender * np + u.pulse + 1];
    for (size_t k = 0; k + 1 < bucket_off.size(); ++k) bucket_off[k + 1] += bucket_off[k];
    {
        std::vector<int32_t> fill(bucket_off.begin(), bucket_off.end() - 1);
        for (int32_t r = 0; r < (int32_t)n_raw; ++r)
            by_bucket[(size_t)fill[(size_t)raw[r].sender * np + raw[r].pulse]++] = r;
    }
    // classes and positions: pulse by pulse, roots first (forwarders first in
    // the last pulse), pieces in order
    std::vector<int32_t> pulse_off((size_t)np + 1, 0), by_pulse(n_raw);
    for (const LocalRun &u : raw) ++pulse_off[(size_t)u.pulse + 1];
    for (int32_t p = 0; p < np; ++p) pulse_off[(size_t)p + 1] += pulse_off[(size_t)p];
    {
        std::vector<int32_t> fill(pulse_off.begin(), pulse_off.end() - 1);
        for (int32_t r = 0; r < (int32_t)n_raw; ++r) by_pulse[(size_t)fill[raw[r].pulse]++] = r;
    }
    std::vector<int32_t> cls_n(kXcdClasses, 0), pos_of(n_raw, -1);
    for (int32_t p = 0; p < np; ++p) {
        const bool last = p + 1 == np;
        for (int pass = 0; pass < 2; ++pass) {
            const bool roots = (pass == 0) != last;
            for (int32_t k = pulse_off[(size_t)p]; k < pulse_off[(size_t)p + 1]; ++k) {
                const int32_t r = by_pulse[(size_t)k];
                if ((raw[r].zone < 0) != roots) continue;
                const int c = raw[r].origin % kXcdClasses;
                pos_of[(size_t)r] = cls_n[c]++ * kXcdClasses + c;
            }
        }
    }
    int32_t k_max = 0;
    for (int c = 0; c < kXcdClasses; ++c) k_max = std::max(k_max, cls_n[c]);
    P.local_k = k_max;
    P.lunits.assign((size_t)k_max * kXcdClasses, LocalUnit{});

    // the pieces of sender D and pulse p
    auto bucket = [&](int32_t D, int32_t p) {
        return std::make_pair(by_bucket.data() + bucket_off[(size_t)D * np + p],
                              by_bucket.data() + bucket_off[(size_t)D * np + p + 1]);
    };
    P.lwaits.reserve(raw.size() * 4);
    for (int32_t r = 0; r < (int32_t)raw.size(); ++r) {
        const LocalRun &u = raw[r];
        const Segment &g = P.at(u.pulse, u.sender);
        LocalUnit &L = P.lunits[(size_t)pos_of[r]];
        L.map_begin = (int32_t)(g.map_off + u.e0);
        L.n_total = u.n;
        L.region_begin = (int32_t)(P.base[g.send_to] + P.at(u.pulse, g.send_to).atom_offset + u.e0);
        L.seg = u.pulse * nd + u.sender;
        for (int c = 0; c < 3; ++c) L.shift[c] = g.shift[c];
        L.origin = u.origin;
        // coordinates: the writers of the stretch of region `zone` it reads
        L.wx_off = (int32_t)P.lwaits.size();
        if (u.zone >= 0) {
            const int32_t q = u.zone, Dq = P.recv_from[(size_t)q * nd + u.sender];
            const int64_t r0 = P.base[u.sender] + P.at(q, u.sender).atom_offset;
            const int64_t i_lo = u.src_lo - r0, i_hi = u.src_hi - r0;
            for (auto [it, end] = bucket(Dq, q); it != end; ++it) {
                const LocalRun &w = raw[(size_t)*it];
                if (w.e0 <= i_hi && w.e0 + w.n - 1 >= i_lo) {
                    P.lwaits.push_back(pos_of[(size_t)*it]);
                    P.lunits[(size_t)pos_of[(size_t)*it]].flags |= kLocalXWaited;
                }
            }
        }
        L.wx_n = (int32_t)P.lwaits.size() - L.wx_off;
        // forces: later units adding into the region slots it reads or into
        // its own source slots
        L.wf_off = (int32_t)P.lwaits.size();
        const int64_t reg_lo = L.region_begin, reg_hi = reg_lo + u.n - 1;
        for (int32_t q = u.pulse + 1; q < np; ++q)
            for (auto [it, end] = bucket(g.send_to, q); it != end; ++it) {
                const LocalRun &w = raw[(size_t)*it];
                if (w.src_lo <= reg_hi && w.src_hi >= reg_lo) P.lwaits.push_back(pos_of[(size_t)*it]);
            }
        const size_t first_own = P.lwaits.size();
        for (int32_t q = u.pulse + 1; q < np; ++q)
            for (auto [it, end] = bucket(u.sender, q); it != end; ++it) {
                const LocalRun &w = raw[(size_t)*it];
                if (w.src_lo <= u.src_hi && w.src_hi >= u.src_lo &&
                    (g.send_to != u.sender ||
                     std::find(P.lwaits.begin() + L.wf_off,
                               P.lwaits.begin() + (ptrdiff_t)first_own,
                               pos_of[(size_t)*it]) == P.lwaits.begin() + (ptrdiff_t)first_own))
                    P.lwaits.push_back(pos_of[(size_t)*it]);
            }
        L.wf_n = (int32_t)P.lwaits.size() - L.wf_off;
        for (int32_t k = L.wf_off; k < L.wf_off + L.wf_n; ++k)
            P.lunits[(size_t)P.lwaits[(size_t)k]].flags |= kLocalFWaited;
    }
    for (const LocalUnit &u : P.lunits) P.local_entries = std::max(P.local_entries, u.n_total);
    P.has_local = true;
}

bool plan_has_chunks(const HostPlan &P)
{
    return P.n_pulse > 0 && P.n_pulse <= kMaxMaskPulses && P.total_slots > 0;
}

std::vector<Piece> chunk_pieces(const HostPlan &P, int32_t chunk_slots)
{
    std::vector<Piece> out;
    for (int32_t D = 0; D < P.n_dom; ++D)
        for (int32_t z = -1; z < P.n_pulse; ++z) {
            int32_t lo, hi;
            if (z < 0) {
                lo = 0;
                hi = P.n_home[D];
            } else {
                lo = P.at(z, D).atom_offset;
                hi = lo + P.at(z, D).recv_size;
            }
            const int32_t len = hi - lo;
            const int32_t pieces = len > 0 ? (len + chunk_slots - 1) / chunk_slots : 0;
            for (int32_t k = 0; k < pieces; ++k) {
                const int32_t a = lo + (int32_t)((int64_t)len * k / pieces);
                const int32_t b = lo + (int32_t)((int64_t)len * (k + 1) / pieces);
                out.push_back(Piece{(int32_t)(P.base[D] + a), b - a, D, z});
            }
        }
    return out;
}

void finish_chunks(HostPlan &P, int32_t chunk_slots, const std::vector<Piece> &pieces,
                   const std::vector<PieceStats> &stats)
{
    const int32_t nd = P.n_dom, np = P.n_pulse;
    P.chunk_slots = chunk_slots;
    P.dest_start.assign((size_t)np * nd, 0);
    P.shift4.assign((size_t)np * nd * 4, 0.f);
    P.x_arrivals.assign((size_t)np * nd, 0);
    P.zone_chunks.assign((size_t)np * nd, 0);
    for (int32_t p = 0; p < np; ++p)
        for (int32_t D = 0; D < nd; ++D) {
            const Segment &s = P.at(p, D);
            const Segment &r = P.at(p, s.send_to);
            P.dest_start[(size_t)p * nd + D] = (int32_t)(P.base[s.send_to] + r.atom_offset);
            for (int c = 0; c < 3; ++c) P.shift4[((size_t)p * nd + D) * 4 + c] = s.shift[c];
        }
    // Pieces come per domain in slot order (home, then the region of each
    // pulse); a chunk's rank[q] counts the bit-q slots of its domain before it.
    // Kept chunks are placed zone-major (stable within a zone): a first pass
    // counts them per zone, the second writes each at its place.
    // zone_first[z + 1] = first chunk of zone z (z = -1 .. np-1)
    std::vector<int32_t> zone_first(np + 2, 0);
    for (size_t i = 0; i < pieces.size(); ++i)
        if (stats[i].mask != 0) ++zone_first[pieces[i].zone + 2];
    for (int32_t z = 0; z <= np; ++z) zone_first[z + 1] += zone_first[z];
    P.chunks.resize((size_t)zone_first[np + 1]);
    std::vector<int32_t> fill(zone_first.begin(), zone_first.end() - 1);
    int32_t rank[kMaxMaskPulses] = {0};
    int32_t cur = -1;
    for (size_t i = 0; i < pieces.size(); ++i) {
        const Piece &pc = pieces[i];
        if (pc.domain != cur) {
            if (cur >= 0)
                for (int32_t q = 0; q < np; ++q)
                    if (rank[q] != P.at(q, cur).send_size)
                        throw std::logic_error("mask ranks disagree");
            cur = pc.domain;
            for (int32_t q = 0; q < kMaxMaskPulses; ++q) rank[q] = 0;
        }
        const uint32_t m = stats[i].mask;
        if (m != 0) {  // else nothing to send from or add into
            Chunk &c = P.chunks[(size_t)fill[pc.zone + 1]++];
            c.first = pc.first;
            c.count = pc.count;
            c.domain = pc.domain;
            c.zone = pc.zone;
            c.mask = m;
            c.xwait = pc.zone < 0 ? -1 : pc.zone * nd + P.at(pc.zone, pc.domain).recv_from;
            c.top_sends = np > 0 ? stats[i].count[np - 1] : 0;
            c.pad = 0;
            for (int32_t q = 0; q < kMaxMaskPulses; ++q) c.rank[q] = rank[q];
            for (int32_t q = 0; q < np; ++q)
                if ((m >> q) & 1u) P.x_arrivals[(size_t)q * nd + pc.domain] += 1;
            if (pc.zone >= 0) P.zone_chunks[(size_t)pc.zone * nd + pc.domain] += 1;
        }
        for (int32_t q = 0; q < np; ++q) rank[q] += stats[i].count[q];
    }
    if (cur >= 0)
        for (int32_t q = 0; q < np; ++q)
            if (rank[q] != P.at(q, cur).send_size) throw std::logic_error("mask ranks disagree");
    // Force direction: regions of later pulses first (their sums feed earlier
    // pulses), home slots last.
    P.chunk_forder.clear();
    P.chunk_forder.reserve(P.chunks.size());
    for (int32_t z = np; z >= 0; --z)
        for (int32_t i = zone_first[z]; i < zone_first[z + 1]; ++i) P.chunk_forder.push_back(i);
}

void make_chunks(HostPlan &P, int32_t chunk_slots)
{
    P.chunk_slots = chunk_slots;
    P.chunks.clear();
    P.chunk_forder.clear();
    P.has_chunks = plan_has_chunks(P);
    if (!P.has_chunks) return;
    P.slot_mask.assign((size_t)P.total_slots, 0);
    parallel_for(P.n_dom, [&](int32_t D) {  // a domain's indexMaps name its own slots
        for (int32_t p = 0; p < P.n_pulse; ++p) {
            const Segment &s = P.at(p, D);
            for (int32_t i = 0; i < s.send_size; ++i)
                P.slot_mask[(size_t)(P.base[D] + P.local_map[s.map_off + i])] |= (uint8_t)(1u << p);
        }
    });
    const std::vector<Piece> pieces = chunk_pieces(P, chunk_slots);
    std::vector<PieceStats> stats(pieces.size());
    parallel_for((int32_t)pieces.size(), [&](int32_t i) {
        PieceStats &st = stats[i];
        st.mask = 0;
        for (int32_t q = 0; q < kMaxMaskPulses; ++q) st.count[q] = 0;
        for (int32_t sl = pieces[i].first; sl < pieces[i].first + pieces[i].count; ++sl) {
            const uint32_t m = P.slot_mask[(size_t)sl];
            st.mask |= m;
            for (int32_t q = 0; q < P.n_pulse; ++q) st.count[q] += (int32_t)((m >> q) & 1u);
        }
    });
    finish_chunks(P, chunk_slots, pieces, stats);
}

}  // namespace halo
