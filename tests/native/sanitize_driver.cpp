// Host-code check under AddressSanitizer and UndefinedBehaviorSanitizer: the
// library's host plan builder (plan.cpp, items and chunks included) and the
// serial C oracle run on small boxes with both selection tests, and their
// PulseData are compared. Built
// and run by tests/test_host_sanitizers.py; exits non-zero on a mismatch, and
// the sanitizers abort on any memory or UB error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "plan.hpp"

extern "C" {
struct oracle;
int oracle_build_ex(const float *pos, int64_t n_atoms, const float *box, const int32_t *grid,
                    float cutoff, int32_t criterion, oracle **out);
void oracle_free(oracle *o);
int64_t oracle_total_slots(const oracle *o);
int oracle_pulse(const oracle *o, int32_t p, int32_t d, int32_t *send_to, int32_t *send_size,
                 int32_t *recv_from, int32_t *recv_size, int32_t *atom_offset,
                 int32_t *dep_start, float *shift, int32_t *index_map);
int oracle_exchange_x(const oracle *o, float *x);
int oracle_exchange_f(const oracle *o, float *f);
}

namespace {

// The XCD-local units of a host plan (plan.hpp, LocalUnit), checked against
// the plan's indexMaps entry by entry: every entry is in exactly one unit;
// a unit's atoms share one origin, whose class is the unit's position mod 8;
// every coordinate dependency (an entry reads a slot another entry wrote)
// and every force dependency (a later pulse adds into a slot the unit reads
// or adds into) is on the unit's wait list, on its own class, at a smaller
// (coordinates) or larger (forces) position; the flag bits mark exactly the
// units on some list. Returns the number of violations.
int check_local_units(const halo::HostPlan &P, int32_t unit_entries)
{
    if (!P.has_local) return P.n_entries > 0 && P.n_pulse > 0;
    int bad = 0;
    const int32_t nd = P.n_dom;
    const size_t nl = P.lunits.size();
    if (nl != (size_t)P.local_k * halo::kXcdClasses) return 1;
    // entry -> position
    std::vector<int32_t> unit_of((size_t)P.n_entries, -1);
    for (size_t b = 0; b < nl; ++b) {
        const halo::LocalUnit &u = P.lunits[b];
        if (u.n_total == 0) continue;
        if (u.n_total > unit_entries) ++bad;
        for (int32_t e = 0; e < u.n_total; ++e) {
            int32_t &o = unit_of[(size_t)u.map_begin + e];
            if (o != -1) ++bad;
            o = (int32_t)b;
        }
    }
    for (int32_t o : unit_of) bad += o < 0;
    // writer entry of every halo slot, and origins (recomputed here)
    std::vector<int64_t> writer((size_t)P.total_slots, -1);
    std::vector<int32_t> origin((size_t)P.total_slots, -1);
    for (int32_t D = 0; D < nd; ++D)
        for (int32_t l = 0; l < P.n_home[D]; ++l) origin[(size_t)(P.base[D] + l)] = D;
    for (int32_t p = 0; p < P.n_pulse; ++p)
        for (int32_t D = 0; D < nd; ++D) {
            const halo::Segment &g = P.at(p, D);
            const int64_t dst = P.base[g.send_to] + P.at(p, g.send_to).atom_offset;
            for (int32_t i = 0; i < g.send_size; ++i) {
                writer[(size_t)(dst + i)] = g.map_off + i;
                origin[(size_t)(dst + i)] = origin[(size_t)P.abs_map[(size_t)g.map_off + i]];
            }
        }
    auto on_list = [&](int32_t off, int32_t n, int32_t pos) {
        for (int32_t i = 0; i < n; ++i)
            if (P.lwaits[(size_t)off + i] == pos) return true;
        return false;
    };
    std::vector<char> xw(nl, 0), fw(nl, 0);
    for (size_t b = 0; b < nl; ++b) {
        const halo::LocalUnit &u = P.lunits[b];
        for (int32_t i = 0; i < u.wx_n; ++i) {
            const int32_t v = P.lwaits[(size_t)u.wx_off + i];
            xw[(size_t)v] = 1;
            bad += v >= (int32_t)b || v % 8 != (int32_t)b % 8;
        }
        for (int32_t i = 0; i < u.wf_n; ++i) {
            const int32_t v = P.lwaits[(size_t)u.wf_off + i];
            fw[(size_t)v] = 1;
            bad += v <= (int32_t)b || v % 8 != (int32_t)b % 8;
        }
    }
    for (size_t b = 0; b < nl; ++b) {
        const halo::LocalUnit &u = P.lunits[b];
        bad += ((u.flags & halo::kLocalXWaited) != 0) != (xw[b] != 0);
        bad += ((u.flags & halo::kLocalFWaited) != 0) != (fw[b] != 0);
    }
    // per entry: origin class, coordinate writer on the wait list
    std::vector<std::vector<int64_t>> readers((size_t)P.total_slots);
    std::vector<int32_t> pulse_of((size_t)P.n_entries);
    for (int32_t p = 0; p < P.n_pulse; ++p)
        for (int32_t D = 0; D < nd; ++D) {
            const halo::Segment &g = P.at(p, D);
            for (int32_t i = 0; i < g.send_size; ++i) pulse_of[(size_t)g.map_off + i] = p;
        }
    for (int64_t e = 0; e < P.n_entries; ++e) {
        const int32_t b = unit_of[(size_t)e];
        const halo::LocalUnit &u = P.lunits[(size_t)b];
        const int32_t src = P.abs_map[(size_t)e];
        bad += origin[(size_t)src] != u.origin || u.origin % 8 != b % 8;
        readers[(size_t)src].push_back(e);
        if (writer[(size_t)src] >= 0 &&
            !on_list(u.wx_off, u.wx_n, unit_of[(size_t)writer[(size_t)src]]))
            ++bad;
    }
    // forces: every later-pulse reader of the entry's source slot or of the
    // region slot it fills
    for (int32_t p = 0; p < P.n_pulse; ++p)
        for (int32_t D = 0; D < nd; ++D) {
            const halo::Segment &g = P.at(p, D);
            const int64_t dst = P.base[g.send_to] + P.at(p, g.send_to).atom_offset;
            for (int32_t i = 0; i < g.send_size; ++i) {
                const int64_t e = g.map_off + i;
                const halo::LocalUnit &u = P.lunits[(size_t)unit_of[(size_t)e]];
                for (int64_t slot : {(int64_t)P.abs_map[(size_t)e], dst + i})
                    for (int64_t r : readers[(size_t)slot])
                        if (pulse_of[(size_t)r] > p &&
                            !on_list(u.wf_off, u.wf_n, unit_of[(size_t)r]))
                            ++bad;
            }
        }
    return bad;
}

// splitmix64: reproducible positions without any library generator
uint64_t next(uint64_t &s)
{
    uint64_t z = (s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

struct Case {
    float box[3];
    int32_t grid[3];
    float cutoff;
    int64_t n;
};

int run(const Case &c, uint64_t seed, int32_t selection)
{
    std::vector<float> pos(3 * (size_t)c.n);
    uint64_t s = seed;
    for (int64_t a = 0; a < c.n; ++a)
        for (int d = 0; d < 3; ++d) {
            const double u = (double)(next(s) >> 11) * (1.0 / 9007199254740992.0);
            float v = (float)(u * c.box[d]);
            if (!(v < c.box[d])) v = std::nextafter(c.box[d], 0.f);
            pos[3 * a + d] = v;
        }
    halo::HostPlan P;
    std::string msg;
    int rc = halo::build_plan(pos.data(), c.n, c.box, c.grid, c.cutoff, selection, 64, P, msg);
    if (rc == 0) {
        const int lb = check_local_units(P, 64);
        if (lb) {
            std::printf("XCD-local units: %d violation(s)\n", lb);
            return 1;
        }
    }
    oracle *o = nullptr;
    int orc = oracle_build_ex(pos.data(), c.n, c.box, c.grid, c.cutoff, selection, &o);
    if (rc != orc) {
        std::printf("status differs: plan %d oracle %d (%s)\n", rc, orc, msg.c_str());
        oracle_free(o);
        return 1;
    }
    if (rc != 0) return 0;
    int bad = P.total_slots != oracle_total_slots(o);
    for (int32_t p = 0; p < P.n_pulse && !bad; ++p)
        for (int32_t d = 0; d < P.n_dom && !bad; ++d) {
            int32_t st, ss, rf, rs, ao, ds;
            float sh[3];
            oracle_pulse(o, p, d, &st, &ss, &rf, &rs, &ao, &ds, sh, nullptr);
            const halo::Segment &g = P.at(p, d);
            std::vector<int32_t> im((size_t)ss + 1);
            oracle_pulse(o, p, d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         im.data());
            bad |= st != g.send_to || ss != g.send_size || rf != g.recv_from ||
                   rs != g.recv_size || ao != g.atom_offset || ds != g.dep_start;
            for (int32_t i = 0; i < ss && !bad; ++i) bad |= im[i] != P.local_map[g.map_off + i];
        }
    // the oracle's exchanges, on buffers sized exactly, for the sanitizers' sake
    std::vector<float> x(3 * (size_t)P.total_slots, 0.f), f(3 * (size_t)P.total_slots, 1.f);
    oracle_exchange_x(o, x.data());
    oracle_exchange_f(o, f.data());
    oracle_free(o);
    if (bad) std::printf("plan differs from the oracle\n");
    return bad;
}

}  // namespace

int main()
{
    const Case cases[] = {
        {{3.f, 3.f, 6.f}, {1, 1, 2}, 1.0f, 600},
        {{6.f, 6.f, 6.f}, {2, 2, 2}, 1.0f, 2000},
        {{6.f, 6.f, 6.f}, {3, 3, 3}, 1.0f, 2500},
        {{4.f, 6.f, 8.f}, {2, 3, 4}, 1.2f, 3000},
        {{4.f, 4.f, 3.f}, {2, 2, 3}, 1.2f, 1500},
        {{2.f, 2.f, 8.f}, {1, 1, 4}, 2.5f, 1200},
        {{8.f, 8.f, 8.f}, {4, 4, 8}, 1.2f, 6000},
        {{4.f, 4.f, 4.f}, {2, 2, 2}, 1.0f, 0},
        {{2.f, 2.f, 2.f}, {1, 1, 1}, 0.9f, 50},
        {{2.f, 2.f, 2.f}, {2, 2, 2}, 1.5f, 10},
    };
    int fails = 0;
    for (const Case &c : cases)
        for (uint64_t seed = 1; seed <= 2; ++seed)
            for (int32_t sel = halo::kSelectSlab; sel <= halo::kSelectCorner; ++sel)
                fails += run(c, seed, sel);
    std::printf("%d case(s) differ\n", fails);
    return fails ? 1 : 0;
}
