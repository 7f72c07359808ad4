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
