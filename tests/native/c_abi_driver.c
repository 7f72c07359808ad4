/* The C ABI from plain C, with no Python and no torch: HIP memory and a HIP
 * stream of the caller's own, plans built on the host and on the device, every
 * exchange form, compared bit for bit with the serial C oracle (test
 * infrastructure, linked only into this test program). Built by
 * __graft_entry__.build() and run by tests/test_gpu_c_abi.py on a GPU; exits
 * non-zero on the first difference or unexpected status. With --time it
 * instead prints how long back-to-back exchanges take when a C caller issues
 * them (GPU time and host time per call).
 */
#define _POSIX_C_SOURCE 199309L  /* clock_gettime */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "halo.h"

typedef struct oracle oracle;
int oracle_build_ex(const float *pos, int64_t n_atoms, const float *box, const int32_t *grid,
                    float cutoff, int32_t criterion, oracle **out);
void oracle_free(oracle *o);
int64_t oracle_total_slots(const oracle *o);
int oracle_home_slots(const oracle *o, int64_t *slot_of_atom);
int oracle_exchange_x(const oracle *o, float *x);
int oracle_exchange_f(const oracle *o, float *f);

#define CHECK_HIP(call)                                                                  \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            exit(2);                                                                     \
        }                                                                                \
    } while (0)

#define CHECK_HALO(call)                                                                  \
    do {                                                                                  \
        halo_status s_ = (call);                                                          \
        if (s_ != HALO_OK) {                                                              \
            printf("halo status %d (%s) at %s:%d\n", (int)s_, halo_last_error(), __FILE__, \
                   __LINE__);                                                             \
            exit(3);                                                                      \
        }                                                                                 \
    } while (0)

/* splitmix64: reproducible inputs without a library generator */
static uint64_t next_u64(uint64_t *s)
{
    uint64_t z = (*s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static double next_unit(uint64_t *s) { return (double)(next_u64(s) >> 11) * (1.0 / 9007199254740992.0); }

typedef struct {
    float box[3];
    int32_t grid[3];
    float cutoff;
    int64_t n;
    int32_t selection;
} Case;

typedef halo_status (*exchange_fn)(halo_plan *, float *, void *);

static int same_bits(const float *a, const float *b, int64_t n, const char *what)
{
    if (n == 0 || memcmp(a, b, (size_t)n * sizeof(float)) == 0) return 1;
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u, v;
        memcpy(&u, a + i, 4);
        memcpy(&v, b + i, 4);
        if (u != v) {
            printf("%s: first difference at float %lld: %.9g vs %.9g\n", what, (long long)i,
                   (double)a[i], (double)b[i]);
            break;
        }
    }
    return 0;
}

/* Run one exchange form on a fresh copy of `init` and compare with `want`. */
static int run_form(halo_plan *plan, exchange_fn fn, const char *name, float *dev, const float *init,
                    const float *want, float *host, int64_t nf, hipStream_t stream)
{
    const size_t bytes = (size_t)nf * sizeof(float);
    CHECK_HIP(hipMemcpyAsync(dev, init, bytes, hipMemcpyHostToDevice, stream));
    CHECK_HALO(fn(plan, dev, stream));
    CHECK_HIP(hipMemcpyAsync(host, dev, bytes, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HALO(halo_plan_sync(plan, stream));
    return same_bits(host, want, nf, name);
}

static int run_case(const Case *c, uint64_t seed, hipStream_t stream)
{
    uint64_t s = seed;
    const int64_t n = c->n;
    float *pos = (float *)malloc((size_t)(3 * n + 1) * sizeof(float));
    for (int64_t a = 0; a < n; ++a)
        for (int d = 0; d < 3; ++d) {
            float v = (float)(next_unit(&s) * c->box[d]);
            if (!(v < c->box[d])) v = nextafterf(c->box[d], 0.f);
            pos[3 * a + d] = v;
        }

    oracle *o = NULL;
    if (oracle_build_ex(pos, n, c->box, c->grid, c->cutoff, c->selection, &o) != 0) {
        printf("oracle build failed\n");
        exit(4);
    }
    halo_plan *hp = NULL, *dp = NULL;
    CHECK_HALO(halo_plan_create_ex(pos, n, c->box, c->grid, c->cutoff, c->selection, &hp));
    float *pos_dev = NULL;
    CHECK_HIP(hipMalloc((void **)&pos_dev, (size_t)(3 * n + 1) * sizeof(float)));
    CHECK_HIP(hipMemcpy(pos_dev, pos, (size_t)(3 * n) * sizeof(float), hipMemcpyHostToDevice));
    CHECK_HALO(halo_plan_create_device_ex(n ? pos_dev : NULL, n, c->box, c->grid, c->cutoff,
                                          c->selection, stream, &dp));

    /* A device build on a stream that is being captured is refused before
     * anything is queued or freed: both calls return HALO_ERR_ARG, the graph
     * stays empty, and dp still exchanges bit for bit below. */
    int capture_ok = 1;
    {
        hipGraph_t g = NULL;
        halo_plan *q = dp;
        size_t nodes = 1;
        CHECK_HIP(hipStreamBeginCapture(stream, hipStreamCaptureModeRelaxed));
        const halo_status s1 = halo_plan_create_device_ex(n ? pos_dev : NULL, n, c->box, c->grid,
                                                          c->cutoff, c->selection, stream, &q);
        const halo_status s2 = halo_plan_rebuild_device(dp, n ? pos_dev : NULL, n, c->box, stream);
        CHECK_HIP(hipStreamEndCapture(stream, &g));
        CHECK_HIP(hipGraphGetNodes(g, NULL, &nodes));
        CHECK_HIP(hipGraphDestroy(g));
        capture_ok = s1 == HALO_ERR_ARG && q == NULL && s2 == HALO_ERR_ARG && nodes == 0;
        if (!capture_ok)
            printf("device build under capture: create %d rebuild %d, %zu graph node(s)\n",
                   (int)s1, (int)s2, nodes);
    }

    const int64_t slots = oracle_total_slots(o);
    int ok = capture_ok && halo_plan_total_slots(hp) == slots && halo_plan_total_slots(dp) == slots &&
             halo_plan_selection(hp) == c->selection && halo_plan_selection(dp) == c->selection;
    int64_t *hs_o = (int64_t *)malloc((size_t)(n + 1) * 8), *hs_h = (int64_t *)malloc((size_t)(n + 1) * 8),
            *hs_d = (int64_t *)malloc((size_t)(n + 1) * 8);
    oracle_home_slots(o, hs_o);
    CHECK_HALO(halo_plan_home_slots(hp, hs_h));
    CHECK_HALO(halo_plan_home_slots(dp, hs_d));
    ok = ok && memcmp(hs_o, hs_h, (size_t)n * 8) == 0 && memcmp(hs_o, hs_d, (size_t)n * 8) == 0;
    if (!ok) printf("plan layout differs from the oracle\n");

    /* coordinates: home slots hold the positions, halo slots NaN */
    const int64_t nf = 3 * slots;
    float *x0 = (float *)malloc((size_t)(nf + 3) * sizeof(float));
    float *want = (float *)malloc((size_t)(nf + 3) * sizeof(float));
    float *host = (float *)malloc((size_t)(nf + 3) * sizeof(float));
    for (int64_t i = 0; i < nf; ++i) x0[i] = NAN;
    for (int64_t a = 0; a < n; ++a)
        for (int d = 0; d < 3; ++d) x0[3 * hs_o[a] + d] = pos[3 * a + d];
    memcpy(want, x0, (size_t)nf * sizeof(float));
    oracle_exchange_x(o, want);
    float *dev = NULL;
    CHECK_HIP(hipMalloc((void **)&dev, (size_t)(nf + 3) * sizeof(float)));

    const int32_t pulses = halo_plan_num_pulses(hp);
    struct {
        exchange_fn fn;
        const char *name;
    } xf[] = {{halo_exchange_x, "x"},
              {halo_exchange_x_indexmap, "x_indexmap"},
              {halo_exchange_x_transposed, "x_transposed"},
              {halo_exchange_x_pulsewise, "x_pulsewise"},
              {halo_exchange_x_staged, "x_staged"},
              {halo_exchange_x_direct, "x_direct"},
              {halo_exchange_x_items, "x_items"},
              {halo_exchange_x_indexmap_lds, "x_indexmap_lds"}},
      ff[] = {{halo_exchange_f, "f"},
              {halo_exchange_f_indexmap, "f_indexmap"},
              {halo_exchange_f_transposed, "f_transposed"},
              {halo_exchange_f_pulsewise, "f_pulsewise"},
              {halo_exchange_f_staged, "f_staged"},
              {halo_exchange_f_atomic, "f_atomic"},
              {halo_exchange_f_items, "f_items"}};
    halo_plan *plans[2] = {hp, dp};
    for (int k = 0; k < 2 && ok; ++k)
        for (size_t i = 0; i < sizeof(xf) / sizeof(xf[0]) && ok; ++i) {
            if (xf[i].fn == halo_exchange_x_transposed && pulses > 8) continue;
            ok = run_form(plans[k], xf[i].fn, xf[i].name, dev, x0, want, host, nf, stream);
        }

    /* the same coordinates through halo_scatter_home from the atom order */
    for (int k = 0; k < 2 && ok && n > 0; ++k) {
        float *nan_fill = (float *)malloc((size_t)(nf + 3) * sizeof(float));
        for (int64_t i = 0; i < nf; ++i) nan_fill[i] = NAN;
        CHECK_HIP(hipMemcpyAsync(dev, nan_fill, (size_t)nf * sizeof(float), hipMemcpyHostToDevice,
                                 stream));
        CHECK_HALO(halo_scatter_home(plans[k], pos_dev, dev, stream));
        CHECK_HALO(halo_exchange_x(plans[k], dev, stream));
        CHECK_HIP(hipMemcpyAsync(host, dev, (size_t)nf * sizeof(float), hipMemcpyDeviceToHost,
                                 stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        ok = same_bits(host, want, nf, "scatter_home + x");
        free(nan_fill);
    }

    /* forces: small integers on halo slots, 0 on home slots, so that every
     * partial sum is exact and the atomic form is bitwise too */
    for (int64_t i = 0; i < nf; ++i) x0[i] = (float)((int)(next_u64(&s) % 17u) - 8);
    for (int64_t a = 0; a < n; ++a)
        for (int d = 0; d < 3; ++d) x0[3 * hs_o[a] + d] = 0.f;
    memcpy(want, x0, (size_t)nf * sizeof(float));
    oracle_exchange_f(o, want);
    for (int k = 0; k < 2 && ok; ++k)
        for (size_t i = 0; i < sizeof(ff) / sizeof(ff[0]) && ok; ++i) {
            if (ff[i].fn == halo_exchange_f_transposed && pulses > 8) continue;
            ok = run_form(plans[k], ff[i].fn, ff[i].name, dev, x0, want, host, nf, stream);
        }

    /* every atom's force back in atom order through halo_gather_home */
    for (int k = 0; k < 2 && ok && n > 0; ++k) {
        float *atoms_dev = NULL, *atoms = (float *)malloc((size_t)(3 * n) * sizeof(float));
        CHECK_HIP(hipMalloc((void **)&atoms_dev, (size_t)(3 * n) * sizeof(float)));
        CHECK_HIP(hipMemcpyAsync(dev, x0, (size_t)nf * sizeof(float), hipMemcpyHostToDevice,
                                 stream));
        CHECK_HALO(halo_exchange_f(plans[k], dev, stream));
        CHECK_HALO(halo_gather_home(plans[k], dev, atoms_dev, stream));
        CHECK_HIP(hipMemcpyAsync(atoms, atoms_dev, (size_t)(3 * n) * sizeof(float),
                                 hipMemcpyDeviceToHost, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        for (int64_t a = 0; a < n && ok; ++a)
            ok = same_bits(atoms + 3 * a, want + 3 * hs_o[a], 3, "gather_home");
        CHECK_HIP(hipFree(atoms_dev));
        free(atoms);
    }

    /* an argument error is synchronous and leaves a message */
    if (ok && slots > 0) {
        ok = halo_exchange_x(hp, NULL, stream) == HALO_ERR_ARG && halo_last_error()[0] != '\0';
        if (!ok) printf("NULL buffer was not refused\n");
    }

    printf("case grid %dx%dx%d n=%lld selection=%d pulses=%d slots=%lld: %s\n", c->grid[0],
           c->grid[1], c->grid[2], (long long)n, c->selection, pulses, (long long)slots,
           ok ? "bitwise equal" : "DIFFERS");
    fflush(stdout);
    CHECK_HIP(hipFree(dev));
    CHECK_HIP(hipFree(pos_dev));
    halo_plan_destroy(hp);
    halo_plan_destroy(dp);
    oracle_free(o);
    free(pos);
    free(hs_o);
    free(hs_h);
    free(hs_d);
    free(x0);
    free(want);
    free(host);
    return ok;
}

/* Host cost of issuing exchanges from C: back-to-back calls of the default
 * exchanges on a plan of the given shape, timed with HIP events and with the
 * host clock (printed, not checked). */
static void time_case(const Case *c, hipStream_t stream)
{
    uint64_t s = 7;
    const int64_t n = c->n;
    float *pos = (float *)malloc((size_t)(3 * n) * sizeof(float));
    for (int64_t a = 0; a < 3 * n; ++a) pos[a] = (float)(next_unit(&s) * c->box[a % 3]);
    for (int64_t a = 0; a < n; ++a)
        for (int d = 0; d < 3; ++d)
            if (!(pos[3 * a + d] < c->box[d])) pos[3 * a + d] = nextafterf(c->box[d], 0.f);
    halo_plan *p = NULL;
    CHECK_HALO(halo_plan_create(pos, n, c->box, c->grid, c->cutoff, &p));
    CHECK_HALO(halo_plan_upload(p));
    const int64_t nf = 3 * halo_plan_total_slots(p);
    float *x = NULL, *f = NULL;
    CHECK_HIP(hipMalloc((void **)&x, (size_t)nf * sizeof(float)));
    CHECK_HIP(hipMalloc((void **)&f, (size_t)nf * sizeof(float)));
    CHECK_HIP(hipMemsetAsync(x, 0, (size_t)nf * sizeof(float), stream));
    CHECK_HIP(hipMemsetAsync(f, 0, (size_t)nf * sizeof(float), stream));
    const int reps = 2000;
    hipEvent_t e0, e1;
    CHECK_HIP(hipEventCreate(&e0));
    CHECK_HIP(hipEventCreate(&e1));
    for (int which = 0; which < 2; ++which) {
        for (int i = 0; i < 50; ++i)
            CHECK_HALO(which ? halo_exchange_f(p, f, stream) : halo_exchange_x(p, x, stream));
        CHECK_HIP(hipStreamSynchronize(stream));
        struct timespec t0, t1;
        clock_gettime(CLOCK_MONOTONIC, &t0);
        CHECK_HIP(hipEventRecord(e0, stream));
        for (int i = 0; i < reps; ++i)
            CHECK_HALO(which ? halo_exchange_f(p, f, stream) : halo_exchange_x(p, x, stream));
        clock_gettime(CLOCK_MONOTONIC, &t1);
        CHECK_HIP(hipEventRecord(e1, stream));
        CHECK_HIP(hipEventSynchronize(e1));
        float ms = 0.f;
        CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
        const double host_us = ((t1.tv_sec - t0.tv_sec) * 1e9 + (t1.tv_nsec - t0.tv_nsec)) / 1e3;
        printf("time grid %dx%dx%d n=%lld %s: %.2f us per exchange on the GPU, %.2f us per "
               "call on the host\n", c->grid[0], c->grid[1], c->grid[2], (long long)n,
               which ? "f" : "x", ms * 1e3 / reps, host_us / reps);
    }
    CHECK_HALO(halo_plan_sync(p, stream));
    CHECK_HIP(hipEventDestroy(e0));
    CHECK_HIP(hipEventDestroy(e1));
    CHECK_HIP(hipFree(x));
    CHECK_HIP(hipFree(f));
    halo_plan_destroy(p);
    free(pos);
}

int main(int argc, char **argv)
{
    if (argc > 1 && strcmp(argv[1], "--time") == 0) {
        const Case tc[] = {{{3.f, 3.f, 6.f}, {1, 1, 2}, 1.0f, 5400, HALO_SELECT_SLAB},
                           {{6.f, 6.f, 6.f}, {2, 2, 2}, 1.0f, 21600, HALO_SELECT_SLAB},
                           {{15.f, 15.f, 15.f}, {4, 4, 4}, 1.2f, 337500, HALO_SELECT_SLAB},
                           {{8.f, 8.f, 8.f}, {4, 4, 8}, 1.2f, 51200, HALO_SELECT_SLAB},
                           {{22.f, 22.f, 22.f}, {8, 8, 8}, 1.2f, 1064800, HALO_SELECT_SLAB}};
        hipStream_t stream;
        CHECK_HIP(hipSetDevice(0));
        CHECK_HIP(hipStreamCreate(&stream));
        for (size_t i = 0; i < sizeof(tc) / sizeof(tc[0]); ++i) time_case(&tc[i], stream);
        {
            /* the capture query every eager fused launch makes */
            const int reps = 100000;
            hipStreamCaptureStatus cs;
            struct timespec t0, t1;
            clock_gettime(CLOCK_MONOTONIC, &t0);
            for (int i = 0; i < reps; ++i) CHECK_HIP(hipStreamIsCapturing(stream, &cs));
            clock_gettime(CLOCK_MONOTONIC, &t1);
            printf("time hipStreamIsCapturing: %.3f us per call\n",
                   ((t1.tv_sec - t0.tv_sec) * 1e9 + (t1.tv_nsec - t0.tv_nsec)) / 1e3 / reps);
        }
        CHECK_HIP(hipStreamDestroy(stream));
        return 0;
    }
    const Case cases[] = {
        {{6.f, 6.f, 6.f}, {2, 2, 2}, 1.0f, 21600, HALO_SELECT_SLAB},
        {{8.f, 8.f, 8.f}, {4, 4, 8}, 1.2f, 51200, HALO_SELECT_SLAB},
        {{8.f, 8.f, 8.f}, {4, 4, 8}, 1.2f, 51200, HALO_SELECT_CORNER},
        {{6.f, 6.f, 6.f}, {3, 3, 3}, 2.5f, 20000, HALO_SELECT_CORNER},
        {{4.f, 4.f, 4.f}, {2, 2, 2}, 1.0f, 0, HALO_SELECT_SLAB},
    };
    hipStream_t stream;
    CHECK_HIP(hipSetDevice(0));
    CHECK_HIP(hipStreamCreate(&stream));
    int ok = 1;
    for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]) && ok; ++i)
        ok = run_case(&cases[i], 100 + i, stream);
    CHECK_HIP(hipStreamDestroy(stream));
    printf(ok ? "c_abi_driver: all cases bitwise equal to the oracle\n"
              : "c_abi_driver: FAILED\n");
    return ok ? 0 : 1;
}
