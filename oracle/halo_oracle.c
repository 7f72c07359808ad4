/*
 * halo_oracle.c -- serial CPU oracle of the eighth-shell halo exchange.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark load this library. The product path (the
 * HIP library under the package's csrc/) never includes, links or calls it,
 * and this file includes nothing from there.
 *
 * It is written to be read against the pages, not to be fast: one loop per
 * step, in the order the method states, no blocking and no reordering.
 *
 * Sources (page title, then section / algorithm):
 *  [REV]  "Redesigning GROMACS Halo Exchange: Improving Strong Scaling with
 *         GPU-initiated NVSHMEM" (paper review):
 *           s.3 "GROMACS domain decomposition halo exchange" (domains, cutoff,
 *               eighth-shell forwarding, pulses in z then y then x);
 *           Algorithm 1 (PulseData: sendSize, recvSize, atomOffset, coordShift,
 *               indexMap);
 *           Algorithm 3 (FusedPackCommX: x[indexMap] + coordShift stored at
 *               the receiver's atomOffset);
 *           Algorithm 4 (packWithDeps: split of indexMap at depOffset);
 *           Algorithm 6 (FusedCommUnpackF: pulses walked in reverse, forces
 *               of the receiver's region added onto indexMap targets);
 *           s.4 "Core formulas" (total pulses = np(x)+np(y)+np(z); chain of
 *               first dependent pulses).
 *  [GUIDE] "GPU-Initiated Halo Exchange Cuts CPU Bottlenecks in GROMACS",
 *           "The CPU bottleneck in halo exchange" (staged forwarding through
 *           intermediate ranks, one pack per pulse, Z to Y to X).
 *
 * Readings where the pages leave a step open (each one is restated where it
 * is used below):
 *  R1 pulses per dimension: np(d) = ceil(rc / w_d) when the dimension is
 *     decomposed (n_d > 1), else 0; np(d) must not exceed n_d - 1.
 *  R2 data moves to the lower neighbour; a domain's halo lies above its upper
 *     faces; a send that wraps the periodic boundary adds +L_d (coordShift).
 *  R3 selection: slot s of sender D is sent in pulse (dd, k) to R = D - e_dd
 *     iff delta < rc / w_dd, with delta the distance (in units of w_dd) of the
 *     atom's original position above R's upper face, computed in double:
 *       delta = t_dd - (c_dd(R) + 1), plus n_dd if negative.
 *     Candidates: every local slot when k = 0; the region received in pulse
 *     (dd, k-1) when k >= 1.
 *  R4 home atoms in ascending global id; indexMap ascending; local layout
 *     [home | region of pulse 0 | region of pulse 1 | ...]; domains laid out
 *     one after another in id order, id = cx + nx*(cy + ny*cz).
 *  R5 depOffset = number of home atoms: entries below it are independent.
 *  R6 force order: pulses strictly in reverse, one fp32 add per component.
 *  R7 corner selection (an option; the pages do not spell the test out): an
 *     atom belongs to the halo of domain D only if its Euclidean distance to
 *     D's box, over the upper faces it lies beyond, is below the cutoff:
 *       sum_d (delta_d * w_d)^2 < rc^2,  delta_d = 0 where the atom's cell
 *     equals D's along d, else its distance above D's upper face (as in R3),
 *     summed over d = x, y, z in that order, in double. In the pulses the
 *     test is made against each receiver; the partial sums only grow along
 *     the forwarding path, so the final receiver's test decides.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off (no -ffast-math).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_ERR_ARG (-1)
#define OR_ERR_GEOMETRY (-2)
#define OR_ERR_RANGE (-3)
#define OR_ERR_NOMEM (-7)

typedef struct {
    int32_t dim;        /* 0 = x, 1 = y, 2 = z */
    int32_t k;          /* pulse number within the dimension */
} or_pulse;

/* PulseData of one (pulse, sending domain), [REV] Algorithm 1. */
typedef struct {
    int32_t send_to;      /* receiver R = D - e_dim (periodic)              */
    int32_t send_size;    /* number of indexMap entries                     */
    int32_t *index_map;   /* local slots of D, ascending                    */
    int32_t dep_start;    /* count of entries below depOffset (= n_home)    */
    float shift[3];       /* coordShift                                     */
    int32_t recv_from;    /* the domain that sends to D in this pulse       */
    int32_t recv_size;    /* entries D receives in this pulse               */
    int32_t atom_offset;  /* local slot where D's region of this pulse starts */
} or_pd;

typedef struct {
    int64_t *gid;         /* global atom id of every local slot */
    int32_t size;
    int32_t cap;
} or_slots;

typedef struct oracle {
    int64_t n_atoms;
    int32_t criterion;    /* 0 slab (R3), 1 corner (R7) */
    float box[3];
    int32_t grid[3];
    float cutoff;
    double w[3];          /* domain width */
    double u[3];          /* cutoff in units of the domain width */
    int32_t np[3];        /* pulses per dimension */
    int32_t n_dom;
    int32_t n_pulse;
    or_pulse *pulse;      /* [n_pulse] */
    double *t;            /* [n_atoms][3] position in units of w */
    int32_t *c;           /* [n_atoms][3] cell coordinate */
    int32_t *n_home;      /* [n_dom] */
    or_slots *slots;      /* [n_dom] */
    int64_t *base;        /* [n_dom] first global slot of each domain */
    int64_t total_slots;
    or_pd *pd;            /* [n_pulse][n_dom] */
} oracle;

static int push_slot(or_slots *s, int64_t gid)
{
    if (s->size == s->cap) {
        int32_t ncap = s->cap ? 2 * s->cap : 16;
        int64_t *g = (int64_t *)realloc(s->gid, (size_t)ncap * sizeof(int64_t));
        if (!g) return OR_ERR_NOMEM;
        s->gid = g;
        s->cap = ncap;
    }
    s->gid[s->size++] = gid;
    return OR_OK;
}

void oracle_free(oracle *o)
{
    if (!o) return;
    if (o->pd) {
        for (int64_t i = 0; i < (int64_t)o->n_pulse * o->n_dom; ++i) free(o->pd[i].index_map);
        free(o->pd);
    }
    if (o->slots) {
        for (int32_t d = 0; d < o->n_dom; ++d) free(o->slots[d].gid);
        free(o->slots);
    }
    free(o->pulse);
    free(o->t);
    free(o->c);
    free(o->n_home);
    free(o->base);
    free(o);
}

/* Domain id from cell coordinates (R4). */
static int32_t dom_id(const oracle *o, int32_t cx, int32_t cy, int32_t cz)
{
    return cx + o->grid[0] * (cy + o->grid[1] * cz);
}

static void dom_cell(const oracle *o, int32_t id, int32_t cell[3])
{
    cell[0] = id % o->grid[0];
    cell[1] = (id / o->grid[0]) % o->grid[1];
    cell[2] = id / (o->grid[0] * o->grid[1]);
}

/* Geometry: domain widths and pulse counts, [REV] s.3 / s.4 and reading R1. */
static int geometry(oracle *o)
{
    for (int d = 0; d < 3; ++d) {
        if (!(o->box[d] > 0.0f) || !isfinite(o->box[d])) return OR_ERR_GEOMETRY;
        if (o->grid[d] < 1) return OR_ERR_GEOMETRY;
    }
    if (!(o->cutoff > 0.0f) || !isfinite(o->cutoff)) return OR_ERR_GEOMETRY;
    for (int d = 0; d < 3; ++d) {
        o->w[d] = (double)o->box[d] / (double)o->grid[d];
        o->u[d] = (double)o->cutoff / o->w[d];
        if (o->grid[d] > 1) {
            double p = ceil(o->u[d]);
            if (p > (double)(o->grid[d] - 1)) return OR_ERR_GEOMETRY;
            o->np[d] = (int32_t)p;
        } else {
            o->np[d] = 0;
        }
    }
    return OR_OK;
}

/* Pulse order z, then y, then x; np(d) pulses in each ([REV] s.3, s.4). */
static int make_pulses(oracle *o)
{
    o->n_pulse = o->np[0] + o->np[1] + o->np[2];
    o->pulse = (or_pulse *)calloc((size_t)(o->n_pulse ? o->n_pulse : 1), sizeof(or_pulse));
    if (!o->pulse) return OR_ERR_NOMEM;
    int32_t p = 0;
    for (int dim = 2; dim >= 0; --dim)
        for (int32_t k = 0; k < o->np[dim]; ++k) {
            o->pulse[p].dim = dim;
            o->pulse[p].k = k;
            ++p;
        }
    return OR_OK;
}

/* Selection test of reading R3: is atom a within the cutoff slab above the
 * upper face (in dimension dim) of the domain whose cell coordinate is cr? */
static int in_slab(const oracle *o, int64_t a, int dim, int32_t cr)
{
    double delta = o->t[3 * a + dim] - (double)(cr + 1);
    if (delta < 0.0) delta += (double)o->grid[dim];
    return delta < o->u[dim];
}

int oracle_build_ex(const float *pos, int64_t n_atoms, const float *box, const int32_t *grid,
                    float cutoff, int32_t criterion, oracle **out);

/* Corner test of reading R7 for atom a sent towards the receiver of cell cr
 * in a pulse along dim: the slab test, and the squared distance to the
 * receiver's box over the faces the atom lies beyond below rc^2. */
static int in_corner(const oracle *o, int64_t a, int dim, const int32_t cr[3])
{
    if (!in_slab(o, a, dim, cr[dim])) return 0;
    double s = 0.0;
    for (int d = 0; d < 3; ++d) {
        double delta = 0.0;
        if (d == dim || o->c[3 * a + d] != cr[d]) {
            delta = o->t[3 * a + d] - (double)(cr[d] + 1);
            if (delta < 0.0) delta += (double)o->grid[d];
        }
        const double dist = delta * o->w[d];
        s += dist * dist;
    }
    return s < (double)o->cutoff * (double)o->cutoff;
}

int oracle_build(const float *pos, int64_t n_atoms, const float *box, const int32_t *grid,
                 float cutoff, oracle **out)
{
    return oracle_build_ex(pos, n_atoms, box, grid, cutoff, 0, out);
}

int oracle_build_ex(const float *pos, int64_t n_atoms, const float *box, const int32_t *grid,
                    float cutoff, int32_t criterion, oracle **out)
{
    if (!out) return OR_ERR_ARG;
    *out = NULL;
    if (n_atoms < 0 || !box || !grid || (n_atoms > 0 && !pos)) return OR_ERR_ARG;
    if (criterion != 0 && criterion != 1) return OR_ERR_ARG;

    oracle *o = (oracle *)calloc(1, sizeof(oracle));
    if (!o) return OR_ERR_NOMEM;
    o->n_atoms = n_atoms;
    o->criterion = criterion;
    for (int d = 0; d < 3; ++d) {
        o->box[d] = box[d];
        o->grid[d] = grid[d];
    }
    o->cutoff = cutoff;
    int rc = geometry(o);
    if (rc) goto fail;

    /* every position finite and inside [0, L) */
    for (int64_t a = 0; a < n_atoms; ++a)
        for (int d = 0; d < 3; ++d) {
            float v = pos[3 * a + d];
            if (!isfinite(v) || !(v >= 0.0f) || !(v < box[d])) {
                rc = OR_ERR_RANGE;
                goto fail;
            }
        }

    if ((int64_t)grid[0] * grid[1] * grid[2] > INT32_MAX) {
        rc = OR_ERR_GEOMETRY;
        goto fail;
    }
    o->n_dom = grid[0] * grid[1] * grid[2];
    rc = make_pulses(o);
    if (rc) goto fail;

    /* Domain of every atom ([REV] s.3): t = x / w in double, clamped below n
     * so that rounding never yields cell n; c = floor(t). */
    size_t na = (size_t)(n_atoms ? n_atoms : 1);
    o->t = (double *)malloc(na * 3 * sizeof(double));
    o->c = (int32_t *)malloc(na * 3 * sizeof(int32_t));
    o->n_home = (int32_t *)calloc((size_t)o->n_dom, sizeof(int32_t));
    o->slots = (or_slots *)calloc((size_t)o->n_dom, sizeof(or_slots));
    o->base = (int64_t *)calloc((size_t)o->n_dom, sizeof(int64_t));
    o->pd = (or_pd *)calloc((size_t)(o->n_pulse ? o->n_pulse : 1) * o->n_dom, sizeof(or_pd));
    if (!o->t || !o->c || !o->n_home || !o->slots || !o->base || !o->pd) {
        rc = OR_ERR_NOMEM;
        goto fail;
    }
    for (int64_t a = 0; a < n_atoms; ++a)
        for (int d = 0; d < 3; ++d) {
            double t = (double)pos[3 * a + d] / o->w[d];
            double top = nextafter((double)grid[d], 0.0);
            if (t > top) t = top;
            o->t[3 * a + d] = t;
            o->c[3 * a + d] = (int32_t)floor(t);
        }

    /* Home atoms of each domain in ascending global id (R4). */
    for (int64_t a = 0; a < n_atoms; ++a) {
        int32_t id = dom_id(o, o->c[3 * a + 0], o->c[3 * a + 1], o->c[3 * a + 2]);
        rc = push_slot(&o->slots[id], a);
        if (rc) goto fail;
        o->n_home[id] += 1;
    }

    /* The pulses, one after the other. Within one pulse every domain first
     * selects from its state before the pulse; then every receiver appends. */
    for (int32_t p = 0; p < o->n_pulse; ++p) {
        int dim = o->pulse[p].dim;
        int32_t k = o->pulse[p].k;
        or_pd *row = &o->pd[(int64_t)p * o->n_dom];

        for (int32_t D = 0; D < o->n_dom; ++D) {
            int32_t cell[3];
            dom_cell(o, D, cell);
            int32_t cr[3] = {cell[0], cell[1], cell[2]};
            cr[dim] = (cell[dim] - 1 + grid[dim]) % grid[dim];   /* R2 */
            or_pd *q = &row[D];
            q->send_to = dom_id(o, cr[0], cr[1], cr[2]);

            /* candidates (R3) */
            int32_t lo, hi;
            if (k == 0) {
                lo = 0;
                hi = o->slots[D].size;
            } else {
                const or_pd *prev = &o->pd[(int64_t)(p - 1) * o->n_dom + D];
                lo = prev->atom_offset;
                hi = prev->atom_offset + prev->recv_size;
            }
            q->index_map = (int32_t *)malloc((size_t)(hi > lo ? hi - lo : 1) * sizeof(int32_t));
            if (!q->index_map) {
                rc = OR_ERR_NOMEM;
                goto fail;
            }
            q->send_size = 0;
            for (int32_t s = lo; s < hi; ++s) {
                const int64_t a = o->slots[D].gid[s];
                if (o->criterion ? in_corner(o, a, dim, cr) : in_slab(o, a, dim, cr[dim]))
                    q->index_map[q->send_size++] = s;
            }

            /* depOffset split, [REV] Algorithm 4 (R5) */
            q->dep_start = 0;
            for (int32_t i = 0; i < q->send_size; ++i)
                if (q->index_map[i] < o->n_home[D]) q->dep_start += 1;

            /* coordShift: the send wraps when D is in cell 0 (R2) */
            q->shift[0] = q->shift[1] = q->shift[2] = 0.0f;
            if (cell[dim] == 0) q->shift[dim] = box[dim];
        }

        /* append to receivers: atomOffset = the receiver's size so far */
        for (int32_t D = 0; D < o->n_dom; ++D) {
            or_pd *q = &row[D];
            or_pd *r = &row[q->send_to];
            r->recv_from = D;
            r->recv_size = q->send_size;
            r->atom_offset = o->slots[q->send_to].size;
            for (int32_t i = 0; i < q->send_size; ++i) {
                rc = push_slot(&o->slots[q->send_to], o->slots[D].gid[q->index_map[i]]);
                if (rc) goto fail;
            }
        }
    }

    /* global layout: domains one after the other (R4) */
    int64_t acc = 0;
    for (int32_t D = 0; D < o->n_dom; ++D) {
        o->base[D] = acc;
        acc += o->slots[D].size;
    }
    o->total_slots = acc;
    if (acc > INT32_MAX) {
        rc = OR_ERR_RANGE;
        goto fail;
    }
    *out = o;
    return OR_OK;

fail:
    oracle_free(o);
    return rc;
}

/* ---- read-out of the plan ------------------------------------------------ */

int64_t oracle_total_slots(const oracle *o) { return o ? o->total_slots : -1; }
int32_t oracle_num_domains(const oracle *o) { return o ? o->n_dom : -1; }
int32_t oracle_num_pulses(const oracle *o) { return o ? o->n_pulse : -1; }

int oracle_geometry(const oracle *o, double *w, double *u, int32_t *np)
{
    if (!o) return OR_ERR_ARG;
    for (int d = 0; d < 3; ++d) {
        if (w) w[d] = o->w[d];
        if (u) u[d] = o->u[d];
        if (np) np[d] = o->np[d];
    }
    return OR_OK;
}

int oracle_pulse_dim(const oracle *o, int32_t p, int32_t *dim, int32_t *k)
{
    if (!o || p < 0 || p >= o->n_pulse) return OR_ERR_ARG;
    if (dim) *dim = o->pulse[p].dim;
    if (k) *k = o->pulse[p].k;
    return OR_OK;
}

int oracle_domain(const oracle *o, int32_t d, int64_t *base, int32_t *n_home, int32_t *n_halo)
{
    if (!o || d < 0 || d >= o->n_dom) return OR_ERR_ARG;
    if (base) *base = o->base[d];
    if (n_home) *n_home = o->n_home[d];
    if (n_halo) *n_halo = o->slots[d].size - o->n_home[d];
    return OR_OK;
}

/* Global id of the atom held in every slot of the global layout. */
int oracle_slot_gids(const oracle *o, int64_t *gid_of_slot)
{
    if (!o || (!gid_of_slot && o->total_slots > 0)) return OR_ERR_ARG;
    for (int32_t D = 0; D < o->n_dom; ++D)
        for (int32_t s = 0; s < o->slots[D].size; ++s)
            gid_of_slot[o->base[D] + s] = o->slots[D].gid[s];
    return OR_OK;
}

/* Home slot (global layout) of every atom. */
int oracle_home_slots(const oracle *o, int64_t *slot_of_atom)
{
    if (!o || (!slot_of_atom && o->n_atoms > 0)) return OR_ERR_ARG;
    for (int32_t D = 0; D < o->n_dom; ++D)
        for (int32_t s = 0; s < o->n_home[D]; ++s)
            slot_of_atom[o->slots[D].gid[s]] = o->base[D] + s;
    return OR_OK;
}

int oracle_pulse(const oracle *o, int32_t p, int32_t d, int32_t *send_to, int32_t *send_size,
                 int32_t *recv_from, int32_t *recv_size, int32_t *atom_offset, int32_t *dep_start,
                 float *shift, int32_t *index_map)
{
    if (!o || p < 0 || p >= o->n_pulse || d < 0 || d >= o->n_dom) return OR_ERR_ARG;
    const or_pd *q = &o->pd[(int64_t)p * o->n_dom + d];
    if (send_to) *send_to = q->send_to;
    if (send_size) *send_size = q->send_size;
    if (recv_from) *recv_from = q->recv_from;
    if (recv_size) *recv_size = q->recv_size;
    if (atom_offset) *atom_offset = q->atom_offset;
    if (dep_start) *dep_start = q->dep_start;
    if (shift)
        for (int c = 0; c < 3; ++c) shift[c] = q->shift[c];
    if (index_map)
        for (int32_t i = 0; i < q->send_size; ++i) index_map[i] = q->index_map[i];
    return OR_OK;
}

/* ---- the two exchanges ---------------------------------------------------- */

/* Coordinate exchange, [REV] Algorithms 3 and 4 run one pulse at a time: for
 * every pulse in order, every sender D writes x[indexMap[i]] + coordShift to
 * slot atomOffset + i of its receiver. x holds the global layout; its home
 * slots are read, every halo slot is written. */
int oracle_exchange_x(const oracle *o, float *x)
{
    if (!o || (!x && o->total_slots > 0)) return OR_ERR_ARG;
    for (int32_t p = 0; p < o->n_pulse; ++p)
        for (int32_t D = 0; D < o->n_dom; ++D) {
            const or_pd *q = &o->pd[(int64_t)p * o->n_dom + D];
            int32_t R = q->send_to;
            const or_pd *r = &o->pd[(int64_t)p * o->n_dom + R];
            for (int32_t i = 0; i < q->send_size; ++i) {
                const float *src = &x[3 * (o->base[D] + q->index_map[i])];
                float *dst = &x[3 * (o->base[R] + r->atom_offset + i)];
                for (int c = 0; c < 3; ++c) dst[c] = src[c] + q->shift[c];
            }
        }
    return OR_OK;
}

/* Force exchange, [REV] Algorithm 6 with reading R6: pulses from the last to
 * the first; in pulse p every sender D adds the forces held in its receiver's
 * region of pulse p onto its own indexMap targets, one fp32 add per
 * component. f holds the global layout and is updated in place. */
int oracle_exchange_f(const oracle *o, float *f)
{
    if (!o || (!f && o->total_slots > 0)) return OR_ERR_ARG;
    for (int32_t p = o->n_pulse - 1; p >= 0; --p)
        for (int32_t D = 0; D < o->n_dom; ++D) {
            const or_pd *q = &o->pd[(int64_t)p * o->n_dom + D];
            int32_t R = q->send_to;
            const or_pd *r = &o->pd[(int64_t)p * o->n_dom + R];
            for (int32_t i = 0; i < q->send_size; ++i) {
                float *dst = &f[3 * (o->base[D] + q->index_map[i])];
                const float *src = &f[3 * (o->base[R] + r->atom_offset + i)];
                for (int c = 0; c < 3; ++c) dst[c] = dst[c] + src[c];
            }
        }
    return OR_OK;
}
