/*
 * CPU oracle for exhaustive QUBO search.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
 * load this library.  The solver (the HIP kernels behind the C-ABI library)
 * never calls it, and it shares no code, header or table with the solver.
 *
 * What it computes is the plain definition from Maltsev et al., "Terastate-per-
 * second QUBO Brute-Force on a Single GPU: A Matrix Prefix-Suffix
 * Decomposition", sec. I:
 *     E(x) = sum_{i,j} Q_ij x_i x_j,   x in {0,1}^n,
 * over the full (not folded) int32 matrix Q, accumulated in int64.
 *   min_energy = min_x E(x)
 *   count      = |{x : E(x) = min_energy}|
 *   argmin     = the smallest index idx(x) = sum_i x_i 2^(n-1-i) among minimisers
 * (variable 0 is the most significant bit: the lexicographic row order of the
 * state matrix U_N, sec. II.B, Fig. 2).  The pages never say which minimiser to
 * return or that the minimisers are counted; the lowest index and the exact
 * count are this library's reading.
 *
 * Two independent tiers, both from sec. I.D of the same paper:
 *   tier A ("naive", O(n^2) per state): every state's energy from scratch, in
 *          increasing index order;
 *   tier B (Gray code, O(n) per state): states visited in binary-reflected Gray
 *          order g(i) = i ^ (i >> 1); one variable flips per step and the energy
 *          moves by that variable's local field, which is kept for every
 *          variable and updated in O(n) after each flip.  Ties are resolved by an
 *          explicit index comparison, because Gray order is not index order.
 * Work is split into contiguous ranges over POSIX threads and merged with the
 * rule (min energy; sum of counts at the min; min index at the min).
 *
 * The low-energy spectrum (same paper, sec. VI.B, "Future Work": keep a list of
 * the k lowest energies instead of one minimum): the first k states in the
 * order (E ascending, index ascending), each walker keeping its own sorted list
 * and the lists of disjoint ranges merged by the same order.  Which of several
 * equal energies at the k-th place to keep is not said; the lower index is this
 * library's reading, as for the single minimiser.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

#define ORACLE_MAX_N 63
#define ORACLE_MAX_THREADS 512
#define ORACLE_MAX_LOWEST 1024

/* Mutation testing of the pins: building with -DORACLE_MUTATION=k (k > 0)
 * plants one deliberate, plausible mistake so that the test suite can show
 * that some pin fails for it.  The default build (k = 0) contains none. */
#ifndef ORACLE_MUTATION
#define ORACLE_MUTATION 0
#endif
#define MUTANT(k) (ORACLE_MUTATION == (k))

/* ------------------------------------------------------------------ */
/* The definition.                                                    */
/* ------------------------------------------------------------------ */

int64_t oracle_energy(const int32_t *Q, int n, uint64_t idx)
{
    int64_t e = 0;
    for (int i = 0; i < n; ++i) {
        int xi = (int)((idx >> (MUTANT(2) ? i : n - 1 - i)) & 1u);
        if (!xi)
            continue; /* every term of row i carries the factor x_i = 0 */
        for (int j = 0; j < n; ++j) {
            int xj = (int)((idx >> (MUTANT(2) ? j : n - 1 - j)) & 1u);
            if (MUTANT(1) && j == i)
                continue;
            e += (int64_t)Q[(size_t)i * n + j] * (MUTANT(8) ? 1 : xj);
        }
    }
    return e;
}

void oracle_energy_many(const int32_t *Q, int n, const uint64_t *idx, uint64_t m, int64_t *out)
{
    for (uint64_t k = 0; k < m; ++k)
        out[k] = oracle_energy(Q, n, idx[k]);
}

/* Merge rule for partial results over disjoint state sets. */
static void merge(oracle_result *acc, const oracle_result *part)
{
    if (part->count == 0)
        return;
    if (acc->count == 0 || part->min_energy < acc->min_energy) {
        acc->min_energy = part->min_energy;
        acc->count = part->count;
        acc->argmin = part->argmin;
    } else if (part->min_energy == acc->min_energy) {
        acc->count += part->count;
        if (part->argmin < acc->argmin)
            acc->argmin = part->argmin;
    }
    if (part->max_abs_energy > acc->max_abs_energy)
        acc->max_abs_energy = part->max_abs_energy;
}

static void record(oracle_result *r, int64_t e, uint64_t idx)
{
    int64_t a = e < 0 ? -e : e;
    if (a > r->max_abs_energy)
        r->max_abs_energy = a;
    if (r->count == 0 || e < r->min_energy) {
        r->min_energy = e;
        r->count = 1;
        r->argmin = idx;
    } else if (e == r->min_energy) {
        r->count += MUTANT(6) ? 0 : 1;
        if (idx < r->argmin && !MUTANT(5))
            r->argmin = idx;
    }
}

static int clamp_threads(int threads)
{
    if (threads < 1)
        threads = 1;
    if (threads > ORACLE_MAX_THREADS)
        threads = ORACLE_MAX_THREADS;
    return threads;
}

/* ------------------------------------------------------------------ */
/* Tier A: direct evaluation over an index range [lo, hi).            */
/* ------------------------------------------------------------------ */

typedef struct {
    const int32_t *Q;
    int n;
    uint64_t lo, hi;
    oracle_result res;
} direct_job;

static void *direct_worker(void *arg)
{
    direct_job *job = (direct_job *)arg;
    memset(&job->res, 0, sizeof(job->res));
    for (uint64_t idx = job->lo; idx < job->hi; ++idx)
        record(&job->res, oracle_energy(job->Q, job->n, idx), idx);
    return NULL;
}

int oracle_search_direct(const int32_t *Q, int n, uint64_t lo, uint64_t hi, int threads,
                         oracle_result *out)
{
    if (!Q || !out || n < 1 || n > ORACLE_MAX_N)
        return -1;
    uint64_t total = 1ull << n;
    if (hi > total || lo > hi)
        return -1;
    memset(out, 0, sizeof(*out));
    threads = clamp_threads(threads);
    uint64_t span = hi - lo;
    if ((uint64_t)threads > span)
        threads = span ? (int)span : 1;
    direct_job *jobs = (direct_job *)calloc((size_t)threads, sizeof(direct_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -2;
    }
    for (int t = 0; t < threads; ++t) {
        jobs[t].Q = Q;
        jobs[t].n = n;
        jobs[t].lo = lo + span * (uint64_t)t / (uint64_t)threads;
        jobs[t].hi = lo + span * (uint64_t)(t + 1) / (uint64_t)threads;
    }
    for (int t = 1; t < threads; ++t)
        pthread_create(&tids[t], NULL, direct_worker, &jobs[t]);
    direct_worker(&jobs[0]);
    for (int t = 1; t < threads; ++t)
        pthread_join(tids[t], NULL);
    for (int t = 0; t < threads; ++t)
        merge(out, &jobs[t].res);
    free(jobs);
    free(tids);
    return 0;
}

/* ------------------------------------------------------------------ */
/* The k lowest states: the first k states in the order (E ascending,  */
/* index ascending).  A walker keeps a sorted list of at most k        */
/* (E, idx) pairs; lists of disjoint ranges merge by the same order.   */
/* ------------------------------------------------------------------ */

typedef struct {
    int64_t e;
    uint64_t idx;
} oracle_state;

static int state_less(const oracle_state *a, int64_t e, uint64_t idx)
{
    /* MUTANT(5) here: equal energies stay in the order they were met */
    return a->e < e || (a->e == e && (MUTANT(5) || a->idx < idx));
}

/* Inserts (e, idx) into the sorted list l of *len <= k entries. */
static void keep_lowest(oracle_state *l, int *len, int k, int64_t e, uint64_t idx)
{
    int pos = *len;
    while (pos > 0 && !state_less(&l[pos - 1], e, idx))
        --pos;
    if (pos >= (MUTANT(10) ? k - 1 : k))
        return;
    int last = *len < k ? *len : k - 1;
    for (int i = last; i > pos; --i)
        l[i] = l[i - 1];
    l[pos].e = e;
    l[pos].idx = idx;
    if (*len < k)
        ++*len;
}

/* ------------------------------------------------------------------ */
/* Tier B: incremental Gray-code walk over a sub-cube.                */
/*                                                                    */
/* The sub-cube fixes variables 0..k-1 to the k-bit number `top`       */
/* (variable 0 most significant) and walks the m = n - k free          */
/* variables.  k = 0 walks the whole space.                            */
/* ------------------------------------------------------------------ */

typedef struct {
    const int32_t *Q;
    int n, k;
    uint64_t top;
    uint64_t i_lo, i_hi; /* Gray counter range over the free variables */
    oracle_result res;
    int keep;             /* > 0: also keep the `keep` lowest states in list */
    int len;
    oracle_state list[ORACLE_MAX_LOWEST];
} gray_job;

static uint64_t gray(uint64_t i) { return i ^ (i >> 1); }

static int ctz64(uint64_t v)
{
    int t = 0;
    while (!(v & 1u)) {
        v >>= 1;
        ++t;
    }
    return t;
}

static void gray_range(gray_job *job)
{
    const int32_t *Q = job->Q;
    const int n = job->n, m = n - job->k;
    memset(&job->res, 0, sizeof(job->res));
    job->len = 0;
    if (job->i_lo >= job->i_hi)
        return;

    /* coupling[v][j] = Q_vj + Q_jv for j != v and 0 for j == v, so that the
     * local field of v is F_v = Q_vv + sum_j coupling[v][j] x_j and flipping v
     * leaves F_v itself unchanged. */
    static __thread int64_t coupling[ORACLE_MAX_N * ORACLE_MAX_N];
    int64_t field[ORACLE_MAX_N];
    int x[ORACLE_MAX_N];

    for (int v = 0; v < n; ++v)
        for (int j = 0; j < n; ++j)
            coupling[v * n + j] =
                (j == v) ? 0 : (int64_t)Q[(size_t)v * n + j] + (int64_t)Q[(size_t)j * n + v];

    uint64_t idx = (job->top << m) | gray(job->i_lo);
    for (int v = 0; v < n; ++v)
        x[v] = (int)((idx >> (n - 1 - v)) & 1u);
    int64_t e = oracle_energy(Q, n, idx);
    for (int v = 0; v < n; ++v) {
        int64_t f = MUTANT(7) ? 0 : Q[(size_t)v * n + v];
        for (int j = 0; j < n; ++j)
            f += coupling[v * n + j] * x[j];
        field[v] = f;
    }
    record(&job->res, e, idx);
    if (job->keep)
        keep_lowest(job->list, &job->len, job->keep, e, idx);

    for (uint64_t i = job->i_lo; i + 1 < job->i_hi; ++i) {
        int t = ctz64(i + 1);   /* Gray counter bit that flips ... */
        int v = MUTANT(9) ? t : n - 1 - t; /* ... is variable n-1-t */
        const int64_t *row = &coupling[v * n];
        if (x[v]) {             /* 1 -> 0: E drops by F_v, fields lose the coupling */
            e += MUTANT(3) ? field[v] : -field[v];
            x[v] = 0;
            for (int j = 0; j < n && !MUTANT(4); ++j)
                field[j] -= row[j];
        } else {                /* 0 -> 1: E rises by F_v, fields gain the coupling */
            e += field[v];
            x[v] = 1;
            for (int j = 0; j < n && !MUTANT(4); ++j)
                field[j] += row[j];
        }
        idx ^= 1ull << t;
        record(&job->res, e, idx);
        if (job->keep)
            keep_lowest(job->list, &job->len, job->keep, e, idx);
    }
}

typedef struct {
    gray_job *jobs;
    uint64_t first, stride, pieces;
} gray_rr;

static void *gray_worker(void *arg)
{
    gray_rr *a = (gray_rr *)arg;
    for (uint64_t p = a->first; p < a->pieces; p += a->stride)
        gray_range(&a->jobs[p]);
    return NULL;
}

/* Runs the Gray walk of the sub-cube (k, top) in pieces over the threads;
 * returns the pieces (caller frees) or NULL when out of memory. */
static gray_job *run_gray(const int32_t *Q, int n, int k, uint64_t top, int threads, int keep,
                          uint64_t *npieces)
{
    const int m = n - k;
    const uint64_t total = 1ull << m;
    threads = clamp_threads(threads);
    /* about 8 ranges per thread, each started from a direct evaluation */
    uint64_t pieces = (uint64_t)threads * 8u;
    if (pieces > total)
        pieces = total;
    if ((uint64_t)threads > pieces)
        threads = (int)pieces;
    gray_job *jobs = (gray_job *)calloc((size_t)pieces, sizeof(gray_job));
    gray_rr *args = (gray_rr *)calloc((size_t)threads, sizeof(gray_rr));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!jobs || !args || !tids) {
        free(jobs);
        free(args);
        free(tids);
        return NULL;
    }
    for (uint64_t p = 0; p < pieces; ++p) {
        jobs[p].Q = Q;
        jobs[p].n = n;
        jobs[p].k = k;
        jobs[p].top = top;
        jobs[p].keep = keep;
        jobs[p].i_lo = total * p / pieces;      /* total <= 2^63, pieces <= 4096 */
        jobs[p].i_hi = total * (p + 1) / pieces;
    }
    for (int t = 0; t < threads; ++t) {
        args[t].jobs = jobs;
        args[t].first = (uint64_t)t;
        args[t].stride = (uint64_t)threads;
        args[t].pieces = pieces;
    }
    for (int t = 1; t < threads; ++t)
        pthread_create(&tids[t], NULL, gray_worker, &args[t]);
    gray_worker(&args[0]);
    for (int t = 1; t < threads; ++t)
        pthread_join(tids[t], NULL);
    free(args);
    free(tids);
    *npieces = pieces;
    return jobs;
}

int oracle_search_gray(const int32_t *Q, int n, int k, uint64_t top, int threads,
                       oracle_result *out)
{
    if (!Q || !out || n < 1 || n > ORACLE_MAX_N || k < 0 || k > n)
        return -1;
    if (top >= (1ull << k))
        return -1;
    memset(out, 0, sizeof(*out));
    uint64_t pieces = 0;
    gray_job *jobs = run_gray(Q, n, k, top, threads, 0, &pieces);
    if (!jobs)
        return -2;
    for (uint64_t p = 0; p < pieces; ++p)
        merge(out, &jobs[p].res);
    free(jobs);
    return 0;
}

int oracle_lowest(const int32_t *Q, int n, int k, int gray_walk, int fixed, uint64_t top,
                  int threads, int64_t *energies, uint64_t *indices, int *found)
{
    if (!Q || !energies || !indices || !found || n < 1 || n > ORACLE_MAX_N || k < 1 ||
        k > ORACLE_MAX_LOWEST || fixed < 0 || fixed > n)
        return -1;
    if (top >= (1ull << fixed))
        return -1;
    oracle_state merged[ORACLE_MAX_LOWEST];
    int len = 0;
    if (gray_walk) {
        uint64_t pieces = 0;
        gray_job *jobs = run_gray(Q, n, fixed, top, threads, k, &pieces);
        if (!jobs)
            return -2;
        for (uint64_t p = 0; p < pieces; ++p)
            for (int i = 0; i < jobs[p].len; ++i)
                keep_lowest(merged, &len, k, jobs[p].list[i].e, jobs[p].list[i].idx);
        free(jobs);
    } else {
        /* tier A: every state of the sub-cube from the definition, in index order */
        const int m = n - fixed;
        for (uint64_t idx = top << m; idx < ((top + 1) << m); ++idx)
            keep_lowest(merged, &len, k, oracle_energy(Q, n, idx), idx);
    }
    for (int i = 0; i < len; ++i) {
        energies[i] = merged[i].e;
        indices[i] = merged[i].idx;
    }
    *found = len;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Floating-point Q (fp64).  The energy is the definition summed in a   */
/* fixed order: e = 0; for i ascending with x_i = 1, for j ascending    */
/* with x_j = 1: e += Q_ij, every add an IEEE binary64 add rounded to   */
/* nearest.  (Adding the zero products Q_ij x_i x_j of unset variables  */
/* would leave e unchanged: e starts at +0 and never becomes -0.)       */
/* The minimum, the lowest minimiser and the count of states with       */
/* exactly that value follow as for integers.                           */
/* ------------------------------------------------------------------ */

double oracle_energy_f64(const double *Q, int n, uint64_t idx)
{
    double e = 0.0;
    for (int i = 0; i < n; ++i) {
        if (!((idx >> (n - 1 - i)) & 1u))
            continue;
        for (int j = 0; j < n; ++j) {
            if (!((idx >> (n - 1 - j)) & 1u))
                continue;
            /* MUTANT(11): the terms in column-major order */
            e += MUTANT(11) ? Q[(size_t)j * n + i] : Q[(size_t)i * n + j];
        }
    }
    return e;
}

void oracle_energy_many_f64(const double *Q, int n, const uint64_t *idx, uint64_t m, double *out)
{
    for (uint64_t k = 0; k < m; ++k)
        out[k] = oracle_energy_f64(Q, n, idx[k]);
}

typedef struct {
    const double *Q;
    int n;
    uint64_t lo, hi;
    oracle_result_f64 res;
} direct_job_f64;

static int near_tie(double a, double b)
{
    double d = a - b, m = (a < 0 ? -a : a);
    return (d < 0 ? -d : d) <= 1e-12 * m;
}

static void record_f64(oracle_result_f64 *r, double e, uint64_t idx)
{
    if (MUTANT(12) && r->count != 0 && near_tie(e, r->min_energy))
        e = r->min_energy; /* MUTANT(12): a tolerance decides ties */
    if (r->count == 0 || e < r->min_energy) {
        r->min_energy = e;
        r->count = 1;
        r->argmin = idx;
    } else if (e == r->min_energy) {
        r->count += 1;
        if (idx < r->argmin)
            r->argmin = idx;
    }
    double a = e < 0 ? -e : e;
    if (a > r->max_abs_energy)
        r->max_abs_energy = a;
}

static void merge_f64(oracle_result_f64 *acc, const oracle_result_f64 *part)
{
    if (part->count == 0)
        return;
    if (acc->count == 0 || part->min_energy < acc->min_energy) {
        acc->min_energy = part->min_energy;
        acc->count = part->count;
        acc->argmin = part->argmin;
    } else if (part->min_energy == acc->min_energy) {
        acc->count += part->count;
        if (part->argmin < acc->argmin)
            acc->argmin = part->argmin;
    }
    if (part->max_abs_energy > acc->max_abs_energy)
        acc->max_abs_energy = part->max_abs_energy;
}

static void *direct_worker_f64(void *arg)
{
    direct_job_f64 *job = (direct_job_f64 *)arg;
    memset(&job->res, 0, sizeof(job->res));
    for (uint64_t idx = job->lo; idx < job->hi; ++idx)
        record_f64(&job->res, oracle_energy_f64(job->Q, job->n, idx), idx);
    return NULL;
}

int oracle_search_direct_f64(const double *Q, int n, uint64_t lo, uint64_t hi, int threads,
                             oracle_result_f64 *out)
{
    if (!Q || !out || n < 1 || n > ORACLE_MAX_N)
        return -1;
    uint64_t total = 1ull << n;
    if (hi > total || lo > hi)
        return -1;
    memset(out, 0, sizeof(*out));
    threads = clamp_threads(threads);
    uint64_t span = hi - lo;
    if ((uint64_t)threads > span)
        threads = span ? (int)span : 1;
    direct_job_f64 *jobs = (direct_job_f64 *)calloc((size_t)threads, sizeof(direct_job_f64));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -2;
    }
    for (int t = 0; t < threads; ++t) {
        jobs[t].Q = Q;
        jobs[t].n = n;
        jobs[t].lo = lo + span * (uint64_t)t / (uint64_t)threads;
        jobs[t].hi = lo + span * (uint64_t)(t + 1) / (uint64_t)threads;
    }
    for (int t = 1; t < threads; ++t)
        pthread_create(&tids[t], NULL, direct_worker_f64, &jobs[t]);
    direct_worker_f64(&jobs[0]);
    for (int t = 1; t < threads; ++t)
        pthread_join(tids[t], NULL);
    for (int t = 0; t < threads; ++t)
        merge_f64(out, &jobs[t].res);
    free(jobs);
    free(tids);
    return 0;
}

/* The k lowest states of a floating-point Q: the first k states in the order
 * (E ascending, index ascending) with E the fixed-order binary64 sum above,
 * each thread keeping its own sorted list over a contiguous index range and
 * the lists merged by the same order. */
typedef struct {
    double e;
    uint64_t idx;
} oracle_state_f64;

static int state_less_f64(const oracle_state_f64 *a, double e, uint64_t idx)
{
    /* MUTANT(13), with the merge below: equal energies stay in the order met */
    return a->e < e || (a->e == e && (MUTANT(13) || a->idx < idx));
}

static void keep_lowest_f64(oracle_state_f64 *l, int *len, int k, double e, uint64_t idx)
{
    int pos = *len;
    while (pos > 0 && !state_less_f64(&l[pos - 1], e, idx))
        --pos;
    if (pos >= k)
        return;
    int last = *len < k ? *len : k - 1;
    for (int i = last; i > pos; --i)
        l[i] = l[i - 1];
    l[pos].e = e;
    l[pos].idx = idx;
    if (*len < k)
        ++*len;
}

typedef struct {
    const double *Q;
    int n, k;
    uint64_t lo, hi;
    int len;
    oracle_state_f64 list[ORACLE_MAX_LOWEST];
} lowest_job_f64;

static void *lowest_worker_f64(void *arg)
{
    lowest_job_f64 *job = (lowest_job_f64 *)arg;
    job->len = 0;
    for (uint64_t idx = job->lo; idx < job->hi; ++idx)
        keep_lowest_f64(job->list, &job->len, job->k, oracle_energy_f64(job->Q, job->n, idx), idx);
    return NULL;
}

int oracle_lowest_f64(const double *Q, int n, int k, uint64_t lo, uint64_t hi, int threads,
                      double *energies, uint64_t *indices, int *found)
{
    if (!Q || !energies || !indices || !found || n < 1 || n > ORACLE_MAX_N || k < 1 ||
        k > ORACLE_MAX_LOWEST)
        return -1;
    if (hi > (1ull << n) || lo > hi)
        return -1;
    threads = clamp_threads(threads);
    const uint64_t span = hi - lo;
    if ((uint64_t)threads > span)
        threads = span ? (int)span : 1;
    lowest_job_f64 *jobs = (lowest_job_f64 *)calloc((size_t)threads, sizeof(lowest_job_f64));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -2;
    }
    for (int t = 0; t < threads; ++t) {
        jobs[t].Q = Q;
        jobs[t].n = n;
        jobs[t].k = k;
        jobs[t].lo = lo + span * (uint64_t)t / (uint64_t)threads;
        jobs[t].hi = lo + span * (uint64_t)(t + 1) / (uint64_t)threads;
    }
    for (int t = 1; t < threads; ++t)
        pthread_create(&tids[t], NULL, lowest_worker_f64, &jobs[t]);
    lowest_worker_f64(&jobs[0]);
    for (int t = 1; t < threads; ++t)
        pthread_join(tids[t], NULL);
    oracle_state_f64 merged[ORACLE_MAX_LOWEST];
    int len = 0;
    for (int s = 0; s < threads; ++s) {
        const int t = MUTANT(13) ? threads - 1 - s : s; /* MUTANT(13): last thread's list first */
        for (int i = 0; i < jobs[t].len; ++i)
            keep_lowest_f64(merged, &len, k, jobs[t].list[i].e, jobs[t].list[i].idx);
    }
    for (int i = 0; i < len; ++i) {
        energies[i] = merged[i].e;
        indices[i] = merged[i].idx;
    }
    *found = len;
    free(jobs);
    free(tids);
    return 0;
}

const char *oracle_version(void) { return "qubo-oracle 3 (tier A direct, tier B Gray; fp64 tier A and k lowest)"; }
