/*
 * CPU oracle for exhaustive QUBO search.  TEST INFRASTRUCTURE ONLY: only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark use it.
 *
 * E(x) = sum_{i,j} Q_ij x_i x_j over a full row-major n x n int32 Q (Maltsev et
 * al., "Terastate-per-second QUBO Brute-Force on a Single GPU", sec. I), with the
 * state index idx(x) = sum_i x_i 2^(n-1-i) (variable 0 most significant,
 * sec. II.B Fig. 2).  All energies are int64.  Functions return 0 on success,
 * -1 on a bad argument and -2 when memory runs out.
 */
#ifndef QUBO_ORACLE_H
#define QUBO_ORACLE_H
#include <stdint.h>

typedef struct {
    int64_t min_energy;     /* min over the searched states */
    uint64_t argmin;        /* smallest index attaining it */
    uint64_t count;         /* number of searched states attaining it (0 = none searched) */
    int64_t max_abs_energy; /* largest |E| seen (overflow audit for int32 solvers) */
} oracle_result;

/* E(x) for the state with index idx. */
int64_t oracle_energy(const int32_t *Q, int n, uint64_t idx);
void oracle_energy_many(const int32_t *Q, int n, const uint64_t *idx, uint64_t m, int64_t *out);

/* Tier A: direct O(n^2) evaluation of every idx in [lo, hi). */
int oracle_search_direct(const int32_t *Q, int n, uint64_t lo, uint64_t hi, int threads,
                         oracle_result *out);

/* Tier B: Gray-code walk over the sub-cube whose variables 0..k-1 equal the k-bit
 * number `top` (variable 0 most significant); k = 0, top = 0 is the full space. */
int oracle_search_gray(const int32_t *Q, int n, int k, uint64_t top, int threads,
                       oracle_result *out);

/* The k lowest states (1 <= k <= 1024): the first k states in the order
 * (E ascending, index ascending) of the sub-cube whose first `fixed` variables
 * spell `top` (fixed = 0: the whole space); gray_walk = 0 evaluates every state
 * directly (tier A, one thread), 1 walks in Gray order (tier B).  Writes
 * min(k, 2^(n - fixed)) pairs and their number to *found. */
int oracle_lowest(const int32_t *Q, int n, int k, int gray_walk, int fixed, uint64_t top,
                  int threads, int64_t *energies, uint64_t *indices, int *found);

/* Floating-point Q (row-major n x n binary64).  E(x) is the sum, in this
 * order, of Q_ij over i ascending with x_i = 1 and, inside, j ascending with
 * x_j = 1, each add rounded to nearest; ties are exact equality. */
typedef struct {
    double min_energy;
    uint64_t argmin;
    uint64_t count;
    double max_abs_energy;
} oracle_result_f64;

double oracle_energy_f64(const double *Q, int n, uint64_t idx);
void oracle_energy_many_f64(const double *Q, int n, const uint64_t *idx, uint64_t m, double *out);
/* Tier A over idx in [lo, hi). */
int oracle_search_direct_f64(const double *Q, int n, uint64_t lo, uint64_t hi, int threads,
                             oracle_result_f64 *out);
/* Tier A over idx in [lo, hi): the k lowest states (k <= 1024) in the order
 * (E ascending, index ascending); *found = min(k, hi - lo). */
int oracle_lowest_f64(const double *Q, int n, int k, uint64_t lo, uint64_t hi, int threads,
                      double *energies, uint64_t *indices, int *found);

const char *oracle_version(void);
#endif
