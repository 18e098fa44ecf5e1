/*
 * qubo.h -- C-ABI of the exhaustive dense-QUBO solver for AMD Instinct MI355X (gfx950).
 *
 * The solver minimises E(x) = sum_{i,j} Q_ij x_i x_j over all x in {0,1}^n for an
 * int32 matrix Q (Maltsev, Remnev, Kapranov and Krivtsova, "Terastate-per-second
 * QUBO Brute-Force on a Single GPU: A Matrix Prefix-Suffix Decomposition",
 * sec. I), with the prefix-suffix decomposition of sec. II (eq. 4 and eq. 8), the
 * Gray-code prefix walk of sec. III.B (eq. 9, Algorithm 2) and the parallel
 * splits of sec. III.C.  Every call is exact: integer arithmetic throughout.  The
 * qubo_*_f64 entry points search a binary64 Q (sec. VI.B, floating-point
 * matrices): they return the exact answer of a fixed-order binary64 definition
 * of E, from an integer walk over rounded tables and a re-evaluation of every
 * state the rounding could not rank.
 *
 * Conventions shared by every entry point
 *   - Q is a dense n x n int32 matrix, row-major and contiguous.  It need not be
 *     symmetric: only Q_ij + Q_ji (i != j) and Q_ii enter E, so it is folded into
 *     the upper triangle internally (sec. II.A uses an upper-triangular Q).
 *   - A state is the index idx(x) = sum_i x_i 2^(n-1-i): variable 0 is the most
 *     significant bit, the lexicographic row order of the state matrix U_N
 *     (sec. II.B, Fig. 2).  Variable i of the minimiser is (argmin >> (n-1-i)) & 1.
 *   - Overflow guard: the sum over all entries of |Q_ij| must not exceed
 *     2^30 - 1.  Every energy, partial energy and table entry the solver forms is
 *     a sum over distinct entries of the folded matrix, each taken with its sign
 *     or as its positive or negative part, so at most that sum in magnitude, and
 *     every comparison is between two such sums, so int32 is then exact everywhere.  (The paper instead bounds
 *     the spectrum with simulated annealing, sec. IV.B.5; this guard is exact.)
 *   - Status codes: 0 on success, a negative QUBO_E* code otherwise.  On error
 *     the output struct is left untouched.
 *   - The library keeps no global mutable state except the per-device HIP
 *     runtime; calls on different streams may run concurrently.
 */
#ifndef QUBO_H
#define QUBO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef QUBO_API
#define QUBO_API __attribute__((visibility("default")))
#endif

#define QUBO_OK 0
#define QUBO_EINVAL (-1)  /* null pointer, n or a split parameter out of range */
#define QUBO_ERANGE (-2)  /* int32 Q: sum |Q_ij| exceeds 2^30 - 1 (int32 would not be exact);
                             binary64 Q: an entry not finite, or sum |Q_ij| above 2^100 or
                             in (0, 2^-100) */
#define QUBO_EPLAN (-3)   /* the requested split does not fit the kernel's registers/LDS/limits */
#define QUBO_EDEVICE (-4) /* no usable gfx950 device, or a HIP runtime error */
#define QUBO_ENOMEM (-5)  /* device or host allocation failed */
#define QUBO_ESCRATCH (-6) /* qubo_search_noalloc: the search needs more device memory than
                              its static buffer holds (QUBO_NOALLOC_BYTES) */

#define QUBO_MAX_N 63

/* Result of a search (24 bytes). */
typedef struct {
    int32_t min_energy; /* min over the searched states of E(x) */
    uint32_t reserved;  /* zero */
    uint64_t argmin;    /* smallest state index attaining min_energy */
    uint64_t count;     /* exact number of searched states attaining min_energy */
} qubo_result;

/* The decomposition the solver runs (sec. II.A partition sizes and the
 * parallel split of sec. III.C), as chosen by the host planner. */
typedef struct {
    int32_t n;               /* variables as given */
    int32_t n_search;        /* variables searched per launch: n - split_bits, at least 5 */
    int32_t prefix_bits;     /* A: prefix variables 0..A-1, walked in Gray order */
    int32_t suffix_bits;     /* B = n_search - A: suffix variables, one per column bit */
    int32_t cache_bits;      /* l: Gray bits whose M_int rows are cached on chip
                                (the lowest reg_bits in VGPRs, the rest in LDS);
                                rows of higher bits are read from L2/HBM.  The
                                effective value: at most seg_bits */
    int32_t reg_bits;        /* Gray bits whose rows live in VGPRs (5) */
    int32_t cols_per_lane;   /* suffix columns held by one lane (8 or 16) */
    int32_t wave_size;       /* 64 */
    int32_t waves_per_block; /* waves of a workgroup, sharing one column group */
    int32_t seg_bits;        /* each wave walks 2^seg_bits consecutive Gray steps per work unit */
    int32_t blocks;          /* persistent workgroups launched */
    int32_t lds_bytes;       /* LDS per workgroup for cached rows */
    int32_t split_bits;      /* k > 0: the search runs 2^k sub-problems of n - k variables,
                                one per assignment of variables 0..k-1 (sec. III.C.1);
                                the other fields describe one sub-problem */
    int32_t reserved;
    uint64_t col_groups;     /* groups of wave_size * cols_per_lane columns */
    uint64_t work_units;     /* (column group, segment) pairs */
    uint64_t workspace_bytes;/* device memory the search allocates */
} qubo_plan;

/* Host only; touches no device.  Plans a search of n variables.
 *   prefix_bits: A in [5, n], or -1 to let the planner choose;
 *   cache_bits:  l in [5, A], or -1 to let the planner choose.
 * Planned for a 256-CU MI355X (qubo_search re-plans for the device it runs on).
 * Above 58 variables the search fixes the first n - 58 variables and runs one
 * launch per assignment (split_bits > 0); prefix_bits and cache_bits then
 * refer to the 58-variable sub-problems.
 * Returns QUBO_EINVAL for n outside [1, 63], or a split value outside the ranges
 * above, and QUBO_EPLAN when the split exceeds the kernel's limits (prefix-energy
 * table over 2^32 entries, M_int over 2^33 bytes, LDS over 64 KiB). */
QUBO_API int qubo_make_plan(int n, int prefix_bits, int cache_bits, qubo_plan *out);

/* Host only; touches no device.  Checks the overflow guard on a host copy of Q
 * (n x n int32, row-major): sum |Q_ij| <= 2^30 - 1.
 * Returns QUBO_OK, QUBO_EINVAL (null Q, n outside [1, 63]) or QUBO_ERANGE. */
QUBO_API int qubo_check_q(const int32_t *Q_host, int n);

/* Host only; touches no device.  Writes sum |Q_ij| of a host int32 matrix
 * (n x n, row-major), in int64, to *abs_sum; no range check.
 * Returns QUBO_OK or QUBO_EINVAL (null pointer, n outside [1, 63]). */
QUBO_API int qubo_abs_sum(const int32_t *Q_host, int n, int64_t *abs_sum);

/* Host only; touches no device.  The guard of the binary64 searches
 * (qubo_search_f64 and its relatives) on a host copy of Q (n x n binary64,
 * row-major): every entry finite and S = sum |Q_ij| either 0 or in
 * [2^-100, 2^100].  The range keeps the walk's scale factor 2^(17 - e)
 * (S < 2^e) and every binary64 sum of the tables and the definition well
 * inside binary64's normal range, with room to spare at both ends.
 * Returns QUBO_OK, QUBO_EINVAL (null Q, n outside [1, 63]) or QUBO_ERANGE. */
QUBO_API int qubo_check_q_f64(const double *Q_host, int n);

/* Host only; touches no device.  The exact int32 form of a dyadic binary64
 * matrix, which the binary64 searches hand to the integer search (sec. VI.B:
 * floating-point matrices).  Q_host: n x n binary64, row-major.  When every
 * entry is an integer multiple of 2^-f and sum |2^f Q_ij| <= 2^30 - 1 (f the
 * smallest such exponent, possibly negative; f = 0 for the zero matrix),
 * writes the n x n int32 matrix 2^f Q to Q_int (host, n*n entries) and f to
 * *f and returns QUBO_OK: every partial sum of the binary64 definition is then
 * exact, so E(x) = E_int(x) / 2^f for every state.  Returns QUBO_ERANGE when Q
 * has no such form (a non-finite entry included; Q_int and *f are then left
 * unspecified), QUBO_EINVAL for null pointers or n outside [1, 63]. */
QUBO_API int qubo_f64_as_int32(const double *Q_host, int n, int32_t *Q_int, int *f);

/* Exhaustive search over all 2^n states (sec. III.B Algorithm 2 with the
 * splits of sec. III.C), on the HIP stream `stream` (a hipStream_t; NULL is the
 * null stream) of the current device.
 *   Q: device pointer, n x n int32, row-major; read only, owned by the caller.
 *   n: 1..63.  For n < 5 the solver appends 5 - n dummy variables with
 *      Q_ii = +1 and no couplings (they are 0 in every minimiser, so min, argmin
 *      and count are those of the original problem).  For n > 58 it fixes the
 *      first n - 58 variables and runs one launch per assignment (hours to days
 *      of GPU time at these sizes).
 *   prefix_bits, cache_bits: as for qubo_make_plan (-1 = planner's choice).  The
 *      result does not depend on them.
 *   out: host pointer; receives {min_energy, argmin, count}.
 * The library allocates its workspace with hipMallocAsync on `stream` and frees
 * it before returning; the call is blocking (it synchronises `stream`).
 * Ties: argmin is the lowest index among all minimisers, count is exact. */
QUBO_API int qubo_search(const int32_t *Q, int n, int prefix_bits, int cache_bits, void *stream,
                qubo_result *out);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): qubo_search without
 * any allocation.  Same arguments, result, blocking and error behaviour as
 * qubo_search; in place of the stream-ordered workspace, every call on a GPU
 * uses one static device buffer of QUBO_NOALLOC_BYTES (128 MiB) that the
 * library holds on each GPU it runs on until the process ends.
 *   - Sizes: the plan's workspace (U, E_s, M_int, 4 x 2^prefix_bits bytes of
 *     prefix energies with their body and group minima, 64 bytes per
 *     workgroup, 256 bytes) must fit the buffer, else QUBO_ESCRATCH before any
 *     device work.  The planner's default split fits up to n = 40 (73 MiB at
 *     n = 40); larger n fit with a smaller prefix_bits while M_int stays small
 *     (n = 42 at prefix_bits 24: 92 MiB); n = 48 does not fit.
 *   - The buffer keeps the last call's contents; every call writes what it
 *     reads before reading it (its tables, partials and counters come from its
 *     own kernels, with no memset), so nothing carries over between calls.
 *   - Calls that overlap on one GPU race on the buffer: serialise them (one
 *     stream, or one call at a time per GPU).
 *   - No HIP events are created: qubo_last_timing then reports the coverage
 *     counters and the zero stage times. */
#define QUBO_NOALLOC_BYTES (128u << 20)
QUBO_API int qubo_search_noalloc(const int32_t *Q, int n, int prefix_bits, int cache_bits, void *stream,
                                 qubo_result *out);

/* Per-stage device times and coverage counters of the last search on this host
 * thread; times come from HIP events recorded on the call's stream around each
 * stage.  Zero before any call. */
typedef struct {
    float build_ms;   /* cache-builder kernels: E_s, M_int, Gray-ordered E_p */
    float search_ms;  /* the Gray-walk search kernel */
    float reduce_ms;  /* the final min/argmin/count reduction */
    float total_ms;   /* from the first upload to the result download */
    uint64_t states;  /* states searched */
    int32_t blocks;   /* workgroups launched */
    uint32_t cols_per_lane; /* suffix columns per lane of the search kernel (8 or 16; 8 for a
                               binary64 Q) */
    uint64_t bodies;  /* 32-step bodies walked, each over the 64 x cols_per_lane suffix
                         columns of one wave (coverage: bodies x 32 x 64 x cols_per_lane
                         = Gray steps x 2^B rounded up to whole column groups) */
    uint64_t checked_bodies; /* bodies that ran the per-step minimum (all of them in strict mode) */
    uint64_t slow_bodies;    /* bodies re-walked on the exact path (records and ties) */
    uint64_t candidates;     /* real-valued search: states re-evaluated from the definition */
} qubo_timing;
QUBO_API int qubo_last_timing(qubo_timing *out);

/* Search a slice of the state space: every suffix of every prefix g(j) =
 * j ^ (j >> 1) (as an A-bit number, variable 0 most significant) for
 * gray_lo <= j < gray_hi, where A is the prefix size of the plan (prefix_bits
 * must be given explicitly, 5 <= prefix_bits <= n).  gray_lo and gray_hi must be
 * multiples of 32 with gray_lo < gray_hi <= 2^A.  The range [m 2^(A-k),
 * (m+1) 2^(A-k)) is exactly the sub-cube whose first k variables spell g(m)
 * (the straightforward split of sec. III.C.1).  n must be at least 5.  Same
 * ownership, blocking and error behaviour as qubo_search; count may be 0 only
 * if the slice is empty (it never is for valid arguments). */
QUBO_API int qubo_search_range(const int32_t *Q, int n, int prefix_bits, int cache_bits, uint64_t gray_lo,
                      uint64_t gray_hi, void *stream, qubo_result *out);

/* Search with options.  gray_lo = gray_hi = 0 searches the whole space (as
 * qubo_search); any other pair selects a slice exactly as qubo_search_range.
 * flags: 0, or QUBO_FLAG_STRICT_MIN to take the minimum over every prefix's
 * suffix vector after every Gray step, as Algorithm 2 does.  By default the
 * kernel first bounds, for each block of 32 consecutive Gray steps, the lowest
 * energy any of its states can have (its suffix-dependent energies can fall by
 * at most the sum of the negative parts of the 5 row updates it applies, and its
 * prefix energies are at least their minimum over the block); blocks whose bound
 * exceeds the best energy found so far apply only the row updates (one add per
 * state).  Both modes return identical results; unknown flag bits are
 * rejected with QUBO_EINVAL. */
#define QUBO_FLAG_STRICT_MIN 1u
/* Kernel build: 8 or 16 suffix columns per lane (default: the planner's choice).
 * Both give identical results; at most one may be set. */
#define QUBO_FLAG_COLS8 2u
#define QUBO_FLAG_COLS16 4u
/* Outer split (sec. III.C.1): QUBO_FLAG_SPLIT(k) fixes the first k variables
 * (1 <= k <= n - 5) and searches the 2^k sub-problems one launch after another,
 * each capped by the best energy found so far; 0 = automatic (only above 58
 * variables).  Not combinable with a slice (gray_lo/gray_hi). */
#define QUBO_FLAG_SPLIT_SHIFT 8
#define QUBO_FLAG_SPLIT_MASK (0x3fu << QUBO_FLAG_SPLIT_SHIFT)
#define QUBO_FLAG_SPLIT(k) (((uint32_t)(k) << QUBO_FLAG_SPLIT_SHIFT) & QUBO_FLAG_SPLIT_MASK)
QUBO_API int qubo_search_ex(const int32_t *Q, int n, int prefix_bits, int cache_bits, uint64_t gray_lo,
                            uint64_t gray_hi, uint32_t flags, void *stream, qubo_result *out);

/* The low-energy spectrum: the k lowest states (sec. VI.B, "Future Work",
 * proposes keeping a list of the k lowest energies in the kernel instead of one
 * minimum; sec. I.D notes that brute force gives the low-energy spectrum).
 * The order is energy ascending, then index ascending: the result is the first
 * k states of that order, which is unique.  One entry (16 bytes): */
typedef struct {
    int32_t energy;   /* E(x) */
    uint32_t reserved;/* zero */
    uint64_t index;   /* idx(x), variable 0 most significant */
} qubo_state;
#define QUBO_MAX_LOWEST 64
/* Q, n, prefix_bits, cache_bits, gray_lo, gray_hi, stream: as for
 * qubo_search_ex (a slice restricts the spectrum to the slice's states).
 *   k: 1..QUBO_MAX_LOWEST.
 *   flags: QUBO_FLAG_COLS8 / QUBO_FLAG_COLS16 / QUBO_FLAG_SPLIT(k) as for
 *      qubo_search_ex; QUBO_FLAG_STRICT_MIN is rejected (the spectrum search is
 *      always bound-gated).  Above 58 variables the sub-problems run in order,
 *      each capped by the k-th energy found so far.
 *   out: host pointer to k entries; entries 0..*found-1 receive the states in
 *      order, the rest are left untouched.
 *   found: host pointer; min(k, number of states searched).
 * Each wave of the search keeps its own k lowest states, one per lane; the
 * threshold of the bound gate is the lowest k-th energy of any wave so far.  A
 * final one-workgroup kernel merges the per-wave lists.  Blocking; same
 * ownership and error behaviour as qubo_search_ex. */
QUBO_API int qubo_search_lowest(const int32_t *Q, int n, int k, int prefix_bits, int cache_bits,
                                uint64_t gray_lo, uint64_t gray_hi, uint32_t flags, void *stream,
                                qubo_state *out, int *found);

/* A real-valued Q (sec. VI.B names floating-point matrices as future work,
 * with the rounding that long incremental Gray-code updates accumulate as the
 * difficulty).  Definition used here: E(x) is the binary64 sum of Q_ij over i
 * ascending with x_i = 1 and, inside, j ascending with x_j = 1, each add
 * rounded to nearest (the sum of sec. I in one fixed order); min_energy is the
 * smallest such value, argmin the lowest index attaining it exactly, count the
 * number of states attaining it exactly.  Result (24 bytes): */
typedef struct {
    double min_energy;
    uint64_t argmin;
    uint64_t count;
} qubo_result_f64;
/* Q: device pointer, n x n binary64, row-major; read only.  n: 1..58 (no
 * outer split).  prefix_bits, cache_bits, gray_lo, gray_hi, stream: as for
 * qubo_search_ex (the same planner and defaults).
 * flags: 0 or QUBO_FLAG_COLS8.  Every entry must be finite and S = sum |Q_ij|
 * either 0 or in [2^-100, 2^100] (else QUBO_ERANGE; qubo_check_q_f64).
 * The walk is the integer kernel's (one int32 add per state) over the tables
 * of eq. 8 formed in binary64, scaled by s = 2^e (s S <= 2^17, or up to 2^28
 * for a matrix whose entries spread over many orders of magnitude) and rounded
 * to integers once each; a state's walked value then lies within A/2 + 2 of
 * s E(x), and a state whose walked value comes within M = A/2 + 3 of s times
 * the best exact energy so far (about 2^-13 S) is re-evaluated from the
 * definition on the GPU, so the result is exactly the definition's.  A dyadic
 * Q (every entry an integer multiple of 2^-f with sum |2^f Q_ij| <= 2^30 - 1,
 * integer-valued matrices included), whose definition sums are all exact, is
 * searched as the int32 matrix 2^f Q by the integer search instead.  Other
 * instances with many states that close to the minimum are correct but slow:
 * each such state costs an O(n^2) evaluation.  Blocking; same ownership
 * and error behaviour as qubo_search_ex; qubo_last_timing reports the
 * re-evaluated states. */
QUBO_API int qubo_search_f64(const double *Q, int n, int prefix_bits, int cache_bits,
                             uint64_t gray_lo, uint64_t gray_hi, uint32_t flags, void *stream,
                             qubo_result_f64 *out);

/* The k lowest states of a binary64 Q (the definition of qubo_search_f64): the
 * first k states in the order (energy ascending, index ascending), as
 * qubo_search_lowest does for int32.  k: 1..QUBO_MAX_LOWEST.  Arguments, limits
 * and errors as for qubo_search_f64; out: host pointer to k entries, entries
 * 0..*found-1 receive the states in order; found: min(k, states searched).
 * Every state whose walked value comes within the margin of the lowest k-th
 * exact energy of any wave is re-evaluated from the definition, so the list is
 * exactly the definition's. */
typedef struct {
    double energy;
    uint64_t index;
} qubo_state_f64;
QUBO_API int qubo_search_lowest_f64(const double *Q, int n, int k, int prefix_bits, int cache_bits,
                                    uint64_t gray_lo, uint64_t gray_hi, uint32_t flags, void *stream,
                                    qubo_state_f64 *out, int *found);

/* A search run in steps, so that a long search (n = 58 takes about an hour,
 * n = 63 about 35 hours) can be stopped and resumed, or its steps spread over
 * time.  The work units are independent (sec. III.C), so the state space is
 * walked as the 2^k sub-problems of the outer split (sec. III.C.1; k = 0 for
 * n <= 58 unless asked for), each as consecutive slices of 2^chunk_bits Gray
 * steps of its prefix walk (qubo_search_range), and the slices' results are
 * combined by the rule of the final reduction (sec. III.C: minimum, count at
 * the minimum, lowest index).  The whole state of the run is this plain struct
 * (96 bytes, no pointers): the caller keeps it between calls, in memory or in
 * a file, and the same Q continues the run from it. */
typedef struct {
    uint64_t q_hash;      /* fingerprint of n and Q (FNV-1a over the int32 entries) */
    int32_t n;            /* variables */
    int32_t split_bits;   /* k: first k variables fixed per sub-problem (0: one problem) */
    int32_t prefix_bits;  /* A of each (sub-)problem of n - k variables */
    int32_t chunk_bits;   /* each step searches 2^chunk_bits Gray steps (all suffixes) */
    uint64_t sub;         /* current sub-problem: the values of the first k variables */
    uint64_t next;        /* first Gray step of the next slice of the current sub-problem */
    uint64_t steps_done;  /* slices searched or skipped so far */
    uint64_t steps_total; /* 2^k * 2^(A - chunk_bits) */
    int32_t done;         /* 1 once every state has been searched */
    int32_t have_best;    /* 1 once best holds a searched state */
    union {                         /* the combined result of the slices searched so far */
        qubo_result best;           /* kind 0 */
        qubo_result_f64 best_f64;   /* kind 1 */
    };
    uint32_t kind;        /* 0: int32 Q (qubo_progress_init), 1: binary64 Q (qubo_progress_init_f64) */
    uint32_t reserved;    /* zero */
} qubo_progress;

/* Starts a run: fills *p for Q (device pointer, n x n int32, as for qubo_search).
 *   prefix_bits: A of each (sub-)problem, or -1 for the planner's choice.
 *   chunk_bits:  Gray steps per step as a power of two, 5 <= chunk_bits <= A, or
 *                -1 for slices of about 2^48 states (a few seconds each).
 *   flags: 0 or QUBO_FLAG_SPLIT(k) as for qubo_search_ex (above 58 variables
 *          the split is automatic).  n - k must be at least 5.
 * Blocking (Q is read to form the fingerprint); error codes as qubo_search. */
QUBO_API int qubo_progress_init(const int32_t *Q, int n, int prefix_bits, int chunk_bits, uint32_t flags,
                                void *stream, qubo_progress *p);

/* Searches the next slice of the run in *p and folds its result into p->best.
 * Q and n must be the ones *p was started with (QUBO_EINVAL otherwise, checked
 * against the fingerprint).  A sub-problem whose every state lies above the
 * best energy found so far is skipped whole.  Once p->done is 1 the call does
 * nothing and returns QUBO_OK; p->best is then exactly qubo_search's result.
 * On error *p is untouched, so the step can be retried.  Blocking; same
 * ownership and error behaviour as qubo_search; qubo_last_timing reports the
 * step. */
QUBO_API int qubo_search_step(const int32_t *Q, int n, void *stream, qubo_progress *p);

/* A spectrum run in steps (the k lowest states, as qubo_search_lowest): the
 * run's header (kind 2; its best is unused) and the k lowest states found so
 * far (1128 bytes, no pointers).  Once k states are known, their k-th energy
 * caps every later slice and a sub-problem wholly above it is skipped. */
typedef struct {
    qubo_progress head;
    int32_t k;                               /* 1 .. QUBO_MAX_LOWEST */
    int32_t found;                           /* entries of states[] in use (<= k) */
    qubo_state states[QUBO_MAX_LOWEST];      /* (energy, index) ascending */
} qubo_progress_lowest;

/* Starts a spectrum run: arguments as for qubo_progress_init, plus k. */
QUBO_API int qubo_progress_init_lowest(const int32_t *Q, int n, int k, int prefix_bits, int chunk_bits,
                                       uint32_t flags, void *stream, qubo_progress_lowest *p);
/* Searches the next slice and merges its k lowest states into p->states; once
 * p->head.done is 1, states[0 .. found) is exactly qubo_search_lowest's list. */
QUBO_API int qubo_search_step_lowest(const int32_t *Q, int n, void *stream, qubo_progress_lowest *p);

/* The same for a binary64 Q (qubo_search_f64's definition and limits: n from
 * 5 to 58, no outer split, so split_bits is 0).  The record has kind 1 and its
 * result in best_f64; every later slice starts from the best energy found so
 * far.  The int32 and binary64 steps refuse each other's records. */
QUBO_API int qubo_progress_init_f64(const double *Q, int n, int prefix_bits, int chunk_bits, void *stream,
                                    qubo_progress *p);
QUBO_API int qubo_search_step_f64(const double *Q, int n, void *stream, qubo_progress *p);

/* Builds the cache tables of a plan into caller-provided device buffers, for
 * inspection (sec. III.A preprocessing steps 1-3, eq. 8):
 *   Es:     2^B entries (int32): E_s(c), the energy of the suffix alone, c the
 *           column index of the suffix (suffix variable A+i is bit B-1-i of c);
 *   Mint:   A x 2^B entries (int32), row v = prefix variable v:
 *           M_int[v][c] = sum_j U_{v,A+j} xs_j(c), the prefix-suffix interaction;
 *   EpGray: 2^A entries (int32): E_p(g(j)), the energy of the prefix alone in
 *           Gray order (sec. IV.B.3).
 * U is Q folded to the upper triangle.  Requires n >= 5 and an explicit
 * prefix_bits.  Blocking; same error codes as qubo_search. */
QUBO_API int qubo_build_tables(const int32_t *Q, int n, int prefix_bits, int32_t *Es, int32_t *Mint,
                      int32_t *EpGray, void *stream);

/* Human-readable name of a status code; never NULL. */
QUBO_API const char *qubo_strerror(int status);

/* Library version and build target. */
QUBO_API const char *qubo_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QUBO_H */
