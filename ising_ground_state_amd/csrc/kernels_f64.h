// Device-side pieces of the search for a real-valued (binary64) Q and their
// launchers (HIP, gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qubo {

// Suffix columns per lane of the binary64 search (four waves per SIMD).  Four columns fit six waves but ran 10 % slower: a body's fixed work
// then covers half as many states.
constexpr int kColsPerLaneF64 = 8;

// The lowest Gray bit whose binary64 row the search keeps in LDS: the anchor of
// a column moves once per aligned group of 32 32-step bodies, by the rows of
// Gray bit 9 and of one bit above it.
constexpr int kLdsFirstBitF64 = 9;

// One workgroup's partial result (48 bytes).
struct PartialF64 {
    double e;            // min energy seen (+inf when count == 0)
    uint64_t count;      // states with exactly that energy
    uint64_t arg;        // smallest index attaining it
    uint64_t bodies;     // 32-step bodies walked
    uint32_t slow;       // bodies walked exactly
    uint32_t pad;
    uint64_t candidates; // states re-evaluated from the definition
};

// One entry of a k-lowest list: a state's binary64 energy and index (16 bytes).
struct LowEntryF64 {
    double e;    // +inf for an empty slot
    uint64_t x;
};

struct CtrlF64 {
    unsigned long long counter;  // next work item
    long long gbest;             // upper bound of the minimum, as an order-preserving integer key
    uint64_t pad[6];
    PartialF64 result;           // final reduction (offset 64)
    uint64_t slow_total;
    uint64_t bodies_total;
    uint64_t candidates_total;
};

struct SearchArgsF64 {
    const double *es;       // [cols_padded]       E_s(c)
    const double *mint;     // [A][cols_padded]    M_int rows by prefix variable
    const float *mint32;    // [A][cols_padded]    the same rows rounded to fp32 (the walk's rows)
    const double *ep;       // [2^A]               E_p(g(j))
    const float *epmin;     // [2^A / 32 + 2]      min over each body of ep rounded to fp32, + 2 padding
    const float *epmin4;    // [2^A / 128 + 1]     min of epmin over each aligned group of 4 bodies, + 1 padding
    const double *Q;        // [n][n]              the caller's matrix (the definition's terms)
    PartialF64 *partials;   // [gridDim.x]: one per workgroup
    CtrlF64 *ctrl;
    LowEntryF64 *lists;     // k-lowest search: [gridDim.x * 4][k_low], else unused
    uint64_t cols_padded;
    uint64_t gray_lo, gray_hi;
    uint64_t seg_first, segs, seg_blocks, items;
    int32_t A, B;
    int32_t n;              // variables of Q
    int32_t pad;            // padding variables appended below n (n < 5), the lowest index bits
    int32_t l_eff;          // Gray bits with rows on chip (registers + LDS)
    int32_t seg_bits;
    float delta;            // filter margin: bounds every fp32 rounding of the walk and the gate
    int32_t k_low;          // k-lowest search: states kept per wave (1..64), else 0
};

// E_s, M_int and E_p(g(j)) in binary64 from the folded matrix, M_int rounded to
// fp32, and the per-body minima of E_p rounded to fp32.
// Only the prefix energies of the Gray steps [j_lo, j_hi) are written (multiples
// of 32; the tables keep their full size).
hipError_t launch_build_tables_f64(const double *U, int ns, int A, int B, uint64_t cols_padded,
                                   double *es, double *mint, float *mint32, double *ep,
                                   float *epmin, float *epmin4, uint64_t j_lo, uint64_t j_hi,
                                   hipStream_t stream);

hipError_t launch_init_ctrl_f64(CtrlF64 *ctrl, double t0, float *epmin_pad, float *epmin4_pad,
                                hipStream_t stream);

// lowest: the k-lowest search (each wave keeps its k lowest states in
// args.lists) instead of the minimum, count and lowest minimiser.
hipError_t launch_search_f64(const SearchArgsF64 &args, bool lowest, int blocks, int lds_bytes,
                             hipStream_t stream);

hipError_t search_occupancy_f64(bool lowest, int *blocks_per_cu, int lds_bytes);

// Merges `count` entries (the per-wave lists, each sorted) into the k lowest
// by (energy, index); writes k entries to out and their number to *found.
hipError_t launch_lowest_merge_f64(const LowEntryF64 *lists, uint64_t count, int k, LowEntryF64 *out,
                                   int32_t *found, hipStream_t stream);

hipError_t launch_reduce_f64(const PartialF64 *partials, int count, CtrlF64 *ctrl,
                             hipStream_t stream);

}  // namespace qubo
