// Device-side pieces of the search for a real-valued (binary64) Q and their
// launchers (HIP, gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"  // kItemParts

namespace qubo {

// Suffix columns per lane of the binary64 search (the integer search's default).
constexpr int kColsPerLaneF64 = 8;

// The walk's tables are the binary64 tables scaled by s = 2^e and rounded to
// integers, with e chosen so that s * sum |Q_ij| <= 2^q.  q = kQuantBits keeps
// about as many significant bits as the integer workloads of that size (wider
// words switch more bits per add and the chip then runs at a lower clock);
// matrices whose entries spread over many orders of magnitude get up to
// kQuantBitsMax, so that their small entries still rank states.
constexpr int kQuantBits = 17;
constexpr int kQuantBitsMax = 28;

// Padding columns of the rounded suffix energies: above every threshold the
// filter can take (at most 2^(q + 2) + 19 + 2^q + 67 <= 2^30 + 2^28 + 86 after
// subtracting a prefix energy, offsets included), so they are never
// candidates, and the sums the walk and its gates form from them (at most
// 3 * 2^29 + 2^28 + 67) stay below 2^31.  (A prefix energy with its offsets is
// at least -(s S + 2 A + 3): the rounded energy and the at most A + 1 offset
// bounds, each the ceiling of s times a part of S plus 1.)
constexpr int32_t kPadQ = 3 << 29;

// Integer offsets of the rounded tables, added after rounding: E_s is raised
// by es_add, the row of prefix variable v < rows by k[v], and every prefix
// energy lowered by es_add and by k[v] of its set variables v < rows.  Each
// state's walked value W(x) is unchanged; the offsets only keep the rows and
// the walked suffix energies at or above zero (the integer search's table
// offsets, with k[v] >= -min_c of the rounded row and es_add >= -min_c of the
// rounded E_s).  Every k[v] and es_add is at most 2^q + 2.  kgate[t] = k[A-1-t]
// for the Gray bits t < 9 (zero past A): the gates' share (walk.h).
struct TableOffsetsF64 {
    int32_t rows;
    int32_t es_add;
    int32_t k[32];
    int32_t kgate[16];
};

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
    long long gbest;             // upper bound of the minimum, as an order-preserving integer key
    uint64_t pad[7];
    PartialF64 result;           // final reduction (offset 64)
    uint64_t slow_total;
    uint64_t bodies_total;
    uint64_t candidates_total;
    unsigned long long counter[kItemParts];  // next work item of each part
};

struct SearchArgsF64 {
    const int32_t *es;      // [cols_padded]       rint(s E_s(c)); kPadQ for padding columns
    const int32_t *mint;    // [A][cols_padded]    rint(s M_int) rows by prefix variable
    const int32_t *ep;      // [2^A]               rint(s E_p(g(j)))
    const int32_t *epmin;   // [2^A / 32 + 2]      min of ep over each 32-step body, + 2 padding
    const int32_t *gates;   // [gate_lane_bounds_at(A) + 6 cols_padded / 8]  the gates' table (walk.h)
    const double *Q;        // [n][n]              the caller's matrix (the definition's terms)
    PartialF64 *partials;   // [gridDim.x]: one per workgroup
    CtrlF64 *ctrl;
    LowEntryF64 *lists;     // k-lowest search: [gridDim.x * 4][k_low], else unused
    uint64_t cols_padded;
    uint64_t gray_lo, gray_hi;
    uint64_t seg_first, segs, seg_blocks, items;
    double scale;           // s = 2^e
    int32_t A, B;
    int32_t n;              // variables of Q
    int32_t pad;            // padding variables appended below n (n < 5), the lowest index bits
    int32_t l_eff;          // Gray bits with rows on chip (registers + LDS)
    int32_t seg_bits;
    int32_t margin;         // M: |W(x) - s E(x)| < M - 1 for every state (rounding and binary64 error)
    int32_t cap;            // filter threshold above every rounded energy (2^(q + 2))
    int32_t k_low;          // k-lowest search: states kept per wave (1..64), else 0
    int32_t pad1;
};

// The rounded tables from the folded binary64 matrix U (ns x ns upper triangle):
// E_s and M_int per column, E_p(g(j)) for the Gray steps [j_lo, j_hi)
// (multiples of 32; the tables keep their full size), each sum formed in
// binary64 and then scaled by `scale` and rounded to the nearest integer once;
// the per-body minima of the rounded prefix energies (relative to each body's
// first step); with the integer offsets `off` added after rounding.  The
// gates' other tables come from launch_gate_tables (kernels.h).
hipError_t launch_build_tables_f64(const double *U, int ns, int A, int B, uint64_t cols_padded,
                                   double scale, const TableOffsetsF64 &off, int32_t *es, int32_t *mint,
                                   int32_t *ep, int32_t *epmin, uint64_t j_lo, uint64_t j_hi,
                                   hipStream_t stream);

// Resets the work counter, seeds the shared bound with t0 and fills the
// padding entries of the body and group minima.
hipError_t launch_init_ctrl_f64(CtrlF64 *ctrl, double t0, int32_t *epmin_pad, int32_t *gates_pad,
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
