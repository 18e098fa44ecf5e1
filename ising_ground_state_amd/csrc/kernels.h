// Device-side pieces of the QUBO search and their launchers (HIP, gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "walk.h"

namespace qubo {

// One workgroup's partial result (40 bytes) with its coverage counters.
struct Partial {
    int32_t e;         // min energy seen (INT32_MAX when count == 0)
    uint32_t slow;     // bodies re-walked on the exact path (records and ties)
    uint64_t count;    // states attaining e
    uint64_t arg;      // smallest index attaining e
    uint64_t bodies;   // 32-step bodies walked (each over 64 x cols_per_lane columns)
    uint32_t checked;  // bodies that ran the per-step minimum
    uint32_t pad;
};
constexpr int kPartialBytes = 64;  // workspace bytes reserved per workgroup's partial
static_assert(sizeof(Partial) <= kPartialBytes, "partial slot");

// One entry of a low-energy list: a state's energy and index (16 bytes).
// e == INT32_MAX marks an empty slot (no energy reaches it: |E| <= 2^30 - 1).
struct LowEntry {
    int32_t e;
    uint32_t pad;
    uint64_t x;
};

constexpr int kMaxLowest = 64;  // one list entry per lane of a wave

struct Ctrl {
    int32_t gbest;               // best energy found by any wave so far (a real state's energy)
    int32_t pad0;
    uint64_t pad1[7];
    Partial result;              // final reduction (offset 64)
    uint64_t slow_total;
    uint64_t bodies_total;
    uint64_t checked_total;
    unsigned long long counter[kItemParts];  // next work item of each part
};
static_assert(sizeof(Ctrl) <= 256, "control block slot");

// Row offsets of the Gray bits t < 9 whose rows the bound gates read (K of
// prefix variable A-1-t; zero past A, and zero for tables without offsets).
struct GateOffsets {
    int32_t k[16];
};

struct SearchArgs {
    const int32_t *es;      // [cols_padded]       suffix energies E_s(c)
    const int32_t *mint;    // [A][cols_padded]    M_int rows by prefix variable
    const int32_t *ep;      // [2^A]               prefix energies in Gray order
    const int32_t *epmin;   // [2^A / 32 + 2]      min of ep over each 32-step body, + 2 padding
    const int32_t *gates;   // [gate_lane_bounds_at(A) + 6 cols_padded / R]  the gates' table (walk.h)
    Partial *partials;      // [gridDim.x]: one per workgroup
    Ctrl *ctrl;
    LowEntry *lists;        // [gridDim.x * waves per block][k_low] (spectrum search only)
    uint64_t cols_padded;
    uint64_t gray_lo, gray_hi;  // Gray steps searched: [gray_lo, gray_hi)
    uint64_t seg_first;         // first segment (2^seg_bits steps each) touching the range
    uint64_t segs;              // segments touching the range
    uint64_t seg_blocks;        // ceil(segs / waves per block)
    uint64_t items;             // col_groups * seg_blocks
    int32_t A, B;
    int32_t l_eff;              // Gray bits with rows on chip (registers + LDS)
    int32_t seg_bits;
    int32_t k_low;              // spectrum search: states kept per wave (1..64); else 0
    int32_t pad;
};

// Cache builder (Maltsev et al., sec. III.A preprocessing, eq. 8): E_s, M_int
// and the Gray-ordered prefix energies, from the folded upper-triangular U.
// Only the prefix energies a search of the Gray steps [j_lo, j_hi) reads are
// written (j_lo, j_hi multiples of 32; the tables keep their full size),
// with the minimum of each 32-step body (epmin).
// Offsets (zero for eq. 8's own tables): E_s is raised by es_add and the prefix
// energies lowered by it; the rows of the prefix variables v < offset_rows are
// raised by K[v] = sum_j max(0, -U[v][A+j]), which U's prefix diagonal must
// carry lowered by K[v] (the caller's copy of U), so that E_s + the rows of the
// set prefix variables + E_p stays E(x) for every state.  kg: the offsets of
// the rows of Gray bits 0..6 (K[A-1-t]); the body minima epmin are taken
// relative to each body's first step (walk.h).
hipError_t launch_build_tables(const int32_t *U, int ns, int A, int B, uint64_t cols_padded,
                               int offset_rows, int32_t es_add, const GateOffsets &kg, int32_t *es,
                               int32_t *mint, int32_t *ep, int32_t *epmin, uint64_t j_lo, uint64_t j_hi,
                               hipStream_t stream);

// The gates' table of a search (integer or over rounded tables; layout in
// walk.h), from its rows and body minima (epmin, relative to each body's first
// step) for the Gray steps [j_lo, j_hi):
//   gates[k]           the group bound of bodies 16k .. 16k+15, relative to the
//                      group's first step (A >= 9);
//   gates[gate_pairs_at(A) + p]  the pair bound of bodies 2p and 2p+1,
//                      relative to the pair's first step (A >= 6);
//   then the lane bounds, six rows of 64 per column group (one entry per lane,
//   R columns each): the bound on the fall of its suffix energies within a body
//   (bit 4 clear or set at its start), a pair (bit 5) and a group (bit 8), over
//   the rows less their offsets kg; padding columns count 0.
// Pairs and groups that straddle the slice's ends get values that are never
// read; the padding group bound (gates[gate_groups(A)]) is set by the
// control-block reset.
hipError_t launch_gate_tables(const int32_t *mint, uint64_t cols_padded, int A, int B, int R,
                              const GateOffsets &kg, const int32_t *epmin, int32_t *gates, uint64_t j_lo,
                              uint64_t j_hi, hipStream_t stream);

// Entries of the gates' table of a plan.
inline uint64_t gate_table_len(int A, uint64_t cols_padded, int R)
{
    return gate_lane_bounds_at(A) + 6 * (cols_padded / (uint64_t)R);
}

// Resets the work counter, seeds the shared best with t0 (a real energy or an
// upper bound) and fills the body-minimum table's two padding entries and the
// group bound of the gates' table's padding record.
hipError_t launch_init_ctrl(Ctrl *ctrl, int32_t t0, int32_t *epmin_pad, int32_t *gates_pad,
                            hipStream_t stream);

// gated = true skips the per-step minimum of bodies whose lower bound cannot
// reach the threshold; gated = false takes it after every prefix (strict).
// cols_per_lane selects the instantiation (8 or 16 suffix columns per lane).
// lowest = true (gated only) keeps each wave's k_low lowest states in
// args.lists instead of the minimum, count and lowest minimiser.
hipError_t launch_search(const SearchArgs &args, int cols_per_lane, bool gated, bool lowest,
                         int blocks, int lds_bytes, hipStream_t stream);

// Resident workgroups of the search kernel per CU for a given dynamic LDS size.
hipError_t search_occupancy(int cols_per_lane, bool gated, bool lowest, int *blocks_per_cu,
                            int lds_bytes);

hipError_t launch_reduce(const Partial *partials, int count, Ctrl *ctrl, hipStream_t stream);

// Merges `lists` (count entries: the per-wave lists of k states each, empty
// slots allowed) into the k lowest states overall, ordered by energy then
// index, in out[0..k); *found = number of non-empty entries written.
hipError_t launch_lowest_merge(const LowEntry *lists, uint64_t count, int k, LowEntry *out,
                               int32_t *found, hipStream_t stream);

}  // namespace qubo
