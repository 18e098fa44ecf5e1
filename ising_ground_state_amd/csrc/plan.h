// Host-side planning for the QUBO search: folding Q, the overflow guard and the
// choice of the prefix/suffix split and cache size.  Pure C++, no HIP.
#pragma once

#include <cstdint>
#include <vector>

#include "qubo.h"

namespace qubo {

// Compile-time shape of the search kernel.
constexpr int kRegBits = 5;        // Gray bits whose M_int rows live in VGPRs
constexpr int kGateBits = kRegBits + 4;  // and with the pair and group gates' bits: rows the gates read
constexpr int kDefaultColsPerLane = 8;  // suffix columns per lane (R); 16 is the other build
constexpr int kWave = 64;                // CDNA wavefront
constexpr int kWavesPerBlock = 4;        // one wave per SIMD of a CU
constexpr int kMinSearchVars = kRegBits; // n below this is padded
constexpr int kMaxPrefixBits = 32;       // prefix-energy table <= 2^32 entries
constexpr int kMaxLdsBytes = 65536;      // cached rows per workgroup
constexpr uint64_t kMaxMintBytes = 1ull << 33;  // 8 GiB
constexpr int kMaxSingleVars = 58;       // largest n searched by a single launch
constexpr int kMaxSplitBits = 32;        // at most 2^32 sub-problems
constexpr int kMaxSegBits = 18;          // Gray steps per work unit at most 2^18 (a fine tail)
constexpr int kMinSegBits = 12;          // and at least 2^12 where the prefix walk allows,
constexpr int kMinSegBitsIdle = 10;      // or 2^10 when longer units would leave waves idle
// Work items are handed out in kItemParts parts, one per XCD of an MI355X, in
// tiles of 2^kTileGroupBits column groups by 2^kTileBlockBits segment blocks
// (item_place, item_part; walk.h).
constexpr int kItemParts = 8;
constexpr int kTileGroupBits = 5;
constexpr int kTileBlockBits = 5;

// ceil(log2(v)) for v >= 1.
constexpr int ceil_log2_u64(uint64_t v) { return v <= 1 ? 0 : 64 - __builtin_clzll(v - 1); }

// The order of the work items of a search with G column groups and SB segment
// blocks (an item: one column group, four consecutive segments).  The items
// run over the 2^lg_g x 2^lg_s slots of the grid rounded up to powers of two
// (lg_g = ceil_log2(G), lg_s = ceil_log2(SB)); slots outside G x SB are empty.
// Slot i lies in a tile of up to 2^kTileGroupBits column groups by
// 2^kTileBlockBits segment blocks; the tiles run in rows, row after row, and
// inside a tile the column group runs fastest: the bits of i are, from the top,
// the row, the tile in the row, the block in the tile and the group in the
// tile.  A bijection of [0, 2^(lg_g + lg_s)) onto the (group, block) slots,
// by shifts and masks.  constexpr: the device code and the host's checks call
// the same function.
struct ItemPlace {
    uint64_t group, block;
};
constexpr ItemPlace item_place(uint64_t i, int lg_g, int lg_s)
{
    const int tg = lg_g < kTileGroupBits ? lg_g : kTileGroupBits;
    const int ts = lg_s < kTileBlockBits ? lg_s : kTileBlockBits;
    const uint64_t in_tile = i & ((1ull << (tg + ts)) - 1);
    const uint64_t tile = (i >> (tg + ts)) & ((1ull << (lg_s - ts)) - 1);
    const uint64_t row = i >> (tg + lg_s);
    return ItemPlace{(row << tg) | (in_tile & ((1ull << tg) - 1)), (tile << ts) | (in_tile >> tg)};
}

// Part p of the slot order: kItemParts contiguous ranges [lo, lo + len) of
// ceil(slots / kItemParts) slots (the last ones shorter or empty).
struct ItemPart {
    uint64_t lo, len;
};
constexpr ItemPart item_part(uint64_t slots, uint32_t p)
{
    const uint64_t part_len = (slots + kItemParts - 1) / kItemParts;
    const uint64_t lo = (uint64_t)p * part_len;
    const uint64_t len = lo >= slots ? 0 : (slots - lo < part_len ? slots - lo : part_len);
    return ItemPart{lo, len};
}

constexpr int64_t kAbsSumLimit = (1ll << 30) - 1;

// The gates' table of a search (built by launch_gate_tables, read by the walk):
// the group bound of each aligned group of sixteen 32-step bodies (at least one)
// and a padding entry; from gate_pairs_at(A) the pair bound of each aligned
// pair of bodies; from gate_lane_bounds_at(A) the lane bounds, per column group
// six rows of 64 (one entry per lane).  The group bounds, read once per group,
// stay 4 bytes apart.
constexpr uint64_t gate_groups(int A) { return A > kRegBits + 4 ? 1ull << (A - kRegBits - 4) : 1ull; }
constexpr uint64_t gate_pair_count(int A) { return A > kRegBits + 1 ? 1ull << (A - kRegBits - 1) : 1ull; }
constexpr uint64_t gate_pairs_at(int A) { return gate_groups(A) + 1; }
constexpr uint64_t gate_lane_bounds_at(int A) { return (gate_pairs_at(A) + gate_pair_count(A) + 63) & ~63ull; }

// Folds a full n x n matrix into the upper triangle U (U_ii = Q_ii,
// U_ij = Q_ij + Q_ji for i < j, 0 below), so x^T Q x = x^T U x, after checking
// sum |Q_ij| <= 2^30 - 1.  Returns QUBO_OK or QUBO_ERANGE; writes the sum.
int fold_upper(const int32_t *Q, int n, std::vector<int32_t> &U, int64_t *abs_sum);

// Pads a folded n x n matrix to n_search >= n variables: the extra variables get
// U_ii = +1 and no couplings, so they are 0 in every minimiser.
std::vector<int32_t> pad_upper(const std::vector<int32_t> &U, int n, int n_search);

// Energies of distinct states of the folded matrix U (n x n upper triangle,
// n <= 63), ascending: the states that steepest single-flip descents reach
// from state 0 and from starts - 1 fixed pseudo-random states (SplitMix64, a
// fixed seed), and their single-flip neighbours, with the first `fixed`
// variables held at the bits of fixed_value (variable 0 its most significant
// of `fixed` bits) throughout: states of that sub-cube only.  Exact in int64.
// The first is a real energy and the j-th bounds the j-th lowest energy of the
// sub-cube (and of any set holding it) from above: first thresholds of a
// search, so that the bound gates clear bodies from the start.  Only the
// thresholds depend on the starts, never a search's result.
std::vector<int64_t> descent_energies(const std::vector<int32_t> &U, int n, int starts, int fixed = 0,
                                      uint64_t fixed_value = 0);
constexpr int kDescentStarts = 16;

// The states of the Gray steps [lo, hi) of an A-bit prefix walk (lo < hi <=
// 2^A) hold a sub-cube: the prefixes g(j) of the largest aligned block of steps
// [m 2^s, (m + 1) 2^s) inside the range share their first A - s variables,
// which spell g(m) (sec. III.C.1).  Writes A - s and g(m).
void largest_subcube(uint64_t lo, uint64_t hi, int A, int *fixed, uint64_t *fixed_value);

// Fills `out` for n variables on a device with `num_cus` compute units;
// cols_per_lane is 8 or 16, or 0 for the default.  split_bits: -1 splits only
// above kMaxSingleVars (by n - kMaxSingleVars fixed variables), 0 never, k > 0
// fixes the first k variables; the plan then describes each sub-problem of
// n - k variables (prefix_bits and cache_bits apply to it).
int make_plan(int n, int prefix_bits, int cache_bits, int num_cus, int cols_per_lane,
              int split_bits, qubo_plan *out);

// The straightforward split of sec. III.C.1 for the k-bit assignment f of the
// first k variables (variable 0 is the most significant bit of f): the folded
// (n-k) x (n-k) matrix of the remaining variables, with U_ii increased by the
// couplings to the fixed ones that are set, and the constant c(x_f) = energy of
// the fixed variables alone.  Writes sum |Usub_ij| to *sub_abs.
void reduce_fixed(const std::vector<int32_t> &U, int n, int k, uint64_t f,
                  std::vector<int32_t> &Usub, int64_t *c, int64_t *sub_abs);

// Offsets of the search's tables that keep the walked energies E_s(c) + sum of
// the set prefix variables' rows, and every row, at or above zero, so that the
// walk's registers and the rows it adds never change sign (a register that
// crosses zero switches all of its high bits, and so does the operand path
// between rows of either sign; a walk over values of one sign ran the chip at a
// higher clock).  Each row v < A is raised by K[v] = sum_j max(0, -U[v][A+j]),
// E_s by es_add = sum_{A <= i <= j} max(0, -U_ij), and the prefix energies carry
// the same amounts lowered: -es_add, and U's prefix diagonal lowered by K[v]
// (Uoff, the builders' copy of U).  E(x) = E_s + rows + E_p holds unchanged for
// every state, and every entry stays within sum |U_ij| of zero.  kgate: K of the
// rows of Gray bits 0..8 (variable A-1-t), which the bound gates take off their
// rows and out of their prefix minima (walk.h).
struct TableOffsets {
    int rows;
    int64_t es_add;
    std::vector<int32_t> Uoff;
    int32_t kgate[16];
};
TableOffsets table_offsets(const std::vector<int32_t> &U, int ns, int A);

// Device workspace layout of a plan (byte offsets, all 256-aligned).
struct Layout {
    uint64_t cols_padded;  // 2^B rounded up to a multiple of the column-group size
    uint64_t off_u, off_es, off_mint, off_ep, off_epmin, off_gates, off_partials, off_ctrl;
    uint64_t total;
};
Layout layout_of(const qubo_plan &p);

}  // namespace qubo
