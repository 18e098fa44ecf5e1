// Host-side planning: fold, overflow guard, prefix/suffix split and cache size.
//
// The split follows Maltsev et al., "Terastate-per-second QUBO Brute-Force on a
// Single GPU", sec. II.A (x = [x_p, x_s], A + B = N) and sec. III.C: suffix
// columns are spread over lanes and workgroups (column-wise split, III.C.2) and
// the Gray walk over the prefix is cut into segments handed to waves (a split
// over ranges of the prefix walk, in the spirit of III.C.1).  The paper tunes
// A and B empirically for the register file of its GPU (sec. IV.B.1); here the
// register budget is fixed by the kernel's compile-time shape (8 or 16 columns
// and 5 cached rows per lane) and the planner only sizes tables and work units.
#include "plan.h"

#include <algorithm>
#include <cstdlib>
#include <unordered_set>

namespace qubo {

int fold_upper(const int32_t *Q, int n, std::vector<int32_t> &U, int64_t *abs_sum)
{
    int64_t s = 0;
    for (int64_t k = 0; k < (int64_t)n * n; ++k)
        s += std::llabs((int64_t)Q[k]);
    if (abs_sum)
        *abs_sum = s;
    if (s > kAbsSumLimit)
        return QUBO_ERANGE;
    U.assign((size_t)n * n, 0);
    for (int i = 0; i < n; ++i) {
        U[(size_t)i * n + i] = Q[(size_t)i * n + i];
        for (int j = i + 1; j < n; ++j)
            U[(size_t)i * n + j] = Q[(size_t)i * n + j] + Q[(size_t)j * n + i];
    }
    return QUBO_OK;
}

std::vector<int32_t> pad_upper(const std::vector<int32_t> &U, int n, int n_search)
{
    std::vector<int32_t> P((size_t)n_search * n_search, 0);
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j)
            P[(size_t)i * n_search + j] = U[(size_t)i * n + j];
    for (int i = n; i < n_search; ++i)
        P[(size_t)i * n_search + i] = 1;
    return P;
}

TableOffsets table_offsets(const std::vector<int32_t> &U, int ns, int A)
{
    TableOffsets t;
    t.rows = A;
    t.es_add = 0;
    t.Uoff = U;
    for (int g = 0; g < 16; ++g)
        t.kgate[g] = 0;
    for (int v = 0; v < A; ++v) {
        int64_t k = 0;
        for (int j = A; j < ns; ++j)
            k += std::max<int64_t>(0, -(int64_t)U[(size_t)v * ns + j]);
        t.Uoff[(size_t)v * ns + v] = (int32_t)(U[(size_t)v * ns + v] - k);
        const int bit = A - 1 - v;  // the Gray bit of variable v
        if (bit < kGateBits)
            t.kgate[bit] = (int32_t)k;
    }
    for (int i = A; i < ns; ++i)
        for (int j = i; j < ns; ++j)
            t.es_add += std::max<int64_t>(0, -(int64_t)U[(size_t)i * ns + j]);
    return t;
}

std::vector<int64_t> descent_energies(const std::vector<int32_t> &U, int n, int starts, int fixed,
                                      uint64_t fixed_value)
{
    // F[v]: the change of E when variable v goes from 0 to 1 given the others
    // (U_vv plus the couplings to the set variables); flipping v moves E by F[v]
    // if x_v = 0 and by -F[v] if x_v = 1.
    auto coupling = [&U, n](int a, int b) { return a < b ? U[(size_t)a * n + b] : U[(size_t)b * n + a]; };
    std::unordered_set<uint64_t> seen;
    std::vector<int64_t> es;
    std::vector<int64_t> F((size_t)n);
    std::vector<int> x((size_t)n);
    uint64_t sm = 0x51a7e5eedull;  // SplitMix64 state (Steele, Lea and Flood)
    for (int st = 0; st < starts; ++st) {
        uint64_t start = 0;
        if (st > 0) {
            uint64_t z = (sm += 0x9e3779b97f4a7c15ull);
            z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
            z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
            start = z ^ (z >> 31);
        }
        int64_t e = 0;
        for (int v = 0; v < n; ++v)
            x[(size_t)v] = v < fixed ? (int)((fixed_value >> (fixed - 1 - v)) & 1u) : (int)((start >> v) & 1u);
        for (int v = 0; v < n; ++v) {
            int64_t f = U[(size_t)v * n + v];
            for (int j = 0; j < n; ++j)
                if (j != v && x[(size_t)j])
                    f += coupling(v, j);
            F[(size_t)v] = f;
            if (x[(size_t)v])
                for (int j = v; j < n; ++j)
                    e += x[(size_t)j] ? U[(size_t)v * n + j] : 0;
        }
        for (int step = 0; step < 4 * n + 4; ++step) {
            int best = -1;
            int64_t best_d = 0;
            for (int v = fixed; v < n; ++v) {
                const int64_t d = x[(size_t)v] ? -F[(size_t)v] : F[(size_t)v];
                if (d < best_d) {
                    best_d = d;
                    best = v;
                }
            }
            if (best < 0)
                break;  // a local minimum under single flips
            const int64_t sg = x[(size_t)best] ? -1 : 1;
            x[(size_t)best] ^= 1;
            e += best_d;
            for (int j = 0; j < n; ++j)
                if (j != best)
                    F[(size_t)j] += sg * coupling(j, best);
        }
        uint64_t key = 0;
        for (int v = 0; v < n; ++v)
            key |= (uint64_t)x[(size_t)v] << v;
        if (seen.insert(key).second)
            es.push_back(e);
        for (int v = fixed; v < n; ++v)  // the single-flip neighbours
            if (seen.insert(key ^ (1ull << v)).second)
                es.push_back(e + (x[(size_t)v] ? -F[(size_t)v] : F[(size_t)v]));
    }
    std::sort(es.begin(), es.end());
    return es;
}

void largest_subcube(uint64_t lo, uint64_t hi, int A, int *fixed, uint64_t *fixed_value)
{
    // the largest aligned block [m 2^s, (m + 1) 2^s) inside [lo, hi); its Gray
    // codes share their top A - s bits, g(m) (g(j) >> s = g(j >> s))
    for (int sb = A; sb >= 0; --sb) {
        const uint64_t size = 1ull << sb;
        const uint64_t m = (lo + size - 1) >> sb;
        if ((m + 1) << sb <= hi && m < (1ull << (A - sb))) {
            *fixed = A - sb;
            *fixed_value = m ^ (m >> 1);
            return;
        }
    }
    *fixed = A;
    *fixed_value = lo ^ (lo >> 1);
}

static int ceil_log2(uint64_t v)
{
    int k = 0;
    while ((1ull << k) < v)
        ++k;
    return k;
}

static uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

void reduce_fixed(const std::vector<int32_t> &U, int n, int k, uint64_t f,
                  std::vector<int32_t> &Usub, int64_t *c, int64_t *sub_abs)
{
    const int m = n - k;
    int64_t cc = 0;
    for (int v = 0; v < k; ++v) {
        if (!((f >> (k - 1 - v)) & 1u))
            continue;
        for (int w = v; w < k; ++w)
            if ((f >> (k - 1 - w)) & 1u)
                cc += U[(size_t)v * n + w];
    }
    Usub.assign((size_t)m * m, 0);
    int64_t s = 0;
    for (int i = 0; i < m; ++i) {
        int64_t d = U[(size_t)(k + i) * n + (k + i)];
        for (int v = 0; v < k; ++v)
            if ((f >> (k - 1 - v)) & 1u)
                d += U[(size_t)v * n + (k + i)];
        Usub[(size_t)i * m + i] = (int32_t)d;
        s += d < 0 ? -d : d;
        for (int j = i + 1; j < m; ++j) {
            const int32_t u = U[(size_t)(k + i) * n + (k + j)];
            Usub[(size_t)i * m + j] = u;
            s += u < 0 ? -(int64_t)u : u;
        }
    }
    *c = cc;
    *sub_abs = s;
}

int make_plan(int n_total, int prefix_bits, int cache_bits, int num_cus, int cols_per_lane,
              int split_bits, qubo_plan *out)
{
    if (!out || n_total < 1 || n_total > QUBO_MAX_N || num_cus < 1)
        return QUBO_EINVAL;
    int k = split_bits;
    if (k < 0)
        k = n_total > kMaxSingleVars ? n_total - kMaxSingleVars : 0;
    if (k > 0 && n_total - k < kMinSearchVars)
        return QUBO_EINVAL;
    if (k > kMaxSplitBits)
        return QUBO_EPLAN;
    const int n = n_total - k;  // variables of each (sub-)problem
    if (cols_per_lane == 0)
        cols_per_lane = kDefaultColsPerLane;
    if (cols_per_lane != 8 && cols_per_lane != 16)
        return QUBO_EINVAL;
    const int group = kWave * cols_per_lane;  // columns of a wave and of a workgroup
    if (prefix_bits < -1 || prefix_bits > n)
        return QUBO_EINVAL;
    if (cache_bits < -1 || cache_bits > (prefix_bits >= 0 ? prefix_bits : n))
        return QUBO_EINVAL;

    qubo_plan p{};
    p.n = n_total;
    p.split_bits = k;
    p.n_search = std::max(n, kMinSearchVars);
    const int ns = p.n_search;

    int A;
    if (n < kMinSearchVars) {
        A = ns;  // tiny problems: one fixed split over the padded variables
    } else if (prefix_bits >= 0) {
        A = prefix_bits;
        if (A < kRegBits)
            return QUBO_EPLAN;
    } else {
        // 2^16 suffix columns (128 column groups), fewer for small n, more
        // where the prefix table would pass 2^28 entries (1 GiB): n = 48 and 50
        // take A = 28, n = 40 A = 24, n = 32 A = 16, n = 24 A = 8.  Measured
        // splits (whole searches on the MI355X): A = 24 is the fastest at
        // n = 40 (17.5 ms against 25.1 ms at A = 28, which spends 7 ms building
        // its prefix table), A = 8 at n = 24; at n = 32, A = 16 is within 20 %
        // of the fastest (A = 18).
        int B = std::max(std::min(ns - kRegBits, 16), ns - 28);
        A = ns - B;
        while (A < kMaxPrefixBits && (uint64_t)A * 4ull * (1ull << (ns - A)) > kMaxMintBytes)
            ++A;
    }
    const int B = ns - A;
    if (A > kMaxPrefixBits)
        return QUBO_EPLAN;
    const uint64_t cols = 1ull << B;
    const uint64_t cols_padded = (cols + group - 1) / group * group;
    if ((uint64_t)A * 4ull * cols_padded > kMaxMintBytes)
        return QUBO_EPLAN;

    int l;
    if (n < kMinSearchVars || cache_bits < 0)
        l = std::min(A, 13);
    else
        l = cache_bits;
    if (l < kRegBits)
        return QUBO_EPLAN;

    p.prefix_bits = A;
    p.suffix_bits = B;
    p.reg_bits = kRegBits;
    p.cols_per_lane = cols_per_lane;
    p.wave_size = kWave;
    p.waves_per_block = kWavesPerBlock;
    p.col_groups = cols_padded / group;

    // Segments: enough work units for ~32 per resident wave (the gated kernel
    // keeps six workgroups of four waves per CU), each at least one unrolled
    // body (2^5 steps) and at most 2^18 steps, so that the last round of the
    // persistent grid is short.  n = 48 and 50 reach the 2^18 cap either way;
    // at n = 40 (2^13-step units) this measured 4 % faster than ~5 units per
    // wave, while 2^11-step units ran 20 % slower (their start-up dominates).
    const uint64_t resident_waves = (uint64_t)num_cus * 6 * kWavesPerBlock;
    const uint64_t target_units = 32 * resident_waves;
    int split = 0;
    if (target_units > p.col_groups)
        split = ceil_log2((target_units + p.col_groups - 1) / p.col_groups);
    int c = A - split;
    // but at least 2^12 steps (128 bodies) per unit where the walk is that long:
    // a unit's start (its rows from memory) must stay small against its walk,
    // even when fewer units result (at n = 34..38, 2^10-step units ran 1.2 to
    // 2.1 times slower than 2^12-step ones; larger sizes reach 2^12 anyway) --
    // unless that leaves fewer units than resident waves: then down to 2^10
    // steps until there are enough (n = 32 ran 30 % slower on 2,048 units)
    c = std::max(c, std::min(A, kMinSegBits));
    while (c > kMinSegBitsIdle && p.col_groups * (1ull << (A - c)) < resident_waves)
        --c;
    c = std::max(c, kRegBits);
    c = std::min(c, kMaxSegBits);
    c = std::min(c, A);
    p.seg_bits = c;

    const int l_eff = std::min(l, c);
    const int lds_rows = std::max(0, l_eff - kRegBits);
    if (lds_rows * group * 4 > kMaxLdsBytes)
        return QUBO_EPLAN;
    p.cache_bits = l_eff;  // bits above the segment length never flip inside a unit
    p.lds_bytes = lds_rows * group * 4;

    const uint64_t segs = 1ull << (A - c);
    p.work_units = p.col_groups * segs;
    const uint64_t block_items = p.col_groups * ((segs + kWavesPerBlock - 1) / kWavesPerBlock);
    // Two resident workgroups per CU for the host-only plan; the search re-sizes
    // the grid from the runtime's occupancy query of the chosen kernel.
    p.blocks = (int)std::min<uint64_t>((uint64_t)num_cus * 2, block_items);

    p.workspace_bytes = layout_of(p).total;
    *out = p;
    return QUBO_OK;
}

Layout layout_of(const qubo_plan &p)
{
    Layout L{};
    const uint64_t cols = 1ull << p.suffix_bits;
    const uint64_t group = (uint64_t)kWave * p.cols_per_lane;
    L.cols_padded = (cols + group - 1) / group * group;
    uint64_t off = 0;
    L.off_u = off;
    off = align256(off + (uint64_t)p.n_search * p.n_search * 4);
    L.off_es = off;
    off = align256(off + L.cols_padded * 4);
    L.off_mint = off;
    off = align256(off + (uint64_t)p.prefix_bits * L.cols_padded * 4);
    L.off_ep = off;
    off = align256(off + (1ull << p.prefix_bits) * 4);
    L.off_epmin = off;
    off = align256(off + ((1ull << (p.prefix_bits - kRegBits)) + 2) * 4);  // + 2 padding entries
    L.off_gates = off;  // the gates' table (plan.h)
    off = align256(off + (gate_lane_bounds_at(p.prefix_bits) + 6 * (L.cols_padded / p.cols_per_lane)) * 4);
    L.off_partials = off;
    off = align256(off + (uint64_t)p.blocks * 64);  // one partial (at most 64 bytes) per workgroup
    L.off_ctrl = off;
    off = align256(off + 256);
    L.total = off;
    return L;
}

}  // namespace qubo
