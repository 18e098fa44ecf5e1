// Host checks of plan.h's layout functions that the search kernels use: the
// gates' table layout, and the work-item order (item_place and item_part):
// for grids of G column groups by SB segment blocks, the slots
// [0, 2^(lg_g + lg_s)) map one-to-one onto the
// (group, block) pairs of the grid rounded up to powers of two, every pair of
// the grid G x SB is the image of exactly one slot, and the kItemParts parts
// cover the slots once, in order.  Prints "ok" or the first failure.
#include <cstdio>
#include <vector>

#include "plan.h"

using namespace qubo;

static int check(uint64_t G, uint64_t SB)
{
    const int lg_g = ceil_log2_u64(G), lg_s = ceil_log2_u64(SB);
    if ((1ull << lg_g) < G || (lg_g > 0 && (1ull << (lg_g - 1)) >= G) || (1ull << lg_s) < SB ||
        (lg_s > 0 && (1ull << (lg_s - 1)) >= SB)) {
        std::printf("ceil_log2 G=%llu SB=%llu\n", (unsigned long long)G, (unsigned long long)SB);
        return 1;
    }
    const uint64_t slots = 1ull << (lg_g + lg_s);
    const uint64_t Gp = 1ull << lg_g, Sp = 1ull << lg_s;
    std::vector<unsigned char> seen(slots, 0);
    uint64_t inside = 0;
    for (uint64_t i = 0; i < slots; ++i) {
        const ItemPlace p = item_place(i, lg_g, lg_s);
        if (p.group >= Gp || p.block >= Sp || seen[p.group * Sp + p.block]) {
            std::printf("place G=%llu SB=%llu i=%llu\n", (unsigned long long)G, (unsigned long long)SB,
                        (unsigned long long)i);
            return 1;
        }
        seen[p.group * Sp + p.block] = 1;
        inside += p.group < G && p.block < SB;
        // inside a tile the column group runs fastest
        const int tg = lg_g < kTileGroupBits ? lg_g : kTileGroupBits;
        if ((i & ((1ull << tg) - 1)) != 0) {
            const ItemPlace q = item_place(i - 1, lg_g, lg_s);
            if (q.group + 1 != p.group || q.block != p.block) {
                std::printf("tile order G=%llu SB=%llu i=%llu\n", (unsigned long long)G, (unsigned long long)SB,
                            (unsigned long long)i);
                return 1;
            }
        }
    }
    if (inside != G * SB) {
        std::printf("inside G=%llu SB=%llu\n", (unsigned long long)G, (unsigned long long)SB);
        return 1;
    }
    uint64_t next = 0;
    for (uint32_t p = 0; p < (uint32_t)kItemParts; ++p) {
        const ItemPart part = item_part(slots, p);
        if (part.len != 0 && part.lo != next) {
            std::printf("part G=%llu SB=%llu p=%u\n", (unsigned long long)G, (unsigned long long)SB, p);
            return 1;
        }
        next += part.len;
    }
    if (next != slots) {
        std::printf("parts G=%llu SB=%llu\n", (unsigned long long)G, (unsigned long long)SB);
        return 1;
    }
    return 0;
}

// The gates' table layout (plan.h): group bounds (one per aligned group of
// sixteen bodies) with a padding entry, then one pair bound per aligned pair,
// then the lane bounds at a 64-entry boundary, with no overlap.
static int check_gates_layout()
{
    for (int A = kRegBits; A <= kMaxPrefixBits; ++A) {
        const uint64_t bodies = 1ull << (A - kRegBits);
        const uint64_t groups = gate_groups(A), pairs = gate_pair_count(A);
        const bool ok = groups >= 1 && (A < kRegBits + 4 || groups * 16 == bodies) &&
                        (A < kRegBits + 1 || pairs * 2 == bodies) && gate_pairs_at(A) == groups + 1 &&
                        gate_lane_bounds_at(A) >= gate_pairs_at(A) + pairs && gate_lane_bounds_at(A) % 64 == 0;
        if (!ok) {
            std::printf("gates layout A=%d\n", A);
            return 1;
        }
    }
    return 0;
}

int main()
{
    if (check_gates_layout())
        return 1;
    const uint64_t sizes[] = {1, 2, 3, 5, 7, 8, 31, 32, 33, 63, 64, 65, 100, 256, 257, 1000, 2048};
    for (uint64_t G : sizes)
        for (uint64_t SB : sizes)
            if (G * SB <= (1ull << 22) && check(G, SB))
                return 1;
    // the n = 48 benchmark's grid (2048 column groups by 256 segment blocks) and a tall one
    if (check(2048, 256) || check(8192, 64) || check(1, 4096))
        return 1;
    std::printf("ok\n");
    return 0;
}
