// The Gray walk of the QUBO search on CDNA4 (gfx950), shared by the integer
// search and the search of a real-valued matrix (whose walk runs on rounded,
// scaled integer tables): the helpers of one unrolled 32-step body and the loop
// over work units with its bound gates (Maltsev, Remnev, Kapranov and
// Krivtsova, "Terastate-per-second QUBO Brute-Force on a Single GPU", sec. III.B,
// eq. 9 and Algorithm 2; sec. III.C for the units).  What happens to a body
// whose bound reaches the threshold is up to the caller's mode.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "plan.h"  // kRegBits, the gates' table layout

namespace qubo {

constexpr int kU = kRegBits;  // Gray bits with rows in VGPRs
constexpr int kBody = 1 << kU;
constexpr int kWaves = 4;    // waves per workgroup

__device__ __forceinline__ uint64_t gray(uint64_t i) { return i ^ (i >> 1); }

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }

// Marks a value that is equal in every lane as wave-uniform (kept in SGPRs).
__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

template <int R>
__device__ __forceinline__ int row_min(const int (&E)[R]);

// Min of 8 values: 3 x v_min3_i32 + 1 x v_min_i32.
template <>
__device__ __forceinline__ int row_min<8>(const int (&E)[8])
{
    const int a = imin(imin(E[0], E[1]), E[2]);
    const int b = imin(imin(E[3], E[4]), E[5]);
    const int c = imin(E[6], E[7]);
    return imin(imin(a, b), c);
}

// Min of 16 values as a tree of 3-input mins (7 x v_min3_i32 + 1 x v_min_i32).
template <>
__device__ __forceinline__ int row_min<16>(const int (&E)[16])
{
    const int a = imin(imin(E[0], E[1]), E[2]);
    const int b = imin(imin(E[3], E[4]), E[5]);
    const int c = imin(imin(E[6], E[7]), E[8]);
    const int d = imin(imin(E[9], E[10]), E[11]);
    const int e = imin(imin(E[12], E[13]), E[14]);
    const int f = imin(imin(a, b), c);
    const int h = imin(imin(d, e), E[15]);
    return imin(f, h);
}

template <int R>
__device__ __forceinline__ void add_row(int (&E)[R], const int (&M)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r)
        E[r] += M[r];
}

template <int R>
__device__ __forceinline__ void sub_row(int (&E)[R], const int (&M)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r)
        E[r] -= M[r];
}

// Keeps each column's energy of the current state in a VGPR: the compiler may
// not fold a run of row updates into its net effect, so every state of the walk
// is materialised by its own add (the O(1)-per-state evaluation of eq. 9).
template <int R>
__device__ __forceinline__ void materialise(int (&E)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r)
        asm volatile("" : "+v"(E[r]));
}

// One unrolled body of 32 Gray steps with only the row updates (eq. 9): every
// flip has a compile-time row and sign except the flip of bit 4, whose sign
// alternates between bodies.
template <int R>
__device__ __forceinline__ void adds_body(int (&E)[R], const int (&Mr)[kU][R], bool top_plus)
{
#pragma unroll
    for (int m = 0; m + 1 < kBody; ++m) {
        const int t = __builtin_ctz((unsigned)(m + 1));
        if (t < kU - 1) {
            if ((((m + 1) >> (t + 1)) & 1) == 0)
                add_row(E, Mr[t]);
            else
                sub_row(E, Mr[t]);
        } else {
            if (top_plus)
                add_row(E, Mr[kU - 1]);
            else
                sub_row(E, Mr[kU - 1]);
        }
        materialise(E);
    }
}

// The same body with the per-step test of Algorithm 2: after each state, the
// lane's minimum over its R columns (a v_min3 tree) is compared with the
// threshold T - E_p(g(j)).  Returns the OR over the body of the wave's hit masks.
template <int R>
__device__ __forceinline__ uint64_t checked_body(int (&E)[R], const int (&Mr)[kU][R],
                                                 bool top_plus, int T,
                                                 const int32_t *__restrict__ epb)
{
    uint64_t acc = 0;
#pragma unroll
    for (int m = 0; m < kBody; ++m) {
        const int th = T - epb[m];
        const int cm = row_min<R>(E);
        acc |= __builtin_amdgcn_ballot_w64(cm <= th);
        if (m + 1 < kBody) {
            const int t = __builtin_ctz((unsigned)(m + 1));
            if (t < kU - 1) {
                if ((((m + 1) >> (t + 1)) & 1) == 0)
                    add_row(E, Mr[t]);
                else
                    sub_row(E, Mr[t]);
            } else {
                if (top_plus)
                    add_row(E, Mr[kU - 1]);
                else
                    sub_row(E, Mr[kU - 1]);
            }
        }
    }
    return acc;
}

// The next work item (slot) of a workgroup, by thread 0.  The slot order
// (item_place in plan.h) is cut into kItemParts contiguous parts (item_part), each with a
// counter.  Workgroup w draws from part w mod kItemParts first, which is the
// XCD the dispatcher places it on (workgroups go to the XCDs in turn), then
// from the parts after it once one is used up (a used-up part stays used up:
// its counter only grows).  So the workgroups that share an L2 walk the rows of
// a few column groups and the gate entries of a few segments at a time.  A
// workgroup's next item lies about as many items on as its part has
// workgroups (192 at six per CU), which keeps it in the same column group, and
// its rows in LDS, while that count is a multiple of kTileGroups.
// state: the parts this workgroup has found used up (thread 0's, kept in LDS).
// Returns `slots` once every part is used up.
template <class Ctl>
__device__ __forceinline__ uint64_t next_item(Ctl *ctrl, uint64_t slots, unsigned long long &state)
{
    while (state < (unsigned long long)kItemParts) {
        const uint32_t p = (blockIdx.x + (uint32_t)state) % kItemParts;
        const ItemPart part = item_part(slots, p);
        if (part.len != 0) {
            const uint64_t k = atomicAdd(&ctrl->counter[p], 1ull);
            if (k < part.len)
                return part.lo + k;
        }
        ++state;
    }
    return slots;
}

// The loop over work units of one workgroup (a persistent grid: items come
// from the counters of next_item; an item is one column group and four
// consecutive segments of the Gray walk, one per wave).  Per unit: E_sd at the segment's
// first prefix (eq. 8), the rows of the five lowest Gray bits in registers,
// the lane bounds of the gates, then the bodies of 32 Gray steps.
//
// Gated = true: before a body, a lower bound on every energy the body will
// produce decides whether the per-step minimum is needed at all.  The body
// visits all 32 patterns y of the 5 low Gray bits with the higher prefix bits
// fixed; from the body's first state (low pattern s<<4, s = bit 5 of the step
// index) a column's suffix-dependent energy can fall by at most
//   beta0(c) - s M_4(c),   beta0(c) = sum_{t<5} min(0, M_t(c)),
// and the prefix energy of any step is at least epmin[body].  A lane bounds all
// its columns at once: min_c E(c) + min_c (beta0(c) - s M_4(c)), the second term
// fixed per work unit for s = 0 and s = 1.  If no lane's bound reaches
// T - epmin, no state of the body can reach the threshold T, and the body runs
// the row updates only; otherwise it is walked exactly.  Every state still
// costs its one add.  Gated = false (strict): every body runs the per-step test
// of Algorithm 2 and is walked exactly where it hits.
// The lane bounds depend only on the lane's columns, so the cache builders
// compute them once per column group and lane (six rows in the gates' table:
// body s = 0 and 1, pair for bit 5 = 0 and 1, group of sixteen bodies for bit
// 8 = 0 and 1), and the prefix bounds of a body (epmin), an aligned pair and an
// aligned group (the gates' table).
//
// The tables may carry offsets: the row of Gray bit t is M_t + K_t and the
// prefix energies carry -K_t for each set bit t, so E and E_p each hold a share
// of sum_{t set} K_t that cancels in their sum.  The lane bounds are then taken
// over M_t = row - K_t, and the prefix bounds are, for each body (pair, group),
// the minimum of E_p + sum_{t < 9 set} K_t over its steps less that sum at its
// first step: the same bounds as without offsets, with no offset in this loop.
//
// The mode provides
//   int refresh(int T): T lowered to the threshold shared between waves;
//   exact(E, Mr, base, top_plus, T, colbase, from_end): the exact walk of the
//     body whose first Gray step is base (E holds its first state, or its last
//     with from_end), leaving E at the body's last state and T lowered.
// T only falls, so a body that a group or pair bound cleared stays cleared.
// gates: the gates' table, a __restrict__ kernel argument of the caller, so
// that its wave-uniform reads are scalar loads (read through the argument
// struct, they were vector loads into VGPRs, with a VALU address and copies);
// item_sh: four __shared__ words of the calling kernel; lds_rows: its dynamic LDS
// ([l_eff - kU][64 R] rows of Gray bits kU .. l_eff - 1).
template <int R, bool Gated, class Args, class Ctl, class Mode>
__device__ __forceinline__ void walk_units(const Args &a, Ctl *__restrict__ ctrl,
                                           const int32_t *__restrict__ es,
                                           const int32_t *__restrict__ mint,
                                           const int32_t *__restrict__ ep,
                                           const int32_t *__restrict__ epmin,
                                           const int32_t *__restrict__ gates, int32_t *lds_rows,
                                           unsigned long long *item_sh, Mode &mode, int &T,
                                           uint32_t &bodies, uint32_t &checked, uint32_t &slow_bodies)
{
    constexpr int kGroup = 64 * R;  // columns of a wave (and of a workgroup)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // This lane's column in the LDS rows, biased so that bit t's row is
    // lds_lane + t * kGroup (one add per outer flip).
    const int32_t *lds_lane = lds_rows - kU * kGroup + lane;
    const int A = a.A;
    const uint64_t cp = a.cols_padded;
    // Thread 0's words: item_sh[2] the parts used up, item_sh[3] the column
    // group whose rows are in LDS (none yet).
    if (threadIdx.x == 0) {
        item_sh[2] = 0;
        item_sh[3] = ~0ull;
    }

    for (;;) {
        if (threadIdx.x == 0) {
            // The grid of items and its slots, recomputed for each item so that
            // none of it holds registers through the body loop.
            uint64_t groups = cp / kGroup, blocks = a.seg_blocks;
            asm volatile("" : "+s"(groups), "+s"(blocks));
            const int lg_g = ceil_log2_u64(groups), lg_s = ceil_log2_u64(blocks);
            const uint64_t slots = 1ull << (lg_g + lg_s);
            uint64_t g = ~0ull, sb = 0;  // ~0: no item left
            for (;;) {
                const uint64_t slot = next_item(ctrl, slots, item_sh[2]);
                if (slot >= slots)
                    break;
                const ItemPlace place = item_place(slot, lg_g, lg_s);
                if (place.group < groups && place.block < blocks) {  // else a slot outside the grid
                    g = place.group;
                    sb = place.block;
                    break;
                }
            }
            // The top bit of the block word asks for the group's rows in LDS.
            const uint64_t reload = g != item_sh[3] ? 1ull << 63 : 0;
            item_sh[3] = g;
            item_sh[0] = g;
            item_sh[1] = sb | reload;
        }
        __syncthreads();
        const uint64_t g = uniform64(item_sh[0]);
        const uint64_t sbw = uniform64(item_sh[1]);
        __syncthreads();
        if (g == ~0ull)
            break;
        const uint64_t sb = sbw & ~(1ull << 63);
        if (sbw >> 63) {
            const int rows = a.l_eff - kU;
            for (int k = threadIdx.x; k < rows * kGroup; k += blockDim.x) {
                const int t = kU + k / kGroup;
                const int col = k % kGroup;
                lds_rows[k] = mint[(uint64_t)(A - 1 - t) * cp + g * kGroup + col];
            }
            __syncthreads();
        }
        const uint64_t seg = a.seg_first + sb * kWaves + (uint64_t)wave;
        if (seg >= a.seg_first + a.segs)
            continue;
        uint64_t j_begin = seg << a.seg_bits;
        uint64_t j_end = (seg + 1) << a.seg_bits;
        j_begin = j_begin > a.gray_lo ? j_begin : a.gray_lo;
        j_end = j_end < a.gray_hi ? j_end : a.gray_hi;
        if (j_begin >= j_end)
            continue;

        const uint64_t col0 = g * kGroup + (uint64_t)lane;  // column of register r is col0 + 64 r

        // E_sd at the first prefix of the segment: E_s + sum of the rows of its set bits (eq. 8).
        int E[R];
        {
            const int32_t *src = es + col0;
#pragma unroll
            for (int r = 0; r < R; ++r)
                E[r] = src[r * 64];
            uint64_t bits = gray(j_begin);
            while (bits) {
                const int t = __builtin_ctzll(bits);
                bits &= bits - 1;
                const int32_t *row = mint + (uint64_t)(A - 1 - t) * cp + col0;
#pragma unroll
                for (int r = 0; r < R; ++r)
                    E[r] += row[r * 64];
            }
        }
        int Mr[kU][R];
#pragma unroll
        for (int t = 0; t < kU; ++t) {
            const int32_t *row = mint + (uint64_t)(A - 1 - t) * cp + col0;
#pragma unroll
            for (int r = 0; r < R; ++r)
                Mr[t][r] = row[r * 64];
        }
        // Lane bounds of the fall within a body, for s = 0 and s = 1; within an
        // aligned pair of bodies (64 steps, Gray bits 0..5), for bit 5 = 0 and 1
        // at the pair's start; and within an aligned group of sixteen bodies (512
        // steps, Gray bits 0..8: bits 0..7 start at 0), for bit 8 = 0 and 1 at
        // the group's start: per column group and lane, from the builders.
        int beta_s0 = 0, beta_s1 = 0, beta_p0 = 0, beta_p1 = 0, beta_q0 = 0, beta_q1 = 0;
        if (Gated) {
            // Column group g's lane bounds: 6 x 64 entries at gate_lane_bounds_at(A)
            // + 384 g, addressed from col0 = g kGroup + lane (live here already; a
            // separate lane offset, hoisted out of the unit loop, held two VGPRs
            // through every body).  The barrier keeps the scalar part here too.
            int64_t at = (int64_t)gate_lane_bounds_at(A) + (int64_t)g * (6 * 64) - (int64_t)(g * kGroup);
            asm volatile("" : "+s"(at));
            const int32_t *lb = gates + at + col0;
            beta_s0 = lb[0];
            beta_s1 = lb[64];
            beta_p0 = lb[128];
            beta_p1 = lb[192];
            beta_q0 = lb[256];
            beta_q1 = lb[320];
        }
        T = mode.refresh(T);

        // The body loop counts with 32-bit scalars (the SALU has no 64-bit
        // less-than): a segment holds at most 2^13 bodies.
        // Bodies are counted by their index b = j >> 5, a 32-bit value (A <= 32),
        // so that the per-body bookkeeping is 32-bit scalar arithmetic; the
        // 64-bit Gray step is formed only where a walk needs it.
        const uint32_t nbodies = (uint32_t)((j_end - j_begin) >> kU);
        const uint32_t b0 = (uint32_t)(j_begin >> kU);
        // The group gate's prefix bound comes from the per-group table, read one
        // group ahead (the table has one padding entry past the last group); the
        // body minima are read only where a pair or body gate needs them.
        int q_next = Gated && A > kU + 3 ? gates[(b0 + 15) >> 4] : 0;
        uint32_t covered = 0;  // bodies ahead that a pair or group bound has cleared
        for (uint32_t bi = 0; bi < nbodies; ++bi) {
            const uint32_t b = b0 + bi;
            const bool last = bi + 1 == nbodies;
            const bool top_plus = (b & 1u) == 0;
            bool check = true;
            if (Gated) {
                // Padding columns hold INT_MAX with zero rows (beta 0), so a lane
                // of padding columns only has the bound INT_MAX.
                if (covered != 0) {
                    // T has not risen since the bound that cleared this body was checked.
                    check = false;
                    --covered;
                } else {
                    const int emin = row_min<R>(E);
                    if ((b & 15u) == 0 && bi + 15 < nbodies && A > kU + 3) {
                        // The first of sixteen aligned bodies: their 512 states of Gray
                        // bits 0..8 fall by at most beta_q(bit 8 at the group's start).
                        const int q = q_next;
                        q_next = gates[(b >> 4) + 1];
                        const int thq = T - q;
                        const int bq = emin + (((b >> 4) & 1u) ? beta_q1 : beta_q0);
                        if (__builtin_amdgcn_ballot_w64(bq <= thq) == 0)
                            covered = 15;
                    }
                    if (covered != 0) {
                        check = false;
                    } else {
                        if (top_plus && !last && A > kU) {
                            // An even body and its partner: the 64 states of Gray bits
                            // 0..5 fall by at most beta_p(bit 5 at the pair's start).
                            const int thp = T - gates[gate_pairs_at(A) + (b >> 1)];
                            const int bp = emin + (((b >> 1) & 1u) ? beta_p1 : beta_p0);
                            if (__builtin_amdgcn_ballot_w64(bp <= thp) == 0)
                                covered = 1;
                        }
                        if (covered != 0) {
                            check = false;
                        } else {
                            const int thb = T - epmin[b];
                            const int bound = emin + (top_plus ? beta_s0 : beta_s1);
                            check = __builtin_amdgcn_ballot_w64(bound <= thb) != 0;
                        }
                    }
                }
            }
            ++bodies;
            if (!check) {
                adds_body(E, Mr, top_plus);
            } else {
                ++checked;
                // Strict mode walks exactly only after the per-step test hit; the
                // gated kernel has already decided that the bound was reached.
                const uint64_t base = (uint64_t)b << kU;
                bool walk = Gated;
                if (!Gated)
                    walk = checked_body(E, Mr, top_plus, T, ep + base) != 0;
                if (walk) {
                    ++slow_bodies;
                    // The group's first column, from lane 0's (every lane is active
                    // here: the walk decision is a ballot): no register holds the
                    // group through the body loop.
                    const uint64_t colbase = uniform64(col0);
                    mode.exact(E, Mr, base, top_plus, T, colbase, !Gated);
                }
            }
            if (!last) {
                // Flip of Gray bit t = 5 + ctz(b + 1) into the next body (its sign is
                // bit t + 1 of the next body's first step): its row comes from LDS or
                // global memory.
                const int t = kU + __builtin_ctz(b + 1);
                const bool plus = (((b + 1) >> (t - kU + 1)) & 1u) == 0;
                int row[R];
                if (t < a.l_eff) {
                    // Bits 5 and 6 (three bodies in four) read at constant offsets: the
                    // general address costs a VALU instruction per body.  The asm
                    // markers keep the compiler from merging the branches into that
                    // address again.
                    if (t == kU) {
                        asm volatile("; exit flip of bit 5");
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            row[r] = lds_lane[kU * kGroup + r * 64];
                    } else if (t == kU + 1) {
                        asm volatile("; exit flip of bit 6");
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            row[r] = lds_lane[(kU + 1) * kGroup + r * 64];
                    } else {
                        const int32_t *src = lds_lane + t * kGroup;  // row of bit t, this lane
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            row[r] = src[r * 64];
                    }
                } else {
                    const int32_t *src = mint + (uint64_t)(A - 1 - t) * cp + col0;
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        row[r] = src[r * 64];
                }
                if (plus)
                    add_row(E, row);
                else
                    sub_row(E, row);
            }
        }
    }
}

}  // namespace qubo
