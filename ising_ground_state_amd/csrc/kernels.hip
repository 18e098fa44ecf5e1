// HIP kernels of the exhaustive QUBO search, written for CDNA4 (gfx950).
//
// Method: Maltsev, Remnev, Kapranov and Krivtsova, "Terastate-per-second QUBO
// Brute-Force on a Single GPU: A Matrix Prefix-Suffix Decomposition".
//   * sec. II, eq. 8: the energies of all states sharing a prefix x_p are
//     E_p(x_p) + x_p M_int + E_s(U_B), with M_int = Q_ps U_B^T;
//   * sec. III.B, eq. 9 and Algorithm 2: walking the prefixes in Gray order,
//     one prefix bit k flips per step and the suffix-dependent vector moves by
//     +-M_int[k,:], one integer add per state;
//   * sec. III.C: suffix columns are split across lanes (column-wise split) and
//     the prefix walk into segments (ranges of the Gray walk), with a final
//     min-reduction over the units;
//   * sec. IV.B.1-3: the rows of M_int and the suffix-dependent vector stay in
//     registers, the prefix energies are read in Gray order.
//
// CDNA4 mapping of the search kernel (its loop over work units and bodies is in
// walk.h, shared with the binary64 search; this file holds the integer mode):
//   * a lane owns R = 8 or 16 suffix columns: c = g*64R + r*64 + lane, so the
//     lanes of a wave read consecutive dwords for each r (coalesced loads,
//     conflict-free LDS reads);
//   * the M_int rows of the 5 lowest Gray bits live in VGPRs (5R registers), the
//     rows of the next Gray bits in LDS, shared by the 4 waves of a workgroup that
//     work on the same column group, and the rest in L2/HBM;
//   * the walk is unrolled over 32 Gray steps: every flip inside the body has a
//     compile-time row and sign except the flip of bit 4, whose sign alternates
//     between bodies (a uniform branch); the flip that leaves the body reads its
//     row from LDS or global memory;
//   * per step: R v_add/v_sub (one per state), a v_min3_i32 tree (R/2 VALU) and one
//     v_cmp against the scalar threshold T - E_p(g(j)) (the prefix energy comes
//     from a Gray-ordered table through scalar loads).  The comparison results are
//     OR-ed over the body; a body with any hit is re-walked on an exact slow path
//     that records every state with E <= T (lowest index and exact counts),
//     then lowers T.  This is the strict mode;
//   * the default (gated) mode drops the per-step minimum: before an aligned
//     group of sixteen bodies, then before an aligned pair, then before a single
//     body, one bound per lane (the smallest column energy at the start plus the
//     largest possible fall over the free Gray bits, plus the smallest prefix
//     energy of those bodies) is compared with T; only bodies some lane's bound
//     reaches are walked on the exact path, and every other state costs its add
//     alone;
//   * the threshold T is shared between waves through a global best-so-far, which
//     is always a real state's energy, so no minimiser is ever skipped;
//   * at the end, each wave combines its lanes' records with DPP lane moves,
//     the workgroup's four waves through LDS, and one small kernel the
//     workgroups' partials (the reduction tree of sec. IV.B.6).
#include "kernels.h"
#include "dpp.h"
#include "walk.h"

#include <climits>
#include <type_traits>

namespace qubo {




// Combine rule for partial results over disjoint state sets.
__device__ __forceinline__ void combine(int &e, uint64_t &cnt, uint64_t &arg, int e2, uint64_t c2,
                                        uint64_t a2)
{
    if (c2 == 0)
        return;
    if (cnt == 0 || e2 < e) {
        e = e2;
        cnt = c2;
        arg = a2;
    } else if (e2 == e) {
        cnt += c2;
        arg = a2 < arg ? a2 : arg;
    }
}

__device__ __forceinline__ int wave_min(int v)
{
    return wave_reduce(v, INT_MAX, [](int a, int b) { return a < b ? a : b; });
}

__device__ __forceinline__ uint64_t wave_sum(uint64_t v)
{
    return wave_reduce(v, (uint64_t)0, [](uint64_t a, uint64_t b) { return a + b; });
}

// The partial result {min energy, count at the min, lowest index at the min} of
// the 64 lanes, by the same DPP steps with `combine` as the operation; the
// result is wave-uniform.
template <int Ctrl, int RowMask>
__device__ __forceinline__ void dpp_combine_step(int &e, uint64_t &cnt, uint64_t &arg)
{
    const int e2 = dpp_i32<Ctrl, RowMask>(INT_MAX, e);
    const uint64_t c2 = dpp_u64<Ctrl, RowMask>(0, cnt);
    const uint64_t a2 = dpp_u64<Ctrl, RowMask>(~0ull, arg);
    combine(e, cnt, arg, e2, c2, a2);
}

__device__ __forceinline__ void wave_combine(int &e, uint64_t &cnt, uint64_t &arg)
{
    dpp_combine_step<kDppSwap1, 0xf>(e, cnt, arg);
    dpp_combine_step<kDppSwap2, 0xf>(e, cnt, arg);
    dpp_combine_step<kDppHalfMirror, 0xf>(e, cnt, arg);
    dpp_combine_step<kDppMirror, 0xf>(e, cnt, arg);
    dpp_combine_step<kDppBcast15, 0xa>(e, cnt, arg);
    dpp_combine_step<kDppBcast31, 0xc>(e, cnt, arg);
    e = __builtin_amdgcn_readlane(e, 63);
    cnt = readlane_u64(cnt, 63);
    arg = readlane_u64(arg, 63);
}

// ---------------------------------------------------------------------------
// Cache builders.
// ---------------------------------------------------------------------------

// One thread per suffix column c (suffix variable A+i is bit B-1-i of c):
//   E_s[c]      = sum_{i <= j} U[A+i][A+j] xs_i xs_j            (eq. 8, E_s(U_B))
//   M_int[v][c] = sum_j U[v][A+j] xs_j, v < A                   (M_int = Q_ps U_B^T)
// plus the offsets: es_add on E_s, and on the rows of the prefix variables
// v < offset_rows, K[v] = sum_j max(0, -U[v][A+j]), i.e. each of their terms
// counts max(U, 0) when x_j = 1 and max(-U, 0) when x_j = 0.
// Padding columns (c >= 2^B) get E_s = INT_MAX and zero rows, so they never
// reach any threshold and stay constant under row updates.
__global__ __launch_bounds__(256) void build_suffix_kernel(const int32_t *__restrict__ U, int ns,
                                                           int A, int B, uint64_t cols_padded,
                                                           int offset_rows, int32_t es_add,
                                                           int32_t *__restrict__ es,
                                                           int32_t *__restrict__ mint)
{
    const uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= cols_padded)
        return;
    if (c >= (1ull << B)) {
        es[c] = INT_MAX;
        for (int v = 0; v < A; ++v)
            mint[(uint64_t)v * cols_padded + c] = 0;
        return;
    }
    int e = 0;
    for (int i = 0; i < B; ++i) {
        const int xi = (int)((c >> (B - 1 - i)) & 1u);
        int rowsum = 0;
        for (int j = i; j < B; ++j) {
            const int xj = (int)((c >> (B - 1 - j)) & 1u);
            rowsum += xj ? U[(A + i) * ns + (A + j)] : 0;
        }
        e += xi ? rowsum : 0;
    }
    es[c] = e + es_add;
    for (int v = 0; v < A; ++v) {
        const bool off = v < offset_rows;
        int m = 0;
        for (int j = 0; j < B; ++j) {
            const int xj = (int)((c >> (B - 1 - j)) & 1u);
            const int u = U[v * ns + (A + j)];
            m += xj ? (off && u < 0 ? 0 : u) : (off && u < 0 ? -u : 0);
        }
        mint[(uint64_t)v * cols_padded + c] = m;
    }
}

// Prefix energies in Gray order, ep[j] = E_p(g(j)) over the A prefix variables
// (prefix variable v is bit A-1-v of the A-bit number).  Block index b covers
// the 2^L consecutive j = b 2^L .. b 2^L + 2^L - 1 (L = min(A, 8)); all of them
// share the high A-L bits of g(j), which equal g(b).  Splitting x_p into high
// and low parts,
//   E_p = E_hi + E_lo + sum_{v in lo, x_v = 1} K[v],   K[v] = sum_{w in hi, x_w = 1} U[w][v],
// so each block evaluates E_hi and K once and each thread only its low part.
// The same kernel writes epmin[k] = min of ep over the 32-step body k (Gray steps
// 32k .. 32k+31), which bounds the prefix energy of every state of that body.
// E_hi is summed in parallel, one high variable per thread, into one of two
// LDS accumulators that alternate between blocks (each is cleared one block
// ahead, so a block needs two barriers).  The A x A prefix part of U sits in
// LDS for the whole launch (A <= 32).  Every entry is raised by ep_add (the
// offsets' constant; the rows' offsets reach the prefix energies through U's
// prefix diagonal, which the caller lowers by K[v]).  With row offsets kg[t] on
// Gray bits t < 5, epmin[k] is taken relative to the body's first step: the
// minimum over the body of ep[j] + sum_{t < 5 set in g(j)} kg[t], less that sum
// at step 32k (only bit 4 can be set there: kg[4] for odd k).
__global__ __launch_bounds__(256) void build_prefix_gray_kernel(const int32_t *__restrict__ U,
                                                                int ns, int A, int L,
                                                                uint64_t blk_first, uint64_t blk_end,
                                                                int32_t ep_add, GateOffsets kg,
                                                                int32_t *__restrict__ ep,
                                                                int32_t *__restrict__ epmin)
{
    __shared__ int K[8];
    __shared__ int Upp[32][32];
    __shared__ int ehi_acc[2];
    const int H = A - L;
    const int tid = threadIdx.x;
    for (int k = tid; k < A * A; k += blockDim.x)
        Upp[k / A][k % A] = k % A >= k / A ? U[(k / A) * ns + (k % A)] : 0;
    if (tid < 2)
        ehi_acc[tid] = 0;
    __syncthreads();
    // Block-stride loop: a dispatch holds fewer than 2^32 work-items, and A = 32
    // needs 2^32 prefixes.  The trip count is the same for every thread of a block.
    // Blocks have 2^L > L + H threads: L = 8 whenever H > 0, and H = A - 8 <= 24.
    int it = 0;
    for (uint64_t blk = blk_first + blockIdx.x; blk < blk_end; blk += gridDim.x, it ^= 1) {
        const uint64_t hi = gray(blk);  // high part of g(j), H bits
        if (tid < L) {
            const int v = H + tid;  // a low variable
            int k = 0;
            for (int w = 0; w < H; ++w)
                k += (int)((hi >> (H - 1 - w)) & 1u) * Upp[w][v];
            K[tid] = k;
        } else if (tid < L + H) {
            const int w = tid - L;  // a high variable: its row of E_hi
            if ((hi >> (H - 1 - w)) & 1u) {
                int e = 0;
                for (int w2 = w; w2 < H; ++w2)
                    e += (int)((hi >> (H - 1 - w2)) & 1u) * Upp[w][w2];
                atomicAdd(&ehi_acc[it], e);
            }
        } else if (tid == L + H) {
            ehi_acc[it ^ 1] = 0;  // the next block's accumulator (last read before this block began)
        }
        __syncthreads();
        const uint64_t j = (blk << L) | (uint64_t)tid;
        const uint32_t lo = (uint32_t)(gray(j) & ((1u << L) - 1));
        int e = ep_add + ehi_acc[it];
        for (int a = 0; a < L; ++a) {
            const int xa = (int)((lo >> (L - 1 - a)) & 1u);
            int row = K[a];
            for (int b = a; b < L; ++b)
                row += (int)((lo >> (L - 1 - b)) & 1u) * Upp[H + a][H + b];
            e += xa * row;
        }
        ep[j] = e;
        // 32 consecutive j are 32 consecutive lanes of one wave (blocks have 2^L >= 32 threads).
        int m = e;
#pragma unroll
        for (int t = 0; t < kU; ++t)
            m += (int)((lo >> t) & 1u) * kg.k[t];  // Gray bit t of g(j) (t < 5 <= L, or a zero kg past A)
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) {
            const int o = __shfl_xor(m, off, 64);
            m = o < m ? o : m;
        }
        if ((tid & 31) == 0)
            epmin[j >> 5] = m - (int)((j >> 5) & 1u) * kg.k[kU - 1];
        __syncthreads();  // K and this block's accumulator are rewritten two blocks on
    }
}

// The offsets of Gray bits 4 to 8 set at the first step of body b: g(32b) has
// bits 0..3 clear, bit 4 = b0, bit 5 = b0 ^ b1, bit 6 = b1 ^ b2, bit 7 = b2 ^ b3,
// bit 8 = b3 ^ b4.
// Unsigned: the gate tables' entries past a slice's ends may be unset.
__device__ __forceinline__ uint32_t body_start_offset(uint32_t b, const GateOffsets &kg)
{
    return (b & 1u) * (uint32_t)kg.k[kU - 1] + ((b ^ (b >> 1)) & 1u) * (uint32_t)kg.k[kU] +
           (((b >> 1) ^ (b >> 2)) & 1u) * (uint32_t)kg.k[kU + 1] +
           (((b >> 2) ^ (b >> 3)) & 1u) * (uint32_t)kg.k[kU + 2] +
           (((b >> 3) ^ (b >> 4)) & 1u) * (uint32_t)kg.k[kU + 3];
}

// Pair bounds (into the gates' pair table): min of the two body minima, each
// moved from its body's first step to the pair's (+ the offsets set at the
// body's first step, - those at the pair's: bits 0..4 clear there, bits 5 to 8
// as at body 2p).
__global__ __launch_bounds__(256) void build_pair_min_kernel(const int32_t *__restrict__ epmin,
                                                             int32_t *__restrict__ pairs,
                                                             uint64_t p_first, uint64_t p_end,
                                                             GateOffsets kg)
{
    const uint64_t p = p_first + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= p_end)
        return;
    const uint32_t b = (uint32_t)(2 * p);
    const uint32_t at0 = body_start_offset(b, kg);
    const int m0 = (int)((uint32_t)epmin[b] + at0);
    const int m1 = (int)((uint32_t)epmin[b + 1] + body_start_offset(b + 1, kg));
    pairs[p] = (int)((uint32_t)imin(m0, m1) - at0);
}

// Group bounds: min of the sixteen body minima, each moved to the group's first
// step (g(512k): bits 0..7 clear, bit 8 = k0).
__global__ __launch_bounds__(256) void build_group_min_kernel(const int32_t *__restrict__ epmin,
                                                              int32_t *__restrict__ gates,
                                                              uint64_t k_first, uint64_t k_end,
                                                              GateOffsets kg)
{
    const uint64_t k = k_first + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= k_end)
        return;
    const int32_t *e = epmin + 16 * k;
    int m = INT_MAX;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        m = imin(m, (int)((uint32_t)e[i] + body_start_offset((uint32_t)(16 * k + i), kg)));
    gates[k] = (int)((uint32_t)m - (uint32_t)(k & 1u) * (uint32_t)kg.k[kU + 3]);
}

// Lane bounds, one thread per column group g and lane (written as six rows of
// 64 per column group: s0, s1, p0, p1, q0, q1): over the lane's R
// columns c = g 64 R + 64 r + lane, with M_t(c) = row of Gray bit t less its
// offset (0 for padding columns and for bits that A does not have),
//   b(c) = sum_{t<5} min(0, M_t(c))          fall within a body from bits 0..4 clear,
//   s0 = min_c b,  s1 = min_c (b - M_4)      bit 4 clear / set at the body's start,
//   p0 = min_c (b + min(0, M_5)),  p1 = min_c (b - max(0, M_5))      pair, bit 5,
//   q0, q1: as p0, p1 from b7 = b + sum_{5<=t<8} min(0, M_t), with M_8   group, bit 8.
template <int R>
__global__ __launch_bounds__(256) void build_lane_bounds_kernel(const int32_t *__restrict__ mint,
                                                                uint64_t cols_padded, int A, int B,
                                                                GateOffsets kg,
                                                                int32_t *__restrict__ out)
{
    const uint64_t nlb = cols_padded / R;
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nlb)
        return;
    const uint64_t g = i / 64, lane = i % 64;
    const uint64_t col0 = g * 64 * R + lane;
    int s0 = INT_MAX, s1 = INT_MAX, p0 = INT_MAX, p1 = INT_MAX, q0 = INT_MAX, q1 = INT_MAX;
    for (int r = 0; r < R; ++r) {
        const uint64_t c = col0 + 64 * (uint64_t)r;
        const bool real = c < (1ull << B);
        int m[kU + 4];
        for (int t = 0; t < kU + 4; ++t)
            m[t] = real && t < A ? mint[(uint64_t)(A - 1 - t) * cols_padded + c] - kg.k[t] : 0;
        int b = 0;
        for (int t = 0; t < kU; ++t)
            b += m[t] < 0 ? m[t] : 0;
        const int b5 = b + (m[kU] < 0 ? m[kU] : 0);
        s0 = imin(s0, b);
        s1 = imin(s1, b - m[kU - 1]);
        p0 = imin(p0, b5);
        p1 = imin(p1, b - (m[kU] > 0 ? m[kU] : 0));
        const int b7 = b5 + (m[kU + 1] < 0 ? m[kU + 1] : 0) + (m[kU + 2] < 0 ? m[kU + 2] : 0);
        q0 = imin(q0, b7 + (m[kU + 3] < 0 ? m[kU + 3] : 0));
        q1 = imin(q1, b7 - (m[kU + 3] > 0 ? m[kU + 3] : 0));
    }
    int32_t *o = out + g * (6 * 64) + lane;  // column group g: six rows of 64
    o[0] = s0;
    o[64] = s1;
    o[128] = p0;
    o[192] = p1;
    o[256] = q0;
    o[320] = q1;
}

hipError_t launch_build_tables(const int32_t *U, int ns, int A, int B, uint64_t cols_padded,
                               int offset_rows, int32_t es_add, const GateOffsets &kg, int32_t *es,
                               int32_t *mint, int32_t *ep, int32_t *epmin, uint64_t j_lo, uint64_t j_hi,
                               hipStream_t stream)
{
    const unsigned g1 = (unsigned)((cols_padded + 255) / 256);
    hipLaunchKernelGGL(build_suffix_kernel, dim3(g1), dim3(256), 0, stream, U, ns, A, B,
                       cols_padded, offset_rows, es_add, es, mint);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    if (j_lo >= j_hi || j_hi > (1ull << A))
        return hipErrorInvalidValue;
    const int L = A < 8 ? A : 8;
    const uint64_t blk_first = j_lo >> L, blk_end = ((j_hi - 1) >> L) + 1;  // blocks holding the range
    const uint64_t nblocks = blk_end - blk_first;
    // Enough blocks to fill the chip several times over; each then walks many
    // prefix blocks with the prefix part of U staged once.
    const uint64_t grid = nblocks < (1ull << 14) ? nblocks : (1ull << 14);
    if (A > 32)
        return hipErrorInvalidValue;  // (the builder stages at most 32 x 32 entries of U)
    hipLaunchKernelGGL(build_prefix_gray_kernel, dim3((unsigned)grid), dim3(1u << L), 0, stream,
                       U, ns, A, L, blk_first, blk_end, -es_add, kg, ep, epmin);
    return hipGetLastError();
}

hipError_t launch_gate_tables(const int32_t *mint, uint64_t cols_padded, int A, int B, int R,
                              const GateOffsets &kg, const int32_t *epmin, int32_t *gates, uint64_t j_lo,
                              uint64_t j_hi, hipStream_t stream)
{
    if ((R != 8 && R != 16) || cols_padded % (64ull * R) != 0 || j_lo >= j_hi || A < kU || A > 32)
        return hipErrorInvalidValue;
    const uint64_t nlb = cols_padded / R;
    const uint64_t g0 = (nlb + 255) / 256;
    if (g0 > 0xffffffffull)
        return hipErrorInvalidValue;
    if (R == 8)
        hipLaunchKernelGGL(build_lane_bounds_kernel<8>, dim3((unsigned)g0), dim3(256), 0, stream, mint,
                           cols_padded, A, B, kg, gates + gate_lane_bounds_at(A));
    else
        hipLaunchKernelGGL(build_lane_bounds_kernel<16>, dim3((unsigned)g0), dim3(256), 0, stream, mint,
                           cols_padded, A, B, kg, gates + gate_lane_bounds_at(A));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || A < kU + 1)
        return err;
    // pairs and groups of bodies holding the slice's bodies
    const uint64_t p_first = j_lo >> (kU + 1), p_end = ((j_hi - 1) >> (kU + 1)) + 1;
    const uint64_t g2 = (p_end - p_first + 255) / 256;
    if (g2 > 0xffffffffull)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(build_pair_min_kernel, dim3((unsigned)g2), dim3(256), 0, stream, epmin,
                       gates + gate_pairs_at(A), p_first, p_end, kg);
    err = hipGetLastError();
    if (err != hipSuccess || A < kU + 4)
        return err;
    const uint64_t k_first = j_lo >> (kU + 4), k_end = ((j_hi - 1) >> (kU + 4)) + 1;
    const uint64_t g3 = (k_end - k_first + 255) / 256;
    if (g3 > 0xffffffffull)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(build_group_min_kernel, dim3((unsigned)g3), dim3(256), 0, stream, epmin, gates,
                       k_first, k_end, kg);
    return hipGetLastError();
}

__global__ void init_ctrl_kernel(Ctrl *ctrl, int32_t t0, int32_t *epmin_pad, int32_t *gates_pad)
{
    epmin_pad[0] = INT_MAX;  // read ahead by the last two bodies of the walk, never used
    epmin_pad[1] = INT_MAX;
    gates_pad[0] = INT_MAX;  // group bound read ahead by the walk's last group, never used
    for (int p = 0; p < kItemParts; ++p)
        ctrl->counter[p] = 0;
    ctrl->gbest = t0;
    ctrl->slow_total = 0;
    ctrl->bodies_total = 0;
    ctrl->checked_total = 0;
}

hipError_t launch_init_ctrl(Ctrl *ctrl, int32_t t0, int32_t *epmin_pad, int32_t *gates_pad,
                            hipStream_t stream)
{
    hipLaunchKernelGGL(init_ctrl_kernel, dim3(1), dim3(1), 0, stream, ctrl, t0, epmin_pad, gates_pad);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The search.
// ---------------------------------------------------------------------------

// Per-thread record slots of a workgroup in LDS (energy and two 64-bit words).
struct RecordSlots {
    int *e;
    uint64_t *a;
    uint64_t *b;
};

// What the exact walk does with the states it visits.  LaneBest keeps, per
// lane, the minimum over the lane's columns with its count and lowest index.
struct LaneBest {
    int e = INT_MAX;
    uint64_t cnt = 0;
    uint64_t arg = ~0ull;

    __device__ __forceinline__ void record(int v, uint64_t idx)
    {
        if (v < e) {
            e = v;
            cnt = 1;
            arg = idx;
        } else if (v == e) {
            cnt += 1;
            arg = idx < arg ? idx : arg;
        }
    }

    // Records every state of one Gray step with E_sd + E_p <= T (E_sd <= T - E_p
    // needs no overflow headroom: both sides are sub-sums of the folded matrix).
    // key = (g(j) << B) | (first column of the group), wave-uniform; column r of
    // a lane is key | r*64 | lane.  The record keeps the index without the
    // lane's 6 bits (equal for all of a lane's states, so comparisons between
    // them are unchanged); they are added once at the end (with_lane), which
    // keeps per-lane column indices out of the registers of the walk.
    template <int R>
    __device__ __forceinline__ void step(const int (&E)[R], int epm, uint64_t key, int &T)
    {
        const int th = T - epm;
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (E[r] <= th)
                record(E[r] + epm, key | ((uint64_t)r << 6));
    }

    __device__ __forceinline__ uint64_t with_lane(int lane) const
    {
        return cnt ? (arg | (uint64_t)lane) : ~0ull;
    }

    // A real energy of the wave's states (or INT_MAX): an upper bound of the minimum.
    __device__ __forceinline__ int bound() const { return wave_min(e); }

    // Between exact walks the record lives in LDS (slot = thread), so the hot
    // loop carries no record registers.
    __device__ __forceinline__ void load(const RecordSlots &s, int slot)
    {
        e = s.e[slot];
        cnt = s.a[slot];
        arg = s.b[slot];
    }
    __device__ __forceinline__ void store(RecordSlots &s, int slot) const
    {
        s.e[slot] = e;
        s.a[slot] = cnt;
        s.b[slot] = arg;
    }
};

// The low-energy spectrum (sec. VI.B, future work: a list of the k lowest
// energies instead of one minimum).  A wave keeps the k lowest states it has
// recorded, in the order (E ascending, index ascending), one per lane: lane i
// holds the i-th (empty slots hold INT_MAX).  A state is inserted by counting
// the entries before it (a ballot) and shifting the later ones up one lane.
// Any wave's k-th energy bounds the k-th lowest energy overall from above (k
// real states reach it), so it is a valid shared threshold; a state among the
// k lowest overall is never displaced from its wave's list, because k states
// before it there would also precede it overall.
struct WaveList {
    int e = INT_MAX;
    uint64_t x = ~0ull;
    int k = 1;     // entries kept (1..64), wave-uniform
    int lane = 0;

    __device__ __forceinline__ void insert(int ce, uint64_t cx)
    {
        const bool before = lane < k && (e < ce || (e == ce && x < cx));
        const int pos = __builtin_popcountll(__builtin_amdgcn_ballot_w64(before));
        if (pos >= k)
            return;
        const int eu = __shfl_up(e, 1, 64);
        const uint64_t xu = __shfl_up(x, 1, 64);
        if (lane > pos) {
            e = eu;
            x = xu;
        }
        if (lane == pos) {
            e = ce;
            x = cx;
        }
    }

    // Inserts the lanes of `mask`, whose entries are (ce, cx) in their own lane.
    __device__ __forceinline__ void insert_lanes(uint64_t mask, int ce, uint64_t cx)
    {
        while (mask) {
            const int l = __builtin_ctzll(mask);
            mask &= mask - 1;
            const int e1 = __builtin_amdgcn_readlane(ce, l);
            const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)cx, l);
            const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(cx >> 32), l);
            insert(e1, ((uint64_t)hi << 32) | lo);
        }
    }

    // The same for entries whose index is key | lane (key wave-uniform).
    __device__ __forceinline__ void insert_lanes_key(uint64_t mask, int ce, uint64_t key)
    {
        while (mask) {
            const int l = __builtin_ctzll(mask);
            mask &= mask - 1;
            insert(__builtin_amdgcn_readlane(ce, l), key | (uint64_t)l);
        }
    }

    // k-th energy of the list (INT_MAX until k states are in it).
    __device__ __forceinline__ int kth() const { return __builtin_amdgcn_readlane(e, k - 1); }

    // Offers every state of one Gray step with E_sd + E_p <= T, then lowers T
    // to the list's k-th energy.
    template <int R>
    __device__ __forceinline__ void step(const int (&E)[R], int epm, uint64_t key, int &T)
    {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint64_t mask = __builtin_amdgcn_ballot_w64(E[r] <= T - epm);
            if (mask) {
                insert_lanes_key(mask, E[r] + epm, key | ((uint64_t)r << 6));
                const int kt = kth();
                T = kt < T ? kt : T;
            }
        }
    }

    __device__ __forceinline__ int bound() const { return kth(); }

    __device__ __forceinline__ void load(const RecordSlots &s, int slot)
    {
        e = s.e[slot];
        x = s.b[slot];
    }
    __device__ __forceinline__ void store(RecordSlots &s, int slot) const
    {
        s.e[slot] = e;
        s.b[slot] = x;
    }
};

__device__ __forceinline__ int read_gbest(const Ctrl *ctrl)
{
    const int v = __hip_atomic_load(&ctrl->gbest, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_amdgcn_readfirstlane(v);
}

// Exact walk of one body of 32 Gray steps starting at `base`: every state with
// E_sd + E_p <= T is offered to the sink (which may lower T).  With from_end, E
// holds the body's last state on entry (a re-walk after the checked body) and
// is first taken back to the body's first state (over a body the low four Gray
// bits return to 0 and only bit 4 flips); otherwise E holds the first state.
// E holds the body's last state on exit.  A compact loop: it runs rarely.
template <int R, class Sink>
__device__ __forceinline__ void exact_body(int (&E)[R], const int (&Mr)[kU][R], uint64_t base,
                                           bool top_plus, int &T, const int32_t *__restrict__ ep,
                                           int B, uint64_t colbase, Sink &sink, bool from_end)
{
    if (from_end) {
        if (top_plus)
            sub_row(E, Mr[kU - 1]);
        else
            add_row(E, Mr[kU - 1]);
    }
    // The body's 32 prefix energies in one coalesced load (lane i holds step
    // i mod 32), read per step from a lane; a scalar load per step made every
    // step wait for memory.
    const int ep_lanes = ep[base + (uint64_t)(threadIdx.x & (kBody - 1))];
    const int neg_top = top_plus ? 0 : -1;
#pragma unroll 1
    for (int m = 0; m < kBody; m += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int mm = m + h;
            const int epm = __builtin_amdgcn_readlane(ep_lanes, mm);
            // Only a step where some lane's minimum reaches T has states to
            // record: the others cost the minimum and a compare.
            if (__builtin_amdgcn_ballot_w64(row_min<R>(E) <= T - epm) != 0)
                sink.step(E, epm, (gray(base + (uint64_t)mm) << B) | colbase, T);
            if (h == 0) {
                // Odd steps flip Gray bit 0; the sign is an integer mask (0: add,
                // -1: subtract, (d ^ neg) - neg), which stays in scalar registers.
                const int neg = -(((mm + 1) >> 1) & 1);
#pragma unroll
                for (int r = 0; r < R; ++r)
                    E[r] += (Mr[0][r] ^ neg) - neg;
            } else {
                // Even steps flip bit t = ctz(m + 2) >= 1, chosen with selects
                // (branches over t made the compiler keep copies of E at every
                // merge).  After the last step t = 5 and no row is chosen.
                const int t = __builtin_ctz((unsigned)(mm + 1));
                const int neg = (t < kU - 1) ? -(((mm + 1) >> (t + 1)) & 1) : neg_top;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    int d = 0;
#pragma unroll
                    for (int tt = 1; tt < kU; ++tt)
                        d = (tt == t) ? Mr[tt][r] : d;
                    E[r] += (d ^ neg) - neg;
                }
            }
        }
    }
}

// The integer mode of the walk: a body is walked exactly into the thread's
// record (LaneBest: minimum, count and lowest index; WaveList: the wave's k
// lowest states), then the wave's bound is offered to the shared best.
template <bool Lowest>
struct IntMode {
    using Sink = typename std::conditional<Lowest, WaveList, LaneBest>::type;
    RecordSlots rec;
    const int32_t *ep;
    Ctrl *ctrl;
    int B, k_low, lane;

    __device__ __forceinline__ int refresh(int T) const
    {
        const int gb = read_gbest(ctrl);
        return gb < T ? gb : T;
    }

    template <int R>
    __device__ __forceinline__ void exact(int (&E)[R], const int (&Mr)[kU][R], uint64_t base,
                                          bool top_plus, int &T, uint64_t colbase, bool from_end)
    {
        Sink sink;
        sink.load(rec, threadIdx.x);
        if constexpr (Lowest) {
            sink.k = k_low;
            sink.lane = lane;
        }
        const int t_in = T;
        exact_body(E, Mr, base, top_plus, T, ep, B, colbase, sink, from_end);
        sink.store(rec, threadIdx.x);
        // Every lane offers the same T to the shared best (a lane-0 branch, a
        // divergent region inside the body loop, made the compiler keep T and
        // the counters in VGPRs), and only when the wave's bound is below the
        // threshold the walk started from (a wave-uniform branch; the
        // spectrum's walk lowers T as it inserts): every value T took before
        // is already in the shared best, and most exact walks find nothing
        // below it.  Offered after every exact walk, the waves queued on the
        // one shared word (the planted n = 32 search ran 3.3 times slower).
        const int wm = sink.bound();
        T = wm < T ? wm : T;
        if (wm < t_in)
            atomicMin(&ctrl->gbest, T);
        const int gb = read_gbest(ctrl);
        T = gb < T ? gb : T;
    }
};

// The search kernel: each workgroup walks work units (walk_units) with the
// exact walks of an integer mode (IntMode), then reduces its lanes' records into
// one partial result per workgroup.
template <int R, bool Gated, bool Lowest>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(R == 8 && Gated ? 6 : 1))) void gray_search_kernel(const int32_t *__restrict__ es,
                                                          const int32_t *__restrict__ mint,
                                                          const int32_t *__restrict__ ep,
                                                          const int32_t *__restrict__ epmin,
                                                          const int32_t *__restrict__ gates,
                                                          Partial *__restrict__ partials,
                                                          Ctrl *__restrict__ ctrl,
                                                          const SearchArgs a)
{
    extern __shared__ int32_t lds_rows[];  // [l_eff - kU][64 R]
    __shared__ unsigned long long item_sh[4];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    using Sink = typename std::conditional<Lowest, WaveList, LaneBest>::type;
    __shared__ int rec_e[64 * kWaves];
    __shared__ uint64_t rec_a[64 * kWaves], rec_b[64 * kWaves];
    RecordSlots rec{rec_e, rec_a, rec_b};
    {
        Sink fresh;
        fresh.store(rec, threadIdx.x);  // each thread only ever touches its own slot
    }
    uint32_t slow_bodies = 0, bodies = 0, checked = 0;
    int T = read_gbest(ctrl);

    IntMode<Lowest> mode{rec, ep, ctrl, a.B, a.k_low, lane};
    walk_units<R, Gated>(a, ctrl, es, mint, ep, epmin, gates, lds_rows, item_sh, mode, T, bodies, checked,
                         slow_bodies);

    Sink sink;
    sink.load(rec, threadIdx.x);
    int e = INT_MAX;
    uint64_t cnt = 0, arg = ~0ull;
    if constexpr (Lowest) {
        if (lane < a.k_low) {
            LowEntry le;
            le.e = sink.e;
            le.pad = 0;
            le.x = sink.x;
            a.lists[((uint64_t)blockIdx.x * kWaves + wave) * (uint64_t)a.k_low + lane] = le;
        }
    } else {
        e = sink.e;
        cnt = sink.cnt;
        arg = sink.with_lane(lane);
        wave_combine(e, cnt, arg);
    }
    // Workgroup stage through LDS: one slot per wave, combined in wave order by
    // one thread into the workgroup's partial (the grid reduction then reads one
    // partial per workgroup).  Every wave of the workgroup leaves the item loop
    // together, so all of them reach the barrier.
    __shared__ Partial wg_part[kWaves];
    if (lane == 0) {
        Partial p;
        p.e = e;
        p.slow = slow_bodies;
        p.count = cnt;
        p.arg = arg;
        p.bodies = bodies;
        p.checked = checked;
        p.pad = 0;
        wg_part[wave] = p;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        Partial p = wg_part[0];
        for (int w = 1; w < kWaves; ++w) {
            const Partial &o = wg_part[w];
            combine(p.e, p.count, p.arg, o.e, o.count, o.arg);
            p.slow += o.slow;
            p.bodies += o.bodies;
            p.checked += o.checked;
        }
        partials[blockIdx.x] = p;
    }
}

template <int R, bool Gated, bool Lowest>
static void launch_one(const SearchArgs &args, int blocks, int lds_bytes, hipStream_t stream)
{
    hipLaunchKernelGGL((gray_search_kernel<R, Gated, Lowest>), dim3(blocks), dim3(64 * kWaves),
                       lds_bytes, stream, args.es, args.mint, args.ep, args.epmin, args.gates, args.partials,
                       args.ctrl, args);
}

// The instantiations: {8, 16} columns per lane x {gated, strict} for the
// minimum, and gated only for the spectrum.
static const void *search_fn(int cols_per_lane, bool gated, bool lowest)
{
    if (cols_per_lane == 8) {
        if (lowest)
            return gated ? reinterpret_cast<const void *>(gray_search_kernel<8, true, true>)
                         : nullptr;
        return gated ? reinterpret_cast<const void *>(gray_search_kernel<8, true, false>)
                     : reinterpret_cast<const void *>(gray_search_kernel<8, false, false>);
    }
    if (cols_per_lane == 16) {
        if (lowest)
            return gated ? reinterpret_cast<const void *>(gray_search_kernel<16, true, true>)
                         : nullptr;
        return gated ? reinterpret_cast<const void *>(gray_search_kernel<16, true, false>)
                     : reinterpret_cast<const void *>(gray_search_kernel<16, false, false>);
    }
    return nullptr;
}

hipError_t launch_search(const SearchArgs &args, int cols_per_lane, bool gated, bool lowest,
                         int blocks, int lds_bytes, hipStream_t stream)
{
    if (!search_fn(cols_per_lane, gated, lowest))
        return hipErrorInvalidValue;
    if (lowest && (args.k_low < 1 || args.k_low > kMaxLowest || !args.lists))
        return hipErrorInvalidValue;
    if (cols_per_lane == 8) {
        if (lowest)
            launch_one<8, true, true>(args, blocks, lds_bytes, stream);
        else if (gated)
            launch_one<8, true, false>(args, blocks, lds_bytes, stream);
        else
            launch_one<8, false, false>(args, blocks, lds_bytes, stream);
    } else {
        if (lowest)
            launch_one<16, true, true>(args, blocks, lds_bytes, stream);
        else if (gated)
            launch_one<16, true, false>(args, blocks, lds_bytes, stream);
        else
            launch_one<16, false, false>(args, blocks, lds_bytes, stream);
    }
    return hipGetLastError();
}

hipError_t search_occupancy(int cols_per_lane, bool gated, bool lowest, int *blocks_per_cu,
                            int lds_bytes)
{
    const void *fn = search_fn(cols_per_lane, gated, lowest);
    if (!fn)
        return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, 64 * kWaves,
                                                        (size_t)lds_bytes);
}

// Final map-reduce step (sec. III.C): min energy, summed counts at the min,
// lowest index at the min, over every workgroup's partial.  Each thread folds a
// strided share, each wave reduces its lanes with DPP, and thread 0 combines the
// waves' results from LDS.
__global__ __launch_bounds__(256) void reduce_kernel(const Partial *__restrict__ partials,
                                                     int count, Ctrl *ctrl)
{
    __shared__ int se[4];
    __shared__ uint64_t sc[4], sa[4], ss[4], sb[4], sk[4];
    int e = INT_MAX;
    uint64_t cnt = 0, arg = ~0ull, slow = 0, bodies = 0, checked = 0;
    for (int k = threadIdx.x; k < count; k += blockDim.x) {
        const Partial p = partials[k];
        combine(e, cnt, arg, p.e, p.count, p.arg);
        slow += p.slow;
        bodies += p.bodies;
        checked += p.checked;
    }
    wave_combine(e, cnt, arg);
    slow = wave_sum(slow);
    bodies = wave_sum(bodies);
    checked = wave_sum(checked);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        se[w] = e;
        sc[w] = cnt;
        sa[w] = arg;
        ss[w] = slow;
        sb[w] = bodies;
        sk[w] = checked;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < (int)(blockDim.x >> 6); ++k) {
            combine(e, cnt, arg, se[k], sc[k], sa[k]);
            slow += ss[k];
            bodies += sb[k];
            checked += sk[k];
        }
        ctrl->result.e = e;
        ctrl->result.slow = 0;
        ctrl->result.count = cnt;
        ctrl->result.arg = arg;
        ctrl->slow_total = slow;
        ctrl->bodies_total = bodies;
        ctrl->checked_total = checked;
    }
}

hipError_t launch_reduce(const Partial *partials, int count, Ctrl *ctrl, hipStream_t stream)
{
    hipLaunchKernelGGL(reduce_kernel, dim3(1), dim3(256), 0, stream, partials, count, ctrl);
    return hipGetLastError();
}

// The k lowest states overall from the per-wave lists (the final map-reduce
// step of sec. III.C with the list merge in place of the min).  One workgroup:
// each wave merges a strided quarter of the entries into its own WaveList,
// admitting only entries at or below its current k-th energy, then wave 0
// merges the other three lists.
__global__ __launch_bounds__(256) void lowest_merge_kernel(const LowEntry *__restrict__ lists,
                                                           uint64_t count, int k,
                                                           LowEntry *__restrict__ out,
                                                           int32_t *__restrict__ found)
{
    __shared__ LowEntry staged[kWaves - 1][kMaxLowest];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    WaveList wl;
    wl.k = k;
    wl.lane = lane;
    for (uint64_t b = (uint64_t)wave * 64; b < count; b += 64 * kWaves) {
        const uint64_t i = b + (uint64_t)lane;
        LowEntry le{INT_MAX, 0, ~0ull};
        if (i < count)
            le = lists[i];
        const int kt = wl.kth();
        const uint64_t mask = __builtin_amdgcn_ballot_w64(le.e != INT_MAX && le.e <= kt);
        wl.insert_lanes(mask, le.e, le.x);
    }
    if (wave > 0 && lane < k) {
        LowEntry le;
        le.e = wl.e;
        le.pad = 0;
        le.x = wl.x;
        staged[wave - 1][lane] = le;
    }
    __syncthreads();
    if (wave != 0)
        return;
    for (int w = 0; w < kWaves - 1; ++w) {
        LowEntry le{INT_MAX, 0, ~0ull};
        if (lane < k)
            le = staged[w][lane];
        const int kt = wl.kth();
        const uint64_t mask = __builtin_amdgcn_ballot_w64(le.e != INT_MAX && le.e <= kt);
        wl.insert_lanes(mask, le.e, le.x);
    }
    const uint64_t filled = __builtin_amdgcn_ballot_w64(lane < k && wl.e != INT_MAX);
    if (lane < k) {
        LowEntry le;
        le.e = wl.e;
        le.pad = 0;
        le.x = wl.x;
        out[lane] = le;
    }
    if (lane == 0)
        *found = (int32_t)__builtin_popcountll(filled);
}

hipError_t launch_lowest_merge(const LowEntry *lists, uint64_t count, int k, LowEntry *out,
                               int32_t *found, hipStream_t stream)
{
    if (k < 1 || k > kMaxLowest)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(lowest_merge_kernel, dim3(1), dim3(64 * kWaves), 0, stream, lists, count, k,
                       out, found);
    return hipGetLastError();
}

}  // namespace qubo
