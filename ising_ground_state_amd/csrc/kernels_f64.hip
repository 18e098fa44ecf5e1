// Exhaustive search of a real-valued (binary64) QUBO matrix on CDNA4 (gfx950).
//
// Maltsev, Remnev, Kapranov and Krivtsova, "Terastate-per-second QUBO
// Brute-Force on a Single GPU: A Matrix Prefix-Suffix Decomposition", name
// floating-point matrices as future work (sec. VI.B): the long incremental
// Gray-code updates accumulate rounding, to be handled by mixed precision or a
// periodic correction.  This kernel does both:
//   * energies are defined as the binary64 sum of Q_ij over i ascending with
//     x_i = 1 and, inside, j ascending with x_j = 1 (the definition of sec. I in
//     one fixed order);
//   * the walk is the integer kernel's decomposition (eq. 8, eq. 9): per column,
//     a binary64 anchor E64 follows the walk once per aligned group of 32
//     32-step bodies (two row updates per group), and every state's energy is
//     one fp32 add (the same 2-cycle rate as int32), re-anchored from E64 at
//     the start of every group, so at most 1023 fp32 adds separate a state
//     from its anchor;
//   * with S = sum |Q_ij|, an fp32 energy is within 1025 * 2^-24 S of exact:
//     the anchor's rounding, each add's (the sums stay below S), and the rows'
//     rounding to fp32 once (a state differs from its anchor by each row at
//     most once, and the rows of one column sum to at most S in magnitude);
//     the compare and gates add a few dozen 2^-24 S more (at most 1060 in
//     all), and the margin delta = 2^-13 S = 2048 * 2^-24 S covers that 1.93
//     times over; a state is
//     re-evaluated from the definition, in binary64 and in the same order as
//     the definition, whenever its fp32 energy is within delta of the threshold T;
//   * T only has to bound the minimum from above: it is lowered to the best
//     exact energy recorded and, before a body is walked exactly, to the body's
//     smallest fp32 energy plus delta (which bounds that state's exact energy).
//     Every minimiser passes every filter, so the minimum, its lowest index and
//     the count of states with exactly that energy are those of the definition.
#include "kernels_f64.h"
#include "dpp.h"

#include <cfloat>
#include <climits>
#include <cmath>

namespace qubo {
namespace {

constexpr int kU = 5;  // Gray bits with rows in VGPRs (fp32)
constexpr int kBody = 1 << kU;
constexpr int kWaves = 4;
constexpr int kR = kColsPerLaneF64;  // columns per lane
// Bodies share one binary64 anchor in aligned groups of 2^kAnchorBits: inside
// a group the fp32 walk runs on through the flips of Gray bits 5 .. 4+kAnchorBits
// (fp32 rows in LDS).
constexpr int kAnchorBits = 5;
constexpr int kAnchorGroup = 1 << kAnchorBits;
// The binary64 rows the anchor moves by at the end of an aligned group: Gray bit
// 4 + kAnchorBits and a bit above it.  Rows of lower bits are needed only when a
// unit starts inside a group, and are read from global memory then.
constexpr int kLdsFirstBit = kU - 1 + kAnchorBits;
static_assert(kLdsFirstBit == kLdsFirstBitF64, "LDS row layout shared with the host");

__device__ __forceinline__ uint64_t gray(uint64_t i) { return i ^ (i >> 1); }

__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ double uniform_f64(double v)
{
    return __longlong_as_double((long long)uniform64((uint64_t)__double_as_longlong(v)));
}

// Order-preserving integer key of a binary64 value (for an atomic minimum).
__device__ __forceinline__ long long order_key(double d)
{
    const long long b = __double_as_longlong(d);
    return b < 0 ? (b ^ 0x7fffffffffffffffLL) : b;
}

__device__ __forceinline__ double from_key(long long k)
{
    return __longlong_as_double(k < 0 ? (k ^ 0x7fffffffffffffffLL) : k);
}

__device__ __forceinline__ float fmin3(float a, float b, float c) { return fminf(fminf(a, b), c); }

// Minimum of two wave-uniform floats (never NaN) on the scalar unit: the
// integer keys b ^ ((b >> 31) & 0x7fffffff) order floats as their values.
__device__ __forceinline__ float uniform_fmin(float a, float b)
{
    const int ia = __float_as_int(a), ib = __float_as_int(b);
    const int ka = ia ^ ((ia >> 31) & 0x7fffffff), kb = ib ^ ((ib >> 31) & 0x7fffffff);
    return __int_as_float(ka < kb ? ia : ib);  // an integer select stays scalar
}

__device__ __forceinline__ float row_min8(const float (&E)[kR])
{
    // four three-input minima (E[5] twice): a two-input fminf would first
    // canonicalise its operands (two more instructions)
    return fmin3(fmin3(E[0], E[1], E[2]), fmin3(E[3], E[4], E[5]), fmin3(E[5], E[6], E[7]));
}

// The definition for one state: binary64, i ascending, j ascending, over the
// set variables of the n-variable index idx (variable 0 most significant).
__device__ double energy_def(const double *__restrict__ Q, int n, uint64_t idx)
{
    double e = 0.0;
    for (int i = 0; i < n; ++i) {
        if (!((idx >> (n - 1 - i)) & 1u))
            continue;
        const double *row = Q + (size_t)i * n;
        for (int j = 0; j < n; ++j)
            if ((idx >> (n - 1 - j)) & 1u)
                e += row[j];
    }
    return e;
}

__device__ __forceinline__ double bits_f64(uint64_t b) { return __longlong_as_double((long long)b); }
__device__ __forceinline__ uint64_t f64_bits(double d) { return (uint64_t)__double_as_longlong(d); }

// Minimum over the wave's lanes (none NaN) by the DPP steps of dpp.h, on the
// order-preserving integer keys; wave-uniform.
__device__ __forceinline__ double wave_min_f64(double v)
{
    const long long k = wave_reduce(order_key(v), (long long)0x7fffffffffffffffLL,
                                    [](long long a, long long b) { return a < b ? a : b; });
    return from_key(k);
}

__device__ __forceinline__ void combine(double &e, uint64_t &cnt, uint64_t &arg, double e2,
                                        uint64_t c2, uint64_t a2)
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

// {min energy, count at the min, lowest index at the min} over the wave's
// lanes: the DPP steps of dpp.h with `combine` as the operation (lanes outside
// a broadcast's rows meet the empty triple); the result is wave-uniform.
template <int Ctrl, int RowMask>
__device__ __forceinline__ void dpp_combine_step(double &e, uint64_t &cnt, uint64_t &arg)
{
    const double e2 = bits_f64(dpp_u64<Ctrl, RowMask>(0x7ff0000000000000ull, f64_bits(e)));
    const uint64_t c2 = dpp_u64<Ctrl, RowMask>(0, cnt);
    const uint64_t a2 = dpp_u64<Ctrl, RowMask>(~0ull, arg);
    combine(e, cnt, arg, e2, c2, a2);
}

__device__ __forceinline__ void wave_combine(double &e, uint64_t &cnt, uint64_t &arg)
{
    dpp_combine_step<kDppSwap1, 0xf>(e, cnt, arg);
    dpp_combine_step<kDppSwap2, 0xf>(e, cnt, arg);
    dpp_combine_step<kDppHalfMirror, 0xf>(e, cnt, arg);
    dpp_combine_step<kDppMirror, 0xf>(e, cnt, arg);
    dpp_combine_step<kDppBcast15, 0xa>(e, cnt, arg);
    dpp_combine_step<kDppBcast31, 0xc>(e, cnt, arg);
    e = bits_f64(readlane_u64(f64_bits(e), 63));
    cnt = readlane_u64(cnt, 63);
    arg = readlane_u64(arg, 63);
}

__device__ __forceinline__ uint64_t wave_sum(uint64_t v)
{
    return wave_reduce(v, (uint64_t)0, [](uint64_t a, uint64_t b) { return a + b; });
}

// ---------------------------------------------------------------------------
// Cache builders (binary64), as in the integer build.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void build_suffix_f64_kernel(const double *__restrict__ U, int ns,
                                                               int A, int B, uint64_t cols_padded,
                                                               double *__restrict__ es,
                                                               double *__restrict__ mint,
                                                               float *__restrict__ mint32)
{
    const uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= cols_padded)
        return;
    if (c >= (1ull << B)) {
        // padding column: +inf never passes a finite threshold, and zero rows keep it there
        es[c] = __longlong_as_double(0x7ff0000000000000LL);
        for (int v = 0; v < A; ++v) {
            mint[(uint64_t)v * cols_padded + c] = 0.0;
            mint32[(uint64_t)v * cols_padded + c] = 0.f;
        }
        return;
    }
    double e = 0.0;
    for (int i = 0; i < B; ++i) {
        if (!((c >> (B - 1 - i)) & 1u))
            continue;
        for (int j = i; j < B; ++j)
            if ((c >> (B - 1 - j)) & 1u)
                e += U[(A + i) * ns + (A + j)];
    }
    es[c] = e;
    for (int v = 0; v < A; ++v) {
        double m = 0.0;
        for (int j = 0; j < B; ++j)
            if ((c >> (B - 1 - j)) & 1u)
                m += U[v * ns + (A + j)];
        mint[(uint64_t)v * cols_padded + c] = m;
        mint32[(uint64_t)v * cols_padded + c] = (float)m;  // the walk's fp32 rows
    }
}

// ep[j] = E_p(g(j)) over the A prefix variables, and epmin[k] = min over body
// k of ep rounded to fp32.  Block-stride loop over 256-prefix blocks, Gray
// steps j_first <= j < j_end (j_first a multiple of 256, j_end of 32).  The
// 256 prefixes of a block share the high H = A - L bits of g(j) (L = min(A, 8)),
// so with x_p split into high and low parts
//   E_p = E_hi + sum_{a in lo, x_a = 1} (K[a] + sum_{b in lo, b >= a, x_b = 1} U[a][b]),
//   K[a] = sum_{w in hi, x_w = 1} U[w][a];
// a block computes K and one row of E_hi per high variable in parallel, and
// every thread adds the rows in the same order (no floating-point atomics, so
// the table does not depend on timing).  The order differs from the
// definition's; the walk only uses these values in its filters, whose margin
// covers any order.
__global__ __launch_bounds__(256) void build_prefix_f64_kernel(const double *__restrict__ U, int ns,
                                                               int A, uint64_t j_first, uint64_t j_end,
                                                               double *__restrict__ ep,
                                                               float *__restrict__ epmin)
{
    __shared__ double K[8];
    __shared__ double Upp[32][32];  // the A x A prefix part of U (A <= 32)
    __shared__ double ehi_row[32];  // H = A - 8 <= 24
    const int L = A < 8 ? A : 8, H = A - L;
    const int tid = threadIdx.x;
    for (int k = tid; k < A * A; k += blockDim.x)
        Upp[k / A][k % A] = k % A >= k / A ? U[(k / A) * ns + (k % A)] : 0.0;
    __syncthreads();
    for (uint64_t j0 = j_first + (uint64_t)blockIdx.x * blockDim.x; j0 < j_end;
         j0 += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t hi = gray(j0 >> L);  // high part of g(j), H bits (j0 is a multiple of 256)
        if (tid < L) {
            double k = 0.0;
            for (int w = 0; w < H; ++w)
                if ((hi >> (H - 1 - w)) & 1u)
                    k += Upp[w][H + tid];
            K[tid] = k;
        } else if (tid < L + H) {
            const int w = tid - L;
            double e = 0.0;
            if ((hi >> (H - 1 - w)) & 1u)
                for (int w2 = w; w2 < H; ++w2)
                    if ((hi >> (H - 1 - w2)) & 1u)
                        e += Upp[w][w2];
            ehi_row[w] = e;
        }
        __syncthreads();
        const uint64_t j = j0 + threadIdx.x;
        float m = __int_as_float(0x7f800000);
        if (j < j_end) {
            double e = 0.0;
            for (int w = 0; w < H; ++w)
                e += ehi_row[w];
            const uint32_t lo = (uint32_t)(gray(j) & ((1u << L) - 1));
            for (int a = 0; a < L; ++a) {
                if (!((lo >> (L - 1 - a)) & 1u))
                    continue;
                double row = K[a];
                for (int b = a; b < L; ++b)
                    if ((lo >> (L - 1 - b)) & 1u)
                        row += Upp[H + a][H + b];
                e += row;
            }
            ep[j] = e;
            m = (float)e;
        }
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1)
            m = fminf(m, __shfl_xor(m, off, 64));
        if (j < j_end && (j & 31) == 0)
            epmin[j >> 5] = m;
        __syncthreads();  // K and ehi_row are rewritten by the next block
    }
}

// The group gate's prefix bound: the minimum of the body minima over each
// aligned group of four bodies.  Groups that straddle the slice's ends get
// values that are never read.
__global__ __launch_bounds__(256) void build_group_min_f64_kernel(const float *__restrict__ epmin,
                                                                  float *__restrict__ epmin4,
                                                                  uint64_t k_first, uint64_t k_end)
{
    const uint64_t k = k_first + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= k_end)
        return;
    const float *e = epmin + 4 * k;
    epmin4[k] = fminf(fminf(e[0], e[1]), fminf(e[2], e[3]));
}

__global__ void init_ctrl_f64_kernel(CtrlF64 *ctrl, double t0, float *epmin_pad, float *epmin4_pad)
{
    epmin_pad[0] = __int_as_float(0x7f800000);
    epmin_pad[1] = __int_as_float(0x7f800000);
    epmin4_pad[0] = __int_as_float(0x7f800000);
    ctrl->counter = 0;
    ctrl->gbest = order_key(t0);
    ctrl->slow_total = 0;
    ctrl->bodies_total = 0;
    ctrl->candidates_total = 0;
}

// ---------------------------------------------------------------------------
// The search.
// ---------------------------------------------------------------------------

// Per-lane record between exact walks, kept in LDS.
struct RecordF64 {
    double e;
    uint64_t cnt;
    uint64_t arg;
};

__device__ __forceinline__ void materialise(float (&E)[kR])
{
#pragma unroll
    for (int r = 0; r < kR; ++r)
        asm volatile("" : "+v"(E[r]));
}

template <bool Plus>
__device__ __forceinline__ void step_rows(float (&E)[kR], const float (&M)[kR])
{
#pragma unroll
    for (int r = 0; r < kR; ++r)
        E[r] = Plus ? E[r] + M[r] : E[r] - M[r];
}

// The flip of Gray bit t (wave-uniform; t >= kU flips no row here) with sign s
// (+-1): one branch per row, each add an fma by +-1 (rounded once, as the add).
__device__ __forceinline__ void flip_row(float (&E)[kR], const float (&Mr)[kU][kR], int t, float s)
{
    switch (t) {
#define QUBO_FLIP_CASE(k)                          \
    case k:                                        \
        _Pragma("unroll") for (int r = 0; r < kR; ++r) \
            E[r] = fmaf(Mr[k][r], s, E[r]);        \
        break;
        QUBO_FLIP_CASE(0)
        QUBO_FLIP_CASE(1)
        QUBO_FLIP_CASE(2)
        QUBO_FLIP_CASE(3)
        QUBO_FLIP_CASE(4)
#undef QUBO_FLIP_CASE
    default:
        break;
    }
}

// Sign of the flip leaving step m of a body (Gray bit t = ctz(m + 1)): bits
// below kU - 1 by the step index, bit kU - 1 by the body (top_plus).
__device__ __forceinline__ float flip_sign(int m, int t, bool top_plus)
{
    if (t < kU - 1)
        return (((m + 1) >> (t + 1)) & 1) ? -1.f : 1.f;
    return top_plus ? 1.f : -1.f;
}

// The low-energy spectrum for a real-valued Q: a wave keeps the k lowest
// states it has evaluated from the definition, in the order (E ascending,
// index ascending), one per lane (lane i holds the i-th; empty slots hold
// +inf).  A state goes in by counting the entries before it (a ballot) and
// shifting the later ones up one lane.  As for integers, any wave's k-th
// energy bounds the k-th lowest energy overall from above, and a state among
// the k lowest overall is never displaced from its wave's list.
struct WaveListF64 {
    double e = __longlong_as_double(0x7ff0000000000000LL);
    uint64_t x = ~0ull;
    int k = 1;     // entries kept (1..64), wave-uniform
    int lane = 0;

    __device__ __forceinline__ void insert(double ce, uint64_t cx)
    {
        const bool before = lane < k && (e < ce || (e == ce && x < cx));
        const int pos = __builtin_popcountll(__builtin_amdgcn_ballot_w64(before));
        if (pos >= k)
            return;
        const double eu = __shfl_up(e, 1, 64);
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
    __device__ __forceinline__ void insert_lanes(uint64_t mask, double ce, uint64_t cx)
    {
        while (mask) {
            const int l = __builtin_ctzll(mask);
            mask &= mask - 1;
            const uint64_t eb = (uint64_t)__double_as_longlong(ce);
            const uint32_t elo = __builtin_amdgcn_readlane((uint32_t)eb, l);
            const uint32_t ehi = __builtin_amdgcn_readlane((uint32_t)(eb >> 32), l);
            const uint32_t xlo = __builtin_amdgcn_readlane((uint32_t)cx, l);
            const uint32_t xhi = __builtin_amdgcn_readlane((uint32_t)(cx >> 32), l);
            insert(__longlong_as_double((long long)(((uint64_t)ehi << 32) | elo)),
                   ((uint64_t)xhi << 32) | xlo);
        }
    }

    // k-th energy of the list (+inf until k states are in it), wave-uniform.
    __device__ __forceinline__ double kth() const
    {
        const uint64_t eb = (uint64_t)__double_as_longlong(e);
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)eb, k - 1);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(eb >> 32), k - 1);
        return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    }
};

// One unrolled body of 32 states: 31 fp32 row updates, every state's energy
// kept in registers (one add per state).
__device__ __forceinline__ void adds_body(float (&E)[kR], const float (&Mr)[kU][kR], bool top_plus)
{
#pragma unroll
    for (int m = 0; m + 1 < kBody; ++m) {
        const int t = __builtin_ctz((unsigned)(m + 1));
        if (t < kU - 1) {
            if ((((m + 1) >> (t + 1)) & 1) == 0)
                step_rows<true>(E, Mr[t]);
            else
                step_rows<false>(E, Mr[t]);
        } else {
            if (top_plus)
                step_rows<true>(E, Mr[kU - 1]);
            else
                step_rows<false>(E, Mr[kU - 1]);
        }
        materialise(E);
    }
}

// Four waves per SIMD: the register budget (128 VGPRs) the compiler must meet.
// Lowest: keep each wave's k lowest states (args.lists) instead of the
// minimum, its count and lowest minimiser; the threshold is then the k-th
// energy, and the first pass of an exact walk (which bounds only the minimum)
// is skipped.
template <bool Lowest>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void gray_search_f64_kernel(const double *__restrict__ es,
                                                              const double *__restrict__ mint,
                                                              const float *__restrict__ mint32,
                                                              const double *__restrict__ ep,
                                                              const float *__restrict__ epmin,
                                                              const double *__restrict__ Q,
                                                              PartialF64 *__restrict__ partials,
                                                              CtrlF64 *__restrict__ ctrl,
                                                              const SearchArgsF64 a)
{
    constexpr int kGroup = 64 * kR;
    extern __shared__ double lds_rows64[];  // [l_eff - 7][kGroup]: rows of Gray bits 7 .. l_eff-1
    __shared__ unsigned long long item_sh;
    __shared__ double rec_e[64 * kWaves];
    __shared__ uint64_t rec_c[64 * kWaves], rec_a[64 * kWaves];
    __shared__ float carry32[kAnchorBits][kGroup];  // fp32 rows of Gray bits 5 .. 4+kAnchorBits

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int A = a.A, B = a.B;
    const uint64_t cp = a.cols_padded;
    const double *lds_lane = lds_rows64 - kLdsFirstBit * kGroup + lane;  // row of bit t: lds_lane + t * kGroup
    // The lane's offset passes through an empty asm: knowing its range, the
    // compiler turned "+ r * 64" into bitwise ors that it does not fold into the
    // LDS reads' immediate offsets, and spent a VALU instruction per register.
    int lane_off = lane;
    asm volatile("" : "+v"(lane_off));
    const float *carry_lane = &carry32[0][0] + lane_off;  // row of bit 5+i: carry_lane + i * kGroup

    rec_e[threadIdx.x] = __longlong_as_double(0x7ff0000000000000LL);
    rec_c[threadIdx.x] = 0;
    rec_a[threadIdx.x] = ~0ull;

    uint32_t bodies = 0, slow = 0, candidates = 0;
    double T = uniform_f64(from_key(
        __hip_atomic_load(&ctrl->gbest, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
    long long cur_g = -1;

    for (;;) {
        if (threadIdx.x == 0)
            item_sh = atomicAdd(&ctrl->counter, 1ull);
        __syncthreads();
        const uint64_t item = uniform64(item_sh);
        __syncthreads();
        if (item >= a.items)
            break;
        const uint64_t g = item / a.seg_blocks;
        const uint64_t sb = item - g * a.seg_blocks;
        if ((long long)g != cur_g) {
            const int rows = a.l_eff > kLdsFirstBit ? a.l_eff - kLdsFirstBit : 0;
            for (int k = threadIdx.x; k < rows * kGroup; k += blockDim.x) {
                const int t = kLdsFirstBit + k / kGroup;
                const int col = k % kGroup;
                lds_rows64[k] = mint[(uint64_t)(A - 1 - t) * cp + g * kGroup + col];
            }
            for (int k = threadIdx.x; k < kAnchorBits * kGroup; k += blockDim.x) {
                const int t = kU + k / kGroup;
                carry32[0][k] = t < A ? mint32[(uint64_t)(A - 1 - t) * cp + g * kGroup + k % kGroup] : 0.f;
            }
            __syncthreads();
            cur_g = (long long)g;
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

        const uint64_t col0 = g * kGroup + (uint64_t)lane;
        // binary64 anchors at the segment's first prefix (eq. 8)
        double E64[kR];
        {
            const double *src = es + col0;
#pragma unroll
            for (int r = 0; r < kR; ++r)
                E64[r] = src[r * 64];
            uint64_t bits = gray(j_begin);
            while (bits) {
                const int t = __builtin_ctzll(bits);
                bits &= bits - 1;
                const double *row = mint + (uint64_t)(A - 1 - t) * cp + col0;
#pragma unroll
                for (int r = 0; r < kR; ++r)
                    E64[r] += row[r * 64];
            }
        }
        float Mr[kU][kR];
#pragma unroll
        for (int t = 0; t < kU; ++t) {
            const float *row = mint32 + (uint64_t)(A - 1 - t) * cp + col0;
#pragma unroll
            for (int r = 0; r < kR; ++r)
                Mr[t][r] = row[r * 64];
        }
        // Lane bounds of the fall within a body (s = bit 4 at its start), a pair
        // of bodies (bit 5 at its start) and an aligned group of four (bits 0..5
        // start at 0; bit 6 at its start), in fp32 (their rounding is in delta).
        float beta_s0 = INFINITY, beta_s1 = INFINITY, beta_p0 = INFINITY, beta_p1 = INFINITY;
        float beta_q0 = INFINITY, beta_q1 = INFINITY;
        {
#pragma unroll
            for (int r = 0; r < kR; ++r) {
                float b = 0.f;
#pragma unroll
                for (int t = 0; t < kU; ++t)
                    b += fminf(Mr[t][r], 0.f);
                beta_s0 = fminf(beta_s0, b);
                beta_s1 = fminf(beta_s1, b - Mr[kU - 1][r]);
                const float m5 = carry_lane[r * 64];           // 0 when A = 5
                const float m6 = carry_lane[kGroup + r * 64];  // 0 when A <= 6
                beta_p0 = fminf(beta_p0, b + fminf(m5, 0.f));
                beta_p1 = fminf(beta_p1, b - fmaxf(m5, 0.f));
                const float b5 = b + fminf(m5, 0.f);
                beta_q0 = fminf(beta_q0, b5 + fminf(m6, 0.f));
                beta_q1 = fminf(beta_q1, b5 - fmaxf(m6, 0.f));
            }
        }
        {
            const double gb = uniform_f64(from_key(__hip_atomic_load(
                &ctrl->gbest, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
            T = gb < T ? gb : T;
        }
        float TD = (float)T + a.delta;  // filter threshold: E32 + E_p32 <= TD

        // Bodies are counted by their index b = j >> 5, a 32-bit value (A <= 32),
        // so that the per-body bookkeeping is 32-bit scalar arithmetic; the
        // 64-bit Gray step is formed only on the rare paths that need it.
        const uint32_t nbodies = (uint32_t)((j_end - j_begin) >> kU);
        const uint32_t b0 = (uint32_t)(j_begin >> kU);
        // The group gate's prefix bound comes from the per-group table, read one
        // group ahead (one padding entry past the last group); the body minima are
        // read only where a pair or body gate needs them.
        float q_next = A > kU + 1 ? a.epmin4[(b0 + 3) >> 2] : 0.f;
        uint32_t covered = 0;  // bodies ahead that a pair or group bound has cleared
        float E[kR];
        uint64_t anchor_j = j_begin;  // E64 holds the suffix energies at prefix g(anchor_j)
        for (uint32_t bi = 0; bi < nbodies; ++bi) {
            uint32_t b = b0 + bi;
            bool last = bi + 1 == nbodies;
            const bool top_plus = (b & 1u) == 0;
            // The first body of an aligned group, and a unit's first body, start
            // from the binary64 anchor E64 (rounded to nearest); the others
            // continue the fp32 walk, so E64 moves once per group.
            uint32_t in_group = b & (kAnchorGroup - 1);
            const bool carried = in_group != 0 && bi != 0;
            if (!carried) {
#pragma unroll
                for (int r = 0; r < kR; ++r)
                    E[r] = (float)E64[r];
            }
            bool check;
            if (covered != 0) {
                check = false;
                --covered;
            } else {
                const float emin = row_min8(E);
                if ((in_group & 3u) == 0 && bi + 3 < nbodies && A > kU + 1) {
                    // four aligned bodies (never across an anchor group)
                    const float q = q_next;
                    q_next = a.epmin4[(b >> 2) + 1];
                    const float bq = emin + (((b >> 2) & 1u) ? beta_q1 : beta_q0);
                    if (__builtin_amdgcn_ballot_w64(bq + q <= TD) == 0)
                        covered = 3;
                }
                if (covered != 0) {
                    check = false;
                } else {
                    const float epm_cur = epmin[b];
                    if (top_plus && !last && A > kU) {
                        const float bp = emin + (((b >> 1) & 1u) ? beta_p1 : beta_p0);
                        if (__builtin_amdgcn_ballot_w64(bp + uniform_fmin(epm_cur, epmin[b + 1]) <= TD) == 0)
                            covered = 1;
                    }
                    if (covered != 0) {
                        check = false;
                    } else {
                        const float bound = emin + (top_plus ? beta_s0 : beta_s1);
                        check = __builtin_amdgcn_ballot_w64(bound + epm_cur <= TD) != 0;
                    }
                }
            }
            ++bodies;
            if (!check && (b & 3u) == 0 && covered >= 3) {
                // An aligned group of four bodies cleared by the group bound: all
                // four run here with their row signs fixed, joined by the flips of
                // Gray bits 5, 6 and 5 (inside the anchor group).
                float row[kR];
                adds_body(E, Mr, true);
#pragma unroll
                for (int r = 0; r < kR; ++r)
                    row[r] = carry_lane[r * 64];
                if ((((b + 1) >> 1) & 1u) == 0)
                    step_rows<true>(E, row);
                else
                    step_rows<false>(E, row);
                adds_body(E, Mr, false);
#pragma unroll
                for (int r = 0; r < kR; ++r)
                    row[r] = carry_lane[kGroup + r * 64];
                if ((((b + 2) >> 2) & 1u) == 0)
                    step_rows<true>(E, row);
                else
                    step_rows<false>(E, row);
                adds_body(E, Mr, true);
#pragma unroll
                for (int r = 0; r < kR; ++r)
                    row[r] = carry_lane[r * 64];
                if ((((b + 3) >> 1) & 1u) == 0)
                    step_rows<true>(E, row);
                else
                    step_rows<false>(E, row);
                covered -= 3;
                bodies += 3;
                bi += 3;
                b += 3;
                last = bi + 1 == nbodies;
                in_group = b & (kAnchorGroup - 1);
                adds_body(E, Mr, false);
            } else if (!check && top_plus && covered != 0) {
                // An even body whose odd partner a bound has cleared too: both run
                // here with their row signs fixed, joined by the flip of Gray bit 5
                // (inside the anchor group: an even body is never its last).
                adds_body(E, Mr, true);
                const uint32_t b1 = b + 1;
                float row5[kR];
#pragma unroll
                for (int r = 0; r < kR; ++r)
                    row5[r] = carry_lane[r * 64];
                if (((b1 >> 1) & 1u) == 0)
                    step_rows<true>(E, row5);
                else
                    step_rows<false>(E, row5);
                --covered;
                ++bodies;
                ++bi;
                b = b1;
                last = bi + 1 == nbodies;
                in_group = b & (kAnchorGroup - 1);
                adds_body(E, Mr, false);
            } else if (!check) {
                adds_body(E, Mr, top_plus);
            } else {
                // Exact walk: every state within delta of T is re-evaluated.
                ++slow;
                const uint64_t base = (uint64_t)b << kU;
                const uint64_t colbase = g * kGroup;
                // First pass: the body's smallest fp32 energy plus delta bounds
                // the best exact energy in the body from above, so T (which only
                // has to bound the minimum from above) falls to it before any
                // state is re-evaluated.
                if (!Lowest) {
                    float W[kR];  // the walk on a copy: E stays at the body's first state
#pragma unroll
                    for (int r = 0; r < kR; ++r)
                        W[r] = E[r];
                    float est = INFINITY;
#pragma unroll 1
                    for (int m = 0; m < kBody; ++m) {
                        const float ep32 = (float)ep[base + (uint64_t)m];
#pragma unroll
                        for (int r = 0; r < kR; ++r)
                            est = fminf(est, W[r] + ep32);
                        const int t = __builtin_ctz((unsigned)(m + 1));
                        flip_row(W, Mr, t, flip_sign(m, t, top_plus));
                    }
#pragma unroll
                    for (int off = 32; off >= 1; off >>= 1)
                        est = fminf(est, __shfl_xor(est, off, 64));
                    const double up = (double)__uint_as_float(
                        __builtin_amdgcn_readfirstlane(__float_as_uint(est + a.delta)));
                    T = up < T ? up : T;
                    TD = (float)T + a.delta;
                }
                if (Lowest) {
                    WaveListF64 wl;
                    wl.k = a.k_low;
                    wl.lane = lane;
                    wl.e = rec_e[threadIdx.x];
                    wl.x = rec_a[threadIdx.x];
#pragma unroll 1
                    for (int m = 0; m < kBody; ++m) {
                        const uint64_t j = base + (uint64_t)m;
                        const float ep32 = (float)ep[j];
                        const uint64_t hi = (gray(j) << B) | colbase;
                        uint32_t hits = 0;
#pragma unroll
                        for (int r = 0; r < kR; ++r)
                            hits |= (E[r] + ep32 <= TD ? 1u : 0u) << r;
                        // one candidate per lane per round, evaluated side by side,
                        // then offered to the list lane by lane
                        while (__builtin_amdgcn_ballot_w64(hits != 0)) {
                            double v = 0.0;
                            uint64_t real = 0;
                            bool ok = false;
                            if (hits) {
                                const int r = __builtin_ctz(hits);
                                hits &= hits - 1;
                                const uint64_t idx = hi | ((uint64_t)r << 6) | (uint64_t)lane;
                                if ((idx & ((1ull << a.pad) - 1)) == 0) {
                                    ++candidates;
                                    real = idx >> a.pad;
                                    v = energy_def(Q, a.n, real);
                                    ok = true;
                                }
                            }
                            wl.insert_lanes(__builtin_amdgcn_ballot_w64(ok), v, real);
                        }
                        const int t = __builtin_ctz((unsigned)(m + 1));
                        flip_row(E, Mr, t, flip_sign(m, t, top_plus));
                    }
                    rec_e[threadIdx.x] = wl.e;
                    rec_a[threadIdx.x] = wl.x;
                    const double kt = wl.kth();
                    T = kt < T ? kt : T;
                } else {
                    RecordF64 rec{rec_e[threadIdx.x], rec_c[threadIdx.x], rec_a[threadIdx.x]};
#pragma unroll 1
                    for (int m = 0; m < kBody; ++m) {
                        const uint64_t j = base + (uint64_t)m;
                        const float ep32 = (float)ep[j];
                        const uint64_t hi = (gray(j) << B) | colbase;
                        uint32_t hits = 0;  // columns r whose state passes the filter
#pragma unroll
                        for (int r = 0; r < kR; ++r)
                            hits |= (E[r] + ep32 <= TD ? 1u : 0u) << r;
                        while (hits) {
                            const int r = __builtin_ctz(hits);
                            hits &= hits - 1;
                            const uint64_t idx = hi | ((uint64_t)r << 6) | (uint64_t)lane;
                            if ((idx & ((1ull << a.pad) - 1)) == 0) {
                                ++candidates;
                                const uint64_t real = idx >> a.pad;
                                const double v = energy_def(Q, a.n, real);
                                if (v < rec.e) {
                                    rec.e = v;
                                    rec.cnt = 1;
                                    rec.arg = real;
                                } else if (v == rec.e) {
                                    rec.cnt += 1;
                                    rec.arg = real < rec.arg ? real : rec.arg;
                                }
                            }
                        }
                        // flip into the next state (after the last one t = 5: no row)
                        const int t = __builtin_ctz((unsigned)(m + 1));
                        flip_row(E, Mr, t, flip_sign(m, t, top_plus));
                    }
                    rec_e[threadIdx.x] = rec.e;
                    rec_c[threadIdx.x] = rec.cnt;
                    rec_a[threadIdx.x] = rec.arg;
                    const double wm = uniform_f64(wave_min_f64(rec.e));
                    T = wm < T ? wm : T;
                }
                atomicMin(&ctrl->gbest, order_key(T));
                const double gb = uniform_f64(from_key(__hip_atomic_load(
                    &ctrl->gbest, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
                T = gb < T ? gb : T;
                TD = (float)T + a.delta;
            }
            // To the next body (after the unit's last body nothing is needed).
            // Signed adds are fma with a wave-uniform +-1: rounded once, with no
            // sign select per register.
            if (!last) {
                if (in_group != kAnchorGroup - 1) {
                    // inside a group: the fp32 walk flips Gray bit 5 + c into the next
                    // body, c = ctz(in_group + 1) < kAnchorBits (two-operand adds: a
                    // three-register fma issues at half rate); its sign is bit c + 1
                    // of the next body's index.  The row's LDS address is one VALU
                    // add of the uniform offset c * kGroup (a branch per carried bit
                    // with constant offsets measured 0.3 % slower).
                    const uint32_t c = __builtin_ctz(in_group + 1);
                    float row[kR];
                    const float *src = carry_lane + c * kGroup;
#pragma unroll
                    for (int r = 0; r < kR; ++r)
                        row[r] = src[r * 64];
                    if ((((b + 1) >> (c + 1)) & 1u) == 0)
                        step_rows<true>(E, row);
                    else
                        step_rows<false>(E, row);
                } else {
                    // E64 from g(anchor_j) to g(next): one signed row per differing
                    // bit (an aligned group: Gray bit 4 + kAnchorBits and the bit
                    // t >= 5 + kAnchorBits of the next group).
                    const uint64_t next = (uint64_t)(b + 1) << kU;
                    const uint64_t gn = gray(next);
                    uint64_t diff = gray(anchor_j) ^ gn;
                    while (diff) {
                        const int t = __builtin_ctzll(diff);
                        diff &= diff - 1;
                        const double st = ((gn >> t) & 1u) ? 1.0 : -1.0;
                        double row[kR];
                        if (t >= kLdsFirstBit && t < a.l_eff) {
                            const double *src = lds_lane + t * kGroup;
#pragma unroll
                            for (int r = 0; r < kR; ++r)
                                row[r] = src[r * 64];
                        } else {
                            const double *src = mint + (uint64_t)(A - 1 - t) * cp + col0;
#pragma unroll
                            for (int r = 0; r < kR; ++r)
                                row[r] = src[r * 64];
                        }
#pragma unroll
                        for (int r = 0; r < kR; ++r)
                            E64[r] = fma(row[r], st, E64[r]);
                    }
                    anchor_j = next;
                }
            }
        }
    }

    double e = rec_e[threadIdx.x];
    uint64_t cnt = rec_c[threadIdx.x], arg = rec_a[threadIdx.x];
    if (Lowest) {
        if (lane < a.k_low) {
            LowEntryF64 le;
            le.e = e;
            le.x = arg;
            a.lists[((uint64_t)blockIdx.x * kWaves + wave) * (uint64_t)a.k_low + (uint64_t)lane] = le;
        }
        cnt = 0;  // the partials carry the statistics only
    }
    wave_combine(e, cnt, arg);
    const uint64_t cand = wave_sum(candidates);
    // Workgroup stage through LDS: one slot per wave, combined in wave order by
    // one thread into the workgroup's partial.  The waves of a workgroup leave
    // the item loop together, so all of them reach the barrier.
    __shared__ PartialF64 wg_part[kWaves];
    if (lane == 0) {
        PartialF64 p;
        p.e = e;
        p.count = cnt;
        p.arg = arg;
        p.bodies = bodies;
        p.slow = slow;
        p.pad = 0;
        p.candidates = cand;
        wg_part[wave] = p;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        PartialF64 p = wg_part[0];
        for (int w = 1; w < kWaves; ++w) {
            const PartialF64 &o = wg_part[w];
            combine(p.e, p.count, p.arg, o.e, o.count, o.arg);
            p.bodies += o.bodies;
            p.slow += o.slow;
            p.candidates += o.candidates;
        }
        partials[blockIdx.x] = p;
    }
}

__global__ __launch_bounds__(256) void reduce_f64_kernel(const PartialF64 *__restrict__ partials,
                                                         int count, CtrlF64 *ctrl)
{
    __shared__ double se[4];
    __shared__ uint64_t sc[4], sa[4], ss[4], sb[4], sk[4];
    double e = __longlong_as_double(0x7ff0000000000000LL);
    uint64_t cnt = 0, arg = ~0ull, slow = 0, bodies = 0, cand = 0;
    for (int k = threadIdx.x; k < count; k += blockDim.x) {
        const PartialF64 p = partials[k];
        combine(e, cnt, arg, p.e, p.count, p.arg);
        slow += p.slow;
        bodies += p.bodies;
        cand += p.candidates;
    }
    wave_combine(e, cnt, arg);
    slow = wave_sum(slow);
    bodies = wave_sum(bodies);
    cand = wave_sum(cand);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        se[w] = e;
        sc[w] = cnt;
        sa[w] = arg;
        ss[w] = slow;
        sb[w] = bodies;
        sk[w] = cand;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < (int)(blockDim.x >> 6); ++k) {
            combine(e, cnt, arg, se[k], sc[k], sa[k]);
            slow += ss[k];
            bodies += sb[k];
            cand += sk[k];
        }
        ctrl->result.e = e;
        ctrl->result.count = cnt;
        ctrl->result.arg = arg;
        ctrl->slow_total = slow;
        ctrl->bodies_total = bodies;
        ctrl->candidates_total = cand;
    }
}

// Merges the per-wave lists into the k lowest: each of the 4 waves of one
// workgroup folds a strided quarter of the entries into its own list (offering
// only entries at or below its current k-th energy), then wave 0 merges the
// other three lists.
__global__ __launch_bounds__(256) void lowest_merge_f64_kernel(const LowEntryF64 *__restrict__ lists,
                                                               uint64_t count, int k,
                                                               LowEntryF64 *__restrict__ out,
                                                               int32_t *__restrict__ found)
{
    __shared__ LowEntryF64 staged[kWaves - 1][64];
    const double inf = __longlong_as_double(0x7ff0000000000000LL);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    WaveListF64 wl;
    wl.k = k;
    wl.lane = lane;
    for (uint64_t b = (uint64_t)wave * 64; b < count; b += 64 * kWaves) {
        const uint64_t i = b + (uint64_t)lane;
        LowEntryF64 le{inf, ~0ull};
        if (i < count)
            le = lists[i];
        const double kt = wl.kth();
        wl.insert_lanes(__builtin_amdgcn_ballot_w64(le.e != inf && le.e <= kt), le.e, le.x);
    }
    if (wave > 0 && lane < k)
        staged[wave - 1][lane] = LowEntryF64{wl.e, wl.x};
    __syncthreads();
    if (wave != 0)
        return;
    for (int w = 0; w < kWaves - 1; ++w) {
        LowEntryF64 le{inf, ~0ull};
        if (lane < k)
            le = staged[w][lane];
        const double kt = wl.kth();
        wl.insert_lanes(__builtin_amdgcn_ballot_w64(le.e != inf && le.e <= kt), le.e, le.x);
    }
    const uint64_t filled = __builtin_amdgcn_ballot_w64(lane < k && wl.e != inf);
    if (lane < k)
        out[lane] = LowEntryF64{wl.e, wl.x};
    if (lane == 0)
        *found = (int32_t)__builtin_popcountll(filled);
}

}  // namespace

hipError_t launch_build_tables_f64(const double *U, int ns, int A, int B, uint64_t cols_padded,
                                   double *es, double *mint, float *mint32, double *ep,
                                   float *epmin, float *epmin4, uint64_t j_lo, uint64_t j_hi,
                                   hipStream_t stream)
{
    const unsigned g1 = (unsigned)((cols_padded + 255) / 256);
    hipLaunchKernelGGL(build_suffix_f64_kernel, dim3(g1), dim3(256), 0, stream, U, ns, A, B,
                       cols_padded, es, mint, mint32);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    if (A < 5 || A > 32 || j_lo >= j_hi || j_hi > (1ull << A) || (j_lo & 31) || (j_hi & 31))
        return hipErrorInvalidValue;  // (the builder stages at most 32 x 32 entries of U)
    const uint64_t j_first = j_lo & ~uint64_t(255);
    const uint64_t blocks = (j_hi - j_first + 255) / 256;
    const uint64_t grid = blocks < (1ull << 14) ? blocks : (1ull << 14);
    hipLaunchKernelGGL(build_prefix_f64_kernel, dim3((unsigned)grid), dim3(256), 0, stream, U, ns,
                       A, j_first, j_hi, ep, epmin);
    err = hipGetLastError();
    if (err != hipSuccess || A < kU + 2)
        return err;
    // groups of four bodies holding the slice's bodies (inside the 256-step
    // blocks the prefix builder just wrote)
    const uint64_t k_first = j_lo >> (kU + 2), k_end = ((j_hi - 1) >> (kU + 2)) + 1;
    const uint64_t g3 = (k_end - k_first + 255) / 256;
    if (g3 > 0xffffffffull)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(build_group_min_f64_kernel, dim3((unsigned)g3), dim3(256), 0, stream, epmin, epmin4,
                       k_first, k_end);
    return hipGetLastError();
}

hipError_t launch_init_ctrl_f64(CtrlF64 *ctrl, double t0, float *epmin_pad, float *epmin4_pad,
                                hipStream_t stream)
{
    hipLaunchKernelGGL(init_ctrl_f64_kernel, dim3(1), dim3(1), 0, stream, ctrl, t0, epmin_pad, epmin4_pad);
    return hipGetLastError();
}

hipError_t launch_search_f64(const SearchArgsF64 &args, bool lowest, int blocks, int lds_bytes,
                             hipStream_t stream)
{
    if (lowest && (args.k_low < 1 || args.k_low > 64 || !args.lists))
        return hipErrorInvalidValue;
    if (lowest)
        hipLaunchKernelGGL(gray_search_f64_kernel<true>, dim3(blocks), dim3(64 * kWaves), lds_bytes,
                           stream, args.es, args.mint, args.mint32, args.ep, args.epmin, args.Q,
                           args.partials, args.ctrl, args);
    else
        hipLaunchKernelGGL(gray_search_f64_kernel<false>, dim3(blocks), dim3(64 * kWaves), lds_bytes,
                           stream, args.es, args.mint, args.mint32, args.ep, args.epmin, args.Q,
                           args.partials, args.ctrl, args);
    return hipGetLastError();
}

hipError_t search_occupancy_f64(bool lowest, int *blocks_per_cu, int lds_bytes)
{
    const void *fn = lowest ? reinterpret_cast<const void *>(gray_search_f64_kernel<true>)
                            : reinterpret_cast<const void *>(gray_search_f64_kernel<false>);
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, 64 * kWaves, (size_t)lds_bytes);
}

hipError_t launch_lowest_merge_f64(const LowEntryF64 *lists, uint64_t count, int k, LowEntryF64 *out,
                                   int32_t *found, hipStream_t stream)
{
    if (k < 1 || k > 64)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(lowest_merge_f64_kernel, dim3(1), dim3(64 * kWaves), 0, stream, lists, count, k,
                       out, found);
    return hipGetLastError();
}

hipError_t launch_reduce_f64(const PartialF64 *partials, int count, CtrlF64 *ctrl,
                             hipStream_t stream)
{
    hipLaunchKernelGGL(reduce_f64_kernel, dim3(1), dim3(256), 0, stream, partials, count, ctrl);
    return hipGetLastError();
}

}  // namespace qubo
