// Exhaustive search of a real-valued (binary64) QUBO matrix on CDNA4 (gfx950).
//
// Maltsev, Remnev, Kapranov and Krivtsova, "Terastate-per-second QUBO
// Brute-Force on a Single GPU: A Matrix Prefix-Suffix Decomposition", name
// floating-point matrices as future work (sec. VI.B): the long incremental
// Gray-code updates accumulate rounding, to be handled by mixed precision or a
// periodic correction.  Here the walk carries no rounding at all:
//   * energies are defined as the binary64 sum of Q_ij over i ascending with
//     x_i = 1 and, inside, j ascending with x_j = 1 (the definition of sec. I in
//     one fixed order);
//   * the tables of the decomposition (eq. 8) are formed in binary64, scaled by
//     s = 2^e (exact) and rounded once each to the nearest integer; the walk is
//     the integer search's walk over these tables (walk.h: eq. 9, one int32 add
//     per state, with its bound gates), so the walked value of a state,
//       W(x) = rint(s E_s(c)) + sum_{k set in x_p} rint(s M_int[k][c]) + rint(s E_p(x_p)),
//     is exact whatever the length of the walk;
//   * W(x) differs from s E(x) by at most (A + 2) / 2 (one half per rounded
//     term: E_s, E_p and at most A rows) plus s times the binary64 rounding of
//     the tables and of the definition (under 2 n^2 2^-53 S with S = sum |Q_ij|,
//     i.e. under 2^-12 for s S <= 2^28), so |W(x) - s E(x)| < M - 1 with
//     M = A / 2 + 3;
//   * a state is re-evaluated from the definition, in binary64 and in the
//     definition's order, whenever W(x) <= floor(s T) + M, where T bounds the
//     minimum from above (the best binary64 energy found, shared between waves,
//     or the first threshold): every minimiser x has E(x) <= T, so
//     W(x) < s E(x) + M - 1 <= floor(s T) + M;
//   * before a body's states are re-evaluated, the filter threshold falls to
//     the body's smallest W plus 2 M: that state's binary64 energy is below
//     (W + M - 1) / s, so every minimiser's W is below W + 2 M - 2.
// The minimum, its lowest index and the count of states with exactly that
// energy are therefore those of the definition.
#include "kernels_f64.h"
#include "dpp.h"
#include "walk.h"

#include <climits>
#include <cmath>

namespace qubo {
namespace {

constexpr int kR = kColsPerLaneF64;  // columns per lane

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

__device__ __forceinline__ double bits_f64(uint64_t b) { return __longlong_as_double((long long)b); }
__device__ __forceinline__ uint64_t f64_bits(double d) { return (uint64_t)__double_as_longlong(d); }

__device__ __forceinline__ double uniform_f64(double v) { return bits_f64(uniform64(f64_bits(v))); }

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

__device__ __forceinline__ int wave_min_i32(int v)
{
    return wave_reduce(v, INT_MAX, [](int a, int b) { return a < b ? a : b; });
}

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
// Cache builders: binary64 sums, each scaled and rounded once.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int32_t round_scaled(double v, double scale)
{
    return (int32_t)rint(v * scale);  // |rint(y) - y| <= 1/2; s v is exact (s a power of two)
}

// One thread per suffix column c (suffix variable A+i is bit B-1-i of c):
// E_s[c] and the rows M_int[v][c] (eq. 8), as in the integer build but summed
// in binary64 and rounded, then offset (E_s by es_add, row v < rows by k[v]).
// Padding columns (c >= 2^B) get kPadQ and zero rows.
__global__ __launch_bounds__(256) void build_suffix_f64_kernel(const double *__restrict__ U, int ns,
                                                               int A, int B, uint64_t cols_padded,
                                                               double scale, TableOffsetsF64 off,
                                                               int32_t *__restrict__ es,
                                                               int32_t *__restrict__ mint)
{
    const uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= cols_padded)
        return;
    if (c >= (1ull << B)) {
        es[c] = kPadQ;
        for (int v = 0; v < A; ++v)
            mint[(uint64_t)v * cols_padded + c] = 0;
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
    es[c] = round_scaled(e, scale) + off.es_add;
    for (int v = 0; v < A; ++v) {
        double m = 0.0;
        for (int j = 0; j < B; ++j)
            if ((c >> (B - 1 - j)) & 1u)
                m += U[v * ns + (A + j)];
        mint[(uint64_t)v * cols_padded + c] = round_scaled(m, scale) + (v < off.rows ? off.k[v] : 0);
    }
}

// ep[j] = rint(s E_p(g(j))) over the A prefix variables, and epmin[k] = min of
// ep over body k.  Block-stride loop over 256-prefix blocks, Gray steps
// j_first <= j < j_end (j_first a multiple of 256, j_end of 32).  The 256
// prefixes of a block share the high H = A - L bits of g(j) (L = min(A, 8)), so
// with x_p split into high and low parts
//   E_p = E_hi + sum_{a in lo, x_a = 1} (K[a] + sum_{b in lo, b >= a, x_b = 1} U[a][b]),
//   K[a] = sum_{w in hi, x_w = 1} U[w][a];
// a block computes K and one row of E_hi per high variable in parallel, and
// every thread adds the rows in the same order (no floating-point atomics, so
// the table does not depend on timing).  The order differs from the
// definition's; the filter's margin covers any order.  The rounded energy is
// then lowered by es_add and by k[v] of the set variables v < rows; the body
// minima are taken relative to the body's first step as in the integer build
// (min over the body of ep + the gate offsets of its set Gray bits t < 5, less
// those at step 32k: kgate[4] for odd k).
__global__ __launch_bounds__(256) void build_prefix_f64_kernel(const double *__restrict__ U, int ns,
                                                               int A, uint64_t j_first, uint64_t j_end,
                                                               double scale, TableOffsetsF64 off,
                                                               int32_t *__restrict__ ep,
                                                               int32_t *__restrict__ epmin)
{
    __shared__ double K[8];
    __shared__ double Upp[32][32];  // the A x A prefix part of U (A <= 32)
    __shared__ double ehi_row[32];  // H = A - 8 <= 24
    __shared__ int koff[32];        // k[v] for v < rows, else 0
    const int L = A < 8 ? A : 8, H = A - L;
    const int tid = threadIdx.x;
    for (int k = tid; k < A * A; k += blockDim.x)
        Upp[k / A][k % A] = k % A >= k / A ? U[(k / A) * ns + (k % A)] : 0.0;
    if (tid < 32)
        koff[tid] = tid < off.rows ? off.k[tid] : 0;
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
        int m = INT_MAX;
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
            const uint64_t gj = gray(j);  // prefix variable v is bit A-1-v
            int koff_sum = off.es_add;
            for (int v = 0; v < A; ++v)
                koff_sum += (int)((gj >> (A - 1 - v)) & 1u) * koff[v];
            m = round_scaled(e, scale) - koff_sum;
            ep[j] = m;
#pragma unroll
            for (int t = 0; t < kU; ++t)
                m += (int)((gj >> t) & 1u) * off.kgate[t];
        }
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1)
            m = imin(m, __shfl_xor(m, o, 64));
        if (j < j_end && (j & 31) == 0)
            epmin[j >> 5] = m - (int)((j >> 5) & 1u) * off.kgate[kU - 1];
        __syncthreads();  // K and ehi_row are rewritten by the next block
    }
}

__global__ void init_ctrl_f64_kernel(CtrlF64 *ctrl, double t0, int32_t *epmin_pad, int32_t *gates_pad)
{
    epmin_pad[0] = INT_MAX;  // read ahead by the last two bodies of the walk, never used
    epmin_pad[1] = INT_MAX;
    gates_pad[0] = INT_MAX;  // group bound read ahead by the walk's last group, never used
    for (int p = 0; p < kItemParts; ++p)
        ctrl->counter[p] = 0;
    ctrl->gbest = order_key(t0);
    ctrl->slow_total = 0;
    ctrl->bodies_total = 0;
    ctrl->candidates_total = 0;
}

// ---------------------------------------------------------------------------
// The search.
// ---------------------------------------------------------------------------

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
            const uint64_t eb = f64_bits(ce);
            const uint32_t elo = __builtin_amdgcn_readlane((uint32_t)eb, l);
            const uint32_t ehi = __builtin_amdgcn_readlane((uint32_t)(eb >> 32), l);
            const uint32_t xlo = __builtin_amdgcn_readlane((uint32_t)cx, l);
            const uint32_t xhi = __builtin_amdgcn_readlane((uint32_t)(cx >> 32), l);
            insert(bits_f64(((uint64_t)ehi << 32) | elo), ((uint64_t)xhi << 32) | xlo);
        }
    }

    // k-th energy of the list (+inf until k states are in it), wave-uniform.
    __device__ __forceinline__ double kth() const
    {
        const uint64_t eb = f64_bits(e);
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)eb, k - 1);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(eb >> 32), k - 1);
        return bits_f64(((uint64_t)hi << 32) | lo);
    }
};

// The flip that leaves step m of a body (Gray bit t = ctz(m + 1)), as in the
// integer exact walk: the row by selects, the sign as an integer mask (0: add,
// -1: subtract); after the last step t = 5 and no row is chosen.
__device__ __forceinline__ void flip_after(int (&E)[kR], const int (&Mr)[kU][kR], int m, int neg_top)
{
    const int t = __builtin_ctz((unsigned)(m + 1));
    const int neg = (t < kU - 1) ? -(((m + 1) >> (t + 1)) & 1) : neg_top;
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        int d = 0;
#pragma unroll
        for (int tt = 0; tt < kU; ++tt)
            d = (tt == t) ? Mr[tt][r] : d;
        E[r] += (d ^ neg) - neg;
    }
}

// The binary64 mode of the walk (walk.h).  The integer threshold T of the walk
// is quant(t) for a binary64 bound t of the minimum (or of the k-th lowest
// energy); a body whose bound reaches T is walked exactly here, and every
// state with W <= T is re-evaluated from the definition into the thread's
// record (minimum, count, lowest index) or the wave's list.
template <bool Lowest>
struct F64Mode {
    double *rec_e;   // per-thread records in LDS
    uint64_t *rec_c, *rec_a;
    const int32_t *ep;
    const double *Q;
    CtrlF64 *ctrl;
    double scale;
    int margin, cap, n, pad, B, k_low, lane;
    uint32_t candidates;

    // floor(s t) + M, or cap when s t reaches cap (t = +inf included).
    __device__ __forceinline__ int quant(double t) const
    {
        const double y = t * scale;
        if (!(y < (double)cap))
            return cap;
        return (int)floor(y) + margin;
    }

    __device__ __forceinline__ double shared_bound() const
    {
        return uniform_f64(
            from_key(__hip_atomic_load(&ctrl->gbest, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
    }

    __device__ __forceinline__ int refresh(int T) const
    {
        const int q = quant(shared_bound());
        return q < T ? q : T;
    }

    template <int R>
    __device__ __forceinline__ void exact(int (&E)[R], const int (&Mr)[kU][R], uint64_t base,
                                          bool top_plus, int &T, uint64_t colbase, bool /*from_end*/)
    {
        static_assert(R == kR, "one instantiation");
        const int neg_top = top_plus ? 0 : -1;

        if (!Lowest) {
            // First pass: the body's smallest W, plus 2 M, bounds the W of every
            // minimiser.  It leaves E at the body's last state, which differs
            // from the first by the row of Gray bit 4 alone (the low four bits
            // return to 0), so one row takes E back.
            int wmin = INT_MAX;
#pragma unroll 1
            for (int m = 0; m < kBody; ++m) {
                wmin = imin(wmin, row_min<kR>(E) + ep[base + (uint64_t)m]);
                flip_after(E, Mr, m, neg_top);
            }
            if (top_plus)
                sub_row(E, Mr[kU - 1]);
            else
                add_row(E, Mr[kU - 1]);
            wmin = wave_min_i32(wmin);
            T = imin(T, wmin + 2 * margin);
        }
        const uint64_t pad_mask = (1ull << pad) - 1;
        if (Lowest) {
            WaveListF64 wl;
            wl.k = k_low;
            wl.lane = lane;
            wl.e = rec_e[threadIdx.x];
            wl.x = rec_a[threadIdx.x];
            // The body's 32 prefix energies in one coalesced load (lane i holds
            // step i mod 32), read per step from a lane: a scalar load per step
            // made every step wait for memory (0.3 % of this search at n = 48).
            const int ep_lanes = ep[base + (uint64_t)(threadIdx.x & (kBody - 1))];
#pragma unroll 1
            for (int m = 0; m < kBody; ++m) {
                const uint64_t j = base + (uint64_t)m;
                const int th = T - __builtin_amdgcn_readlane(ep_lanes, m);
                const uint64_t hi = (gray(j) << B) | colbase;
                uint32_t hits = 0;
#pragma unroll
                for (int r = 0; r < kR; ++r)
                    hits |= (E[r] <= th ? 1u : 0u) << r;
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
                        if ((idx & pad_mask) == 0) {
                            ++candidates;
                            real = idx >> pad;
                            v = energy_def(Q, n, real);
                            ok = true;
                        }
                    }
                    wl.insert_lanes(__builtin_amdgcn_ballot_w64(ok), v, real);
                }
                flip_after(E, Mr, m, neg_top);
            }
            rec_e[threadIdx.x] = wl.e;
            rec_a[threadIdx.x] = wl.x;
            // Offered only below the shared bound (a wave-uniform branch): the
            // waves' unconditional offers after every exact walk queued on the
            // one shared word.
            const double kt = wl.kth();
            const double gb = shared_bound();
            if (kt < gb)
                atomicMin(&ctrl->gbest, order_key(kt));
            T = imin(T, quant(gb < kt ? gb : kt));
        } else {
            // The record stays in LDS and is read and written per candidate
            // only: kept in registers across the walk, it cost the kernel a
            // wave per SIMD.
#pragma unroll 1
            for (int m = 0; m < kBody; ++m) {
                const uint64_t j = base + (uint64_t)m;
                const int th = T - ep[j];
                const uint64_t hi = (gray(j) << B) | colbase;
                uint32_t hits = 0;  // columns r whose state passes the filter
#pragma unroll
                for (int r = 0; r < kR; ++r)
                    hits |= (E[r] <= th ? 1u : 0u) << r;
                while (hits) {
                    const int r = __builtin_ctz(hits);
                    hits &= hits - 1;
                    const uint64_t idx = hi | ((uint64_t)r << 6) | (uint64_t)lane;
                    if ((idx & pad_mask) == 0) {
                        ++candidates;
                        const uint64_t real = idx >> pad;
                        const double v = energy_def(Q, n, real);
                        const double re = rec_e[threadIdx.x];
                        if (v < re) {
                            rec_e[threadIdx.x] = v;
                            rec_c[threadIdx.x] = 1;
                            rec_a[threadIdx.x] = real;
                        } else if (v == re) {
                            rec_c[threadIdx.x] += 1;
                            const uint64_t ra = rec_a[threadIdx.x];
                            rec_a[threadIdx.x] = real < ra ? real : ra;
                        }
                    }
                }
                flip_after(E, Mr, m, neg_top);
            }
            const double wm = wave_min_f64(rec_e[threadIdx.x]);
            const double gb = shared_bound();
            if (wm < gb)
                atomicMin(&ctrl->gbest, order_key(wm));
            T = imin(T, quant(gb < wm ? gb : wm));
        }
    }
};

// The search kernel: the integer walk of walk.h over the rounded tables with
// the binary64 mode, then the lanes' records reduced into one partial result
// per workgroup.  Lowest: keep each wave's k lowest states (args.lists)
// instead of the minimum, its count and lowest minimiser; the threshold is then
// the k-th energy, and the first pass of an exact walk (which bounds only the
// minimum) is skipped.  Six waves per SIMD (80 VGPRs), as for the integer
// search: the compiler then moves a few values of a unit's set-up to scratch,
// outside the body loop.
template <bool Lowest>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6))) void gray_search_f64_kernel(const int32_t *__restrict__ es,
                                                              const int32_t *__restrict__ mint,
                                                              const int32_t *__restrict__ ep,
                                                              const int32_t *__restrict__ epmin,
                                                              const int32_t *__restrict__ gates,
                                                              const double *__restrict__ Q,
                                                              PartialF64 *__restrict__ partials,
                                                              CtrlF64 *__restrict__ ctrl,
                                                              const SearchArgsF64 a)
{
    extern __shared__ int32_t lds_rows[];  // [l_eff - kU][64 kR]
    __shared__ unsigned long long item_sh[4];
    __shared__ double rec_e[64 * kWaves];
    __shared__ uint64_t rec_c[64 * kWaves], rec_a[64 * kWaves];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    rec_e[threadIdx.x] = __longlong_as_double(0x7ff0000000000000LL);  // each thread owns its slot
    rec_c[threadIdx.x] = 0;
    rec_a[threadIdx.x] = ~0ull;

    F64Mode<Lowest> mode{rec_e, rec_c, rec_a, ep, Q, ctrl, a.scale, a.margin, a.cap, a.n, a.pad, a.B,
                         a.k_low, lane, 0u};
    int T = mode.refresh(INT_MAX);
    uint32_t bodies = 0, checked = 0, slow = 0;
    walk_units<kR, true>(a, ctrl, es, mint, ep, epmin, gates, lds_rows, item_sh, mode, T, bodies, checked, slow);

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
    const uint64_t cand = wave_sum(mode.candidates);
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
                                   double scale, const TableOffsetsF64 &off, int32_t *es, int32_t *mint,
                                   int32_t *ep, int32_t *epmin, uint64_t j_lo, uint64_t j_hi,
                                   hipStream_t stream)
{
    if (off.rows < 0 || off.rows > A || A > 32)
        return hipErrorInvalidValue;
    const unsigned g1 = (unsigned)((cols_padded + 255) / 256);
    hipLaunchKernelGGL(build_suffix_f64_kernel, dim3(g1), dim3(256), 0, stream, U, ns, A, B,
                       cols_padded, scale, off, es, mint);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    if (A < kU || A > 32 || j_lo >= j_hi || j_hi > (1ull << A) || (j_lo & 31) || (j_hi & 31))
        return hipErrorInvalidValue;  // (the builder stages at most 32 x 32 entries of U)
    const uint64_t j_first = j_lo & ~uint64_t(255);
    const uint64_t blocks = (j_hi - j_first + 255) / 256;
    const uint64_t grid = blocks < (1ull << 14) ? blocks : (1ull << 14);
    hipLaunchKernelGGL(build_prefix_f64_kernel, dim3((unsigned)grid), dim3(256), 0, stream, U, ns,
                       A, j_first, j_hi, scale, off, ep, epmin);
    return hipGetLastError();
}

hipError_t launch_init_ctrl_f64(CtrlF64 *ctrl, double t0, int32_t *epmin_pad, int32_t *gates_pad,
                                hipStream_t stream)
{
    hipLaunchKernelGGL(init_ctrl_f64_kernel, dim3(1), dim3(1), 0, stream, ctrl, t0, epmin_pad, gates_pad);
    return hipGetLastError();
}

hipError_t launch_search_f64(const SearchArgsF64 &args, bool lowest, int blocks, int lds_bytes,
                             hipStream_t stream)
{
    if (lowest && (args.k_low < 1 || args.k_low > 64 || !args.lists))
        return hipErrorInvalidValue;
    if (lowest)
        hipLaunchKernelGGL(gray_search_f64_kernel<true>, dim3(blocks), dim3(64 * kWaves), lds_bytes,
                           stream, args.es, args.mint, args.ep, args.epmin, args.gates, args.Q, args.partials,
                           args.ctrl, args);
    else
        hipLaunchKernelGGL(gray_search_f64_kernel<false>, dim3(blocks), dim3(64 * kWaves), lds_bytes,
                           stream, args.es, args.mint, args.ep, args.epmin, args.gates, args.Q, args.partials,
                           args.ctrl, args);
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
