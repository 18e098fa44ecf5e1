// Shared host helpers of the C-ABI: device check, copies, fingerprints, the
// binary64 guard and the int32 form of dyadic binary64 matrices, list merging
// and slice checks.
#include "host.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <iterator>

namespace qubo_host {

qubo_timing &last_timing()
{
    thread_local qubo_timing t{};
    return t;
}

int device_info(DeviceInfo *info)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return QUBO_EDEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return QUBO_EDEVICE;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return QUBO_EDEVICE;
    info->num_cus = prop.multiProcessorCount;
    return QUBO_OK;
}

// Copies Q (n x n int32, device) to the host.
int read_q(const int32_t *Q, int n, hipStream_t stream, std::vector<int32_t> &Qh)
{
    Qh.resize((size_t)n * n);
    if (hipMemcpyAsync(Qh.data(), Q, Qh.size() * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return QUBO_EDEVICE;
    return QUBO_OK;
}

// FNV-1a (64 bit) over n (4 little-endian bytes) and the bytes of Q's entries.
uint64_t fingerprint(const void *Qh, size_t bytes, int n)
{
    uint64_t h = 0xcbf29ce484222325ull;
    auto mix = [&h](uint8_t b) {
        h ^= b;
        h *= 0x100000001b3ull;
    };
    for (int b = 0; b < 4; ++b)
        mix((uint8_t)((uint32_t)n >> (8 * b)));
    const uint8_t *q = static_cast<const uint8_t *>(Qh);
    for (size_t i = 0; i < bytes; ++i)
        mix(q[i]);
    return h;
}

// The binary64 guard: finite entries and S = sum |Q_ij| (rounded up) either 0
// or in [2^-100, 2^100].  The walk of the binary64 search runs on its tables
// scaled by s = 2^(17 - e) with S < 2^e and rounded to integers; the range
// keeps s, s S and every binary64 sum of the tables and of the definition well
// inside binary64's normal range (where each rounding errs by at most 2^-53 of
// its result), with room at both ends.  S = 0 means every entry is zero.
int guard_f64(const std::vector<double> &Qh, double *S_out)
{
    double S = 0.0;
    for (double v : Qh) {
        if (!std::isfinite(v))
            return QUBO_ERANGE;
        S += std::fabs(v);
    }
    S *= 1.0 + 0x1p-40;  // rounding of the sum itself (at most n^2 ulp)
    if (!(S <= 0x1p100) || (S > 0.0 && S < 0x1p-100))
        return QUBO_ERANGE;
    *S_out = S;
    return QUBO_OK;
}

// A dyadic matrix: every entry an integer multiple of 2^-f with
// sum |2^f Q_ij| <= 2^30 - 1.  Then every partial sum of the definition is a
// multiple of 2^-f below 2^(30 - f) in magnitude, i.e. at most 30 significant
// bits, so binary64 adds it exactly, in any order: E(x) = E_int(x) / 2^f with
// E_int the energy of the int32 matrix 2^f Q, whose search is exact, ties and
// counts included.  Writes that matrix and f; false when Q is not such a matrix.
bool dyadic_int32(const std::vector<double> &Qh, std::vector<int32_t> &Qi, int *f_out)
{
    // f = -(the lowest exponent of any entry's last set bit)
    int f = INT_MIN;
    for (double v : Qh) {
        if (!std::isfinite(v))
            return false;
        if (v == 0.0)
            continue;
        int ex = 0;
        const double m = std::frexp(std::fabs(v), &ex);      // |v| = m 2^ex, m in [0.5, 1)
        const uint64_t M = (uint64_t)std::ldexp(m, 53);       // 53-bit integer significand
        const int lsb = ex - 53 + __builtin_ctzll(M);         // |v| = odd * 2^lsb
        f = std::max(f, -lsb);
    }
    if (f == INT_MIN)
        f = 0;  // the zero matrix
    Qi.resize(Qh.size());
    int64_t sum = 0;
    for (size_t k = 0; k < Qh.size(); ++k) {
        const double q = std::ldexp(Qh[k], f);  // exact: a power-of-two scale of an integer multiple
        if (!(std::fabs(q) <= (double)qubo::kAbsSumLimit))
            return false;
        Qi[k] = (int32_t)q;
        sum += std::llabs((long long)Qi[k]);
        if (sum > qubo::kAbsSumLimit)
            return false;
    }
    *f_out = f;
    return true;
}

// Keeps the k first states of `acc` merged with `add`, in (energy, index) order.
void merge_lowest(std::vector<qubo_state> &acc, const std::vector<qubo_state> &add, int k)
{
    std::vector<qubo_state> m;
    m.reserve(acc.size() + add.size());
    std::merge(acc.begin(), acc.end(), add.begin(), add.end(), std::back_inserter(m),
               [](const qubo_state &a, const qubo_state &b) {
                   return a.energy < b.energy || (a.energy == b.energy && a.index < b.index);
               });
    if ((int)m.size() > k)
        m.resize((size_t)k);
    acc.swap(m);
}

void add_timing(qubo_timing &acc, const qubo_timing &t)
{
    acc.build_ms += t.build_ms;
    acc.search_ms += t.search_ms;
    acc.reduce_ms += t.reduce_ms;
    acc.total_ms += t.total_ms;
    acc.states += t.states;
    acc.blocks = t.blocks;
    if (t.cols_per_lane != 0)  // (a skipped sub-problem launched nothing)
        acc.cols_per_lane = t.cols_per_lane;
    acc.bodies += t.bodies;
    acc.checked_bodies += t.checked_bodies;
    acc.slow_bodies += t.slow_bodies;
}

// A slice [gray_lo, gray_hi) of the Gray walk over an explicit prefix size:
// whole 32-step bodies, non-empty, inside the 2^prefix_bits steps.
bool valid_slice(int n, int prefix_bits, uint64_t gray_lo, uint64_t gray_hi)
{
    if (n < qubo::kMinSearchVars || prefix_bits < qubo::kRegBits || prefix_bits > n ||
        prefix_bits > qubo::kMaxPrefixBits)
        return false;
    return !(gray_lo & 31u) && !(gray_hi & 31u) && gray_lo < gray_hi &&
           gray_hi <= (1ull << prefix_bits);
}

}  // namespace qubo_host
