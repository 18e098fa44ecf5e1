// C-ABI entry points of the QUBO search (declared in include/qubo.h): argument
// checks and the requests they build; the runs are in run_int.hip,
// run_f64.hip and run_steps.hip.
#include "host.h"

#include <algorithm>

using namespace qubo_host;

static_assert(sizeof(qubo::LowEntry) == sizeof(qubo_state), "list entry layout");
static_assert(sizeof(qubo_progress) == 96, "the run state is a fixed 96-byte record");
static_assert(sizeof(qubo_progress_lowest) == 96 + 8 + QUBO_MAX_LOWEST * 16, "the spectrum run state is a fixed record");

extern "C" {

QUBO_API int qubo_make_plan(int n, int prefix_bits, int cache_bits, qubo_plan *out)
{
    // Host-only planning for a 256-CU MI355X.
    return qubo::make_plan(n, prefix_bits, cache_bits, 256, 0, -1, out);
}

QUBO_API int qubo_check_q(const int32_t *Q_host, int n)
{
    if (!Q_host || n < 1 || n > QUBO_MAX_N)
        return QUBO_EINVAL;
    std::vector<int32_t> U;
    return qubo::fold_upper(Q_host, n, U, nullptr);
}

QUBO_API int qubo_abs_sum(const int32_t *Q_host, int n, int64_t *abs_sum)
{
    if (!Q_host || !abs_sum || n < 1 || n > QUBO_MAX_N)
        return QUBO_EINVAL;
    int64_t s = 0;
    for (size_t i = 0; i < (size_t)n * n; ++i)
        s += Q_host[i] < 0 ? -(int64_t)Q_host[i] : (int64_t)Q_host[i];
    *abs_sum = s;
    return QUBO_OK;
}

QUBO_API int qubo_check_q_f64(const double *Q_host, int n)
{
    if (!Q_host || n < 1 || n > QUBO_MAX_N)
        return QUBO_EINVAL;
    const std::vector<double> Qh(Q_host, Q_host + (size_t)n * n);
    double S = 0.0;
    return guard_f64(Qh, &S);
}

QUBO_API int qubo_f64_as_int32(const double *Q_host, int n, int32_t *Q_int, int *f)
{
    if (!Q_host || !Q_int || !f || n < 1 || n > QUBO_MAX_N)
        return QUBO_EINVAL;
    const std::vector<double> Qh(Q_host, Q_host + (size_t)n * n);
    std::vector<int32_t> Qi;
    int fe = 0;
    if (!dyadic_int32(Qh, Qi, &fe))
        return QUBO_ERANGE;
    std::copy(Qi.begin(), Qi.end(), Q_int);
    *f = fe;
    return QUBO_OK;
}

QUBO_API int qubo_search(const int32_t *Q, int n, int prefix_bits, int cache_bits, void *stream,
                qubo_result *out)
{
    Request rq;
    rq.Q = Q;
    rq.n = n;
    rq.prefix_bits = prefix_bits;
    rq.cache_bits = cache_bits;
    rq.stream = static_cast<hipStream_t>(stream);
    return run(rq, out);
}

QUBO_API int qubo_search_ex(const int32_t *Q, int n, int prefix_bits, int cache_bits, uint64_t gray_lo,
                           uint64_t gray_hi, uint32_t flags, void *stream, qubo_result *out)
{
    const uint32_t known =
        QUBO_FLAG_STRICT_MIN | QUBO_FLAG_COLS8 | QUBO_FLAG_COLS16 | QUBO_FLAG_SPLIT_MASK;
    if ((flags & ~known) || ((flags & QUBO_FLAG_COLS8) && (flags & QUBO_FLAG_COLS16)))
        return QUBO_EINVAL;
    Request rq;
    rq.Q = Q;
    rq.n = n;
    rq.prefix_bits = prefix_bits;
    rq.cache_bits = cache_bits;
    rq.gated = !(flags & QUBO_FLAG_STRICT_MIN);
    rq.cols_per_lane = (flags & QUBO_FLAG_COLS8) ? 8 : (flags & QUBO_FLAG_COLS16) ? 16 : 0;
    rq.split_bits = (int)((flags & QUBO_FLAG_SPLIT_MASK) >> QUBO_FLAG_SPLIT_SHIFT);
    rq.stream = static_cast<hipStream_t>(stream);
    if (gray_lo != 0 || gray_hi != 0) {
        if (!valid_slice(n, prefix_bits, gray_lo, gray_hi))
            return QUBO_EINVAL;
        rq.ranged = true;
        rq.gray_lo = gray_lo;
        rq.gray_hi = gray_hi;
    }
    return run(rq, out);
}

QUBO_API int qubo_search_lowest(const int32_t *Q, int n, int k, int prefix_bits, int cache_bits,
                                uint64_t gray_lo, uint64_t gray_hi, uint32_t flags, void *stream,
                                qubo_state *out, int *found)
{
    const uint32_t known = QUBO_FLAG_COLS8 | QUBO_FLAG_COLS16 | QUBO_FLAG_SPLIT_MASK;
    if ((flags & ~known) || ((flags & QUBO_FLAG_COLS8) && (flags & QUBO_FLAG_COLS16)))
        return QUBO_EINVAL;
    if (!out || !found || k < 1 || k > QUBO_MAX_LOWEST)
        return QUBO_EINVAL;
    Request rq;
    rq.Q = Q;
    rq.n = n;
    rq.prefix_bits = prefix_bits;
    rq.cache_bits = cache_bits;
    rq.cols_per_lane = (flags & QUBO_FLAG_COLS8) ? 8 : (flags & QUBO_FLAG_COLS16) ? 16 : 0;
    rq.split_bits = (int)((flags & QUBO_FLAG_SPLIT_MASK) >> QUBO_FLAG_SPLIT_SHIFT);
    rq.lowest_k = k;
    rq.stream = static_cast<hipStream_t>(stream);
    if (gray_lo != 0 || gray_hi != 0) {
        if (!valid_slice(n, prefix_bits, gray_lo, gray_hi))
            return QUBO_EINVAL;
        rq.ranged = true;
        rq.gray_lo = gray_lo;
        rq.gray_hi = gray_hi;
    }
    return run(rq, nullptr, out, found);
}

QUBO_API int qubo_search_range(const int32_t *Q, int n, int prefix_bits, int cache_bits, uint64_t gray_lo,
                      uint64_t gray_hi, void *stream, qubo_result *out)
{
    if (gray_lo == 0 && gray_hi == 0)
        return QUBO_EINVAL;
    return qubo_search_ex(Q, n, prefix_bits, cache_bits, gray_lo, gray_hi, 0u, stream, out);
}

QUBO_API int qubo_progress_init(const int32_t *Q, int n, int prefix_bits, int chunk_bits, uint32_t flags,
                                void *stream, qubo_progress *p)
{
    return init_progress(Q, n, prefix_bits, chunk_bits, flags, stream, 0, p);
}

QUBO_API int qubo_progress_init_lowest(const int32_t *Q, int n, int k, int prefix_bits, int chunk_bits,
                                       uint32_t flags, void *stream, qubo_progress_lowest *p)
{
    if (!p || k < 1 || k > QUBO_MAX_LOWEST)
        return QUBO_EINVAL;
    qubo_progress head;
    const int rc = init_progress(Q, n, prefix_bits, chunk_bits, flags, stream, 2, &head);
    if (rc != QUBO_OK)
        return rc;
    qubo_progress_lowest q{};
    q.head = head;
    q.k = k;
    *p = q;
    return QUBO_OK;
}

QUBO_API int qubo_search_step_lowest(const int32_t *Q, int n, void *stream, qubo_progress_lowest *p)
{
    if (!Q || !p || n < 1 || n > QUBO_MAX_N || p->head.n != n || p->head.kind != 2)
        return QUBO_EINVAL;
    if (p->head.done)
        return QUBO_OK;
    return run_step_lowest(Q, n, static_cast<hipStream_t>(stream), *p, p);
}

QUBO_API int qubo_search_step(const int32_t *Q, int n, void *stream, qubo_progress *p)
{
    if (!Q || !p || n < 1 || n > QUBO_MAX_N || p->n != n || p->kind != 0)
        return QUBO_EINVAL;
    if (p->done)
        return QUBO_OK;
    return run_step(Q, n, static_cast<hipStream_t>(stream), *p, p);
}

QUBO_API int qubo_progress_init_f64(const double *Q, int n, int prefix_bits, int chunk_bits, void *stream,
                                    qubo_progress *p)
{
    using namespace qubo;
    if (!Q || !p || n < kMinSearchVars || n > kMaxSingleVars)
        return QUBO_EINVAL;
    qubo_plan plan;
    int rc = make_plan(n, prefix_bits, -1, 256, 8, 0, &plan);
    if (rc != QUBO_OK)
        return rc;
    const int A = plan.prefix_bits, B = plan.suffix_bits;
    if (chunk_bits < 0)
        chunk_bits = std::max(kRegBits, std::min(A, 48 - B));  // about 2^48 states per step
    if (chunk_bits < kRegBits || chunk_bits > A)
        return QUBO_EINVAL;
    DeviceInfo dev;
    rc = device_info(&dev);
    if (rc != QUBO_OK)
        return rc;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    std::vector<double> Qh((size_t)n * n);
    if (hipMemcpyAsync(Qh.data(), Q, Qh.size() * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return QUBO_EDEVICE;
    double S = 0.0;
    rc = guard_f64(Qh, &S);
    if (rc != QUBO_OK)
        return rc;
    qubo_progress q{};
    q.q_hash = fingerprint(Qh.data(), Qh.size() * 8, n);
    q.n = n;
    q.prefix_bits = A;
    q.chunk_bits = chunk_bits;
    q.steps_total = 1ull << (A - chunk_bits);
    q.kind = 1;
    *p = q;
    return QUBO_OK;
}

QUBO_API int qubo_search_step_f64(const double *Q, int n, void *stream, qubo_progress *p)
{
    if (!Q || !p || n < 1 || n > QUBO_MAX_N || p->n != n || p->kind != 1)
        return QUBO_EINVAL;
    if (p->done)
        return QUBO_OK;
    return run_step_f64(Q, n, static_cast<hipStream_t>(stream), *p, p);
}

QUBO_API int qubo_search_lowest_f64(const double *Q, int n, int k, int prefix_bits, int cache_bits,
                                    uint64_t gray_lo, uint64_t gray_hi, uint32_t flags, void *stream,
                                    qubo_state_f64 *out, int *found)
{
    if ((flags & ~QUBO_FLAG_COLS8) || !out || !found || k < 1 || k > QUBO_MAX_LOWEST)
        return QUBO_EINVAL;
    RequestF64 rq;
    rq.Q = Q;
    rq.n = n;
    rq.prefix_bits = prefix_bits;
    rq.cache_bits = cache_bits;
    rq.stream = static_cast<hipStream_t>(stream);
    rq.lowest_k = k;
    if (gray_lo != 0 || gray_hi != 0) {
        if (!valid_slice(n, prefix_bits, gray_lo, gray_hi))
            return QUBO_EINVAL;
        rq.ranged = true;
        rq.gray_lo = gray_lo;
        rq.gray_hi = gray_hi;
    }
    std::vector<qubo_state_f64> low;
    const int rc = run_f64(rq, nullptr, false, 0.0, nullptr, &low);
    if (rc != QUBO_OK)
        return rc;
    std::copy(low.begin(), low.end(), out);
    *found = (int)low.size();
    return QUBO_OK;
}

QUBO_API int qubo_search_f64(const double *Q, int n, int prefix_bits, int cache_bits,
                             uint64_t gray_lo, uint64_t gray_hi, uint32_t flags, void *stream,
                             qubo_result_f64 *out)
{
    if (flags & ~QUBO_FLAG_COLS8)
        return QUBO_EINVAL;
    RequestF64 rq;
    rq.Q = Q;
    rq.n = n;
    rq.prefix_bits = prefix_bits;
    rq.cache_bits = cache_bits;
    rq.stream = static_cast<hipStream_t>(stream);
    if (gray_lo != 0 || gray_hi != 0) {
        if (!valid_slice(n, prefix_bits, gray_lo, gray_hi))
            return QUBO_EINVAL;
        rq.ranged = true;
        rq.gray_lo = gray_lo;
        rq.gray_hi = gray_hi;
    }
    return run_f64(rq, out);
}

QUBO_API int qubo_build_tables(const int32_t *Q, int n, int prefix_bits, int32_t *Es, int32_t *Mint,
                      int32_t *EpGray, void *stream)
{
    if (!Es || !Mint || !EpGray)
        return QUBO_EINVAL;
    if (n < qubo::kMinSearchVars || prefix_bits < qubo::kRegBits || prefix_bits > n)
        return QUBO_EINVAL;
    Request rq;
    rq.Q = Q;
    rq.n = n;
    rq.prefix_bits = prefix_bits;
    rq.stream = static_cast<hipStream_t>(stream);
    rq.mode = Mode::Build;
    rq.es_out = Es;
    rq.mint_out = Mint;
    rq.ep_out = EpGray;
    return run(rq, nullptr);
}

QUBO_API int qubo_last_timing(qubo_timing *out)
{
    if (!out)
        return QUBO_EINVAL;
    *out = last_timing();
    return QUBO_OK;
}

QUBO_API const char *qubo_strerror(int status)
{
    switch (status) {
    case QUBO_OK:
        return "ok";
    case QUBO_EINVAL:
        return "invalid argument";
    case QUBO_ERANGE:
        return "Q out of range (int32: sum of |Q_ij| above 2^30-1; binary64: an entry not finite, "
               "or sum of |Q_ij| above 2^100 or in (0, 2^-100))";
    case QUBO_EPLAN:
        return "split does not fit the kernel (prefix/cache bits out of the supported range)";
    case QUBO_EDEVICE:
        return "no usable gfx950 device or HIP runtime error";
    case QUBO_ENOMEM:
        return "out of device memory";
    case QUBO_ESCRATCH:
        return "the search's workspace exceeds the static buffer of qubo_search_noalloc (128 MiB)";
    default:
        return "unknown status";
    }
}

QUBO_API const char *qubo_version(void)
{
    return "qubo-mi355x 0.6 (gfx950; int32 minimum and k-lowest, 8 or 16 columns/lane; binary64 on rounded int32 tables; runs in steps)";
}

}  // extern "C"
