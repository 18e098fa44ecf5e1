// C-ABI entry points of the QUBO search (declared in include/qubo.h).
//
// Orchestration of one search (Maltsev et al., "Terastate-per-second QUBO
// Brute-Force on a Single GPU", sec. III, Algorithms 1-2 and sec. III.C):
//   1. copy Q (n x n int32, at most 16 KiB) to the host, fold it into the upper
//      triangle and check the overflow guard;
//   2. plan the split (prefix A, suffix B, cached Gray bits, work units);
//   3. one stream-ordered allocation for U, E_s, M_int, the Gray-ordered E_p,
//      the per-wave partial results and a control block;
//   4. cache builders, search kernel, final reduction, 64-byte result download;
//   5. free and synchronise the stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstring>
#include <iterator>
#include <vector>

#include <cmath>

#include "kernels.h"
#include "kernels_f64.h"
#include "plan.h"
#include "qubo.h"

namespace {

thread_local qubo_timing g_timing{};

struct DeviceInfo {
    int num_cus = 0;
};

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

// The binary64 guard: finite entries and S = sum |Q_ij| (rounded up) <= 2^100.
int guard_f64(const std::vector<double> &Qh, double *S_out)
{
    double S = 0.0;
    for (double v : Qh) {
        if (!std::isfinite(v))
            return QUBO_ERANGE;
        S += std::fabs(v);
    }
    S *= 1.0 + 0x1p-40;  // rounding of the sum itself (at most n^2 ulp)
    if (!(S <= 0x1p100))
        return QUBO_ERANGE;
    *S_out = S;
    return QUBO_OK;
}

// Everything one call owns; released in the destructor on every path.
struct Call {
    hipStream_t stream = nullptr;
    void *ws = nullptr;
    hipEvent_t ev[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};

    // Every event that was created is destroyed, also after a partial failure.
    bool create_events()
    {
        for (auto &e : ev) {
            hipEvent_t tmp = nullptr;
            if (hipEventCreate(&tmp) != hipSuccess)
                return false;
            e = tmp;
        }
        return true;
    }

    ~Call()
    {
        if (ws) {
            (void)hipFreeAsync(ws, stream);
            (void)hipStreamSynchronize(stream);
        }
        for (auto &e : ev)
            if (e)
                (void)hipEventDestroy(e);
    }
};

enum class Mode { Search, Build };

struct Request {
    const int32_t *Q = nullptr;
    int n = 0;
    int prefix_bits = -1;
    int cache_bits = -1;
    bool ranged = false;
    uint64_t gray_lo = 0, gray_hi = 0;
    hipStream_t stream = nullptr;
    Mode mode = Mode::Search;
    bool gated = true;
    int cols_per_lane = 0;  // 0: planner's default
    int split_bits = 0;     // 0: automatic (only above the single-launch limit)
    int lowest_k = 0;       // > 0: the spectrum search (the lowest_k lowest states)
    int32_t *es_out = nullptr, *mint_out = nullptr, *ep_out = nullptr;
};

static_assert(sizeof(qubo::LowEntry) == sizeof(qubo_state), "list entry layout");
static_assert(sizeof(qubo_progress) == 96, "the run state is a fixed 96-byte record");
static_assert(sizeof(qubo_progress_lowest) == 96 + 8 + QUBO_MAX_LOWEST * 16, "the spectrum run state is a fixed record");

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
    acc.bodies += t.bodies;
    acc.checked_bodies += t.checked_bodies;
    acc.slow_bodies += t.slow_bodies;
}

// One search of the folded upper-triangular matrix U (n x n, host memory) on the
// device.  have_t0: the search only has to find states with E <= t0_cap (the
// caller knows a real energy that low elsewhere, or k of them for the
// spectrum); then an empty result is valid and *found reports whether any
// state was recorded.  The spectrum search (rq.lowest_k > 0) writes its states
// to *low, in order, and leaves *out alone.
int run_one(const Request &rq, const DeviceInfo &dev, std::vector<int32_t> U, int n, int64_t abs_sum,
            bool have_t0, int32_t t0_cap, qubo_result *out, bool *found, qubo_timing *timing,
            std::vector<qubo_state> *low = nullptr)
{
    using namespace qubo;
    Call call;
    call.stream = rq.stream;

    // Plan.
    qubo_plan plan;
    int rc = make_plan(n, rq.prefix_bits, rq.cache_bits, dev.num_cus, rq.cols_per_lane, 0, &plan);
    if (rc != QUBO_OK)
        return rc;
    const int ns = plan.n_search;
    if (ns != n)
        U = pad_upper(U, n, ns);
    const int A = plan.prefix_bits, B = plan.suffix_bits;
    const bool lowest = rq.lowest_k > 0;
    // With padding variables (n < 5, so 2^ns = 32 states) the list keeps every
    // state; the padded ones are dropped afterwards.
    const int k_low = !lowest ? 0 : (ns != n ? (1 << ns) : rq.lowest_k);
    if (lowest && (k_low < 1 || k_low > kMaxLowest))
        return QUBO_EINVAL;

    // Work range in Gray steps and its segments.
    uint64_t lo = 0, hi = 1ull << A;
    if (rq.ranged) {
        lo = rq.gray_lo;
        hi = rq.gray_hi;
        if (hi > (1ull << A))
            return QUBO_EINVAL;
    }
    const uint64_t seg_first = lo >> plan.seg_bits;
    const uint64_t seg_last = (hi - 1) >> plan.seg_bits;
    const uint64_t segs = seg_last - seg_first + 1;
    const uint64_t seg_blocks = (segs + kWavesPerBlock - 1) / kWavesPerBlock;
    const uint64_t items = plan.col_groups * seg_blocks;

    int per_cu = 0;
    if (search_occupancy(plan.cols_per_lane, rq.gated, lowest, &per_cu, plan.lds_bytes) !=
        hipSuccess)
        return QUBO_EDEVICE;
    if (per_cu < 1)
        per_cu = 1;
    const uint64_t want_blocks = (uint64_t)dev.num_cus * (uint64_t)per_cu;
    plan.blocks = (int)(items < want_blocks ? items : want_blocks);
    const Layout L = layout_of(plan);
    // The spectrum search appends the per-wave lists, the merged list and its size.
    const uint64_t list_entries = lowest ? (uint64_t)plan.blocks * plan.waves_per_block * k_low : 0;
    const uint64_t off_lists = (L.total + 255) & ~uint64_t(255);
    const uint64_t off_low_out = off_lists + ((list_entries * sizeof(LowEntry) + 255) & ~uint64_t(255));
    const uint64_t off_low_found = off_low_out + kMaxLowest * sizeof(LowEntry);
    const uint64_t ws_total = lowest ? off_low_found + 256 : L.total;

    // Workspace.
    if (hipMallocAsync(&call.ws, ws_total, rq.stream) != hipSuccess) {
        call.ws = nullptr;
        return QUBO_ENOMEM;
    }
    char *base = static_cast<char *>(call.ws);
    int32_t *dU = reinterpret_cast<int32_t *>(base + L.off_u);
    int32_t *des = reinterpret_cast<int32_t *>(base + L.off_es);
    int32_t *dmint = reinterpret_cast<int32_t *>(base + L.off_mint);
    int32_t *dep = reinterpret_cast<int32_t *>(base + L.off_ep);
    int32_t *depmin = reinterpret_cast<int32_t *>(base + L.off_epmin);
    Partial *dpart = reinterpret_cast<Partial *>(base + L.off_partials);
    Ctrl *dctrl = reinterpret_cast<Ctrl *>(base + L.off_ctrl);

    if (!call.create_events())
        return QUBO_EDEVICE;

    // Upload, build, search, reduce.
    if (hipEventRecord(call.ev[0], rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    if (hipMemcpyAsync(dU, U.data(), U.size() * 4, hipMemcpyHostToDevice, rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    if (launch_build_tables(dU, ns, A, B, L.cols_padded, des, dmint, dep, depmin, lo, hi, rq.stream) !=
        hipSuccess)
        return QUBO_EDEVICE;
    if (hipEventRecord(call.ev[1], rq.stream) != hipSuccess)
        return QUBO_EDEVICE;

    if (rq.mode == Mode::Build) {
        const uint64_t cols = 1ull << B;
        if (hipMemcpyAsync(rq.es_out, des, cols * 4, hipMemcpyDeviceToDevice, rq.stream) !=
                hipSuccess ||
            hipMemcpy2DAsync(rq.mint_out, cols * 4, dmint, L.cols_padded * 4, cols * 4, (size_t)A,
                             hipMemcpyDeviceToDevice, rq.stream) != hipSuccess ||
            hipMemcpyAsync(rq.ep_out, dep, (1ull << A) * 4, hipMemcpyDeviceToDevice, rq.stream) !=
                hipSuccess)
            return QUBO_EDEVICE;
        if (hipStreamSynchronize(rq.stream) != hipSuccess)
            return QUBO_EDEVICE;
        return QUBO_OK;
    }

    // The first threshold must be a real energy of the searched set or an upper
    // bound of all of them: E(0) = 0 when state 0 is searched, else sum |Q_ij|
    // (always sum |Q_ij| for the spectrum, whose threshold bounds the k-th
    // energy).  A caller's cap (an energy found elsewhere) may only lower it; it
    // is never below -sum |U_ij| here, so every threshold stays within
    // +-2 sum |U_ij|.
    int32_t t0 = (lo == 0 && !lowest) ? 0 : (int32_t)abs_sum;
    if (have_t0 && t0_cap < t0)
        t0 = t0_cap;
    if (launch_init_ctrl(dctrl, t0, depmin + (1ull << (A - kRegBits)), rq.stream) != hipSuccess)
        return QUBO_EDEVICE;

    SearchArgs sa{};
    sa.es = des;
    sa.mint = dmint;
    sa.ep = dep;
    sa.epmin = depmin;
    sa.partials = dpart;
    sa.ctrl = dctrl;
    sa.cols_padded = L.cols_padded;
    sa.gray_lo = lo;
    sa.gray_hi = hi;
    sa.seg_first = seg_first;
    sa.segs = segs;
    sa.seg_blocks = seg_blocks;
    sa.items = items;
    sa.A = A;
    sa.B = B;
    sa.l_eff = plan.cache_bits < plan.seg_bits ? plan.cache_bits : plan.seg_bits;
    sa.seg_bits = plan.seg_bits;
    LowEntry *dlists = reinterpret_cast<LowEntry *>(base + off_lists);
    LowEntry *dlow = reinterpret_cast<LowEntry *>(base + off_low_out);
    int32_t *dlow_found = reinterpret_cast<int32_t *>(base + off_low_found);
    if (lowest) {
        sa.lists = dlists;
        sa.k_low = k_low;
    }
    if (launch_search(sa, plan.cols_per_lane, rq.gated, lowest, plan.blocks, plan.lds_bytes,
                      rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    if (hipEventRecord(call.ev[2], rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    if (launch_reduce(dpart, plan.blocks * plan.waves_per_block, dctrl, rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    if (lowest && launch_lowest_merge(dlists, list_entries, k_low, dlow, dlow_found, rq.stream) !=
                      hipSuccess)
        return QUBO_EDEVICE;
    if (hipEventRecord(call.ev[3], rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    Ctrl host_ctrl;
    LowEntry host_low[kMaxLowest];
    int32_t host_low_found = 0;
    if (hipMemcpyAsync(&host_ctrl, dctrl, sizeof(Ctrl), hipMemcpyDeviceToHost, rq.stream) !=
        hipSuccess)
        return QUBO_EDEVICE;
    if (lowest &&
        (hipMemcpyAsync(host_low, dlow, sizeof(host_low), hipMemcpyDeviceToHost, rq.stream) !=
             hipSuccess ||
         hipMemcpyAsync(&host_low_found, dlow_found, sizeof(int32_t), hipMemcpyDeviceToHost,
                        rq.stream) != hipSuccess))
        return QUBO_EDEVICE;
    if (hipEventRecord(call.ev[4], rq.stream) != hipSuccess ||
        hipStreamSynchronize(rq.stream) != hipSuccess)
        return QUBO_EDEVICE;

    qubo_timing t{};
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, call.ev[0], call.ev[1]) == hipSuccess)
        t.build_ms = ms;
    if (hipEventElapsedTime(&ms, call.ev[1], call.ev[2]) == hipSuccess)
        t.search_ms = ms;
    if (hipEventElapsedTime(&ms, call.ev[2], call.ev[3]) == hipSuccess)
        t.reduce_ms = ms;
    if (hipEventElapsedTime(&ms, call.ev[0], call.ev[4]) == hipSuccess)
        t.total_ms = ms;
    t.states = (hi - lo) << B;
    t.slow_bodies = host_ctrl.slow_total;
    t.bodies = host_ctrl.bodies_total;
    t.checked_bodies = host_ctrl.checked_total;
    t.blocks = plan.blocks;
    *timing = t;

    if (lowest) {
        if (host_low_found < 0 || host_low_found > k_low)
            return QUBO_EDEVICE;
        low->clear();
        const int pad = ns - n;
        for (int i = 0; i < host_low_found; ++i) {
            const LowEntry &le = host_low[i];
            if (le.x & ((1ull << pad) - 1))
                continue;  // a padding variable is set: not a state of the problem
            qubo_state st;
            st.energy = le.e;
            st.reserved = 0;
            st.index = le.x >> pad;
            low->push_back(st);
            if ((int)low->size() == rq.lowest_k)
                break;
        }
        // Without a cap the first threshold bounds every energy of the problem
        // (padded states may exceed it; they are dropped anyway), so every state
        // was offered and min(k, states searched) of them must be listed.
        const uint64_t states = t.states >> pad;
        const uint64_t expect = states < (uint64_t)rq.lowest_k ? states : (uint64_t)rq.lowest_k;
        if (!have_t0 && low->size() != expect)
            return QUBO_EDEVICE;
        *found = !low->empty();
        return QUBO_OK;
    }

    const Partial &r = host_ctrl.result;
    *found = r.count != 0;
    if (!*found) {
        // Without a cap the threshold was a searched state's energy or an upper
        // bound, so some state must have been recorded.
        return have_t0 ? QUBO_OK : QUBO_EDEVICE;
    }
    qubo_result res{};
    res.min_energy = r.e;
    res.reserved = 0;
    res.argmin = r.arg >> (ns - n);  // padding variables are the lowest bits and 0 at the min
    res.count = r.count;
    *out = res;
    return QUBO_OK;
}

int run(const Request &rq, qubo_result *out, qubo_state *low_out = nullptr,
        int *low_found = nullptr)
{
    using namespace qubo;
    const bool lowest = rq.lowest_k > 0;
    if (!rq.Q || rq.n < 1 || rq.n > QUBO_MAX_N)
        return QUBO_EINVAL;
    if (rq.mode == Mode::Search && !lowest && !out)
        return QUBO_EINVAL;
    if (lowest && (!low_out || !low_found || rq.lowest_k > kMaxLowest || !rq.gated))
        return QUBO_EINVAL;
    const int n = rq.n;
    // Outer split: fixed first k variables (the straightforward split of sec. III.C.1).
    int k = rq.split_bits;
    if (k == 0 && n > kMaxSingleVars)
        k = n - kMaxSingleVars;
    if (k < 0 || (k > 0 && (n - k < kMinSearchVars || rq.mode == Mode::Build || rq.ranged)))
        return QUBO_EINVAL;
    if (k > kMaxSplitBits)
        return QUBO_EPLAN;
    {
        // Reject an unplannable split before touching the device.
        qubo_plan probe;
        const int rc0 = make_plan(n, rq.prefix_bits, rq.cache_bits, 256, rq.cols_per_lane, k, &probe);
        if (rc0 != QUBO_OK)
            return rc0;
    }
    DeviceInfo dev;
    int rc = device_info(&dev);
    if (rc != QUBO_OK)
        return rc;

    // Q to the host; fold and guard.
    std::vector<int32_t> Qh;
    rc = read_q(rq.Q, n, rq.stream, Qh);
    if (rc != QUBO_OK)
        return rc;
    std::vector<int32_t> U;
    int64_t abs_sum = 0;
    rc = fold_upper(Qh.data(), n, U, &abs_sum);
    if (rc != QUBO_OK)
        return rc;

    if (k == 0) {
        bool found = false;
        qubo_timing t{};
        std::vector<qubo_state> low;
        rc = run_one(rq, dev, std::move(U), n, abs_sum, false, 0, out, &found, &t, &low);
        if (rc == QUBO_OK && rq.mode == Mode::Search)
            g_timing = t;
        if (rc == QUBO_OK && lowest) {
            std::copy(low.begin(), low.end(), low_out);
            *low_found = (int)low.size();
        }
        return rc;
    }

    if (lowest) {
        // 2^k sub-problems; once k states are known, their k-th energy caps the
        // later sub-problems, and a sub-cube whose every state lies above it is
        // skipped.
        const int m = n - k;
        qubo_timing acc{};
        std::vector<qubo_state> best, sub;
        std::vector<int32_t> Usub;
        for (uint64_t f = 0; f < (1ull << k); ++f) {
            int64_t c = 0, sub_abs = 0;
            reduce_fixed(U, n, k, f, Usub, &c, &sub_abs);
            bool have_cap = false;
            int32_t cap = 0;
            if ((int)best.size() == rq.lowest_k) {
                const int64_t cap64 = (int64_t)best.back().energy - c;
                if (cap64 < -sub_abs)
                    continue;
                have_cap = true;
                cap = (int32_t)(cap64 < sub_abs ? cap64 : sub_abs);
            }
            bool found = false;
            qubo_timing t{};
            rc = run_one(rq, dev, Usub, m, sub_abs, have_cap, cap, nullptr, &found, &t, &sub);
            if (rc != QUBO_OK)
                return rc;
            add_timing(acc, t);
            for (auto &st : sub) {
                st.energy = (int32_t)((int64_t)st.energy + c);
                st.index |= f << m;
            }
            merge_lowest(best, sub, rq.lowest_k);
        }
        g_timing = acc;
        std::copy(best.begin(), best.end(), low_out);
        *low_found = (int)best.size();
        return QUBO_OK;
    }

    // 2^k sub-problems of n - k variables, each with the reduced matrix and the
    // constant c(x_f); the best energy found so far caps the later ones.
    const int m = n - k;
    qubo_timing acc{};
    qubo_result best{};
    bool have_best = false;
    std::vector<int32_t> Usub;
    for (uint64_t f = 0; f < (1ull << k); ++f) {
        int64_t c = 0, sub_abs = 0;
        reduce_fixed(U, n, k, f, Usub, &c, &sub_abs);
        bool have_cap = false;
        int32_t cap = 0;
        if (have_best) {
            const int64_t cap64 = (int64_t)best.min_energy - c;
            if (cap64 < -sub_abs)
                continue;  // every state of this sub-cube is above the best energy found
            have_cap = true;
            cap = (int32_t)(cap64 < 0 ? cap64 : 0);
        }
        qubo_result sub{};
        bool found = false;
        qubo_timing t{};
        rc = run_one(rq, dev, Usub, m, sub_abs, have_cap, cap, &sub, &found, &t);
        if (rc != QUBO_OK)
            return rc;
        add_timing(acc, t);
        if (!found)
            continue;
        const int64_t e = (int64_t)sub.min_energy + c;
        const uint64_t idx = (f << m) | sub.argmin;
        if (!have_best || e < best.min_energy) {
            best.min_energy = (int32_t)e;
            best.argmin = idx;
            best.count = sub.count;
            have_best = true;
        } else if (e == best.min_energy) {
            best.count += sub.count;
            best.argmin = idx < best.argmin ? idx : best.argmin;
        }
    }
    if (!have_best)
        return QUBO_EDEVICE;  // the first sub-problem is searched without a cap
    g_timing = acc;
    *out = best;
    return QUBO_OK;
}

// What one step of an int32 run needs: the device, and the folded matrix of
// the current sub-problem with its constant c(x_f) and sum of |entries|.
struct StepInput {
    DeviceInfo dev;
    std::vector<int32_t> Usub;
    int64_t c = 0, sub_abs = 0;
};

// Checks the run record against n, Q (its fingerprint) and the record's kind,
// then reads and folds Q and reduces it to the current sub-problem.
int prepare_step(const int32_t *Q, int n, hipStream_t stream, const qubo_progress &p, uint32_t kind,
                 StepInput *in)
{
    using namespace qubo;
    const int k = p.split_bits, A = p.prefix_bits, cb = p.chunk_bits, m = n - k;
    if (k < 0 || k > kMaxSplitBits || m < kMinSearchVars || m > kMaxSingleVars || A < kRegBits ||
        A > m || A > kMaxPrefixBits || cb < kRegBits || cb > A || p.sub >= (1ull << k) ||
        p.next >= (1ull << A) || (p.next & ((1ull << cb) - 1)) || p.steps_total == 0 || p.kind != kind)
        return QUBO_EINVAL;
    int rc = device_info(&in->dev);
    if (rc != QUBO_OK)
        return rc;
    std::vector<int32_t> Qh;
    rc = read_q(Q, n, stream, Qh);
    if (rc != QUBO_OK)
        return rc;
    if (fingerprint(Qh.data(), Qh.size() * 4, n) != p.q_hash)
        return QUBO_EINVAL;  // not the matrix this run was started with
    std::vector<int32_t> U;
    int64_t abs_sum = 0;
    rc = fold_upper(Qh.data(), n, U, &abs_sum);
    if (rc != QUBO_OK)
        return rc;
    in->c = 0;
    in->sub_abs = abs_sum;
    if (k > 0)
        reduce_fixed(U, n, k, p.sub, in->Usub, &in->c, &in->sub_abs);
    else
        in->Usub.swap(U);
    return QUBO_OK;
}

// The request for the slice of the current sub-problem that a step searches.
Request slice_request(const int32_t *Q, int n, hipStream_t stream, const qubo_progress &p)
{
    Request rq;
    rq.Q = Q;
    rq.n = n - p.split_bits;
    rq.prefix_bits = p.prefix_bits;
    rq.ranged = true;
    rq.gray_lo = p.next;
    rq.gray_hi = p.next + (1ull << p.chunk_bits);
    rq.stream = stream;
    return rq;
}

// Moves the run in q (a copy of p) past the slice just searched, or past the
// rest of the sub-problem when it was skipped.
void advance(qubo_progress &q, const qubo_progress &p, bool skip_sub)
{
    const int A = p.prefix_bits, cb = p.chunk_bits;
    if (skip_sub) {
        q.steps_done += (1ull << (A - cb)) - (p.next >> cb);
        q.next = 1ull << A;
    } else {
        q.steps_done += 1;
        q.next = p.next + (1ull << cb);
    }
    if (q.next == (1ull << A)) {
        q.next = 0;
        q.sub = p.sub + 1;
        if (q.sub == (1ull << p.split_bits))
            q.done = 1;
    }
}

// One step of a run in slices (qubo_search_step): the next slice of the
// current sub-problem, folded into the run's result by the final reduction's
// rule; the new state goes to *next (the caller's struct is left alone on error).
int run_step(const int32_t *Q, int n, hipStream_t stream, const qubo_progress &p, qubo_progress *next)
{
    StepInput in;
    int rc = prepare_step(Q, n, stream, p, 0, &in);
    if (rc != QUBO_OK)
        return rc;
    const int m = n - p.split_bits;
    qubo_progress q = p;
    qubo_timing t{};
    bool skip = false, have_cap = false;
    int32_t cap = 0;
    if (p.have_best) {
        const int64_t cap64 = (int64_t)p.best.min_energy - in.c;
        if (cap64 < -in.sub_abs) {
            skip = true;  // every state of this sub-problem lies above the best energy found so far
        } else {
            have_cap = true;
            cap = (int32_t)(cap64 < in.sub_abs ? cap64 : in.sub_abs);
        }
    }
    if (!skip) {
        qubo_result r{};
        bool found = false;
        rc = run_one(slice_request(Q, n, stream, p), in.dev, std::move(in.Usub), m, in.sub_abs, have_cap,
                     cap, &r, &found, &t);
        if (rc != QUBO_OK)
            return rc;
        if (found) {
            const int32_t e = (int32_t)((int64_t)r.min_energy + in.c);  // a state's energy: |e| <= abs_sum
            const uint64_t idx = (p.split_bits > 0 ? (p.sub << m) : 0) | r.argmin;
            if (!q.have_best || e < q.best.min_energy) {
                q.best.min_energy = e;
                q.best.reserved = 0;
                q.best.argmin = idx;
                q.best.count = r.count;
                q.have_best = 1;
            } else if (e == q.best.min_energy) {
                q.best.count += r.count;
                q.best.argmin = idx < q.best.argmin ? idx : q.best.argmin;
            }
        }
    }
    advance(q, p, skip);
    g_timing = t;
    *next = q;
    return QUBO_OK;
}

// One step of a spectrum run (qubo_search_step_lowest): the k lowest states of
// the next slice, merged into the run's list; once the list is full its k-th
// energy caps the slice, and a sub-problem wholly above it is skipped.
int run_step_lowest(const int32_t *Q, int n, hipStream_t stream, const qubo_progress_lowest &p,
                    qubo_progress_lowest *next)
{
    using namespace qubo;
    if (p.k < 1 || p.k > kMaxLowest || p.found < 0 || p.found > p.k)
        return QUBO_EINVAL;
    StepInput in;
    int rc = prepare_step(Q, n, stream, p.head, 2, &in);
    if (rc != QUBO_OK)
        return rc;
    const int m = n - p.head.split_bits;
    qubo_progress_lowest q = p;
    qubo_timing t{};
    bool skip = false, have_cap = false;
    int32_t cap = 0;
    if (p.found == p.k) {
        const int64_t cap64 = (int64_t)p.states[p.k - 1].energy - in.c;
        if (cap64 < -in.sub_abs) {
            skip = true;  // every state of this sub-problem lies above the k-th energy found so far
        } else {
            have_cap = true;
            cap = (int32_t)(cap64 < in.sub_abs ? cap64 : in.sub_abs);
        }
    }
    if (!skip) {
        Request rq = slice_request(Q, n, stream, p.head);
        rq.lowest_k = p.k;
        std::vector<qubo_state> sub;
        bool found = false;
        rc = run_one(rq, in.dev, std::move(in.Usub), m, in.sub_abs, have_cap, cap, nullptr, &found, &t,
                     &sub);
        if (rc != QUBO_OK)
            return rc;
        for (auto &st : sub) {
            st.energy = (int32_t)((int64_t)st.energy + in.c);
            st.index |= p.head.split_bits > 0 ? (p.head.sub << m) : 0;
        }
        std::vector<qubo_state> best(p.states, p.states + p.found);
        merge_lowest(best, sub, p.k);
        std::copy(best.begin(), best.end(), q.states);
        q.found = (int32_t)best.size();
        q.head.have_best = q.found > 0;
    }
    advance(q.head, p.head, skip);
    g_timing = t;
    *next = q;
    return QUBO_OK;
}

// ---------------------------------------------------------------------------
// Real-valued (binary64) Q.
// ---------------------------------------------------------------------------

struct RequestF64 {
    const double *Q = nullptr;
    int n = 0;
    int prefix_bits = -1;
    int cache_bits = -1;
    bool ranged = false;
    uint64_t gray_lo = 0, gray_hi = 0;
    hipStream_t stream = nullptr;
    int lowest_k = 0;  // > 0: the k-lowest search (its states go to *low)
};

static_assert(sizeof(qubo::LowEntryF64) == sizeof(qubo_state_f64), "list entry layout");

// have_cap: the search only has to find states with E <= cap (a real energy
// found elsewhere); an empty result is then valid and *found says whether any
// state was recorded.
int run_f64(const RequestF64 &rq, qubo_result_f64 *out, bool have_cap = false, double cap = 0.0,
            bool *found = nullptr, std::vector<qubo_state_f64> *low = nullptr)
{
    using namespace qubo;
    const bool lowest = rq.lowest_k > 0;
    if (!rq.Q || rq.n < 1 || rq.n > kMaxSingleVars || (lowest ? (!low || rq.lowest_k > kMaxLowest) : !out))
        return QUBO_EINVAL;
    const int n = rq.n;
    // The binary64 rows of Gray bits 4 .. l-1 sit in LDS (4 KiB each per
    // workgroup): the default keeps 6 of them, so that with the fp32 rows of
    // the walk's carries four workgroups fit a CU.
    int cache_bits = rq.cache_bits;
    if (cache_bits < 0 && n >= kMinSearchVars) {  // (tiny problems: the planner's fixed split)
        qubo_plan probe;
        const int rc0 = make_plan(n, rq.prefix_bits, -1, 256, 8, 0, &probe);
        if (rc0 != QUBO_OK)
            return rc0;
        cache_bits = probe.prefix_bits < 10 ? probe.prefix_bits : 10;
    }
    DeviceInfo dev;
    int rc = device_info(&dev);
    if (rc != QUBO_OK)
        return rc;
    qubo_plan plan;
    rc = make_plan(n, rq.prefix_bits, cache_bits, dev.num_cus, 8, 0, &plan);
    if (rc != QUBO_OK)
        return rc;
    const int ns = plan.n_search, A = plan.prefix_bits, B = plan.suffix_bits;
    const int l_eff = plan.cache_bits;
    const int group = kWave * 8;
    const int lds_bytes = (l_eff - 4) * group * 8;
    if (lds_bytes > kMaxLdsBytes)
        return QUBO_EPLAN;

    // Q to the host; the guard: finite entries and sum |Q_ij| <= 2^100, so that
    // fp32 energies never overflow.
    std::vector<double> Qh((size_t)n * n);
    if (hipMemcpyAsync(Qh.data(), rq.Q, Qh.size() * 8, hipMemcpyDeviceToHost, rq.stream) !=
            hipSuccess ||
        hipStreamSynchronize(rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    double S = 0.0;
    rc = guard_f64(Qh, &S);
    if (rc != QUBO_OK)
        return rc;
    // Fold to the upper triangle in binary64 (the walk's tables only; states
    // are scored against Q itself) and pad small problems.
    std::vector<double> U((size_t)ns * ns, 0.0);
    for (int i = 0; i < n; ++i) {
        U[(size_t)i * ns + i] = Qh[(size_t)i * n + i];
        for (int j = i + 1; j < n; ++j)
            U[(size_t)i * ns + j] = Qh[(size_t)i * n + j] + Qh[(size_t)j * n + i];
    }
    for (int i = n; i < ns; ++i)
        U[(size_t)i * ns + i] = 1.0;

    uint64_t lo = 0, hi = 1ull << A;
    if (rq.ranged) {
        lo = rq.gray_lo;
        hi = rq.gray_hi;
        if (hi > (1ull << A))
            return QUBO_EINVAL;
    }
    const uint64_t seg_first = lo >> plan.seg_bits;
    const uint64_t seg_last = (hi - 1) >> plan.seg_bits;
    const uint64_t segs = seg_last - seg_first + 1;
    const uint64_t seg_blocks = (segs + kWavesPerBlock - 1) / kWavesPerBlock;
    const uint64_t items = plan.col_groups * seg_blocks;
    int per_cu = 0;
    if (search_occupancy_f64(lowest, &per_cu, lds_bytes) != hipSuccess)
        return QUBO_EDEVICE;
    if (per_cu < 1)
        per_cu = 1;
    const uint64_t want_blocks = (uint64_t)dev.num_cus * (uint64_t)per_cu;
    const int blocks = (int)(items < want_blocks ? items : want_blocks);

    // Workspace.
    const uint64_t cols_padded = (((1ull << B) + group - 1) / group) * group;
    auto al = [](uint64_t v) { return (v + 255) & ~uint64_t(255); };
    const uint64_t off_u = 0;
    const uint64_t off_es = al(off_u + (uint64_t)ns * ns * 8);
    const uint64_t off_mint = al(off_es + cols_padded * 8);
    const uint64_t off_mint32 = al(off_mint + (uint64_t)A * cols_padded * 8);
    const uint64_t off_ep = al(off_mint32 + (uint64_t)A * cols_padded * 4);
    const uint64_t off_epmin = al(off_ep + (1ull << A) * 8);
    const uint64_t off_part = al(off_epmin + ((1ull << (A - kRegBits)) + 2) * 4);
    const uint64_t off_ctrl = al(off_part + (uint64_t)blocks * kWavesPerBlock * sizeof(PartialF64));
    // the k-lowest search: the per-wave lists, the merged list and its length
    const uint64_t list_entries = lowest ? (uint64_t)blocks * kWavesPerBlock * rq.lowest_k : 0;
    const uint64_t off_lists = al(off_ctrl + sizeof(CtrlF64));
    const uint64_t off_low = al(off_lists + list_entries * sizeof(LowEntryF64));
    const uint64_t off_low_found = al(off_low + kMaxLowest * sizeof(LowEntryF64));
    const uint64_t total = lowest ? al(off_low_found + 4) : off_lists;
    Call call;
    call.stream = rq.stream;
    if (hipMallocAsync(&call.ws, total, rq.stream) != hipSuccess) {
        call.ws = nullptr;
        return QUBO_ENOMEM;
    }
    char *base = static_cast<char *>(call.ws);
    double *dU = reinterpret_cast<double *>(base + off_u);
    double *des = reinterpret_cast<double *>(base + off_es);
    double *dmint = reinterpret_cast<double *>(base + off_mint);
    float *dmint32 = reinterpret_cast<float *>(base + off_mint32);
    double *dep = reinterpret_cast<double *>(base + off_ep);
    float *depmin = reinterpret_cast<float *>(base + off_epmin);
    PartialF64 *dpart = reinterpret_cast<PartialF64 *>(base + off_part);
    CtrlF64 *dctrl = reinterpret_cast<CtrlF64 *>(base + off_ctrl);
    if (!call.create_events())
        return QUBO_EDEVICE;

    // A state passes the filter when its fp32 energy is within delta of the
    // best binary64 energy so far; delta = 1024 * 2^-24 S bounds every fp32
    // rounding of the walk, the compare and the gates (at most about
    // 290 * 2^-24 S) more than three times over.
    const double delta = std::ldexp(S, -14);
    float delta32 = (float)delta;
    if ((double)delta32 < delta)
        delta32 = std::nextafter(delta32, INFINITY);
    // The first threshold: E(0) = 0 when state 0 is searched, else above every energy.
    // (for the k-lowest search: always the bound, E(0) bounds only the minimum)
    double t0 = (lo == 0 && !lowest) ? 0.0 : 4.0 * S + 1.0;
    if (have_cap && cap < t0)
        t0 = cap;

    if (hipEventRecord(call.ev[0], rq.stream) != hipSuccess ||
        hipMemcpyAsync(dU, U.data(), U.size() * 8, hipMemcpyHostToDevice, rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    if (launch_build_tables_f64(dU, ns, A, B, cols_padded, des, dmint, dmint32, dep, depmin, lo, hi,
                                rq.stream) !=
        hipSuccess)
        return QUBO_EDEVICE;
    if (hipEventRecord(call.ev[1], rq.stream) != hipSuccess ||
        launch_init_ctrl_f64(dctrl, t0, depmin + (1ull << (A - kRegBits)), rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    SearchArgsF64 sa{};
    sa.es = des;
    sa.mint = dmint;
    sa.mint32 = dmint32;
    sa.ep = dep;
    sa.epmin = depmin;
    sa.Q = rq.Q;
    sa.partials = dpart;
    sa.ctrl = dctrl;
    sa.cols_padded = cols_padded;
    sa.gray_lo = lo;
    sa.gray_hi = hi;
    sa.seg_first = seg_first;
    sa.segs = segs;
    sa.seg_blocks = seg_blocks;
    sa.items = items;
    sa.A = A;
    sa.B = B;
    sa.n = n;
    sa.pad = ns - n;
    sa.l_eff = l_eff;
    sa.seg_bits = plan.seg_bits;
    sa.delta = delta32;
    LowEntryF64 *dlists = reinterpret_cast<LowEntryF64 *>(base + off_lists);
    LowEntryF64 *dlow = reinterpret_cast<LowEntryF64 *>(base + off_low);
    int32_t *dlow_found = reinterpret_cast<int32_t *>(base + off_low_found);
    if (lowest) {
        sa.lists = dlists;
        sa.k_low = rq.lowest_k;
    }
    if (launch_search_f64(sa, lowest, blocks, lds_bytes, rq.stream) != hipSuccess ||
        hipEventRecord(call.ev[2], rq.stream) != hipSuccess ||
        launch_reduce_f64(dpart, blocks * kWavesPerBlock, dctrl, rq.stream) != hipSuccess ||
        (lowest && launch_lowest_merge_f64(dlists, list_entries, rq.lowest_k, dlow, dlow_found,
                                           rq.stream) != hipSuccess) ||
        hipEventRecord(call.ev[3], rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    CtrlF64 host_ctrl;
    LowEntryF64 host_low[kMaxLowest];
    int32_t host_low_found = 0;
    if (hipMemcpyAsync(&host_ctrl, dctrl, sizeof(CtrlF64), hipMemcpyDeviceToHost, rq.stream) !=
            hipSuccess ||
        (lowest &&
         (hipMemcpyAsync(host_low, dlow, sizeof(host_low), hipMemcpyDeviceToHost, rq.stream) != hipSuccess ||
          hipMemcpyAsync(&host_low_found, dlow_found, 4, hipMemcpyDeviceToHost, rq.stream) !=
              hipSuccess)) ||
        hipEventRecord(call.ev[4], rq.stream) != hipSuccess ||
        hipStreamSynchronize(rq.stream) != hipSuccess)
        return QUBO_EDEVICE;

    qubo_timing t{};
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, call.ev[0], call.ev[1]) == hipSuccess)
        t.build_ms = ms;
    if (hipEventElapsedTime(&ms, call.ev[1], call.ev[2]) == hipSuccess)
        t.search_ms = ms;
    if (hipEventElapsedTime(&ms, call.ev[2], call.ev[3]) == hipSuccess)
        t.reduce_ms = ms;
    if (hipEventElapsedTime(&ms, call.ev[0], call.ev[4]) == hipSuccess)
        t.total_ms = ms;
    t.states = (hi - lo) << B;
    t.blocks = blocks;
    t.bodies = host_ctrl.bodies_total;
    t.checked_bodies = host_ctrl.slow_total;
    t.slow_bodies = host_ctrl.slow_total;
    t.candidates = host_ctrl.candidates_total;
    g_timing = t;

    if (lowest) {
        // Only states of the problem are offered (padding variables unset), and
        // without a cap the first threshold bounds every energy, so every state
        // was offered and min(k, states searched) of them must be listed.
        const uint64_t states = t.states >> (ns - n);
        const uint64_t expect = states < (uint64_t)rq.lowest_k ? states : (uint64_t)rq.lowest_k;
        if (host_low_found < 0 || host_low_found > rq.lowest_k ||
            (!have_cap && (uint64_t)host_low_found != expect))
            return QUBO_EDEVICE;
        low->clear();
        for (int i = 0; i < host_low_found; ++i)
            low->push_back(qubo_state_f64{host_low[i].e, host_low[i].x});
        if (found)
            *found = host_low_found > 0;
        return QUBO_OK;
    }
    const PartialF64 &r = host_ctrl.result;
    if (found)
        *found = r.count != 0;
    if (r.count == 0)  // without a cap every state passes the first threshold
        return have_cap ? QUBO_OK : QUBO_EDEVICE;
    out->min_energy = r.e;
    out->argmin = r.arg;
    out->count = r.count;
    return QUBO_OK;
}

// One step of a binary64 run: the next slice, capped by the best energy so far.
int run_step_f64(const double *Q, int n, hipStream_t stream, const qubo_progress &p, qubo_progress *next)
{
    using namespace qubo;
    const int A = p.prefix_bits, cb = p.chunk_bits;
    if (p.kind != 1 || p.split_bits != 0 || n < kMinSearchVars || n > kMaxSingleVars || A < kRegBits ||
        A > n || A > kMaxPrefixBits || cb < kRegBits || cb > A || p.sub != 0 || p.next >= (1ull << A) ||
        (p.next & ((1ull << cb) - 1)) || p.steps_total == 0)
        return QUBO_EINVAL;
    std::vector<double> Qh((size_t)n * n);
    if (hipMemcpyAsync(Qh.data(), Q, Qh.size() * 8, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return QUBO_EDEVICE;
    if (fingerprint(Qh.data(), Qh.size() * 8, n) != p.q_hash)
        return QUBO_EINVAL;  // not the matrix this run was started with
    RequestF64 rq;
    rq.Q = Q;
    rq.n = n;
    rq.prefix_bits = A;
    rq.ranged = true;
    rq.gray_lo = p.next;
    rq.gray_hi = p.next + (1ull << cb);
    rq.stream = stream;
    qubo_result_f64 r{};
    bool found = false;
    const int rc = run_f64(rq, &r, p.have_best != 0, p.best_f64.min_energy, &found);
    if (rc != QUBO_OK)
        return rc;
    qubo_progress q = p;
    if (found) {
        if (!q.have_best || r.min_energy < q.best_f64.min_energy) {
            q.best_f64 = r;
            q.have_best = 1;
        } else if (r.min_energy == q.best_f64.min_energy) {
            q.best_f64.count += r.count;
            q.best_f64.argmin = r.argmin < q.best_f64.argmin ? r.argmin : q.best_f64.argmin;
        }
    }
    q.steps_done += 1;
    q.next = p.next + (1ull << cb);
    if (q.next == (1ull << A)) {
        q.next = 0;
        q.done = 1;
    }
    *next = q;
    return QUBO_OK;
}

// Starts an int32 run (kind 0: minimum, kind 2: spectrum): checks the
// arguments, reads and folds Q (the guard) and fills the run header.
int init_progress(const int32_t *Q, int n, int prefix_bits, int chunk_bits, uint32_t flags, void *stream,
                  uint32_t kind, qubo_progress *p)
{
    using namespace qubo;
    if (!Q || !p || n < 1 || n > QUBO_MAX_N || (flags & ~QUBO_FLAG_SPLIT_MASK))
        return QUBO_EINVAL;
    int k = (int)((flags & QUBO_FLAG_SPLIT_MASK) >> QUBO_FLAG_SPLIT_SHIFT);
    if (k == 0 && n > kMaxSingleVars)
        k = n - kMaxSingleVars;
    if (n - k < kMinSearchVars)
        return QUBO_EINVAL;
    qubo_plan plan;
    int rc = make_plan(n, prefix_bits, -1, 256, 0, k, &plan);
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
    std::vector<int32_t> Qh;
    rc = read_q(Q, n, static_cast<hipStream_t>(stream), Qh);
    if (rc != QUBO_OK)
        return rc;
    std::vector<int32_t> U;
    int64_t abs_sum = 0;
    rc = fold_upper(Qh.data(), n, U, &abs_sum);
    if (rc != QUBO_OK)
        return rc;
    qubo_progress q{};
    q.q_hash = fingerprint(Qh.data(), Qh.size() * 4, n);
    q.n = n;
    q.split_bits = k;
    q.prefix_bits = A;
    q.chunk_bits = chunk_bits;
    q.steps_total = (1ull << k) << (A - chunk_bits);
    q.kind = kind;
    *p = q;
    return QUBO_OK;
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

}  // namespace

extern "C" {

QUBO_API int qubo_make_plan(int n, int prefix_bits, int cache_bits, qubo_plan *out)
{
    // Host-only planning for a 256-CU MI355X.
    return qubo::make_plan(n, prefix_bits, cache_bits, 256, 0, -1, out);
}

QUBO_API int qubo_check_q(const int32_t *Q_host, int n, int64_t *abs_sum)
{
    if (!Q_host || n < 1 || n > QUBO_MAX_N)
        return QUBO_EINVAL;
    std::vector<int32_t> U;
    return qubo::fold_upper(Q_host, n, U, abs_sum);
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
    *out = g_timing;
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
        return "Q out of range (int32: sum of |Q_ij| above 2^30-1; binary64: an entry not finite "
               "or sum of |Q_ij| above 2^100)";
    case QUBO_EPLAN:
        return "split does not fit the kernel (prefix/cache bits out of the supported range)";
    case QUBO_EDEVICE:
        return "no usable gfx950 device or HIP runtime error";
    case QUBO_ENOMEM:
        return "out of device memory";
    default:
        return "unknown status";
    }
}

QUBO_API const char *qubo_version(void)
{
    return "qubo-mi355x 0.5 (gfx950; int32 minimum and k-lowest, 8 or 16 columns/lane; binary64; runs in steps)";
}

}  // extern "C"
