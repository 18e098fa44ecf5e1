// One search of a real-valued (binary64) Q on the device, and one step of a
// binary64 run in slices.
#include "host.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdlib>
#include <unordered_set>

namespace qubo_host {

static_assert(sizeof(qubo::LowEntryF64) == sizeof(qubo_state_f64), "list entry layout");

// The definition's energy of one state (binary64, i ascending, j ascending over
// the set variables; the same sums in the same order as the device).
static double energy_def_host(const std::vector<double> &Qh, int n, const std::vector<char> &x)
{
    double e = 0.0;
    for (int i = 0; i < n; ++i) {
        if (!x[i])
            continue;
        for (int j = 0; j < n; ++j)
            if (x[j])
                e += Qh[(size_t)i * n + j];
    }
    return e;
}

// Energies of distinct real states, ascending: the states that steepest
// single-flip descents reach (fields in binary64; at most 4n flips each) from
// state 0 and from qubo::kDescentStarts - 1 fixed pseudo-random states (SplitMix64,
// a fixed seed: only the first threshold depends on them, never the result),
// and their single-flip neighbours, each scored by the definition, with the
// first `fixed` variables held at the bits of fixed_value (variable 0 its most
// significant of `fixed` bits): states of that sub-cube only.  The j-th value
// bounds the j-th lowest energy of the sub-cube (and of any set holding it)
// from above.
static std::vector<double> descent_energies(const std::vector<double> &Qh, int n, int fixed,
                                            uint64_t fixed_value)
{
    std::unordered_set<uint64_t> seen;
    std::vector<double> es;
    uint64_t sm = 0x51a7e5eedull;  // SplitMix64 state
    auto next = [&sm]() {
        uint64_t z = (sm += 0x9e3779b97f4a7c15ull);
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        return z ^ (z >> 31);
    };
    std::vector<char> x(n);
    std::vector<double> F(n);  // F_v = Q_vv + sum_{j != v, x_j = 1} (Q_vj + Q_jv): the change of setting v
    for (int s = 0; s < qubo::kDescentStarts; ++s) {
        const uint64_t start = s == 0 ? 0 : next();
        for (int v = 0; v < n; ++v)
            x[v] = v < fixed ? (char)((fixed_value >> (fixed - 1 - v)) & 1u) : (char)((start >> v) & 1u);
        for (int v = 0; v < n; ++v) {
            double f = Qh[(size_t)v * n + v];
            for (int j = 0; j < n; ++j)
                if (j != v && x[j])
                    f += Qh[(size_t)v * n + j] + Qh[(size_t)j * n + v];
            F[v] = f;
        }
        for (int it = 0; it < 4 * n; ++it) {
            int best = -1;
            double gain = 0.0;
            for (int v = fixed; v < n; ++v) {
                const double d = x[v] ? -F[v] : F[v];
                if (d < gain) {
                    gain = d;
                    best = v;
                }
            }
            if (best < 0)
                break;
            const double sgn = x[best] ? -1.0 : 1.0;
            x[best] ^= 1;
            for (int j = 0; j < n; ++j)
                if (j != best)
                    F[j] += sgn * (Qh[(size_t)j * n + best] + Qh[(size_t)best * n + j]);
        }
        uint64_t key = 0;
        for (int v = 0; v < n; ++v)
            key |= (uint64_t)x[v] << v;
        for (int v = -1; v < n; ++v) {  // y, then its neighbours over the free variables
            if (v >= 0 && v < fixed)
                continue;
            const uint64_t k = v < 0 ? key : key ^ (1ull << v);
            if (!seen.insert(k).second)
                continue;
            if (v >= 0)
                x[v] ^= 1;
            es.push_back(energy_def_host(Qh, n, x));
            if (v >= 0)
                x[v] ^= 1;
        }
    }
    std::sort(es.begin(), es.end());
    return es;
}

// A dyadic binary64 request (Qi = 2^f Q exactly; dyadic_int32) on the integer
// search: states with E <= cap are those with E_int <= floor(2^f cap), and
// energies come back divided by 2^f (exact: at least 2^-130 in magnitude when
// not 0, since 2^f sum |Q_ij| <= 2^30 - 1 and sum |Q_ij| >= 2^-100).
static int run_dyadic(const RequestF64 &rq, const DeviceInfo &dev, const std::vector<int32_t> &Qi, int f,
                      qubo_result_f64 *out, bool have_cap, double cap, bool *found,
                      std::vector<qubo_state_f64> *low)
{
    using namespace qubo;
    const bool lowest = rq.lowest_k > 0;
    std::vector<int32_t> Ui;
    int64_t abs_sum = 0;
    int rc = fold_upper(Qi.data(), rq.n, Ui, &abs_sum);
    if (rc != QUBO_OK)
        return rc;
    Request irq;
    irq.n = rq.n;
    irq.prefix_bits = rq.prefix_bits;
    irq.cache_bits = rq.cache_bits;
    irq.ranged = rq.ranged;
    irq.gray_lo = rq.gray_lo;
    irq.gray_hi = rq.gray_hi;
    irq.stream = rq.stream;
    irq.cols_per_lane = kColsPerLaneF64;
    irq.lowest_k = rq.lowest_k;
    int32_t icap = 0;
    if (have_cap) {
        const double c = std::floor(std::ldexp(cap, f));
        icap = c > (double)abs_sum ? (int32_t)abs_sum : c < -(double)abs_sum ? (int32_t)-abs_sum - 1 : (int32_t)c;
    }
    qubo_result ir{};
    bool ifound = false;
    qubo_timing t{};
    std::vector<qubo_state> ilow;
    rc = run_one(irq, dev, std::move(Ui), rq.n, abs_sum, have_cap, icap, lowest ? nullptr : &ir, &ifound, &t,
                 lowest ? &ilow : nullptr);
    if (rc != QUBO_OK)
        return rc;
    last_timing() = t;
    if (found)
        *found = ifound;
    if (lowest) {
        low->clear();
        for (const qubo_state &st : ilow)
            low->push_back(qubo_state_f64{std::ldexp((double)st.energy, -f), st.index});
    } else if (ifound) {
        out->min_energy = std::ldexp((double)ir.min_energy, -f);
        out->argmin = ir.argmin;
        out->count = ir.count;
    }
    return QUBO_OK;
}

// have_cap: the search only has to find states with E <= cap (a real energy
// found elsewhere); an empty result is then valid and *found says whether any
// state was recorded.
int run_f64(const RequestF64 &rq, qubo_result_f64 *out, bool have_cap, double cap, bool *found,
            std::vector<qubo_state_f64> *low)
{
    using namespace qubo;
    const bool lowest = rq.lowest_k > 0;
    if (!rq.Q || rq.n < 1 || rq.n > kMaxSingleVars || (lowest ? (!low || rq.lowest_k > kMaxLowest) : !out))
        return QUBO_EINVAL;
    const int n = rq.n;
    DeviceInfo dev;
    int rc = device_info(&dev);
    if (rc != QUBO_OK)
        return rc;
    // The integer search's plan: the walk runs on int32 tables of the same shape.
    qubo_plan plan;
    rc = make_plan(n, rq.prefix_bits, rq.cache_bits, dev.num_cus, kColsPerLaneF64, 0, &plan);
    if (rc != QUBO_OK)
        return rc;
    const int ns = plan.n_search, A = plan.prefix_bits, B = plan.suffix_bits;
    const int group = kWave * kColsPerLaneF64;
    const int lds_bytes = plan.lds_bytes;

    // Q to the host; the guard: finite entries and sum |Q_ij| either 0 or in
    // [2^-100, 2^100].
    std::vector<double> Qh((size_t)n * n);
    if (hipMemcpyAsync(Qh.data(), rq.Q, Qh.size() * 8, hipMemcpyDeviceToHost, rq.stream) !=
            hipSuccess ||
        hipStreamSynchronize(rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    double S = 0.0;
    rc = guard_f64(Qh, &S);
    if (rc != QUBO_OK)
        return rc;

    // A dyadic matrix (integer-valued ones included) is searched as the int32
    // matrix 2^f Q by the integer search, which is exact for it.
    {
        std::vector<int32_t> Qi;
        int f = 0;
        if (dyadic_int32(Qh, Qi, &f))
            return run_dyadic(rq, dev, Qi, f, out, have_cap, cap, found, low);
    }
    // Fold to the upper triangle in binary64 (the walk's tables only; states
    // are scored against Q itself) and pad small problems: a padding variable
    // gets the positive diagonal S (1 for the zero matrix) and no couplings, so
    // setting it raises a state's energy and keeps the tables on Q's scale.
    std::vector<double> U((size_t)ns * ns, 0.0);
    for (int i = 0; i < n; ++i) {
        U[(size_t)i * ns + i] = Qh[(size_t)i * n + i];
        for (int j = i + 1; j < n; ++j)
            U[(size_t)i * ns + j] = Qh[(size_t)i * n + j] + Qh[(size_t)j * n + i];
    }
    const double pad_diag = S > 0.0 ? S : 1.0;
    for (int i = n; i < ns; ++i)
        U[(size_t)i * ns + i] = pad_diag;
    // The scale s = 2^e with s * S_walk <= 2^q, S_walk bounding the magnitude
    // sum of the folded, padded matrix (and so of every table entry and every
    // sub-sum the walk forms).  q = kQuantBits unless S_walk exceeds n^2 times
    // the median nonzero |Q_ij| by more than 8: then by the excess, up to
    // kQuantBitsMax (entries over many orders of magnitude would otherwise round
    // to a few bits, leave many states with one walked value and send them all
    // to re-evaluation).  Any q up to kQuantBitsMax keeps the proof below.
    const double S_walk = S + (double)(ns - n) * pad_diag;
    int qbits = kQuantBits;
    {
        std::vector<double> mags;
        mags.reserve(Qh.size());
        for (double v : Qh)
            if (v != 0.0)
                mags.push_back(std::fabs(v));
        if (!mags.empty()) {
            std::nth_element(mags.begin(), mags.begin() + mags.size() / 2, mags.end());
            const double spread = S_walk / ((double)n * n * mags[mags.size() / 2]);
            const int extra = (int)std::floor(std::log2(spread)) - 3;
            qbits = std::min(kQuantBitsMax, kQuantBits + std::max(0, extra));
        }
    }
    int ex = 0;
    (void)std::frexp(S_walk, &ex);  // S_walk < 2^ex
    const double scale = std::ldexp(1.0, qbits - ex);

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
    const uint64_t off_mint = al(off_es + cols_padded * 4);
    const uint64_t off_ep = al(off_mint + (uint64_t)A * cols_padded * 4);
    const uint64_t off_epmin = al(off_ep + (1ull << A) * 4);
    const uint64_t groups = A > kRegBits + 2 ? 1ull << (A - kRegBits - 2) : 1ull;
    const uint64_t off_gates = al(off_epmin + ((1ull << (A - kRegBits)) + 2) * 4);
    const uint64_t off_part = al(off_gates + gate_table_len(A, cols_padded, kColsPerLaneF64) * 4);
    const uint64_t off_ctrl = al(off_part + (uint64_t)blocks * sizeof(PartialF64));  // one per workgroup
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
    int32_t *des = reinterpret_cast<int32_t *>(base + off_es);
    int32_t *dmint = reinterpret_cast<int32_t *>(base + off_mint);
    int32_t *dep = reinterpret_cast<int32_t *>(base + off_ep);
    int32_t *depmin = reinterpret_cast<int32_t *>(base + off_epmin);
    int32_t *dgates = reinterpret_cast<int32_t *>(base + off_gates);
    PartialF64 *dpart = reinterpret_cast<PartialF64 *>(base + off_part);
    CtrlF64 *dctrl = reinterpret_cast<CtrlF64 *>(base + off_ctrl);
    if (!call.create_events())
        return QUBO_EDEVICE;

    // A state is re-evaluated when its rounded walk value W is at most
    // floor(s T) + M for the bound T of the minimum: |W - s E| is at most
    // (A + 2) / 2 for the rounded terms plus under 2^-20 of binary64 rounding,
    // below M - 1 = A / 2 + 2 (the binary64 part stays under 2^-12 at q = 28).
    // The filter's cap 2^(q + 2) lies above every W.
    const int margin = A / 2 + 3;
    const int filter_cap = 1 << (qbits + 2);
    // The first threshold: E(0) = 0 when state 0 is searched, else above every
    // energy (for the k-lowest search: always that bound, E(0) bounds only the
    // minimum).  A whole-space search starts from real energies instead: the
    // lowest of the descents' states for the minimum, their k-th lowest for
    // the k lowest (each wave's own list bounds the k-th lowest energy only
    // loosely: it holds the lowest states of its share of the space), raised
    // by 2^-40 S against any difference between the host's sums and the
    // device's.
    double t0 = (lo == 0 && !lowest) ? 0.0 : 4.0 * S + 1.0;
    if (n >= kMinSearchVars) {
        int fixed = 0;
        uint64_t fixed_value = 0;
        largest_subcube(lo, hi, A, &fixed, &fixed_value);  // the whole space: nothing fixed
        const std::vector<double> es = descent_energies(Qh, n, fixed, fixed_value);
        const size_t j = lowest ? (size_t)rq.lowest_k - 1 : 0;
        if (j < es.size()) {
            const double t = es[j] + std::ldexp(S, -40);
            t0 = t < t0 ? t : t0;
        }
    }
    if (have_cap && cap < t0)
        t0 = cap;

    // Integer offsets that keep the rows and the walked suffix energies at or
    // above zero (the integer search's table offsets, on the rounded tables):
    // each row entry is rint(s m) with m a binary64 sub-sum of the row's terms,
    // so rint(s m) >= -(s sum of the row's negative parts) - 1 > -k[v] with k[v]
    // the ceiling of that scaled sum plus 1 (the sum's own rounding is far below
    // 1/2); likewise es_add for E_s.
    TableOffsetsF64 off{};
    off.rows = A;
    {
        auto neg_bound = [scale](double neg) { return (int32_t)std::ceil(neg * scale) + 1; };
        double neg = 0.0;
        for (int i = A; i < ns; ++i)
            for (int j = i; j < ns; ++j)
                neg += std::max(0.0, -U[(size_t)i * ns + j]);
        off.es_add = neg_bound(neg);
        for (int v = 0; v < A; ++v) {
            double nv = 0.0;
            for (int j = A; j < ns; ++j)
                nv += std::max(0.0, -U[(size_t)v * ns + j]);
            off.k[v] = neg_bound(nv);
            if (A - 1 - v < kGateBits)
                off.kgate[A - 1 - v] = off.k[v];
        }
    }

    if (hipEventRecord(call.ev[0], rq.stream) != hipSuccess ||
        hipMemcpyAsync(dU, U.data(), U.size() * 8, hipMemcpyHostToDevice, rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    GateOffsets kg;
    std::copy(off.kgate, off.kgate + 16, kg.k);
    if (launch_build_tables_f64(dU, ns, A, B, cols_padded, scale, off, des, dmint, dep, depmin, lo, hi,
                                rq.stream) != hipSuccess ||
        launch_gate_tables(dmint, cols_padded, A, B, kColsPerLaneF64, kg, depmin, dgates, lo, hi, rq.stream) !=
            hipSuccess)
        return QUBO_EDEVICE;
    if (hipEventRecord(call.ev[1], rq.stream) != hipSuccess ||
        launch_init_ctrl_f64(dctrl, t0, depmin + (1ull << (A - kRegBits)), dgates + gate_groups(A), rq.stream) !=
            hipSuccess)
        return QUBO_EDEVICE;
    SearchArgsF64 sa{};
    sa.es = des;
    sa.mint = dmint;
    sa.ep = dep;
    sa.epmin = depmin;
    sa.gates = dgates;
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
    sa.l_eff = plan.cache_bits < plan.seg_bits ? plan.cache_bits : plan.seg_bits;
    sa.seg_bits = plan.seg_bits;
    sa.scale = scale;
    sa.margin = margin;
    sa.cap = filter_cap;
    LowEntryF64 *dlists = reinterpret_cast<LowEntryF64 *>(base + off_lists);
    LowEntryF64 *dlow = reinterpret_cast<LowEntryF64 *>(base + off_low);
    int32_t *dlow_found = reinterpret_cast<int32_t *>(base + off_low_found);
    if (lowest) {
        sa.lists = dlists;
        sa.k_low = rq.lowest_k;
    }
    if (launch_search_f64(sa, lowest, blocks, lds_bytes, rq.stream) != hipSuccess ||
        hipEventRecord(call.ev[2], rq.stream) != hipSuccess ||
        launch_reduce_f64(dpart, blocks, dctrl, rq.stream) != hipSuccess ||
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
    t.cols_per_lane = kColsPerLaneF64;
    t.bodies = host_ctrl.bodies_total;
    t.checked_bodies = host_ctrl.slow_total;
    t.slow_bodies = host_ctrl.slow_total;
    t.candidates = host_ctrl.candidates_total;
    last_timing() = t;

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

}  // namespace qubo_host
