// One search of an int32 Q on the device (Maltsev et al., "Terastate-per-second
// QUBO Brute-Force on a Single GPU", sec. III, Algorithms 1-2 and sec. III.C):
//   1. copy Q (n x n int32, at most 16 KiB) to the host, fold it into the upper
//      triangle and check the overflow guard;
//   2. plan the split (prefix A, suffix B, cached Gray bits, work units);
//   3. one stream-ordered allocation for U, E_s, M_int, the Gray-ordered E_p,
//      the per-workgroup partial results and a control block (or the caller's
//      device buffer, for the entry point that allocates nothing);
//   4. cache builders, search kernel, final reduction, 64-byte result download;
//   5. free and synchronise the stream.
// Above 58 variables (or when asked for) the 2^k sub-problems of the
// straightforward split of sec. III.C.1 run one after another.
#include "host.h"

#include <algorithm>
#include <climits>

namespace qubo_host {

static_assert(qubo::kPartialBytes == 64, "layout_of reserves 64 bytes per workgroup's partial");

// One search of the folded upper-triangular matrix U (n x n, host memory) on the
// device.  have_t0: the search only has to find states with E <= t0_cap (the
// caller knows a real energy that low elsewhere, or k of them for the
// spectrum); then an empty result is valid and *found reports whether any
// state was recorded.  The spectrum search (rq.lowest_k > 0) writes its states
// to *low, in order, and leaves *out alone.
int run_one(const Request &rq, const DeviceInfo &dev, std::vector<int32_t> U, int n, int64_t abs_sum,
            bool have_t0, int32_t t0_cap, qubo_result *out, bool *found, qubo_timing *timing,
            std::vector<qubo_state> *low)
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

    // Workspace: one stream-ordered allocation, or the caller's buffer.
    char *base = nullptr;
    if (rq.scratch) {
        if (ws_total > rq.scratch_bytes)
            return QUBO_ESCRATCH;
        base = static_cast<char *>(rq.scratch);
        call.enqueued = true;
    } else {
        if (hipMallocAsync(&call.ws, ws_total, rq.stream) != hipSuccess) {
            call.ws = nullptr;
            return QUBO_ENOMEM;
        }
        base = static_cast<char *>(call.ws);
    }
    int32_t *dU = reinterpret_cast<int32_t *>(base + L.off_u);
    int32_t *des = reinterpret_cast<int32_t *>(base + L.off_es);
    int32_t *dmint = reinterpret_cast<int32_t *>(base + L.off_mint);
    int32_t *dep = reinterpret_cast<int32_t *>(base + L.off_ep);
    int32_t *depmin = reinterpret_cast<int32_t *>(base + L.off_epmin);
    int32_t *dgates = reinterpret_cast<int32_t *>(base + L.off_gates);
    Partial *dpart = reinterpret_cast<Partial *>(base + L.off_partials);
    Ctrl *dctrl = reinterpret_cast<Ctrl *>(base + L.off_ctrl);

    // Stage times come from events, which a call that must not allocate skips.
    const bool timed = !rq.scratch;
    if (timed && !call.create_events())
        return QUBO_EDEVICE;
    auto mark = [&](int i) { return !timed || hipEventRecord(call.ev[i], rq.stream) == hipSuccess; };

    // Upload, build, search, reduce.
    if (!mark(0))
        return QUBO_EDEVICE;
    // The search's tables are offset so that the walked energies keep one sign
    // (table_offsets); the exported ones are eq. 8's own.
    const bool offset = rq.mode != Mode::Build;
    const TableOffsets off = offset ? table_offsets(U, ns, A) : TableOffsets{0, 0, U, {}};
    GateOffsets kg;
    std::copy(off.kgate, off.kgate + 16, kg.k);
    if (hipMemcpyAsync(dU, off.Uoff.data(), off.Uoff.size() * 4, hipMemcpyHostToDevice, rq.stream) !=
        hipSuccess)
        return QUBO_EDEVICE;
    if (launch_build_tables(dU, ns, A, B, L.cols_padded, off.rows, (int32_t)off.es_add, kg, des, dmint, dep,
                            depmin, lo, hi, rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    if (offset && launch_gate_tables(dmint, L.cols_padded, A, B, plan.cols_per_lane, kg, depmin, dgates, lo, hi,
                                     rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    if (!mark(1))
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
    // (for the spectrum, whose threshold bounds the k-th energy, sum |Q_ij|).
    // A search starts from the energies of single-flip descents inside the
    // largest sub-cube its range holds instead (real states of the range; the
    // lowest for the minimum, the k-th lowest for the spectrum), so that its
    // gates clear bodies from the first one.  With padding variables (whole
    // spaces only: slices need n >= 5) the spectrum keeps sum |Q_ij|: a
    // neighbour that sets one is not a state of the problem.  A caller's cap (an energy found
    // elsewhere) may only lower it; it is never below -sum |U_ij| here, so
    // every threshold stays within +-2 sum |U_ij|.
    int32_t t0 = (lo == 0 && !lowest) ? 0 : (int32_t)abs_sum;
    if (!lowest || ns == n) {
        int fixed = 0;
        uint64_t fixed_value = 0;
        largest_subcube(lo, hi, A, &fixed, &fixed_value);  // the whole space: nothing fixed
        const std::vector<int64_t> es = descent_energies(U, ns, kDescentStarts, fixed, fixed_value);
        const size_t j = lowest ? (size_t)k_low - 1 : 0;
        if (j < es.size() && es[j] < t0)
            t0 = (int32_t)es[j];
    }
    if (have_t0 && t0_cap < t0)
        t0 = t0_cap;
    const uint64_t groups = A > kRegBits + 2 ? 1ull << (A - kRegBits - 2) : 1ull;
    if (launch_init_ctrl(dctrl, t0, depmin + (1ull << (A - kRegBits)), dgates + gate_groups(A), rq.stream) !=
        hipSuccess)
        return QUBO_EDEVICE;

    SearchArgs sa{};
    sa.es = des;
    sa.mint = dmint;
    sa.ep = dep;
    sa.epmin = depmin;
    sa.gates = dgates;
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
    if (!mark(2))
        return QUBO_EDEVICE;
    if (launch_reduce(dpart, plan.blocks, dctrl, rq.stream) != hipSuccess)
        return QUBO_EDEVICE;
    if (lowest && launch_lowest_merge(dlists, list_entries, k_low, dlow, dlow_found, rq.stream) !=
                      hipSuccess)
        return QUBO_EDEVICE;
    if (!mark(3))
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
    if (!mark(4) || hipStreamSynchronize(rq.stream) != hipSuccess)
        return QUBO_EDEVICE;

    qubo_timing t{};
    float ms = 0.f;
    if (timed) {
        if (hipEventElapsedTime(&ms, call.ev[0], call.ev[1]) == hipSuccess)
            t.build_ms = ms;
        if (hipEventElapsedTime(&ms, call.ev[1], call.ev[2]) == hipSuccess)
            t.search_ms = ms;
        if (hipEventElapsedTime(&ms, call.ev[2], call.ev[3]) == hipSuccess)
            t.reduce_ms = ms;
        if (hipEventElapsedTime(&ms, call.ev[0], call.ev[4]) == hipSuccess)
            t.total_ms = ms;
    }
    t.states = (hi - lo) << B;
    t.slow_bodies = host_ctrl.slow_total;
    t.bodies = host_ctrl.bodies_total;
    t.checked_bodies = host_ctrl.checked_total;
    t.blocks = plan.blocks;
    t.cols_per_lane = (uint32_t)plan.cols_per_lane;
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

int run(const Request &rq, qubo_result *out, qubo_state *low_out, int *low_found)
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
            last_timing() = t;
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
        last_timing() = acc;
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
    last_timing() = acc;
    *out = best;
    return QUBO_OK;
}

}  // namespace qubo_host
