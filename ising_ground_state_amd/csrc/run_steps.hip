// Runs of an int32 Q in steps (qubo_progress, qubo_progress_lowest): the
// record checks, one slice per call, and the starting of a run.
#include "host.h"

#include <algorithm>

namespace qubo_host {

namespace {

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

}  // namespace

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
    last_timing() = t;
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
    last_timing() = t;
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

}  // namespace qubo_host
