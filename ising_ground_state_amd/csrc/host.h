// Host side of the C-ABI (internal): the request structs, the helpers the
// entry points share, and the runs behind them.  Not installed; include/qubo.h
// is the interface.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "kernels.h"
#include "kernels_f64.h"
#include "plan.h"
#include "qubo.h"

namespace qubo_host {

// The calling thread's timing of its last search (qubo_last_timing).
qubo_timing &last_timing();

struct DeviceInfo {
    int num_cus = 0;
};

// The current device's compute units; QUBO_EDEVICE unless it is a gfx950.
int device_info(DeviceInfo *info);

// Copies Q (n x n int32, device) to the host.
int read_q(const int32_t *Q, int n, hipStream_t stream, std::vector<int32_t> &Qh);

// FNV-1a (64 bit) over n (4 little-endian bytes) and the bytes of Q's entries.
uint64_t fingerprint(const void *Qh, size_t bytes, int n);

// The binary64 guard: finite entries and S = sum |Q_ij| (rounded up) either 0
// or in [2^-100, 2^100] (QUBO_ERANGE otherwise).
int guard_f64(const std::vector<double> &Qh, double *S_out);

// Everything one call owns; released in the destructor on every path.
struct Call {
    hipStream_t stream = nullptr;
    void *ws = nullptr;
    // Work enqueued on a caller-provided workspace: the destructor waits for it,
    // so that no call returns while its kernels still use that buffer.
    bool enqueued = false;
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
        } else if (enqueued) {
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
    // Caller-provided device workspace (qubo_search_noalloc): used instead of a
    // stream-ordered allocation, and no HIP events are created (no stage times).
    void *scratch = nullptr;
    uint64_t scratch_bytes = 0;
};

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

// A dyadic binary64 matrix as int32: true, with Qi = 2^f Q exactly, when every
// entry is an integer multiple of 2^-f and sum |2^f Q_ij| <= 2^30 - 1 (then
// every partial sum of the binary64 definition is exact); false otherwise.
bool dyadic_int32(const std::vector<double> &Qh, std::vector<int32_t> &Qi, int *f_out);

// Keeps the k first states of `acc` merged with `add`, in (energy, index) order.
void merge_lowest(std::vector<qubo_state> &acc, const std::vector<qubo_state> &add, int k);

// Sums the timings of the sub-problems of one search.
void add_timing(qubo_timing &acc, const qubo_timing &t);

// A slice [gray_lo, gray_hi) of the Gray walk over an explicit prefix size:
// whole 32-step bodies, non-empty, inside the 2^prefix_bits steps.
bool valid_slice(int n, int prefix_bits, uint64_t gray_lo, uint64_t gray_hi);

// int32 Q (run_int.hip).  run_one: one launch on the folded matrix U; run: a
// whole request, with the outer split above 58 variables or when asked for.
int run_one(const Request &rq, const DeviceInfo &dev, std::vector<int32_t> U, int n, int64_t abs_sum,
            bool have_t0, int32_t t0_cap, qubo_result *out, bool *found, qubo_timing *timing,
            std::vector<qubo_state> *low = nullptr);
int run(const Request &rq, qubo_result *out, qubo_state *low_out = nullptr, int *low_found = nullptr);

// binary64 Q (run_f64.hip).
int run_f64(const RequestF64 &rq, qubo_result_f64 *out, bool have_cap = false, double cap = 0.0,
            bool *found = nullptr, std::vector<qubo_state_f64> *low = nullptr);

// Runs in steps (run_steps.hip, run_f64.hip).
int init_progress(const int32_t *Q, int n, int prefix_bits, int chunk_bits, uint32_t flags, void *stream,
                  uint32_t kind, qubo_progress *p);
int run_step(const int32_t *Q, int n, hipStream_t stream, const qubo_progress &p, qubo_progress *next);
int run_step_lowest(const int32_t *Q, int n, hipStream_t stream, const qubo_progress_lowest &p,
                    qubo_progress_lowest *next);
int run_step_f64(const double *Q, int n, hipStream_t stream, const qubo_progress &p, qubo_progress *next);

}  // namespace qubo_host
