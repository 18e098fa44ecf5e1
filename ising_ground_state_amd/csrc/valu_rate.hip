// Issue rate of the vector ALU on gfx950 for the instruction forms the search
// kernels are built from.  A stand-alone program (not part of libqubo.so): it
// measures the peak that the search kernels' roofline is priced against.
//
// Each kernel runs a fixed chain of 16 independent registers per lane, updated
// 8 x 16 times per loop trip, with an empty asm after each round so that every
// update is issued (the compiler may not fold or vectorise across it).  Per
// form it prints:
//   * lane-ops/s = threads x trips x 128 updates / kernel time (HIP events);
//   * the shader clock during the loop: s_memtime ticks (shader clock) over
//     s_memrealtime ticks (a constant 100 MHz), summed over one wave per workgroup;
//   * cycles per wave-instruction on one SIMD: kernel time x that clock, over the
//     instructions each SIMD issues (waves per SIMD x updates per wave).
// Forms: v_add_u32 with two VGPR operands, with an inline constant and with an
// SGPR; v_min3_i32 over three VGPRs; v_pk_add_u16 (two 16-bit adds per lane);
// v_add_f32 with two VGPRs.
//
//     ising_ground_state_amd/lib/qubo_valu_rate
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

namespace {

constexpr int kThreads = 256;  // 4 waves per workgroup, one per SIMD of a CU
constexpr int kRegs = 16;
constexpr int kRounds = 8;

enum Form { AddVV, AddVC, AddVS, Min3, PkAddU16, AddF32, kForms };
const char *kNames[kForms] = {"v_add_u32 v,v", "v_add_u32 v,const", "v_add_u32 v,s", "v_min3_i32 v,v,v",
                              "v_pk_add_u16 v,v", "v_add_f32 v,v"};
const int kElems[kForms] = {1, 1, 1, 1, 2, 1};  // results per lane per instruction

typedef short short2_t __attribute__((ext_vector_type(2)));

template <int F>
__global__ __launch_bounds__(kThreads) void rate_kernel(int *__restrict__ out, uint64_t *__restrict__ ticks,
                                                        int trips, int seed)
{
    int a[kRegs];
    float f[kRegs];
    short2_t p[kRegs];
#pragma unroll
    for (int r = 0; r < kRegs; ++r) {
        a[r] = (int)threadIdx.x + r * 7;
        f[r] = (float)(threadIdx.x + r);
        p[r] = short2_t{(short)(threadIdx.x + r), (short)(seed - r)};
    }
    const int s = __builtin_amdgcn_readfirstlane(seed);
    const uint64_t c0 = clock64();
    const uint64_t w0 = wall_clock64();
    for (int i = 0; i < trips; ++i) {
#pragma unroll
        for (int rep = 0; rep < kRounds; ++rep) {
#pragma unroll
            for (int r = 0; r < kRegs; ++r) {
                if constexpr (F == AddVV)
                    a[r] += a[(r + 1) & (kRegs - 1)];
                else if constexpr (F == AddVC)
                    a[r] += 7;
                else if constexpr (F == AddVS)
                    a[r] += s;
                else if constexpr (F == Min3) {
                    const int b = a[(r + 1) & (kRegs - 1)], c = a[(r + 2) & (kRegs - 1)];
                    const int m = a[r] < b ? a[r] : b;
                    a[r] = m < c ? m : c;
                } else if constexpr (F == PkAddU16)
                    p[r] = p[r] + p[(r + 1) & (kRegs - 1)];
                else
                    f[r] += f[(r + 1) & (kRegs - 1)];
            }
#pragma unroll
            for (int r = 0; r < kRegs; ++r) {
                if constexpr (F == PkAddU16)
                    asm volatile("" : "+v"(p[r]));
                else if constexpr (F == AddF32)
                    asm volatile("" : "+v"(f[r]));
                else
                    asm volatile("" : "+v"(a[r]));
            }
        }
    }
    const uint64_t c1 = clock64();
    const uint64_t w1 = wall_clock64();
    int t = 0;
#pragma unroll
    for (int r = 0; r < kRegs; ++r)
        t += a[r] + (int)f[r] + (int)p[r].x + (int)p[r].y;
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = t;
    if (threadIdx.x == 0) {
        ticks[2 * (size_t)blockIdx.x] = c1 - c0;
        ticks[2 * (size_t)blockIdx.x + 1] = w1 - w0;
    }
}

template <int F>
void launch(int blocks, int *out, uint64_t *ticks, int trips)
{
    hipLaunchKernelGGL(rate_kernel<F>, dim3(blocks), dim3(kThreads), 0, 0, out, ticks, trips, 3);
}

void launch_form(int form, int blocks, int *out, uint64_t *ticks, int trips)
{
    switch (form) {
    case AddVV: launch<AddVV>(blocks, out, ticks, trips); break;
    case AddVC: launch<AddVC>(blocks, out, ticks, trips); break;
    case AddVS: launch<AddVS>(blocks, out, ticks, trips); break;
    case Min3: launch<Min3>(blocks, out, ticks, trips); break;
    case PkAddU16: launch<PkAddU16>(blocks, out, ticks, trips); break;
    default: launch<AddF32>(blocks, out, ticks, trips); break;
    }
}

bool ok(hipError_t e, const char *what)
{
    if (e != hipSuccess) {
        std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        return false;
    }
    return true;
}

}  // namespace

int main()
{
    hipDeviceProp_t prop;
    if (!ok(hipGetDeviceProperties(&prop, 0), "hipGetDeviceProperties"))
        return 1;
    const int cus = prop.multiProcessorCount;
    const int trips = 20000;
    const int max_waves_per_simd = 8;
    const size_t max_blocks = (size_t)cus * max_waves_per_simd;
    int *out = nullptr;
    uint64_t *ticks = nullptr;
    if (!ok(hipMalloc(&out, max_blocks * kThreads * sizeof(int)), "hipMalloc") ||
        !ok(hipMalloc(&ticks, max_blocks * 2 * sizeof(uint64_t)), "hipMalloc"))
        return 1;
    hipEvent_t e0, e1;
    if (!ok(hipEventCreate(&e0), "hipEventCreate") || !ok(hipEventCreate(&e1), "hipEventCreate"))
        return 1;
    std::printf("device %s, %d CUs; %d threads per workgroup; %d updates per lane per trip, %d trips\n",
                prop.gcnArchName, cus, kThreads, kRegs * kRounds, trips);
    std::printf("%-18s %10s %9s %14s %16s %12s\n", "form", "waves/SIMD", "ms", "lane-ops/s", "cycles/wave-instr",
                "clock (MHz)");
    std::vector<uint64_t> h(max_blocks * 2);
    for (int wps = 2; wps <= max_waves_per_simd; wps *= 2) {
        // one workgroup holds one wave per SIMD, so wps workgroups per CU give wps waves per SIMD
        const int blocks = cus * wps;
        for (int form = 0; form < kForms; ++form) {
            float best = 1e30f;
            double mhz = 0.0;
            for (int rep = 0; rep < 2; ++rep) {
                if (!ok(hipEventRecord(e0), "hipEventRecord"))
                    return 1;
                launch_form(form, blocks, out, ticks, trips);
                if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(e1), "hipEventRecord") ||
                    !ok(hipEventSynchronize(e1), "hipEventSynchronize"))
                    return 1;
                float ms = 0.f;
                if (!ok(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime") ||
                    !ok(hipMemcpy(h.data(), ticks, (size_t)blocks * 2 * sizeof(uint64_t), hipMemcpyDeviceToHost),
                        "hipMemcpy"))
                    return 1;
                if (ms < best) {
                    best = ms;
                    double c = 0.0, w = 0.0;
                    for (int b = 0; b < blocks; ++b) {
                        c += (double)h[2 * b];
                        w += (double)h[2 * b + 1];
                    }
                    mhz = w > 0 ? c / w * 100.0 : 0.0;  // s_memrealtime runs at 100 MHz
                }
            }
            const double instr_per_wave = (double)trips * kRounds * kRegs;
            const double cyc = best * 1e-3 * mhz * 1e6 / (instr_per_wave * wps);
            const double ops = (double)blocks * kThreads * trips * kRounds * kRegs * kElems[form];
            std::printf("%-18s %10d %9.2f %14.4e %16.3f %12.0f\n", kNames[form], wps, best, ops / (best * 1e-3),
                        cyc, mhz);
        }
    }
    (void)hipFree(out);
    (void)hipFree(ticks);
    return 0;
}
