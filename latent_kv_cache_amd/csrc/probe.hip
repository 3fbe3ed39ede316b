// Device peak probes for the path selector: achievable HBM read bandwidth and dense
// MFMA rate of the current device.
//
// Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
// Decoding", technical summary section 2 (Path selection): the runtime picks the
// decode path from the device's compute-to-bandwidth ratio (section 1 gives the
// ridges of the two devices it discusses).  These kernels measure the two
// quantities on the device at hand so the ratio is the measured one.
#include "common.h"
#include "launch.h"

namespace gqla {

namespace {

// Four 256-thread blocks per CU with four 16-byte loads in flight per lane read fastest
// of the shapes tried on MI355X (7.01 TB/s over 4 GiB; two 512-thread blocks with eight
// loads 6.86, 16 or more blocks per CU 6.0-6.5).
constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;       // 16-byte loads in flight per lane
constexpr int kReadBlocksPerCu = 4;

// Streams [base, base + n16 * 16) once, with nontemporal loads (the policy of the
// streaming decode kernel).  Block k reads its own contiguous span (the
// access pattern of the decode kernels, one chunk of one sequence per workgroup);
// lanes read 16 bytes each with kReadUnroll loads in flight.  The values only feed a
// comparison with a runtime value that never holds (never_lane = -1), so nothing is
// stored but the loads cannot be dropped.
__global__ __launch_bounds__(kReadThreads) void read_probe_kernel(const u32x4* __restrict__ base, size_t n16,
                                                                  uint32_t* __restrict__ sink, int never_lane) {
    uint32_t acc = 0;
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t lo = (size_t)blockIdx.x * per;
    const size_t hi = lo + per < n16 ? lo + per : n16;
    size_t i = lo + threadIdx.x;
    constexpr size_t step = (size_t)kReadThreads;
    for (; i + (kReadUnroll - 1) * step < hi; i += kReadUnroll * step) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int k = 0; k < kReadUnroll; ++k) v[k] = __builtin_nontemporal_load(base + i + k * step);
#pragma unroll
        for (int k = 0; k < kReadUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    for (; i < hi; i += step) {
        const u32x4 v = __builtin_nontemporal_load(base + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if ((int)threadIdx.x == never_lane && acc == 0x9e3779b9u) sink[0] = acc;
}

// Four independent 16x16x32 bf16 MFMA chains per wave.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ out) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (float)(threadIdx.x + e));
        b[e] = (__bf16)(0.5f);
    }
    floatx4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    for (int i = 0; i < iters; ++i) {
        c0 = mfma16(a, b, c0);
        c1 = mfma16(a, b, c1);
        c2 = mfma16(a, b, c2);
        c3 = mfma16(a, b, c3);
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = c0[0] + c1[1] + c2[2] + c3[3];
}

}  // namespace

hipError_t probe_read_bandwidth(const void* buf, size_t bytes, int cus, hipStream_t st, double* bytes_per_s) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    const size_t n16 = bytes / 16;
    double best = 0.0;
    for (int rep = 0; rep < 4 && e == hipSuccess; ++rep) {   // the first pass warms up
        e = hipEventRecord(e0, st);
        if (e != hipSuccess) break;
        hipLaunchKernelGGL(read_probe_kernel, dim3(kReadBlocksPerCu * cus), dim3(kReadThreads), 0, st,
                           (const u32x4*)buf, n16,
                           (uint32_t*)buf, -1);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipEventRecord(e1, st);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (e == hipSuccess && rep > 0 && ms > 0.f) best = std::max(best, (double)(n16 * 16) / (ms * 1e-3));
    }
    if (e0) hipEventDestroy(e0);
    if (e1) hipEventDestroy(e1);
    *bytes_per_s = best;
    return e;
}

hipError_t probe_mfma_rate(void* out, int cus, hipStream_t st, double* flops_per_s) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    const int blocks = 8 * cus;            // 32 waves per CU
    const int iters = 16384;             // about 4 ms: long enough for the clock to settle
    double best = 0.0;
    for (int rep = 0; rep < 4 && e == hipSuccess; ++rep) {
        e = hipEventRecord(e0, st);
        if (e != hipSuccess) break;
        hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, st, iters, (float*)out);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipEventRecord(e1, st);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        const double flops = (double)blocks * 4 /* waves */ * iters * 4 /* chains */ * 16.0 * 16.0 * 32.0 * 2.0;
        if (e == hipSuccess && rep > 0 && ms > 0.f) best = std::max(best, flops / (ms * 1e-3));
    }
    if (e0) hipEventDestroy(e0);
    if (e1) hipEventDestroy(e1);
    *flops_per_s = best;
    return e;
}

}  // namespace gqla
