// Throughput probes of the MI355X execution units and of HBM, for the roofline denominators: each kernel
// keeps every compute unit busy with independent instruction streams (no data dependence between the
// accumulators of a thread, no memory traffic in the loop), and the copy moves a buffer far larger than
// the caches. Built into its own library (libkqprobe.so), outside the solver's C ABI.
//
//   kind 0: fp64 vector FMA       (v_fma_f64, 8 independent chains per thread)
//   kind 1: fp64 matrix core      (v_mfma_f64_16x16x4_f64, 4 independent accumulators per wave)
//   kind 2: fp32 matrix core      (v_mfma_f32_16x16x4_f32, 4 independent accumulators per wave)
//   kind 3: bf16 matrix core      (v_mfma_f32_16x16x32_bf16, 4 independent accumulators per wave)
//   kind 4: fp32 vector FMA       (v_fma_f32, 8 independent chains per thread)
//   kind 5: HBM copy              (16-byte loads and stores over `bytes`)
//   kind 6: fp64 matrix core and vector FMA side by side (alternate waves; 4x the vector trips)
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef double d4p __attribute__((ext_vector_type(4)));
typedef float f4p __attribute__((ext_vector_type(4)));
typedef __bf16 b8p __attribute__((ext_vector_type(8)));

constexpr int PR_THREADS = 256;

__global__ __launch_bounds__(PR_THREADS) void probe_fma64(int iters, double seed, double* out) {
    double x[8];
#pragma unroll
    for (int c = 0; c < 8; c++) x[c] = seed + threadIdx.x + c;
    const double a = 1.0000000001, b = -1e-12;
    for (int it = 0; it < iters; it++)
#pragma unroll
        for (int c = 0; c < 8; c++) x[c] = fma(x[c], a, b);
    double s = 0.0;
#pragma unroll
    for (int c = 0; c < 8; c++) s += x[c];
    out[blockIdx.x * PR_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(PR_THREADS) void probe_fma32(int iters, float seed, float* out) {
    float x[8];
#pragma unroll
    for (int c = 0; c < 8; c++) x[c] = seed + threadIdx.x + c;
    const float a = 1.0000001f, b = -1e-7f;
    for (int it = 0; it < iters; it++)
#pragma unroll
        for (int c = 0; c < 8; c++) x[c] = fmaf(x[c], a, b);
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; c++) s += x[c];
    out[blockIdx.x * PR_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(PR_THREADS) void probe_mfma64(int iters, double seed, double* out) {
    d4p acc[4];
#pragma unroll
    for (int c = 0; c < 4; c++) acc[c] = d4p{seed, 0.0, 0.0, 0.0};
    const double a = 1e-3 * (threadIdx.x & 7), b = 1e-3;
    for (int it = 0; it < iters; it++)
#pragma unroll
        for (int c = 0; c < 4; c++) acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[c], 0, 0, 0);
    double s = 0.0;
#pragma unroll
    for (int c = 0; c < 4; c++) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[blockIdx.x * PR_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(PR_THREADS) void probe_mfma32(int iters, float seed, float* out) {
    f4p acc[4];
#pragma unroll
    for (int c = 0; c < 4; c++) acc[c] = f4p{seed, 0.0f, 0.0f, 0.0f};
    const float a = 1e-3f * (threadIdx.x & 7), b = 1e-3f;
    for (int it = 0; it < iters; it++)
#pragma unroll
        for (int c = 0; c < 4; c++) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; c++) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[blockIdx.x * PR_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(PR_THREADS) void probe_mfma_bf16(int iters, float seed, float* out) {
    f4p acc[4];
#pragma unroll
    for (int c = 0; c < 4; c++) acc[c] = f4p{seed, 0.0f, 0.0f, 0.0f};
    b8p a, b;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        a[e] = (__bf16)(0.001f * (float)((threadIdx.x + e) & 7));
        b[e] = (__bf16)0.001f;
    }
    for (int it = 0; it < iters; it++)
#pragma unroll
        for (int c = 0; c < 4; c++) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; c++) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[blockIdx.x * PR_THREADS + threadIdx.x] = s;
}

// Half of the waves of every work-group run the fp64 matrix-core loop, the other half the fp64 vector
// FMA loop: whether the two pipes add up when they share the compute units.
__global__ __launch_bounds__(PR_THREADS) void probe_mixed64(int iters, double seed, double* out) {
    const int wave = threadIdx.x >> 6;
    double s = 0.0;
    if (wave & 1) {
        double x[8];
#pragma unroll
        for (int c = 0; c < 8; c++) x[c] = seed + threadIdx.x + c;
        const double a = 1.0000000001, b = -1e-12;
        for (int it = 0; it < 4 * iters; it++)
#pragma unroll
            for (int c = 0; c < 8; c++) x[c] = fma(x[c], a, b);
#pragma unroll
        for (int c = 0; c < 8; c++) s += x[c];
    } else {
        d4p acc[4];
#pragma unroll
        for (int c = 0; c < 4; c++) acc[c] = d4p{seed, 0.0, 0.0, 0.0};
        const double a = 1e-3 * (threadIdx.x & 7), b = 1e-3;
        for (int it = 0; it < iters; it++)
#pragma unroll
            for (int c = 0; c < 4; c++) acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < 4; c++) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    }
    out[blockIdx.x * PR_THREADS + threadIdx.x] = s;
}

struct alignas(16) P16 {
    uint32_t w[4];
};

__global__ __launch_bounds__(PR_THREADS) void probe_copy(const P16* __restrict__ src, P16* __restrict__ dst, int64_t n) {
    for (int64_t e = blockIdx.x * (int64_t)PR_THREADS + threadIdx.x; e < n; e += (int64_t)gridDim.x * PR_THREADS)
        dst[e] = src[e];
}

// Runs probe `kind` once to warm up and once timed; *seconds = the timed kernel's duration (HIP events),
// *work = its FLOP (kinds 0-4) or bytes moved (kind 5, read + written). `iters`: loop trips per thread
// (kinds 0-4); `bytes`: buffer size (kind 5, a multiple of 16). Device buffers are the caller's:
// scratch (>= 4 * 256 * 256 * 8 bytes) for the compute kinds, src and dst (bytes each) for the copy.
// Returns 0, or a HIP error code.
extern "C" int kq_probe_run(int kind, int iters, int64_t bytes, void* scratch, void* src, void* dst, double* seconds,
                            double* work) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
    const unsigned blocks = (unsigned)(cus * 4);
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
    double flop_per_trip = 0;  // per thread
    auto launch = [&]() {
        switch (kind) {
            case 0: hipLaunchKernelGGL(probe_fma64, dim3(blocks), dim3(PR_THREADS), 0, 0, iters, 1.0, (double*)scratch); break;
            case 1: hipLaunchKernelGGL(probe_mfma64, dim3(blocks), dim3(PR_THREADS), 0, 0, iters, 1.0, (double*)scratch); break;
            case 2: hipLaunchKernelGGL(probe_mfma32, dim3(blocks), dim3(PR_THREADS), 0, 0, iters, 1.0f, (float*)scratch); break;
            case 3: hipLaunchKernelGGL(probe_mfma_bf16, dim3(blocks), dim3(PR_THREADS), 0, 0, iters, 1.0f, (float*)scratch); break;
            case 4: hipLaunchKernelGGL(probe_fma32, dim3(blocks), dim3(PR_THREADS), 0, 0, iters, 1.0f, (float*)scratch); break;
            case 6: hipLaunchKernelGGL(probe_mixed64, dim3(blocks), dim3(PR_THREADS), 0, 0, iters, 1.0, (double*)scratch); break;
            default: hipLaunchKernelGGL(probe_copy, dim3(blocks * 8), dim3(PR_THREADS), 0, 0, (const P16*)src, (P16*)dst,
                                        bytes / 16); break;
        }
    };
    // FLOP per thread and trip: vector FMA 8 chains x 2; a 16x16xK MFMA is 2 * 16 * 16 * K per wave of 64,
    // four per trip
    switch (kind) {
        case 0: case 4: flop_per_trip = 16.0; break;
        case 1: case 2: flop_per_trip = 4.0 * 2 * 16 * 16 * 4 / 64.0; break;
        case 3: flop_per_trip = 4.0 * 2 * 16 * 16 * 32 / 64.0; break;
        case 6: flop_per_trip = 0.5 * (4.0 * 2 * 16 * 16 * 4 / 64.0) + 0.5 * 4 * 16.0; break;  // per thread, averaged
        default: break;
    }
    launch();
    if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) return 2;
    if (kind == 6) flop_per_trip = 0.5 * (4.0 * 2 * 16 * 16 * 4 / 64.0) + 0.5 * 4 * 16.0;
    hipEventRecord(e0, 0);
    launch();
    hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess) return 3;
    float ms = 0.0f;
    hipEventElapsedTime(&ms, e0, e1);
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    *seconds = ms / 1e3;
    *work = kind == 5 ? 2.0 * (double)(bytes / 16 * 16) : flop_per_trip * iters * (double)blocks * PR_THREADS;
    return 0;
}
