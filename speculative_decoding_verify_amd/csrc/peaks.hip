// Achievable MFMA rate on this GPU, for the measurement harness only (not
// part of the ldv ABI; built into its own library, libldv_peaks.so).
//
// Every wave runs kIters rounds of eight independent accumulation chains of
// v_mfma_f32_16x16x32_bf16 (the instruction every kernel of the library
// uses), so the matrix pipe never waits on a result.  Each lane then writes
// one value derived from all eight accumulators, so nothing is dead code.
// The round count is a compile-time constant: with a run-time count the
// compiler rotates the accumulators through copies every round.
// Flops per launch: blocks * 4 waves * kIters * 8 * (2 * 16 * 16 * 32).
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // four waves: one per SIMD of a CU
constexpr int kChains = 8;
constexpr int kIters = 2000;

__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(float seed, float* out) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
        b[i] = (__bf16)(seed * (float)(i - (int)threadIdx.x));
    }
    floatx4 acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < kIters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

// Enqueue one launch of `blocks` workgroups (out: blocks * 256 floats).
// Returns 0, or the HIP error code of the launch.
extern "C" __attribute__((visibility("default"))) int ldv_peak_mfma(int blocks, float* out, void* stream) {
    if (blocks <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       1e-3f, out);
    return (int)hipGetLastError();
}

// Floating-point operations of one launch.
extern "C" __attribute__((visibility("default"))) double ldv_peak_mfma_flops(int blocks) {
    return (double)blocks * (kThreads / 64) * kIters * kChains * (2.0 * 16 * 16 * 32);
}
