// Achievable rates on this GPU, for the measurement harness only (not part of
// the ldv ABI; built into its own library, libldv_peaks.so).
//
// MFMA: every wave runs kIters rounds of eight independent accumulation
// chains of v_mfma_f32_16x16x32_bf16 (the instruction every kernel of the
// library uses), so the matrix pipe never waits on a result.  Each lane then
// writes one value derived from all eight accumulators, so nothing is dead
// code.  The round count is a compile-time constant: with a run-time count
// the compiler rotates the accumulators through copies every round.
// Flops per launch: blocks * 4 waves * kIters * 8 * (2 * 16 * 16 * 32).
//
// HBM streams: grid-stride kernels over a buffer of float4 in the read/write
// mixes of the library's kernels: reads only (the selection's logits), one
// write per read (commit: a state in, a state out, in place or not), and one
// write per two, four or eight reads (verify, the gathers and the in-block
// reads write less than they read), each with 2, 4 or 8 loads in flight per
// thread.  Each kernel of the library is graded against the best rate
// measured at its own read:write ratio or a more write-heavy one.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Stream probes: each thread keeps L 16-byte non-temporal loads in flight
// per step (2, 4 or 8; non-temporal loads measured fastest on MI355X: 7.1-7.2
// TB/s for reads alone against about 6.0 TB/s with ordinary loads) and
// writes, with non-temporal stores, one float4 per R float4 read (their sum,
// so the loads are live); R = 0 reads only and writes one float4 per thread
// at the end.  A block step covers L * 256 consecutive float4, each wave load
// 1 KiB of consecutive bytes.  Step w writes its sums at float4
// w * (L / R) * 256 + ..., so with R = 1 and dst == src every float4 is
// rewritten in place right after it is read.
constexpr int kMaxLoads = 8;

// With `spread` (a grid of one block per step), the steps are grouped in
// units of 128 KiB (two heads' states at d = 128) and consecutive units go to
// different XCDs, the steps of a unit staying on one XCD (hardware block i
// runs on XCD i % 8): the block-to-data map of the library's per-head
// kernels.  Blocks past the last whole group of 8 units keep their step.
template <int R, int L>
__global__ __launch_bounds__(kThreads) void stream_kernel(const floatx4* src, floatx4* dst, size_t n, int spread) {
    static_assert(R == 0 || L % R == 0, "R divides L");
    constexpr int W = R > 0 ? L / R : 0;  // float4 written per thread and step
    const size_t per_block = (size_t)L * kThreads;
    const size_t nsteps = n / per_block;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    size_t w0 = blockIdx.x;
    if (spread) {
        constexpr size_t per = 32 / L;  // steps per 128 KiB unit
        const size_t full = (nsteps / per / 8) * 8 * per;
        if (w0 < full) {
            const size_t x = w0 % 8, t = w0 / 8;
            w0 = ((t / per) * 8 + x) * per + t % per;
        }
    }
    for (size_t w = w0; w < nsteps; w += gridDim.x) {
        const size_t base = w * per_block + threadIdx.x;
        floatx4 v[L];
#pragma unroll
        for (int i = 0; i < L; ++i) v[i] = __builtin_nontemporal_load(src + base + (size_t)i * kThreads);
        if constexpr (R == 0) {
#pragma unroll
            for (int i = 0; i < L; ++i) acc += v[i];
        } else {
#pragma unroll
            for (int j = 0; j < W; ++j) {
                floatx4 s = v[j * R];
#pragma unroll
                for (int i = 1; i < R; ++i) s += v[j * R + i];
                __builtin_nontemporal_store(s, dst + w * (size_t)W * kThreads + (size_t)j * kThreads + threadIdx.x);
            }
        }
    }
    if constexpr (R == 0) dst[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

#define PEAKS_EXPORT extern "C" __attribute__((visibility("default")))

// Enqueue one launch of `blocks` workgroups (out: blocks * 256 floats).
// Returns 0, or the HIP error code of the launch.
PEAKS_EXPORT int ldv_peak_mfma(int blocks, float* out, void* stream) {
    if (blocks <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       1e-3f, out);
    return (int)hipGetLastError();
}

// Floating-point operations of one launch.
PEAKS_EXPORT double ldv_peak_mfma_flops(int blocks) {
    return (double)blocks * (kThreads / 64) * kIters * kChains * (2.0 * 16 * 16 * 32);
}

// Float4 granule of the stream probes: n4 must be a multiple of it.
PEAKS_EXPORT long long ldv_peak_stream_granule(void) { return (long long)kMaxLoads * kThreads; }

// One launch of the stream probe reading n4 float4 of src with `loads`
// (2, 4 or 8) loads in flight per thread and writing one float4 per `ratio`
// read (ratio 1, 2, 4 or 8, at most `loads`; 0 = reads only).  dst holds at
// least n4 / ratio float4 (ratio 0: blocks * 256 float4); dst == src with
// ratio 1 rewrites src in place.  spread != 0 maps steps to XCDs as above
// (only on a grid of one block per step).  Returns 0 or a HIP error code (an invalid
// size, ratio, load count or pointer gives hipErrorInvalidValue before any
// launch).
PEAKS_EXPORT int ldv_peak_stream(int ratio, int loads, const void* src, void* dst, long long n4, int blocks,
                                 int spread, void* stream) {
    if (!src || !dst || blocks <= 0 || n4 <= 0 || n4 % ldv_peak_stream_granule() != 0) return (int)hipErrorInvalidValue;
    // the spread map is meant for a grid of one block per step
    if (spread && (loads <= 0 || n4 / ((long long)loads * kThreads) != blocks)) return (int)hipErrorInvalidValue;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const floatx4* s = static_cast<const floatx4*>(src);
    floatx4* d = static_cast<floatx4*>(dst);
    const dim3 g((unsigned)blocks), b(kThreads);
#define PEAKS_CASE(R, L) \
    if (ratio == R && loads == L) { \
        hipLaunchKernelGGL((stream_kernel<R, L>), g, b, 0, st, s, d, (size_t)n4, spread); \
        return (int)hipGetLastError(); \
    }
    PEAKS_CASE(0, 2) PEAKS_CASE(0, 4) PEAKS_CASE(0, 8)
    PEAKS_CASE(1, 2) PEAKS_CASE(1, 4) PEAKS_CASE(1, 8)
    PEAKS_CASE(2, 2) PEAKS_CASE(2, 4) PEAKS_CASE(2, 8)
    PEAKS_CASE(4, 4) PEAKS_CASE(4, 8)
    PEAKS_CASE(8, 8)
#undef PEAKS_CASE
    return (int)hipErrorInvalidValue;
}
