// Device helpers of the library run on caller data, for the tests only (not
// part of the ldv ABI; built into its own library, libldv_checks.so).
//
// ldv_check_split: the fp32 -> bf16 hi + lo split (split4 in ldv_device.hpp)
// that every MFMA product with an fp32 operand uses, applied to n values so
// that a test can compare it bit for bit with its definition.
#include <stdint.h>

#include "ldv_device.hpp"

namespace {

__global__ __launch_bounds__(256) void split_kernel(const float4* x, unsigned short* hi, unsigned short* lo,
                                                    long long n4) {
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n4) return;
    ldv::u16x4 h, l;
    ldv::split4(x[t], h, l);
    *reinterpret_cast<ldv::u16x4*>(hi + 4 * t) = h;
    *reinterpret_cast<ldv::u16x4*>(lo + 4 * t) = l;
}

}  // namespace

// x: n fp32 values (device, 16-byte aligned, n a multiple of 4); hi, lo: n
// bf16 bit patterns each (device, 8-byte aligned).  Returns 0, or -1 for bad
// arguments, or the HIP error of the launch.
extern "C" __attribute__((visibility("default"))) int ldv_check_split(const float* x, unsigned short* hi,
                                                                      unsigned short* lo, long long n,
                                                                      void* stream) {
    if (n < 0 || n % 4 || (n > 0 && (!x || !hi || !lo))) return -1;
    if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(hi) & 7) ||
        (reinterpret_cast<uintptr_t>(lo) & 7))
        return -1;
    const long long n4 = n / 4;
    if (n4 == 0) return 0;
    const long long blocks = (n4 + 255) / 256;
    if (blocks > 0x7fffffffLL) return -1;
    hipLaunchKernelGGL(split_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<const float4*>(x), hi, lo, n4);
    return (int)hipGetLastError();
}
