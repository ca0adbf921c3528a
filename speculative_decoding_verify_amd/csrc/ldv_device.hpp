// Device helpers shared by the verify, commit, gather, read and selection
// kernels (gfx950).
//
// MFMA tile used throughout: v_mfma_f32_16x16x32_bf16.  For one wave (64
// lanes, g = lane / 16, c = lane % 16):
//   A operand (16 x 32): lane holds row c, eight k-slots 8g .. 8g+7
//   B operand (32 x 16): lane holds column c, the same eight k-slots
//   C/D (16 x 16, 4 VGPRs): lane holds column c, rows 4g .. 4g+3
// The k-slots of A and B are paired identically, so any fixed map from
// k-slot to the true contraction index, applied to both operands, gives the
// same product.  The map used here makes each lane's eight values two runs of
// four consecutive k (k0 = 32s + 4g and k0 + 16), so a wave reading 16 rows
// of an fp32 matrix touches 64 contiguous bytes per row per load.
//
// fp32 operands are carried as two bf16 terms, x = hi + lo with
// hi = bf16(x) and lo = bf16(x - hi) (both round-to-nearest-even); the pair
// holds x to about 2^-16 relative.  A bf16 operand times (hi + lo) in two
// MFMAs with fp32 accumulation keeps fp32-state products near fp32 accuracy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ldv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
// 16 raw bytes as a native vector: copies stay in registers (HIP's uint4 is
// a struct whose copies can be lowered to memcpy through private memory)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A pointer into global memory (address space 1): loads through it are
// global_load instructions, never flat ones (a pending flat load makes the
// compiler wait for every outstanding memory operation).
template <typename T>
using global_ptr = __attribute__((address_space(1))) T*;

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each

__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ unsigned short bf16_bits(float x) {
    __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(unsigned short, h);
}

__device__ __forceinline__ float bf16_val(unsigned short b) {
    return __uint_as_float(((unsigned)b) << 16);
}

// hi/lo bf16 split of four fp32 values.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// A packed bf16 pair held in a scalar register.  As an immediate, the
// multiplier (-1, 0) of split4 is encoded by the compiler as the inline
// constant -1.0, which the hardware applies to a packed bf16 operand as the
// fp32 pattern 0xBF800000, that is (0, -1); a value the compiler cannot see
// through keeps it in a register (the asm has no side effects, so it is
// shared and hoisted), and a scalar one costs no vector register.
__device__ __forceinline__ bf16x2 bf16x2_sreg(unsigned bits) {
    asm("" : "+s"(bits));
    return __builtin_bit_cast(bf16x2, bits);
}

// x = hi + lo with hi = x rounded to bf16 (nearest even) and lo = x - hi
// rounded the same way.  x - hi is exact (hi holds the top 8 of x's 24
// mantissa bits) and comes from one packed bf16 dot product per element,
// dot((-1, 0), (hi_0, hi_1)) + x_0, so hi is never unpacked: two VALU per
// element instead of three.  Checked bit for bit against the subtraction on
// MI355X over 4M values: identical for every |x| from 1e-30 to 1e30; 3 of the
// values outside that range differed (denormals, whose lo term is below
// 2^-126 in magnitude, or values near the largest float).
__device__ __forceinline__ void split4(const float4 x, u16x4& hi, u16x4& lo) {
    const bf16x2 nlo = bf16x2_sreg(0x0000BF80u), nhi = bf16x2_sreg(0xBF800000u);
    const bf16x2 h01 = {(__bf16)x.x, (__bf16)x.y}, h23 = {(__bf16)x.z, (__bf16)x.w};
    const bf16x2 l01 = {(__bf16)__builtin_amdgcn_fdot2_f32_bf16(nlo, h01, x.x, false),
                        (__bf16)__builtin_amdgcn_fdot2_f32_bf16(nhi, h01, x.y, false)};
    const bf16x2 l23 = {(__bf16)__builtin_amdgcn_fdot2_f32_bf16(nlo, h23, x.z, false),
                        (__bf16)__builtin_amdgcn_fdot2_f32_bf16(nhi, h23, x.w, false)};
    const u16x4 hb = __builtin_bit_cast(u16x4, __builtin_shufflevector(h01, h23, 0, 1, 2, 3));
    const u16x4 lb = __builtin_bit_cast(u16x4, __builtin_shufflevector(l01, l23, 0, 1, 2, 3));
    hi = hb;
    lo = lb;
}

__device__ __forceinline__ bf16x8 join(const u16x4 a, const u16x4 b) {
    u16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ u16x4 zero4() {
    u16x4 z = {0, 0, 0, 0};
    return z;
}

// hi/lo split of eight fp32 values (two runs of four) into MFMA operands.
__device__ __forceinline__ void split8(const float4 a, const float4 b, bf16x8& hi, bf16x8& lo) {
    u16x4 h0, l0, h1, l1;
    split4(a, h0, l0);
    split4(b, h1, l1);
    hi = join(h0, h1);
    lo = join(l0, l1);
}

// acc + A B for fp32 operands carried as hi + lo bf16 terms; the lo * lo term
// (about 2^-16 of the others) is dropped.
__device__ __forceinline__ floatx4 mma3(floatx4 acc, bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl) {
    acc = mfma16x16x32(ah, bh, acc);
    acc = mfma16x16x32(ah, bl, acc);
    return mfma16x16x32(al, bh, acc);
}

// Streaming accesses: data read or written exactly once per call (states,
// outputs).  Outputs go through non-temporal stores, which let HBM mix the
// write stream with the read stream at less loss.  Reads depend on their
// pattern:
//   - ld_nt, a non-temporal load, where each wave load covers whole
//     contiguous 128-byte lines (commit's state rows, the gather's state
//     rows before their LDS transpose, the logits): measured 7-13% faster
//     than ordinary loads on MI355X (commit 36.2 -> 33.7 us on the
//     27B-hybrid shape, 197.9 -> 175.3 us on batch-256);
//   - ld_stream, an ordinary load, where each load instruction covers 64-byte
//     halves of lines (state rows loaded straight into MFMA operand
//     registers): non-temporal loads measured no faster there in verify and
//     the in-block read, and 12% slower in a gather of that form.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld_stream(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ float4 ld_nt(const float* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<global_ptr<const f32x4>>((global_ptr<const float>)p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void st_stream(float* p, const float4 v) {
    const f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<global_ptr<f32x4>>((global_ptr<float>)p));
}

// Raw buffer views.  A view covers `bytes` bytes from a base address held in
// scalar registers; the memory unit range-checks every access against it,
// so loads at or past the end return zero and stores there are dropped.
// The draft-row loads and output stores use one view per (sequence, head)
// whose range ends at row T: rows past T then need no clamping, selects or
// branches, and each access costs only its 32-bit offset.  Offsets go in
// the vector operand (the scalar offset is left 0), and no access straddles
// the end of a view.
typedef __amdgpu_buffer_rsrc_t buf_t;
constexpr int kBufWord3 = 0x00020000;  // descriptor word 3 of a raw (untyped) gfx9 buffer
constexpr int kBufNT = 2;              // cache policy bits: non-temporal

__device__ __forceinline__ buf_t make_buf(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kBufWord3);
}
__device__ __forceinline__ u32x4 buf_ld128(buf_t b, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(b, off, 0, 0);
}
__device__ __forceinline__ float4 buf_ldf4(buf_t b, uint32_t off) {
    const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(b, off, 0, 0);
    return make_float4(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[2]), __uint_as_float(r[3]));
}
__device__ __forceinline__ float buf_ldf(buf_t b, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(b, off, 0, 0));
}
__device__ __forceinline__ unsigned short buf_ld16(buf_t b, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(b, off, 0, 0);
}
__device__ __forceinline__ void buf_st_stream(buf_t b, uint32_t off, const float4 v) {
    const f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), b, off, 0, kBufNT);
}

// Four consecutive output values at element `off` of `base`: fp32 (16 bytes)
// or bf16 rounded to nearest even (8 bytes), non-temporal either way.
__device__ __forceinline__ void st_stream_out4(void* base, int bf16, size_t off, const float4 v) {
    if (bf16) {
        const u16x4 w = {bf16_bits(v.x), bf16_bits(v.y), bf16_bits(v.z), bf16_bits(v.w)};
        __builtin_nontemporal_store(w, reinterpret_cast<global_ptr<u16x4>>(
                                           (global_ptr<unsigned short>)(static_cast<unsigned short*>(base) + off)));
    } else {
        st_stream(static_cast<float*>(base) + off, v);
    }
}

// Four bf16 values (8 bytes) from LDS or global memory.
__device__ __forceinline__ u16x4 load_u16x4(const unsigned short* p) {
    return *reinterpret_cast<const u16x4*>(p);
}

// A/B fragment of k-step s from a bf16 row of length D (row = &M[r][0]).
template <int D>
__device__ __forceinline__ bf16x8 frag_row(const unsigned short* row, int s, int g) {
    const int k0 = 32 * s + 4 * g;
    u16x4 c0 = (k0 < D) ? load_u16x4(row + k0) : zero4();
    u16x4 c1 = (k0 + 16 < D) ? load_u16x4(row + k0 + 16) : zero4();
    return join(c0, c1);
}

// Block index remap (the dispatcher places hardware block i on XCD i % 8,
// and each XCD has its own L2).  A unit is `per` consecutive logical blocks,
// e.g. the row blocks of one head: the blocks of a unit stay on one XCD (and
// share its L2), and consecutive units go to different XCDs, so that uneven
// units (heads with nothing to commit next to heads with long paths) spread
// over all eight XCDs.  Hardware block
// 8 t + x runs on XCD x and becomes block (t % per) of unit
// 8 (t / per) + x; the units past the last multiple of 8 keep their order.
// Blocks past the last whole group of 8 units (any remainder of the grid
// included) keep their order, so that the map is a bijection on the grid.
__host__ __device__ __forceinline__ unsigned xcd_spread(unsigned bid, unsigned units, unsigned per) {
    const unsigned full = (units / kXcds) * kXcds * per;  // blocks of the first 8 * (units / 8) units
    if (bid >= full) return bid;
    const unsigned x = bid % kXcds, t = bid / kXcds;
    return ((t / per) * kXcds + x) * per + t % per;
}

// Heads per spread unit in the per-head kernels (verify, commit, in-block
// read), which share one head-to-XCD map: units of two heads measured as
// fast as single heads on the 27B-hybrid, tree-64 and GDN-1.3B shapes and 6%
// faster for the batch-256 commit (longer contiguous runs of state per XCD).
constexpr unsigned kSpreadHeads = 2;

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
    unsigned lo = (unsigned)v, hi = (unsigned)(v >> 32);
    lo = __shfl(lo, src, kWave);
    hi = __shfl(hi, src, kWave);
    return ((uint64_t)hi << 32) | lo;
}

}  // namespace ldv
