// Batched state reads at chosen positions (gfx950).
//
// ReaDy page (arXiv 2610.20503): the drafter combines target features with
// position-specific reads from committed recurrent states (Fig. 2a); the
// state reader gathers the states directly, without an intermediate tensor
// (Fig. 3), which is what cut its state-gathering latency (Fig. 4).  Here:
//   s = slot[b, p];  o[b, p, h, i, :] = pool[s, h] q_i  for i < Qn;
//   states_out[b, p, h] = pool[s, h]  (optional bit copy).
//
// One block of four waves per 64 rows of a (sequence, position, head) state
// (two blocks per state at d = 128: small blocks keep more loads in flight
// per CU).  Each wave's 16 rows of the fp32 state are 8 KiB of consecutive
// bytes at d = 128; the wave reads them with non-temporal loads of which
// each covers 1 KiB (whole 128-byte lines), writes the optional copy from the
// same registers, and passes them through LDS into the MFMA operand layout
// (lane (c, g) holds row c).  Loading the operands straight from memory, as
// before, made every load instruction cover only 64-byte halves of lines:
// measured 119.1 us against 103.1 us now on the 27B-hybrid shape (106.4 us
// with ordinary loads in the new form).  o = S q is formed on MFMA with the
// state split into bf16 hi + lo terms; the o tile of the block goes through
// LDS, so that every store instruction writes whole rows of o (measured 5%
// faster for bf16 outputs, 1.5% for fp32).  The read of the 64 KiB state
// dominates: the kernel is bound by HBM.
#include "ldv_device.hpp"
#include "ldv_kernels.hpp"

#include "../../include/ldv.h"

namespace ldv {

template <int D>
struct GShape {
    static constexpr int MBT = D / 16;             // 16-row blocks per state
    static constexpr int NWA = MBT < 4 ? MBT : 4;  // waves per block
    static constexpr int MBW = 1;                  // 16-row blocks per wave
    static constexpr int NSPLIT = MBT / (NWA * MBW);  // blocks per (sequence, position, head)
    static constexpr int KS = (D + 31) / 32;       // MFMA k-steps
};

template <int D, bool F32Q>
__global__ __launch_bounds__((GShape<D>::NWA * kWave)) void gather_kernel(const GatherArgs p) {
    using S = GShape<D>;
    constexpr int NWA = S::NWA, KS = S::KS;
    constexpr int RB = NWA * 16;        // state rows per block
    constexpr int SP = D + 4;           // padded LDS row of the state tile (floats)
    constexpr int NL = 16 * D / 4 / kWave > 0 ? 16 * D / 4 / kWave : 1;  // float4 per lane of a wave's 16 rows
    __shared__ __align__(16) float s_st[NWA][16 * SP];  // each wave's 16 state rows
    __shared__ __align__(16) float s_o[16][RB + 4];     // padded: the 16 query rows start on different banks
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int H = p.H;
    // (sequence, position, head) units spread over the XCDs, the blocks of a
    // unit together (they share its queries): measured faster than
    // contiguous ranges of units per XCD
    const unsigned bid = xcd_spread(blockIdx.x, gridDim.x / S::NSPLIT, S::NSPLIT);
    const int part = (int)(bid % S::NSPLIT);  // which 16 * NWA rows of the state
    const int h = (int)((bid / S::NSPLIT) % H);
    const size_t bp = bid / S::NSPLIT / H;  // b * P + p

    const int s = p.slot[bp];
    if (s < 0 || s >= p.num_slots) {
        if (tid == 0 && p.status && h == 0 && part == 0) atomicOr(p.status, LDV_STATUS_BAD_SLOT);
        return;
    }
    const size_t row0 = (size_t)(part * NWA + wave) * 16;  // the wave's first state row
    const float* src = p.pool + ((size_t)s * H + h) * D * D + row0 * D;
    const bool reads = p.queries && p.o.base && p.Qn > 0;
    const size_t qo_base = ((size_t)bp * H + h) * (size_t)p.Qn;           // queries row of query 0
    const size_t o_base = bp * p.o.ld + p.o.col + (size_t)h * p.Qn * D;  // o element of query 0

    // queries of the first 16-column block (the common case is Qn <= 16)
    // before the state, so that waiting for them leaves the state in flight.
    // The loads are unconditional per lane (row clamped into range); lanes
    // past Qn drop their values when the operand is formed.
    u16x4 qc[KS][2];
    float4 qf[KS][2];
    if (reads) {
        const size_t qrow = (qo_base + min(c, p.Qn - 1)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k0 = 32 * ks + 4 * g;
            if constexpr (F32Q) {
                const float* qr = static_cast<const float*>(p.queries) + qrow;
                if (k0 < D) qf[ks][0] = *reinterpret_cast<const float4*>(qr + k0);
                if (k0 + 16 < D) qf[ks][1] = *reinterpret_cast<const float4*>(qr + k0 + 16);
            } else {
                const unsigned short* qr = static_cast<const unsigned short*>(p.queries) + qrow;
                if (k0 < D) qc[ks][0] = load_u16x4(qr + k0);
                if (k0 + 16 < D) qc[ks][1] = load_u16x4(qr + k0 + 16);
            }
        }
    }
    // the wave's 16 rows are 16 * D consecutive floats: each load instruction
    // covers 1 KiB of them (whole lines), read non-temporally
    float4 v[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e = 4 * (lane + kWave * i);
        if (16 * D >= 4 * kWave || e < 16 * D) v[i] = ld_nt(src + e);
    }
    asm volatile("" ::: "memory");  // keep the loads above ahead of any use of them
    if (p.states_out) {  // the bit copy, from the same registers, whole lines per store
        float* dst = p.states_out + ((size_t)bp * H + h) * D * D + row0 * D;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int e = 4 * (lane + kWave * i);
            if (16 * D >= 4 * kWave || e < 16 * D) st_stream(dst + e, v[i]);
        }
    }
    if (!reads) return;
    // through LDS into the MFMA operand layout: lane (c, g) takes row c
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e = 4 * (lane + kWave * i);
        if (16 * D >= 4 * kWave || e < 16 * D)
            *reinterpret_cast<float4*>(&s_st[wave][(e / D) * SP + e % D]) = v[i];
    }
    __syncthreads();
    float4 st[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int k0 = 32 * ks + 4 * g;
        st[ks][0] = (k0 < D) ? *reinterpret_cast<const float4*>(&s_st[wave][c * SP + k0]) : make_float4(0.f, 0.f, 0.f, 0.f);
        st[ks][1] = (k0 + 16 < D) ? *reinterpret_cast<const float4*>(&s_st[wave][c * SP + k0 + 16])
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    for (int nb = 0; nb * 16 < p.Qn; ++nb) {
        const int col = nb * 16 + c;  // query index held by this lane
        const bool cval = col < p.Qn;
        if (nb > 0) {  // later 16-query blocks (Qn > 16)
            const size_t qrow = (qo_base + min(col, p.Qn - 1)) * D;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int k0 = 32 * ks + 4 * g;
                if constexpr (F32Q) {
                    const float* qr = static_cast<const float*>(p.queries) + qrow;
                    if (k0 < D) qf[ks][0] = *reinterpret_cast<const float4*>(qr + k0);
                    if (k0 + 16 < D) qf[ks][1] = *reinterpret_cast<const float4*>(qr + k0 + 16);
                } else {
                    const unsigned short* qr = static_cast<const unsigned short*>(p.queries) + qrow;
                    if (k0 < D) qc[ks][0] = load_u16x4(qr + k0);
                    if (k0 + 16 < D) qc[ks][1] = load_u16x4(qr + k0 + 16);
                }
            }
        }
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k0 = 32 * ks + 4 * g;
            bf16x8 bq, bql;
            if constexpr (F32Q) {
                const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                u16x4 h0, l0, h1, l1;
                split4((cval && k0 < D) ? qf[ks][0] : z, h0, l0);
                split4((cval && k0 + 16 < D) ? qf[ks][1] : z, h1, l1);
                bq = join(h0, h1);
                bql = join(l0, l1);
            } else {
                bq = join((cval && k0 < D) ? qc[ks][0] : zero4(), (cval && k0 + 16 < D) ? qc[ks][1] : zero4());
            }
            u16x4 h0, l0, h1, l1;
            split4(st[ks][0], h0, l0);
            split4(st[ks][1], h1, l1);
            const bf16x8 ah = join(h0, h1), al = join(l0, l1);
            acc = mfma16x16x32(ah, bq, acc);
            acc = mfma16x16x32(al, bq, acc);
            if constexpr (F32Q) acc = mfma16x16x32(ah, bql, acc);
        }
        // the block's o tile (16 queries x RB rows) goes through LDS, so that
        // each store instruction covers whole rows of o: 16 consecutive lanes
        // write one query's RB values
        __syncthreads();  // the previous query block's tile has been stored
        {
            const int r0 = wave * 16 + 4 * g;
            *reinterpret_cast<float4*>(&s_o[c][r0]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        __syncthreads();
        for (int j = tid; j < 16 * (RB / 4); j += NWA * kWave) {
            const int qi = j / (RB / 4), r4 = (j % (RB / 4)) * 4;
            if (nb * 16 + qi < p.Qn)
                st_stream_out4(p.o.base, p.o.bf16, o_base + (size_t)(nb * 16 + qi) * D + part * RB + r4,
                               *reinterpret_cast<const float4*>(&s_o[qi][r4]));
        }
    }
}

template <int D, bool F32Q>
static hipError_t launch_t(const GatherArgs& a, hipStream_t st) {
    const long long nblk = (long long)a.B * a.P * a.H * GShape<D>::NSPLIT;
    if (nblk <= 0) return hipSuccess;
    hipLaunchKernelGGL((gather_kernel<D, F32Q>), dim3((unsigned)nblk), dim3(GShape<D>::NWA * kWave), 0, st, a);
    return hipGetLastError();
}

template <bool F32Q>
static hipError_t launch_f(const GatherArgs& a, hipStream_t st) {
    switch (a.D) {
        case 16: return launch_t<16, F32Q>(a, st);
        case 32: return launch_t<32, F32Q>(a, st);
        case 64: return launch_t<64, F32Q>(a, st);
        case 128: return launch_t<128, F32Q>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gather(const GatherArgs& a, bool f32_queries, hipStream_t stream) {
    return f32_queries ? launch_f<true>(a, stream) : launch_f<false>(a, stream);
}

}  // namespace ldv
