// Parallel verification of a draft chain or tree through a gated-delta-rule
// layer, all nodes at once from the committed state (gfx950).
//
// Closed form (Bole page, arXiv 2608.01651, section IV, Eq. (2)), written in
// the o = S q orientation (S_pre of the page is S0 transposed):
//   P_n   = prod of a over the root-to-n path          (D_P)
//   B0    = D_P (Q S0^T)                               (Eq. (7), B0)
//   R     = D_beta (V - D_P (K S0^T))                  (Eq. (7), R)
//   U     = (I + G)^{-1} R                             (Eq. (7), U)
//   O     = B0 + C U                                   (Eq. (7), O)
// with, for m on the root-to-n path (the page only says G and C depend on
// the topology, Q/K and the gates; these follow from unrolling the
// recurrence):
//   C[n, m] = (P_n / P_m) q_n . k_m        (m = n included)
//   G[n, m] = beta_n (P_n / P_m) k_n . k_m (m a strict ancestor)
// G is strictly lower in topological order, so (I + G) U = R is solved by
// substitution; nodes of equal depth are independent, so the solve runs
// level by level (at most 8 levels for the draft trees, T for a chain).
//
// One workgroup per (sequence, head, value tile of BV columns): G and C do
// not depend on the value channel (Eq. (7) context), so value tiles are
// independent.  Per block:
//   1. issue the loads of its BV x D slice of S0 (fp32) straight into the
//      registers of the MFMA B operand;
//   2. stage Q, K (bf16) and the V tile in LDS; wave 0 turns the parent row
//      into ancestor masks, depths and log P by pointer doubling;
//   3. Q K^T and K K^T (MFMA), masked and decay-scaled into C and G in LDS;
//   4. Q S0^T and K S0^T on MFMA, S0 split into bf16 hi + lo terms;
//   5. B0 and R into LDS, then the level-by-level solve for U and O, with
//      one wave per node and one lane per value column.
// P_n / P_m is evaluated as exp(log P_n - log P_m), only for ancestor pairs
// (so the exponent is <= 0 for gates in [0, 1]); log a is clamped at -87 so
// that a zero gate gives a finite log.
#include "ldv_device.hpp"
#include "ldv_kernels.hpp"

#include "../../include/ldv.h"

namespace ldv {

template <int D>
struct VShape {
    static constexpr int BV = D >= 64 ? 64 : D;  // value columns per block
    static constexpr int NT = D / BV;            // value tiles per head
    static constexpr int NW = BV / 16;           // waves per block
    static constexpr int KS = (D + 31) / 32;     // MFMA k-steps over d_k
    static constexpr int QKLD = D + 8;           // bf16 row stride of Q/K in LDS
    static constexpr int BRLD = BV + 4;          // fp32 row stride of B0/R in LDS
};

template <int D, int TM, bool F32IN>
struct VLds {
    using S = VShape<D>;
    static constexpr int NPLANE = F32IN ? 4 : 2;  // q, k (hi and lo for fp32 input)
    static constexpr size_t qk = (size_t)NPLANE * TM * S::QKLD * 2;
    static constexpr size_t br = (size_t)2 * TM * S::BRLD * 4;
    static constexpr size_t regionA = ((qk > br ? qk : br) + 15) / 16 * 16;
    static constexpr size_t gc = (size_t)TM * TM * 8;
    static constexpr size_t vt = ((size_t)TM * S::BV * (F32IN ? 4 : 2) + 15) / 16 * 16;
    static constexpr size_t off_gc = regionA;
    static constexpr size_t off_v = off_gc + gc;
    static constexpr size_t off_anc = off_v + vt;          // uint64 [TM]
    static constexpr size_t off_lvl = off_anc + 8 * TM;    // uint64 [TM + 1]
    static constexpr size_t off_f = off_lvl + 8 * (TM + 8);  // float logp, P, beta [TM] each
    static constexpr size_t off_i = off_f + 12 * TM;        // int maxdep, bad
    static constexpr size_t total = off_i + 16;
};

template <int D, int TM, bool F32IN>
__global__ __launch_bounds__(VShape<D>::NW * kWave) void verify_kernel(const VerifyArgs p) {
    using S = VShape<D>;
    using L = VLds<D, TM, F32IN>;
    constexpr int BV = S::BV, NW = S::NW, KS = S::KS, QKLD = S::QKLD, BRLD = S::BRLD;
    constexpr int NTHR = NW * kWave;
    constexpr int MBMAX = TM / 16;

    __shared__ __align__(16) unsigned char smem[L::total];
    unsigned short* s_q = reinterpret_cast<unsigned short*>(smem);
    unsigned short* s_k = s_q + TM * QKLD;
    unsigned short* s_qlo = s_k + TM * QKLD;  // fp32 input only
    unsigned short* s_klo = s_qlo + TM * QKLD;
    float* s_b0 = reinterpret_cast<float*>(smem);  // aliases Q/K after the products
    float* s_r = s_b0 + TM * BRLD;                 // R, then U in place
    float2* s_gc = reinterpret_cast<float2*>(smem + L::off_gc);  // (G, C)[n][m]
    void* s_v = smem + L::off_v;
    uint64_t* s_anc = reinterpret_cast<uint64_t*>(smem + L::off_anc);
    uint64_t* s_lvl = reinterpret_cast<uint64_t*>(smem + L::off_lvl);
    float* s_logp = reinterpret_cast<float*>(smem + L::off_f);
    float* s_P = s_logp + TM;
    float* s_beta = s_P + TM;
    int* s_int = reinterpret_cast<int*>(smem + L::off_i);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int T = p.T, H = p.H;
    const unsigned bid = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = (int)(bid % S::NT);
    const int bh = (int)(bid / S::NT);
    const int h = bh % H, b = bh / H;
    const int NB = (T + 15) >> 4;  // 16-node blocks in use
    const int T16 = NB * 16;

    // 1. this lane's S0 row (one MFMA B-operand column) for every k-step
    const int jl = wave * 16 + c;  // column within the value tile
    const float* s0row = p.S0 + (((size_t)b * H + h) * D + (size_t)tile * BV + jl) * D;
    float4 sreg[KS][2];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int k0 = 32 * s + 4 * g;
        sreg[s][0] = (k0 < D) ? *reinterpret_cast<const float4*>(s0row + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
        sreg[s][1] = (k0 + 16 < D) ? *reinterpret_cast<const float4*>(s0row + k0 + 16)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // 2a. Q, K rows into LDS (rows T .. T16-1 zero)
    if constexpr (!F32IN) {
        constexpr int CPR = D / 8;  // 16-byte chunks per row
        const unsigned short* qg = static_cast<const unsigned short*>(p.q);
        const unsigned short* kg = static_cast<const unsigned short*>(p.k);
        for (int ch = tid; ch < T16 * CPR; ch += NTHR) {
            const int row = ch / CPR, col = (ch % CPR) * 8;
            uint4 qv = make_uint4(0, 0, 0, 0), kv = qv;
            if (row < T) {
                const size_t off = (((size_t)b * T + row) * H + h) * D + col;
                qv = *reinterpret_cast<const uint4*>(qg + off);
                kv = *reinterpret_cast<const uint4*>(kg + off);
            }
            *reinterpret_cast<uint4*>(s_q + row * QKLD + col) = qv;
            *reinterpret_cast<uint4*>(s_k + row * QKLD + col) = kv;
        }
        constexpr int VPR = BV / 8;
        const unsigned short* vg = static_cast<const unsigned short*>(p.v);
        unsigned short* sv = static_cast<unsigned short*>(s_v);
        for (int ch = tid; ch < T * VPR; ch += NTHR) {
            const int row = ch / VPR, col = (ch % VPR) * 8;
            const size_t off = (((size_t)b * T + row) * H + h) * D + (size_t)tile * BV + col;
            *reinterpret_cast<uint4*>(sv + row * BV + col) = *reinterpret_cast<const uint4*>(vg + off);
        }
    } else {
        constexpr int CPR = D / 4;
        const float* qg = static_cast<const float*>(p.q);
        const float* kg = static_cast<const float*>(p.k);
        for (int ch = tid; ch < T16 * CPR; ch += NTHR) {
            const int row = ch / CPR, col = (ch % CPR) * 4;
            float4 qv = make_float4(0.f, 0.f, 0.f, 0.f), kv = qv;
            if (row < T) {
                const size_t off = (((size_t)b * T + row) * H + h) * D + col;
                qv = *reinterpret_cast<const float4*>(qg + off);
                kv = *reinterpret_cast<const float4*>(kg + off);
            }
            u16x4 hi, lo;
            split4(qv, hi, lo);
            *reinterpret_cast<u16x4*>(s_q + row * QKLD + col) = hi;
            *reinterpret_cast<u16x4*>(s_qlo + row * QKLD + col) = lo;
            split4(kv, hi, lo);
            *reinterpret_cast<u16x4*>(s_k + row * QKLD + col) = hi;
            *reinterpret_cast<u16x4*>(s_klo + row * QKLD + col) = lo;
        }
        constexpr int VPR = BV / 4;
        const float* vg = static_cast<const float*>(p.v);
        float* sv = static_cast<float*>(s_v);
        for (int ch = tid; ch < T * VPR; ch += NTHR) {
            const int row = ch / VPR, col = (ch % VPR) * 4;
            const size_t off = (((size_t)b * T + row) * H + h) * D + (size_t)tile * BV + col;
            *reinterpret_cast<float4*>(sv + row * BV + col) = *reinterpret_cast<const float4*>(vg + off);
        }
    }

    // 2b. topology: lane n of wave 0 is node n
    if (wave == 0) {
        const int n = lane;
        const bool valid = n < T;
        int par = -1;
        float la = 0.f, be = 0.f;
        if (valid) {
            par = p.parent ? p.parent[(size_t)b * T + n] : n - 1;
            const size_t gi = ((size_t)b * T + n) * H + h;
            la = fmaxf(logf(p.a[gi]), -87.f);
            be = p.beta[gi];
        }
        const bool bad = valid && (par < -1 || par >= n);
        const uint64_t badm = __ballot(bad);
        // pointer doubling: (set, ls, dep) summarise the path segment from n
        // up to (not including) jmp
        uint64_t set = valid ? (1ull << n) : 0ull;
        int jmp = (valid && !bad) ? par : -1;
        float ls = la;
        int dep = valid ? 1 : 0;
#pragma unroll
        for (int it = 0; it < 6; ++it) {
            const int src = jmp >= 0 ? jmp : n;
            const uint64_t set_j = shfl_u64(set, src);
            const float ls_j = __shfl(ls, src, kWave);
            const int dep_j = __shfl(dep, src, kWave);
            const int jmp_j = __shfl(jmp, src, kWave);
            if (jmp >= 0) {
                set |= set_j;
                ls += ls_j;
                dep += dep_j;
                jmp = jmp_j;
            }
        }
        if (n < TM) {
            s_anc[n] = valid ? (set & ~(1ull << n)) : 0ull;
            s_logp[n] = ls;
            s_P[n] = valid ? expf(ls) : 0.f;
            s_beta[n] = be;
        }
        const int maxdep = wave_max_i(dep);
        for (int lv = 1; lv <= maxdep; ++lv) {
            const uint64_t m = __ballot(valid && dep == lv);
            if (lane == 0) s_lvl[lv] = m;
        }
        if (lane == 0) {
            s_int[0] = maxdep;
            s_int[1] = badm != 0ull;
            if (badm != 0ull && p.status && h == 0 && tile == 0) atomicOr(p.status, LDV_STATUS_BAD_PARENT);
        }
        if (badm == 0ull && valid && tile == 0 && p.logp_out) p.logp_out[((size_t)b * T + n) * H + h] = ls;
    }
    __syncthreads();
    if (s_int[1]) return;  // invalid parent row: nothing is written

    // 3. C and G: lower-triangular 16x16 blocks of Q K^T and K K^T
    {
        const int npairs = NB * (NB + 1) / 2;
        for (int it = wave; it < 2 * npairs; it += NW) {
            const int kind = it & 1;  // 0: Q K^T -> C, 1: K K^T -> G
            const int pr = it >> 1;
            int mb = 0;
            while ((mb + 1) * (mb + 2) / 2 <= pr) ++mb;
            const int nb = pr - mb * (mb + 1) / 2;
            const unsigned short* arow = (kind ? s_k : s_q) + (mb * 16 + c) * QKLD;
            const unsigned short* brow = s_k + (nb * 16 + c) * QKLD;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 af = frag_row<D>(arow, s, g);
                const bf16x8 bfr = frag_row<D>(brow, s, g);
                acc = mfma16x16x32(af, bfr, acc);
                if constexpr (F32IN) {
                    const unsigned short* arow_lo = (kind ? s_klo : s_qlo) + (mb * 16 + c) * QKLD;
                    const unsigned short* brow_lo = s_klo + (nb * 16 + c) * QKLD;
                    acc = mfma16x16x32(af, frag_row<D>(brow_lo, s, g), acc);
                    acc = mfma16x16x32(frag_row<D>(arow_lo, s, g), bfr, acc);
                }
            }
            const int m = nb * 16 + c;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = mb * 16 + 4 * g + r;
                float val = 0.f;
                if (n < T && m < T) {
                    const uint64_t anc = s_anc[n];
                    if (kind == 0) {
                        if (((anc | (1ull << n)) >> m) & 1ull) val = expf(s_logp[n] - s_logp[m]) * acc[r];
                    } else {
                        if ((anc >> m) & 1ull) val = s_beta[n] * expf(s_logp[n] - s_logp[m]) * acc[r];
                    }
                }
                float* cell = reinterpret_cast<float*>(s_gc + n * TM + m);
                cell[kind ? 0 : 1] = val;
            }
        }
    }

    // 4. state products Q S0^T and K S0^T for this wave's 16 value columns
    floatx4 accq[MBMAX], acck[MBMAX];
#pragma unroll
    for (int mb = 0; mb < MBMAX; ++mb) {
        accq[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
        acck[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u16x4 h0, l0, h1, l1;
        split4(sreg[s][0], h0, l0);
        split4(sreg[s][1], h1, l1);
        const bf16x8 bh = join(h0, h1), bl = join(l0, l1);
#pragma unroll
        for (int mb = 0; mb < MBMAX; ++mb) {
            if (mb < NB) {
                const bf16x8 aq = frag_row<D>(s_q + (mb * 16 + c) * QKLD, s, g);
                const bf16x8 ak = frag_row<D>(s_k + (mb * 16 + c) * QKLD, s, g);
                accq[mb] = mfma16x16x32(aq, bh, accq[mb]);
                accq[mb] = mfma16x16x32(aq, bl, accq[mb]);
                acck[mb] = mfma16x16x32(ak, bh, acck[mb]);
                acck[mb] = mfma16x16x32(ak, bl, acck[mb]);
                if constexpr (F32IN) {
                    accq[mb] = mfma16x16x32(frag_row<D>(s_qlo + (mb * 16 + c) * QKLD, s, g), bh, accq[mb]);
                    acck[mb] = mfma16x16x32(frag_row<D>(s_klo + (mb * 16 + c) * QKLD, s, g), bh, acck[mb]);
                }
            }
        }
    }
    // B0 = P (Q S0^T), R = beta (v - P (K S0^T)) at (node, column jl)
    float b0v[MBMAX][4], rv[MBMAX][4];
#pragma unroll
    for (int mb = 0; mb < MBMAX; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = mb * 16 + 4 * g + r;
            b0v[mb][r] = 0.f;
            rv[mb][r] = 0.f;
            if (mb < NB && n < T) {
                float vv;
                if constexpr (F32IN) vv = static_cast<const float*>(s_v)[n * BV + jl];
                else vv = bf16_val(static_cast<const unsigned short*>(s_v)[n * BV + jl]);
                const float P = s_P[n];
                b0v[mb][r] = P * accq[mb][r];
                rv[mb][r] = s_beta[n] * (vv - P * acck[mb][r]);
            }
        }
    }
    __syncthreads();  // Q/K no longer read; C and G complete
#pragma unroll
    for (int mb = 0; mb < MBMAX; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = mb * 16 + 4 * g + r;
            if (mb < NB && n < T) {
                s_b0[n * BRLD + jl] = b0v[mb][r];
                s_r[n * BRLD + jl] = rv[mb][r];
            }
        }
    }
    __syncthreads();

    // 5. (I + G) U = R and O = B0 + C U, level by level
    const int maxdep = s_int[0];
    for (int lv = 1; lv <= maxdep; ++lv) {
        const uint64_t lvm = s_lvl[lv];
        const int cnt = __builtin_popcountll(lvm);
        for (int it = wave; it < cnt; it += NW) {
            const int n = nth_set_bit(lvm, it);
            if (lane < BV) {
                const int j = lane;
                float u = s_r[n * BRLD + j];
                float o = s_b0[n * BRLD + j];
                uint64_t an = s_anc[n];
                while (an) {
                    const int m = __builtin_ctzll(an);
                    an &= an - 1;
                    const float2 gc = s_gc[n * TM + m];
                    const float um = s_r[m * BRLD + j];
                    u -= gc.x * um;
                    o += gc.y * um;
                }
                o += s_gc[n * TM + n].y * u;
                s_r[n * BRLD + j] = u;
                const size_t off = (((size_t)b * T + n) * H + h) * D + (size_t)tile * BV + j;
                p.o[off] = o;
                if (p.u_out) p.u_out[off] = u;
            }
        }
        __syncthreads();
    }
}

template <int D, int TM, bool F32IN>
static hipError_t launch_t(const VerifyArgs& a, hipStream_t st) {
    using S = VShape<D>;
    const long long nblk = (long long)a.B * a.H * S::NT;
    if (nblk <= 0) return hipSuccess;
    hipLaunchKernelGGL((verify_kernel<D, TM, F32IN>), dim3((unsigned)nblk), dim3(S::NW * kWave), 0, st, a);
    return hipGetLastError();
}

template <int D, bool F32IN>
static hipError_t launch_d(const VerifyArgs& a, hipStream_t st) {
    if (a.T <= 16) return launch_t<D, 16, F32IN>(a, st);
    if (a.T <= 32) return launch_t<D, 32, F32IN>(a, st);
    return launch_t<D, 64, F32IN>(a, st);
}

template <bool F32IN>
static hipError_t launch_f(const VerifyArgs& a, hipStream_t st) {
    switch (a.D) {
        case 16: return launch_d<16, F32IN>(a, st);
        case 32: return launch_d<32, F32IN>(a, st);
        case 64: return launch_d<64, F32IN>(a, st);
        case 128: return launch_d<128, F32IN>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_verify(const VerifyArgs& a, bool f32_inputs, hipStream_t stream) {
    return f32_inputs ? launch_f<true>(a, stream) : launch_f<false>(a, stream);
}

}  // namespace ldv
