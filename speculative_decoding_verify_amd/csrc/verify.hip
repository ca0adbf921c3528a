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
// G is strictly lower in topological order, so over 16-node blocks
//   U_i = X_ii (R_i - sum_{k < i} G_ik U_k),   X_ii = (I + G_ii)^{-1}
// (block forward substitution: only the diagonal blocks of (I + G)^{-1} are
// ever formed), and O_j = B0_j + sum_{i <= j} C_ji U_i.
//
// All 16 x 16 products use one identity.  With a matrix P held in the MFMA
// C layout (lane (c, g), register r holds P[4 g + r][c]), the same registers
// are the B operand of a 16-deep product as they stand and the A operand of
// one with P transposed, so mm(P, Q) = P^T Q needs no data movement; fp32
// operands go in as bf16 hi + lo terms (two MFMAs, lo * lo dropped).
//
// Drafts of up to 16 nodes go to verify_t16_kernel (below).  Longer ones
// use one workgroup per (sequence, head, value tile of BV columns): G and C
// do not depend on the value channel (Eq. (7) context), so value tiles are
// independent; at d = 128 a tile is the whole head, so the T x T factor work
// is done once per head.  Each wave owns one 16-row value block of the tile
// (two at 32 nodes).  Per workgroup:
//   1. issue the loads of q, k, v, the gates and the parent row, then of the
//      wave's S0 rows (fp32) straight into MFMA operand registers; the S0
//      loads stay in flight through steps 2-3;
//   2. stage Q, K (bf16) in LDS; wave 0 turns the parent row into ancestor
//      masks and log P by pointer doubling;
//   3. the factor tiles, spread over the waves: each is a 16 x 16 product of
//      K or Q rows on MFMA, masked and decay-scaled in the accumulators and
//      kept in LDS in the C layout as hi + lo terms:
//        X_ii^T  (forward substitution in registers from G_ii),
//        -G_ik^T (k < i),  C_ji^T (i <= j);
//   4. S0 Q^T (value-major) and K S0^T (node-major) on MFMA give B0^T and R
//      for the wave's value rows;
//   5. per node block i: Y = R_i - sum_k G_ik U_k, then U_i = X_ii Y (kept
//      for the later blocks) and U_i^T = Y^T X_ii^T (stored), and
//      O_j^T += U_i^T C_ji^T for j >= i; O_i^T is then complete and stored,
//      each lane writing four consecutive values of one node (float4).
// Two workgroup barriers in all (after step 2 and after step 3).
// P_n / P_m is exp(log P_n - log P_m), evaluated only for ancestor pairs
// (exponent <= 0 for gates in [0, 1]); log a is clamped at -87 so that a
// zero gate gives a finite log.
#include "ldv_device.hpp"
#include "ldv_kernels.hpp"

#include "../../include/ldv.h"

namespace ldv {

// acc + P^T Q for 16 x 16 fp32 matrices in the C layout, given as hi + lo
// bf16 terms: the 32 k-slots of the first MFMA pair P_hi and P_lo with
// Q_hi, the second adds P_hi^T Q_lo (lo * lo dropped).
__device__ __forceinline__ floatx4 mm16_acc(floatx4 acc, u16x4 ph, u16x4 pl, u16x4 qh, u16x4 ql) {
    acc = mfma16x16x32(join(ph, pl), join(qh, qh), acc);
    return mfma16x16x32(join(ph, zero4()), join(ql, zero4()), acc);
}

// Makes v be computed at this point of the program.  An MFMA whose result
// feeds only a store under a per-lane condition may otherwise be sunk into
// that condition's exec-masked block together with its operand set-up,
// which the masked lanes then skip although the MFMA reads their registers.
__device__ __forceinline__ void keep_here(floatx4& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ void split_x4(const floatx4 v, u16x4& hi, u16x4& lo) {
    split4(make_float4(v[0], v[1], v[2], v[3]), hi, lo);
}

// A 16 x 16 factor tile in LDS: the hi terms of the 64 lanes' C-layout
// registers, then the lo terms (8 bytes per lane each, conflict-free).
__device__ __forceinline__ void tile_store(u16x4* tiles, int t, int lane, const floatx4 v) {
    u16x4 hi, lo;
    split_x4(v, hi, lo);
    tiles[(2 * t) * kWave + lane] = hi;
    tiles[(2 * t + 1) * kWave + lane] = lo;
}

__device__ __forceinline__ void tile_load(const u16x4* tiles, int t, int lane, u16x4& hi, u16x4& lo) {
    hi = tiles[(2 * t) * kWave + lane];
    lo = tiles[(2 * t + 1) * kWave + lane];
}

template <int D, int TM>
struct VShape {
    // At d = 128 a block keeps the whole head (BV = 128), so the factor work
    // is done once per head: eight waves of 16 value rows at 64 nodes, four
    // waves of two 16-row blocks (MBW = 2) at 32 nodes, where each factor
    // tile read from LDS then serves two row blocks.
    static constexpr int BV = (D >= 128) ? 128 : (D >= 64 ? 64 : D);
    static constexpr int MBW = (TM == 32 && D >= 128) ? 2 : 1;  // 16-row blocks per wave
    static constexpr int NT = D / BV;         // value tiles per head
    static constexpr int NW = BV / (16 * MBW);  // waves per block
    static constexpr int KS = (D + 31) / 32;  // MFMA k-steps over d_k
    static constexpr int QKLD = D + 8;        // bf16 row stride of Q/K in LDS
    static constexpr int NBM = TM / 16;       // 16-node blocks at most
    // factor tiles: X_ii^T (NBM), -G_ik^T (k < i), C_ji^T (i <= j)
    static constexpr int NTILE = NBM * (NBM + 1);
    static constexpr int TG0 = NBM;                        // first -G tile
    static constexpr int TC0 = NBM + NBM * (NBM - 1) / 2;  // first C tile
    // waves per SIMD the registers must allow: two blocks per CU at 64 nodes
    // (eight waves each), three at 32 nodes with two row blocks per wave,
    // four otherwise
    static constexpr int WPE = MBW == 2 ? 3 : 4;
};

template <int D, int TM, bool F32IN>
struct VLds {
    using S = VShape<D, TM>;
    static constexpr int NPLANE = F32IN ? 4 : 2;  // q, k (hi and lo planes for fp32 input)
    static constexpr size_t qk = (size_t)NPLANE * TM * S::QKLD * 2;
    static constexpr size_t off_t = (qk + 15) / 16 * 16;                          // factor tiles
    static constexpr size_t off_anc = off_t + (size_t)S::NTILE * 2 * kWave * 8;  // uint64 [TM]
    static constexpr size_t off_f = off_anc + 8 * TM;  // float logp, P, beta [TM] each
    static constexpr size_t off_i = off_f + 12 * TM;   // int: bad flag
    static constexpr size_t total = off_i + 16;
};

template <int D, int TM, bool F32IN>
__global__ __launch_bounds__((VShape<D, TM>::NW * kWave))
__attribute__((amdgpu_waves_per_eu(VShape<D, TM>::WPE))) void verify_kernel(const VerifyArgs p) {
    using S = VShape<D, TM>;
    using L = VLds<D, TM, F32IN>;
    constexpr int BV = S::BV, NW = S::NW, KS = S::KS, QKLD = S::QKLD, NBM = S::NBM, MBW = S::MBW;
    constexpr int NTHR = NW * kWave;
    constexpr int EPC = F32IN ? 4 : 8;                 // elements per 16-byte chunk
    constexpr int CPR = D / EPC;                       // chunks per q/k row
    constexpr int QKC = (TM * CPR + NTHR - 1) / NTHR;  // q (and k) chunks per thread
    constexpr int LO = 2 * TM * QKLD;                  // offset of the lo planes (fp32 input)

    __shared__ __align__(16) unsigned char smem[L::total];
    unsigned short* s_q = reinterpret_cast<unsigned short*>(smem);
    unsigned short* s_k = s_q + TM * QKLD;
    u16x4* s_tl = reinterpret_cast<u16x4*>(smem + L::off_t);
    uint64_t* s_anc = reinterpret_cast<uint64_t*>(smem + L::off_anc);
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
    const size_t nb0 = (size_t)b * p.Ts + p.t0;  // node 0 of this sequence's (chunk of the) draft
    const int NB = (T + 15) >> 4;  // 16-node blocks in use
    const int T16 = NB * 16;
    const int vrow0 = tile * BV + wave * 16 * MBW;  // first value row (of S0, o, u) of this wave

    // 1. global loads.  Every small per-node input first, so that, loads
    // completing in issue order, steps 2-3 can run while the S0 rows are in
    // flight.  The loads are branch-free (indices clamped into range, values
    // of rows past T dropped later by selects): a load under a branch, or a
    // register overwritten while its load is pending, would make the
    // compiler wait for every earlier memory operation.
    u32x4 qreg[QKC], kreg[QKC];
#pragma unroll
    for (int i = 0; i < QKC; ++i) {
        const int ch = tid + i * NTHR, row = min(ch / CPR, T - 1), col = (ch % CPR) * EPC;
        const size_t off = (((nb0 + row) * H + h) * D + col) * (F32IN ? 4 : 2);
        qreg[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.q) + off);
        kreg[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.k) + off);
    }
    // v[n][vrow0 + 16 mi + c] for the nodes n = 16 nb + 4 g + r this lane
    // holds in R (node-major C layout)
    float vf[MBW][NBM][4];
    unsigned short vb[MBW][NBM][4];
#pragma unroll
    for (int mi = 0; mi < MBW; ++mi) {
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = min(nb * 16 + 4 * g + r, T - 1);
                const size_t off = ((nb0 + n) * H + h) * D + vrow0 + 16 * mi + c;
                if constexpr (F32IN) vf[mi][nb][r] = static_cast<const float*>(p.v)[off];
                else vb[mi][nb][r] = static_cast<const unsigned short*>(p.v)[off];
            }
        }
    }
    const int nl = min(lane, T - 1);
    // a chain has no parent array: read the gate array instead (it has at
    // least B * T entries) and discard the value
    const global_ptr<const int32_t> parp =
        (global_ptr<const int32_t>)(p.parent ? p.parent : reinterpret_cast<const int32_t*>(p.a));
    const int par_ld = parp[(size_t)b * T + nl];
    const size_t gi = (nb0 + nl) * H + h;
    const float ga = p.a[gi];
    const float gb = p.beta[gi];
    // log P at the node before a chunk (read from any valid entry otherwise)
    const float* lbp = p.logp_out ? p.logp_out : p.a;
    const float lbase_ld = lbp[((p.t0 > 0 ? nb0 - 1 : nb0)) * H + h];
    // this lane's S0 rows (A operand row c of each of the wave's 16-row
    // blocks, and the B operand column c of K S0^T)
    // (one row block is written without the row-block loop: with it the
    // compiler's allocation of the 64-node kernel spills)
    float4 sreg[MBW][KS][2];
    if constexpr (MBW == 1) {
        const float* s0row = p.S0 + (((size_t)b * H + h) * D + vrow0 + c) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int k0 = 32 * s + 4 * g;
            sreg[0][s][0] = (k0 < D) ? ld_stream(s0row + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
            sreg[0][s][1] = (k0 + 16 < D) ? ld_stream(s0row + k0 + 16) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else {
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) {
            const float* s0row = p.S0 + (((size_t)b * H + h) * D + vrow0 + 16 * mi + c) * D;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int k0 = 32 * s + 4 * g;
                sreg[mi][s][0] = (k0 < D) ? ld_stream(s0row + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
                sreg[mi][s][1] = (k0 + 16 < D) ? ld_stream(s0row + k0 + 16) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    }
    asm volatile("" ::: "memory");  // keep the loads above ahead of any use of them
    const int par = p.parent ? par_ld : lane - 1;

    // 2a. Q, K rows into LDS (rows T .. T16-1 zero)
#pragma unroll
    for (int i = 0; i < QKC; ++i) {
        const int ch = tid + i * NTHR, row = ch / CPR, col = (ch % CPR) * EPC;
        if (row < T16) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 qv = row < T ? qreg[i] : z, kv = row < T ? kreg[i] : z;
            if constexpr (!F32IN) {
                *reinterpret_cast<u32x4*>(s_q + row * QKLD + col) = qv;
                *reinterpret_cast<u32x4*>(s_k + row * QKLD + col) = kv;
            } else {
                u16x4 hi, lo;
                split4(__builtin_bit_cast(float4, qv), hi, lo);
                *reinterpret_cast<u16x4*>(s_q + row * QKLD + col) = hi;
                *reinterpret_cast<u16x4*>(s_q + LO + row * QKLD + col) = lo;
                split4(__builtin_bit_cast(float4, kv), hi, lo);
                *reinterpret_cast<u16x4*>(s_k + row * QKLD + col) = hi;
                *reinterpret_cast<u16x4*>(s_k + LO + row * QKLD + col) = lo;
            }
        }
    }

    // 2b. topology: lane n of wave 0 is node n
    if (wave == 0) {
        const int n = lane;
        const bool valid = n < T;
        const bool bad = valid && (par < -1 || par >= n);
        const uint64_t badm = __ballot(bad);
        const float la = valid ? fmaxf(logf(ga), -87.f) : 0.f;
        // pointer doubling: (set, ls) summarise the path segment from n up to
        // (not including) jmp
        uint64_t set = valid ? (1ull << n) : 0ull;
        int jmp = (valid && !bad) ? par : -1;
        float ls = la;
        for (int it = 0; it < 6; ++it) {
            if (__ballot(jmp >= 0) == 0ull) break;  // every path complete
            const int src = jmp >= 0 ? jmp : n;
            const uint64_t set_j = shfl_u64(set, src);
            const float ls_j = __shfl(ls, src, kWave);
            const int jmp_j = __shfl(jmp, src, kWave);
            if (jmp >= 0) {
                set |= set_j;
                ls += ls_j;
                jmp = jmp_j;
            }
        }
        if (n < TM) {
            s_anc[n] = valid ? (set & ~(1ull << n)) : 0ull;
            s_logp[n] = ls;
            s_P[n] = valid ? expf(ls) : 0.f;
            s_beta[n] = valid ? gb : 0.f;
        }
        if (lane == 0) {
            s_int[0] = badm != 0ull;
            if (badm != 0ull && p.status && h == 0 && tile == 0) atomicOr(p.status, LDV_STATUS_BAD_PARENT);
        }
        if (badm == 0ull && valid && tile == 0 && p.logp_out)
            p.logp_out[(nb0 + n) * H + h] = ls + (p.t0 > 0 ? lbase_ld : 0.f);
    }
    __syncthreads();
    if (s_int[0]) return;  // invalid parent row: nothing is written

    // 3a. diagonal blocks: X_ii^T.  K_i K_i^T in the C layout is G_ii[n][m]
    //     before scaling (rows n = 16 i + 4 g + r, column m = 16 i + c).
    for (int i = wave; i < NB; i += NW) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        const unsigned short* krow = s_k + (16 * i + c) * QKLD;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 bk = frag_row<D>(krow, s, g);
            acc = mfma16x16x32(bk, bk, acc);
            if constexpr (F32IN) {
                const bf16x8 bkl = frag_row<D>(krow + LO, s, g);
                acc = mfma16x16x32(bk, bkl, acc);
                acc = mfma16x16x32(bkl, bk, acc);
            }
        }
        const int m = 16 * i + c;
        const float lpm = s_logp[m];
        float gv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = 16 * i + 4 * g + r;
            const bool strict = ((s_anc[n] >> m) & 1ull) != 0ull;
            gv[r] = strict ? s_beta[n] * expf(s_logp[n] - lpm) * acc[r] : 0.f;
        }
        // row c of X = (I + G_ii)^{-1} in every lane of column c: from
        // X (I + G) = I, X[c][t] = [t == c] - sum_{s > t} X[c][s] G[s][t],
        // with G[s][t] read from lane t + 16 (s / 4), register s % 4
        float x[16];
#pragma unroll
        for (int t = 15; t >= 0; --t) {
            float a = (t == c) ? 1.f : 0.f;
#pragma unroll
            for (int s = t + 1; s < 16; ++s) a -= x[s] * readlane_f(gv[s & 3], t + 16 * (s >> 2));
            x[t] = a;
        }
        // X_ii^T in the C layout: register r of lane (c, g) is X[c][4 g + r]
        floatx4 xt;
#pragma unroll
        for (int r = 0; r < 4; ++r) xt[r] = g == 0 ? x[r] : g == 1 ? x[4 + r] : g == 2 ? x[8 + r] : x[12 + r];
        tile_store(s_tl, i, lane, xt);
    }

    // 3b. -G_ik^T (k < i) and C_ji^T (i <= j).  Item it covers the tile of
    //     rows n in node block bn and columns m in block bm: A = k rows of
    //     block bm, B = k or q rows of block bn, so the accumulator holds
    //     k_m . k_n (or k_m . q_n) at register r of lane (c, g) for
    //     m = 16 bm + 4 g + r, n = 16 bn + c.  The items start at wave NB so
    //     that the waves holding a diagonal block take fewer of them.
    {
        const int nneg = NB * (NB - 1) / 2;
        for (int it = (wave + NW - NB % NW) % NW; it < NB * NB; it += NW) {
            const bool isc = it >= nneg;
            int bn, bm, t;
            if (!isc) {
                int i = 1;
                while (i * (i + 1) / 2 <= it) ++i;
                bn = i;
                bm = it - i * (i - 1) / 2;
                t = S::TG0 + i * (i - 1) / 2 + bm;
            } else {
                const int rr = it - nneg;
                int j = 0;
                while ((j + 1) * (j + 2) / 2 <= rr) ++j;
                bn = j;
                bm = rr - j * (j + 1) / 2;
                t = S::TC0 + j * (j + 1) / 2 + bm;
            }
            const unsigned short* arow = s_k + (16 * bm + c) * QKLD;
            const unsigned short* brow = (isc ? s_q : s_k) + (16 * bn + c) * QKLD;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 fa = frag_row<D>(arow, s, g), fb = frag_row<D>(brow, s, g);
                acc = mfma16x16x32(fa, fb, acc);
                if constexpr (F32IN) {
                    acc = mfma16x16x32(fa, frag_row<D>(brow + LO, s, g), acc);
                    acc = mfma16x16x32(frag_row<D>(arow + LO, s, g), fb, acc);
                }
            }
            const int n = 16 * bn + c;
            // m on the path of n (C: n itself included; G: strict ancestors)
            const uint64_t pathn = s_anc[n] | (isc ? (1ull << n) : 0ull);
            const float lpn = s_logp[n], sc = isc ? 1.f : -s_beta[n];
            floatx4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * bm + 4 * g + r;
                v[r] = ((pathn >> m) & 1ull) ? sc * expf(lpn - s_logp[m]) * acc[r] : 0.f;
            }
            tile_store(s_tl, t, lane, v);
        }
    }

    // 4. S0 Q^T (A = S0 rows, B = q rows: value-major, lane (c, g) holds
    //    value rows 4 g + r of node 16 nb + c) and K S0^T (A = k rows,
    //    B = S0 rows: node-major, nodes 16 nb + 4 g + r of value row c).
    //    Both read only Q, K and registers, so they go before the barrier.
    floatx4 accq[MBW][NBM], acck[MBW][NBM];
#pragma unroll
    for (int mi = 0; mi < MBW; ++mi) {
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
            accq[mi][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
            acck[mi][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        bf16x8 sh[MBW], sl[MBW];
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) split8(sreg[mi][s][0], sreg[mi][s][1], sh[mi], sl[mi]);
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
            if (nb < NB) {
                const unsigned short* qrow = s_q + (nb * 16 + c) * QKLD;
                const unsigned short* krow = s_k + (nb * 16 + c) * QKLD;
                const bf16x8 bq = frag_row<D>(qrow, s, g);
                const bf16x8 bk = frag_row<D>(krow, s, g);
#pragma unroll
                for (int mi = 0; mi < MBW; ++mi) {
                    accq[mi][nb] = mfma16x16x32(sh[mi], bq, accq[mi][nb]);
                    accq[mi][nb] = mfma16x16x32(sl[mi], bq, accq[mi][nb]);
                    acck[mi][nb] = mfma16x16x32(bk, sh[mi], acck[mi][nb]);
                    acck[mi][nb] = mfma16x16x32(bk, sl[mi], acck[mi][nb]);
                }
                if constexpr (F32IN) {
                    const bf16x8 bql = frag_row<D>(qrow + LO, s, g);
                    const bf16x8 bkl = frag_row<D>(krow + LO, s, g);
#pragma unroll
                    for (int mi = 0; mi < MBW; ++mi) {
                        accq[mi][nb] = mfma16x16x32(sh[mi], bql, accq[mi][nb]);
                        acck[mi][nb] = mfma16x16x32(bkl, sh[mi], acck[mi][nb]);
                    }
                }
            }
        }
    }
    // B0^T[v][n] = P_n (S0 q_n)[v] (the O^T accumulators start there);
    // R[n][v] = beta_n (v_n[v] - P_n (S0 k_n)[v]), zero past T (beta = 0)
    floatx4 acco[MBW][NBM], rn[MBW][NBM];
#pragma unroll
    for (int nb = 0; nb < NBM; ++nb) {
        if (nb < NB) {
            const float Pc = s_P[nb * 16 + c];
            const float4 P4 = *reinterpret_cast<const float4*>(s_P + nb * 16 + 4 * g);
            const float4 B4 = *reinterpret_cast<const float4*>(s_beta + nb * 16 + 4 * g);
            const float Pr[4] = {P4.x, P4.y, P4.z, P4.w}, Br[4] = {B4.x, B4.y, B4.z, B4.w};
#pragma unroll
            for (int mi = 0; mi < MBW; ++mi) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float vv;
                    if constexpr (F32IN) vv = vf[mi][nb][r];
                    else vv = bf16_val(vb[mi][nb][r]);
                    acco[mi][nb][r] = Pc * accq[mi][nb][r];
                    rn[mi][nb][r] = Br[r] * (vv - Pr[r] * acck[mi][nb][r]);
                }
            }
        }
    }
    __syncthreads();  // every factor tile written

    // 5. forward substitution over node blocks; O^T block by block
    u16x4 uh[MBW][NBM], ul[MBW][NBM];
#pragma unroll
    for (int i = 0; i < NBM; ++i) {
        if (i < NB) {
            floatx4 y[MBW];
#pragma unroll
            for (int mi = 0; mi < MBW; ++mi) y[mi] = rn[mi][i];
#pragma unroll
            for (int k = 0; k < i; ++k) {  // Y -= G_ik U_k
                u16x4 th, tl;
                tile_load(s_tl, S::TG0 + i * (i - 1) / 2 + k, lane, th, tl);
#pragma unroll
                for (int mi = 0; mi < MBW; ++mi) y[mi] = mm16_acc(y[mi], th, tl, uh[mi][k], ul[mi][k]);
            }
            u16x4 xh, xl;
            tile_load(s_tl, i, lane, xh, xl);
            const int n = 16 * i + c;
#pragma unroll
            for (int mi = 0; mi < MBW; ++mi) {
                u16x4 yh, yl;
                split_x4(y[mi], yh, yl);
                const floatx4 z = {0.f, 0.f, 0.f, 0.f};
                split_x4(mm16_acc(z, xh, xl, yh, yl), uh[mi][i], ul[mi][i]);  // U_i = X_ii Y
                if (p.u_out) {
                    floatx4 ut = mm16_acc(z, yh, yl, xh, xl);  // U_i^T = Y^T X_ii^T
                    keep_here(ut);
                    if (n < T)
                        st_stream(p.u_out + ((nb0 + n) * H + h) * D + vrow0 + 16 * mi + 4 * g,
                                  make_float4(ut[0], ut[1], ut[2], ut[3]));
                }
            }
#pragma unroll
            for (int j = i; j < NBM; ++j) {  // O_j^T += U_i^T C_ji^T
                if (j < NB) {
                    u16x4 ch, cl;
                    tile_load(s_tl, S::TC0 + j * (j + 1) / 2 + i, lane, ch, cl);
#pragma unroll
                    for (int mi = 0; mi < MBW; ++mi) acco[mi][j] = mm16_acc(acco[mi][j], uh[mi][i], ul[mi][i], ch, cl);
                }
            }
#pragma unroll
            for (int mi = 0; mi < MBW; ++mi) keep_here(acco[mi][i]);
            if (n < T) {
#pragma unroll
                for (int mi = 0; mi < MBW; ++mi)
                    st_stream(p.o + ((nb0 + n) * H + h) * D + vrow0 + 16 * mi + 4 * g,
                              make_float4(acco[mi][i][0], acco[mi][i][1], acco[mi][i][2], acco[mi][i][3]));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// T <= 16: one 16 x 16 node block, so one wave does the whole factor algebra
// of the head in registers, and every wave of the block then handles 16
// value rows of the head, all products being mm(P, Q) = P^T Q on C-layout
// registers (top of this file).  K K^T is symmetric, so G and G^T (and C and C^T
// from Q K^T and K Q^T) come out of the accumulators directly, and
//   X = (I + G)^-1 = (I - G)(I + G^2)(I + G^4)(I + G^8)      (G^16 = 0)
// is built by repeated squaring, stopping at the stage the tree depth
// allows.  Then M^T = X^T C^T, R and B0^T from the state products, and
// U^T = R^T X^T, O^T = B0^T + R^T M^T.  X^T and M^T reach the other waves
// through LDS in the same C layout (one float4 per lane), and the only LDS
// staging is Q and K.

// P^T Q for 16 x 16 fp32 matrices in the C layout
__device__ __forceinline__ floatx4 mm16(const floatx4 P, const floatx4 Q) {
    u16x4 ph, pl, qh, ql;
    split_x4(P, ph, pl);
    split_x4(Q, qh, ql);
    return mm16_acc(floatx4{0.f, 0.f, 0.f, 0.f}, ph, pl, qh, ql);
}

// I + s P for a C-layout matrix (s = +1 or -1), lane (c, g)
__device__ __forceinline__ floatx4 ident_plus(const floatx4 P, float sgn, int c, int g) {
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = sgn * P[i] + ((4 * g + i == c) ? 1.f : 0.f);
    return r;
}

template <int D>
struct W16Shape {
    static constexpr int BV = D >= 64 ? 64 : D;  // value rows per block
    static constexpr int NT = D / BV;            // blocks per head
    static constexpr int NW = BV / 16;           // waves per block, 16 value rows each
    static constexpr int KS = (D + 31) / 32;     // MFMA k-steps over d_k
    static constexpr int QKLD = D + 8;           // bf16 row stride of Q/K in LDS
};

template <int D, bool F32IN>
__global__ __launch_bounds__((W16Shape<D>::NW * kWave)) void verify_t16_kernel(const VerifyArgs p) {
    using S = W16Shape<D>;
    constexpr int BV = S::BV, NW = S::NW, KS = S::KS, QKLD = S::QKLD;
    constexpr int NTHR = NW * kWave;
    constexpr int EPC = F32IN ? 4 : 8;                 // elements per 16-byte chunk
    constexpr int CPR = D / EPC;                       // chunks per q/k row
    constexpr int QKC = (16 * CPR + NTHR - 1) / NTHR;  // q (and k) chunks per thread
    constexpr int NPLANE = F32IN ? 4 : 2;

    __shared__ __align__(16) unsigned short s_qk[NPLANE * 16 * QKLD];
    __shared__ float4 s_xt[kWave], s_mt[kWave];  // X^T and M^T in the C layout, one float4 per lane
    unsigned short* s_q = s_qk;
    unsigned short* s_k = s_qk + 16 * QKLD;
    unsigned short* s_qlo = s_k + 16 * QKLD;  // fp32 input only
    unsigned short* s_klo = s_qlo + 16 * QKLD;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int T = p.T, H = p.H;
    const unsigned bid = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = (int)(bid % S::NT);
    const int bh = (int)(bid / S::NT);
    const int h = bh % H, b = bh / H;
    const size_t nb0 = (size_t)b * p.Ts + p.t0;  // node 0 of this sequence's (chunk of the) draft
    const int vrow0 = tile * BV + wave * 16;

    // 1. loads, small ones first, branch-free (rows clamped into range)
    u32x4 qreg[QKC], kreg[QKC];
#pragma unroll
    for (int i = 0; i < QKC; ++i) {
        const int ch = tid + i * NTHR, row = min(ch / CPR, T - 1), col = (ch % CPR) * EPC;
        const size_t off = (((nb0 + row) * H + h) * D + col) * (F32IN ? 4 : 2);
        qreg[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.q) + off);
        kreg[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.k) + off);
    }
    // v[n][vrow0 + c] for the nodes n = 4 g + r this lane holds in R
    float vv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const size_t off = ((nb0 + min(4 * g + r, T - 1)) * H + h) * D + vrow0 + c;
        if constexpr (F32IN) vv[r] = static_cast<const float*>(p.v)[off];
        else vv[r] = bf16_val(static_cast<const unsigned short*>(p.v)[off]);
    }
    const int nq = min(c, T - 1);
    const global_ptr<const int32_t> parp =
        (global_ptr<const int32_t>)(p.parent ? p.parent : reinterpret_cast<const int32_t*>(p.a));
    const int par_ld = parp[(size_t)b * T + nq];
    const size_t gi = (nb0 + nq) * H + h;
    const float ga = p.a[gi];
    const float gb = p.beta[gi];
    const float* lbp = p.logp_out ? p.logp_out : p.a;  // log P before a chunk
    const float lbase_ld = lbp[((p.t0 > 0 ? nb0 - 1 : nb0)) * H + h];
    const float* s0row = p.S0 + (((size_t)b * H + h) * D + vrow0 + c) * D;
    float4 sreg[KS][2];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int k0 = 32 * s + 4 * g;
        sreg[s][0] = (k0 < D) ? ld_stream(s0row + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
        sreg[s][1] = (k0 + 16 < D) ? ld_stream(s0row + k0 + 16) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    asm volatile("" ::: "memory");  // keep the loads above ahead of any use of them

    // 2a. Q, K rows into LDS (rows T .. 15 zero)
#pragma unroll
    for (int i = 0; i < QKC; ++i) {
        const int ch = tid + i * NTHR, row = ch / CPR, col = (ch % CPR) * EPC;
        if (row < 16) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 qv = row < T ? qreg[i] : z, kv = row < T ? kreg[i] : z;
            if constexpr (!F32IN) {
                *reinterpret_cast<u32x4*>(s_q + row * QKLD + col) = qv;
                *reinterpret_cast<u32x4*>(s_k + row * QKLD + col) = kv;
            } else {
                u16x4 hi, lo;
                split4(__builtin_bit_cast(float4, qv), hi, lo);
                *reinterpret_cast<u16x4*>(s_q + row * QKLD + col) = hi;
                *reinterpret_cast<u16x4*>(s_qlo + row * QKLD + col) = lo;
                split4(__builtin_bit_cast(float4, kv), hi, lo);
                *reinterpret_cast<u16x4*>(s_k + row * QKLD + col) = hi;
                *reinterpret_cast<u16x4*>(s_klo + row * QKLD + col) = lo;
            }
        }
    }

    // 2b. topology, in every wave and every 16-lane group: lane (c, g) is node c
    const bool valid = c < T;
    const int par = p.parent ? par_ld : c - 1;
    const bool bad = valid && (par < -1 || par >= c);
    if (__ballot(bad) != 0ull) {  // the same verdict in every wave of the block
        if (tid == 0 && tile == 0 && p.status) atomicOr(p.status, LDV_STATUS_BAD_PARENT);
        return;  // invalid parent row: nothing is written
    }
    unsigned set = valid ? (1u << c) : 0u;  // path segment from c up to (not including) jmp
    int jmp = valid ? par : -1;
    float ls = valid ? fmaxf(logf(ga), -87.f) : 0.f;
    int dep = valid ? 1 : 0;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int src = (jmp >= 0 ? jmp : c) + 16 * g;
        const unsigned set_j = __shfl(set, src, kWave);
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
    const unsigned anc = set & ~(1u << c);
    const float lp = ls, Pc = valid ? expf(ls) : 0.f, bec = valid ? gb : 0.f;
    if (tile == 0 && wave == 0 && g == 0 && valid && p.logp_out)
        p.logp_out[(nb0 + c) * H + h] = lp + (p.t0 > 0 ? lbase_ld : 0.f);
    // node data for the rows n = 4 g + r of the C layout
    unsigned anc_r[4];
    float lp_r[4], P_r[4], be_r[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int src = 4 * g + r;
        anc_r[r] = __shfl(anc, src, kWave);
        lp_r[r] = __shfl(lp, src, kWave);
        P_r[r] = __shfl(Pc, src, kWave);
        be_r[r] = __shfl(bec, src, kWave);
    }
    __syncthreads();  // Q, K staged

    // 3. wave 0: G, G^T, C, C^T from K K^T, Q K^T, K Q^T (rows 4 g + r,
    //    column c); X = (I + G)^-1 by repeated squaring; M^T = X^T C^T
    if (wave == 0) {
        const int maxdep = wave_max_i(dep);
        floatx4 kk = {0.f, 0.f, 0.f, 0.f}, qk = kk, kq = kk;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 bq = frag_row<D>(s_q + c * QKLD, s, g), bk = frag_row<D>(s_k + c * QKLD, s, g);
            kk = mfma16x16x32(bk, bk, kk);
            qk = mfma16x16x32(bq, bk, qk);
            kq = mfma16x16x32(bk, bq, kq);
            if constexpr (F32IN) {
                const bf16x8 bql = frag_row<D>(s_qlo + c * QKLD, s, g), bkl = frag_row<D>(s_klo + c * QKLD, s, g);
                kk = mfma16x16x32(bk, bkl, kk);
                kk = mfma16x16x32(bkl, bk, kk);
                qk = mfma16x16x32(bq, bkl, qk);
                qk = mfma16x16x32(bql, bk, qk);
                kq = mfma16x16x32(bk, bql, kq);
                kq = mfma16x16x32(bkl, bq, kq);
            }
        }
        floatx4 G, Gt, Ct;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = 4 * g + r, m = c;
            const bool both = n < T && m < T;
            const bool m_on_n = both && ((((anc_r[r] | (1u << n)) >> m) & 1u) != 0u);
            const bool n_on_m = both && ((((anc | (1u << m)) >> n) & 1u) != 0u);
            const float dnm = m_on_n ? expf(lp_r[r] - lp) : 0.f;  // P_n / P_m
            const float dmn = n_on_m ? expf(lp - lp_r[r]) : 0.f;  // P_m / P_n
            G[r] = (m_on_n && m != n) ? be_r[r] * dnm * kk[r] : 0.f;
            Gt[r] = (n_on_m && m != n) ? bec * dmn * kk[r] : 0.f;
            Ct[r] = dmn * kq[r];
        }
        floatx4 X = ident_plus(G, -1.f, c, g), Xt = ident_plus(Gt, -1.f, c, g);  // I - G
        if (maxdep > 2) {
            floatx4 Gp = mm16(Gt, G), Gpt = mm16(G, Gt);  // G^2, (G^2)^T
            for (int stage = 2; stage < maxdep; stage *= 2) {
                const floatx4 Bm = ident_plus(Gp, 1.f, c, g);
                const floatx4 Xn = mm16(Xt, Bm), Xnt = mm16(Bm, Xt);  // X (I + G^p) and its transpose
                X = Xn;
                Xt = Xnt;
                if (2 * stage < maxdep) {
                    const floatx4 Gq = mm16(Gpt, Gp), Gqt = mm16(Gp, Gpt);
                    Gp = Gq;
                    Gpt = Gqt;
                }
            }
        }
        const floatx4 Mt = mm16(X, Ct);  // M^T = X^T C^T
        s_xt[lane] = make_float4(Xt[0], Xt[1], Xt[2], Xt[3]);
        s_mt[lane] = make_float4(Mt[0], Mt[1], Mt[2], Mt[3]);
    }
    __syncthreads();

    // 4. state products for this wave's 16 value rows: B0^T from S0 Q^T
    //    (rows = values, column c = node), K S0^T for R (rows = nodes)
    floatx4 sq = {0.f, 0.f, 0.f, 0.f}, ks = sq;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        bf16x8 sh, sl;
        split8(sreg[s][0], sreg[s][1], sh, sl);
        const bf16x8 bq = frag_row<D>(s_q + c * QKLD, s, g), bk = frag_row<D>(s_k + c * QKLD, s, g);
        sq = mfma16x16x32(sh, bq, sq);
        sq = mfma16x16x32(sl, bq, sq);
        ks = mfma16x16x32(bk, sh, ks);
        ks = mfma16x16x32(bk, sl, ks);
        if constexpr (F32IN) {
            sq = mfma16x16x32(sh, frag_row<D>(s_qlo + c * QKLD, s, g), sq);
            ks = mfma16x16x32(frag_row<D>(s_klo + c * QKLD, s, g), sh, ks);
        }
    }
    floatx4 B0t, R;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        B0t[r] = Pc * sq[r];                        // B0^T[value 4g+r][node c]
        R[r] = be_r[r] * (vv[r] - P_r[r] * ks[r]);  // R[node 4g+r][value c]; 0 past T
    }

    // 5. U^T = R^T X^T and O^T = B0^T + R^T M^T; lane (c, g) holds node c,
    //    values vrow0 + 4 g .. +3
    const float4 xt4 = s_xt[lane], mt4 = s_mt[lane];
    const floatx4 Xt = {xt4.x, xt4.y, xt4.z, xt4.w}, Mt = {mt4.x, mt4.y, mt4.z, mt4.w};
    const floatx4 Ut = mm16(R, Xt);
    const floatx4 RMt = mm16(R, Mt);
    if (c < T) {
        const size_t off = ((nb0 + c) * H + h) * D + vrow0 + 4 * g;
        st_stream(p.o + off, make_float4(B0t[0] + RMt[0], B0t[1] + RMt[1], B0t[2] + RMt[2], B0t[3] + RMt[3]));
        if (p.u_out) st_stream(p.u_out + off, make_float4(Ut[0], Ut[1], Ut[2], Ut[3]));
    }
}

template <int D, bool F32IN>
static hipError_t launch_t16(const VerifyArgs& a, hipStream_t st) {
    using S = W16Shape<D>;
    const long long nblk = (long long)a.B * a.H * S::NT;
    if (nblk <= 0) return hipSuccess;
    hipLaunchKernelGGL((verify_t16_kernel<D, F32IN>), dim3((unsigned)nblk), dim3(S::NW * kWave), 0, st, a);
    return hipGetLastError();
}

template <int D, int TM, bool F32IN>
static hipError_t launch_t(const VerifyArgs& a, hipStream_t st) {
    using S = VShape<D, TM>;
    const long long nblk = (long long)a.B * a.H * S::NT;
    if (nblk <= 0) return hipSuccess;
    hipLaunchKernelGGL((verify_kernel<D, TM, F32IN>), dim3((unsigned)nblk), dim3(S::NW * kWave), 0, st, a);
    return hipGetLastError();
}

template <int D, bool F32IN>
static hipError_t launch_d(const VerifyArgs& a, hipStream_t st) {
    if (a.T <= 16) return launch_t16<D, F32IN>(a, st);
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
