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
// G is strictly lower in topological order.  X = (I + G)^{-1} and M = C X
// depend only on Q, K, the gates and the topology; with them U = X R and
// O = B0 + M R.
//
// Drafts of up to 16 nodes go to verify_t16_kernel (below).  Longer ones
// use one workgroup per (sequence, head, value tile of BV columns): G and C
// do not depend on the value channel (Eq. (7) context), so value tiles are
// independent; at d = 128 a tile is the whole head, so the T x T factor work
// is done once per head.  Each wave owns one 16-row block of the tile (two
// at 32 nodes).  Per block:
//   1. issue the loads of q, k, v, the gates and the parent row, then of the
//      block's S0 rows (fp32) straight into MFMA operand registers; the S0
//      loads stay in flight through steps 2-4;
//   2. stage Q, K (bf16) in LDS; wave 0 turns the parent row into ancestor
//      masks and log P by pointer doubling;
//   3. 16 x 16 blocks of K K^T on MFMA, masked and decay-scaled into G;
//      the diagonal blocks of X are solved by forward substitution in
//      registers, reading G from the MFMA accumulators with readlane;
//   4. the off-diagonal blocks of X, X_ij = -X_ii sum_k G_ik X_kj (one stage
//      per block diagonal), then M = C X on MFMA, with the blocks of C made
//      on the fly from K Q^T (so C never takes LDS);
//   5. S0 Q^T and S0 K^T on MFMA (S0 split into bf16 hi + lo terms) give
//      B0^T and R^T for the wave's rows;
//   6. U^T = R^T X^T and O^T = B0^T + R^T M^T on MFMA (with eight waves
//      reading X and M, they are first packed once as bf16 hi | lo words);
//      each lane then holds four consecutive values of one node and stores
//      them as a float4.
// Products with fp32 operands on both sides (X, M, R) carry both as hi + lo
// bf16 terms (three MFMAs per step).  P_n / P_m is exp(log P_n - log P_m),
// evaluated only for ancestor pairs (exponent <= 0 for gates in [0, 1]);
// log a is clamped at -87 so that a zero gate gives a finite log.
#include "ldv_device.hpp"
#include "ldv_kernels.hpp"

#include "../../include/ldv.h"

namespace ldv {

template <int D, int TM>
struct VShape {
    // At d = 128 a block keeps the whole head (BV = 128), so the factor work
    // is done once per head: eight waves of 16 value rows at 64 nodes, four
    // waves of two 16-row blocks (MBW = 2) at 32 nodes, where each operand
    // fragment read from LDS then serves two MFMA row blocks.
    static constexpr int BV = (D >= 128) ? 128 : (D >= 64 ? 64 : D);
    static constexpr int MBW = (TM == 32 && D >= 128) ? 2 : 1;  // 16-row blocks per wave
    static constexpr int NT = D / BV;         // value tiles per head
    static constexpr int NW = BV / (16 * MBW);  // waves per block
    static constexpr int KS = (D + 31) / 32;  // MFMA k-steps over d_k
    static constexpr int QKLD = D + 8;        // bf16 row stride of Q/K in LDS
    static constexpr int FLD = TM + 4;        // fp32 row stride of the T x T factors and of R^T
    static constexpr int NBM = TM / 16;       // 16-node blocks at most
    // waves per SIMD the registers must allow: two blocks per CU at 64 nodes
    // (eight waves each), three at 32 nodes with two row blocks per wave,
    // four otherwise
    static constexpr int WPE = MBW == 2 ? 3 : 4;
    // pack X, M and R^T as bf16 hi | lo once before step 6 when eight waves
    // read them (fewer waves: splitting at each read is cheaper than the
    // extra pass and barrier)
    static constexpr bool PACK = NW >= 8;
};

template <int D, int TM, bool F32IN>
struct VLds {
    using S = VShape<D, TM>;
    static constexpr int NPLANE = F32IN ? 4 : 2;  // q, k (hi and lo planes for fp32 input)
    static constexpr size_t qk = (size_t)NPLANE * TM * S::QKLD * 2;
    static constexpr size_t rt = (size_t)S::BV * S::FLD * 4;  // R^T, after Q/K are dead
    static constexpr size_t regionA = ((qk > rt ? qk : rt) + 15) / 16 * 16;
    static constexpr size_t fac = (size_t)TM * S::FLD * 4;
    static constexpr size_t off_g = regionA;    // G, later M
    static constexpr size_t off_x = off_g + fac;
    static constexpr size_t off_anc = off_x + fac;   // uint64 [TM]
    static constexpr size_t off_f = off_anc + 8 * TM;  // float logp, P, beta [TM] each
    static constexpr size_t off_i = off_f + 12 * TM;   // int: bad flag
    static constexpr size_t total = off_i + 16;
};

template <int D, int TM, bool F32IN>
__global__ __launch_bounds__((VShape<D, TM>::NW * kWave))
__attribute__((amdgpu_waves_per_eu(VShape<D, TM>::WPE))) void verify_kernel(const VerifyArgs p) {
    using S = VShape<D, TM>;
    using L = VLds<D, TM, F32IN>;
    constexpr int BV = S::BV, NW = S::NW, KS = S::KS, QKLD = S::QKLD, FLD = S::FLD, NBM = S::NBM, MBW = S::MBW;
    constexpr int NTHR = NW * kWave;
    constexpr int EPC = F32IN ? 4 : 8;                 // elements per 16-byte chunk
    constexpr int CPR = D / EPC;                       // chunks per q/k row
    constexpr int QKC = (TM * CPR + NTHR - 1) / NTHR;  // q (and k) chunks per thread

    __shared__ __align__(16) unsigned char smem[L::total];
    unsigned short* s_q = reinterpret_cast<unsigned short*>(smem);
    unsigned short* s_k = s_q + TM * QKLD;
    unsigned short* s_qlo = s_k + TM * QKLD;  // fp32 input only
    unsigned short* s_klo = s_qlo + TM * QKLD;
    float* s_rt = reinterpret_cast<float*>(smem);  // R^T [BV][FLD], aliases Q/K once they are dead
    float* s_g = reinterpret_cast<float*>(smem + L::off_g);  // G [TM][FLD], then M
    float* s_x = reinterpret_cast<float*>(smem + L::off_x);  // X [TM][FLD]
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
    const int wrow0 = wave * 16 * MBW;        // first value row of this wave within the tile
    const int vrow0 = tile * BV + wrow0;      // first value row (of S0, o, u) of this wave

    // 1. global loads.  Every small per-node input first, so that, loads
    // completing in issue order, steps 2-4 can run while the S0 rows are in
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
    // v[n][vrow0 + 16 mi + 4g .. +3] for the node n = 16 nb + c this lane
    // holds in step 5
    u16x4 vb[MBW][NBM];
    float4 vf[MBW][NBM];
#pragma unroll
    for (int mi = 0; mi < MBW; ++mi) {
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
            const int n = min(nb * 16 + c, T - 1);
            const size_t off = ((nb0 + n) * H + h) * D + vrow0 + 16 * mi + 4 * g;
            if constexpr (F32IN) vf[mi][nb] = *reinterpret_cast<const float4*>(static_cast<const float*>(p.v) + off);
            else vb[mi][nb] = load_u16x4(static_cast<const unsigned short*>(p.v) + off);
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
    // this lane's S0 rows (A operand row c of each of the wave's 16-row blocks)
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
                *reinterpret_cast<u16x4*>(s_qlo + row * QKLD + col) = lo;
                split4(__builtin_bit_cast(float4, kv), hi, lo);
                *reinterpret_cast<u16x4*>(s_k + row * QKLD + col) = hi;
                *reinterpret_cast<u16x4*>(s_klo + row * QKLD + col) = lo;
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

    // 3. G blocks (mb, nb), nb <= mb, from K K^T; zero above the block
    //    diagonal.  Items 0 .. NB-1 are the diagonal blocks: block (i, i)
    //    goes to wave i % NW, which also solves the diagonal block of X from
    //    its G registers.
    for (int it = wave; it < NB * NB; it += NW) {
        int mb, nb;
        if (it < NB) {
            mb = nb = it;
        } else {
            const int r = it - NB;  // ordered pairs mb != nb
            mb = r / (NB - 1);
            nb = r % (NB - 1);
            if (nb >= mb) ++nb;
        }
        if (nb > mb) {  // above the diagonal: zero G (later M) and X
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = mb * 16 + 4 * g + r, m = nb * 16 + c;
                s_g[n * FLD + m] = 0.f;
                s_x[n * FLD + m] = 0.f;
            }
            continue;
        }
        floatx4 acc_g = {0.f, 0.f, 0.f, 0.f};
        const unsigned short* krow_a = s_k + (mb * 16 + c) * QKLD;
        const unsigned short* krow_b = s_k + (nb * 16 + c) * QKLD;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 bk = frag_row<D>(krow_b, s, g);
            const bf16x8 ak = frag_row<D>(krow_a, s, g);
            acc_g = mfma16x16x32(ak, bk, acc_g);
            if constexpr (F32IN) {
                acc_g = mfma16x16x32(ak, frag_row<D>(s_klo + (nb * 16 + c) * QKLD, s, g), acc_g);
                acc_g = mfma16x16x32(frag_row<D>(s_klo + (mb * 16 + c) * QKLD, s, g), bk, acc_g);
            }
        }
        // lane (c, g) holds rows n = 16 mb + 4 g + r, column m = 16 nb + c
        const int m = nb * 16 + c;
        const float lpm = s_logp[m];
        float gv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = mb * 16 + 4 * g + r;
            const uint64_t anc = s_anc[n];
            const bool on_path = m < T && n < T && (((anc | (1ull << n)) >> m) & 1ull);
            const bool strict = on_path && m != n;
            const float dec = on_path ? expf(s_logp[n] - lpm) : 0.f;
            gv[r] = strict ? s_beta[n] * dec * acc_g[r] : 0.f;
            s_g[n * FLD + m] = gv[r];
        }
        if (mb == nb) {
            // X_ii = (I + G_ii)^{-1}: lane j < 16 solves column j,
            //   x[r] = [r == j] - sum_{t < r} G[r][t] x[t],
            // with G[r][t] read from lane t + 16 (r / 4), register r % 4
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
                for (int t = 0; t < r; ++t) acc -= readlane_f(gv[r & 3], t + 16 * (r >> 2)) * x[t];
                x[r] = acc;
            }
            if (g == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s_x[(mb * 16 + r) * FLD + mb * 16 + c] = x[r];
            }
        }
    }
    __syncthreads();

    // 4a. off-diagonal blocks of X, one block diagonal d = i - j per stage:
    //     X_ij = -X_ii S, S = sum_{k=j}^{i-1} G_ik X_kj
    for (int d = 1; d < NB; ++d) {
        for (int it = wave; it < NB - d; it += NW) {
            const int j = it, i = it + d;
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
            floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
            const float* grow = s_g + (16 * i + c) * FLD;
            const float* xcol = s_x + 16 * j + c;
            // k-steps of 32 nodes over [16 j, 16 i); runs outside read as zero
            for (int s = j / 2; 32 * s < 16 * i; ++s) {
                const int k0 = 32 * s + 4 * g;
                const bool v0 = k0 >= 16 * j && k0 < 16 * i;
                const bool v1 = k0 + 16 >= 16 * j && k0 + 16 < 16 * i;
                const float4 a0 = v0 ? *reinterpret_cast<const float4*>(grow + k0) : z;
                const float4 a1 = v1 ? *reinterpret_cast<const float4*>(grow + k0 + 16) : z;
                // B[k][n] = X[k][16 j + n]: four rows down one column
                const float4 b0 = v0 ? make_float4(xcol[(k0 + 0) * FLD], xcol[(k0 + 1) * FLD], xcol[(k0 + 2) * FLD],
                                                   xcol[(k0 + 3) * FLD])
                                     : z;
                const float4 b1 = v1 ? make_float4(xcol[(k0 + 16) * FLD], xcol[(k0 + 17) * FLD],
                                                   xcol[(k0 + 18) * FLD], xcol[(k0 + 19) * FLD])
                                     : z;
                bf16x8 ah, al, bh, bl;
                split8(a0, a1, ah, al);
                split8(b0, b1, bh, bl);
                sacc = mma3(sacc, ah, al, bh, bl);
            }
            // S in C layout (lane (c, g): rows 4 g .. 4 g + 3 of column c) is
            // already the B operand of a 16-deep product
            bf16x8 sh, sl, ah, al;
            split8(make_float4(sacc[0], sacc[1], sacc[2], sacc[3]), z, sh, sl);
            split8(*reinterpret_cast<const float4*>(s_x + (16 * i + c) * FLD + 16 * i + 4 * g), z, ah, al);
            floatx4 xacc = {0.f, 0.f, 0.f, 0.f};
            xacc = mma3(xacc, ah, al, sh, sl);
#pragma unroll
            for (int r = 0; r < 4; ++r) s_x[(16 * i + 4 * g + r) * FLD + 16 * j + c] = -xacc[r];
        }
        __syncthreads();
    }

    // 4b. M = C X on the blocks (i, j), j <= i, into the G area
    //     (M_ij = sum_{k=j}^{i} C_ik X_kj; every X block is final, so G is
    //     no longer read).  The A operand, row n = 16 i + c of C at the
    //     k-slots m = 32 s + 4 g + r and m + 16, comes from the K Q^T blocks
    //     of node blocks 2 s and 2 s + 1 against block i: in the MFMA C
    //     layout those hold exactly k_m . q_n for this lane's (n, m).
    for (int it = wave; it < NB * (NB + 1) / 2; it += NW) {
        int i = 0;
        while ((i + 1) * (i + 2) / 2 <= it) ++i;
        const int j = it - i * (i + 1) / 2;
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        const int n = 16 * i + c;
        const uint64_t path_n = s_anc[n] | (1ull << n);
        const float lpn = s_logp[n];
        const unsigned short* qrow = s_q + n * QKLD;
        floatx4 macc = {0.f, 0.f, 0.f, 0.f};
        const float* xcol = s_x + 16 * j + c;
        for (int s = j / 2; 32 * s < 16 * (i + 1); ++s) {
            const int k0 = 32 * s + 4 * g;
            const bool v0 = k0 >= 16 * j && k0 < 16 * (i + 1);
            const bool v1 = k0 + 16 >= 16 * j && k0 + 16 < 16 * (i + 1);
            floatx4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = t0;  // k_m . q_n, m in blocks 2 s and 2 s + 1
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 bq = frag_row<D>(qrow, ks, g);
                const bf16x8 ak0 = frag_row<D>(s_k + (32 * s + c) * QKLD, ks, g);
                const bf16x8 ak1 = frag_row<D>(s_k + (32 * s + 16 + c) * QKLD, ks, g);
                t0 = mfma16x16x32(ak0, bq, t0);
                t1 = mfma16x16x32(ak1, bq, t1);
                if constexpr (F32IN) {
                    const bf16x8 bql = frag_row<D>(s_qlo + n * QKLD, ks, g);
                    t0 = mfma16x16x32(ak0, bql, t0);
                    t0 = mfma16x16x32(frag_row<D>(s_klo + (32 * s + c) * QKLD, ks, g), bq, t0);
                    t1 = mfma16x16x32(ak1, bql, t1);
                    t1 = mfma16x16x32(frag_row<D>(s_klo + (32 * s + 16 + c) * QKLD, ks, g), bq, t1);
                }
            }
            float ca[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m0 = k0 + r, m1 = k0 + 16 + r;
                ca[r] = (v0 && ((path_n >> m0) & 1ull)) ? expf(lpn - s_logp[m0]) * t0[r] : 0.f;
                ca[4 + r] = (v1 && ((path_n >> m1) & 1ull)) ? expf(lpn - s_logp[m1]) * t1[r] : 0.f;
            }
            const float4 b0 = v0 ? make_float4(xcol[(k0 + 0) * FLD], xcol[(k0 + 1) * FLD], xcol[(k0 + 2) * FLD],
                                               xcol[(k0 + 3) * FLD])
                                 : z;
            const float4 b1 = v1 ? make_float4(xcol[(k0 + 16) * FLD], xcol[(k0 + 17) * FLD],
                                               xcol[(k0 + 18) * FLD], xcol[(k0 + 19) * FLD])
                                 : z;
            bf16x8 ah, al, bh, bl;
            split8(make_float4(ca[0], ca[1], ca[2], ca[3]), make_float4(ca[4], ca[5], ca[6], ca[7]), ah, al);
            split8(b0, b1, bh, bl);
            macc = mma3(macc, ah, al, bh, bl);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) s_g[(16 * i + 4 * g + r) * FLD + 16 * j + c] = macc[r];
    }

    // 5. S0 Q^T and S0 K^T for the wave's value rows (A = S0 rows, split
    //    hi + lo; B = Q / K rows).  Lane (c, g) ends with value rows
    //    16 mi + 4 g + r and node n = 16 nb + c of each node block.
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
                const bf16x8 bq = frag_row<D>(s_q + (nb * 16 + c) * QKLD, s, g);
                const bf16x8 bk = frag_row<D>(s_k + (nb * 16 + c) * QKLD, s, g);
#pragma unroll
                for (int mi = 0; mi < MBW; ++mi) {
                    accq[mi][nb] = mfma16x16x32(sh[mi], bq, accq[mi][nb]);
                    accq[mi][nb] = mfma16x16x32(sl[mi], bq, accq[mi][nb]);
                    acck[mi][nb] = mfma16x16x32(sh[mi], bk, acck[mi][nb]);
                    acck[mi][nb] = mfma16x16x32(sl[mi], bk, acck[mi][nb]);
                }
                if constexpr (F32IN) {
                    const bf16x8 bql = frag_row<D>(s_qlo + (nb * 16 + c) * QKLD, s, g);
                    const bf16x8 bkl = frag_row<D>(s_klo + (nb * 16 + c) * QKLD, s, g);
#pragma unroll
                    for (int mi = 0; mi < MBW; ++mi) {
                        accq[mi][nb] = mfma16x16x32(sh[mi], bql, accq[mi][nb]);
                        acck[mi][nb] = mfma16x16x32(sh[mi], bkl, acck[mi][nb]);
                    }
                }
            }
        }
    }
    // B0^T[i][n] = P_n (S0 q_n)[i];  R^T[i][n] = beta_n (v_n[i] - P_n (S0 k_n)[i])
    floatx4 b0t[MBW][NBM];
    float rtv[MBW][NBM][4];
#pragma unroll
    for (int nb = 0; nb < NBM; ++nb) {
        const int n = nb * 16 + c;
        const bool nv = nb < NB && n < T;
        const float P = nv ? s_P[n] : 0.f, be = nv ? s_beta[n] : 0.f;
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) {
            float vv[4];
            if constexpr (F32IN) {
                vv[0] = vf[mi][nb].x;
                vv[1] = vf[mi][nb].y;
                vv[2] = vf[mi][nb].z;
                vv[3] = vf[mi][nb].w;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) vv[r] = bf16_val(vb[mi][nb][r]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                b0t[mi][nb][r] = P * accq[mi][nb][r];
                rtv[mi][nb][r] = nv ? be * (vv[r] - P * acck[mi][nb][r]) : 0.f;
            }
        }
    }
    __syncthreads();  // Q/K dead in every wave; X and M complete

    // 6. U^T = R^T X^T and O^T = B0^T + R^T M^T (K = nodes, 32 per step).
    //    R^T goes to the Q/K area; each wave reads back only the rows it
    //    wrote (LDS keeps one wave's operations in order).
    const int ksteps = (T16 + 31) / 32;
    floatx4 accu[MBW][NBM], acco[MBW][NBM];
#pragma unroll
    for (int mi = 0; mi < MBW; ++mi) {
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
            accu[mi][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
            acco[mi][nb] = b0t[mi][nb];
        }
    }
    if constexpr (S::PACK) {
        // R^T, X and M as packed hi | lo words, X and M converted in place
        uint32_t* s_rtp = reinterpret_cast<uint32_t*>(s_rt);
        uint32_t* s_xp = reinterpret_cast<uint32_t*>(s_x);
        uint32_t* s_mp = reinterpret_cast<uint32_t*>(s_g);
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) {
#pragma unroll
            for (int nb = 0; nb < NBM; ++nb) {
                if (nb < NB) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        s_rtp[(wrow0 + 16 * mi + 4 * g + r) * FLD + nb * 16 + c] = pack_hilo(rtv[mi][nb][r]);
                }
            }
        }
        for (int e = tid; e < T16 * T16; e += NTHR) {
            const int row = e / T16, col = e - row * T16;
            s_xp[row * FLD + col] = pack_hilo(s_x[row * FLD + col]);
            s_mp[row * FLD + col] = pack_hilo(s_g[row * FLD + col]);
        }
        __syncthreads();
        for (int s = 0; s < ksteps; ++s) {
            bf16x8 rh[MBW], rl[MBW];
#pragma unroll
            for (int mi = 0; mi < MBW; ++mi) frag_packed(s_rtp + (wrow0 + 16 * mi + c) * FLD, s, g, T16, rh[mi], rl[mi]);
#pragma unroll
            for (int nb = 0; nb < NBM; ++nb) {
                // rows of node block nb of X and M vanish past the block
                // (both are lower triangular): skip k-steps starting there
                // (with at most 32 nodes there is one k-step, never skipped)
                if (nb < NB && (TM <= 32 || 32 * s < 16 * (nb + 1))) {
                    bf16x8 xh, xl, mh, ml;
                    frag_packed(s_xp + (nb * 16 + c) * FLD, s, g, T16, xh, xl);
                    frag_packed(s_mp + (nb * 16 + c) * FLD, s, g, T16, mh, ml);
#pragma unroll
                    for (int mi = 0; mi < MBW; ++mi) {
                        accu[mi][nb] = mma3(accu[mi][nb], rh[mi], rl[mi], xh, xl);
                        acco[mi][nb] = mma3(acco[mi][nb], rh[mi], rl[mi], mh, ml);
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int mi = 0; mi < MBW; ++mi) {
#pragma unroll
            for (int nb = 0; nb < NBM; ++nb) {
                if (nb < NB) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        s_rt[(wrow0 + 16 * mi + 4 * g + r) * FLD + nb * 16 + c] = rtv[mi][nb][r];
                }
            }
        }
        for (int s = 0; s < ksteps; ++s) {
            bf16x8 rh[MBW], rl[MBW];
#pragma unroll
            for (int mi = 0; mi < MBW; ++mi) {
                float4 a0, a1;
                frag_f32(s_rt + (wrow0 + 16 * mi + c) * FLD, s, g, T16, a0, a1);
                split8(a0, a1, rh[mi], rl[mi]);
            }
#pragma unroll
            for (int nb = 0; nb < NBM; ++nb) {
                if (nb < NB && (TM <= 32 || 32 * s < 16 * (nb + 1))) {  // as above
                    float4 x0, x1, m0, m1;
                    frag_f32(s_x + (nb * 16 + c) * FLD, s, g, T16, x0, x1);
                    frag_f32(s_g + (nb * 16 + c) * FLD, s, g, T16, m0, m1);
                    bf16x8 xh, xl, mh, ml;
                    split8(x0, x1, xh, xl);
                    split8(m0, m1, mh, ml);
#pragma unroll
                    for (int mi = 0; mi < MBW; ++mi) {
                        accu[mi][nb] = mma3(accu[mi][nb], rh[mi], rl[mi], xh, xl);
                        acco[mi][nb] = mma3(acco[mi][nb], rh[mi], rl[mi], mh, ml);
                    }
                }
            }
        }
    }
    // lane (c, g): node n = 16 nb + c, value rows vrow0 + 16 mi + 4 g .. +3
#pragma unroll
    for (int mi = 0; mi < MBW; ++mi) {
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
            const int n = nb * 16 + c;
            if (nb < NB && n < T) {
                const size_t off = ((nb0 + n) * H + h) * D + vrow0 + 16 * mi + 4 * g;
                st_stream(p.o + off, make_float4(acco[mi][nb][0], acco[mi][nb][1], acco[mi][nb][2], acco[mi][nb][3]));
                if (p.u_out)
                    st_stream(p.u_out + off, make_float4(accu[mi][nb][0], accu[mi][nb][1], accu[mi][nb][2], accu[mi][nb][3]));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// T <= 16: one 16 x 16 node block, so one wave does the whole factor algebra
// of the head in registers, and every wave of the block then handles 16
// value rows of the head.  With a matrix P held in the MFMA C layout (lane (c, g), register r holds
// P[4 g + r][c]), the same registers are the B operand of a 16-deep product
// as they stand and the A operand of one with P transposed, so
//   mm(P, Q) = P^T Q
// needs no data movement.  K K^T is symmetric, so G and G^T (and C and C^T
// from Q K^T and K Q^T) come out of the accumulators directly, and
//   X = (I + G)^-1 = (I - G)(I + G^2)(I + G^4)(I + G^8)      (G^16 = 0)
// is built by repeated squaring, stopping at the stage the tree depth
// allows.  Then M^T = X^T C^T, R and B0^T from the state products, and
// U^T = R^T X^T, O^T = B0^T + R^T M^T.  X^T and M^T reach the other waves
// through LDS in the same C layout (one float4 per lane), and the only LDS
// staging is Q and K.

// P^T Q for 16 x 16 fp32 matrices in C layout (hi + lo split, lo * lo dropped)
__device__ __forceinline__ floatx4 mm16(const floatx4 P, const floatx4 Q) {
    u16x4 ph, pl, qh, ql;
    split4(make_float4(P[0], P[1], P[2], P[3]), ph, pl);
    split4(make_float4(Q[0], Q[1], Q[2], Q[3]), qh, ql);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma16x16x32(join(ph, pl), join(qh, qh), acc);  // (P_hi + P_lo)^T Q_hi
    return mfma16x16x32(join(ph, zero4()), join(ql, zero4()), acc);  // + P_hi^T Q_lo
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
