// Reads of states inside the verified block, without forming them (gfx950).
//
// The ReaDy page (arXiv 2610.20503, Fig. 2a) has the drafter read recurrent
// states at chosen positions.  For a position inside the block that verify
// just processed, the Bole page (arXiv 2608.01651, section IV, Eq. (9) and
// its "Lemma 1") writes every node state through the factors verify leaves:
//   S_j = P_j S0 + sum_{m on path(j)} (P_j / P_m) u_m k_m^T,
// so a read is
//   S_j q = P_j (S0 q) + sum_{m on path(j)} (P_j / P_m) (k_m . q) u_m,
// and position -1 reads S0 itself.  All positions of a (sequence, head)
// share S0, so it is read once for all P x Qn queries and no S_j is formed:
// per head the traffic is S0 plus the queries and outputs, where a gather of
// formed states reads one state per position.
//
// One workgroup per (sequence, head, value tile of BV rows, chunk of 64
// queries), one wave per 16 value rows:
//   1. issue the loads of the query chunk, K, the U tile, log P, the
//      positions and the parent row, then the wave's S0 rows straight into
//      MFMA operand registers (they stay in flight through steps 2-3);
//   2. stage Q, K in LDS; wave 0 turns the parent row into ancestor-or-self
//      masks by pointer doubling;
//   3. W[m, f] = [m on path(j_f)] exp(log P_j - log P_m) (k_m . q_f) on
//      MFMA, one 16-query column block per wave, into registers, then
//      S0 Q^T on MFMA; once every wave is done with Q and K, W^T and U^T go
//      as bf16 hi and lo planes into their place, so that LDS holds little
//      more than Q and K (four blocks per CU at 64 nodes) and step 4 splits
//      nothing;
//   4. O^T = (S0 Q^T) diag(P_j) + U^T W on MFMA (S0, U and W carried as
//      bf16 hi + lo terms); on large grids the O tile goes through LDS so
//      that every store writes whole rows of o, else float4 stores straight
//      from the accumulators.
#include <limits.h>

#include "ldv_device.hpp"
#include "ldv_kernels.hpp"

#include "../../include/ldv.h"

namespace ldv {

constexpr float kLog2e = 1.44269504088896341f;  // log2 of e

// Grids above this many blocks (more than about two rounds on 256 CUs) stage
// the O tile in LDS before storing it: measured 8.6% faster on the 27B-hybrid
// shape (4096 blocks) and 5.7% on batch-256, 2-3% slower on the tree-64 and
// GDN-1.3B shapes (1024 and 512 blocks).
constexpr long long kReadStageBlocks = 2048;

template <int D, int TM>
struct RShape {
    static constexpr int BV = D >= 64 ? 64 : D;  // value rows per block
    static constexpr int NT = D / BV;            // value tiles per head
    static constexpr int NW = BV / 16;           // waves per block
    static constexpr int KS = (D + 31) / 32;     // MFMA k-steps over d_k
    static constexpr int NQ = 64;                // queries per block (one per lane of wave 0)
    static constexpr int NCB = NQ / 16;          // 16-query column blocks
    static constexpr int QKLD = D + 8;           // bf16 row stride of Q / K in LDS
    static constexpr int WTLD = TM + 8;          // bf16 row stride of the W^T planes
    static constexpr int OLD = BV + 4;           // fp32 row stride of the staged O tile
    static constexpr int NKS = (TM + 31) / 32;   // MFMA k-steps over nodes
    static constexpr int LOG2TM = TM <= 16 ? 4 : (TM <= 32 ? 5 : 6);
};

template <int D, int TM, bool F32IN>
struct RLds {
    using S = RShape<D, TM>;
    static constexpr int NPL = F32IN ? 2 : 1;  // bf16 planes per operand (hi, then lo)
    static constexpr size_t off_k = (size_t)NPL * S::NQ * S::QKLD * 2;
    static constexpr size_t qk = off_k + (size_t)NPL * TM * S::QKLD * 2;
    // once Q and K are dead, their area holds the W^T hi and lo planes
    // [NQ][WTLD] and the U^T hi and lo planes [BV][WTLD] (bf16)
    static constexpr size_t off_ut = (size_t)2 * S::NQ * S::WTLD * 2;
    static constexpr size_t wu = off_ut + (size_t)2 * S::BV * S::WTLD * 2;
    // once the planes are dead too, the fp32 O tile [NQ][OLD] for the stores
    static constexpr size_t ot = (size_t)S::NQ * S::OLD * 4;
    static constexpr size_t big = qk > wu ? (qk > ot ? qk : ot) : (wu > ot ? wu : ot);
    static constexpr size_t off_anc = (big + 15) / 16 * 16;
    static constexpr size_t off_lp = off_anc + 8 * TM;
    static constexpr size_t off_pos = off_lp + 4 * TM;
    static constexpr size_t off_flag = off_pos + 4 * S::NQ;
    static constexpr size_t total = off_flag + 16;
    // waves per SIMD the registers must allow: what this block's LDS
    // (160 KiB per CU) lets reside, at most four
    static constexpr int lds_waves = (int)(163840 / total) * S::NW / 4;
    static constexpr int WPE = lds_waves < 1 ? 1 : (lds_waves < 4 ? lds_waves : 4);
};

template <int D, int TM, bool F32IN>
__global__ __launch_bounds__((RShape<D, TM>::NW * kWave))
__attribute__((amdgpu_waves_per_eu(RLds<D, TM, F32IN>::WPE))) void read_kernel(const ReadArgs p) {
    using S = RShape<D, TM>;
    using L = RLds<D, TM, F32IN>;
    constexpr int BV = S::BV, NW = S::NW, KS = S::KS, NQ = S::NQ, NCB = S::NCB;
    constexpr int QKLD = S::QKLD, WTLD = S::WTLD, NKS = S::NKS;
    constexpr int NTHR = NW * kWave;
    constexpr int EPC = F32IN ? 4 : 8;  // elements per 16-byte chunk
    constexpr int CPR = D / EPC;        // chunks per q/k row
    constexpr int QC = (NQ * CPR + NTHR - 1) / NTHR;
    constexpr int KC = (TM * CPR + NTHR - 1) / NTHR;
    static_assert(NQ == kWave, "one query column per lane of wave 0");
    // On grids of one round (every block resident at once) the blocks run in
    // lockstep and each CU's older blocks win the issue arbitration; each wave
    // lowers its priority as it advances (3, then 2 after staging, 1 once Q
    // and K are dead, 0 for step 4), so that issue goes to the waves that are
    // behind: tree-64 20.4 -> 19.5 us, GDN-1.3B 9.85 -> 9.55 us.
    // blocks of this kernel resident per CU: what its LDS and its register
    // bound (waves per SIMD) allow
    constexpr int RES = (163840 / (int)L::total) < (4 * L::WPE / NW) ? (163840 / (int)L::total) : (4 * L::WPE / NW);
    const bool lockstep = gridDim.x <= (unsigned)(RES * kCus);
    if (lockstep) __builtin_amdgcn_s_setprio(3);

    __shared__ __align__(16) unsigned char smem[L::total];
    unsigned short* s_q = reinterpret_cast<unsigned short*>(smem);           // [NQ][QKLD] hi, then lo
    unsigned short* s_k = reinterpret_cast<unsigned short*>(smem + L::off_k);  // [TM][QKLD] hi, then lo
    unsigned short* s_wt = reinterpret_cast<unsigned short*>(smem);          // [NQ][WTLD] hi, then lo (after Q, K)
    unsigned short* s_ut = reinterpret_cast<unsigned short*>(smem + L::off_ut);  // [BV][WTLD] hi, then lo (after Q, K)
    uint64_t* s_anc = reinterpret_cast<uint64_t*>(smem + L::off_anc);       // [TM]
    float* s_lp = reinterpret_cast<float*>(smem + L::off_lp);                // [TM]
    int* s_pos = reinterpret_cast<int*>(smem + L::off_pos);                  // [NQ]
    int* s_flag = reinterpret_cast<int*>(smem + L::off_flag);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int T = p.T, H = p.H, P = p.P, Qn = p.Qn;
    const int NQT = P * Qn;  // queries per (sequence, head), flattened f = p Qn + i
    const int nch = (NQT + NQ - 1) / NQ;
    // units of kSpreadHeads heads spread over the XCDs as in verify and
    // commit (a unit's blocks stay on one XCD)
    const unsigned per = kSpreadHeads * (unsigned)(S::NT * nch);  // blocks of a unit of heads
    const unsigned bid = xcd_spread(blockIdx.x, gridDim.x / per, per);
    const int ch = (int)(bid % (unsigned)nch);
    const unsigned r1 = bid / (unsigned)nch;
    const int tile = (int)(r1 % S::NT);
    const unsigned bh = r1 / S::NT;
    const int h = (int)(bh % (unsigned)H), b = (int)(bh / (unsigned)H);
    const int f0 = ch * NQ;
    const int vrow0 = tile * BV + __builtin_amdgcn_readfirstlane(wave) * 16;

    // 1. loads, small ones first, branch-free (indices clamped into range;
    // values past the ends are dropped when LDS is written)
    const char* qbase = static_cast<const char*>(p.queries);
    u32x4 qreg[QC];
#pragma unroll
    for (int i = 0; i < QC; ++i) {
        const int chunk = tid + i * NTHR, col = (chunk % CPR) * EPC;
        const int f = min(f0 + min(chunk / CPR, NQ - 1), NQT - 1);
        const int pp = f / Qn, ii = f - pp * Qn;
        const size_t off = (((((size_t)b * P + pp) * H + h) * Qn + ii) * D + col) * (F32IN ? 4 : 2);
        qreg[i] = *reinterpret_cast<const u32x4*>(qbase + off);
    }
    u32x4 kreg[KC];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int chunk = tid + i * NTHR, col = (chunk % CPR) * EPC;
        const int m = min(chunk / CPR, T - 1);
        const size_t off = ((((size_t)b * T + m) * H + h) * D + col) * (F32IN ? 4 : 2);
        kreg[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.k) + off);
    }
    const int nl = min(lane, T - 1);
    const float lp_ld = p.logp[((size_t)b * T + nl) * H + h];
    // a chain has no parent array: read the log-gate array instead (it has at
    // least B * T entries) and discard the value
    const global_ptr<const int32_t> parp =
        (global_ptr<const int32_t>)(p.parent ? p.parent : reinterpret_cast<const int32_t*>(p.logp));
    const int par_ld = parp[(size_t)b * T + nl];
    const global_ptr<const int32_t> posp = (global_ptr<const int32_t>)p.pos;
    const int pos_ld = posp[(size_t)b * P + min(f0 + lane, NQT - 1) / Qn];  // position of query column `lane`
    const int need_ld = posp[(size_t)b * P + min(tid, P - 1)];                // for the parent-row check
    const float* s0row = p.S0 + (((size_t)b * H + h) * D + vrow0 + c) * D;
    float4 sreg[KS][2];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int k0 = 32 * s + 4 * g;
        sreg[s][0] = (k0 < D) ? ld_stream(s0row + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
        sreg[s][1] = (k0 + 16 < D) ? ld_stream(s0row + k0 + 16) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // the U tile (nodes x this block's BV values), float4 per thread
    constexpr int U4 = BV / 4;  // float4 chunks per U row of the tile
    constexpr int UC = (TM * U4 + NTHR - 1) / NTHR;
    float4 ureg[UC];
#pragma unroll
    for (int i = 0; i < UC; ++i) {
        const int chunk = tid + i * NTHR;
        const int m = min(chunk / U4, T - 1);
        ureg[i] = *reinterpret_cast<const float4*>(p.u + (((size_t)b * T + m) * H + h) * D + tile * BV +
                                                   4 * (chunk % U4));
    }
    asm volatile("" ::: "memory");  // keep the loads above ahead of any use of them

    // 2a. stage Q, K (rows past the ends zero)
    const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < QC; ++i) {
        const int chunk = tid + i * NTHR, row = chunk / CPR, col = (chunk % CPR) * EPC;
        if (row < NQ) {
            const u32x4 qv = (f0 + row < NQT) ? qreg[i] : z4;
            if constexpr (!F32IN) {
                *reinterpret_cast<u32x4*>(s_q + row * QKLD + col) = qv;
            } else {
                u16x4 hi, lo;
                split4(__builtin_bit_cast(float4, qv), hi, lo);
                *reinterpret_cast<u16x4*>(s_q + row * QKLD + col) = hi;
                *reinterpret_cast<u16x4*>(s_q + (NQ + row) * QKLD + col) = lo;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int chunk = tid + i * NTHR, row = chunk / CPR, col = (chunk % CPR) * EPC;
        if (row < TM) {
            const u32x4 kv = row < T ? kreg[i] : z4;
            if constexpr (!F32IN) {
                *reinterpret_cast<u32x4*>(s_k + row * QKLD + col) = kv;
            } else {
                u16x4 hi, lo;
                split4(__builtin_bit_cast(float4, kv), hi, lo);
                *reinterpret_cast<u16x4*>(s_k + row * QKLD + col) = hi;
                *reinterpret_cast<u16x4*>(s_k + (TM + row) * QKLD + col) = lo;
            }
        }
    }

    // 2b. wave 0: per-query positions, log P, ancestor-or-self masks
    if (wave == 0) {
        s_pos[lane] = (f0 + lane < NQT) ? pos_ld : INT_MIN;
        const int n = lane;
        const bool valid = n < T;
        const int par = p.parent ? par_ld : n - 1;
        const bool bad = valid && (par < -1 || par >= n);
        const bool anybad = __ballot(bad) != 0ull;
        // pointer doubling: `set` covers the path segment from n up to (not
        // including) jmp
        uint64_t set = valid ? (1ull << n) : 0ull;
        int jmp = (valid && !bad) ? par : -1;
#pragma unroll
        for (int it = 0; it < S::LOG2TM; ++it) {
            const int src = jmp >= 0 ? jmp : n;
            const uint64_t set_j = shfl_u64(set, src);
            const int jmp_j = __shfl(jmp, src, kWave);
            if (jmp >= 0) {
                set |= set_j;
                jmp = jmp_j;
            }
        }
        if (n < TM) {
            s_anc[n] = set;
            s_lp[n] = valid ? lp_ld : 0.f;
        }
        if (lane == 0) s_flag[0] = anybad ? 1 : 0;
    }
    // the parent row matters only if some valid position of the sequence is a node
    int need = tid < P && need_ld >= 0 && need_ld < T;
    for (int pp = tid + NTHR; pp < P; pp += NTHR) {
        const int j = p.pos[(size_t)b * P + pp];
        need |= (j >= 0 && j < T);
    }
    need = __syncthreads_or(need);  // also the barrier after staging
    if (lockstep) __builtin_amdgcn_s_setprio(2);
    if (s_flag[0] && need) {
        if (tid == 0 && h == 0 && tile == 0 && ch == 0 && p.status) atomicOr(p.status, LDV_STATUS_BAD_PARENT);
        return;  // invalid parent row: nothing of the sequence is written
    }

    // 3a. W[m][f] = [m on path(j_f)] (P_j / P_m) k_m . q_f for the wave's
    //     column blocks (needs only Q, K: it runs while the S0 rows are in
    //     flight), kept in registers until Q and K are dead
    constexpr int CBW = (NCB + NW - 1) / NW;  // column blocks per wave
    floatx4 wreg[CBW][TM / 16];
#pragma unroll
    for (int t = 0; t < CBW; ++t) {
        const int cb = wave + t * NW;
        if (cb < NCB) {
            const int fcol = cb * 16 + c;
            const int j = s_pos[fcol];
            const bool node = j >= 0 && j < T;
            const uint64_t am = node ? s_anc[j] : 0ull;
            const float lpj = node ? s_lp[j] : 0.f;
#pragma unroll
            for (int mb = 0; mb < TM / 16; ++mb) {
                const float4 lm4 = *reinterpret_cast<const float4*>(s_lp + mb * 16 + 4 * g);
                const float lm[4] = {lm4.x, lm4.y, lm4.z, lm4.w};
                floatx4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 bk = frag_row<D>(s_k + (mb * 16 + c) * QKLD, s, g);
                    const bf16x8 bq = frag_row<D>(s_q + fcol * QKLD, s, g);
                    w = mfma16x16x32(bk, bq, w);
                    if constexpr (F32IN) {
                        w = mfma16x16x32(bk, frag_row<D>(s_q + (NQ + fcol) * QKLD, s, g), w);
                        w = mfma16x16x32(frag_row<D>(s_k + (TM + mb * 16 + c) * QKLD, s, g), bq, w);
                    }
                }
                // (no branch: the mask selects; P_j / P_m as the hardware's 2^x of the
                // difference in log2 units, which loses accuracy only where the
                // ratio is too small to matter)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = mb * 16 + 4 * g + r;
                    const float x = __builtin_amdgcn_exp2f((lpj - lm[r]) * kLog2e) * w[r];
                    wreg[t][mb][r] = ((am >> m) & 1ull) ? x : 0.f;
                }
            }
        }
    }
    // 3b. S0 Q^T for the wave's 16 value rows (once the S0 rows are in):
    //     lane (c, g) of column block cb holds query f0 + 16 cb + c, values
    //     vrow0 + 4 g .. +3
    floatx4 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        bf16x8 sh, sl;
        split8(sreg[s][0], sreg[s][1], sh, sl);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const bf16x8 bq = frag_row<D>(s_q + (cb * 16 + c) * QKLD, s, g);
            acc[cb] = mfma16x16x32(sh, bq, acc[cb]);
            acc[cb] = mfma16x16x32(sl, bq, acc[cb]);
            if constexpr (F32IN) acc[cb] = mfma16x16x32(sh, frag_row<D>(s_q + (NQ + cb * 16 + c) * QKLD, s, g), acc[cb]);
        }
    }

    __syncthreads();  // Q and K dead in every wave
    if (lockstep) __builtin_amdgcn_s_setprio(1);
    // 3c. W^T into the Q / K area as bf16 hi and lo planes: row f, the four
    //     nodes 16 mb + 4 g .. +3 of this lane
#pragma unroll
    for (int t = 0; t < CBW; ++t) {
        const int cb = wave + t * NW;
        if (cb < NCB) {
            const int f = cb * 16 + c;
#pragma unroll
            for (int mb = 0; mb < TM / 16; ++mb) {
                u16x4 hi, lo;
                split4(make_float4(wreg[t][mb][0], wreg[t][mb][1], wreg[t][mb][2], wreg[t][mb][3]), hi, lo);
                *reinterpret_cast<u16x4*>(s_wt + f * WTLD + mb * 16 + 4 * g) = hi;
                *reinterpret_cast<u16x4*>(s_wt + (NQ + f) * WTLD + mb * 16 + 4 * g) = lo;
            }
        }
    }
    //     U^T likewise: the four values of this thread's chunk of node m go
    //     to rows v .. v + 3 of the U^T planes (nodes past T zero)
#pragma unroll
    for (int i = 0; i < UC; ++i) {
        const int chunk = tid + i * NTHR, m = chunk / U4, v = 4 * (chunk % U4);
        if (m < TM) {
            const float4 uv = m < T ? ureg[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            u16x4 hi, lo;
            split4(uv, hi, lo);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s_ut[(v + e) * WTLD + m] = hi[e];
                s_ut[(BV + v + e) * WTLD + m] = lo[e];
            }
        }
    }
    __syncthreads();
    if (lockstep) __builtin_amdgcn_s_setprio(0);

    // 4. O^T = (S0 Q^T) diag(P_j) + U^T W
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int j = s_pos[cb * 16 + c];
        const float Pj = (j >= 0 && j < T) ? __builtin_amdgcn_exp2f(s_lp[j] * kLog2e) : 1.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[cb][r] *= Pj;
    }
    const unsigned short* urow = s_ut + (wave * 16 + c) * WTLD;  // U^T row of value vrow0 + c
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        const bf16x8 uh = frag_row<TM>(urow, s, g), ul = frag_row<TM>(urow + BV * WTLD, s, g);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const unsigned short* wrow = s_wt + (cb * 16 + c) * WTLD;
            const bf16x8 wh = frag_row<TM>(wrow, s, g);
            const bf16x8 wl = frag_row<TM>(wrow + NQ * WTLD, s, g);
            acc[cb] = mma3(acc[cb], uh, ul, wh, wl);
        }
    }
    // Stores.  With many blocks the block's O tile goes through LDS (over the
    // dead planes), so that each store instruction writes whole rows (16
    // consecutive lanes cover one query's BV values); a grid of one or two
    // rounds of blocks is latency-bound and stores straight from the
    // accumulators (each lane four values of one query).
    if (p.stage_o) {
        constexpr int OLD = S::OLD;
        float* s_ot = reinterpret_cast<float*>(smem);  // [NQ][OLD]
        __syncthreads();  // every wave is done with the W^T and U^T planes
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            *reinterpret_cast<float4*>(s_ot + (cb * 16 + c) * OLD + wave * 16 + 4 * g) =
                make_float4(acc[cb][0], acc[cb][1], acc[cb][2], acc[cb][3]);
        __syncthreads();
        for (int k = tid; k < NQ * (BV / 4); k += NTHR) {
            const int fl = k / (BV / 4), v4 = 4 * (k % (BV / 4));
            const int f = f0 + fl, j = s_pos[fl];
            if (f < NQT && j >= -1 && j < T) {
                const int pp = f / Qn, ii = f - pp * Qn;
                const size_t off = ((size_t)b * P + pp) * p.o.ld + p.o.col + ((size_t)h * Qn + ii) * D + tile * BV + v4;
                st_stream_out4(p.o.base, p.o.bf16, off, *reinterpret_cast<const float4*>(s_ot + fl * OLD + v4));
            }
        }
    } else {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int f = f0 + cb * 16 + c, j = s_pos[cb * 16 + c];
            if (f < NQT && j >= -1 && j < T) {
                const int pp = f / Qn, ii = f - pp * Qn;
                const size_t off = ((size_t)b * P + pp) * p.o.ld + p.o.col + ((size_t)h * Qn + ii) * D + vrow0 + 4 * g;
                st_stream_out4(p.o.base, p.o.bf16, off, make_float4(acc[cb][0], acc[cb][1], acc[cb][2], acc[cb][3]));
            }
        }
    }
    // positions outside [-1, T-1]: reported by the blocks of head 0, tile 0
    if (h == 0 && tile == 0 && wave == 0 && p.status) {
        const int j = s_pos[lane];
        const bool badp = f0 + lane < NQT && (j < -1 || j >= T);
        if (__ballot(badp) != 0ull && lane == 0) atomicOr(p.status, LDV_STATUS_BAD_POSITION);
    }
}

template <int D, int TM, bool F32IN>
static hipError_t launch_t(const ReadArgs& a, hipStream_t st) {
    using S = RShape<D, TM>;
    const long long nch = ((long long)a.P * a.Qn + S::NQ - 1) / S::NQ;
    const long long nblk = (long long)a.B * a.H * S::NT * nch;
    if (nblk <= 0) return hipSuccess;
    ReadArgs a2 = a;
    a2.stage_o = nblk > kReadStageBlocks;
    hipLaunchKernelGGL((read_kernel<D, TM, F32IN>), dim3((unsigned)nblk), dim3(S::NW * kWave), 0, st, a2);
    return hipGetLastError();
}

template <int D, bool F32IN>
static hipError_t launch_d(const ReadArgs& a, hipStream_t st) {
    if (a.T <= 16) return launch_t<D, 16, F32IN>(a, st);
    if (a.T <= 32) return launch_t<D, 32, F32IN>(a, st);
    return launch_t<D, 64, F32IN>(a, st);
}

template <bool F32IN>
static hipError_t launch_f(const ReadArgs& a, hipStream_t st) {
    switch (a.D) {
        case 16: return launch_d<16, F32IN>(a, st);
        case 32: return launch_d<32, F32IN>(a, st);
        case 64: return launch_d<64, F32IN>(a, st);
        case 128: return launch_d<128, F32IN>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_read(const ReadArgs& a, bool f32_inputs, hipStream_t stream) {
    return f32_inputs ? launch_f<true>(a, stream) : launch_f<false>(a, stream);
}

}  // namespace ldv
