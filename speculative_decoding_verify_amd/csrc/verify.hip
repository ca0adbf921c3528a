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
// operands go in as bf16 hi + lo terms (two MFMAs, see Frag16).
//
// One kernel serves drafts of up to 16, 32 and 64 nodes (TM), with one
// workgroup per (sequence, head, value tile of BV columns): G and C do not
// depend on the value channel (Eq. (7) context), so value tiles are
// independent; at d = 128 a tile is the whole head, so the T x T factor
// work is done once per head.  Each wave owns one 16-row value block of the
// tile (two at 32 nodes).  Per workgroup:
//   1. issue the loads of the parent row and gates, q, k and v (through
//      buffer views that end at node T - 1), then of the wave's S0 rows
//      (fp32) straight into MFMA operand registers; the S0 loads stay in
//      flight through steps 2-3;
//   2. stage Q, K (bf16) in LDS; wave 0 turns the parent row into ancestor
//      masks and log P by pointer doubling;
//   3. the factor tiles, spread over the waves: each is a 16 x 16 product of
//      K or Q rows on MFMA, masked and decay-scaled in the accumulators and
//      kept in LDS as doubled bf16 operands:
//        X_ii^T  (by repeated squaring of G_ii, on MFMA),
//        -G_ik^T (k < i),  C_ji^T (i <= j);
//   4. S0 Q^T (value-major) and K S0^T (node-major) on MFMA give B0^T and R
//      for the wave's value rows;
//   5. per node block i: Y = R_i - sum_k G_ik U_k, then U_i = X_ii Y (kept
//      for the later blocks) and U_i^T = Y^T X_ii^T (stored), and
//      O_j^T += U_i^T C_ji^T for j >= i; O_i^T is then complete and stored,
//      each lane writing four consecutive values of one node (float4), or,
//      on large grids, node block i's U^T and O^T tiles go through LDS so
//      that every store writes whole rows of one node (at 64 nodes all four
//      node blocks at the end, over the dead Q/K rows and factor tiles).
//   6. (long chains, every 64-node chunk but the last) the state at node
//      T - 1,
//        S = P S0 + sum_{m on its path} (P / P_m) u_m k_m^T   (Eq. (9)),
//      from the U blocks still in registers: K goes transposed into the
//      factor-tile area, and each wave forms its 16 value rows of S on MFMA,
//      so the next chunk's base costs one read and one write of the state
//      instead of a commit kernel's second pass over S0, u and k.  One
//      launch may run several chunks: each block then runs steps 1-6 for its
//      head's chunks in order.
// Two workgroup barriers (after step 2 and after step 3), and two more per
// node block when the outputs are staged (two in all at 64 nodes; two more
// for step 6).
// Inside the kernel log P is kept in base 2: log2 a from the hardware's
// log2 (clamped at -126, so that a zero gate gives a finite log), summed
// along the path; P_n / P_m = 2^(log2 P_n - log2 P_m) from the hardware's
// 2^x, used only for ancestor pairs (exponent <= 0 for gates in [0, 1]).
// The natural log P is what the kernel writes out.
#include "ldv_device.hpp"
#include "ldv_kernels.hpp"

#include "../../include/ldv.h"

namespace ldv {

constexpr float kLn2 = 0.693147180559945309f;  // natural log of 2

// A 16 x 16 fp32 matrix held in the C layout, as bf16 operand forms: the
// pair [hi | lo] (k-slots 8 g .. 8 g + 3 take rows 4 g .. 4 g + 3 of the hi
// term, 8 g + 4 .. 8 g + 7 the same rows of the lo term) and the doubled
// forms [hi | hi], [lo | lo].  mm(P, Q) = P^T Q takes one operand as a pair
// and the other doubled, on either side:
//   P^T Q = MFMA([P_hi|P_lo], [Q_hi|Q_hi]) + MFMA([P_hi|P_lo], [Q_lo|Q_lo])
//         = MFMA([P_hi|P_hi], [Q_hi|Q_lo]) + MFMA([P_lo|P_lo], [Q_hi|Q_lo])
//         = (P_hi + P_lo)^T (Q_hi + Q_lo),
// every cross term kept.  Factor tiles are stored doubled (read straight
// into operand registers); values a wave produces and reuses are kept as
// pairs (four registers).
struct Frag16 {
    bf16x8 pr, dh, dl;
};

__device__ __forceinline__ Frag16 frag16(const floatx4 v) {
    u16x4 hi, lo;
    split4(make_float4(v[0], v[1], v[2], v[3]), hi, lo);
    return Frag16{join(hi, lo), join(hi, hi), join(lo, lo)};
}

__device__ __forceinline__ bf16x8 pair16(const floatx4 v) {
    u16x4 hi, lo;
    split4(make_float4(v[0], v[1], v[2], v[3]), hi, lo);
    return join(hi, lo);
}

// acc + P^T Q, P as a pair and Q doubled
__device__ __forceinline__ floatx4 mm16f(floatx4 acc, const bf16x8 p_pr, const bf16x8 q_dh, const bf16x8 q_dl) {
    acc = mfma16x16x32(p_pr, q_dh, acc);
    return mfma16x16x32(p_pr, q_dl, acc);
}

// acc + P^T Q, P doubled and Q as a pair
__device__ __forceinline__ floatx4 mm16d(floatx4 acc, const bf16x8 p_dh, const bf16x8 p_dl, const bf16x8 q_pr) {
    acc = mfma16x16x32(p_dh, q_pr, acc);
    return mfma16x16x32(p_dl, q_pr, acc);
}

// P^T Q for 16 x 16 fp32 matrices in the C layout
__device__ __forceinline__ floatx4 mm16(const floatx4 P, const floatx4 Q) {
    const Frag16 fp = frag16(P), fq = frag16(Q);
    return mm16f(floatx4{0.f, 0.f, 0.f, 0.f}, fp.pr, fq.dh, fq.dl);
}

// I + s P for a C-layout matrix (s = +1 or -1), lane (c, g)
__device__ __forceinline__ floatx4 ident_plus(const floatx4 P, float sgn, int c, int g) {
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = sgn * P[i] + ((4 * g + i == c) ? 1.f : 0.f);
    return r;
}

// Factor tiles in LDS, one operand form per slot: 16 bytes per lane, so
// that a wave reads or writes a slot with conflict-free 128-bit accesses
// straight from or into its operand registers.
__device__ __forceinline__ void slot_store(bf16x8* slots, int s, int lane, const bf16x8 v) { slots[s * kWave + lane] = v; }
__device__ __forceinline__ bf16x8 slot_load(const bf16x8* slots, int s, int lane) { return slots[s * kWave + lane]; }

template <int D, int TM>
struct VShape {
    // At d = 128 a block keeps the whole head (BV = 128), so the factor work
    // is done once per head: eight waves of 16 value rows at 16 and 64
    // nodes, four waves of two 16-row blocks (MBW = 2) at 32 nodes, where
    // each factor tile read from LDS then serves two row blocks.
    static constexpr int BV = (D >= 128) ? 128 : (D >= 64 ? 64 : D);
    static constexpr int MBW = (TM == 32 && D >= 128) ? 2 : 1;  // 16-row blocks per wave
    static constexpr int NT = D / BV;         // value tiles per head
    static constexpr int NW = BV / (16 * MBW);  // waves per block
    static constexpr int KS = (D + 31) / 32;  // MFMA k-steps over d_k
    static constexpr int QKLD = D + 8;        // bf16 row stride of Q/K in LDS
    static constexpr int NBM = TM / 16;       // 16-node blocks at most
    // factor tiles, doubled ([hi | hi] at slot s, [lo | lo] at s + 1):
    // X_ii^T at 2 i, -G_ik^T (k < i) at SG0 + 2 (i (i - 1) / 2 + k),
    // C_ji^T (i <= j) at SC0 + 2 (j (j + 1) / 2 + i)
    static constexpr int SG0 = 2 * NBM;
    static constexpr int SC0 = SG0 + NBM * (NBM - 1);
    static constexpr int NSLOT = SC0 + NBM * (NBM + 1);
    // waves per SIMD the registers must allow: two blocks per CU at 64 nodes
    // (eight waves each), three at 32 nodes with two row blocks per wave,
    // four otherwise
    static constexpr int WPE = MBW == 2 ? 3 : 4;
};

template <int D, int TM, bool F32IN, bool STG>
struct VLds {
    using S = VShape<D, TM>;
    static constexpr int NPLANE = F32IN ? 4 : 2;  // q, k (hi and lo planes for fp32 input)
    static constexpr size_t qk = (size_t)NPLANE * TM * S::QKLD * 2;
    static constexpr size_t off_t = (qk + 15) / 16 * 16;                        // factor-tile slots
    static constexpr size_t off_anc = off_t + (size_t)S::NSLOT * kWave * 16;  // uint64 [TM]
    static constexpr size_t off_f = off_anc + 8 * TM;  // float logp, P, beta [TM] each
    static constexpr size_t off_i = off_f + 12 * TM;   // int: bad flag
    // staged outputs (large grids): the O^T and U^T tiles of one node block
    // as fp32 [node][value] rows of SLD.  With one node block they go over
    // everything above once the substitution is done.  With more, the
    // factor tiles are still in use, and they go over the Q and K rows (dead
    // once the state products are done) where those are large enough, else
    // into an area of their own.
    static constexpr int SLD = S::BV + 4;
    static constexpr size_t stage = STG ? (size_t)2 * 16 * SLD * 4 : 0;
    static constexpr bool own = S::NBM > 1 && qk < stage;
    static constexpr size_t off_stg = own ? (off_i + 16 + 15) / 16 * 16 : 0;
    // S0 rows through LDS (16- and 32-node kernels at d = 128, bf16 inputs): each wave's
    // rows, S0C columns at a time (two passes with one row block per wave,
    // four with two, so that three 32-node blocks still fit a CU); the
    // staged outputs may overlay this area (S0 is used up by then)
    static constexpr bool cs0 = D == 128 && !F32IN && (TM == 16 || TM == 32);
    static constexpr int S0C = S::MBW == 1 ? 64 : 32;  // columns per pass
    static constexpr int S0LD = S0C + 4;                // padded LDS row (floats)
    static constexpr size_t end_i = own ? off_stg + stage : off_i + 16;
    static constexpr size_t off_s0 = (end_i + 15) / 16 * 16;
    static constexpr size_t end_s0 = cs0 ? off_s0 + (size_t)S::NW * 16 * S::MBW * S0LD * 4 : end_i;
    static constexpr size_t total = (own || S::NBM > 1 || end_s0 > stage) ? end_s0 : stage;
    // waves per SIMD that the registers must allow: the shape's target, or
    // fewer where this block's LDS (160 KiB per CU) already caps residency
    static constexpr int lds_waves = (int)(163840 / total) * S::NW / 4;
    static constexpr int WPE = lds_waves < 1 ? 1 : (lds_waves < S::WPE ? lds_waves : S::WPE);
};

// STG: outputs staged in LDS and stored as whole rows.  CMT: a 64-node chunk
// of a long chain of pa.Ts nodes, with step 6; with LOOP, pa.chunks chunks.
// The looping form runs one block per CU, so its registers need only allow
// that block's waves (two per SIMD at d = 128): with the four-wave limit of
// the other forms it spilled, and measured 290 vs 274 us on the GDN-1.3B
// shape's 1024-node chain.
template <int D, int TM, bool F32IN, bool STG, bool CMT, bool LOOP>
__global__ __launch_bounds__((VShape<D, TM>::NW * kWave))
__attribute__((amdgpu_waves_per_eu(LOOP ? (VShape<D, TM>::NW + 3) / 4 : VLds<D, TM, F32IN, STG>::WPE)))
void verify_kernel(const VerifyArgs pa) {
    using S = VShape<D, TM>;
    using L = VLds<D, TM, F32IN, STG>;
    constexpr int BV = S::BV, NW = S::NW, KS = S::KS, QKLD = S::QKLD, NBM = S::NBM, MBW = S::MBW;
    constexpr int NTHR = NW * kWave;
    constexpr int EPC = F32IN ? 4 : 8;                 // elements per 16-byte chunk
    constexpr int CPR = D / EPC;                       // chunks per q/k row
    constexpr int QKC = (TM * CPR + NTHR - 1) / NTHR;  // q (and k) chunks per thread
    constexpr int LO = 2 * TM * QKLD;                  // offset of the lo planes (fp32 input)

    __shared__ __align__(16) unsigned char smem[L::total];
    unsigned short* s_q = reinterpret_cast<unsigned short*>(smem);
    unsigned short* s_k = s_q + TM * QKLD;
    bf16x8* s_sl = reinterpret_cast<bf16x8*>(smem + L::off_t);
    uint64_t* s_anc = reinterpret_cast<uint64_t*>(smem + L::off_anc);
    float* s_logp = reinterpret_cast<float*>(smem + L::off_f);
    float* s_P = s_logp + TM;
    float* s_beta = s_P + TM;
    int* s_int = reinterpret_cast<int*>(smem + L::off_i);

    // CMT: pa.chunks chunks of a long chain from node pa.t0.  Each block
    // walks its head's chunks in order, each from the state the previous
    // chunk formed in S_next (step 6).  Within a launch, every element a
    // chunk reads of that state was written by the same lane at the end of
    // the previous chunk, and the log P base is carried in a register, so no
    // block reads what another block wrote in the same launch.
    static_assert(!LOOP || CMT, "only chunks of a long chain loop");
    // One round of staged 64-node blocks (the tree-64 shape: two per CU) runs
    // in lockstep, and the older block of each CU wins the issue arbitration:
    // it ended about 5 us before the other, which then ran alone at half
    // occupancy.  Each wave lowers its priority as it advances (3 until the
    // barrier after the topology, 2 until the one after the factor tiles, 1
    // through the first two node blocks, then 0), so that issue goes to the
    // waves that are behind (tree-64 21.9 -> 21.65 us, its step 33.3 -> 32.55
    // us).  Only on grids of one round: where rounds overlap it held back the
    // blocks the next round waits for.
    // blocks of this kernel resident per CU: what its LDS and its register
    // bound (waves per SIMD) allow
    constexpr int RES = (163840 / (int)L::total) < (4 * L::WPE / NW) ? (163840 / (int)L::total) : (4 * L::WPE / NW);
    const bool lockstep = TM == 64 && STG && !CMT && gridDim.x <= (unsigned)(RES * kCus);
    if (lockstep) __builtin_amdgcn_s_setprio(3);
    float lcarry = 0.f;  // log P at the previous chunk's last node, counted from S0
    const int nchunk = LOOP ? pa.chunks : 1;
    for (int ch = 0; ch < nchunk; ++ch) {
        VerifyArgs p = pa;
        if constexpr (CMT) {
            p.t0 = pa.t0 + TM * ch;
            p.T = min(TM, pa.Ts - p.t0);
            p.S0 = p.t0 == 0 ? pa.S0 : pa.S_next;
            p.S_next = p.t0 + p.T < pa.Ts ? pa.S_next : nullptr;
            if (ch > 0) __syncthreads();  // every read of the previous chunk's LDS is done
        }

        // (looping over chunks, the thread index is made a new value per
        // chunk, so that no lane address derived from it is kept live across
        // chunks: hoisted out of the loop they made the compiler spill)
        int tid_v = threadIdx.x;
        if constexpr (LOOP) asm volatile("" : "+v"(tid_v));
        const int tid = tid_v, lane = tid & 63, wave = tid >> 6;
        const int c = lane & 15, g = lane >> 4;
        const int T = p.T, H = p.H;
        // units of kSpreadHeads heads spread over the XCDs as in commit and the
        // in-block read, so that a head's S0 is in the same L2 for the calls that
        // follow
        const unsigned bid = xcd_spread(blockIdx.x, gridDim.x / (kSpreadHeads * S::NT), kSpreadHeads * S::NT);
        const int tile = (int)(bid % S::NT);
        const int bh = (int)(bid / S::NT);
        const int h = bh % H, b = bh / H;
        const size_t nb0 = (size_t)b * p.Ts + p.t0;  // node 0 of this sequence's (chunk of the) draft
        // 16-node blocks in use.  The launch picks TM as the smallest of 16, 32
        // and 64 that holds T, so at 16 and 32 every node block is in use and at
        // 64 all but possibly the last.  Saying so at compile time keeps those
        // node-block branches out of the kernels (at 64 nodes only where the
        // outputs are staged: it measured 2% slower on the one-round tree grid).
        // Every chunk of a long chain but the last is full; the last one runs
        // all four node blocks too (its nodes past T are zero rows that no
        // store reaches, so they cost only time).
        static_assert(!CMT || (TM == 64 && MBW == 1), "step 6 is written for 64-node chunks");
        const int NB = (TM <= 32 || CMT) ? NBM : (STG ? max(NBM - 1, (T + 15) >> 4) : (T + 15) >> 4);
        const int T16 = NB * 16;
        // first value row (of S0, o, u) of this wave; the wave index is read
        // into a scalar register so that every view base below is scalar
        const int vrow0 = tile * BV + __builtin_amdgcn_readfirstlane(wave) * 16 * MBW;
        constexpr int ES = F32IN ? 4 : 2;  // bytes per q/k/v element
        const uint32_t HD = (uint32_t)H * D;             // elements from one node to the next
        const uint32_t span = (uint32_t)(T - 1) * HD;    // elements from node 0 to node T-1
        const size_t hrow0 = nb0 * H + h;                // (node 0, head h) as a row of the [.., H, D] arrays

        // 1. global loads, through views that end at node T - 1 (rows past T
        // read as zero, see make_buf).  Every small per-node input first, so
        // that, loads completing in issue order, steps 2-3 can run while the S0
        // rows are in flight; the parent row and gates go before q and k (a
        // wait for them, which the compiler also places where their registers
        // are reused, then waits for nothing else).  No load is under a branch:
        // a load under a branch, or a register overwritten while its load is
        // pending, would make the compiler wait for every earlier memory
        // operation.  Lane n of each wave reads node n's parent and gates (a
        // chain has no parent array: its view is empty).
        const buf_t bpar = make_buf(p.parent ? p.parent + (size_t)b * T : nullptr, p.parent ? 4u * T : 0u);
        const uint32_t gbytes = ((uint32_t)(T - 1) * H + 1) * 4;
        const int par_ld = (int)__builtin_amdgcn_raw_buffer_load_b32(bpar, 4u * lane, 0, 0);
        const float ga = buf_ldf(make_buf(p.a + hrow0, gbytes), 4u * lane * H);
        const float gb = buf_ldf(make_buf(p.beta + hrow0, gbytes), 4u * lane * H);
        // log P at the node before a chunk (read from any valid entry otherwise)
        const float* lbp = p.logp_out ? p.logp_out : p.a;
        const float lbase_ld = (CMT && ch > 0) ? lcarry : lbp[((p.t0 > 0 ? nb0 - 1 : nb0)) * H + h];
        u32x4 qreg[QKC], kreg[QKC];
        {
            const uint32_t qkbytes = (span + D) * ES;
            const buf_t bq = make_buf(static_cast<const char*>(p.q) + hrow0 * D * ES, qkbytes);
            const buf_t bk = make_buf(static_cast<const char*>(p.k) + hrow0 * D * ES, qkbytes);
    #pragma unroll
            for (int i = 0; i < QKC; ++i) {
                const int ch = tid + i * NTHR, row = ch / CPR, col = (ch % CPR) * EPC;
                const uint32_t off = ((uint32_t)row * HD + col) * ES;
                qreg[i] = buf_ld128(bq, off);
                kreg[i] = buf_ld128(bk, off);
            }
        }
        // v[n][vrow0 + 16 mi + c] for the nodes n = 16 nb + 4 g + r this lane
        // holds in R (node-major C layout)
        float vf[MBW][NBM][4];
        unsigned short vb[MBW][NBM][4];
        {
            const buf_t bv = make_buf(static_cast<const char*>(p.v) + (hrow0 * D + vrow0) * ES, (span + 16 * MBW) * ES);
            const uint32_t voff = ((uint32_t)(4 * g) * HD + c) * ES;
    #pragma unroll
            for (int mi = 0; mi < MBW; ++mi) {
    #pragma unroll
                for (int nb = 0; nb < NBM; ++nb) {
    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t off = voff + ((uint32_t)(16 * nb + r) * HD + 16 * mi) * ES;
                        if constexpr (F32IN) vf[mi][nb][r] = buf_ldf(bv, off);
                        else vb[mi][nb][r] = buf_ld16(bv, off);
                    }
                }
            }
        }
        // this lane's S0 rows (A operand row c of each of the wave's 16-row
        // blocks, and the B operand column c of K S0^T)
        // (one row block is written without the row-block loop: with it the
        // compiler's allocation of the 64-node kernel spills)
        float4 sreg[MBW][KS][2];
        // 16 and 32 nodes at d = 128: the wave's 16 MBW rows are 8 MBW KiB of
        // consecutive bytes, read with non-temporal loads that each cover 1 KiB
        // (whole lines), and put into the operand layout through LDS before
        // step 4 (verify 36.7 -> 33.6 us on the 27B-hybrid shape); loading the
        // operand layout straight from memory covers 64-byte halves of lines
        // per load
        constexpr bool CS0 = L::cs0 && !CMT;
        constexpr int NS0 = CS0 ? 8 * MBW : 1;
        float4 s0c[NS0];  // float4 lane + 64 i of the wave's rows: row 2 i + lane / 32, columns 4 (lane % 32) ..
        if constexpr (CS0) {
            const float* wsrc = p.S0 + (((size_t)b * H + h) * D + vrow0) * D;
    #pragma unroll
            for (int i = 0; i < NS0; ++i) s0c[i] = ld_nt(wsrc + 4 * (lane + kWave * i));
        } else {
            const buf_t bs = make_buf(p.S0 + (((size_t)b * H + h) * D + vrow0) * D, 16u * MBW * D * 4);
            const uint32_t soff = (uint32_t)(c * D + 4 * g) * 4;
            const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (MBW == 1) {
    #pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const int k0 = 32 * s + 4 * g;
                    sreg[0][s][0] = (k0 < D) ? buf_ldf4(bs, soff + 128u * s) : z4;
                    sreg[0][s][1] = (k0 + 16 < D) ? buf_ldf4(bs, soff + 128u * s + 64u) : z4;
                }
            } else {
    #pragma unroll
                for (int mi = 0; mi < MBW; ++mi) {
    #pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const int k0 = 32 * s + 4 * g;
                        const uint32_t o = soff + 64u * mi * D + 128u * s;
                        sreg[mi][s][0] = (k0 < D) ? buf_ldf4(bs, o) : z4;
                        sreg[mi][s][1] = (k0 + 16 < D) ? buf_ldf4(bs, o + 64u) : z4;
                    }
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
                const u32x4 qv = qreg[i], kv = kreg[i];  // zero past T
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
            const float la = valid ? fmaxf(__builtin_amdgcn_logf(ga), -126.f) : 0.f;  // log2 a
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
                s_P[n] = valid ? __builtin_amdgcn_exp2f(ls) : 0.f;
                s_beta[n] = valid ? gb : 0.f;
            }
            if (lane == 0) {
                s_int[0] = badm != 0ull;
                if (badm != 0ull && p.status && h == 0 && tile == 0) atomicOr(p.status, LDV_STATUS_BAD_PARENT);
            }
            if (badm == 0ull && valid && tile == 0 && p.logp_out)
                p.logp_out[(nb0 + n) * H + h] = ls * kLn2 + (p.t0 > 0 ? lbase_ld : 0.f);
        }
        __syncthreads();
        if (lockstep) __builtin_amdgcn_s_setprio(2);
        if (s_int[0]) return;  // invalid parent row: nothing is written

        // 3a. diagonal blocks: X_ii^T.  K_i K_i^T is symmetric, so one
        //     accumulator gives G_ii and G_ii^T in the C layout (register r of
        //     lane (c, g): rows 16 i + 4 g + r, column 16 i + c), and
        //       X_ii = (I + G_ii)^{-1} = (I - G)(I + G^2)(I + G^4)(I + G^8)
        //     (G_ii is nilpotent: G^L = 0 for L the longest ancestor chain
        //     inside the block, so the product stops at the first power >= L).
        // (the factor work is spread over the waves by the wave index read into a
        // scalar register, so that the item loops and index searches are scalar)
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        for (int i = wv; i < NB; i += NW) {
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
            // rows 16 i + 4 g + r (read as vectors, with no branch: the masks
            // select), column nc; of the two entries at most one is nonzero, so
            // each takes one 2^x
            const int nc = 16 * i + c, n0 = 16 * i + 4 * g;
            const uint64_t anc_c = s_anc[nc];
            const float lpc = s_logp[nc], bec = s_beta[nc];
            const float4 lp4 = *reinterpret_cast<const float4*>(s_logp + n0);
            const float4 be4 = *reinterpret_cast<const float4*>(s_beta + n0);
            const float lpr[4] = {lp4.x, lp4.y, lp4.z, lp4.w}, ber[4] = {be4.x, be4.y, be4.z, be4.w};
            floatx4 G, Gt;  // G[16 i + 4 g + r][nc] and G[nc][16 i + 4 g + r]
    #pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool below = (s_anc[n0 + r] >> nc) & 1ull;  // nc an ancestor of row n0 + r
                const bool above = (anc_c >> (n0 + r)) & 1ull;    // row n0 + r an ancestor of nc
                const float x = __builtin_amdgcn_exp2f(below ? lpr[r] - lpc : lpc - lpr[r]) * acc[r];
                G[r] = below ? ber[r] * x : 0.f;
                Gt[r] = above ? bec * x : 0.f;
            }
            const int L = __builtin_amdgcn_readfirstlane(wave_max_i(__popcll((anc_c >> (16 * i)) & 0xffffull) + 1));
            floatx4 Xt = ident_plus(Gt, -1.f, c, g);  // (I - G)^T
            if (L > 2) {
                const floatx4 z = {0.f, 0.f, 0.f, 0.f};
                floatx4 G2, G2t;
                {
                    const Frag16 fg = frag16(G), fgt = frag16(Gt);
                    G2 = mm16f(z, fgt.pr, fg.dh, fg.dl);
                    G2t = L > 4 ? mm16f(z, fg.pr, fgt.dh, fgt.dl) : z;
                }
                Xt = mm16(ident_plus(G2, 1.f, c, g), Xt);  // ((I - G)(I + G^2))^T
                if (L > 4) {
                    floatx4 G4, G4t;
                    {
                        const Frag16 fg2 = frag16(G2), fg2t = frag16(G2t);
                        G4 = mm16f(z, fg2t.pr, fg2.dh, fg2.dl);
                        G4t = L > 8 ? mm16f(z, fg2.pr, fg2t.dh, fg2t.dl) : z;
                    }
                    Xt = mm16(ident_plus(G4, 1.f, c, g), Xt);
                    if (L > 8) Xt = mm16(ident_plus(mm16(G4t, G4), 1.f, c, g), Xt);
                }
            }
            const Frag16 fx = frag16(Xt);
            slot_store(s_sl, 2 * i, lane, fx.dh);
            slot_store(s_sl, 2 * i + 1, lane, fx.dl);
        }

        // 3b. -G_ik^T (k < i) and C_ji^T (i <= j).  Item it covers the tile of
        //     rows n in node block bn and columns m in block bm: A = k rows of
        //     block bm, B = k or q rows of block bn, so the accumulator holds
        //     k_m . k_n (or k_m . q_n) at register r of lane (c, g) for
        //     m = 16 bm + 4 g + r, n = 16 bn + c.  With more waves than node
        //     blocks, a diagonal block counts as two items: the waves without
        //     one take C consecutive items each, the others share the rest.
        {
            const int nneg = NB * (NB - 1) / 2, nitem = NB * NB;
            int it0 = wv, it1 = nitem, step = NW;
            if (NW > NB) {
                const int C = (2 * NB + nitem + NW - 1) / NW;
                if (wv >= NB) {
                    it0 = (wv - NB) * C;
                    it1 = min(it0 + C, nitem);
                    step = 1;
                } else {
                    it0 = (NW - NB) * C + wv;
                    step = NB;
                }
            }
            for (int it = it0; it < it1; it += step) {
                const bool isc = it >= nneg;
                int bn, bm, t;
                if (!isc) {
                    int i = 1;
                    while (i * (i + 1) / 2 <= it) ++i;
                    bn = i;
                    bm = it - i * (i - 1) / 2;
                    t = S::SG0 + 2 * (i * (i - 1) / 2 + bm);
                } else {
                    const int rr = it - nneg;
                    int j = 0;
                    while ((j + 1) * (j + 2) / 2 <= rr) ++j;
                    bn = j;
                    bm = rr - j * (j + 1) / 2;
                    t = S::SC0 + 2 * (j * (j + 1) / 2 + bm);
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
                const float4 lm4 = *reinterpret_cast<const float4*>(s_logp + 16 * bm + 4 * g);
                const float lm[4] = {lm4.x, lm4.y, lm4.z, lm4.w};
                floatx4 v;
    #pragma unroll
                for (int r = 0; r < 4; ++r) {  // (no branch: the mask selects)
                    const int m = 16 * bm + 4 * g + r;
                    const float x = sc * __builtin_amdgcn_exp2f(lpn - lm[r]) * acc[r];
                    v[r] = ((pathn >> m) & 1ull) ? x : 0.f;
                }
                const Frag16 fv = frag16(v);
                slot_store(s_sl, t, lane, fv.dh);
                slot_store(s_sl, t + 1, lane, fv.dl);
            }
        }

        // 4. S0 Q^T (A = S0 rows, B = q rows: value-major, lane (c, g) holds
        //    value rows 4 g + r of node 16 nb + c) and K S0^T (A = k rows,
        //    B = S0 rows: node-major, nodes 16 nb + 4 g + r of value row c).
        //    Both read only Q, K and registers, so they go before the barrier.
        //    Two passes keep the register peak down: K S0^T and R (the v
        //    registers die), then S0 Q^T and B0^T from the S0 operands kept as
        //    hi / lo terms.  With one row block per wave, all S0 registers are
        //    split first and R is formed node block by node block; with two
        //    (and the registers to spare) each k-step splits its own S0
        //    registers, so the S0 loads are waited for one step at a time.  (The
        //    other orders make the compiler spill.)
        if constexpr (CS0) {
            // lane (c, g) takes row c of each row block, S0C columns per pass:
            // the lanes holding the pass's columns write them, every lane
            // reads its operands back (wave-local: the wave's own rows)
            constexpr int S0C = L::S0C, S0LD = L::S0LD, LPP = S0C / 4;  // lanes (mod 32) per pass
            float* s0t = reinterpret_cast<float*>(smem + L::off_s0) + wave * 16 * MBW * S0LD;
    #pragma unroll
            for (int ps = 0; ps < D / S0C; ++ps) {
                if ((lane & 31) / LPP == ps) {
    #pragma unroll
                    for (int i = 0; i < NS0; ++i)
                        *reinterpret_cast<float4*>(&s0t[(2 * i + (lane >> 5)) * S0LD + 4 * (lane & 31) - S0C * ps]) =
                            s0c[i];
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    #pragma unroll
                for (int s = ps * S0C / 32; s < (ps + 1) * S0C / 32; ++s) {
                    const int k = 32 * s + 4 * g - S0C * ps;
    #pragma unroll
                    for (int mi = 0; mi < MBW; ++mi) {
                        sreg[mi][s][0] = *reinterpret_cast<const float4*>(&s0t[(16 * mi + c) * S0LD + k]);
                        sreg[mi][s][1] = *reinterpret_cast<const float4*>(&s0t[(16 * mi + c) * S0LD + k + 16]);
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
        bf16x8 sh[MBW][KS], sl[MBW][KS];
        floatx4 acck[MBW][NBM];
        if constexpr (MBW > 1) {
    #pragma unroll
            for (int mi = 0; mi < MBW; ++mi) {
    #pragma unroll
                for (int nb = 0; nb < NBM; ++nb) acck[mi][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
    #pragma unroll
            for (int s = 0; s < KS; ++s) {
    #pragma unroll
                for (int mi = 0; mi < MBW; ++mi) split8(sreg[mi][s][0], sreg[mi][s][1], sh[mi][s], sl[mi][s]);
    #pragma unroll
                for (int nb = 0; nb < NBM; ++nb) {
                    if (nb < NB) {
                        const unsigned short* krow = s_k + (nb * 16 + c) * QKLD;
                        const bf16x8 bk = frag_row<D>(krow, s, g);
    #pragma unroll
                        for (int mi = 0; mi < MBW; ++mi) {
                            acck[mi][nb] = mfma16x16x32(bk, sh[mi][s], acck[mi][nb]);
                            acck[mi][nb] = mfma16x16x32(bk, sl[mi][s], acck[mi][nb]);
                        }
                        if constexpr (F32IN) {
                            const bf16x8 bkl = frag_row<D>(krow + LO, s, g);
    #pragma unroll
                            for (int mi = 0; mi < MBW; ++mi) acck[mi][nb] = mfma16x16x32(bkl, sh[mi][s], acck[mi][nb]);
                        }
                    }
                }
            }
        } else {
    #pragma unroll
            for (int s = 0; s < KS; ++s) split8(sreg[0][s][0], sreg[0][s][1], sh[0][s], sl[0][s]);
        }
        // R[n][v] = beta_n (v_n[v] - P_n (S0 k_n)[v]), zero past T (beta = 0)
        floatx4 rn[MBW][NBM];
    #pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
            if (nb < NB) {
                if constexpr (MBW == 1) {
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                    const unsigned short* krow = s_k + (nb * 16 + c) * QKLD;
    #pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const bf16x8 bk = frag_row<D>(krow, s, g);
                        acc = mfma16x16x32(bk, sh[0][s], acc);
                        acc = mfma16x16x32(bk, sl[0][s], acc);
                        if constexpr (F32IN) acc = mfma16x16x32(frag_row<D>(krow + LO, s, g), sh[0][s], acc);
                    }
                    acck[0][nb] = acc;
                }
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
                        rn[mi][nb][r] = Br[r] * (vv - Pr[r] * acck[mi][nb][r]);
                    }
                }
            }
        }
        // B0^T[v][n] = P_n (S0 q_n)[v]; the O^T accumulators start there
        floatx4 acco[MBW][NBM];
    #pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
            if (nb < NB) {
                floatx4 acc[MBW];
    #pragma unroll
                for (int mi = 0; mi < MBW; ++mi) acc[mi] = floatx4{0.f, 0.f, 0.f, 0.f};
                const unsigned short* qrow = s_q + (nb * 16 + c) * QKLD;
    #pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const bf16x8 bq = frag_row<D>(qrow, s, g);
    #pragma unroll
                    for (int mi = 0; mi < MBW; ++mi) {
                        acc[mi] = mfma16x16x32(sh[mi][s], bq, acc[mi]);
                        acc[mi] = mfma16x16x32(sl[mi][s], bq, acc[mi]);
                    }
                    if constexpr (F32IN) {
                        const bf16x8 bql = frag_row<D>(qrow + LO, s, g);
    #pragma unroll
                        for (int mi = 0; mi < MBW; ++mi) acc[mi] = mfma16x16x32(sh[mi][s], bql, acc[mi]);
                    }
                }
                const float Pc = s_P[nb * 16 + c];
    #pragma unroll
                for (int mi = 0; mi < MBW; ++mi) {
    #pragma unroll
                    for (int r = 0; r < 4; ++r) acco[mi][nb][r] = Pc * acc[mi][r];
                }
            }
        }
        __syncthreads();  // every factor tile written
        if (lockstep) __builtin_amdgcn_s_setprio(1);

        // 5. forward substitution over node blocks; O^T block by block.  Output
        //    views: lane (c, g) stores node 16 i + c, values vrow0 + 16 mi + 4 g
        //    .. +3; stores of nodes past T fall outside the views and are
        //    dropped (no per-lane branch around the MFMAs that feed them).
        const uint32_t obytes = (span + 16 * MBW) * 4;
        const buf_t bo = make_buf(p.o + hrow0 * D + vrow0, obytes);
        const buf_t bu = make_buf(p.u_out ? p.u_out + hrow0 * D + vrow0 : nullptr, p.u_out ? obytes : 0u);
        const uint32_t ooff = ((uint32_t)c * HD + 4 * g) * 4;
        bf16x8 upr[MBW][NBM];  // U_i as pairs
        floatx4 ukeep[MBW], okeep[MBW];  // STG: the finished U^T and O^T tiles
        // STG with four node blocks (outside long-chain chunks, whose step 6
        // still reads K): one pass of whole-row stores for all 64 nodes after
        // the substitution instead of one per node block, two workgroup
        // barriers instead of eight.  Node blocks 0 and 1 go into the Q/K rows
        // (dead for every wave after the barrier that ends step 4) as soon as
        // they are done; block 2 waits in registers, and blocks 2 and 3 go over
        // the factor tiles once every wave has read its last one.  With the
        // priorities above: tree-64 verify 22.2 -> 21.85 us, its step 32.0 ->
        // 30.9 us.
        constexpr bool STG4 = STG && NBM == 4 && !CMT;
        constexpr int SLOT = 2 * 16 * L::SLD;  // floats per staged node block: O rows, then U rows
        static_assert(!STG4 || (L::qk >= 2 * SLOT * 4 && (size_t)S::NSLOT * kWave * 16 >= 2 * SLOT * 4),
                      "two staged node blocks fit the Q/K rows and two the factor tiles");
        float* const s_stg_qk = reinterpret_cast<float*>(smem);
        float* const s_stg_t = reinterpret_cast<float*>(smem + L::off_t);
        floatx4 ukeep2[MBW], okeep2[MBW];  // STG4: node block 2's tiles
        auto stage_put = [&](float* s_so, const floatx4 (&ok)[MBW], const floatx4 (&uk)[MBW]) {
    #pragma unroll
            for (int mi = 0; mi < MBW; ++mi) {
                const int v = (wave * MBW + mi) * 16 + 4 * g;
                *reinterpret_cast<float4*>(s_so + c * L::SLD + v) = make_float4(ok[mi][0], ok[mi][1], ok[mi][2], ok[mi][3]);
                *reinterpret_cast<float4*>(s_so + (16 + c) * L::SLD + v) = make_float4(uk[mi][0], uk[mi][1], uk[mi][2], uk[mi][3]);
            }
        };
        // STG: node block i's finished tiles through the staging area, then whole
        // rows of its 16 nodes (BV values each) to o and u, so that each store
        // instruction writes whole rows; nodes past T fall outside the views and
        // are dropped
        auto stage_store = [&](int i) {
            constexpr int SLD = L::SLD;
            float* s_so = reinterpret_cast<float*>(smem + L::off_stg);  // [16][SLD] O rows, then [16][SLD] U rows
            // what the staging area overlays is no longer read: the previous node
            // block's rows (or, with one node block, every factor tile)
            __syncthreads();
    #pragma unroll
            for (int mi = 0; mi < MBW; ++mi) {
                const int v = (wave * MBW + mi) * 16 + 4 * g;
                *reinterpret_cast<float4*>(s_so + c * SLD + v) = make_float4(okeep[mi][0], okeep[mi][1], okeep[mi][2], okeep[mi][3]);
                *reinterpret_cast<float4*>(s_so + (16 + c) * SLD + v) =
                    make_float4(ukeep[mi][0], ukeep[mi][1], ukeep[mi][2], ukeep[mi][3]);
            }
            __syncthreads();
            const uint32_t tbytes = (span + BV) * 4;
            const buf_t to = make_buf(p.o + hrow0 * D + tile * BV, tbytes);
            const buf_t tu = make_buf(p.u_out ? p.u_out + hrow0 * D + tile * BV : nullptr, p.u_out ? tbytes : 0u);
            for (int k = tid; k < 16 * (BV / 4); k += NTHR) {
                const int n = k / (BV / 4), v4 = 4 * (k % (BV / 4));
                const uint32_t off = ((uint32_t)(16 * i + n) * HD + v4) * 4;
                buf_st_stream(to, off, *reinterpret_cast<const float4*>(s_so + n * SLD + v4));
                buf_st_stream(tu, off, *reinterpret_cast<const float4*>(s_so + (16 + n) * SLD + v4));
            }
        };
    #pragma unroll
        for (int i = 0; i < NBM; ++i) {
            if (i < NB) {
                floatx4 y[MBW];
    #pragma unroll
                for (int mi = 0; mi < MBW; ++mi) y[mi] = rn[mi][i];
    #pragma unroll
                for (int k = 0; k < i; ++k) {  // Y -= G_ik U_k
                    const int sg = S::SG0 + 2 * (i * (i - 1) / 2 + k);
                    const bf16x8 gdh = slot_load(s_sl, sg, lane), gdl = slot_load(s_sl, sg + 1, lane);
    #pragma unroll
                    for (int mi = 0; mi < MBW; ++mi) y[mi] = mm16d(y[mi], gdh, gdl, upr[mi][k]);
                }
                const bf16x8 xdh = slot_load(s_sl, 2 * i, lane), xdl = slot_load(s_sl, 2 * i + 1, lane);
                const uint32_t oo = ooff + (uint32_t)(16 * i) * HD * 4;
                const floatx4 z = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                for (int mi = 0; mi < MBW; ++mi) {
                    const bf16x8 ypr = pair16(y[mi]);
                    upr[mi][i] = pair16(mm16d(z, xdh, xdl, ypr));  // U_i = X_ii Y
                    if constexpr (STG) {
                        ukeep[mi] = mm16f(z, ypr, xdh, xdl);  // U_i^T = Y^T X_ii^T
                    } else if (p.u_out) {
                        const floatx4 ut = mm16f(z, ypr, xdh, xdl);  // U_i^T = Y^T X_ii^T
                        buf_st_stream(bu, oo + 64u * mi, make_float4(ut[0], ut[1], ut[2], ut[3]));
                    }
                }
                {  // O_i^T += U_i^T C_ii^T completes block i: store it at once (in
                   // the same basic block as the MFMA that feeds it)
                    const int sc = S::SC0 + 2 * (i * (i + 1) / 2 + i);
                    const bf16x8 cdh = slot_load(s_sl, sc, lane), cdl = slot_load(s_sl, sc + 1, lane);
    #pragma unroll
                    for (int mi = 0; mi < MBW; ++mi) {
                        const floatx4 ov = mm16f(acco[mi][i], upr[mi][i], cdh, cdl);
                        if constexpr (STG) okeep[mi] = ov;
                        else buf_st_stream(bo, oo + 64u * mi, make_float4(ov[0], ov[1], ov[2], ov[3]));
                    }
                }
    #pragma unroll
                for (int j = i + 1; j < NBM; ++j) {  // O_j^T += U_i^T C_ji^T
                    if (j < NB) {
                        const int sc = S::SC0 + 2 * (j * (j + 1) / 2 + i);
                        const bf16x8 cdh = slot_load(s_sl, sc, lane), cdl = slot_load(s_sl, sc + 1, lane);
    #pragma unroll
                        for (int mi = 0; mi < MBW; ++mi) acco[mi][j] = mm16f(acco[mi][j], upr[mi][i], cdh, cdl);
                    }
                }
                if constexpr (STG4) {
                    if (i < 2) {
                        stage_put(s_stg_qk + i * SLOT, okeep, ukeep);
                    } else if (i == 2) {
                        if (lockstep) __builtin_amdgcn_s_setprio(0);
    #pragma unroll
                        for (int mi = 0; mi < MBW; ++mi) {
                            okeep2[mi] = okeep[mi];
                            ukeep2[mi] = ukeep[mi];
                        }
                    }
                } else if constexpr (STG) {
                    stage_store(i);
                }
            }
        }
        if constexpr (STG4) {
            __syncthreads();  // every factor tile has been read
            stage_put(s_stg_t, okeep2, ukeep2);
            stage_put(s_stg_t + SLOT, okeep, ukeep);  // node block 3 (block 2 again when NB = 3: past T, dropped)
            __syncthreads();
            const uint32_t tbytes = (span + BV) * 4;
            const buf_t to = make_buf(p.o + hrow0 * D + tile * BV, tbytes);
            const buf_t tu = make_buf(p.u_out ? p.u_out + hrow0 * D + tile * BV : nullptr, p.u_out ? tbytes : 0u);
            for (int k = tid; k < NB * 16 * (BV / 4); k += NTHR) {
                const int i = k / (16 * (BV / 4)), n = (k / (BV / 4)) % 16, v4 = 4 * (k % (BV / 4));
                const float* s_so = (i < 2 ? s_stg_qk : s_stg_t - 2 * SLOT) + i * SLOT;
                const uint32_t off = ((uint32_t)(16 * i + n) * HD + v4) * 4;
                buf_st_stream(to, off, *reinterpret_cast<const float4*>(s_so + n * L::SLD + v4));
                buf_st_stream(tu, off, *reinterpret_cast<const float4*>(s_so + (16 + n) * L::SLD + v4));
            }
        }

        // 6. the state at node T - 1 into S_next.  Per key tile kt the wave forms
        //    M = (K^T)_kt U_w for its 16 value rows: A = the k column 16 kt + c at
        //    four nodes, doubled like a factor tile (the nodes of U's k-slots), B
        //    = U_i weighted by w_m = P / P_m as a pair; M[key 16 kt + 4 g + r]
        //    [value c] is then S - P S0 at four consecutive keys of one value row.
        if constexpr (CMT) {
            if (p.S_next) {
                constexpr int KTLD = TM + 8;        // bf16 row stride of K^T (rows are keys)
                constexpr int NPK = F32IN ? 2 : 1;  // K planes (hi, lo)
                static_assert((size_t)NPK * D * KTLD * 2 <= (size_t)S::NSLOT * kWave * 16, "K^T fits the factor tiles' area");
                unsigned short* s_kt = reinterpret_cast<unsigned short*>(smem + L::off_t);
                __syncthreads();  // every factor tile has been read
                for (int e = tid; e < NPK * D * (TM / 4); e += NTHR) {
                    const int pl = e / (D * (TM / 4)), r = e % (D * (TM / 4));
                    const int x = r % D, n4 = 4 * (r / D);
                    const unsigned short* kr = s_k + pl * LO + n4 * QKLD + x;
                    const u16x4 w4 = {kr[0], kr[QKLD], kr[2 * QKLD], kr[3 * QKLD]};
                    *reinterpret_cast<u16x4*>(s_kt + (pl * D + x) * KTLD + n4) = w4;
                }
                __syncthreads();
                const int last = T - 1;
                const uint64_t path = s_anc[last] | (1ull << last);
                const float lpl = s_logp[last], Pl = s_P[last];
                bf16x8 uw[NBM];
    #pragma unroll
                for (int i = 0; i < NBM; ++i) {
                    const u16x8 ub = __builtin_bit_cast(u16x8, upr[0][i]);  // [hi | lo] of nodes 16 i + 4 g + r
                    float x[4];
    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = 16 * i + 4 * g + r;
                        const float w = ((path >> m) & 1ull) ? __builtin_amdgcn_exp2f(lpl - s_logp[m]) : 0.f;
                        x[r] = w * (bf16_val(ub[r]) + bf16_val(ub[4 + r]));
                    }
                    uw[i] = pair16(floatx4{x[0], x[1], x[2], x[3]});
                }
                const size_t srow = (((size_t)b * H + h) * D + vrow0 + c) * D + 4 * g;
    #pragma unroll
                for (int kt = 0; kt < D / 16; ++kt) {
                    const float4 s4 = ld_stream(p.S0 + srow + 16 * kt);
                    floatx4 acc = {Pl * s4.x, Pl * s4.y, Pl * s4.z, Pl * s4.w};
    #pragma unroll
                    for (int i = 0; i < NBM; ++i) {
                        const u16x4 k4 = load_u16x4(s_kt + (16 * kt + c) * KTLD + 16 * i + 4 * g);
                        acc = mfma16x16x32(join(k4, k4), uw[i], acc);
                        if constexpr (F32IN) {
                            const u16x4 kl4 = load_u16x4(s_kt + (D + 16 * kt + c) * KTLD + 16 * i + 4 * g);
                            acc = mfma16x16x32(join(kl4, kl4), uw[i], acc);
                        }
                    }
                    // (looping: the same block reads the state back in its next
                    // chunk, so it is stored through the caches: GDN-1.3B
                    // 1024-node chain 259.2 -> 257.3 us)
                    if constexpr (LOOP)
                        *reinterpret_cast<float4*>(p.S_next + srow + 16 * kt) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                    else
                        st_stream(p.S_next + srow + 16 * kt, make_float4(acc[0], acc[1], acc[2], acc[3]));
                }
            }
        }
        if constexpr (LOOP)  // (the same in every lane: kept in a scalar register)
            lcarry = __int_as_float(__builtin_amdgcn_readfirstlane(
                __float_as_int(s_logp[p.T - 1] * kLn2 + (p.t0 > 0 ? lbase_ld : 0.f))));
    }
}

// Grids of at least this many blocks stage their outputs in LDS and store
// whole rows.  Measured: 27B-hybrid 38.3 -> 36.5 us (2048 blocks), tree-64
// 23.5 -> 21.3 us (512), batch-256 191 -> 175 us (8192); the GDN-1.3B grid
// (256 blocks) is the same either way and stores straight from the
// accumulators.
constexpr long long kVerifyStageBlocks = 512;

template <int D, int TM, bool F32IN, bool STG, bool CMT = false, bool LOOP = false>
static hipError_t launch_t(const VerifyArgs& a, hipStream_t st) {
    using S = VShape<D, TM>;
    const long long nblk = (long long)a.B * a.H * S::NT;
    if (nblk <= 0) return hipSuccess;
    hipLaunchKernelGGL((verify_kernel<D, TM, F32IN, STG, CMT, LOOP>), dim3((unsigned)nblk), dim3(S::NW * kWave), 0,
                       st, a);
    return hipGetLastError();
}

template <int D, bool F32IN>
static hipError_t launch_d(const VerifyArgs& a, hipStream_t st) {
    if (a.S_next) {  // chunks of a chain longer than 64 nodes, in one launch
        if (a.Ts <= 64 || a.chunks < 1 || a.t0 % 64 || a.t0 + 64LL * (a.chunks - 1) >= a.Ts)
            return hipErrorInvalidValue;
        // several chunks per launch: grids of at most one block per CU, which
        // never stage their outputs (the looping kernel holds a few more
        // registers and measured slower per chunk on larger grids)
        if (a.chunks > 1) return launch_t<D, 64, F32IN, false, true, true>(a, st);
        if constexpr (D == 128) {
            if ((long long)a.B * a.H * VShape<D, 64>::NT >= kVerifyStageBlocks)
                return launch_t<D, 64, F32IN, true, true>(a, st);
        }
        return launch_t<D, 64, F32IN, false, true>(a, st);
    }
    if (a.T <= 16) {
        if ((long long)a.B * a.H * VShape<D, 16>::NT >= kVerifyStageBlocks) return launch_t<D, 16, F32IN, true>(a, st);
        return launch_t<D, 16, F32IN, false>(a, st);
    }
    if (a.T <= 32) {
        if ((long long)a.B * a.H * VShape<D, 32>::NT >= kVerifyStageBlocks) return launch_t<D, 32, F32IN, true>(a, st);
        return launch_t<D, 32, F32IN, false>(a, st);
    }
    // 64-node staging at d = 128 only: at d = 64 the compiler's code for it
    // leaves an MFMA result one wait state short of the others before its
    // LDS write on one path, so that shape keeps the direct stores
    if constexpr (D == 128) {
        if ((long long)a.B * a.H * VShape<D, 64>::NT >= kVerifyStageBlocks) return launch_t<D, 64, F32IN, true>(a, st);
    }
    return launch_t<D, 64, F32IN, false>(a, st);
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
