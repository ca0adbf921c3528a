// State commit: form only the accepted node's state from the committed state
// and the node factors (gfx950).
//
// Bole page (arXiv 2608.01651): its summary has only the state of the node
// kept after sampling built; section IV, Eq. (9) and its "Lemma 1"
// keep the node factors P, K, U next to the single committed state.  Unrolling
// the recurrence S_n = a_n S_p + u_n k_n^T gives, for the accepted node n,
//   S_n = P_n S0 + sum_{m on root-to-n path} (P_n / P_m) u_m k_m^T,
// a rank-L update of S0 with L the path length (at most 8 for the draft
// trees, T for a chain).
//
// A chain (no parent array) may be longer than 64 nodes: its path is
// n, n-1, ..., 0 and is generated instead of walked.  (The state at the end
// of each 64-node chunk of a long chain is formed by the verify kernel of
// that chunk, from the factors it already holds.)
//
// The work is a streaming read of S0 and write of S_out (64 KiB each per head
// at d = 128), so it is bound by HBM.  One block of 256 threads per
// (sequence, head, row block of 8 KiB, or 16 KiB where that alone makes the
// grid one round of resident blocks; see launch_t); each thread owns
// float4 chunks of consecutive columns so that every wave reads and writes
// contiguous 1 KiB runs, so the state is read with non-temporal loads
// (whole lines, used once).  The block loads the parent row, then its S0 rows; walks the parent
// row in LDS from the accepted node to the root while the state is in
// flight; issues the loads of u, k and log P on the path; stages w_m u_m (its
// rows) and k_m (all columns) for up to 16 path nodes at a time in LDS; and
// applies the update.
#include "ldv_device.hpp"
#include "ldv_kernels.hpp"

#include "../../include/ldv.h"

namespace ldv {

// EMAX: float4 per block at most (512: 8 KiB row blocks, 1024: 16 KiB)
template <int D, int EMAX>
struct CShape {
    static constexpr int NTHR = 256;
    static constexpr int C4 = D / 4;                                  // float4 per state row (divides NTHR)
    static constexpr int E4 = (D * D / 4 < EMAX) ? D * D / 4 : EMAX;  // float4 per block
    static constexpr int RB = E4 / C4;                                // rows per block
    static constexpr int NRB = D / RB;                                // row blocks per head
    static constexpr int F4 = (E4 + NTHR - 1) / NTHR;                 // float4 per thread
    static constexpr int PCH = 16;                                    // path nodes staged per pass
};

template <int D, bool F32K, int EMAX>
__global__ __launch_bounds__(256) void commit_kernel(const CommitArgs p) {
    using S = CShape<D, EMAX>;
    constexpr int C4 = S::C4, E4 = S::E4, RB = S::RB, F4 = S::F4, NTHR = S::NTHR, PCH = S::PCH;
    constexpr int KI = (PCH * C4 + NTHR - 1) / NTHR;  // k chunks staged per thread and pass
    constexpr int UI = (PCH * RB + NTHR - 1) / NTHR;  // u values staged per thread and pass
    __shared__ float4 s_k[PCH * C4];  // k rows of up to PCH path nodes (fp32)
    __shared__ float s_uw[PCH * RB];  // (P_n / P_m) u_m over this block's rows
    __shared__ int s_par[LDV_MAX_T];
    __shared__ int s_path[LDV_MAX_T];
    __shared__ int s_len, s_bad;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = p.T, H = p.H;
    // units of kSpreadHeads heads spread over the XCDs (a unit's row blocks
    // stay together): the heads that commit nothing cost nothing, so whole
    // sequences per XCD would leave some XCDs with far more work than others
    const unsigned bid = xcd_spread(blockIdx.x, gridDim.x / (kSpreadHeads * S::NRB), kSpreadHeads * S::NRB);
    const int rb = (int)(bid % S::NRB);
    const int bh = (int)(bid / S::NRB);
    const int h = bh % H, b = bh / H;
    const size_t nb0 = (size_t)b * p.Ts + p.t0;  // node 0 of this sequence's (chunk of the) draft
    const bool chain = p.parent == nullptr;

    const int nacc = p.acc_const >= -1 ? p.acc_const : p.accepted[b];
    if (nacc < -1 || nacc >= T) {
        if (tid == 0 && p.status && h == 0 && rb == 0) atomicOr(p.status, LDV_STATUS_BAD_ACCEPTED);
        return;
    }
    if (nacc < 0 && p.S_out == p.S0) return;  // in place, nothing accepted: no traffic

    // Loads: the parent row, then this block's S0 rows; nothing waits for the
    // parent row before the S0 loads are issued (branch-free, clamped index;
    // a chain reads its log P array instead and discards the value).
    const global_ptr<const int32_t> parp =
        (global_ptr<const int32_t>)(p.parent ? p.parent : reinterpret_cast<const int32_t*>(p.logp));
    const int par_ld = (T > 0) ? parp[(size_t)b * T + min(lane, T - 1)] : -1;
    const size_t base = ((size_t)b * H + h) * D * D + (size_t)rb * RB * D;
    const float* src = p.S0 + base;
    float* dst = p.S_out + base;
    float4 sv[F4];
#pragma unroll
    for (int i = 0; i < F4; ++i) {
        const int f = tid + NTHR * i;
        if (F4 * NTHR == E4 || f < E4) sv[i] = ld_nt(src + 4 * f);
    }
    asm volatile("" ::: "memory");  // keep the loads above ahead of any use of them
    if (nacc < 0) {  // nothing accepted, out of place: copy the committed state
#pragma unroll
        for (int i = 0; i < F4; ++i) {
            const int f = tid + NTHR * i;
            if (F4 * NTHR == E4 || f < E4) st_stream(dst + 4 * f, sv[i]);
        }
        return;
    }

    // log P at the node before a chunk (0: the path starts at the committed state)
    const float lbase = p.t0 > 0 ? p.logp[(nb0 - 1) * H + h] : 0.f;
    // validate the parent row (as verify does) and walk from the accepted node
    if (wave == 0 && !chain) {
        const int par = p.parent ? par_ld : lane - 1;
        const bool bad = lane < T && (par < -1 || par >= lane);
        const uint64_t badm = __ballot(bad);
        if (lane < T) s_par[lane] = par;
        if (lane == 0) {
            s_bad = badm != 0ull;
            if (badm != 0ull && p.status && h == 0 && rb == 0) atomicOr(p.status, LDV_STATUS_BAD_PARENT);
        }
    }
    if (chain && tid == 0) s_bad = 0;
    __syncthreads();
    if (s_bad) return;
    if (!chain && tid == 0) {  // parents strictly decrease, so the walk ends within T steps
        int len = 0;
        for (int m = nacc; m >= 0; m = s_par[m]) s_path[len++] = m;
        s_len = len;
    }
    __syncthreads();
    const int len = chain ? nacc + 1 : s_len;
    // i-th node of the path from the accepted node towards the root
    auto path_node = [&](int i) { return chain ? nacc - i : s_path[i]; };
    const int col4 = tid % C4;  // this thread's chunks share one column group (C4 divides NTHR)

    for (int c0 = 0; c0 < len; c0 += PCH) {
        const int cl = min(PCH, len - c0);
        // issue every load of this pass before using any of them
        const float lp_n = p.logp[(nb0 + nacc) * H + h];
        float4 kf[KI];
        u16x4 kb[KI];
        float uval[UI], lval[UI];
#pragma unroll
        for (int j = 0; j < KI; ++j) {
            const int idx = tid + NTHR * j, i = min(idx / C4, cl - 1), c4 = idx % C4;
            const size_t krow = ((nb0 + path_node(c0 + i)) * H + h) * D;
            if constexpr (F32K) kf[j] = *reinterpret_cast<const float4*>(static_cast<const float*>(p.k) + krow + 4 * c4);
            else kb[j] = load_u16x4(static_cast<const unsigned short*>(p.k) + krow + 4 * c4);
        }
#pragma unroll
        for (int j = 0; j < UI; ++j) {
            const int idx = tid + NTHR * j, i = min(idx / RB, cl - 1), r = idx % RB;
            const size_t node = (nb0 + path_node(c0 + i)) * H + h;
            uval[j] = p.u[node * D + (size_t)rb * RB + r];
            lval[j] = p.logp[node];
        }
#pragma unroll
        for (int j = 0; j < KI; ++j) {
            const int idx = tid + NTHR * j;
            if (idx < cl * C4) {
                if constexpr (F32K) s_k[idx] = kf[j];
                else s_k[idx] = make_float4(bf16_val(kb[j][0]), bf16_val(kb[j][1]), bf16_val(kb[j][2]), bf16_val(kb[j][3]));
            }
        }
#pragma unroll
        for (int j = 0; j < UI; ++j) {
            const int idx = tid + NTHR * j;
            if (idx < cl * RB) s_uw[idx] = expf(lp_n - lval[j]) * uval[j];
        }
        if (c0 == 0) {
            const float Pn = expf(lp_n - lbase);
#pragma unroll
            for (int i = 0; i < F4; ++i) sv[i] = make_float4(Pn * sv[i].x, Pn * sv[i].y, Pn * sv[i].z, Pn * sv[i].w);
        }
        __syncthreads();
        for (int m = 0; m < cl; ++m) {
            const float4 kk = s_k[m * C4 + col4];
#pragma unroll
            for (int i = 0; i < F4; ++i) {
                const int f = tid + NTHR * i;
                if (F4 * NTHR == E4 || f < E4) {
                    const float w = s_uw[m * RB + f / C4];
                    sv[i].x += w * kk.x;
                    sv[i].y += w * kk.y;
                    sv[i].z += w * kk.z;
                    sv[i].w += w * kk.w;
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < F4; ++i) {
        const int f = tid + NTHR * i;
        if (F4 * NTHR == E4 || f < E4) st_stream(dst + 4 * f, sv[i]);
    }
}

// Resident 256-thread commit blocks per CU (8 waves per SIMD).
constexpr long long kCommitBlocksPerCu = 8;

template <int D, bool F32K, int EMAX>
static hipError_t launch_e(const CommitArgs& a, hipStream_t st) {
    const long long nblk = (long long)a.B * a.H * CShape<D, EMAX>::NRB;
    if (nblk <= 0) return hipSuccess;
    hipLaunchKernelGGL((commit_kernel<D, F32K, EMAX>), dim3((unsigned)nblk), dim3(CShape<D, EMAX>::NTHR), 0, st, a);
    return hipGetLastError();
}

// 8 KiB row blocks keep more loads in flight per CU than 16 KiB ones and
// measured faster (27B-hybrid 33.6 -> 30.9 us, batch-256 175.3 -> 163.7 us,
// GDN-1.3B 5.8 -> 5.3 us), except where the 16 KiB grid is one round of
// resident blocks and the 8 KiB grid would need two (tree-64: 8.1 vs 9.5 us).
template <int D, bool F32K>
static hipError_t launch_t(const CommitArgs& a, hipStream_t st) {
    const long long heads = (long long)a.B * a.H, round = kCommitBlocksPerCu * kCus;
    if (heads * CShape<D, 512>::NRB > round && heads * CShape<D, 1024>::NRB <= round)
        return launch_e<D, F32K, 1024>(a, st);
    return launch_e<D, F32K, 512>(a, st);
}

template <bool F32K>
static hipError_t launch_f(const CommitArgs& a, hipStream_t st) {
    switch (a.D) {
        case 16: return launch_t<16, F32K>(a, st);
        case 32: return launch_t<32, F32K>(a, st);
        case 64: return launch_t<64, F32K>(a, st);
        case 128: return launch_t<128, F32K>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_commit(const CommitArgs& a, bool f32_k, hipStream_t stream) {
    return f32_k ? launch_f<true>(a, stream) : launch_f<false>(a, stream);
}

}  // namespace ldv
