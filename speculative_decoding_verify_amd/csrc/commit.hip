// State commit: form only the accepted node's state from the committed state
// and the node factors (gfx950).
//
// Bole page (arXiv 2608.01651): the summary says only the post-sampling
// selected state is materialised; section IV, Eq. (9) and its "Lemma 1"
// keep the node factors P, K, U next to the single committed state.  Unrolling
// the recurrence S_n = a_n S_p + u_n k_n^T gives, for the accepted node n,
//   S_n = P_n S0 + sum_{m on root-to-n path} (P_n / P_m) u_m k_m^T,
// a rank-L update of S0 with L the path length (at most 8 for the draft
// trees, T for a chain).
//
// The work is a streaming read of S0 and write of S_out (64 KiB each per head
// at d = 128), so it is bound by HBM.  One block of 256 threads per
// (sequence, head, row block of RB rows); each thread owns float4 chunks of
// consecutive columns so that every wave reads and writes contiguous 1 KiB
// runs.  The block first issues its S0 loads, then walks the parent row in
// LDS from the accepted node to the root, stages w_m u_m (its RB rows) and
// k_m (all columns) for the path in LDS, and applies the update.
#include "ldv_device.hpp"
#include "ldv_kernels.hpp"

#include "../../include/ldv.h"

namespace ldv {

template <int D>
struct CShape {
    static constexpr int E = D * D < 4096 ? D * D : 4096;  // floats per block
    static constexpr int RB = E / D;                       // rows per block
    static constexpr int NRB = D / RB;                     // row blocks per head
    static constexpr int NTHR = 256;
    static constexpr int F4 = (E / 4 + NTHR - 1) / NTHR;   // float4 chunks per thread
};

template <int D, bool F32K>
__global__ __launch_bounds__(256) void commit_kernel(const CommitArgs p) {
    using S = CShape<D>;
    constexpr int E = S::E, RB = S::RB, F4 = S::F4, NTHR = S::NTHR;
    __shared__ __align__(16) float s_k[LDV_MAX_T * D];
    __shared__ float s_uw[LDV_MAX_T * RB];
    __shared__ int s_par[LDV_MAX_T];
    __shared__ int s_path[LDV_MAX_T];
    __shared__ int s_len, s_bad;

    const int tid = threadIdx.x;
    const int T = p.T, H = p.H;
    const unsigned bid = xcd_remap(blockIdx.x, gridDim.x);
    const int rb = (int)(bid % S::NRB);
    const int bh = (int)(bid / S::NRB);
    const int h = bh % H, b = bh / H;

    const int nacc = p.accepted[b];
    if (nacc < -1 || nacc >= T) {
        if (tid == 0 && p.status && h == 0 && rb == 0) atomicOr(p.status, LDV_STATUS_BAD_ACCEPTED);
        return;
    }
    if (nacc < 0 && p.S_out == p.S0) return;  // in place, nothing accepted: no traffic
    const size_t base = ((size_t)b * H + h) * D * D + (size_t)rb * E;
    const float4* src = reinterpret_cast<const float4*>(p.S0 + base);
    float4* dst = reinterpret_cast<float4*>(p.S_out + base);

    float4 sv[F4];
#pragma unroll
    for (int i = 0; i < F4; ++i) {
        const int f = tid + NTHR * i;
        if (f < E / 4) sv[i] = src[f];
    }
    if (nacc < 0) {  // nothing accepted, out of place: copy the committed state
#pragma unroll
        for (int i = 0; i < F4; ++i) {
            const int f = tid + NTHR * i;
            if (f < E / 4) dst[f] = sv[i];
        }
        return;
    }

    // parent row: validate (as verify does) and keep it in LDS
    if (tid < kWave) {
        const int n = tid;
        const bool valid = n < T;
        int par = -1;
        if (valid) par = p.parent ? p.parent[(size_t)b * T + n] : n - 1;
        const bool bad = valid && (par < -1 || par >= n);
        const uint64_t badm = __ballot(bad);
        if (valid) s_par[n] = par;
        if (tid == 0) {
            s_bad = badm != 0ull;
            if (badm != 0ull && p.status && h == 0 && rb == 0) atomicOr(p.status, LDV_STATUS_BAD_PARENT);
        }
    }
    __syncthreads();
    if (s_bad) return;
    if (tid == 0) {  // parents strictly decrease, so the walk ends within T steps
        int len = 0;
        for (int m = nacc; m >= 0; m = s_par[m]) s_path[len++] = m;
        s_len = len;
    }
    __syncthreads();
    const int len = s_len;
    const float lp_n = p.logp[((size_t)b * T + nacc) * H + h];
    const float Pn = expf(lp_n);

    if constexpr (F32K) {
        const float* kg = static_cast<const float*>(p.k);
        for (int idx = tid; idx < len * (D / 4); idx += NTHR) {
            const int i = idx / (D / 4), col = (idx % (D / 4)) * 4;
            const int m = s_path[i];
            *reinterpret_cast<float4*>(s_k + i * D + col) =
                *reinterpret_cast<const float4*>(kg + (((size_t)b * T + m) * H + h) * D + col);
        }
    } else {
        const unsigned short* kg = static_cast<const unsigned short*>(p.k);
        for (int idx = tid; idx < len * (D / 4); idx += NTHR) {
            const int i = idx / (D / 4), col = (idx % (D / 4)) * 4;
            const int m = s_path[i];
            const u16x4 kv = load_u16x4(kg + (((size_t)b * T + m) * H + h) * D + col);
            *reinterpret_cast<float4*>(s_k + i * D + col) =
                make_float4(bf16_val(kv[0]), bf16_val(kv[1]), bf16_val(kv[2]), bf16_val(kv[3]));
        }
    }
    for (int idx = tid; idx < len * RB; idx += NTHR) {
        const int i = idx / RB, r = idx % RB;
        const int m = s_path[i];
        const size_t node = ((size_t)b * T + m) * H + h;
        const float w = expf(lp_n - p.logp[node]);
        s_uw[i * RB + r] = w * p.u[node * D + (size_t)rb * RB + r];
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < F4; ++i) {
        const int f = tid + NTHR * i;
        if (f < E / 4) {
            const int row = f / (D / 4), col = (f % (D / 4)) * 4;
            float4 acc = make_float4(Pn * sv[i].x, Pn * sv[i].y, Pn * sv[i].z, Pn * sv[i].w);
            for (int m = 0; m < len; ++m) {
                const float w = s_uw[m * RB + row];
                const float4 kk = *reinterpret_cast<const float4*>(s_k + m * D + col);
                acc.x += w * kk.x;
                acc.y += w * kk.y;
                acc.z += w * kk.z;
                acc.w += w * kk.w;
            }
            dst[f] = acc;
        }
    }
}

template <int D, bool F32K>
static hipError_t launch_t(const CommitArgs& a, hipStream_t st) {
    const long long nblk = (long long)a.B * a.H * CShape<D>::NRB;
    if (nblk <= 0) return hipSuccess;
    hipLaunchKernelGGL((commit_kernel<D, F32K>), dim3((unsigned)nblk), dim3(CShape<D>::NTHR), 0, st, a);
    return hipGetLastError();
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
