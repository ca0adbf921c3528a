// Greedy accepted-node selection on the device (gfx950).
//
// Verification fixes the accepted prefix (ReaDy page, arXiv 2610.20503,
// Fig. 2a) and only the state of the node selected after sampling is kept
// (Bole page, arXiv 2608.01651, summary and section IV).  Under greedy
// decoding that node is found by walking down from the committed state: at
// each step the target's most likely next token (the argmax of its logits at
// the current position) is compared with the draft tokens of the current
// node's children, and the walk moves to the lowest-index child that
// matches.  The result feeds ldv_commit_state with no host round trip.
//
// Two launches on the caller's stream:
//   1. argmax_kernel: one workgroup per logits row (B x (T+1) rows of V
//      values; 256 threads, or 512 when there are few rows), 16-byte
//      non-temporal loads (each wave load covers 1 KiB of the row; measured
//      10-12% faster than ordinary loads) with eight in flight per thread; or, when the caller gives a
//      workspace and the rows are few, np workgroups per row, each over one
//      part of it (whole 16-byte chunks), writing its part's (maximum,
//      index) to the workspace.  The rule,
//      identical everywhere: the larger value wins, equal values go to the
//      lower index, NaN never wins (+0 == -0), an all-NaN row gives 0.
//      Each thread visits its 16-byte chunks in increasing index order and
//      keeps the chunk with the strictly largest maximum (so the earliest
//      of equal maxima), with one max per element (fmaxf, which never
//      returns NaN over a number) and one compare per chunk; it keeps that
//      chunk's 16 bytes in registers and at the end finds in them the first
//      element equal to the maximum.  Elements outside whole chunks, the wave and workgroup
//      reductions, and rows whose largest value is -inf (where no chunk
//      maximum beats the starting value) use the full rule.  The
//      comparisons are exact in fp32 (bf16 widens exactly), so the argmax
//      does not depend on the order of the reduction.  HBM-bound: the
//      logits are read once.
//   2. walk_kernel: one wave per sequence; lane n holds node n's parent and
//      token and lane r the target of row r, so each step of the walk is a
//      shuffle and a ballot (at most T steps).  With split rows, lane r first
//      combines row r's parts under the same rule and writes target.
#include <limits.h>

#include <mutex>

#include "ldv_device.hpp"
#include "ldv_kernels.hpp"

#include "../../include/ldv.h"

namespace ldv {

// Threads per logits row: 256 when there are enough rows to fill the GPU
// (kArgFillRows or more), else 512 so that a few rows still keep more loads
// in flight (1024 measured slower: fewer chunks per thread, a longer
// reduction).
constexpr int kArgThreadsWide = 512;
constexpr int kArgThreadsNarrow = 256;
constexpr int kArgFillRows = 1024;
constexpr int kArgUnroll = 8;  // 16-byte loads in flight per thread

// With one workgroup per row, a grid that is not a large multiple of the CU
// count leaves CUs idle at its end (measured, rows of 151936 bf16 values:
// 1024 rows 57.9 us, 1088 rows 66.1 us, 544 rows 37.4 us).  Given a
// workspace, fewer rows than kArgSplitRows are split so that the grid holds
// about kArgSplitBlocks workgroups, each part at least kArgMinPart values
// (1088 rows: 61.9 us in four parts each; 544 rows: 34.9 us).  Shorter parts
// measured slower: 144 rows of 32000 values take 6.5 us whole, 7.2 us in
// three parts and 11.2 us in fifteen.
constexpr long long kArgSplitRows = 2048;
constexpr long long kArgSplitBlocks = 4096;
constexpr int kArgMinPart = 32768;

int select_parts(long long rows, int V) {
    if (rows <= 0 || rows >= kArgSplitRows) return 1;
    long long np = (kArgSplitBlocks + rows - 1) / rows;
    if (np > V / kArgMinPart) np = V / kArgMinPart;
    return np < 1 ? 1 : (int)np;
}

// The split-row partial results of ldv_select_accepted_noalloc, for callers
// that cannot allocate: a fixed array of the library, one copy per GPU, held
// until the process ends.  Rows are split only when there are fewer than
// kArgSplitRows of them, into at most ceil(kArgSplitBlocks / rows) parts, so
// a call never needs more than kSelectScratchParts entries (48 KiB).  Every
// call on a GPU uses that GPU's array: calls that overlap on one GPU (on
// different streams) race.  No entry needs to start at any value (each part
// writes its entry before the walk kernel reads it), so nothing is cleared.
static_assert(kSelectScratchParts >= kArgSplitBlocks + kArgSplitRows - 1, "scratch smaller than a split");
static __device__ __align__(256) ArgPart scratch[kSelectScratchParts];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
ArgPart* g_scratch_ptr[kMaxDevices];  // the array's device address on each GPU (null: not resolved yet)
}  // namespace

// In host code `scratch` names a host-side handle, not device memory: its
// device address is resolved once per device, with that device current, and
// only that address is handed to kernels.  The device is the one the
// kernels will run on: the stream's (the current device for the null
// stream); a stream of another device makes that device current for the
// lookup, and the caller's device is restored.
hipError_t select_scratch(hipStream_t stream, ArgPart** out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(stream, &sd);
        if (e != hipSuccess) return e;
        dev = sd;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur) {
            e = hipSetDevice(dev);
            if (e != hipSuccess) return e;
        }
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<ArgPart*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// (v, i) replaces (bv, bi) when v is larger, or equal with a lower index;
// NaN compares false both ways and never replaces.
__device__ __forceinline__ void take_max(float v, int i, float& bv, int& bi) {
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

template <bool F32>
__device__ __forceinline__ float elem(const unsigned char* row, int i) {
    if constexpr (F32) return reinterpret_cast<const float*>(row)[i];
    else return bf16_val(reinterpret_cast<const unsigned short*>(row)[i]);
}

// Value k of a 16-byte chunk.
template <bool F32>
__device__ __forceinline__ float chunk_elem(const u32x4 r, int k) {
    if constexpr (F32) return __uint_as_float(r[k]);
    else return __uint_as_float((k & 1) ? (r[k >> 1] & 0xffff0000u) : (r[k >> 1] << 16));
}

// Largest value of a chunk; NaN never wins (fmaxf returns the number), a
// chunk of NaN gives NaN.
template <bool F32>
__device__ __forceinline__ float chunk_max(const u32x4 r) {
    constexpr int EPC = F32 ? 4 : 8;
    float m = chunk_elem<F32>(r, 0);
#pragma unroll
    for (int k = 1; k < EPC; ++k) m = fmaxf(m, chunk_elem<F32>(r, k));
    return m;
}

// Position of the first element of a chunk equal to v.
template <bool F32>
__device__ __forceinline__ int chunk_find(const u32x4 r, float v) {
    constexpr int EPC = F32 ? 4 : 8;
    int e = EPC - 1;
#pragma unroll
    for (int k = EPC - 2; k >= 0; --k) e = chunk_elem<F32>(r, k) == v ? k : e;
    return e;
}

// Workgroup-wide argmax of (bv, bi) under the full rule; every thread gets
// the result.
template <int NTHR>
__device__ __forceinline__ void block_take_max(float& bv, int& bi, float* s_v, int* s_i, int tid) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        take_max(ov, oi, bv, bi);
    }
    __syncthreads();  // earlier readers of s_v / s_i are done
    if ((tid & (kWave - 1)) == 0) {
        s_v[tid / kWave] = bv;
        s_i[tid / kWave] = bi;
    }
    __syncthreads();
    bv = s_v[0];
    bi = s_i[0];
#pragma unroll
    for (int w = 1; w < NTHR / kWave; ++w) take_max(s_v[w], s_i[w], bv, bi);
}

template <bool F32, int NTHR>
__global__ __launch_bounds__(NTHR) void argmax_kernel(const SelectArgs p) {
    constexpr int ES = F32 ? 4 : 2;    // bytes per element
    constexpr int EPC = 16 / ES;       // elements per 16-byte chunk
    constexpr int STEP = NTHR * kArgUnroll;
    __shared__ float s_v[NTHR / kWave];
    __shared__ int s_i[NTHR / kWave];

    const int tid = threadIdx.x;
    const int np = p.np;
    const size_t row = blockIdx.x / np;
    // this workgroup's part of the row, elements [lo, lo + V): parts of whole
    // 16-byte chunks (each the same distance from a chunk boundary as the
    // row), the last one shorter or empty
    const long long seg = (((long long)p.V + np - 1) / np + EPC - 1) / EPC * EPC;
    const int lo = (int)min((long long)(blockIdx.x % np) * seg, (long long)p.V);
    const int V = (int)(min(lo + seg, (long long)p.V) - lo);
    const unsigned char* base = static_cast<const unsigned char*>(p.logits) + (row * (size_t)p.V + lo) * ES;
    // elements up to the first 16-byte boundary of the row, 16-byte chunks,
    // then the elements past the last whole chunk
    const int mis = (int)((reinterpret_cast<uintptr_t>(base) & 15) / ES);
    const int head = mis ? min(EPC - mis, V) : 0;
    const int nbody = (V - head) / EPC;
    const int tail0 = head + nbody * EPC;
    const global_ptr<const u32x4> body = (global_ptr<const u32x4>)(base + (size_t)head * ES);

    // the thread's chunks c0 + tid + u * NTHR, in increasing order:
    // a strictly larger maximum is the only update needed
    float cv = -__builtin_inff();
    int cb = -1;
    u32x4 cr = {0u, 0u, 0u, 0u};  // the chosen chunk itself (re-reading it would miss L2)
    const int nfull = nbody / STEP;
    for (int it = 0; it < nfull; ++it) {
        const int c0 = it * STEP + tid;
        u32x4 r[kArgUnroll];
#pragma unroll
        for (int u = 0; u < kArgUnroll; ++u) r[u] = __builtin_nontemporal_load(&body[c0 + u * NTHR]);
#pragma unroll
        for (int u = 0; u < kArgUnroll; ++u) {
            const float m = chunk_max<F32>(r[u]);
            if (m > cv) {
                cv = m;
                cb = c0 + u * NTHR;
                cr = r[u];
            }
        }
    }
    if (nfull * STEP < nbody) {  // the last, partial step (loads clamped into the row)
        const int c0 = nfull * STEP + tid;
        u32x4 r[kArgUnroll];
#pragma unroll
        for (int u = 0; u < kArgUnroll; ++u) r[u] = __builtin_nontemporal_load(&body[min(c0 + u * NTHR, nbody - 1)]);
#pragma unroll
        for (int u = 0; u < kArgUnroll; ++u) {
            const float m = chunk_max<F32>(r[u]);
            if (c0 + u * NTHR < nbody && m > cv) {
                cv = m;
                cb = c0 + u * NTHR;
                cr = r[u];
            }
        }
    }
    float bv = -__builtin_inff();
    int bi = INT_MAX;
    if (cb >= 0) {  // the first element of the chosen chunk equal to its maximum
        bv = cv;
        bi = head + cb * EPC + chunk_find<F32>(cr, cv);
    }
    if (tid < head) take_max(elem<F32>(base, tid), tid, bv, bi);
    for (int i = tail0 + tid; i < V; i += NTHR) take_max(elem<F32>(base, i), i, bv, bi);
    block_take_max<NTHR>(bv, bi, s_v, s_i, tid);

    if (bi == INT_MAX || bv == -__builtin_inff()) {
        // the row's largest value is -inf (or every value is NaN): no chunk
        // maximum beat the starting value, so scan every element under the
        // full rule (the same decision in every thread)
        bv = -__builtin_inff();
        bi = INT_MAX;
        for (int i = tid; i < V; i += NTHR) take_max(elem<F32>(base, i), i, bv, bi);
        block_take_max<NTHR>(bv, bi, s_v, s_i, tid);
    }
    if (tid == 0) {
        if (np == 1) p.target[row] = bi == INT_MAX ? 0 : bi;  // a row of NaN: 0
        else p.part[blockIdx.x] = ArgPart{bv, bi == INT_MAX ? INT_MAX : lo + bi};
    }
}

// The argmax of a split row from its parts (same rule; no number: 0).  The
// parts are loaded eight at a time (a repeated part, from the clamp, changes
// nothing), so that the loads are in flight together.
__device__ __forceinline__ int combine_row(const SelectArgs& p, size_t row) {
    const ArgPart* pp = p.part + row * p.np;
    float bv = -__builtin_inff();
    int bi = INT_MAX;
    for (int q0 = 0; q0 < p.np; q0 += 8) {
        ArgPart e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = pp[min(q0 + j, p.np - 1)];
#pragma unroll
        for (int j = 0; j < 8; ++j) take_max(e[j].v, e[j].i, bv, bi);
    }
    return bi == INT_MAX ? 0 : bi;
}

__global__ __launch_bounds__(256) void walk_kernel(const SelectArgs p) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= p.B) return;  // whole waves
    const int T = p.T;
    const int n = lane;
    const bool valid = n < T;
    // node n's parent and token (lanes past the last node, and every lane
    // when T = 0, read nothing)
    int par = n - 1, tok = -1;
    if (valid) {
        if (p.parent) par = p.parent[(size_t)b * T + n];
        tok = p.tokens[(size_t)b * T + n];
    }
    const size_t rb = (size_t)b * (T + 1);
    int tgt, tgt_last;  // target of row n (rows 0 .. 63), and of row T (the only row past 63 when T = 64)
    if (p.np > 1) {  // split rows: combine the parts and write target (every row, as the argmax does)
        tgt = combine_row(p, rb + min(n, T));
        if (n <= T) p.target[rb + n] = tgt;
        if (T == 64) {
            tgt_last = combine_row(p, rb + 64);
            if (lane == 0) p.target[rb + 64] = tgt_last;
        } else {
            tgt_last = __shfl(tgt, T, kWave);
        }
    } else {
        tgt = p.target[rb + min(n, T)];
        tgt_last = p.target[rb + T];
    }
    if (__ballot(valid && (par < -1 || par >= n)) != 0ull) {
        if (lane == 0 && p.status) atomicOr(p.status, LDV_STATUS_BAD_PARENT);
        return;  // outputs of the sequence left unwritten
    }
    int cur = -1, len = 0;
    for (int it = 0; it < T; ++it) {  // a path has at most T nodes
        const int r = cur + 1;
        const int sh = __shfl(tgt, r & 63, kWave);
        const int want = r < 64 ? sh : tgt_last;
        const uint64_t m = __ballot(valid && par == cur && tok == want);
        if (m == 0ull) break;
        cur = __builtin_ctzll(m);
        ++len;
    }
    const int r = cur + 1;
    const int sh = __shfl(tgt, r & 63, kWave);
    const int bonus = r < 64 ? sh : tgt_last;
    if (lane == 0) {
        p.accepted[b] = cur;
        if (p.accepted_len) p.accepted_len[b] = len;
        if (p.bonus) p.bonus[b] = bonus;
    }
}

hipError_t launch_select(const SelectArgs& a, bool f32_logits, hipStream_t stream) {
    const long long rows = (long long)a.B * (a.T + 1);
    if (rows <= 0) return hipSuccess;
    const dim3 grid((unsigned)(rows * a.np));
    if (rows >= kArgFillRows || a.np > 1) {
        if (f32_logits)
            hipLaunchKernelGGL((argmax_kernel<true, kArgThreadsNarrow>), grid, dim3(kArgThreadsNarrow), 0, stream, a);
        else
            hipLaunchKernelGGL((argmax_kernel<false, kArgThreadsNarrow>), grid, dim3(kArgThreadsNarrow), 0, stream, a);
    } else {
        if (f32_logits)
            hipLaunchKernelGGL((argmax_kernel<true, kArgThreadsWide>), grid, dim3(kArgThreadsWide), 0, stream, a);
        else
            hipLaunchKernelGGL((argmax_kernel<false, kArgThreadsWide>), grid, dim3(kArgThreadsWide), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(walk_kernel, dim3((unsigned)((a.B + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ldv
