// The C ABI: host-side argument checks, then one kernel launch per call.
// Every check happens before any HIP call, so argument errors are reported
// without touching a device.
#include <stdint.h>

#include "ldv_kernels.hpp"

#include "../../include/ldv.h"

#define LDV_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// A launch dispatches at most 2^32 - 1 work-items (the dispatch packet's grid
// size is 32 bits).  `units` independent units of at most `per_unit`
// work-items each must fit: verify 512 per (sequence, head), commit 2048 per
// (sequence, head), gather 512 per (sequence, position, head), the in-block
// read 512 per (sequence, head, chunk of 64 queries), selection 512 per row.
bool grid_fits(long long units, long long per_unit) { return units * per_unit <= 0xffffffffLL; }

// Shared checks of the verify calls.
int check_verify(int B, int T, int H, int dk, int dv, int dt, const void* q, const void* k, const void* v,
                 const float* a, const float* beta, const float* S0, const float* o, const float* u_out,
                 const float* logp_out, const int* status) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return LDV_ERR_ARG;
    if (dt != LDV_BF16 && dt != LDV_F32) return LDV_ERR_ARG;
    if ((u_out == nullptr) != (logp_out == nullptr)) return LDV_ERR_ARG;
    if (dk != dv || !supported_d(dk) || T > LDV_MAX_T) return LDV_ERR_UNSUPPORTED;
    if (B == 0 || T == 0 || H == 0) return LDV_OK;
    if (!q || !k || !v || !a || !beta || !S0 || !o) return LDV_ERR_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(S0, 16) || !aligned(o, 16) ||
        !aligned(u_out, 16) || !aligned(a, 4) || !aligned(beta, 4) || !aligned(logp_out, 4) ||
        !aligned(status, 4))
        return LDV_ERR_ARG;
    if (!grid_fits((long long)B * H, 512) || (long long)B * T > 0x7fffffffLL) return LDV_ERR_UNSUPPORTED;
    // each (sequence, head) is read and written through views of T rows of
    // H * d elements with 32-bit byte offsets
    if ((long long)T * H * dk * 4 > 0xffffffffLL) return LDV_ERR_UNSUPPORTED;
    return 1;  // proceed
}

int verify_common(int B, int T, int H, int d, int dt, const void* q, const void* k, const void* v, const float* a,
                  const float* beta, const float* S0, const int32_t* parent, float* o, float* u_out,
                  float* logp_out, int* status, void* stream) {
    ldv::VerifyArgs args{B, T, H, d, T, 0, q, k, v, a, beta, S0, parent, o, u_out, logp_out, status, nullptr, 0};
    hipError_t e = ldv::launch_verify(args, dt == LDV_F32, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LDV_OK : LDV_ERR_LAUNCH;
}

}  // namespace

LDV_EXPORT int ldv_verify_tree(int B, int T, int H, int dk, int dv, int qkv_dtype, const void* q, const void* k,
                               const void* v, const float* a, const float* beta, const float* S0,
                               const int32_t* parent, float* o, float* u_out, float* logp_out, int* status,
                               void* stream) {
    int rc = check_verify(B, T, H, dk, dv, qkv_dtype, q, k, v, a, beta, S0, o, u_out, logp_out, status);
    if (rc != 1) return rc;
    if (!parent || !aligned(parent, 4)) return LDV_ERR_ARG;
    return verify_common(B, T, H, dk, qkv_dtype, q, k, v, a, beta, S0, parent, o, u_out, logp_out, status, stream);
}

LDV_EXPORT int ldv_verify_chain(int B, int T, int H, int dk, int dv, int qkv_dtype, const void* q, const void* k,
                                const void* v, const float* a, const float* beta, const float* S0, float* o,
                                float* u_out, float* logp_out, int* status, void* stream) {
    int rc = check_verify(B, T, H, dk, dv, qkv_dtype, q, k, v, a, beta, S0, o, u_out, logp_out, status);
    if (rc != 1) return rc;
    return verify_common(B, T, H, dk, qkv_dtype, q, k, v, a, beta, S0, nullptr, o, u_out, logp_out, status,
                         stream);
}

LDV_EXPORT int ldv_verify_chain_long(int B, int T, int H, int dk, int dv, int qkv_dtype, const void* q,
                                     const void* k, const void* v, const float* a, const float* beta,
                                     const float* S0, float* o, float* u_out, float* logp_out, float* S_work,
                                     int* status, void* stream) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return LDV_ERR_ARG;
    if (qkv_dtype != LDV_BF16 && qkv_dtype != LDV_F32) return LDV_ERR_ARG;
    if (dk != dv || !supported_d(dk) || T > LDV_MAX_LONG_T) return LDV_ERR_UNSUPPORTED;
    if (B == 0 || T == 0 || H == 0) return LDV_OK;
    if (!q || !k || !v || !a || !beta || !S0 || !o || !u_out || !logp_out) return LDV_ERR_ARG;
    if (T > LDV_MAX_T && !S_work) return LDV_ERR_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(S0, 16) || !aligned(o, 16) ||
        !aligned(u_out, 16) || !aligned(S_work, 16) || !aligned(a, 4) || !aligned(beta, 4) ||
        !aligned(logp_out, 4) || !aligned(status, 4))
        return LDV_ERR_ARG;
    if (!grid_fits((long long)B * H, 1024) || (long long)B * T > 0x7fffffffLL) return LDV_ERR_UNSUPPORTED;
    if ((long long)(T < LDV_MAX_T ? T : LDV_MAX_T) * H * dk * 4 > 0xffffffffLL) return LDV_ERR_UNSUPPORTED;
    if (S_work) {  // S_work must not overlap S0 (the first chunk reads S0 while later ones write S_work)
        const char *w0 = reinterpret_cast<const char*>(S_work), *s0 = reinterpret_cast<const char*>(S0);
        const size_t bytes = (size_t)B * H * dk * dv * 4;
        if (w0 < s0 + bytes && s0 < w0 + bytes) return LDV_ERR_ARG;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const bool f32 = qkv_dtype == LDV_F32;
    const int nch = (T + LDV_MAX_T - 1) / LDV_MAX_T;
    // Every 64-node chunk but the last also forms the state at its last node,
    // the next chunk's base, in S_work (in place from the second chunk on).
    // A grid of at most one block per CU runs every chunk in one launch,
    // each block walking its head's chunks in order (GDN-1.3B shape, 1024
    // nodes: 280 vs 320 us); larger grids measured faster with a launch per
    // chunk (27B-hybrid shape, 256 nodes: 444 vs 465 us), where the chunk
    // boundaries cost little against several rounds of blocks per chunk.
    if (nch > 1 && (long long)B * H <= ldv::kCus) {
        ldv::VerifyArgs va{B, LDV_MAX_T, H, dk, T, 0, q, k, v, a, beta, S0, nullptr, o, u_out, logp_out,
                           status, S_work, nch};
        return ldv::launch_verify(va, f32, st) == hipSuccess ? LDV_OK : LDV_ERR_LAUNCH;
    }
    for (int c = 0; c < nch; ++c) {
        const int t0 = c * LDV_MAX_T, len = T - t0 < LDV_MAX_T ? T - t0 : LDV_MAX_T;
        const bool last = c + 1 == nch;  // the last chunk: the ordinary verify, from S_work
        ldv::VerifyArgs va{B, len, H, dk, T, t0, q, k, v, a, beta, c == 0 ? S0 : S_work, nullptr, o, u_out,
                           logp_out, status, last ? nullptr : S_work, last ? 0 : 1};
        if (ldv::launch_verify(va, f32, st) != hipSuccess) return LDV_ERR_LAUNCH;
    }
    return LDV_OK;
}

LDV_EXPORT int ldv_commit_state(int B, int T, int H, int dk, int dv, int k_dtype, const void* k, const float* u,
                                const float* logp, const int32_t* parent, const int32_t* accepted,
                                const float* S0, float* S_out, int* status, void* stream) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return LDV_ERR_ARG;
    if (k_dtype != LDV_BF16 && k_dtype != LDV_F32) return LDV_ERR_ARG;
    // a chain (no parent array) may be of any length, a tree at most 64 nodes
    if (dk != dv || !supported_d(dk) || (parent && T > LDV_MAX_T) || T > LDV_MAX_LONG_T)
        return LDV_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return LDV_OK;
    if (!accepted || !S0 || !S_out) return LDV_ERR_ARG;
    if (T > 0 && (!k || !u || !logp)) return LDV_ERR_ARG;
    if (!aligned(k, 16) || !aligned(u, 16) || !aligned(S0, 16) || !aligned(S_out, 16) || !aligned(logp, 4) ||
        !aligned(parent, 4) || !aligned(accepted, 4) || !aligned(status, 4))
        return LDV_ERR_ARG;
    if (!grid_fits((long long)B * H, 2048) || (long long)B * T > 0x7fffffffLL) return LDV_ERR_UNSUPPORTED;
    ldv::CommitArgs args{B, T, H, dk, T, 0, -2, k, u, logp, parent, accepted, S0, S_out, status};
    hipError_t e = ldv::launch_commit(args, k_dtype == LDV_F32, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LDV_OK : LDV_ERR_LAUNCH;
}

namespace {

// Checks of a packed destination: fp32 or bf16, rows of ld elements holding
// H * Qn * dv values from column col, vector-aligned.
int check_packed(int H, int Qn, int dv, const void* feat, long long ld, long long col, int dt) {
    if (!feat || (dt != LDV_BF16 && dt != LDV_F32)) return LDV_ERR_ARG;
    if (ld < 0 || col < 0 || col + (long long)H * Qn * dv > ld) return LDV_ERR_ARG;
    if (ld % 4 != 0 || col % 4 != 0 || !aligned(feat, dt == LDV_F32 ? 16 : 8)) return LDV_ERR_ARG;
    return 1;
}

int gather_common(int B, int P, int H, int dk, int dv, int num_slots, int Qn, int q_dtype, const float* pool,
                  const int32_t* slot, const void* queries, ldv::ReadOut o, float* states_out, int* status,
                  void* stream) {
    if (B < 0 || P < 0 || H < 0 || dk <= 0 || dv <= 0 || num_slots < 0) return LDV_ERR_ARG;
    if (q_dtype != LDV_BF16 && q_dtype != LDV_F32) return LDV_ERR_ARG;
    if ((queries == nullptr) != (o.base == nullptr)) return LDV_ERR_ARG;
    if (queries && Qn < 0) return LDV_ERR_ARG;
    if (dk != dv || !supported_d(dk)) return LDV_ERR_UNSUPPORTED;
    if (B == 0 || P == 0 || H == 0) return LDV_OK;
    if (!pool || !slot) return LDV_ERR_ARG;
    if (!aligned(pool, 16) || !aligned(queries, 16) || !aligned(o.base, o.bf16 ? 8 : 16) ||
        !aligned(states_out, 16) || !aligned(slot, 4) || !aligned(status, 4))
        return LDV_ERR_ARG;
    if (!grid_fits((long long)B * P * H, 512)) return LDV_ERR_UNSUPPORTED;
    ldv::GatherArgs args{B, P, H, dk, num_slots, queries ? Qn : 0, pool, slot, queries, o, states_out, status};
    hipError_t e = ldv::launch_gather(args, q_dtype == LDV_F32, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LDV_OK : LDV_ERR_LAUNCH;
}

int read_common(int B, int T, int H, int dk, int dv, int P, int Qn, int qk_dtype, const void* k, const float* u,
                const float* logp, const int32_t* parent, const float* S0, const int32_t* pos, const void* queries,
                ldv::ReadOut o, int* status, void* stream) {
    if (B < 0 || T < 0 || H < 0 || P < 0 || Qn < 0 || dk <= 0 || dv <= 0) return LDV_ERR_ARG;
    if (qk_dtype != LDV_BF16 && qk_dtype != LDV_F32) return LDV_ERR_ARG;
    if (dk != dv || !supported_d(dk) || T > LDV_MAX_T) return LDV_ERR_UNSUPPORTED;
    if (B == 0 || T == 0 || H == 0 || P == 0 || Qn == 0) return LDV_OK;
    if (!k || !u || !logp || !S0 || !pos || !queries || !o.base) return LDV_ERR_ARG;
    if (!aligned(k, 16) || !aligned(u, 16) || !aligned(S0, 16) || !aligned(queries, 16) ||
        !aligned(o.base, o.bf16 ? 8 : 16) || !aligned(logp, 4) || !aligned(parent, 4) || !aligned(pos, 4) ||
        !aligned(status, 4))
        return LDV_ERR_ARG;
    if ((long long)P * Qn > 0x7fffffffLL || !grid_fits((long long)B * H * (((long long)P * Qn + 63) / 64), 512))
        return LDV_ERR_UNSUPPORTED;
    ldv::ReadArgs args{B, T, H, dk, P, Qn, k, u, logp, parent, S0, pos, queries, o, status, 0};
    hipError_t e = ldv::launch_read(args, qk_dtype == LDV_F32, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LDV_OK : LDV_ERR_LAUNCH;
}

}  // namespace

LDV_EXPORT int ldv_gather_states(int B, int P, int H, int dk, int dv, int num_slots, int Qn, int q_dtype,
                                 const float* pool, const int32_t* slot, const void* queries, float* o,
                                 float* states_out, int* status, void* stream) {
    const ldv::ReadOut out{o, (size_t)(H > 0 ? H : 0) * (Qn > 0 ? Qn : 0) * (dv > 0 ? dv : 0), 0, 0};
    return gather_common(B, P, H, dk, dv, num_slots, Qn, q_dtype, pool, slot, queries, out, states_out, status,
                         stream);
}

LDV_EXPORT int ldv_gather_states_packed(int B, int P, int H, int dk, int dv, int num_slots, int Qn, int q_dtype,
                                        const float* pool, const int32_t* slot, const void* queries, void* feat,
                                        long long feat_ld, long long feat_col, int feat_dtype, int* status,
                                        void* stream) {
    if (!queries || Qn <= 0) return LDV_ERR_ARG;
    const int c = check_packed(H, Qn, dv, feat, feat_ld, feat_col, feat_dtype);
    if (c != 1) return c;
    const ldv::ReadOut out{feat, (size_t)feat_ld, (size_t)feat_col, feat_dtype == LDV_BF16};
    return gather_common(B, P, H, dk, dv, num_slots, Qn, q_dtype, pool, slot, queries, out, nullptr, status, stream);
}

LDV_EXPORT int ldv_read_block_states(int B, int T, int H, int dk, int dv, int P, int Qn, int qk_dtype,
                                     const void* k, const float* u, const float* logp, const int32_t* parent,
                                     const float* S0, const int32_t* pos, const void* queries, float* o,
                                     int* status, void* stream) {
    const ldv::ReadOut out{o, (size_t)(H > 0 ? H : 0) * (Qn > 0 ? Qn : 0) * (dv > 0 ? dv : 0), 0, 0};
    return read_common(B, T, H, dk, dv, P, Qn, qk_dtype, k, u, logp, parent, S0, pos, queries, out, status, stream);
}

LDV_EXPORT int ldv_read_block_states_packed(int B, int T, int H, int dk, int dv, int P, int Qn, int qk_dtype,
                                            const void* k, const float* u, const float* logp, const int32_t* parent,
                                            const float* S0, const int32_t* pos, const void* queries, void* feat,
                                            long long feat_ld, long long feat_col, int feat_dtype, int* status,
                                            void* stream) {
    if (Qn <= 0) return LDV_ERR_ARG;
    const int c = check_packed(H, Qn, dv, feat, feat_ld, feat_col, feat_dtype);
    if (c != 1) return c;
    const ldv::ReadOut out{feat, (size_t)feat_ld, (size_t)feat_col, feat_dtype == LDV_BF16};
    return read_common(B, T, H, dk, dv, P, Qn, qk_dtype, k, u, logp, parent, S0, pos, queries, out, status, stream);
}

LDV_EXPORT size_t ldv_select_workspace_bytes(int B, int T, int V) {
    if (B <= 0 || T < 0 || V <= 0 || T > LDV_MAX_T) return 0;
    const long long rows = (long long)B * (T + 1);
    const int np = ldv::select_parts(rows, V);
    return np > 1 ? (size_t)rows * np * sizeof(ldv::ArgPart) : 0;
}

namespace {

// Shared checks of the selection calls: 1 = proceed.
int check_select(int B, int T, int V, int dt, const void* logits, const int32_t* tokens, const int32_t* parent,
                 const int32_t* target, const int32_t* accepted, const int32_t* accepted_len, const int32_t* bonus,
                 const int* status) {
    if (B < 0 || T < 0 || V <= 0) return LDV_ERR_ARG;
    if (dt != LDV_BF16 && dt != LDV_F32) return LDV_ERR_ARG;
    if (T > LDV_MAX_T) return LDV_ERR_UNSUPPORTED;
    if (B == 0) return LDV_OK;
    // T = 0 (no draft nodes): row 0 is still read, nothing is accepted and
    // the bonus token is row 0's argmax; tokens may then be NULL
    if (!logits || (T > 0 && !tokens) || !target || !accepted) return LDV_ERR_ARG;
    if (!aligned(logits, dt == LDV_F32 ? 4 : 2) || !aligned(tokens, 4) || !aligned(parent, 4) ||
        !aligned(target, 4) || !aligned(accepted, 4) || !aligned(accepted_len, 4) || !aligned(bonus, 4) ||
        !aligned(status, 4))
        return LDV_ERR_ARG;
    if (!grid_fits((long long)B * (T + 1), 512)) return LDV_ERR_UNSUPPORTED;
    return 1;
}

int select_launch(int B, int T, int V, int dt, const void* logits, const int32_t* tokens, const int32_t* parent,
                  int32_t* target, int32_t* accepted, int32_t* accepted_len, int32_t* bonus, int* status, int np,
                  ldv::ArgPart* part, void* stream) {
    if (!grid_fits((long long)B * (T + 1) * np, 512)) return LDV_ERR_UNSUPPORTED;
    ldv::SelectArgs args{B, T, V, logits, tokens, parent, target, accepted, accepted_len, bonus, status, np, part};
    hipError_t e = ldv::launch_select(args, dt == LDV_F32, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LDV_OK : LDV_ERR_LAUNCH;
}

}  // namespace

LDV_EXPORT int ldv_select_accepted(int B, int T, int V, int logits_dtype, const void* logits,
                                   const int32_t* tokens, const int32_t* parent, int32_t* target,
                                   int32_t* accepted, int32_t* accepted_len, int32_t* bonus, int* status,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    const int rc = check_select(B, T, V, logits_dtype, logits, tokens, parent, target, accepted, accepted_len, bonus,
                                status);
    if (rc != 1) return rc;
    // with a workspace, rows may be split over several workgroups
    const long long rows = (long long)B * (T + 1);
    int np = 1;
    if (workspace) {
        if (!aligned(workspace, 8)) return LDV_ERR_ARG;
        const int want = ldv::select_parts(rows, V);
        if (want > 1) {
            if (workspace_bytes < (size_t)rows * want * sizeof(ldv::ArgPart)) return LDV_ERR_ARG;
            np = want;
        }
    }
    return select_launch(B, T, V, logits_dtype, logits, tokens, parent, target, accepted, accepted_len, bonus, status,
                         np, static_cast<ldv::ArgPart*>(workspace), stream);
}

LDV_EXPORT int ldv_select_accepted_noalloc(int B, int T, int V, int logits_dtype, const void* logits,
                                           const int32_t* tokens, const int32_t* parent, int32_t* target,
                                           int32_t* accepted, int32_t* accepted_len, int32_t* bonus, int* status,
                                           void* stream) {
    const int rc = check_select(B, T, V, logits_dtype, logits, tokens, parent, target, accepted, accepted_len, bonus,
                                status);
    if (rc != 1) return rc;
    // rows split exactly as ldv_select_accepted splits them with a workspace,
    // the partial results in the library's own array
    const long long rows = (long long)B * (T + 1);
    const int np = ldv::select_parts(rows, V);
    ldv::ArgPart* part = nullptr;
    if (np > 1) {
        if (rows * np > ldv::kSelectScratchParts) return LDV_ERR_UNSUPPORTED;  // beyond the array (no valid split is)
        if (ldv::select_scratch(static_cast<hipStream_t>(stream), &part) != hipSuccess) return LDV_ERR_LAUNCH;
    }
    return select_launch(B, T, V, logits_dtype, logits, tokens, parent, target, accepted, accepted_len, bonus, status,
                         np, part, stream);
}

LDV_EXPORT const char* ldv_status_string(int code) {
    switch (code) {
        case LDV_OK: return "ok";
        case LDV_ERR_ARG: return "invalid argument (null pointer, negative size, bad dtype or misaligned pointer)";
        case LDV_ERR_UNSUPPORTED:
            return "unsupported size (d_k == d_v in {16, 32, 64, 128}, T <= 64 except for chains, and the size "
                   "limits of the call)";
        case LDV_ERR_LAUNCH: return "HIP kernel launch failed";
        default: return "unknown status code";
    }
}

LDV_EXPORT int ldv_version(void) { return 100; }
