// Kernel argument blocks and launchers (host side of the HIP library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ldv {

constexpr int kCus = 256;  // MI355X: compute units

// Node arrays ([B, T, H, ...] and [B, T, H]) are addressed as node
// b * Ts + t0 + n for n < T: a call on a whole draft has Ts = T and t0 = 0;
// a chunk of a longer chain views nodes [t0, t0 + T) of arrays with Ts nodes
// per sequence.  For t0 > 0, log P is counted from the committed state: the
// value at node t0 - 1 (already written) is the chunk's base.

struct VerifyArgs {
    int B, T, H, D;
    int Ts, t0;
    const void* q;
    const void* k;
    const void* v;
    const float* a;
    const float* beta;
    const float* S0;
    const int32_t* parent;  // NULL: chain
    float* o;
    float* u_out;     // may be NULL (together with logp_out)
    float* logp_out;  // may be NULL
    int* status;      // may be NULL
    // may be NULL; else the call verifies `chunks` 64-node chunks of a chain
    // of Ts > 64 nodes from node t0, each from the state at the end of the
    // one before (S0 for the chunk at node 0, else S_next, the work state),
    // and forms each chunk's end state in S_next unless it ends the chain
    float* S_next;
    int chunks;
};

struct CommitArgs {
    int B, T, H, D;
    int Ts, t0;
    int acc_const;  // >= -1: the accepted node of every sequence; -2: read accepted[]
    const void* k;
    const float* u;
    const float* logp;
    const int32_t* parent;  // NULL: chain
    const int32_t* accepted;
    const float* S0;
    float* S_out;
    int* status;
};

// Destination of the o values of state reads: for reading p of sequence b,
// row b * P + p of a matrix with a row stride of `ld` elements, elements
// col + (h * Qn + i) * D + v for head h, query i, value v; fp32, or bf16
// rounded to nearest even.  The o tensor [B, P, H, Qn, D] is the case
// ld = H * Qn * D, col = 0, fp32; a drafter feature buffer is any other.
struct ReadOut {
    void* base;  // NULL: no reads
    size_t ld, col;
    int bf16;
};
struct GatherArgs {
    int B, P, H, D, num_slots, Qn;
    const float* pool;
    const int32_t* slot;
    const void* queries;  // may be NULL
    ReadOut o;            // base may be NULL
    float* states_out;    // may be NULL
    int* status;
};

struct ReadArgs {
    int B, T, H, D, P, Qn;
    const void* k;
    const float* u;
    const float* logp;
    const int32_t* parent;  // NULL: chain
    const float* S0;
    const int32_t* pos;
    const void* queries;
    ReadOut o;
    int* status;  // may be NULL
    int stage_o;  // set by the launch: 1 = the O tile goes through LDS before the stores
};

// The argmax of one part of a logits row: the largest value and its index
// in the row (INT_MAX: no element of the part is a number above -inf, or the
// part is empty).
struct ArgPart {
    float v;
    int i;
};

struct SelectArgs {
    int B, T, V;
    const void* logits;      // [B, T+1, V]
    const int32_t* tokens;   // [B, T]
    const int32_t* parent;   // NULL: chain
    int32_t* target;         // [B, T+1]
    int32_t* accepted;       // [B]
    int32_t* accepted_len;   // may be NULL
    int32_t* bonus;          // may be NULL
    int* status;             // may be NULL
    int np;                  // workgroups per logits row (1: the row's argmax goes straight to target)
    ArgPart* part;           // np > 1: [B, T+1, np] partial results, combined by the walk
};

// Workgroups per logits row for B * (T + 1) = rows rows of V elements when
// the caller provides the workspace for the partial results (1 otherwise).
int select_parts(long long rows, int V);

// Entries of the library's own split-row workspace (ldv_select_accepted_noalloc):
// every split select_parts makes fits (fewer than 2048 rows, at most
// ceil(4096 / rows) parts each).
constexpr long long kSelectScratchParts = 6144;

// The address of that workspace on the GPU the stream belongs to (the
// current GPU for the null stream), resolved once per device.
hipError_t select_scratch(hipStream_t stream, ArgPart** out);

// Each launcher assumes arguments already validated by the C ABI layer and
// returns the HIP launch status.
hipError_t launch_verify(const VerifyArgs& a, bool f32_inputs, hipStream_t stream);
hipError_t launch_commit(const CommitArgs& a, bool f32_k, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, bool f32_queries, hipStream_t stream);
hipError_t launch_read(const ReadArgs& a, bool f32_inputs, hipStream_t stream);
hipError_t launch_select(const SelectArgs& a, bool f32_logits, hipStream_t stream);

}  // namespace ldv
