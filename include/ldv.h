/*
 * ldv.h - draft verification through a gated-delta-rule linear-attention
 * layer on AMD Instinct MI355X (gfx950).
 *
 * The layer's recurrence, per head, over a draft tree in topological order:
 *
 *     S_n = a_n * S_p(n) * (I - beta_n k_n k_n^T) + beta_n v_n k_n^T,
 *     o_n = S_n q_n,                 S_p(n) = S0 when p(n) = -1,
 *
 * with S a d_v x d_k matrix stored row-major ([d_v][d_k], row = value index).
 * The Bole page (arXiv 2608.01651, section IV, Eq. (2)) gives the closed form
 * that verifies every proposal node at once from the committed state; its
 * S_pre is S0 transposed.  Eq. (7) of the same section splits the value
 * columns into independent tiles; Eq. (9) and its "Lemma 1" keep only the
 * node factors (gate products P, keys K, corrections U) plus the one
 * committed state, so that only the accepted node's state is ever formed
 * (the page's summary makes the same point: of all proposal nodes, only
 * the one kept after sampling gets its state built).  The ReaDy page (arXiv 2610.20503, Fig. 2a, 3, 4) reads committed
 * recurrent states at chosen positions for the drafter.
 *
 * Conventions shared by every call:
 *   - Pointers are device memory owned by the caller (hipMalloc or a PyTorch
 *     tensor).  The library allocates nothing and keeps no state, so calls
 *     are thread-safe.  Tensors are dense and row-major in the shapes given.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     null stream) and returns without synchronising.
 *   - The return value reports argument errors found on the host before
 *     anything is enqueued: LDV_OK, LDV_ERR_ARG (NULL required pointer,
 *     negative size, bad dtype code, misaligned pointer), LDV_ERR_UNSUPPORTED
 *     (a size outside what the kernels implement), LDV_ERR_LAUNCH (the HIP
 *     launch failed).  A size of zero in B, T, H or P is a no-op returning
 *     LDV_OK.
 *   - Data errors can only be seen on the device: each kernel ORs
 *     LDV_STATUS_* bits into *status (a device int; NULL = do not report) and
 *     leaves the outputs of the affected sequence or position unwritten.
 *   - Alignment: q, k, v, S0, o, u, S_out, pool, queries, states_out need 16
 *     bytes; the [B, T, H] gate/log arrays, index arrays and status need 4.
 *   - Supported sizes: d_k == d_v in {16, 32, 64, 128}; 1 <= T <= 64.
 *   - One launch holds at most 2^32 - 1 work-items (the dispatch grid size
 *     is 32 bits), so B * H <= 2^23 - 1 for verify, B * H <= 2^22 - 1 for
 *     long chains, B * H <= 2^21 - 1 for commit, B * P * H <= 2^23 - 1 for
 *     the gathers,
 *     B * H * ceil(P * Qn / 64) <= 2^23 - 1 for the in-block reads and
 *     B * (T + 1) <= 2^23 - 1 for selection; larger shapes return
 *     LDV_ERR_UNSUPPORTED.
 *   - Drafts of different lengths in one batch: T is the batch's largest
 *     draft; a shorter draft is padded with nodes placed after its real
 *     ones (each under any earlier node, or a root) with draft token -1.
 *     A node's outputs depend only on its own root-to-node path (Eq. (2)),
 *     so padding leaves every real node's o, u and log P unchanged, and
 *     ldv_select_accepted never accepts a node whose token is outside
 *     [0, V), so the committed state is always a real node's.
 */
#ifndef LDV_H
#define LDV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LDV_OK 0
#define LDV_ERR_ARG (-1)
#define LDV_ERR_UNSUPPORTED (-2)
#define LDV_ERR_LAUNCH (-3)

/* Bits ORed into *status by the kernels. */
#define LDV_STATUS_BAD_PARENT 1   /* parent[b, n] outside [-1, n-1] */
#define LDV_STATUS_BAD_ACCEPTED 2 /* accepted[b] outside [-1, T-1] */
#define LDV_STATUS_BAD_SLOT 4     /* slot[b, p] outside [0, num_slots) */
#define LDV_STATUS_BAD_POSITION 8 /* pos[b, p] outside [-1, T-1] */

/* Element type of q / k / v / queries. */
#define LDV_BF16 0
#define LDV_F32 1

#define LDV_MAX_T 64
/* Longest chain ldv_verify_chain_long and ldv_commit_state (chain) accept.
 * log P is an fp32 sum counted from S0, and commit forms its weights as
 * exp(log P_n - log P_m): each weight carries a relative error of about one
 * fp32 ulp of |log P|, which grows with the chain.  At 8192 nodes, with
 * decay gates a = exp(-softplus(x)), x ~ N(0, 1) or N(2, 1), a simulation of
 * these fp32 sums keeps the committed state within 2.3e-4 of the exact one;
 * at 16384 nodes it reached 1.4e-3 and at 65536 nodes 1.3e-3 to 8e-4, near
 * the 2e-3 bound, so longer chains are not accepted. */
#define LDV_MAX_LONG_T 8192

/*
 * Verify a draft tree: for every node n of every (sequence b, head h),
 *     o[b, n, h, :] = S_n q_n
 * computed from the committed state S0 for all nodes at once (Bole page,
 * section IV, Eq. (2), evaluated per value tile as in Eq. (7)).
 *
 *   q, k      [B, T, H, dk]  element type qkv_dtype
 *   v         [B, T, H, dv]  element type qkv_dtype
 *   a, beta   [B, T, H] fp32; a in [0, 1] (decay gate), beta in [0, 1]
 *   S0        [B, H, dv, dk] fp32, the committed state (read only)
 *   parent    [B, T] int32, parent[b, n] in [-1, n-1] (-1: child of S0);
 *             nodes are in topological order, several roots are allowed
 *   o         [B, T, H, dv] fp32 (written)
 *   u_out     [B, T, H, dv] fp32, the node corrections U of Eq. (2)
 *             (u_n = beta_n (v_n - a_n S_p(n) k_n)), written
 *   logp_out  [B, T, H] fp32, log P_n = sum of log a over the root-to-n path
 *             (natural log), each log a clamped below at -126 ln 2 = -87.34
 *             (a zero gate stays finite)
 *   u_out and logp_out are the factors ldv_commit_state needs; pass both or
 *   neither (NULL, NULL: no commit will follow).
 * A sequence whose parent row is invalid gets LDV_STATUS_BAD_PARENT and none
 * of its outputs are written.  T * H * dk * 4 must stay below 4 GiB (each
 * (sequence, head) is accessed through views with 32-bit byte offsets);
 * larger shapes return LDV_ERR_UNSUPPORTED.
 */
int ldv_verify_tree(int B, int T, int H, int dk, int dv, int qkv_dtype,
                    const void* q, const void* k, const void* v,
                    const float* a, const float* beta, const float* S0,
                    const int32_t* parent,
                    float* o, float* u_out, float* logp_out,
                    int* status, void* stream);

/*
 * Verify a chain (a draft block): ldv_verify_tree with parent[b, n] = n - 1,
 * no parent array needed.  The block-of-drafts case of the ReaDy page
 * (Fig. 2a: verification determines the accepted prefix).
 */
int ldv_verify_chain(int B, int T, int H, int dk, int dv, int qkv_dtype,
                     const void* q, const void* k, const void* v,
                     const float* a, const float* beta, const float* S0,
                     float* o, float* u_out, float* logp_out,
                     int* status, void* stream);

/*
 * Verify a chain of any length up to LDV_MAX_LONG_T (a long draft block).
 * The chain is cut into chunks of LDV_MAX_T consecutive nodes; chunk c is
 * verified with the closed form from the state at the end of chunk c - 1,
 * which the verify of chunk c - 1 also forms, in S_work, from its own
 * factors (the chunk form: the Bole page's Eq. (2) per chunk, Eq. (9) at the
 * chunk's last node to pass the state on).  When B * H is at most the CU
 * count (256) one kernel launch verifies every chunk, each workgroup taking
 * its head's chunks in order; larger grids get one launch per chunk, in
 * order on `stream`.  Results are those of ldv_verify_chain on the whole
 * chain: o, the node corrections u_n = beta_n (v_n - a_n S_{n-1} k_n) and
 * log P_n counted from S0, so ldv_commit_state (no parent array) commits any
 * node from S0 (see LDV_MAX_LONG_T for the precision of log P).
 *
 *   q, k, v, a, beta, S0, o: as for ldv_verify_chain; u_out and logp_out are
 *             required
 *   S_work    [B, H, dv, dk] fp32 scratch owned by the caller, not
 *             overlapping S0; needed when T > LDV_MAX_T (may be NULL
 *             otherwise); its contents on return are unspecified
 * T <= LDV_MAX_T is the same as ldv_verify_chain.
 */
int ldv_verify_chain_long(int B, int T, int H, int dk, int dv, int qkv_dtype,
                          const void* q, const void* k, const void* v,
                          const float* a, const float* beta, const float* S0,
                          float* o, float* u_out, float* logp_out, float* S_work,
                          int* status, void* stream);

/*
 * Commit: form only the state of the accepted node (Bole page, summary and
 * section IV, Eq. (9) / "Lemma 1"):
 *     n = accepted[b];  n = -1: S_out[b, h] = S0[b, h]
 *     else S_out[b, h] = P_n S0[b, h] + sum_{m on root-to-n path} (P_n / P_m) u_m k_m^T
 * with P = exp(logp) and u, logp as written by the verify call on the same
 * k, parent and S0.
 *
 *   k         [B, T, H, dk] element type k_dtype
 *   u         [B, T, H, dv] fp32, logp [B, T, H] fp32 (from verify)
 *   parent    [B, T] int32 or NULL for a chain; T <= LDV_MAX_T with a
 *             parent array, T <= LDV_MAX_LONG_T for a chain
 *   accepted  [B] int32 in [-1, T-1]
 *   S0        [B, H, dv, dk] fp32; S_out [B, H, dv, dk] fp32.  S_out == S0
 *             (in place) is allowed and then heads with accepted = -1 are not
 *             touched; any other overlap of S_out and S0 is undefined.
 * Bad accepted[b] -> LDV_STATUS_BAD_ACCEPTED, bad parent on the sequence ->
 * LDV_STATUS_BAD_PARENT; that sequence's S_out is left unwritten.
 */
int ldv_commit_state(int B, int T, int H, int dk, int dv, int k_dtype,
                     const void* k, const float* u, const float* logp,
                     const int32_t* parent, const int32_t* accepted,
                     const float* S0, float* S_out,
                     int* status, void* stream);

/*
 * Gather committed states at chosen positions and read them with drafter
 * queries (ReaDy page, Fig. 2a: position-specific reads from committed
 * recurrent states; Fig. 3: direct gathering without an intermediate copy):
 *     s = slot[b, p]
 *     o[b, p, h, i, :]        = pool[s, h] queries[b, p, h, i, :]   (i < Qn)
 *     states_out[b, p, h]     = pool[s, h]                          (bit copy)
 *
 *   pool        [num_slots, H, dv, dk] fp32
 *   slot        [B, P] int32 in [0, num_slots); duplicates allowed
 *   queries     [B, P, H, Qn, dk] element type q_dtype, or NULL (Qn ignored)
 *   o           [B, P, H, Qn, dv] fp32 or NULL (both queries and o, or neither)
 *   states_out  [B, P, H, dv, dk] fp32 or NULL
 * A bad slot -> LDV_STATUS_BAD_SLOT and that position's outputs are unwritten.
 */
int ldv_gather_states(int B, int P, int H, int dk, int dv, int num_slots, int Qn, int q_dtype,
                      const float* pool, const int32_t* slot, const void* queries,
                      float* o, float* states_out, int* status, void* stream);

/*
 * Read states inside the verified block without forming them.  The drafter
 * of the ReaDy page (arXiv 2610.20503, Fig. 2a) reads recurrent states at
 * chosen positions; for a node j of the block just verified, the Bole page
 * (arXiv 2608.01651, section IV, Eq. (9) / "Lemma 1") writes its state from
 * the verify factors, so that
 *     j = pos[b, p] in [-1, T-1]
 *     o[b, p, h, i, :] = S_j q = P_j S0[b, h] q + sum_{m on root-to-j path} (P_j / P_m) (k_m . q) u_m
 * with q = queries[b, p, h, i, :] and P = exp(logp); j = -1 reads S0 itself.
 * Each head's S0 is read once for all P x Qn queries.
 *
 *   k         [B, T, H, dk] element type qk_dtype (the verified block's keys)
 *   u, logp   [B, T, H, dv], [B, T, H] fp32, as written by the verify call
 *   parent    [B, T] int32 or NULL for a chain
 *   S0        [B, H, dv, dk] fp32, the committed state the block was verified from
 *   pos       [B, P] int32 in [-1, T-1]; duplicates allowed
 *   queries   [B, P, H, Qn, dk] element type qk_dtype
 *   o         [B, P, H, Qn, dv] fp32 (written)
 * A position outside [-1, T-1] -> LDV_STATUS_BAD_POSITION and its outputs are
 * unwritten.  The parent row is needed only when a valid position of the
 * sequence is a node; if it is then invalid -> LDV_STATUS_BAD_PARENT and
 * nothing of that sequence is written.  Qn == 0 is a no-op.
 */
int ldv_read_block_states(int B, int T, int H, int dk, int dv, int P, int Qn, int qk_dtype,
                          const void* k, const float* u, const float* logp, const int32_t* parent,
                          const float* S0, const int32_t* pos, const void* queries, float* o,
                          int* status, void* stream);

/*
 * The state reads written straight into packed drafter features.  The
 * ReaDy page's drafter combines target hidden features with the
 * position-specific state reads (Fig. 2a); its state reader fuses state
 * preparation and feature packing so that no intermediate tensor is
 * materialised (Fig. 3).  The pages do not give the feature layout, so the
 * destination is any row-major matrix: reading p of sequence b fills row
 * b * P + p (row stride feat_ld elements) at
 *     feat[(b * P + p) * feat_ld + feat_col + (h * Qn + i) * dv + v]
 *         = o[b, p, h, i, v]
 * for every head h, query i < Qn and value v (the o of ldv_gather_states /
 * ldv_read_block_states); every other element of feat is left as it is (the
 * caller's hidden features, for instance).  feat_dtype is LDV_F32, or
 * LDV_BF16 for values rounded to nearest even from the same fp32 results.
 * Requirements (LDV_ERR_ARG otherwise): queries given and Qn > 0;
 * feat_col + H * Qn * dv <= feat_ld; feat_ld and feat_col multiples of 4;
 * feat aligned to 16 bytes (fp32) or 8 bytes (bf16).  The other arguments,
 * checks and status bits are those of the unpacked call; the gather form
 * writes no state copies.
 */
int ldv_gather_states_packed(int B, int P, int H, int dk, int dv, int num_slots, int Qn, int q_dtype,
                             const float* pool, const int32_t* slot, const void* queries,
                             void* feat, long long feat_ld, long long feat_col, int feat_dtype,
                             int* status, void* stream);
int ldv_read_block_states_packed(int B, int T, int H, int dk, int dv, int P, int Qn, int qk_dtype,
                                 const void* k, const float* u, const float* logp,
                                 const int32_t* parent, const float* S0, const int32_t* pos,
                                 const void* queries,
                                 void* feat, long long feat_ld, long long feat_col, int feat_dtype,
                                 int* status, void* stream);

/*
 * Greedy selection of the accepted node, on the device.  Verification fixes
 * the accepted prefix (ReaDy page, Fig. 2a) and only the node selected after
 * sampling keeps its state (Bole page, summary and section IV); with greedy
 * decoding the selection is a walk from the committed state:
 *     target[b, r] = argmax_v logits[b, r, v]     (r = 0 .. T)
 *     cur = -1; while some node c with parent[c] == cur has
 *               tokens[b, c] == target[b, cur + 1]: cur = the lowest such c
 *     accepted[b] = cur;  accepted_len[b] = nodes walked (cur's depth);
 *     bonus[b] = target[b, cur + 1] (the target's token after the accepted node)
 * argmax: the larger value wins, equal values go to the lower index, NaN
 * never wins (+0 equals -0) and an all-NaN row gives 0.
 *
 *   logits        [B, T+1, V] element type logits_dtype (LDV_BF16 / LDV_F32);
 *                 row 0 is the target's prediction at the committed position,
 *                 row n+1 its prediction after draft node n
 *   tokens        [B, T] int32 draft token of each node (any value; one
 *                 outside [0, V) never matches)
 *   parent        [B, T] int32 or NULL for a chain
 *   target        [B, T+1] int32 (written: every row's argmax)
 *   accepted      [B] int32 in [-1, T-1] (written), ready for ldv_commit_state
 *   accepted_len, bonus  [B] int32 or NULL
 *   workspace     NULL, or device memory of at least
 *                 ldv_select_workspace_bytes(B, T, V) bytes, 8-byte aligned,
 *                 owned by the caller; its contents on entry and return do
 *                 not matter.  With it, when there are few rows, each row is
 *                 split over several workgroups (their partial results go
 *                 through the workspace), which keeps every CU busy; the
 *                 results are the same either way.  Calls that share a
 *                 workspace must not overlap.
 *   workspace_bytes  its size; a non-NULL workspace smaller than needed
 *                 returns LDV_ERR_ARG
 * The logits need element alignment only.  A sequence with an invalid parent
 * row -> LDV_STATUS_BAD_PARENT; its target row is written, its accepted,
 * accepted_len and bonus are not.  V must be >= 1; 0 <= T <= 64.  With T = 0
 * (no draft nodes) tokens may be NULL: target row 0 is written, accepted is
 * -1, accepted_len 0 and bonus row 0's argmax.
 */
int ldv_select_accepted(int B, int T, int V, int logits_dtype, const void* logits,
                        const int32_t* tokens, const int32_t* parent, int32_t* target,
                        int32_t* accepted, int32_t* accepted_len, int32_t* bonus,
                        int* status, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ldv_select_accepted without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  It
 * splits few, long rows exactly as ldv_select_accepted does when given a
 * workspace, with the partial results in an array of the library instead: a
 * fixed 48 KiB (6144 entries) per GPU, reserved on each GPU the library runs
 * on until the process ends, its address resolved on the first call on that
 * GPU (the GPU of `stream`, or the current GPU for the null stream).  Every split the selection makes fits it; a larger one would return
 * LDV_ERR_UNSUPPORTED.  Results are those of ldv_select_accepted.  Every call
 * on a GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different host threads) race and must be
 * ordered by the caller.  Arguments, checks and status bits are those of
 * ldv_select_accepted; LDV_ERR_LAUNCH also reports a failure to resolve the
 * array's address.  The caller still passes every output.
 */
int ldv_select_accepted_noalloc(int B, int T, int V, int logits_dtype, const void* logits,
                                const int32_t* tokens, const int32_t* parent, int32_t* target,
                                int32_t* accepted, int32_t* accepted_len, int32_t* bonus,
                                int* status, void* stream);

/*
 * Bytes of workspace ldv_select_accepted uses for B sequences of T nodes and
 * rows of V logits: 0 when it would not split the rows (then the workspace
 * may be NULL at no cost), and 0 for sizes the call rejects.
 */
size_t ldv_select_workspace_bytes(int B, int T, int V);

/* Text for an LDV_OK / LDV_ERR_* return code (static storage). */
const char* ldv_status_string(int code);

/* Library version: major * 10000 + minor * 100 + patch. */
int ldv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LDV_H */
