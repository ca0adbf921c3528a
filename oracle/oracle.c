/*
 * fp64 CPU oracle for draft verification through a gated-delta-rule layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it is used by tests/, by the smoke check and by the
 * benchmark's CPU-baseline leg, and by nothing else.  It shares no code with
 * the HIP library.
 *
 * What it computes is the plain definition, walked token by token:
 *
 *   S_n = a_n * S_{p(n)} * (I - b_n k_n k_n^T) + b_n v_n k_n^T,   o_n = S_n q_n,
 *   S_{p(n)} = S0 when p(n) = -1,
 *
 * with S a d_v x d_k matrix (row-major, S[i][j], i over values, j over keys).
 * This is the gated delta rule that the Bole page (arXiv 2608.01651, section
 * IV, context of Eq. (2)) says is executed sequentially over the draft tree;
 * its closed form O = D_P Q S_pre + C (I+G)^{-1} D_beta (V - D_P K S_pre) of
 * Eq. (2) uses the transposed orientation S_pre = S0^T.  The oracle never
 * uses the closed form: every node's state is rebuilt from S0 along the
 * node's root-to-node path.
 *
 * Commit (Bole page, summary: of all proposal nodes only the one kept
 * after sampling gets its state built) is the walk's state at the accepted node; gather (ReaDy page,
 * Fig. 2a-3: position-specific reads from committed recurrent states) is a
 * copy of a pool entry plus o = S q for each query.
 *
 * Inputs are the exact fp32 values handed to the GPU (bf16 inputs arrive as
 * their exact fp32 widening); all arithmetic is fp64.
 *
 * Two steps around verify follow from the same definitions:
 *   - reads inside the verified block (ReaDy page, Fig. 2a: the drafter reads
 *     recurrent states at chosen positions): o = S_j q for a node j of the
 *     block, S_j rebuilt by the same walk (S0 itself for j = -1);
 *   - greedy accepted-node selection (Bole page, summary and section IV:
 *     verification decides the accepted prefix, then only the selected state
 *     is kept): walk down from the committed state, at each step taking the
 *     child whose draft token equals the target's most likely token there.
 *
 * Status bits (returned, OR-ed): 1 = a parent index outside [-1, n-1],
 * 2 = an accepted index outside [-1, T-1], 4 = a slot index outside
 * [0, num_slots), 8 = a read position outside [-1, T-1].  The outputs of an
 * affected sequence (or position) are left untouched.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BAD_PARENT 1
#define OR_BAD_ACCEPTED 2
#define OR_BAD_SLOT 4
#define OR_BAD_POSITION 8

/* ---------------------------------------------------------------- threads */

typedef struct {
    void (*fn)(void* ctx, long item, double* work);
    void* ctx;
    long n_items;
    long next;
    long work_doubles;
    pthread_mutex_t lock;
} pool_t;

static void* pool_worker(void* arg) {
    pool_t* p = (pool_t*)arg;
    double* work = (double*)malloc(sizeof(double) * (size_t)(p->work_doubles > 0 ? p->work_doubles : 1));
    for (;;) {
        pthread_mutex_lock(&p->lock);
        long it = p->next++;
        pthread_mutex_unlock(&p->lock);
        if (it >= p->n_items) break;
        p->fn(p->ctx, it, work);
    }
    free(work);
    return NULL;
}

/* Run fn(ctx, item, work) for item in [0, n_items) on nthreads threads.  Each
 * thread owns a private work buffer of work_doubles doubles. */
static void run_items(void (*fn)(void*, long, double*), void* ctx, long n_items,
                      long work_doubles, int nthreads) {
    pool_t p;
    p.fn = fn;
    p.ctx = ctx;
    p.n_items = n_items;
    p.next = 0;
    p.work_doubles = work_doubles;
    pthread_mutex_init(&p.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((long)nthreads > n_items) nthreads = (int)(n_items > 0 ? n_items : 1);
    pthread_t tid[256];
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&tid[t], NULL, pool_worker, &p) == 0) started = t;
        else break;
    pool_worker(&p);
    for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
    pthread_mutex_destroy(&p.lock);
}

/* ------------------------------------------------------- the definition */

/* One token of the gated delta rule on S (dv x dk, row-major):
 *   x = S k;   S <- a * (S - b x k^T) + b v k^T
 * which is S <- a S (I - b k k^T) + b v k^T with x formed before the update.
 * If u is not NULL it receives the token's correction u = b (v - a x), the
 * vector with S_new = a S_old + u k^T. */
static void gdr_token(double* S, int dk, int dv, const float* k, const float* v,
                      double a, double b, double* x, double* u) {
    for (int i = 0; i < dv; ++i) {
        double s = 0.0;
        for (int j = 0; j < dk; ++j) s += S[(size_t)i * dk + j] * (double)k[j];
        x[i] = s;
    }
    if (u)
        for (int i = 0; i < dv; ++i) u[i] = b * ((double)v[i] - a * x[i]);
    for (int i = 0; i < dv; ++i) {
        double bx = b * x[i];
        double bv = b * (double)v[i];
        double* row = S + (size_t)i * dk;
        for (int j = 0; j < dk; ++j) {
            double kj = (double)k[j];
            row[j] = a * (row[j] - bx * kj) + bv * kj;
        }
    }
}

/* out[i] = sum_j S[i][j] * q[j] */
static void read_state(const double* S, int dk, int dv, const float* q, double* out) {
    for (int i = 0; i < dv; ++i) {
        double s = 0.0;
        for (int j = 0; j < dk; ++j) s += S[(size_t)i * dk + j] * (double)q[j];
        out[i] = s;
    }
}

/* parent of node n in sequence b; a NULL parent array means a chain. */
static int parent_of(const int32_t* parent, int T, int b, int n) {
    return parent ? parent[(size_t)b * T + n] : n - 1;
}

static int parents_valid(const int32_t* parent, int T, int b) {
    if (!parent) return 1;
    for (int n = 0; n < T; ++n) {
        int p = parent[(size_t)b * T + n];
        if (p < -1 || p >= n) return 0;
    }
    return 1;
}

/* Root-to-n path into path[0..len-1]; returns len (node count, root first). */
static int root_path(const int32_t* parent, int T, int b, int n, int* path) {
    int len = 0;
    for (int m = n; m >= 0; m = parent_of(parent, T, b, m)) path[len++] = m;
    for (int i = 0; i < len / 2; ++i) {
        int t = path[i];
        path[i] = path[len - 1 - i];
        path[len - 1 - i] = t;
    }
    return len;
}

typedef struct {
    int B, T, H, dk, dv;
    const float *q, *k, *v, *a, *beta, *S0;
    const int32_t* parent;
    const int32_t* accepted;
    double* o;
    double* u;
    double* states;
    double* S_out;
    const unsigned char* seq_ok;
} walk_ctx;

/* Offsets of the [B, T, H, d] node tensors and [B, T, H] gates. */
#define NODE_VEC(base, c, b, n, h, d) ((base) + ((((size_t)(b) * (c)->T + (n)) * (c)->H + (h)) * (size_t)(d)))
#define NODE_GATE(base, c, b, n, h) ((base)[(((size_t)(b) * (c)->T + (n)) * (c)->H + (h))])

/* Rebuild S at node n of (b, h) from S0 along the root-to-n path; u_n (the
 * correction of the last token) goes to u when u is not NULL. */
static void walk_to(const walk_ctx* c, int b, int h, int n, double* S, double* x, int* path, double* u) {
    const size_t dd = (size_t)c->dk * c->dv;
    const float* s0 = c->S0 + ((size_t)b * c->H + h) * dd;
    for (size_t e = 0; e < dd; ++e) S[e] = (double)s0[e];
    if (n < 0) return;
    int len = root_path(c->parent, c->T, b, n, path);
    for (int i = 0; i < len; ++i) {
        int m = path[i];
        gdr_token(S, c->dk, c->dv, NODE_VEC(c->k, c, b, m, h, c->dk), NODE_VEC(c->v, c, b, m, h, c->dv),
                  (double)NODE_GATE(c->a, c, b, m, h), (double)NODE_GATE(c->beta, c, b, m, h), x,
                  i == len - 1 ? u : NULL);
    }
}

static void verify_item(void* vctx, long item, double* work) {
    const walk_ctx* c = (const walk_ctx*)vctx;
    int b = (int)(item / c->H), h = (int)(item % c->H);
    if (!c->seq_ok[b]) return;
    const size_t dd = (size_t)c->dk * c->dv;
    double* S = work;
    double* x = S + dd;
    int* path = (int*)(x + c->dv);
    for (int n = 0; n < c->T; ++n) {
        walk_to(c, b, h, n, S, x, path, c->u ? NODE_VEC(c->u, c, b, n, h, c->dv) : NULL);
        read_state(S, c->dk, c->dv, NODE_VEC(c->q, c, b, n, h, c->dk), NODE_VEC(c->o, c, b, n, h, c->dv));
        if (c->states) memcpy(c->states + ((((size_t)b * c->T + n) * c->H + h) * dd), S, dd * sizeof(double));
    }
}

static long walk_work(int T, int dk, int dv) {
    /* S, x, then T ints of path (stored in doubles) */
    return (long)dk * dv + dv + T + 1;
}

/*
 * Verify every draft node: o[b, n, h, :] = S_n q_n for all nodes.
 *   q, k: [B, T, H, dk]; v: [B, T, H, dv]; a, beta: [B, T, H]; S0: [B, H, dv, dk]
 *   parent: [B, T] (parent[n] in [-1, n-1]) or NULL for a chain (parent[n] = n-1)
 *   o: [B, T, H, dv] fp64; u: [B, T, H, dv] fp64 or NULL, the node corrections
 *   u_n = beta_n (v_n - a_n S_p(n) k_n); states: [B, T, H, dv, dk] fp64 or NULL
 * Returns status bits (OR_BAD_PARENT).
 */
int oracle_verify(int B, int T, int H, int dk, int dv, const float* q, const float* k, const float* v,
                  const float* a, const float* beta, const float* S0, const int32_t* parent, double* o,
                  double* u, double* states, int nthreads) {
    if (B <= 0 || T <= 0 || H <= 0) return 0;
    unsigned char* ok = (unsigned char*)malloc((size_t)B);
    int status = 0;
    for (int b = 0; b < B; ++b) {
        ok[b] = (unsigned char)parents_valid(parent, T, b);
        if (!ok[b]) status |= OR_BAD_PARENT;
    }
    walk_ctx c = {B, T, H, dk, dv, q, k, v, a, beta, S0, parent, NULL, o, u, states, NULL, ok};
    run_items(verify_item, &c, (long)B * H, walk_work(T, dk, dv), nthreads);
    free(ok);
    return status;
}

/*
 * Log decay of every node: logp[b, n, h] = log P_n, where P_n is the product
 * of the decay gates a_m over the root-to-n path (m = n included), multiplied
 * in fp64 node by node along the walk (a zero gate gives -inf).  This is the
 * gate product that multiplies S0 in the unrolled recurrence (with b = 0 the
 * walk gives S_n = P_n S0), the factor P of the Bole page's Eq. (2) / Eq. (9).
 * The running product is kept as m * 2^e with m in [1/2, 1) (frexp after
 * every factor), so that long paths, whose product is far below the fp64
 * range, keep full precision: log P = log m + e log 2.
 *   a: [B, T, H]; parent: [B, T] or NULL (chain); logp: [B, T, H] fp64
 * Returns status bits (OR_BAD_PARENT; the rows of such a sequence are left
 * untouched).
 */
int oracle_log_decay(int B, int T, int H, const float* a, const int32_t* parent, double* logp) {
    if (B <= 0 || T <= 0 || H <= 0) return 0;
    int status = 0;
    int* path = (int*)malloc(sizeof(int) * (size_t)T);
    for (int b = 0; b < B; ++b) {
        if (!parents_valid(parent, T, b)) {
            status |= OR_BAD_PARENT;
            continue;
        }
        for (int n = 0; n < T; ++n) {
            int len = root_path(parent, T, b, n, path);
            for (int h = 0; h < H; ++h) {
                double P = 1.0;
                long e2 = 0;
                for (int i = 0; i < len; ++i) {
                    int e;
                    P = frexp(P * (double)a[((size_t)b * T + path[i]) * H + h], &e);
                    e2 += e;
                }
                logp[((size_t)b * T + n) * H + h] = log(P) + (double)e2 * log(2.0);
            }
        }
    }
    free(path);
    return status;
}

static void commit_item(void* vctx, long item, double* work) {
    const walk_ctx* c = (const walk_ctx*)vctx;
    int b = (int)(item / c->H), h = (int)(item % c->H);
    if (!c->seq_ok[b]) return;
    const size_t dd = (size_t)c->dk * c->dv;
    double* S = work;
    double* x = S + dd;
    int* path = (int*)(x + c->dv);
    walk_to(c, b, h, c->accepted[b], S, x, path, NULL);
    memcpy(c->S_out + ((size_t)b * c->H + h) * dd, S, dd * sizeof(double));
}

/*
 * Committed state at the accepted node: S_out[b, h] = S_{accepted[b]} of the
 * walk, or S0[b, h] when accepted[b] = -1.  S_out: [B, H, dv, dk] fp64.
 * Returns status bits (OR_BAD_PARENT when a node is accepted and the
 * sequence's parent row is invalid, OR_BAD_ACCEPTED).
 */
int oracle_commit(int B, int T, int H, int dk, int dv, const float* k, const float* v, const float* a,
                  const float* beta, const float* S0, const int32_t* parent, const int32_t* accepted,
                  double* S_out, int nthreads) {
    if (B <= 0 || H <= 0) return 0;
    unsigned char* ok = (unsigned char*)malloc((size_t)B);
    int status = 0;
    for (int b = 0; b < B; ++b) {
        int n = accepted[b];
        int good_acc = (n >= -1 && n < T);
        /* the parent row is only needed (and only checked) when a node is accepted */
        int good_par = (!good_acc || n < 0) ? 1 : parents_valid(parent, T, b);
        if (!good_acc) status |= OR_BAD_ACCEPTED;
        if (!good_par) status |= OR_BAD_PARENT;
        ok[b] = (unsigned char)(good_acc && good_par);
    }
    walk_ctx c = {B, T, H, dk, dv, NULL, k, v, a, beta, S0, parent, accepted, NULL, NULL, NULL, S_out, ok};
    run_items(commit_item, &c, (long)B * H, walk_work(T > 0 ? T : 1, dk, dv), nthreads);
    free(ok);
    return status;
}

/* ------------------------------------------- independent cross-checks */

typedef struct {
    int B, T, H, dk, dv;
    const float *q, *k, *v, *a, *beta, *S0;
    const int32_t* parent;
    double* o;
} seq_ctx;

/* Sequential chain decode: one running state, updated token by token,
 * read after every token.  The ordinary autoregressive recurrence. */
static void chain_item(void* vctx, long item, double* work) {
    const seq_ctx* c = (const seq_ctx*)vctx;
    int b = (int)(item / c->H), h = (int)(item % c->H);
    const size_t dd = (size_t)c->dk * c->dv;
    double* S = work;
    double* x = S + dd;
    const float* s0 = c->S0 + ((size_t)b * c->H + h) * dd;
    for (size_t e = 0; e < dd; ++e) S[e] = (double)s0[e];
    for (int n = 0; n < c->T; ++n) {
        size_t nv = (((size_t)b * c->T + n) * c->H + h);
        gdr_token(S, c->dk, c->dv, c->k + nv * c->dk, c->v + nv * c->dv, (double)c->a[nv], (double)c->beta[nv], x,
                  NULL);
        read_state(S, c->dk, c->dv, c->q + nv * c->dk, c->o + nv * c->dv);
    }
}

int oracle_chain_decode(int B, int T, int H, int dk, int dv, const float* q, const float* k, const float* v,
                        const float* a, const float* beta, const float* S0, double* o, int nthreads) {
    if (B <= 0 || T <= 0 || H <= 0) return 0;
    seq_ctx c = {B, T, H, dk, dv, q, k, v, a, beta, S0, NULL, o};
    run_items(chain_item, &c, (long)B * H, (long)dk * dv + dv, nthreads);
    return 0;
}

/* Branch-by-branch traversal (what tree speculation does without a closed
 * form): depth-first over the tree, each child's state computed once from its
 * parent's, with a stack of states along the current branch. */
static void dfs_item(void* vctx, long item, double* work) {
    const seq_ctx* c = (const seq_ctx*)vctx;
    int b = (int)(item / c->H), h = (int)(item % c->H);
    const int T = c->T;
    const size_t dd = (size_t)c->dk * c->dv;
    /* work: (T + 1) states, x, then int scratch: child lists and resume points */
    double* stack = work;
    double* x = stack + (size_t)(T + 1) * dd;
    int* first_child = (int*)(x + c->dv);
    int* next_sib = first_child + T + 1;
    int* resume = next_sib + T + 1;
    const int32_t* par = c->parent + (size_t)b * T;
    /* child lists in increasing node order; virtual root T holds the roots */
    for (int n = 0; n <= T; ++n) first_child[n] = -1;
    for (int n = T - 1; n >= 0; --n) {
        int p = par[n] < 0 ? T : par[n];
        next_sib[n] = first_child[p];
        first_child[p] = n;
    }
    const float* s0 = c->S0 + ((size_t)b * c->H + h) * dd;
    for (size_t e = 0; e < dd; ++e) stack[e] = (double)s0[e];
    int top = 0;
    int cursor = first_child[T];
    /* iterative DFS: descend into cursor, or climb when no child is left */
    for (;;) {
        if (cursor >= 0) {
            int n = cursor;
            resume[top] = next_sib[n];
            memcpy(stack + (size_t)(top + 1) * dd, stack + (size_t)top * dd, dd * sizeof(double));
            ++top;
            size_t nv = (((size_t)b * T + n) * c->H + h);
            double* S = stack + (size_t)top * dd;
            gdr_token(S, c->dk, c->dv, c->k + nv * c->dk, c->v + nv * c->dv, (double)c->a[nv], (double)c->beta[nv], x,
                      NULL);
            read_state(S, c->dk, c->dv, c->q + nv * c->dk, c->o + nv * c->dv);
            cursor = first_child[n];
        } else {
            if (top == 0) break;
            --top;
            cursor = resume[top];
        }
    }
}

int oracle_verify_dfs(int B, int T, int H, int dk, int dv, const float* q, const float* k, const float* v,
                      const float* a, const float* beta, const float* S0, const int32_t* parent, double* o,
                      int nthreads) {
    if (B <= 0 || T <= 0 || H <= 0) return 0;
    for (int b = 0; b < B; ++b)
        if (!parents_valid(parent, T, b)) return OR_BAD_PARENT;
    seq_ctx c = {B, T, H, dk, dv, q, k, v, a, beta, S0, parent, o};
    long work = (long)(T + 1) * dk * dv + dv + 3L * (T + 1);
    run_items(dfs_item, &c, (long)B * H, work, nthreads);
    return 0;
}

/* ------------------------------------------------------------- gather */

typedef struct {
    int B, P, H, dk, dv, num_slots, Qn;
    const float* pool;
    const int32_t* slot;
    const float* queries;
    double* o;
    float* states_out;
} gather_ctx;

static void gather_item(void* vctx, long item, double* work) {
    const gather_ctx* c = (const gather_ctx*)vctx;
    (void)work;
    int h = (int)(item % c->H);
    long bp = item / c->H; /* b * P + p */
    int s = c->slot[bp];
    if (s < 0 || s >= c->num_slots) return;
    const size_t dd = (size_t)c->dk * c->dv;
    const float* src = c->pool + ((size_t)s * c->H + h) * dd;
    if (c->states_out) memcpy(c->states_out + ((size_t)bp * c->H + h) * dd, src, dd * sizeof(float));
    if (c->o && c->queries) {
        for (int i = 0; i < c->Qn; ++i) {
            const float* qv = c->queries + (((size_t)bp * c->H + h) * c->Qn + i) * c->dk;
            double* out = c->o + (((size_t)bp * c->H + h) * c->Qn + i) * c->dv;
            for (int r = 0; r < c->dv; ++r) {
                double acc = 0.0;
                for (int j = 0; j < c->dk; ++j) acc += (double)src[(size_t)r * c->dk + j] * (double)qv[j];
                out[r] = acc;
            }
        }
    }
}

/*
 * State reads at chosen positions.
 *   pool: [num_slots, H, dv, dk]; slot: [B, P]; queries: [B, P, H, Qn, dk] or NULL
 *   o: [B, P, H, Qn, dv] fp64 or NULL; states_out: [B, P, H, dv, dk] fp32 (exact copy) or NULL
 * Returns status bits (OR_BAD_SLOT).
 */
int oracle_gather(int B, int P, int H, int dk, int dv, int num_slots, int Qn, const float* pool,
                  const int32_t* slot, const float* queries, double* o, float* states_out, int nthreads) {
    if (B <= 0 || P <= 0 || H <= 0) return 0;
    int status = 0;
    for (long i = 0; i < (long)B * P; ++i)
        if (slot[i] < 0 || slot[i] >= num_slots) status |= OR_BAD_SLOT;
    gather_ctx c = {B, P, H, dk, dv, num_slots, Qn, pool, slot, queries, o, states_out};
    run_items(gather_item, &c, (long)B * P * H, 1, nthreads);
    return status;
}

/* ------------------------------------------------ reads inside the block */

typedef struct {
    walk_ctx w;
    int P, Qn;
    const int32_t* pos;
    const float* queries;
    double* o;
} read_ctx;

static void read_item(void* vctx, long item, double* work) {
    const read_ctx* c = (const read_ctx*)vctx;
    const walk_ctx* w = &c->w;
    int h = (int)(item % w->H);
    long bp = item / w->H; /* b * P + p */
    int b = (int)(bp / c->P);
    int n = c->pos[bp];
    if (n < -1 || n >= w->T || !w->seq_ok[b]) return;
    const size_t dd = (size_t)w->dk * w->dv;
    double* S = work;
    double* x = S + dd;
    int* path = (int*)(x + w->dv);
    walk_to(w, b, h, n, S, x, path, NULL);
    for (int i = 0; i < c->Qn; ++i)
        read_state(S, w->dk, w->dv, c->queries + (((size_t)bp * w->H + h) * c->Qn + i) * w->dk,
                   c->o + (((size_t)bp * w->H + h) * c->Qn + i) * w->dv);
}

/*
 * Reads of states inside the verified block, without a commit:
 *   o[b, p, h, i, :] = S_j q_{b,p,h,i},   j = pos[b, p] in [-1, T-1],
 * S_j the walk's state at node j (S0 for j = -1).
 *   k, v, a, beta, S0, parent: as for oracle_verify; pos: [B, P];
 *   queries: [B, P, H, Qn, dk]; o: [B, P, H, Qn, dv] fp64.
 * A position outside [-1, T-1] sets OR_BAD_POSITION and is skipped.  The
 * parent row is needed (and checked) only when a valid position of the
 * sequence is a node (>= 0); when it is invalid, OR_BAD_PARENT is set and
 * nothing of that sequence is written.
 */
int oracle_read_states(int B, int T, int H, int dk, int dv, int P, int Qn, const float* k, const float* v,
                       const float* a, const float* beta, const float* S0, const int32_t* parent,
                       const int32_t* pos, const float* queries, double* o, int nthreads) {
    if (B <= 0 || P <= 0 || H <= 0 || Qn <= 0) return 0;
    unsigned char* ok = (unsigned char*)malloc((size_t)B);
    int status = 0;
    for (int b = 0; b < B; ++b) {
        int needs_parent = 0;
        for (int p = 0; p < P; ++p) {
            int n = pos[(size_t)b * P + p];
            if (n < -1 || n >= T) status |= OR_BAD_POSITION;
            else if (n >= 0) needs_parent = 1;
        }
        ok[b] = (unsigned char)(!needs_parent || parents_valid(parent, T, b));
        if (!ok[b]) status |= OR_BAD_PARENT;
    }
    read_ctx c = {{B, T, H, dk, dv, NULL, k, v, a, beta, S0, parent, NULL, NULL, NULL, NULL, NULL, ok},
                  P, Qn, pos, queries, o};
    run_items(read_item, &c, (long)B * P * H, walk_work(T > 0 ? T : 1, dk, dv), nthreads);
    free(ok);
    return status;
}

/* ------------------------------------------- accepted-node selection */

/* Index of the largest value of x[0..V-1]; equal values go to the lowest
 * index, NaN never wins (+0 and -0 are equal), and a row of NaN gives 0. */
static int row_argmax(const float* x, long V) {
    long best = -1;
    float bv = 0.f;
    for (long i = 0; i < V; ++i) {
        float t = x[i];
        if (t != t) continue;
        if (best < 0 || t > bv) {
            best = i;
            bv = t;
        }
    }
    return best < 0 ? 0 : (int)best;
}

typedef struct {
    long V;
    const float* logits;
    int32_t* target;
} argmax_ctx;

static void argmax_item(void* vctx, long item, double* work) {
    const argmax_ctx* c = (const argmax_ctx*)vctx;
    (void)work;
    c->target[item] = row_argmax(c->logits + (size_t)item * c->V, c->V);
}

/*
 * Greedy selection of the accepted node.
 *   logits: [B, T+1, V]; row 0 is the target's prediction at the committed
 *     position, row n+1 its prediction after draft node n.
 *   tokens: [B, T] the draft token of each node; parent: [B, T] or NULL (chain).
 * Outputs: target[B, T+1] = argmax of each row (row_argmax rules);
 *   accepted[b]: start at cur = -1 (the committed state); while some child c
 *   of cur (parent[c] == cur) has tokens[c] == target[cur + 1], move to the
 *   lowest-index such child; accepted[b] = the final cur (-1 if none).
 *   acc_len[b] = number of nodes moved through (the accepted node's depth);
 *   bonus[b] = target[b, accepted[b] + 1], the target's token after it.
 *   acc_len and bonus may be NULL.
 * An invalid parent row sets OR_BAD_PARENT and leaves accepted, acc_len and
 * bonus of that sequence untouched (target is still written).
 */
int oracle_select(int B, int T, long V, const float* logits, const int32_t* tokens, const int32_t* parent,
                  int32_t* target, int32_t* accepted, int32_t* acc_len, int32_t* bonus, int nthreads) {
    if (B <= 0 || T < 0 || V <= 0) return 0;
    argmax_ctx ac = {V, logits, target};
    run_items(argmax_item, &ac, (long)B * (T + 1), 1, nthreads);
    int status = 0;
    for (int b = 0; b < B; ++b) {
        if (!parents_valid(parent, T, b)) {
            status |= OR_BAD_PARENT;
            continue;
        }
        const int32_t* tg = target + (size_t)b * (T + 1);
        int cur = -1, len = 0;
        for (;;) {
            int want = tg[cur + 1], next = -1;
            for (int c = cur + 1; c < T; ++c)
                if (parent_of(parent, T, b, c) == cur && tokens[(size_t)b * T + c] == want) {
                    next = c;
                    break;
                }
            if (next < 0) break;
            cur = next;
            ++len;
        }
        accepted[b] = cur;
        if (acc_len) acc_len[b] = len;
        if (bonus) bonus[b] = tg[cur + 1];
    }
    return status;
}
