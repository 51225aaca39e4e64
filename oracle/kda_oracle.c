/*
 * KDA oracle: plain, slow, obviously correct fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (the per-token Kimi Delta Attention recurrence), from
 *   [P4] "Kimi K3 发布核实与 Moonshot AI 主干架构演变" (dllmharness.com),
 *        section 3 "Kimi Linear：K3 注意力的架构先导", paragraph
 *        "KDA 为什么不同于 MLA": each head keeps a state matrix S_t; a new
 *        token first decays the old state channel by channel with the
 *        retention alpha_t, then corrects it with the write strength beta_t,
 *        the key and the value; the query is read from the updated state.
 *   [P2] "Kimi K3 模型架构解析：KDA、AttnRes 与 Stable LatentMoE"
 *        (blog.baizx.cool), section 二.3 "Delta Rule：写入新记忆前修正旧映射":
 *        the delta rule reads the mapping already stored under the key,
 *        forms the error against the value and writes back only that
 *        difference; section 二.2 gives S_t = Update(S_{t-1}, k_t, v_t),
 *        o_t = Read(S_t, q_t).
 *
 * Per sequence n and head h, with S in R^{K x V} (rows = key channels):
 *   S   <- diag(exp(g_t)) S              decay (g_t is the log-retention)
 *   u   <- S^T k_t                       read the old value (after decay)
 *   S   <- S + beta_t k_t (v_t - u)^T    write the correction
 *   o_t <- S^T q_t                       read the updated state
 * Readings where the pages are silent: alpha = e^g (natural log); no q
 * scaling and no normalisation inside; the read of step 2 uses the decayed
 * state (pinned by the read-after-write identity in the tests).
 *
 * Layouts (row-major, contiguous):
 *   q, k, g : [B, T, H, K]     v, o : [B, T, H, V]     beta : [B, T, H]
 *   S0, S_final : [num_seqs, H, K, V]
 * With cu_seqlens (int64[num_seqs+1]) the batch is packed: B = 1 and
 * sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1. Without it,
 * num_seqs = B and sequence n is batch row n.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *S0;
    const int64_t *cu;
    int64_t B, T, H, K, V, num_seqs;
    double *o, *S_final;
    int64_t next_item; /* shared work counter */
    int only_last;     /* decode: single token per sequence, S updated in place */
} job_t;

/* One (sequence, head): the recurrence above, token by token. */
static void run_item(const job_t *J, int64_t item, double *S, double *u, double *y)
{
    const int64_t H = J->H, K = J->K, V = J->V;
    const int64_t n = item / H, h = item % H;
    int64_t t0, t1; /* flat token range: row index into [B*T] */
    if (J->cu) {
        t0 = J->cu[n];
        t1 = J->cu[n + 1];
    } else {
        t0 = n * J->T;
        t1 = t0 + J->T;
    }
    const size_t state_off = (size_t)(n * H + h) * (size_t)(K * V);
    if (J->S0)
        memcpy(S, J->S0 + state_off, sizeof(double) * (size_t)(K * V));
    else
        memset(S, 0, sizeof(double) * (size_t)(K * V));

    for (int64_t t = t0; t < t1; ++t) {
        const double *qt = J->q + (size_t)(t * H + h) * K;
        const double *kt = J->k + (size_t)(t * H + h) * K;
        const double *gt = J->g + (size_t)(t * H + h) * K;
        const double *vt = J->v + (size_t)(t * H + h) * V;
        const double bt = J->beta[t * H + h];
        double *ot = J->o + (size_t)(t * H + h) * V;

        /* 1. decay every key-channel row of S by alpha = exp(g) */
        for (int64_t a = 0; a < K; ++a) {
            const double alpha = exp(gt[a]);
            for (int64_t b = 0; b < V; ++b) S[a * V + b] *= alpha;
        }
        /* 2. u = S^T k : the value the decayed state returns for this key */
        for (int64_t b = 0; b < V; ++b) u[b] = 0.0;
        for (int64_t a = 0; a < K; ++a)
            for (int64_t b = 0; b < V; ++b) u[b] += S[a * V + b] * kt[a];
        /* 3. S += beta k (v - u)^T : write back only the error */
        for (int64_t a = 0; a < K; ++a)
            for (int64_t b = 0; b < V; ++b) S[a * V + b] += bt * kt[a] * (vt[b] - u[b]);
        /* 4. o = S^T q : read the updated state */
        for (int64_t b = 0; b < V; ++b) y[b] = 0.0;
        for (int64_t a = 0; a < K; ++a)
            for (int64_t b = 0; b < V; ++b) y[b] += S[a * V + b] * qt[a];
        for (int64_t b = 0; b < V; ++b) ot[b] = y[b];
    }
    if (J->S_final) memcpy(J->S_final + state_off, S, sizeof(double) * (size_t)(K * V));
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t K = J->K, V = J->V;
    double *S = (double *)malloc(sizeof(double) * (size_t)(K * V));
    double *u = (double *)malloc(sizeof(double) * (size_t)V);
    double *y = (double *)malloc(sizeof(double) * (size_t)V);
    const int64_t n_items = J->num_seqs * J->H;
    for (;;) {
        const int64_t item = __atomic_fetch_add(&J->next_item, 1, __ATOMIC_RELAXED);
        if (item >= n_items) break;
        run_item(J, item, S, u, y);
    }
    free(S);
    free(u);
    free(y);
    return NULL;
}

static int run_job(job_t *J, int nthreads)
{
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    const int64_t n_items = J->num_seqs * J->H;
    if (nthreads > n_items) nthreads = (int)(n_items > 0 ? n_items : 1);
    J->next_item = 0;
    if (nthreads == 1) {
        worker(J);
        return 0;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, J) != 0) break;
        ++started;
    }
    if (started == 0) worker(J); /* could not spawn: do the work here */
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    return 0;
}

/* Prefill over whole sequences. Returns 0 on success, -1 on bad arguments. */
int kda_oracle_chunk_fwd(const double *q, const double *k, const double *v, const double *g,
                         const double *beta, const double *S0, const int64_t *cu_seqlens,
                         int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, int64_t num_seqs,
                         double *o, double *S_final, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !o) return -1;
    if (B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0 || num_seqs < 0) return -1;
    if (cu_seqlens) {
        if (B != 1) return -1;
        if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -1;
        for (int64_t n = 0; n < num_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    } else if (num_seqs != B) {
        return -1;
    }
    job_t J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.S0 = S0; J.cu = cu_seqlens;
    J.B = B; J.T = T; J.H = H; J.K = K; J.V = V; J.num_seqs = num_seqs;
    J.o = o; J.S_final = S_final;
    return run_job(&J, nthreads);
}

/*
 * One decode step for N independent sequences: the same four steps for a
 * single token, with the state S [N, H, K, V] updated in place and o [N, H, V]
 * written. Inputs q, k, g are [N, H, K], v is [N, H, V], beta is [N, H].
 */
int kda_oracle_decode(const double *q, const double *k, const double *v, const double *g,
                      const double *beta, double *S, double *o, int64_t N, int64_t H, int64_t K,
                      int64_t V, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !S || !o) return -1;
    if (N < 0 || H <= 0 || K <= 0 || V <= 0) return -1;
    /* a decode step is a length-1 prefill of each sequence from S, back into S */
    job_t J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.S0 = S; J.cu = NULL;
    J.B = N; J.T = 1; J.H = H; J.K = K; J.V = V; J.num_seqs = N;
    J.o = o; J.S_final = S; /* each item reads then overwrites only its own state */
    return run_job(&J, nthreads);
}
