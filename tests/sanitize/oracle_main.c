/*
 * Host sanitizer driver for the C oracle (test infrastructure): runs
 * kda_oracle_chunk_fwd and kda_oracle_decode on small batched and packed cases
 * (empty and one-token sequences, several threads, absent S0), checks two
 * exact properties and the argument checks, and exits non-zero on a mismatch.
 * Built with gcc -fsanitize=address,undefined by tests/test_sanitizers_cpu.py,
 * so an out-of-bounds access, a use of freed memory or undefined arithmetic in
 * the oracle ends the run with a sanitizer report.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_chunk_fwd(const double *q, const double *k, const double *v, const double *g,
                         const double *beta, const double *S0, const int64_t *cu_seqlens,
                         int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, int64_t num_seqs,
                         double *o, double *S_final, int nthreads);
int kda_oracle_decode(const double *q, const double *k, const double *v, const double *g,
                      const double *beta, double *S, double *o, int64_t N, int64_t H, int64_t K,
                      int64_t V, int nthreads);

static uint64_t rng_state = 88172645463325252ull;
static double uniform(void) { /* xorshift64, mapped to (-1, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
/* exact-size heap buffers, so that any access past an end is caught */
static double *fill(size_t n, double lo, double hi) {
    double *p = (double *)malloc(n ? n * sizeof(double) : 1);
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (uniform() + 1.0);
    return p;
}

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

static void run_prefill(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, const int64_t *cu, int64_t N,
                        int with_S0, int threads, int passthrough) {
    const size_t nt = (size_t)(B * T);
    double *q = fill(nt * H * K, -1, 1), *k = fill(nt * H * K, -1, 1), *v = fill(nt * H * V, -1, 1);
    double *g = fill(nt * H * K, passthrough ? 0 : -5, 0), *beta = fill(nt * H, passthrough ? 0 : 0, passthrough ? 0 : 1);
    double *S0 = with_S0 ? fill((size_t)N * H * K * V, -0.1, 0.1) : NULL;
    double *o = fill(nt * H * V, 0, 0), *Sf = fill((size_t)N * H * K * V, 0, 0);
    CHECK(kda_oracle_chunk_fwd(q, k, v, g, beta, S0, cu, B, T, H, K, V, N, o, Sf, threads) == 0);
    if (passthrough) /* beta = 0, g = 0: the state passes through bit for bit */
        for (size_t i = 0; i < (size_t)N * H * K * V; ++i) CHECK(Sf[i] == (S0 ? S0[i] : 0.0));
    free(q); free(k); free(v); free(g); free(beta); free(S0); free(o); free(Sf);
}

int main(void) {
    run_prefill(2, 37, 3, 8, 4, NULL, 2, 1, 3, 0);
    run_prefill(1, 50, 2, 4, 8, NULL, 1, 0, 1, 0);
    const int64_t cu[] = {0, 7, 7, 8, 40, 40, 41};
    run_prefill(1, 41, 2, 4, 4, cu, 6, 1, 4, 0);
    run_prefill(1, 41, 2, 4, 4, cu, 6, 1, 2, 1);
    run_prefill(3, 0, 2, 4, 4, NULL, 3, 1, 2, 1); /* no tokens: S_final = S0 */
    /* decode: one step equals a one-token prefill from the same state */
    {
        const int64_t N = 3, H = 2, K = 4, V = 8;
        double *q = fill(N * H * K, -1, 1), *k = fill(N * H * K, -1, 1), *v = fill(N * H * V, -1, 1);
        double *g = fill(N * H * K, -5, 0), *beta = fill(N * H, 0, 1), *S = fill(N * H * K * V, -0.1, 0.1);
        double *S_copy = fill(N * H * K * V, 0, 0), *o = fill(N * H * V, 0, 0), *o2 = fill(N * H * V, 0, 0);
        double *Sf = fill(N * H * K * V, 0, 0);
        memcpy(S_copy, S, sizeof(double) * N * H * K * V);
        CHECK(kda_oracle_decode(q, k, v, g, beta, S, o, N, H, K, V, 2) == 0);
        CHECK(kda_oracle_chunk_fwd(q, k, v, g, beta, S_copy, NULL, N, 1, H, K, V, N, o2, Sf, 1) == 0);
        CHECK(memcmp(S, Sf, sizeof(double) * N * H * K * V) == 0 && memcmp(o, o2, sizeof(double) * N * H * V) == 0);
        free(q); free(k); free(v); free(g); free(beta); free(S); free(S_copy); free(o); free(o2); free(Sf);
    }
    /* argument checks */
    {
        double x[64] = {0}, y[64] = {0};
        const int64_t bad_cu[] = {0, 5, 3};
        CHECK(kda_oracle_chunk_fwd(NULL, x, x, x, x, NULL, NULL, 1, 1, 1, 1, 1, 1, y, y, 1) == -1);
        CHECK(kda_oracle_chunk_fwd(x, x, x, x, x, NULL, bad_cu, 1, 3, 1, 1, 1, 2, y, y, 1) == -1);
        CHECK(kda_oracle_chunk_fwd(x, x, x, x, x, NULL, NULL, 2, 1, 1, 1, 1, 3, y, y, 1) == -1);
        CHECK(kda_oracle_decode(x, x, x, x, x, NULL, y, 1, 1, 1, 1, 1) == -1);
    }
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle sanitizer driver: all checks passed\n");
    return 0;
}
