/*
 * Runs every entry point of the CPU oracle (oracle/dspark_oracle.c) on small
 * inputs that reach its edge cases, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: any out-of-bounds access, use of freed memory
 * or undefined operation aborts the run. The values are checked only for
 * what holds in any case (tokens in range, proposals summing to 1); the
 * oracle's correctness is pinned by the Python tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void dspark_oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t dspark_oracle_noise_word(uint64_t seed, uint64_t offset, uint32_t k, uint32_t v);
double dspark_oracle_uniform(uint32_t x);
float dspark_oracle_gumbel(uint32_t x);
void dspark_oracle_uniform_batch(const uint32_t* x, double* u, int64_t n);
void dspark_oracle_gumbel_batch(const uint32_t* x, float* g, int64_t n);
int dspark_oracle_draft_block(const void* base, int base_is_bf16, const uint16_t* E, const uint16_t* W,
                              const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
                              const float* temperature, int n_real, int B, int K, int V, int r,
                              const int32_t* forced, double tie_eps, int max_cand, int32_t* tokens,
                              int32_t* own_tokens, float* logits, double* q, double* margin, int32_t* ncand,
                              int32_t* cand, int num_threads);
float dspark_oracle_verify_uniform(uint64_t seed, uint64_t offset, uint32_t k);
float dspark_oracle_verify_gumbel(uint64_t seed, uint64_t offset, uint32_t v);
int dspark_oracle_verify_standard(const float* q, const float* p, const int32_t* draft, const int64_t* seed,
                                  const int64_t* offset, int B, int K, int V, double tie_eps, int max_cand,
                                  int32_t* n_accepted, int32_t* out_tokens, int32_t* emit_pos, double* margin,
                                  int32_t* ncand, int32_t* cand);
int dspark_oracle_verify_block_weights(const float* q, const float* p, const int32_t* draft, int B, int K, int V,
                                       double* w, double* S, double* h, float* resid);
int dspark_oracle_verify_block(const float* q, const float* p, const int32_t* draft, const int64_t* seed,
                               const int64_t* offset, int B, int K, int V, double tie_eps, int max_cand,
                               int32_t* n_accepted, int32_t* out_tokens, double* tau_margin, double* margin,
                               int32_t* ncand, int32_t* cand);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {   /* xorshift64*: test inputs only */
    rng_state ^= rng_state >> 12; rng_state ^= rng_state << 25; rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float unif(void) { return (float)((rnd() >> 8) + 0.5) * (1.0f / 16777216.0f); }
static uint16_t bf16_of(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }
static void* xmalloc(size_t n) { void* p = malloc(n ? n : 1); if (!p) abort(); return p; }

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

/* one draft block; base_kind 0: f32, 1: bf16; nan_pad: padding rows' base is NaN */
static void draft_case(int B, int K, int V, int r, int bf16, int n_real, int nan_pad, int force, float T0) {
    const size_t n = (size_t)B * K * V;
    float* basef = xmalloc(n * sizeof(float));
    uint16_t* baseh = xmalloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) {
        const int b = (int)(i / ((size_t)K * V));
        basef[i] = (nan_pad && n_real >= 0 && b >= n_real) ? NAN : 4.0f * (unif() - 0.5f);
        baseh[i] = bf16_of(basef[i]);
    }
    uint16_t* E = xmalloc((size_t)V * r * 2);
    uint16_t* W = xmalloc((size_t)r * V * 2);
    for (size_t i = 0; i < (size_t)V * r; ++i) E[i] = bf16_of(0.3f * (unif() - 0.5f));
    for (size_t i = 0; i < (size_t)V * r; ++i) W[i] = bf16_of(0.3f * (unif() - 0.5f));
    int32_t* prev = xmalloc(B * 4 + 4);
    int64_t* seed = xmalloc(B * 8 + 8);
    int64_t* off = xmalloc(B * 8 + 8);
    float* T = xmalloc(B * 4 + 4);
    int32_t* forced = xmalloc((size_t)B * K * 4 + 4);
    for (int b = 0; b < B; ++b) {
        prev[b] = (b % 3 == 0) ? -5 : (b % 3 == 1) ? V + 7 : (int32_t)(rnd() % V);   /* clamped */
        seed[b] = (int64_t)(((uint64_t)rnd() << 32) | rnd());
        off[b] = (int64_t)rnd();
        T[b] = (b % 2) ? 0.0f : T0 * (1.0f + 0.1f * b);
    }
    for (int i = 0; i < B * K; ++i) forced[i] = force ? (int32_t)(rnd() % V) : -1;
    const int MC = 4;
    int32_t* tok = xmalloc((size_t)B * K * 4 + 4);
    int32_t* own = xmalloc((size_t)B * K * 4 + 4);
    float* lg = xmalloc(n * sizeof(float));
    double* q = xmalloc(n * sizeof(double));
    double* mg = xmalloc((size_t)B * K * 8 + 8);
    int32_t* nc = xmalloc((size_t)B * K * 4 + 4);
    int32_t* cand = xmalloc((size_t)B * K * MC * 4 + 4);
    const int rc = dspark_oracle_draft_block(bf16 ? (const void*)baseh : (const void*)basef, bf16, E, W, prev, seed,
                                             off, T, n_real, B, K, V, r, force ? forced : NULL, 1e-4, MC, tok, own,
                                             lg, q, mg, nc, cand, 1);
    CHECK(rc == 0);
    for (int i = 0; i < B * K; ++i) CHECK(tok[i] >= 0 && tok[i] < V && own[i] >= 0 && own[i] < V);
    for (int i = 0; i < B * K; ++i) {
        double s = 0.0;
        for (int v = 0; v < V; ++v) s += q[(size_t)i * V + v];
        CHECK(fabs(s - 1.0) < 1e-9);   /* every row, padding rows included */
    }
    /* outputs may be omitted */
    CHECK(dspark_oracle_draft_block(bf16 ? (const void*)baseh : (const void*)basef, bf16, E, W, prev, seed, off, T,
                                    n_real, B, K, V, r, NULL, 1e-4, MC, tok, own, NULL, NULL, mg, nc, cand, 1) == 0);
    free(basef); free(baseh); free(E); free(W); free(prev); free(seed); free(off); free(T); free(forced);
    free(tok); free(own); free(lg); free(q); free(mg); free(nc); free(cand);
}

static void verify_case(int B, int K, int V, int pq_equal) {
    const size_t nq = (size_t)B * K * V, np = (size_t)B * (K + 1) * V;
    float* q = xmalloc(nq * 4 + 4);
    float* p = xmalloc(np * 4);
    for (int b = 0; b < B; ++b)
        for (int j = 0; j <= K; ++j) {
            double sp = 0.0, sq = 0.0;
            float* pr = p + ((size_t)b * (K + 1) + j) * V;
            float* qr = j < K ? q + ((size_t)b * K + j) * V : NULL;
            for (int v = 0; v < V; ++v) {
                pr[v] = (v % 5 == 0) ? 0.0f : unif();
                sp += pr[v];
                if (qr) { qr[v] = pq_equal ? pr[v] : ((v % 7 == 0) ? 0.0f : unif()); sq += qr[v]; }
            }
            for (int v = 0; v < V; ++v) {
                pr[v] = (float)(pr[v] / sp);
                if (qr) qr[v] = (float)(qr[v] / sq);
            }
        }
    int32_t* d = xmalloc((size_t)B * K * 4 + 4);
    int64_t* seed = xmalloc(B * 8);
    int64_t* off = xmalloc(B * 8);
    for (int i = 0; i < B * K; ++i) d[i] = (i % 4 == 3) ? -3 : (int32_t)(rnd() % (V + 2));   /* some clamped */
    for (int b = 0; b < B; ++b) { seed[b] = (int64_t)rnd(); off[b] = (int64_t)rnd() << 20; }
    const int MC = 4;
    int32_t* n = xmalloc(B * 4);
    int32_t* out = xmalloc((size_t)B * (K + 1) * 4);
    int32_t* pos = xmalloc(B * 4);
    double* mg = xmalloc(B * 8);
    double* tm = xmalloc(B * 8);
    int32_t* nc = xmalloc(B * 4);
    int32_t* cand = xmalloc((size_t)B * MC * 4);
    CHECK(dspark_oracle_verify_standard(q, p, d, seed, off, B, K, V, 1e-4, MC, n, out, pos, mg, nc, cand) == 0);
    for (int b = 0; b < B; ++b) CHECK(n[b] >= 0 && n[b] <= K && out[(size_t)b * (K + 1) + n[b]] >= 0);
    double* w = xmalloc((size_t)B * (K + 1) * 8);
    double* S = xmalloc((size_t)B * (K + 1) * 8);
    double* h = xmalloc((size_t)B * (K + 1) * 8);
    float* resid = xmalloc(np * 4);
    CHECK(dspark_oracle_verify_block_weights(q, p, d, B, K, V, w, S, h, resid) == 0);
    CHECK(dspark_oracle_verify_block_weights(q, p, d, B, K, V, w, S, h, NULL) == 0);
    CHECK(dspark_oracle_verify_block(q, p, d, seed, off, B, K, V, 1e-4, MC, n, out, tm, mg, nc, cand) == 0);
    for (int b = 0; b < B; ++b) CHECK(n[b] >= 0 && n[b] <= K && out[(size_t)b * (K + 1) + n[b]] >= 0);
    free(q); free(p); free(d); free(seed); free(off); free(n); free(out); free(pos); free(mg); free(tm);
    free(nc); free(cand); free(w); free(S); free(h); free(resid);
}

int main(void) {
    uint32_t c[4] = {1, 2, 3, 4}, k2[2] = {5, 6}, o[4];
    dspark_oracle_philox4x32_10(c, k2, o);
    (void)dspark_oracle_noise_word(~0ull, ~0ull, 254, 0xFFFFFFFFu);
    uint32_t xs[6] = {0, 1, 511, 512, 0xFFFFFE00u, 0xFFFFFFFFu};
    double u[6];
    float g[6];
    dspark_oracle_uniform_batch(xs, u, 6);
    dspark_oracle_gumbel_batch(xs, g, 6);
    for (int i = 0; i < 6; ++i) CHECK(u[i] > 0.0 && u[i] < 1.0 && isfinite(g[i]));
    CHECK(isfinite(dspark_oracle_gumbel(0u)) && dspark_oracle_uniform(0xFFFFFFFFu) < 1.0);
    (void)dspark_oracle_verify_uniform(1, 2, 3);
    (void)dspark_oracle_verify_gumbel(1, 2, 0xFFFFFFFFu);

    draft_case(3, 3, 64, 32, 0, -1, 0, 0, 1.0f);    /* f32 base, greedy and sampling rows, clamped prev */
    draft_case(4, 2, 72, 64, 1, 2, 1, 0, 0.7f);     /* bf16 base, NaN padding rows */
    draft_case(2, 4, 8, 32, 0, 1, 1, 1, 2.5f);      /* tiny vocabulary, forced tokens */
    draft_case(1, 1, 16, 96, 1, 0, 1, 0, 1.0f);     /* every row padding, K = 1 */
    draft_case(5, 0, 16, 32, 0, -1, 0, 0, 1.0f);    /* K = 0 */
    CHECK(dspark_oracle_draft_block(NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, -1, -1, 1, 8, 32, NULL, 1e-4, 4,
                                    NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) != 0);
    verify_case(3, 4, 40, 0);
    verify_case(2, 3, 12, 1);                       /* p = q: empty residuals */
    verify_case(2, 1, 8, 0);
    verify_case(1, 0, 8, 0);                        /* K = 0: the bonus draw only */
    if (fails) { fprintf(stderr, "%d checks failed\n", fails); return 1; }
    printf("oracle driver ok\n");
    return 0;
}
