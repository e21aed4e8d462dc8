/*
 * dspark_oracle.c -- CPU oracle for the DSpark ancestral draft-block sampler.
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow, obviously correct
 * statement of what the sampler computes. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the GPU library
 * never calls it and shares no code with it.
 *
 * Sources (page titles as on the pages):
 *  - "brb-nv/TensorRT-LLM pull 21", section "2. Golden sampling semantics":
 *    the law of a draft block (every position is sampled from the
 *    temperature-scaled softmax of its biased logits, where the bias depends
 *    on the token sampled one position earlier); temperature is the only
 *    transformation applied to draft logits; a greedy request takes the
 *    argmax at every position; what a draft was sampled from is kept as its
 *    proposal distribution.
 *  - "brb-nv/TensorRT-LLM pull 27", section "2. One fused kernel per draft
 *    position": the rank-r Markov bias added to the drafter logits, the
 *    1/T scaling, Gumbel-max sampling with counter-based Philox noise keyed
 *    per request slot (seed, offset) and per position, drafter logits in
 *    float32 or bfloat16 with the biased logits kept in float32, the
 *    proposal written after the block from those same float32 logits with
 *    the scaled values reproduced exactly, and graph-padding rows sampled
 *    from the bias term only.
 *  - Philox4x32-10: Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
 *    As Easy as 1, 2, 3", SC'11, section 3 (the Philox round and key schedule).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *  - bias(d) = E[d] . W with E [V,r] and W [r,V] in bf16; the bias is the
 *    exact sum rounded once to float32 (here: double accumulation of exact
 *    bf16 products, then one rounding).
 *  - logit = float32(base) + float32(bias), one float32 addition. Padding
 *    rows (b >= n_real) use base = 0 and never read their base row.
 *  - Greedy rows are those with !(T > 0): their token is the lowest index of
 *    the largest logit and their proposal is one-hot at that token.
 *  - Sampling rows: invT = float32(1/T); s = float32(logit * invT).
 *    Philox key = (lo32(seed), hi32(seed)); counter = (v >> 2, k,
 *    lo32(offset), hi32(offset)); the noise word is output word (v & 3).
 *    u = ((x >> 9) + 1/2) * 2^-23, which is exact and lies in
 *    [2^-24, 1 - 2^-24]; g = -ln(-ln u), evaluated in double and rounded to
 *    float32; the perturbed score is z = float32(s + g). The draw is the
 *    lowest index of the largest z (the decision is taken in float32, the
 *    precision the GPU kernel uses). A NaN score never wins; a row whose
 *    every score is NaN draws token 0.
 *  - Proposal: M = max s, S = sum exp(s - M), q = exp(s - M) / S, in double.
 *  - prev_token is clamped into [0, V).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math):
 * every float expression above is a single IEEE binary32 operation.
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- Philox4x32-10 (SC'11, section 3) ---------------------------------- */

/* Multipliers and Weyl key increments of Philox4x32 as given in the paper. */
static const uint32_t kPhiloxMul0 = 0xD2511F53u;
static const uint32_t kPhiloxMul1 = 0xCD9E8D57u;
static const uint32_t kPhiloxWeyl0 = 0x9E3779B9u;
static const uint32_t kPhiloxWeyl1 = 0xBB67AE85u;

/* Ten rounds of the Philox4x32 bijection on `ctr` under `key`.
 * One round: the products M0*c0 and M1*c2 are split into high and low
 * words; the new block is (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2),
 * hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)). The key is bumped by the Weyl
 * constants before every round after the first. */
void dspark_oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += kPhiloxWeyl0;
            k1 += kPhiloxWeyl1;
        }
        uint64_t p0 = (uint64_t)kPhiloxMul0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)kPhiloxMul1 * (uint64_t)c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 32-bit noise word of vocabulary entry v at draft position k for the
 * slot (seed, offset). */
uint32_t dspark_oracle_noise_word(uint64_t seed, uint64_t offset, uint32_t k, uint32_t v)
{
    uint32_t ctr[4] = { v >> 2, k, (uint32_t)offset, (uint32_t)(offset >> 32) };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t out[4];
    dspark_oracle_philox4x32_10(ctr, key, out);
    return out[v & 3u];
}

/* Uniform in the open unit interval from the top 23 bits of a word. */
double dspark_oracle_uniform(uint32_t x)
{
    return ((double)(x >> 9) + 0.5) / 8388608.0; /* 2^23 */
}

/* Standard Gumbel variate -ln(-ln u), rounded to float32. */
float dspark_oracle_gumbel(uint32_t x)
{
    double u = dspark_oracle_uniform(x);
    return (float)(-log(-log(u)));
}

void dspark_oracle_uniform_batch(const uint32_t* x, double* u, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) u[i] = dspark_oracle_uniform(x[i]);
}

void dspark_oracle_gumbel_batch(const uint32_t* x, float* g, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) g[i] = dspark_oracle_gumbel(x[i]);
}

/* ---- the draft block ------------------------------------------------------ */

static float bf16_to_float(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

typedef struct {
    const void* base; int base_is_bf16;     /* [B,K,V] */
    const uint16_t* E;                      /* [V,r] bf16 */
    const uint16_t* W;                      /* [r,V] bf16 */
    const int32_t* prev_token;              /* [B] */
    const int64_t* seed;                    /* [B] */
    const int64_t* offset;                  /* [B] */
    const float* temperature;               /* [B] */
    int n_real;                             /* < 0: every row is real */
    int B, K, V, r;
    const int32_t* forced;                  /* [B,K] or NULL; >= 0 replaces the token */
    double tie_eps;
    int max_cand;
    int32_t* tokens;                        /* [B,K] the token each position carries */
    int32_t* own_tokens;                    /* [B,K] or NULL: the oracle's own draw */
    float* logits;                          /* [B,K,V] or NULL */
    double* q;                              /* [B,K,V] or NULL */
    double* margin;                         /* [B,K] or NULL */
    int32_t* ncand;                         /* [B,K] or NULL */
    int32_t* cand;                          /* [B,K,max_cand] or NULL */
} OracleArgs;

static float base_at(const OracleArgs* a, int b, int k, int v)
{
    size_t i = ((size_t)b * a->K + k) * a->V + v;
    if (a->base_is_bf16) return bf16_to_float(((const uint16_t*)a->base)[i]);
    return ((const float*)a->base)[i];
}

/* Does score za at index ia beat zb at index ib?  NaN never wins; equal
 * scores go to the lower index. */
static int beats(float za, int ia, float zb, int ib)
{
    if (isnan(za)) return 0;
    if (ib < 0 || isnan(zb)) return 1;
    if (za > zb) return 1;
    if (za < zb) return 0;
    return ia < ib;
}

static void draft_row(const OracleArgs* a, int b, double* acc, float* lg, float* s, float* z)
{
    const int K = a->K, V = a->V, r = a->r;
    const int pad = (a->n_real >= 0 && b >= a->n_real);
    const float T = a->temperature[b];
    const int greedy = !(T > 0.0f);
    const float invT = greedy ? 0.0f : 1.0f / T;
    const uint64_t seed = (uint64_t)a->seed[b];
    const uint64_t off = (uint64_t)a->offset[b];
    int32_t d = a->prev_token[b];
    if (d < 0) d = 0;
    if (d > V - 1) d = V - 1;

    for (int k = 0; k < K; ++k) {
        /* bias[v] = sum_j E[d,j] * W[j,v]: exact products, double sum, one rounding */
        for (int v = 0; v < V; ++v) acc[v] = 0.0;
        for (int j = 0; j < r; ++j) {
            const double e = (double)bf16_to_float(a->E[(size_t)d * r + j]);
            const uint16_t* wrow = a->W + (size_t)j * V;
            for (int v = 0; v < V; ++v) acc[v] += e * (double)bf16_to_float(wrow[v]);
        }
        for (int v = 0; v < V; ++v) {
            const float base_v = pad ? 0.0f : base_at(a, b, k, v);
            lg[v] = base_v + (float)acc[v];
        }

        /* scores and the draw */
        int best = -1;
        for (int v = 0; v < V; ++v) {
            if (greedy) {
                z[v] = lg[v];
            } else {
                s[v] = lg[v] * invT;
                const float g = dspark_oracle_gumbel(dspark_oracle_noise_word(seed, off, (uint32_t)k, (uint32_t)v));
                z[v] = s[v] + g;
            }
            if (beats(z[v], v, best < 0 ? 0.0f : z[best], best)) best = v;
        }
        const int own = best < 0 ? 0 : best;

        /* runner-up score and the set of near-tied candidates */
        double second = -INFINITY;
        int n_near = 0;
        for (int v = 0; v < V; ++v) {
            if (isnan(z[v])) continue;
            if (v != best && (double)z[v] > second) second = (double)z[v];
            if (best >= 0 && (double)z[v] >= (double)z[best] - a->tie_eps) {
                if (a->cand && n_near < a->max_cand)
                    a->cand[((size_t)b * K + k) * a->max_cand + n_near] = v;
                ++n_near;
            }
        }
        const size_t bk = (size_t)b * K + k;
        if (a->margin) a->margin[bk] = best < 0 ? INFINITY : (double)z[best] - second;
        if (a->ncand) a->ncand[bk] = n_near;
        if (a->own_tokens) a->own_tokens[bk] = own;

        int carried = own;
        if (a->forced && a->forced[bk] >= 0) carried = a->forced[bk];
        a->tokens[bk] = carried;

        if (a->logits) memcpy(a->logits + bk * V, lg, (size_t)V * sizeof(float));

        if (a->q) {
            double* q = a->q + bk * V;
            if (greedy) {
                for (int v = 0; v < V; ++v) q[v] = (v == carried) ? 1.0 : 0.0;
            } else {
                double M = -INFINITY;
                for (int v = 0; v < V; ++v)
                    if ((double)s[v] > M) M = (double)s[v];
                double S = 0.0;
                for (int v = 0; v < V; ++v) S += exp((double)s[v] - M);
                for (int v = 0; v < V; ++v) q[v] = exp((double)s[v] - M) / S;
            }
        }
        d = carried;
    }
}

/* Run the sampler over every row.  Returns 0, or -1 on bad arguments. */
int dspark_oracle_draft_block(
    const void* base, int base_is_bf16, const uint16_t* E, const uint16_t* W,
    const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
    const float* temperature, int n_real, int B, int K, int V, int r,
    const int32_t* forced, double tie_eps, int max_cand,
    int32_t* tokens, int32_t* own_tokens, float* logits, double* q,
    double* margin, int32_t* ncand, int32_t* cand, int num_threads)
{
    if (B < 0 || K < 0 || V <= 0 || r <= 0) return -1;
    if (B == 0 || K == 0) return 0;
    if (!base || !E || !W || !prev_token || !seed || !offset || !temperature || !tokens) return -1;
    if (cand && max_cand <= 0) return -1;
    OracleArgs a = { base, base_is_bf16, E, W, prev_token, seed, offset, temperature, n_real,
                     B, K, V, r, forced, tie_eps, max_cand, tokens, own_tokens, logits, q,
                     margin, ncand, cand };
    int failed = 0;
#ifdef _OPENMP
    if (num_threads <= 0) num_threads = omp_get_max_threads();
#pragma omp parallel num_threads(num_threads)
#endif
    {
        double* acc = (double*)malloc((size_t)V * sizeof(double));
        float* lg = (float*)malloc((size_t)V * sizeof(float));
        float* s = (float*)malloc((size_t)V * sizeof(float));
        float* z = (float*)malloc((size_t)V * sizeof(float));
        if (!acc || !lg || !s || !z) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int b = 0; b < B; ++b)
            if (acc && lg && s && z) draft_row(&a, b, acc, lg, s, z);
        free(acc); free(lg); free(s); free(z);
    }
    return failed ? -2 : 0;
}

/* Number of threads the oracle uses when asked for the default. */
int dspark_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- standard token-level verification ------------------------------------
 *
 * What the draft block feeds: its tokens d_k and proposals q_k are checked
 * against target distributions p_k by the standard rule ("brb-nv/TensorRT-LLM
 * pull 21", section "2. Golden sampling semantics": rejection_sample_method
 * standard, token-level verification, the default). The pages name the rule
 * and do not spell it out; this is the textbook rule of Leviathan, Kalman
 * and Matias, "Fast Inference from Transformers via Speculative Decoding"
 * (ICML 2023), section 2.3, and Chen et al., "Accelerating Large Language
 * Model Decoding with Speculative Sampling" (2023), algorithm 2:
 *   for k = 0 .. K-1: accept d_k with probability min(1, p_k(d_k) / q_k(d_k));
 *   at the first rejection emit a token drawn from max(0, p_k - q_k)
 *   (normalised) and stop; if all K are accepted emit a bonus token drawn
 *   from p_K.
 * Output per row: n (the number accepted) and K+1 tokens: d_0 .. d_{n-1},
 * the emitted token, then -1.
 *
 * Readings (the pages are silent; each is listed in the design notes):
 *  - ratio = float32(p_k(d_k) / q_k(d_k)), one IEEE division; accept iff
 *    u_k < ratio (float32 compare). q = 0 < p gives +inf (accept); 0/0 gives
 *    NaN (reject).
 *  - u_k = ((x >> 9) + 1/2) 2^-23 for the Philox word x = word 0 of counter
 *    (0xFFFFFFFF, 256 + k, lo32(offset), hi32(offset)) under key
 *    (lo32(seed), hi32(seed)): the draft uses counter words y = k < 256, so
 *    the streams never meet.
 *  - The emitted token at position j (j < K: residual; j = K: bonus) is the
 *    Gumbel-max draw over w_v = float32(p_j(v) - q_j(v)) where that is > 0
 *    (residual) or w_v = p_j(v) (bonus), among v with w_v > 0: the lowest
 *    index of the largest ln(w_v) + g_v, g_v = -ln(-ln u) of word (v & 3) of
 *    counter (v >> 2, 512, lo32(offset), hi32(offset)). The counter does not
 *    depend on j: a row emits exactly one drawn token, and which position it
 *    is drawn at is decided by the acceptance uniforms (another stream), so
 *    the positions can share one noise stream. Scores are
 *    rounded to float32 before the argmax, as the kernel decides in float32.
 *    A residual with no positive entry (possible only through rounding, as
 *    p = q then) is replaced by p_j.
 */

static uint32_t verify_word(uint64_t seed, uint64_t offset, uint32_t x, uint32_t y, uint32_t w)
{
    uint32_t ctr[4] = { x, y, (uint32_t)offset, (uint32_t)(offset >> 32) };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t out[4];
    dspark_oracle_philox4x32_10(ctr, key, out);
    return out[w & 3u];
}

/* The acceptance uniform of position k, as float32 (exact). */
float dspark_oracle_verify_uniform(uint64_t seed, uint64_t offset, uint32_t k)
{
    return (float)dspark_oracle_uniform(verify_word(seed, offset, 0xFFFFFFFFu, 256u + k, 0u));
}

/* Gumbel variate of column v for the emitted token (at any position). */
float dspark_oracle_verify_gumbel(uint64_t seed, uint64_t offset, uint32_t v)
{
    return dspark_oracle_gumbel(verify_word(seed, offset, v >> 2, 512u, v));
}

int dspark_oracle_verify_standard(
    const float* q, const float* p, const int32_t* draft, const int64_t* seed, const int64_t* offset,
    int B, int K, int V, double tie_eps, int max_cand,
    int32_t* n_accepted, int32_t* out_tokens, int32_t* emit_pos,
    double* margin, int32_t* ncand, int32_t* cand)
{
    if (B < 0 || K < 0 || V <= 0) return -1;
    if (!q || !p || !draft || !seed || !offset || !n_accepted || !out_tokens) return -1;
    if (cand && max_cand <= 0) return -1;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int b = 0; b < B; ++b) {
        const uint64_t sd = (uint64_t)seed[b], off = (uint64_t)offset[b];
        int n = 0;
        for (; n < K; ++n) {
            int d = draft[(size_t)b * K + n];
            if (d < 0) d = 0;
            if (d > V - 1) d = V - 1;
            const float pv = p[((size_t)b * (K + 1) + n) * V + d];
            const float qv = q[((size_t)b * K + n) * V + d];
            const float ratio = pv / qv;
            const float u = dspark_oracle_verify_uniform(sd, off, (uint32_t)n);
            if (!(u < ratio)) break;
        }
        /* the emitted token */
        const float* pj = p + ((size_t)b * (K + 1) + n) * V;
        const float* qj = n < K ? q + ((size_t)b * K + n) * V : NULL;
        int use_p = (qj == NULL);
        if (!use_p) {
            int any = 0;
            for (int v = 0; v < V && !any; ++v) any = (pj[v] - qj[v]) > 0.0f;
            use_p = !any;
        }
        int best = -1;
        float zbest = 0.0f;
        for (int v = 0; v < V; ++v) {
            const float w = use_p ? pj[v] : pj[v] - qj[v];
            if (!(w > 0.0f)) continue;
            const float z = (float)log((double)w) + dspark_oracle_verify_gumbel(sd, off, (uint32_t)v);
            if (best < 0 || z > zbest) { best = v; zbest = z; }
        }
        double second = -INFINITY;
        int n_near = 0;
        for (int v = 0; v < V && best >= 0; ++v) {
            const float w = use_p ? pj[v] : pj[v] - qj[v];
            if (!(w > 0.0f)) continue;
            const float z = (float)log((double)w) + dspark_oracle_verify_gumbel(sd, off, (uint32_t)v);
            if (v != best && (double)z > second) second = (double)z;
            if ((double)z >= (double)zbest - tie_eps) {
                if (cand && n_near < max_cand) cand[(size_t)b * max_cand + n_near] = v;
                ++n_near;
            }
        }
        n_accepted[b] = n;
        int32_t* out = out_tokens + (size_t)b * (K + 1);
        for (int i = 0; i < n; ++i) {
            int d = draft[(size_t)b * K + i];
            out[i] = d < 0 ? 0 : (d > V - 1 ? V - 1 : d);
        }
        out[n] = best < 0 ? 0 : best;
        for (int i = n + 1; i <= K; ++i) out[i] = -1;
        if (emit_pos) emit_pos[b] = n;
        if (margin) margin[b] = best < 0 ? INFINITY : (double)zbest - second;
        if (ncand) ncand[b] = n_near;
    }
    return 0;
}

/* ---- block verification ----------------------------------------------------
 *
 * The pages' other rule ("brb-nv/TensorRT-LLM pull 21", section "2. Golden
 * sampling semantics": the option rejection_sample_method = block, citing
 * Sun et al., 2024; the page's test coverage claims losslessness under a
 * chi-square test). The pages
 * only name it; the algorithm is the one of Sun, Mendlovic, Leviathan,
 * Aharoni, Beirami, Ro and Suresh, "Block Verification Accelerates
 * Speculative Decoding" (2024), restated here in the indices of the draft
 * block (drafts d_0 .. d_{K-1}, d_j drawn from q_j; p_j the target
 * distribution after d_0 .. d_{j-1}, p_K the one after the whole block):
 *   w_0 = 1,  w_{j+1} = min(1, w_j * p_j(d_j) / q_j(d_j))   (prefix weights)
 *   S_j = sum_v max(w_j p_j(v) - q_j(v), 0)                 (residual mass)
 *   h_j = S_j / (S_j + 1 - w_j) for 1 <= j < K,  h_K = w_K
 *   n = the largest j in 1..K whose uniform eta_j passes h_j, else 0
 *   emit d_0 .. d_{n-1}, then a token drawn from max(w_n p_n - q_n, 0)
 *   (normalised) if n < K, or from p_K if n = K.
 * Unlike the token-level rule, a failed test at j does not end the scan: a
 * later position can still pass and keep the whole prefix.
 *
 * Readings (the pages are silent; each is listed in the design notes):
 *  - Weights, residual masses and thresholds in double. The ratio is one
 *    IEEE double division of the float32 inputs; w_{j+1} is the product
 *    w_j * ratio clamped to [0, 1] (q = 0 < p gives 1; 0/0 gives 0).
 *    Residual entries are w_j * p - q (a product and a difference, no fused
 *    multiply-add) clamped at 0. h_j = 0 when S_j = 0 (a stop there would
 *    need an empty residual; in exact arithmetic such a stop has
 *    probability zero, whatever h_j is).
 *  - eta_j is the acceptance uniform of draft d_{j-1}, the same word as the
 *    token-level rule's u_{j-1}; the test passes iff eta_j < h_j (the
 *    comparison in double).
 *  - The emitted token is drawn as in the token-level rule (the same
 *    position-free Gumbel words), from the weights
 *    float32(max(w_n p_n(v) - q_n(v), 0)) (or p_K(v)); an empty residual is
 *    replaced by p_n.
 */

static int clamp_tok(int d, int V)
{
    return d < 0 ? 0 : (d > V - 1 ? V - 1 : d);
}

/* Prefix weights w[0..K], residual masses S[0..K-1] and thresholds h[1..K]
 * of one row (h[0] = 1: the empty prefix is always kept). */
static void block_weights(const float* q, const float* p, const int32_t* draft, int K, int V,
                          double* w, double* S, double* h)
{
    w[0] = 1.0;
    for (int j = 0; j < K; ++j) {
        const int d = clamp_tok(draft[j], V);
        const double ratio = (double)p[(size_t)j * V + d] / (double)q[(size_t)j * V + d];
        const double t = w[j] * ratio;
        w[j + 1] = t >= 1.0 ? 1.0 : (t > 0.0 ? t : 0.0);
    }
    for (int j = 0; j < K; ++j) {
        double s = 0.0;
        for (int v = 0; v < V; ++v) {
            const double e = w[j] * (double)p[(size_t)j * V + v] - (double)q[(size_t)j * V + v];
            if (e > 0.0) s += e;
        }
        S[j] = s;
    }
    h[0] = 1.0;
    for (int j = 1; j < K; ++j) h[j] = S[j] > 0.0 ? S[j] / (S[j] + (1.0 - w[j])) : 0.0;
    if (K > 0) h[K] = w[K];
}

/* The float32 weight of column v of the distribution the token emitted at
 * position n is drawn from (before the empty-residual fallback). */
static float block_emit_weight(const float* q, const float* p, const double* w, int n, int K, int V, int v)
{
    if (n == K) return p[(size_t)K * V + v];
    const double e = w[n] * (double)p[(size_t)n * V + v] - (double)q[(size_t)n * V + v];
    return (float)(e > 0.0 ? e : 0.0);
}

/* The rule's quantities for inspection: w [B,K+1], S [B,K+1] (S[K] = 0),
 * h [B,K+1] and, if resid is given, the float32 weights of every position's
 * emission distribution [B,K+1,V] (position K: p_K). */
int dspark_oracle_verify_block_weights(
    const float* q, const float* p, const int32_t* draft, int B, int K, int V,
    double* w, double* S, double* h, float* resid)
{
    if (B < 0 || K < 0 || V <= 0 || !q || !p || !draft || !w || !S || !h) return -1;
    for (int b = 0; b < B; ++b) {
        const float* qb = q + (size_t)b * K * V;
        const float* pb = p + (size_t)b * (K + 1) * V;
        double* wb = w + (size_t)b * (K + 1);
        double* Sb = S + (size_t)b * (K + 1);
        double* hb = h + (size_t)b * (K + 1);
        block_weights(qb, pb, draft + (size_t)b * K, K, V, wb, Sb, hb);
        Sb[K] = 0.0;
        if (K == 0) hb[0] = 1.0;
        if (resid)
            for (int n = 0; n <= K; ++n)
                for (int v = 0; v < V; ++v)
                    resid[((size_t)b * (K + 1) + n) * V + v] = block_emit_weight(qb, pb, wb, n, K, V, v);
    }
    return 0;
}

int dspark_oracle_verify_block(
    const float* q, const float* p, const int32_t* draft, const int64_t* seed, const int64_t* offset,
    int B, int K, int V, double tie_eps, int max_cand,
    int32_t* n_accepted, int32_t* out_tokens, double* tau_margin,
    double* margin, int32_t* ncand, int32_t* cand)
{
    if (B < 0 || K < 0 || V <= 0 || K > 255) return -1;
    if (!q || !p || !draft || !seed || !offset || !n_accepted || !out_tokens) return -1;
    if (cand && max_cand <= 0) return -1;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int b = 0; b < B; ++b) {
        double w[256], S[256], h[256];
        const float* qb = q + (size_t)b * K * V;
        const float* pb = p + (size_t)b * (K + 1) * V;
        const uint64_t sd = (uint64_t)seed[b], off = (uint64_t)offset[b];
        block_weights(qb, pb, draft + (size_t)b * K, K, V, w, S, h);
        int n = 0;
        double tm = INFINITY;
        for (int j = 1; j <= K; ++j) {
            const double eta = (double)dspark_oracle_verify_uniform(sd, off, (uint32_t)(j - 1));
            if (eta < h[j]) n = j;
            if (fabs(eta - h[j]) < tm) tm = fabs(eta - h[j]);
        }
        int use_p = 0;
        if (n < K) {
            int any = 0;
            for (int v = 0; v < V && !any; ++v) any = block_emit_weight(qb, pb, w, n, K, V, v) > 0.0f;
            use_p = !any;
        }
        int best = -1;
        float zbest = 0.0f;
        for (int v = 0; v < V; ++v) {
            const float wt = use_p ? pb[(size_t)n * V + v] : block_emit_weight(qb, pb, w, n, K, V, v);
            if (!(wt > 0.0f)) continue;
            const float z = (float)log((double)wt) + dspark_oracle_verify_gumbel(sd, off, (uint32_t)v);
            if (best < 0 || z > zbest) { best = v; zbest = z; }
        }
        double second = -INFINITY;
        int n_near = 0;
        for (int v = 0; v < V && best >= 0; ++v) {
            const float wt = use_p ? pb[(size_t)n * V + v] : block_emit_weight(qb, pb, w, n, K, V, v);
            if (!(wt > 0.0f)) continue;
            const float z = (float)log((double)wt) + dspark_oracle_verify_gumbel(sd, off, (uint32_t)v);
            if (v != best && (double)z > second) second = (double)z;
            if ((double)z >= (double)zbest - tie_eps) {
                if (cand && n_near < max_cand) cand[(size_t)b * max_cand + n_near] = v;
                ++n_near;
            }
        }
        n_accepted[b] = n;
        int32_t* out = out_tokens + (size_t)b * (K + 1);
        for (int i = 0; i < n; ++i) out[i] = clamp_tok(draft[(size_t)b * K + i], V);
        out[n] = best < 0 ? 0 : best;
        for (int i = n + 1; i <= K; ++i) out[i] = -1;
        if (tau_margin) tau_margin[b] = tm;
        if (margin) margin[b] = best < 0 ? INFINITY : (double)zbest - second;
        if (ncand) ncand[b] = n_near;
    }
    return 0;
}
