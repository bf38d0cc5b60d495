/*
 * ORACLE -- test infrastructure only.  Only the tests, the package smoke check
 * and the benchmark's CPU-baseline leg may load this code; the product path
 * never does.
 *
 * Semi-autoregressive chaining of a K-token draft block, written out plainly in
 * double precision, one request row and one position at a time.
 *
 * What it computes (DSpark summary, "Draft better": a first-order Markov term,
 * held as a rank-256 factorisation and indexed by the previous position's
 * token, is added to each position's logits; MAX worklog, "What DSpark is", item 3:
 * the chain adds a rank-r term selected by the token chosen one position
 * earlier and takes an argmax):
 *
 *   prev = prev0[r]
 *   for i = 0 .. K-1:
 *       x[v]        = base[r, i, v] + sum_k A[prev, k] * Bmat[k, v]   (W = A Bmat)
 *       tokens[r,i] = argmax_v x[v]
 *       prev        = tokens[r, i]
 *
 * Readings where the pages are silent:
 *   - the bias is added to the logits as is: no scale, activation or
 *     normalisation; position 0 is keyed on prev0 (the last accepted token);
 *   - argmax returns the lowest index among equal maxima; NaN counts as larger
 *     than every number, so the first NaN wins; a row of -inf returns 0.  The
 *     index is always inside [0, V) (the MAX worklog's ArgMax NaN crash, "Scaling
 *     to 31B", is excluded by construction);
 *   - prev0 outside [0, V) is clamped into range and status bit 1 is set.
 *
 * Arithmetic: every bf16 / fp32 input is widened exactly to double; the bias of
 * column v is summed in increasing k starting from 0.0, then base is added.
 * Built with -O2 -ffp-contract=off, no fast-math.
 *
 * Probabilistic drafting (oracle_chain_sample): each position is a sample from
 * softmax(x / temperature) drawn by the Gumbel-max rule with counter-based random
 * numbers (Philox4x32-10 keyed on the seed, counter (v / 4, i, r, 0)); the argmax
 * conventions above apply to the perturbed values.  The vLLM blog's benchmark
 * samples at temperature 1.0 ("Results").
 *
 * Teacher forcing: when `forced` is non-NULL, position i > 0 is keyed on
 * forced[r, i-1] instead of the oracle's own previous argmax, so a comparison
 * against another implementation continues like for like after a near-tie.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* bf16 is the top half of an IEEE binary32; widening it is exact. */
static double bf16_to_double(uint16_t h) {
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double load_elem(const void* p, int dtype, size_t idx) {
    if (dtype == ORACLE_BF16) return bf16_to_double(((const uint16_t*)p)[idx]);
    return (double)((const float*)p)[idx];
}

/* a > b under "NaN is the largest value; NaNs are equal to each other". */
static int greater(double a, double b) {
    if (isnan(a)) return !isnan(b);
    if (isnan(b)) return 0;
    return a > b;
}

/* First index of the maximum of x[0..n). */
static int argmax_first(const double* x, int n) {
    int best = 0;
    for (int v = 1; v < n; ++v)
        if (greater(x[v], x[best])) best = v;
    return best;
}

/*
 * x[v] = base[r, i, v] + sum_k A[prev, k] * Bmat[k, v] for every v (the chained
 * logits of one request row and position).  a and bias are scratch of rank and V.
 */
static void chained_logits(const void* base, const void* A, const void* Bmat, int dtype, int K, int V,
                           int rank, int r, int i, int prev, double* a, double* bias, double* x) {
    /* a = A[prev, :] */
    for (int k = 0; k < rank; ++k) a[k] = load_elem(A, dtype, (size_t)prev * rank + k);
    /* bias[v] = sum_k a[k] * Bmat[k, v], accumulated in increasing k */
    for (int v = 0; v < V; ++v) bias[v] = 0.0;
    for (int k = 0; k < rank; ++k) {
        double ak = a[k];
        size_t off = (size_t)k * V;
        if (dtype == ORACLE_BF16) {
            const uint16_t* b = (const uint16_t*)Bmat + off;
            for (int v = 0; v < V; ++v) bias[v] += ak * bf16_to_double(b[v]);
        } else {
            const float* b = (const float*)Bmat + off;
            for (int v = 0; v < V; ++v) bias[v] += ak * (double)b[v];
        }
    }
    /* x[v] = base[r, i, v] + bias[v] */
    size_t row = ((size_t)r * K + i) * (size_t)V;
    for (int v = 0; v < V; ++v) x[v] = load_elem(base, dtype, row + v) + bias[v];
}

/*
 * Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3",
 * SC 2011): ten rounds of the Philox S-box over a 4-word counter under a 2-word
 * key, the key bumped by the Weyl constants between rounds.
 */
void oracle_philox4x32(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Standard Gumbel variate of entry v at (r, i): -log(-log u), u = (2 b + 1) / 2^24
 * from the top 23 bits b of Philox4x32-10 word v % 4 at counter (v / 4, i, r, 0). */
static double gumbel_at(uint64_t seed, int r, int i, int v) {
    const uint32_t ctr[4] = {(uint32_t)v >> 2, (uint32_t)i, (uint32_t)r, 0u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oracle_philox4x32(ctr, key, w);
    const uint32_t bits = w[v & 3] >> 9;
    const double u = (2.0 * (double)bits + 1.0) / 16777216.0;
    return -log(-log(u));
}

/*
 * rows[0..n_rows): request rows to evaluate (each row is an independent chain).
 * tokens_out: [n_rows, K].  logits_out: [n_rows, K, V] or NULL.
 * status_out: bit 1 set when a prev0 entry had to be clamped.
 * temperature > 0: sample each position by the Gumbel-max rule,
 *     token = argmax_v x[v] / temperature + gumbel(seed, r, i, v),
 * and logits_out then receives those perturbed values; temperature == 0: argmax of x.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
static int chain_rows(const void* base, const void* A, const void* Bmat, int dtype, const int32_t* prev0, int R,
                      int K, int V, int rank, const int32_t* rows, int n_rows, const int32_t* forced,
                      double temperature, uint64_t seed, int32_t* tokens_out, double* logits_out,
                      uint32_t* status_out) {
    if (R < 0 || K < 0 || V <= 0 || rank < 0 || n_rows < 0 || !(temperature >= 0.0)) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    double* x = (double*)malloc(sizeof(double) * (size_t)V);
    double* bias = (double*)malloc(sizeof(double) * (size_t)V);
    double* a = (double*)malloc(sizeof(double) * (size_t)(rank > 0 ? rank : 1));
    if (!x || !bias || !a) { free(x); free(bias); free(a); return -1; }
    uint32_t status = 0;

    for (int q = 0; q < n_rows; ++q) {
        int r = rows[q];
        if (r < 0 || r >= R) { free(x); free(bias); free(a); return -1; }
        int prev = prev0[r];
        if (prev < 0 || prev >= V) {
            status |= 1u;
            prev = prev < 0 ? 0 : V - 1;
        }
        for (int i = 0; i < K; ++i) {
            if (i > 0 && forced) {
                prev = forced[(size_t)r * K + (i - 1)];
                if (prev < 0 || prev >= V) { free(x); free(bias); free(a); return -1; }
            }
            chained_logits(base, A, Bmat, dtype, K, V, rank, r, i, prev, a, bias, x);
            if (temperature > 0.0)
                for (int v = 0; v < V; ++v) x[v] = x[v] / temperature + gumbel_at(seed, r, i, v);
            int tok = argmax_first(x, V);
            tokens_out[(size_t)q * K + i] = tok;
            if (logits_out) memcpy(logits_out + ((size_t)q * K + i) * (size_t)V, x, sizeof(double) * (size_t)V);
            prev = tok;
        }
    }
    if (status_out) *status_out = status;
    free(x); free(bias); free(a);
    return 0;
}

int oracle_chain(const void* base, const void* A, const void* Bmat, int dtype,
                 const int32_t* prev0, int R, int K, int V, int rank,
                 const int32_t* rows, int n_rows, const int32_t* forced,
                 int32_t* tokens_out, double* logits_out, uint32_t* status_out) {
    return chain_rows(base, A, Bmat, dtype, prev0, R, K, V, rank, rows, n_rows, forced, 0.0, 0, tokens_out,
                      logits_out, status_out);
}

int oracle_chain_sample(const void* base, const void* A, const void* Bmat, int dtype,
                        const int32_t* prev0, int R, int K, int V, int rank,
                        const int32_t* rows, int n_rows, const int32_t* forced, double temperature,
                        uint64_t seed, int32_t* tokens_out, double* perturbed_out, uint32_t* status_out) {
    if (!(temperature > 0.0)) return -1;
    return chain_rows(base, A, Bmat, dtype, prev0, R, K, V, rank, rows, n_rows, forced, temperature, seed,
                      tokens_out, perturbed_out, status_out);
}
