/* oracle_checks.c -- drives every entry point of the fp64 CPU oracle on small
 * inputs, edge cases included (V = 1, empty batches, ragged and out-of-range
 * draft lengths, -inf logits, zero residual mass, out-of-range history ids,
 * histories longer than their buffer, null optional arrays, every dtype), with
 * every array allocated at its exact size so that AddressSanitizer sees any
 * access past it and UndefinedBehaviorSanitizer any overflow or bad shift.
 * A few invariants are checked too (probabilities sum to one, draws stay in
 * range). Exit status 0: every call ran clean. Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sv_oracle.h"

static int failures = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform01(void) { /* splitmix64 */
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1.0p-53;
}

static void* exact(size_t n) { /* exact-size heap block: ASan guards both ends */
    void* p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

static float* logits_f32(int64_t n, int with_ninf) {
    float* z = exact((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; ++i) z[i] = (float)(6.0 * uniform01() - 3.0);
    if (with_ninf && n > 2) z[1] = -INFINITY;
    return z;
}

static uint16_t* to_bf16(const float* z, int64_t n) {
    uint16_t* o = exact((size_t)n * 2);
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &z[i], 4);
        o[i] = (uint16_t)(u >> 16);
    }
    return o;
}

static double* to_f64(const float* z, int64_t n) {
    double* o = exact((size_t)n * 8);
    for (int64_t i = 0; i < n; ++i) o[i] = z[i];
    return o;
}

static double row_sum(const double* p, int64_t V) {
    double s = 0.0;
    for (int64_t i = 0; i < V; ++i) s += p[i];
    return s;
}

static float* probs_f32(int64_t rows, int64_t V) { /* each row normalised */
    float* p = exact((size_t)(rows * V) * sizeof(float));
    for (int64_t r = 0; r < rows; ++r) {
        double s = 0.0;
        for (int64_t x = 0; x < V; ++x) s += (p[r * V + x] = (float)uniform01());
        for (int64_t x = 0; x < V; ++x) p[r * V + x] = (float)(p[r * V + x] / s);
    }
    return p;
}

static int32_t* ints(int64_t n, int32_t lo, int32_t hi) {
    int32_t* t = exact((size_t)n * 4);
    for (int64_t i = 0; i < n; ++i) t[i] = lo + (int32_t)(uniform01() * (double)(hi - lo + 1));
    return t;
}

static void warp_rows(void) {
    const int64_t Vs[] = {1, 2, 7, 300};
    for (int i = 0; i < 4; ++i) {
        const int64_t V = Vs[i];
        float* z = logits_f32(V, 1);
        uint16_t* zb = to_bf16(z, V);
        double* zd = to_f64(z, V);
        double* p = exact((size_t)V * 8);
        const void* rows[3] = {z, zb, zd};
        const int dts[3] = {OR_F32, OR_BF16, OR_F64};
        for (int d = 0; d < 3; ++d) {
            or_warp_row(rows[d], dts[d], V, 0.7, p);
            CHECK(fabs(row_sum(p, V) - 1.0) < 1e-12);
            int32_t fl = 0;
            const int32_t ks[] = {0, 1, (int32_t)V, (int32_t)V + 5};
            const double ps[] = {0.0, 1e-9, 0.5, 1.0, 1.5};
            for (int a = 0; a < 4; ++a)
                for (int b = 0; b < 5; ++b) {
                    or_warp_row_filtered(rows[d], dts[d], V, 1.3, ks[a], ps[b], 1e-5, p, &fl);
                    CHECK(fabs(row_sum(p, V) - 1.0) < 1e-12);
                }
            const int64_t m = or_argmax_row(rows[d], dts[d], V);
            CHECK(m >= 0 && m < V);
            (void)or_top2_margin(rows[d], dts[d], V);
        }
        free(z), free(zb), free(zd), free(p);
    }
}

static void batched_warps(void) {
    const int64_t B = 4, R = 3, V = 33;
    float* z = logits_f32(B * R * V, 1);
    uint16_t* zb = to_bf16(z, B * R * V);
    int32_t lens[4] = {-1, 0, 2, 9};
    double* p = exact((size_t)(B * R * V) * 8);
    int32_t* fl = exact((size_t)(B * R) * 4);
    int32_t tk[4] = {0, 1, 40, -3};
    float tp[4] = {1.0f, 0.3f, 0.0f, 2.0f};
    for (int e = 0; e <= 1; ++e) {
        or_softmax_warp(z, OR_F32, B, R, V, lens, e, 1.0, p);
        or_softmax_warp(zb, OR_BF16, B, R, V, NULL, e, 0.5, p);
        or_softmax_warp_filtered(z, OR_F32, B, R, V, lens, e, 0.8, tk, tp, 1e-5, p, fl);
        or_softmax_warp_filtered(zb, OR_BF16, B, R, V, NULL, e, 0.8, NULL, NULL, 1e-5, p, fl);
    }
    or_softmax_warp(z, OR_F32, 0, R, V, NULL, 1, 1.0, p); /* empty batch */
    free(z), free(zb), free(p), free(fl);
}

static void verifies(void) {
    const int64_t B = 5, V = 17;
    for (int64_t K = 0; K <= 4; K += 4) {
        float* zt = logits_f32(B * (K + 1) * V, 1);
        float* zd = logits_f32(B * (K > 0 ? K : 1) * V, 0);
        float* p = probs_f32(B * (K + 1), V);
        float* q = probs_f32(B * (K > 0 ? K : 1), V);
        if (K > 0) memcpy(p, q, (size_t)V * sizeof(float)); /* p = q in row (0, 0): zero residual */
        int32_t* tok = ints(B * (K > 0 ? K : 1), 0, (int32_t)V - 1);
        int32_t lens[5] = {-2, 0, 1, (int32_t)K, (int32_t)K + 3};
        double* u = exact((size_t)(B * (K + 1)) * 8);
        float* uf = exact((size_t)(B * (K + 1)) * 4);
        for (int64_t i = 0; i < B * (K + 1); ++i) uf[i] = (float)(u[i] = uniform01());
        u[0] = 0.0;
        int32_t* n = exact((size_t)B * 4);
        int32_t* nx = exact((size_t)B * 4);
        int32_t* fl = exact((size_t)B * 4);
        for (int l = 0; l < 2; ++l) {
            const int32_t* ln = l ? lens : NULL;
            or_verify_greedy(zt, OR_F32, B, K, V, tok, ln, n, nx);
            for (int64_t b = 0; b < B; ++b) CHECK(n[b] >= 0 && n[b] <= K && nx[b] >= 0 && nx[b] < V);
            or_accept(p, q, OR_F32, B, K, V, tok, ln, u, OR_F64, 1e-7, n, nx, fl);
            for (int64_t b = 0; b < B; ++b) CHECK(n[b] >= 0 && n[b] <= K && nx[b] >= -1 && nx[b] < V);
            or_accept(p, q, OR_F32, B, K, V, tok, ln, uf, OR_F32, 1e-5, n, nx, fl);
            or_accept_logits(zt, zd, OR_F32, B, K, V, 0.9, tok, ln, u, OR_F64, 1e-5, n, nx, fl);
            for (int64_t b = 0; b < B; ++b) CHECK(n[b] >= 0 && n[b] <= K && nx[b] >= -1 && nx[b] < V);
            /* given draft normalisers: exact-size [B, K] array (one element when K = 0) */
            float* lse = exact((size_t)(B * (K > 0 ? K : 1)) * 4);
            for (int64_t i = 0; i < B * (K > 0 ? K : 1); ++i) lse[i] = (float)(3.0 * uniform01());
            or_accept_logits_lse(zt, zd, OR_F32, B, K, V, 0.9, lse, tok, ln, u, OR_F64, 1e-5, n, nx, fl);
            for (int64_t b = 0; b < B; ++b) CHECK(n[b] >= 0 && n[b] <= K && nx[b] >= -1 && nx[b] < V);
            free(lse);
        }
        for (int kind = 0; kind <= 1; ++kind) {
            int32_t f = 0;
            (void)or_mass(p, q, OR_F32, kind, V);
            const int64_t x = or_icdf(p, q, OR_F32, kind, V, 0.999999, 1e-7, &f);
            CHECK(x >= -1 && x < V);
            (void)or_overlap(p, q, OR_F32, V);
        }
        free(zt), free(zd), free(p), free(q), free(tok), free(u), free(uf), free(n), free(nx), free(fl);
    }
}

static void penalties(void) {
    const int64_t B = 4, K = 3, R = K + 1, V = 9, cap = 6;
    float* z = logits_f32(B * R * V, 1);
    uint16_t* zb = to_bf16(z, B * R * V);
    float* out = exact((size_t)(B * R * V) * sizeof(float));
    int32_t* seq = ints(B * cap, -2, (int32_t)V + 2); /* some ids outside [0, V) */
    int32_t seq_len[4] = {-1, 0, 3, 50};              /* 50 > cap: clamped */
    int32_t* tok = ints(B * K, -1, (int32_t)V);
    int32_t lens[4] = {3, -1, 1, 7};
    float th[4] = {1.0f, 1.5f, 0.5f, 2.0f}, pr[4] = {0.0f, 0.3f, -0.2f, 1.0f}, fq[4] = {0.0f, 0.1f, 0.5f, 0.0f};
    or_apply_penalties(z, OR_F32, B, R, V, lens, 1, seq, seq_len, cap, tok, K, th, pr, fq, out);
    or_apply_penalties(zb, OR_BF16, B, R, V, NULL, 1, NULL, NULL, 0, tok, K, th, NULL, fq, out);
    or_apply_penalties(z, OR_F32, B, K, V, lens, 0, seq, seq_len, cap, NULL, 0, NULL, NULL, NULL, out);
    or_penalize_row(z, OR_F32, V, NULL, 0, 1.3f, 0.2f, 0.1f, out);
    or_penalize_row(zb, OR_BF16, V, seq, B * cap, 1.3f, 0.2f, 0.1f, out);
    or_penalize_row(z, OR_F32, 1, seq, 3, 0.7f, 0.0f, 0.0f, out); /* V = 1 */
    free(z), free(zb), free(out), free(seq), free(tok);
}

static void gate(void) {
    const int64_t B = 3, K = 4, NB = 4;
    double* hits = exact((size_t)(B * NB) * 8);
    double* trials = exact((size_t)(B * NB) * 8);
    for (int64_t i = 0; i < B * NB; ++i) hits[i] = trials[i] = 0.0;
    int32_t lens[3] = {4, 0, 9}, n[3] = {2, 0, 4};
    int32_t* buckets = ints(B * K, -3, (int32_t)NB + 3); /* clamped into [0, NB) */
    float mg[3] = {0.1f, 5.0f, 0.0f};
    int32_t out[3];
    for (int r = 0; r < 3; ++r) {
        or_gate_update(hits, trials, B, NB, K, lens, n, r ? buckets : NULL, 0.9);
        or_gate_choose(hits, trials, B, NB, K, r ? buckets : NULL, r == 2 ? mg : NULL, 1.0, 5.0, 0.1, 4.0, 0.0, 1,
                       r == 2 ? 1.0 : 0.0, out);
        for (int64_t b = 0; b < B; ++b) CHECK(out[b] >= 0 && out[b] <= K);
    }
    free(hits), free(trials), free(buckets);
}

int main(void) {
    CHECK(or_abi_version() > 0);
    warp_rows();
    batched_warps();
    verifies();
    penalties();
    gate();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle checks clean\n");
    return 0;
}
