/*
 * sv_oracle.c -- plain fp64 CPU oracle of the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct
 * definition the HIP library is checked against. Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it. It shares no code,
 * header, table or constant with the HIP library, and includes nothing of it.
 *
 * Every floating-point step runs in double precision. Inputs given as fp32 or
 * bf16 are widened exactly (both embed in binary64), so the only rounding is
 * the oracle's own, in the order written here: left to right over the
 * vocabulary. Nothing is blocked, fused or reordered.
 *
 * Sources (the four web pages on draft-token verification):
 *  [CARD]   "spec-verify" kernels-hub card: sections "Method", "API",
 *           "Correctness", "Requirements and limits".
 *  [BLOG]   llmstudio.ru, "Как работает speculative decoding и MTP при
 *           инференсе LLM": section 13 (greedy verification), 15 (the
 *           min(1, p/q) rule), 16 (p > q), 17 (rejection and the residual
 *           distribution), 22 (what verify needs of the vocabulary),
 *           38 (temperature and the sampler pipeline), 42 (fixed-seed
 *           reproducibility), 47-48 (one iteration; left-to-right checking).
 *  [DSPARK] PocketLLM DSpark notes: the gate's per-position acceptance law
 *           and the early stop at the first mismatch.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  R1  The final draw (correction or bonus) of sequence b uses uniform
 *      column K_b; column i < K_b drives the accept test of position i.
 *  R2  Accept iff u < rho with u in [0,1): accepts with probability min(1,rho).
 *  R3  rho = p/q; q == 0 < p gives rho = +inf (accept); p == q == 0 gives 0.
 *  R4  ICDF(w, u) = smallest x with C(x) = sum_{y<=x} w(y) > u * S; zero-mass
 *      ids are never drawn. If no x qualifies (u >= 1), the last id with
 *      positive mass; if the row has no positive mass, -1.
 *  R5  Residual mass S == 0 after a rejection (impossible in exact arithmetic
 *      for normalised rows): draw from max(0, p) of the same row instead.
 *  R6  Argmax ties go to the lowest index; -0.0 equals +0.0 (IEEE compare).
 *  R7  A draft token outside [0, V) is a greedy miss and a sampled rejection.
 *      draft_lens[b] is clamped to [0, K]; NULL lens means K for every b.
 *  R8  Greedy reads its rows as given (logits or probabilities, no warp).
 *  R9  The bonus and fallback draws weigh ids by max(0, p) (identical to p
 *      for valid probability rows).
 *  R29 A draft distribution given by its log-normaliser (draft_lse) is taken
 *      as given: q_i(x) = exp(z_draft,i(x) / T - lse_i), not renormalised, so
 *      a wrong lse scales q_i (and with it the accept ratio and the residual).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "sv_oracle.h"

/* ---- element access: exact widening to binary64 ---------------------- */

static double elem(const void* base, int dtype, int64_t i) {
    switch (dtype) {
    case OR_F32:
        return (double)((const float*)base)[i];
    case OR_F64:
        return ((const double*)base)[i];
    case OR_BF16: {
        /* a bf16 value is the upper half of the fp32 with the same bits */
        uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    default:
        return NAN;
    }
}

static size_t dtype_size(int dtype) {
    return dtype == OR_BF16 ? 2u : dtype == OR_F32 ? 4u : 8u;
}

static const void* row_ptr(const void* base, int dtype, int64_t row, int64_t V) {
    return (const char*)base + (size_t)row * (size_t)V * dtype_size(dtype);
}

static int32_t clamp_len(const int32_t* lens, int64_t b, int64_t K) {
    if (lens == NULL) return (int32_t)K;
    int64_t k = lens[b];
    if (k < 0) k = 0;
    if (k > K) k = K;
    return (int32_t)k;
}

/* ---- warp: p = softmax(z / T) over one row  [BLOG s.38; CARD "Method"] --- */

void or_warp_row(const void* z, int dtype, int64_t V, double T, double* p) {
    double m = -INFINITY;
    for (int64_t x = 0; x < V; ++x) {
        double v = elem(z, dtype, x) / T;
        if (v > m) m = v;
    }
    double s = 0.0;
    for (int64_t x = 0; x < V; ++x) {
        double e = exp(elem(z, dtype, x) / T - m);
        p[x] = e;
        s += e;
    }
    for (int64_t x = 0; x < V; ++x) p[x] /= s;
}

/* Rows r < min(R, clamp(lens[b], 0, R - extra) + extra) of every sequence b. */
void or_softmax_warp(const void* logits, int dtype, int64_t B, int64_t R, int64_t V,
                     const int32_t* lens, int32_t extra_rows, double T, double* probs) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        int64_t live = (int64_t)clamp_len(lens, b, R - extra_rows) + extra_rows;
        if (live > R) live = R;
        for (int64_t r = 0; r < live; ++r)
            or_warp_row(row_ptr(logits, dtype, b * R + r, V), dtype, V, T, probs + (size_t)(b * R + r) * V);
    }
}

/* ---- argmax with lowest-index ties  [CARD "Method"; reading R6] -------- */

int64_t or_argmax_row(const void* row, int dtype, int64_t V) {
    int64_t best = 0;
    double bv = elem(row, dtype, 0);
    for (int64_t x = 1; x < V; ++x) {
        double v = elem(row, dtype, x);
        if (v > bv) { /* strict: an equal later value never displaces */
            bv = v;
            best = x;
        }
    }
    return best;
}

/* ---- greedy verification  [CARD "Method"; BLOG s.13, s.48] -------------
 * Accept t_i while it equals argmax(target_i); at the first miss emit that
 * row's argmax; if all K_b match, emit argmax(target_{K_b}). Rows after the
 * first miss are never examined. */
void or_verify_greedy(const void* target, int dtype, int64_t B, int64_t K, int64_t V,
                      const int32_t* tokens, const int32_t* lens, int32_t* n_accepted,
                      int32_t* next_token) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        int32_t kb = clamp_len(lens, b, K);
        int32_t n = 0;
        int64_t am = or_argmax_row(row_ptr(target, dtype, b * (K + 1) + 0, V), dtype, V);
        while (n < kb) {
            int64_t t = tokens[b * K + n];
            if (t < 0 || t >= V || t != am) break; /* R7: out-of-range is a miss */
            ++n;
            am = or_argmax_row(row_ptr(target, dtype, b * (K + 1) + n, V), dtype, V);
        }
        n_accepted[b] = n;
        next_token[b] = (int32_t)am;
    }
}

/* ---- inverse CDF  [CARD "Method"; BLOG s.17; reading R4] ---------------
 * kind 0: w(x) = max(0, p(x) - q(x))   (residual after a rejection)
 * kind 1: w(x) = max(0, p(x))          (bonus row, or fallback R5)     */

static double weight(const void* p, const void* q, int dtype, int kind, int64_t x) {
    double w = kind == 0 ? elem(p, dtype, x) - elem(q, dtype, x) : elem(p, dtype, x);
    return w > 0.0 ? w : 0.0;
}

double or_mass(const void* p, const void* q, int dtype, int kind, int64_t V) {
    double s = 0.0;
    for (int64_t x = 0; x < V; ++x) s += weight(p, q, dtype, kind, x);
    return s;
}

/* Returns the drawn id; *flag gets OR_FLAG_CDF when the threshold u*S lies
 * within rel_window (relative) of the cumulative mass on either side of the
 * drawn id, i.e. when a different rounding order could move the draw. */
int64_t or_icdf(const void* p, const void* q, int dtype, int kind, int64_t V, double u,
                double rel_window, int32_t* flag) {
    double S = or_mass(p, q, dtype, kind, V);
    if (!(S > 0.0)) {
        *flag |= OR_FLAG_NO_MASS;
        return -1;
    }
    double thr = u * S;
    double c = 0.0;
    int64_t last_pos = -1;
    for (int64_t x = 0; x < V; ++x) {
        double w = weight(p, q, dtype, kind, x);
        if (w > 0.0) last_pos = x;
        double c_prev = c;
        c += w;
        if (c > thr) {
            if (fabs(thr - c_prev) <= rel_window * c_prev || fabs(c - thr) <= rel_window * c)
                *flag |= OR_FLAG_CDF;
            return x;
        }
    }
    *flag |= OR_FLAG_CDF; /* u >= 1 or rounding at the top: unreachable for u < 1 */
    return last_pos;
}

/* ---- speculative-sampling verification  [CARD "Method"; BLOG s.15-17, s.47] ---
 * For i < K_b: accept t_i iff u[b,i] < p_i(t_i) / q_i(t_i); stop at the first
 * rejection n. If n < K_b draw the correction from norm(max(0, p_n - q_n));
 * else draw the bonus from p_{K_b}. Both draws use u[b, K_b] (R1). */
void or_accept(const void* p, const void* q, int dtype, int64_t B, int64_t K, int64_t V,
               const int32_t* tokens, const int32_t* lens, const void* uniforms, int u_dtype,
               double rel_window, int32_t* n_accepted, int32_t* next_token, int32_t* flags) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        int32_t kb = clamp_len(lens, b, K);
        int32_t flag = 0;
        int32_t n = kb;
        for (int32_t i = 0; i < kb; ++i) {
            int64_t t = tokens[b * K + i];
            double ui = elem(uniforms, u_dtype, b * (K + 1) + i);
            if (t < 0 || t >= V) { /* R7 */
                n = i;
                break;
            }
            double pt = elem(row_ptr(p, dtype, b * (K + 1) + i, V), dtype, t);
            double qt = elem(row_ptr(q, dtype, b * K + i, V), dtype, t);
            double rho;
            if (qt > 0.0)
                rho = pt / qt;
            else
                rho = pt > 0.0 ? INFINITY : 0.0; /* R3 */
            if (isfinite(rho) && fabs(ui - rho) <= rel_window * rho) flag |= OR_FLAG_RATIO;
            if (!(ui < rho)) { /* R2 */
                n = i;
                break;
            }
        }
        double uf = elem(uniforms, u_dtype, b * (K + 1) + kb);
        int64_t next;
        if (n < kb) {
            const void* pn = row_ptr(p, dtype, b * (K + 1) + n, V);
            const void* qn = row_ptr(q, dtype, b * K + n, V);
            if (or_mass(pn, qn, dtype, 0, V) > 0.0) {
                next = or_icdf(pn, qn, dtype, 0, V, uf, rel_window, &flag);
            } else { /* R5 */
                flag |= OR_FLAG_ZERO_RESIDUAL;
                next = or_icdf(pn, NULL, dtype, 1, V, uf, rel_window, &flag);
            }
        } else {
            next = or_icdf(row_ptr(p, dtype, b * (K + 1) + kb, V), NULL, dtype, 1, V, uf, rel_window, &flag);
        }
        n_accepted[b] = n;
        next_token[b] = (int32_t)next;
        if (flags) flags[b] = flag;
    }
}

/* ---- sampled verification from logits  [BLOG s.21-22, s.38; CARD "Method"] ---
 * The same procedure as or_accept on p = softmax(z_target / T) and
 * q = softmax(z_draft / T) of each examined row, warped in fp64 with
 * or_warp_row; only the rows the procedure examines are warped. Flags use
 * the same relative windows as or_accept: a tested u within rel_window * rho
 * of its ratio, a draw threshold within rel_window * C of a cumulative
 * weight C.
 *
 * With draft_lse (or_accept_logits_lse) the draft distribution of position i
 * is given by its log-normaliser instead of being normalised here:
 * q_i(x) = exp(z_draft,i(x) / T - draft_lse[b, i]) (R29). The draft model
 * computes this normaliser when it samples t_i from q_i; with the row's true
 * log-sum-exp the procedure is or_accept_logits exactly, up to the rounding
 * of the value passed in. */

/* q(x) = exp(z(x) / T - lse) over one row (R29). */
static void draft_row_given_lse(const void* z, int dtype, int64_t V, double T, double lse, double* q) {
    for (int64_t x = 0; x < V; ++x) q[x] = exp(elem(z, dtype, x) / T - lse);
}

static void accept_logits_impl(const void* zt, const void* zd, int dtype, int64_t B, int64_t K, int64_t V, double T,
                               const float* draft_lse, const int32_t* tokens, const int32_t* lens,
                               const void* uniforms, int u_dtype, double rel_window, int32_t* n_accepted,
                               int32_t* next_token, int32_t* flags) {
#pragma omp parallel
    {
        double* p = (double*)malloc((size_t)V * sizeof(double));
        double* q = (double*)malloc((size_t)V * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < B; ++b) {
            int32_t kb = clamp_len(lens, b, K);
            int32_t flag = 0;
            int32_t n = kb;
            for (int32_t i = 0; i < kb; ++i) {
                int64_t t = tokens[b * K + i];
                double ui = elem(uniforms, u_dtype, b * (K + 1) + i);
                if (t < 0 || t >= V) {
                    n = i;
                    break;
                }
                or_warp_row(row_ptr(zt, dtype, b * (K + 1) + i, V), dtype, V, T, p);
                if (draft_lse)
                    draft_row_given_lse(row_ptr(zd, dtype, b * K + i, V), dtype, V, T, (double)draft_lse[b * K + i], q);
                else
                    or_warp_row(row_ptr(zd, dtype, b * K + i, V), dtype, V, T, q);
                double rho = q[t] > 0.0 ? p[t] / q[t] : (p[t] > 0.0 ? INFINITY : 0.0);
                if (isfinite(rho) && fabs(ui - rho) <= rel_window * rho) flag |= OR_FLAG_RATIO;
                if (!(ui < rho)) {
                    n = i;
                    break;
                }
            }
            double u_final = elem(uniforms, u_dtype, b * (K + 1) + kb);
            int64_t next;
            int32_t f2 = 0;
            if (n < kb) {
                /* p, q hold row n unless the loop stopped on an out-of-range token */
                or_warp_row(row_ptr(zt, dtype, b * (K + 1) + n, V), dtype, V, T, p);
                if (draft_lse)
                    draft_row_given_lse(row_ptr(zd, dtype, b * K + n, V), dtype, V, T, (double)draft_lse[b * K + n], q);
                else
                    or_warp_row(row_ptr(zd, dtype, b * K + n, V), dtype, V, T, q);
                if (or_mass(p, q, OR_F64, 0, V) > 0.0) {
                    next = or_icdf(p, q, OR_F64, 0, V, u_final, rel_window, &f2);
                } else {
                    flag |= OR_FLAG_ZERO_RESIDUAL;
                    next = or_icdf(p, NULL, OR_F64, 1, V, u_final, rel_window, &f2);
                }
            } else {
                or_warp_row(row_ptr(zt, dtype, b * (K + 1) + kb, V), dtype, V, T, p);
                next = or_icdf(p, NULL, OR_F64, 1, V, u_final, rel_window, &f2);
            }
            n_accepted[b] = n;
            next_token[b] = (int32_t)next;
            if (flags) flags[b] = flag | f2;
        }
        free(p);
        free(q);
    }
}

void or_accept_logits(const void* zt, const void* zd, int dtype, int64_t B, int64_t K, int64_t V, double T,
                      const int32_t* tokens, const int32_t* lens, const void* uniforms, int u_dtype,
                      double rel_window, int32_t* n_accepted, int32_t* next_token, int32_t* flags) {
    accept_logits_impl(zt, zd, dtype, B, K, V, T, NULL, tokens, lens, uniforms, u_dtype, rel_window, n_accepted,
                       next_token, flags);
}

void or_accept_logits_lse(const void* zt, const void* zd, int dtype, int64_t B, int64_t K, int64_t V, double T,
                          const float* draft_lse, const int32_t* tokens, const int32_t* lens, const void* uniforms,
                          int u_dtype, double rel_window, int32_t* n_accepted, int32_t* next_token, int32_t* flags) {
    accept_logits_impl(zt, zd, dtype, B, K, V, T, draft_lse, tokens, lens, uniforms, u_dtype, rel_window, n_accepted,
                       next_token, flags);
}

/* ---- sampler penalties: the pipeline's first stage [BLOG s.38, s.39] ----
 * The sampler turns raw logits into the effective distribution as
 * penalties -> temperature -> top-k -> top-p -> normalise; the penalties are
 * stateful (they depend on the tokens so far), and under speculation their
 * state must follow the speculative branch: the history of verify row r is
 * the committed sequence followed by the draft tokens before position r.
 * Readings (the pages name the stage, not its formulas):
 *  R24 repetition penalty theta, as the transformers library applies it: an
 *      id present in the history has its logit z replaced by z * theta when
 *      z < 0, else by z / theta (theta = 1: off).
 *  R25 presence and frequency penalties (the usual serving-API form): an id
 *      with c > 0 occurrences in the history loses frequency * c + presence.
 *  R26 repetition first, then presence and frequency; ids outside [0, V) in
 *      the history are ignored.
 *  R27 the stage is defined in fp32, one rounding per operation, so that
 *      every later decision (top-k keys, argmax) sees identical values:
 *        z1 = z < 0 ? z * theta : z / theta       (c > 0)
 *        d  = fmaf(frequency, c, presence)
 *        z' = z1 - d                              (c > 0; z' = z otherwise) */
void or_penalize_row(const void* z, int dtype, int64_t V, const int32_t* hist, int64_t nh, float theta,
                     float presence, float frequency, float* out) {
    int32_t* count = (int32_t*)calloc((size_t)V, sizeof(int32_t));
    for (int64_t j = 0; j < nh; ++j)
        if (hist[j] >= 0 && hist[j] < V) count[hist[j]] += 1;
    for (int64_t x = 0; x < V; ++x) {
        float v = (float)elem(z, dtype, x); /* exact: the input is fp32 or bf16 */
        if (count[x] > 0) {
            float z1 = v < 0.0f ? v * theta : v / theta;
            float d = fmaf(frequency, (float)count[x], presence);
            v = z1 - d;
        }
        out[x] = v;
    }
    free(count);
}

/* Live rows r < clamp(lens[b], 0, R - extra) + extra of logits [B, R, V]:
 * history = seq[b, :clamp(seq_len[b], 0, cap)] (none when seq is NULL), then
 * draft tokens tokens[b, 0 .. r-1] (none when tokens is NULL); per-sequence
 * theta / presence / frequency (NULL: 1, 0, 0). Other rows are untouched. */
void or_apply_penalties(const void* logits, int dtype, int64_t B, int64_t R, int64_t V, const int32_t* lens,
                        int32_t extra_rows, const int32_t* seq, const int32_t* seq_len, int64_t cap,
                        const int32_t* tokens, int64_t K, const float* theta, const float* presence,
                        const float* frequency, float* out) {
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t r = 0; r < R; ++r) {
            int64_t live = (int64_t)clamp_len(lens, b, R - extra_rows) + extra_rows;
            if (r >= (live < R ? live : R)) continue;
            int64_t n0 = 0;
            if (seq) {
                n0 = seq_len[b];
                if (n0 < 0) n0 = 0;
                if (n0 > cap) n0 = cap;
            }
            int64_t np = tokens ? r : 0;
            int32_t* hist = (int32_t*)malloc((size_t)(n0 + np + 1) * sizeof(int32_t));
            for (int64_t j = 0; j < n0; ++j) hist[j] = seq[b * cap + j];
            for (int64_t j = 0; j < np; ++j) hist[n0 + j] = tokens[b * K + j];
            or_penalize_row(row_ptr(logits, dtype, b * R + r, V), dtype, V, hist, n0 + np, theta ? theta[b] : 1.0f,
                            presence ? presence[b] : 0.0f, frequency ? frequency[b] : 0.0f,
                            out + (size_t)(b * R + r) * V);
            free(hist);
        }
    }
}

/* ---- filtered warp: temperature, top-k, top-p, normalise [BLOG §38] ---
 * The sampler pipeline turns logits into the effective distribution in the
 * order: temperature, top-k, top-p, renormalisation (penalties and other
 * stateful filters are not part of it here; see BLOG §39). Readings:
 *  R16 top-k keeps every id whose value is at least the k-th largest value
 *      (ties at the boundary are all kept); k <= 0 or k >= V keeps all ids.
 *  R17 top-p acts on the top-k survivors renormalised: an id is kept iff the
 *      mass of the ids strictly more probable than it is below top_p times
 *      their total (equal values share one decision); the most probable
 *      value is always kept; top_p >= 1 (or NaN) keeps all survivors.
 *  R18 ids outside the kept set get probability exactly 0.
 * `flag` gets OR_FLAG_TOPP when the top-p decision of a boundary value lies
 * within `window` (relative to the survivors' mass) of the threshold. */
typedef struct {
    double y;
    int64_t x;
} vy_t;

static int by_value_desc(const void* a, const void* b) {
    double ya = ((const vy_t*)a)->y, yb = ((const vy_t*)b)->y;
    if (ya > yb) return -1;
    if (ya < yb) return 1;
    int64_t xa = ((const vy_t*)a)->x, xb = ((const vy_t*)b)->x;
    return xa < xb ? -1 : (xa > xb);
}

void or_warp_row_filtered(const void* z, int dtype, int64_t V, double T, int32_t top_k, double top_p,
                          double window, double* p, int32_t* flag) {
    int32_t f = 0;
    vy_t* s = (vy_t*)malloc((size_t)V * sizeof(vy_t));
    /* temperature */
    double m = -INFINITY;
    for (int64_t x = 0; x < V; ++x) {
        s[x].y = elem(z, dtype, x) / T;
        s[x].x = x;
        if (s[x].y > m) m = s[x].y;
    }
    /* descending value order (a library sort; ties in index order) */
    qsort(s, (size_t)V, sizeof(vy_t), by_value_desc);
    /* top-k: survivors are the first n entries of the sorted order */
    int64_t n = V;
    if (top_k > 0 && top_k < V) {
        double kth = s[top_k - 1].y;
        n = top_k;
        while (n < V && s[n].y >= kth) ++n;
    }
    for (int64_t x = 0; x < V; ++x) p[x] = 0.0;
    double S = 0.0;
    for (int64_t i = 0; i < n; ++i) S += exp(s[i].y - m);
    /* top-p over the survivors, one decision per group of equal values */
    int64_t kept = n;
    if (top_p < 1.0) {
        double target = top_p * S, above = 0.0;
        int64_t i = 0;
        kept = 0;
        while (i < n) {
            int64_t j = i;
            double g = 0.0;
            while (j < n && s[j].y == s[i].y) g += exp(s[j++].y - m);
            /* the most probable value is kept whatever top_p is: never a close call */
            if (i > 0 && fabs(above - target) <= window * S) f |= OR_FLAG_TOPP;
            if (i > 0 && !(above < target)) break;
            kept = j;
            above += g;
            i = j;
        }
    }
    double Sk = 0.0;
    for (int64_t i = 0; i < kept; ++i) Sk += exp(s[i].y - m);
    for (int64_t i = 0; i < kept; ++i) p[s[i].x] = exp(s[i].y - m) / Sk;
    free(s);
    if (flag) *flag = f;
}

/* Rows r < clamp(lens[b]) + extra_rows of every sequence, with that
 * sequence's top_k[b] / top_p[b] (NULL: the filter is off); rows past the
 * live count are left untouched (the caller pre-fills them). */
void or_softmax_warp_filtered(const void* logits, int dtype, int64_t B, int64_t R, int64_t V,
                              const int32_t* lens, int32_t extra_rows, double T, const int32_t* top_k,
                              const float* top_p, double window, double* probs, int32_t* flags) {
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t r = 0; r < R; ++r) {
            int64_t live = (int64_t)clamp_len(lens, b, R - extra_rows) + extra_rows;
            if (r >= (live < R ? live : R)) continue;
            int32_t f = 0;
            or_warp_row_filtered(row_ptr(logits, dtype, b * R + r, V), dtype, V, T, top_k ? top_k[b] : 0,
                                 top_p ? (double)top_p[b] : 1.0, window, probs + (size_t)(b * R + r) * V, &f);
            if (flags) flags[b * R + r] = f;
        }
    }
}

/* ---- top1 - top2 margin of a row [DSPARK "pre-draft gating"] -----------
 * The largest value minus the largest of the others (one occurrence of the
 * maximum removed, so a tied maximum gives 0); +inf when V == 1. */
double or_top2_margin(const void* row, int dtype, int64_t V) {
    int64_t am = or_argmax_row(row, dtype, V);
    double v1 = elem(row, dtype, am), v2 = -INFINITY;
    for (int64_t x = 0; x < V; ++x)
        if (x != am && elem(row, dtype, x) > v2) v2 = elem(row, dtype, x);
    return v1 - v2;
}

/* ---- acceptance-driven draft-length gate [DSPARK "gating"] --------------
 * Per sequence b, per bucket c (a draft position, or a caller's confidence
 * bucket of it): decayed counts hits[b, c] and trials[b, c].
 * Update after a verify round in which sequence b drafted kb = lens[b]
 * tokens and had n = n_accepted[b] accepted:
 *   if kb > 0: every count of b is multiplied by `decay` (forgetting), then
 *   positions j = 0 .. min(n, kb - 1) are recorded (trials += 1, hits += 1 if
 *   j < n). Positions after the first rejection were not observed (censored)
 *   and are not recorded.
 * Readings: a round without a draft observes nothing and forgets nothing;
 * bucket ids outside [0, NB) are clamped into it. */
static int32_t bucket_of(const int32_t* buckets, int64_t b, int64_t K, int64_t j, int64_t NB) {
    int64_t c = buckets ? buckets[b * K + j] : j;
    return (int32_t)(c < 0 ? 0 : (c >= NB ? NB - 1 : c));
}

void or_gate_update(double* hits, double* trials, int64_t B, int64_t NB, int64_t K, const int32_t* lens,
                    const int32_t* n_accepted, const int32_t* buckets, double decay) {
    for (int64_t b = 0; b < B; ++b) {
        int32_t kb = clamp_len(lens, b, K);
        if (kb == 0) continue;
        for (int64_t c = 0; c < NB; ++c) {
            hits[b * NB + c] *= decay;
            trials[b * NB + c] *= decay;
        }
        int64_t n = n_accepted[b] < 0 ? 0 : (n_accepted[b] > kb ? kb : n_accepted[b]);
        int64_t last = n < kb ? n : kb - 1;
        for (int64_t j = 0; j <= last; ++j) {
            int32_t c = bucket_of(buckets, b, K, j, NB);
            trials[b * NB + c] += 1.0;
            if (j < n) hits[b * NB + c] += 1.0;
        }
    }
}

/* Choice of the next draft length of sequence b, in 0 .. K:
 *   p_j = hits/trials of position j's bucket (1 while the bucket has no
 *         trials: a cold gate drafts and learns; reading),
 *   E(n) = 1 + sum_{i<n} prod_{j<=i} p_j,
 *   cost(0) = plain_ms, cost(n) = draft_ms + verify_base_ms + verify_slope_ms * n,
 *   n* = argmax_n E(n) / cost(n) (ties: the larger n; reading);
 *   a truncation n* < K is taken only if E/cost beats the full draft's by the
 *   factor `margin`; then n >= min_draft; and when margin_threshold > 0 and
 *   the committed token's top1 - top2 logit margin is below it, 0 (skip the
 *   draft). */
void or_gate_choose(const double* hits, const double* trials, int64_t B, int64_t NB, int64_t K,
                    const int32_t* buckets, const float* top2_margin, double draft_ms, double verify_base_ms,
                    double verify_slope_ms, double plain_ms, double margin, int32_t min_draft,
                    double margin_threshold, int32_t* next_lens) {
    for (int64_t b = 0; b < B; ++b) {
        double E = 1.0, prod = 1.0;
        double best = E / plain_ms, full = best;
        int64_t nstar = 0;
        for (int64_t n = 1; n <= K; ++n) {
            int32_t c = bucket_of(buckets, b, K, n - 1, NB);
            double t = trials[b * NB + c];
            double p = t > 0.0 ? hits[b * NB + c] / t : 1.0;
            prod *= p;
            E += prod;
            double r = E / (draft_ms + verify_base_ms + verify_slope_ms * (double)n);
            if (r >= best) {
                best = r;
                nstar = n;
            }
            if (n == K) full = r;
        }
        int64_t len = nstar;
        if (nstar < K && !(best >= margin * full)) len = K;
        if (len < min_draft) len = min_draft > K ? K : min_draft;
        if (margin_threshold > 0.0 && top2_margin && (double)top2_margin[b] < margin_threshold) len = 0;
        next_lens[b] = (int32_t)len;
    }
}

/* ---- per-position acceptance a = sum_x min(p(x), q(x))  [CARD "Measured"] ---
 * The probability that a token drawn from q passes the min(1, p/q) test. */
double or_overlap(const void* p, const void* q, int dtype, int64_t V) {
    double a = 0.0;
    for (int64_t x = 0; x < V; ++x) {
        double pv = elem(p, dtype, x), qv = elem(q, dtype, x);
        a += pv < qv ? pv : qv;
    }
    return a;
}

int or_abi_version(void) { return 1; }

/* Threads the parallel loops over rows use from now on (n >= 1); returns the
 * count in effect. Timing only: results do not depend on it. */
int or_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
