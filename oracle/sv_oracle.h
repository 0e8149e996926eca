/*
 * sv_oracle.h -- entry points of the fp64 CPU oracle (test infrastructure).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg use
 * these. Layouts are row-major with the vocabulary fastest: target/p rows
 * [B, K+1, V], draft/q rows [B, K, V], tokens [B, K], lens [B] (or NULL),
 * uniforms [B, K+1]. All pointers are host memory owned by the caller.
 */
#ifndef SV_ORACLE_H
#define SV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };

enum {
    OR_FLAG_RATIO = 1,         /* a tested u lies within the window of its ratio p/q */
    OR_FLAG_CDF = 2,           /* the draw threshold lies within the window of a CDF step */
    OR_FLAG_ZERO_RESIDUAL = 4, /* residual mass was zero; drew from p instead */
    OR_FLAG_NO_MASS = 8,       /* the final-draw row had no positive mass; next = -1 */
    OR_FLAG_TOPP = 16          /* a top-p decision lies within the window of its threshold */
};

int or_abi_version(void);
int or_set_threads(int n); /* threads of the row loops (timing only); returns the count in effect */

void or_warp_row(const void* z, int dtype, int64_t V, double T, double* p);
void or_softmax_warp(const void* logits, int dtype, int64_t B, int64_t R, int64_t V,
                     const int32_t* lens, int32_t extra_rows, double T, double* probs);

void or_warp_row_filtered(const void* z, int dtype, int64_t V, double T, int32_t top_k, double top_p,
                          double window, double* p, int32_t* flag);
void or_softmax_warp_filtered(const void* logits, int dtype, int64_t B, int64_t R, int64_t V,
                              const int32_t* lens, int32_t extra_rows, double T, const int32_t* top_k,
                              const float* top_p, double window, double* probs, int32_t* flags);

int64_t or_argmax_row(const void* row, int dtype, int64_t V);
void or_verify_greedy(const void* target, int dtype, int64_t B, int64_t K, int64_t V,
                      const int32_t* tokens, const int32_t* lens, int32_t* n_accepted,
                      int32_t* next_token);

double or_mass(const void* p, const void* q, int dtype, int kind, int64_t V);
int64_t or_icdf(const void* p, const void* q, int dtype, int kind, int64_t V, double u,
                double rel_window, int32_t* flag);
void or_accept(const void* p, const void* q, int dtype, int64_t B, int64_t K, int64_t V,
               const int32_t* tokens, const int32_t* lens, const void* uniforms, int u_dtype,
               double rel_window, int32_t* n_accepted, int32_t* next_token, int32_t* flags);

void or_accept_logits(const void* zt, const void* zd, int dtype, int64_t B, int64_t K, int64_t V, double T,
                      const int32_t* tokens, const int32_t* lens, const void* uniforms, int u_dtype,
                      double rel_window, int32_t* n_accepted, int32_t* next_token, int32_t* flags);
/* or_accept_logits with q_i(x) = exp(z_draft,i(x) / T - draft_lse[b*K + i]) (R29). */
void or_accept_logits_lse(const void* zt, const void* zd, int dtype, int64_t B, int64_t K, int64_t V, double T,
                          const float* draft_lse, const int32_t* tokens, const int32_t* lens, const void* uniforms,
                          int u_dtype, double rel_window, int32_t* n_accepted, int32_t* next_token, int32_t* flags);

void or_penalize_row(const void* z, int dtype, int64_t V, const int32_t* hist, int64_t nh, float theta,
                     float presence, float frequency, float* out);
void or_apply_penalties(const void* logits, int dtype, int64_t B, int64_t R, int64_t V, const int32_t* lens,
                        int32_t extra_rows, const int32_t* seq, const int32_t* seq_len, int64_t cap,
                        const int32_t* tokens, int64_t K, const float* theta, const float* presence,
                        const float* frequency, float* out);

double or_top2_margin(const void* row, int dtype, int64_t V);
void or_gate_update(double* hits, double* trials, int64_t B, int64_t NB, int64_t K, const int32_t* lens,
                    const int32_t* n_accepted, const int32_t* buckets, double decay);
void or_gate_choose(const double* hits, const double* trials, int64_t B, int64_t NB, int64_t K,
                    const int32_t* buckets, const float* top2_margin, double draft_ms, double verify_base_ms,
                    double verify_slope_ms, double plain_ms, double margin, int32_t min_draft,
                    double margin_threshold, int32_t* next_lens);

double or_overlap(const void* p, const void* q, int dtype, int64_t V);

#ifdef __cplusplus
}
#endif

#endif
