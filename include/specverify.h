/*
 * specverify.h -- C ABI of libspecverify: the verify step of speculative
 * decoding on AMD Instinct MI355X (gfx950), as hand-written HIP kernels.
 *
 * Over a batch of B sequences a target model scored K+1 positions and a draft
 * model proposed K tokens. The calls below decide, per sequence, how many
 * draft tokens are kept (n_accepted) and which token follows them
 * (next_token). The caller keeps draft_tokens[b, :n_accepted[b]] and appends
 * next_token[b] (spec-verify card, "Usage" and "API").
 *
 * Layouts (row-major, vocabulary fastest, no padding between rows):
 *   target        [B, K+1, V]   row i scores position i; row K_b is the bonus row
 *   draft         [B, K,   V]   row i is the draft distribution of token i
 *   draft_tokens  [B, K]        int32
 *   draft_lens    [B]           int32 per-sequence draft length K_b, clamped to
 *                               [0, K]; NULL means K_b = K for every sequence
 *   uniforms      [B, K+1]      fp32 in [0, 1); column i < K_b drives the accept
 *                               test of position i, column K_b the final draw
 *   n_accepted, next_token  [B] int32 outputs
 *
 * Conventions for every entry point:
 *  - Pointers are device memory owned by the caller. The library never
 *    allocates, frees or retains them; its only scratch memory, the exchange
 *    slots of sv_softmax_warp, sv_verify_greedy(_margin) and sv_accept_logits
 *    (their `workspace` arguments), is passed in by the caller too (the one
 *    exception is sv_softmax_warp_noalloc's fixed array, below).
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the default
 *    stream) and return. Outputs are valid once the stream reaches them.
 *    Calls keep no state between them; concurrent calls on different streams
 *    are safe.
 *  - Results are bitwise deterministic run to run: every reduction has a fixed
 *    order.
 *  - Host-side argument checks return an error before anything is enqueued;
 *    sv_last_error() then describes it. A launch failure returns SV_ERR_HIP.
 *  - Workspaces: a call that takes one accepts either none (a null pointer
 *    or 0 bytes: a path that needs no exchange slots runs instead, with the
 *    same results) or at least the bytes its *_workspace_bytes query returns
 *    for the same sizes, 8-byte aligned; anything in between is
 *    SV_ERR_WORKSPACE, so an undersized buffer never silently selects the
 *    slower path.
 *  - Data-dependent conditions are defined behaviour, not errors: a draft
 *    token outside [0, V) is a greedy miss and a sampled rejection and is
 *    never dereferenced; draft_lens are clamped. Rows, tokens and uniforms a
 *    sequence does not use are never read. NaN inputs are outside the contract.
 *  - B == 0 is a valid empty call and enqueues nothing.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 4
#define SV_MAX_K 64 /* draft lengths up to 64, one wavefront lane per position */

typedef enum {
    SV_OK = 0,
    SV_ERR_INVALID_ARG = 1, /* null pointer, size out of range, misaligned pointer, bad dtype */
    SV_ERR_UNSUPPORTED = 2, /* the current device is not gfx950 */
    SV_ERR_HIP = 3,         /* the HIP runtime reported an error at launch */
    SV_ERR_WORKSPACE = 4    /* a workspace of more than 0 bytes is smaller than its query returns */
} sv_status;

typedef enum {
    SV_F32 = 0,  /* IEEE binary32 */
    SV_BF16 = 1  /* bfloat16: the upper 16 bits of a binary32 */
} sv_dtype;

/* Version of this ABI (SV_ABI_VERSION of the build). */
int sv_abi_version(void);

/* Static description of a status code. */
const char* sv_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* sv_last_error(void);

/*
 * sv_softmax_warp -- temperature warp: probs[r, x] = softmax(logits[r, :] / T)[x].
 *
 * The sampled verify works on the distributions the sampler would draw from,
 * after the temperature step, with target and draft warped identically
 * (llmstudio blog "Как работает speculative decoding и MTP при инференсе
 * LLM", sections 21-22 and 38; spec-verify card, "Method" and "Requirements
 * and limits").
 *
 * logits       [B, R, V] of `dtype` (SV_F32 or SV_BF16), element-aligned.
 * draft_lens   [B] or NULL. Sequence b has live rows r < clamp(draft_lens[b],
 *              0, R - extra_rows) + extra_rows; NULL makes all R rows live.
 *              Use extra_rows = 1 with R = K+1 for target rows and
 *              extra_rows = 0 with R = K for draft rows.
 * temperature  finite, > 0.
 * probs        [B, R, V] fp32 output, 4-byte aligned; only live rows are
 *              written, the others are left untouched.
 * workspace    device memory of at least sv_softmax_warp_workspace_bytes(B,
 *              R, V) bytes, 8-byte aligned, owned by the caller, contents
 *              irrelevant (the call initialises it on `stream`); it holds the
 *              per-row partial statistics the workgroups of a row exchange.
 *              NULL or 0 bytes selects a slower path that needs none;
 *              fewer bytes than the query returns is SV_ERR_WORKSPACE.
 *              Calls that overlap in time must not share a workspace.
 * Accuracy: |probs - exact| <= 1e-5 absolute per element (fp32 arithmetic,
 * exp2 with a folded log2(e)/T scale, fixed-order sums); results are bitwise
 * identical run to run and independent of the workspace path's internal
 * timing.
 * Errors: SV_ERR_INVALID_ARG for a null logits/probs, B < 0, R < 1,
 * extra_rows not in [0, R], V < 1 or V > INT32_MAX, B*R > INT32_MAX, a bad
 * dtype or temperature, or misaligned pointers; SV_ERR_WORKSPACE as above.
 */
sv_status sv_softmax_warp(const void* logits, int dtype, int32_t B, int32_t R, int64_t V,
                          const int32_t* draft_lens, int32_t extra_rows, float temperature,
                          float* probs, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes sv_softmax_warp uses for these sizes (0 when its fast path
 * does not apply: V not a multiple of 4, or V above about 2 million). */
size_t sv_softmax_warp_workspace_bytes(int32_t B, int32_t R, int64_t V);

/*
 * sv_softmax_warp_noalloc -- sv_softmax_warp for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. It calls no allocating routine; the
 * exchange slots that sv_softmax_warp takes from a caller's workspace live in
 * a fixed device array of SV_NOALLOC_SCRATCH_BYTES bytes inside the library
 * (one per device, held until the process ends).
 * Arguments, results (bitwise those of sv_softmax_warp with a workspace) and
 * errors as sv_softmax_warp, plus SV_ERR_WORKSPACE when the call needs more
 * slots than the array holds, i.e. sv_softmax_warp_workspace_bytes(B, R, V)
 * > SV_NOALLOC_SCRATCH_BYTES (up to 131072 row slices: 8704 rows of 256000).
 * Every call on a device shares that device's array and leaves its slots
 * behind (each call resets them on its stream first), so calls that overlap
 * in time on one device race: serialise them on one stream.
 */
#define SV_NOALLOC_SCRATCH_BYTES 1048576
sv_status sv_softmax_warp_noalloc(const void* logits, int dtype, int32_t B, int32_t R, int64_t V,
                                  const int32_t* draft_lens, int32_t extra_rows, float temperature, float* probs,
                                  void* stream);

/* Diagnostic control, process-wide: how many times a workgroup polls for the
 * partial results of the other workgroups that share its row or sequence
 * before computing them all itself (default 16384), for calls made after
 * this one. It governs sv_softmax_warp's fast path, and sv_accept_logits,
 * sv_verify_greedy and sv_verify_greedy_margin with a workspace. Any value
 * gives the same results; 0 forces the self-computation. Returns
 * SV_ERR_INVALID_ARG for a negative value. */
sv_status sv_set_wait_limit(int32_t polls);

/* Tuning control, process-wide: the look-ahead depth L of the split greedy
 * walk (sv_verify_greedy and sv_verify_greedy_margin with a workspace), for
 * calls made after this one. At position i each workgroup reads its slices
 * of target rows up to min(K_b, i + L) before it waits for the rest of row
 * i, so that the wait overlaps the next rows' loads. L = 0 (the default,
 * SV_GREEDY_LOOKAHEAD) is the walk the method describes: row i+1 is read
 * only after row i matched (spec-verify card, "Method"; llmstudio blog
 * "Как работает speculative decoding и MTP при инференсе LLM", section 13).
 * Rows read ahead of a sequence's first miss are read but not needed;
 * L >= K + 1 reads every live row. Every L gives the same results; only the
 * bytes read and the time change. Without a workspace, or for rows of at
 * most 128 KB (one workgroup per sequence, no exchange), L is not used.
 * Returns SV_ERR_INVALID_ARG for rows outside [0, SV_MAX_K + 1]. */
#define SV_GREEDY_LOOKAHEAD 0
sv_status sv_set_greedy_lookahead(int32_t rows);

/*
 * sv_softmax_warp_filtered -- the sampler pipeline temperature -> top-k ->
 * top-p -> renormalise (llmstudio blog "Как работает speculative decoding и
 * MTP при инференсе LLM", section 38: the verify compares the distributions
 * after the sampler's transforms, target and draft filtered alike).
 *
 * Same rows, layouts and live-row rule as sv_softmax_warp, plus per-sequence
 * filter parameters:
 * top_k   [B] int32 device array, or NULL (off for every sequence). Sequence
 *         b keeps every id whose logit is at least its row's top_k[b]-th
 *         largest logit (ties at the boundary are all kept); top_k[b] <= 0 or
 *         >= V turns the filter off.
 * top_p   [B] fp32 device array, or NULL (off). After top-k, with the
 *         survivors renormalised, an id is kept iff the mass of the ids
 *         strictly more probable than it is below top_p[b] times the
 *         survivors' mass; equal logits are kept or dropped together; the
 *         largest logit is always kept (so top_p[b] <= 0 keeps only it);
 *         top_p[b] >= 1 or NaN turns the filter off.
 * probs   live rows get softmax over the kept ids and exactly 0 elsewhere.
 * Kept sets are decided exactly for top-k; top-p decides with fixed-point
 * masses (2^-40 or finer per unit) of fp32 exponentials, so a value within
 * ~1e-5 relative of its threshold may fall either way. Results are bitwise
 * identical run to run. No workspace; one workgroup per live row. When the
 * kept ids lie within 20 log2 units of the row maximum, the row is read once
 * and the output written once (for rows of up to 1,048,576 elements with V a
 * multiple of 8 (bf16) or 4 (fp32) and 16-byte aligned logits and probs);
 * otherwise the row is read several times. Rows with neither filter are
 * correct but read twice: sv_softmax_warp is the faster call for them.
 * Errors: as sv_softmax_warp, plus misaligned top_k / top_p.
 */
sv_status sv_softmax_warp_filtered(const void* logits, int dtype, int32_t B, int32_t R, int64_t V,
                                   const int32_t* draft_lens, int32_t extra_rows, float temperature,
                                   const int32_t* top_k, const float* top_p, float* probs, void* stream);

/*
 * sv_apply_penalties -- the sampler pipeline's first stage: repetition,
 * presence and frequency penalties of the live logit rows, each row with its
 * own token history (llmstudio blog "Как работает speculative decoding и MTP
 * при инференсе LLM", section 38: raw logits -> penalties -> temperature ->
 * top-k -> top-p -> normalise; section 39: a stateful sampler's state must
 * follow the speculative branch).
 *
 * The history of row r of sequence b is seq[b, :clamp(seq_len[b], 0, cap)]
 * followed by draft_tokens[b, 0 .. r-1]; ids outside [0, V) in it are
 * ignored. An id with c > 0 occurrences gets, in fp32 with one rounding per
 * operation,
 *     z1 = z < 0 ? z * theta : z / theta,   z' = z1 - fmaf(frequency, c, presence)
 * (the repetition penalty as the transformers library applies it, then the
 * usual presence and frequency penalties); every other id keeps z. The rest
 * of the pipeline runs on the output: sv_softmax_warp_filtered (or
 * sv_softmax_warp) for the sampled verify, sv_verify_greedy for greedy.
 *
 * logits       [B, R, V] of `dtype`, element-aligned; rows and live-row rule
 *              as sv_softmax_warp (draft_lens, extra_rows).
 * pen          host pointer to the parameters below (read during the call):
 *   seq          [B, cap] int32 token buffers (sv_commit's), or NULL: no
 *                committed history;
 *   seq_len      [B] int32, required with seq;
 *   cap          row stride of seq, >= 1 with seq;
 *   draft_tokens [B, K] int32, or NULL: no draft prefix; with it K >= R - 1;
 *   K            row stride of draft_tokens;
 *   repetition, presence, frequency   [B] fp32 per-sequence parameters, or
 *                NULL (1, 0, 0: off). theta must be finite and > 0 and the
 *                others finite; other values are outside the contract.
 * out          [B, R, V] fp32, 4-byte aligned, not overlapping logits; live
 *              rows are written, the others left untouched.
 * workspace    with seq: at least sv_apply_penalties_workspace_bytes(B, cap)
 *              bytes, 4-byte aligned, contents irrelevant (the call builds
 *              its tables in it); not needed without seq.
 * Result: bitwise the fp32 values above.
 * Errors: SV_ERR_INVALID_ARG for null logits/out/pen, bad sizes (as
 * sv_softmax_warp), seq without seq_len, cap < 1 with seq, K < R - 1 with
 * draft_tokens, misaligned pointers; SV_ERR_WORKSPACE when seq is given and
 * the workspace is missing or too small.
 */
typedef struct {
    const int32_t* seq;
    const int32_t* seq_len;
    int32_t cap;
    const int32_t* draft_tokens;
    int32_t K;
    const float* repetition;
    const float* presence;
    const float* frequency;
} sv_penalties;

sv_status sv_apply_penalties(const void* logits, int dtype, int32_t B, int32_t R, int64_t V,
                             const int32_t* draft_lens, int32_t extra_rows, const sv_penalties* pen, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes sv_apply_penalties needs for B sequences with token buffers
 * of cap tokens (0 for invalid sizes). */
size_t sv_apply_penalties_workspace_bytes(int32_t B, int32_t cap);

/*
 * sv_verify_greedy -- temperature-0 verification.
 *
 * Accept draft token t_i while it equals argmax(target row i); at the first
 * miss emit that row's argmax and stop; if all K_b match emit
 * argmax(target row K_b) (spec-verify card, "Method"; llmstudio blog,
 * sections 13 and 48). Rows after a sequence's first miss are never read.
 * The argmax takes the lowest index among equal maxima; -0.0 equals +0.0.
 * The rows are read as given: logits or probabilities, no warp.
 *
 * target       [B, K+1, V] of `dtype` (SV_F32 or SV_BF16), element-aligned.
 * draft_tokens [B, K] int32 (may be NULL when K == 0).
 * draft_lens   [B] int32 or NULL.
 * workspace    device memory of at least
 *              sv_verify_greedy_workspace_bytes(B, K, V) bytes, 8-byte
 *              aligned, owned by the caller, not used by another call that
 *              may run at the same time. Unlike the other workspaces it must
 *              hold ZEROS before its first use (e.g. hipMemset to 0) and be
 *              written by nothing but sv_verify_greedy and
 *              sv_verify_greedy_margin: every call leaves it all zero again,
 *              so no reset has to run before a launch. With it, each
 *              sequence's rows are split over workgroups (one 32 KB slice of
 *              each row per workgroup, up to 64) that exchange partial
 *              argmaxes, so a long chain of matches is read by many compute
 *              units (see sv_set_greedy_lookahead for how far ahead of its
 *              decision each reads); NULL or 0 bytes selects one workgroup per sequence
 *              (fewer bytes than the query returns is SV_ERR_WORKSPACE). The
 *              results are identical either way.
 * Result: n_accepted[b] in [0, K_b], next_token[b] in [0, V); bit-exact.
 * Errors: SV_ERR_INVALID_ARG for null required pointers, B < 0, K < 0,
 * K > SV_MAX_K, V < 1 or V > INT32_MAX, a bad dtype, misaligned pointers;
 * SV_ERR_WORKSPACE for an undersized workspace.
 */
sv_status sv_verify_greedy(const void* target, int dtype, int32_t B, int32_t K, int64_t V,
                           const int32_t* draft_tokens, const int32_t* draft_lens,
                           int32_t* n_accepted, int32_t* next_token, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Workspace bytes the split path of sv_verify_greedy and
 * sv_verify_greedy_margin uses for these sizes, for fp32 or bf16 rows alike
 * (0 when one workgroup per sequence is used regardless: rows of at most
 * 128 KB, i.e. V up to 32768, or invalid sizes). */
size_t sv_verify_greedy_workspace_bytes(int32_t B, int32_t K, int64_t V);

/*
 * sv_verify_greedy_margin -- sv_verify_greedy plus, per sequence, the top1 -
 * top2 margin of the row next_token is taken from (target row n_accepted[b]):
 * its largest value minus the largest of its other values, computed in fp32
 * (0 for a tied maximum, +inf when V == 1). A serving loop feeds it to the
 * pre-draft gate, which skips drafting when the target is unsure of the
 * committed token (PocketLLM DSpark notes, "gating": the top1 - top2 logit
 * margin of the committed token).
 * top2_margin  [B] fp32 output, 4-byte aligned, required.
 * Same arguments, results and errors as sv_verify_greedy otherwise.
 */
sv_status sv_verify_greedy_margin(const void* target, int dtype, int32_t B, int32_t K, int64_t V,
                                  const int32_t* draft_tokens, const int32_t* draft_lens,
                                  int32_t* n_accepted, int32_t* next_token, float* top2_margin,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Acceptance-driven draft-length gate (PocketLLM DSpark notes, "gating"), on
 * the device: the verify's n_accepted never has to reach the host.
 *
 * State: hits[B, NB] and trials[B, NB], fp64 device arrays owned by the
 * caller, zero-filled for a cold gate; bucket c of sequence b counts the
 * decayed acceptances and observations of the draft positions mapped to c
 * (the position itself when `buckets` is NULL, which needs NB >= K; or a
 * caller's confidence bucket, buckets[b, j] for position j, clamped into
 * [0, NB)).
 *
 * sv_gate_update records one verify round: for each sequence with
 * draft_lens[b] = kb > 0 (clamped to [0, K]; NULL means K), every count of b
 * is multiplied by `decay` in [0, 1], then positions j = 0 .. min(n, kb - 1)
 * with n = n_accepted[b] (clamped to [0, kb]) add 1 to trials, and 1 to hits
 * when j < n. Later positions were not observed (censored) and are not
 * recorded. A sequence without a draft is left unchanged.
 *
 * sv_gate_choose writes next_lens[b] in [0, K]: with p_j = hits / trials of
 * position j's bucket (1 when it has no trials, so a cold gate drafts and
 * learns), E(n) = 1 + sum_{i<n} prod_{j<=i} p_j, cost(0) = plain_ms and
 * cost(n) = draft_ms + verify_base_ms + verify_slope_ms * n, it takes
 * n* = argmax E(n) / cost(n) (ties to the longer draft); a truncation n* < K
 * only if it beats the full draft by the factor `margin`; at least
 * min(min_draft, K); and 0 when margin_threshold > 0, top2_margin is given
 * and top2_margin[b] < margin_threshold (skip the draft). All arithmetic is
 * IEEE fp64 in the order written, identical on every run.
 * params is a host pointer read during the call. The notes' defaults: draft
 * 196, verify 300 + 109 n, plain 303 (ms), margin 1.15, decay 0.9,
 * min_draft 0, margin_threshold 0 (off).
 * Errors: SV_ERR_INVALID_ARG for B < 0, NB < 1, K not in [0, SV_MAX_K],
 * NB < K without buckets, decay outside [0, 1], negative or non-finite
 * costs, plain_ms <= 0, margin <= 0, min_draft < 0, a non-finite
 * margin_threshold, null required pointers, misalignment.
 */
typedef struct {
    double draft_ms;         /* cost of drafting a block */
    double verify_base_ms;   /* fixed cost of a verify forward */
    double verify_slope_ms;  /* verify cost per draft token */
    double plain_ms;         /* cost of a plain single-token decode step */
    double margin;           /* a truncation must beat the full draft by this factor */
    int32_t min_draft;       /* never draft fewer than this (0: no floor) */
    float margin_threshold;  /* skip drafting below this top1 - top2 margin (0: off) */
} sv_gate_params;

sv_status sv_gate_update(double* hits, double* trials, int32_t B, int32_t NB, int32_t K,
                         const int32_t* draft_lens, const int32_t* n_accepted, const int32_t* buckets,
                         double decay, void* stream);

sv_status sv_gate_choose(const double* hits, const double* trials, int32_t B, int32_t NB, int32_t K,
                         const int32_t* buckets, const float* top2_margin, const sv_gate_params* params,
                         int32_t* next_lens, void* stream);

/*
 * sv_accept -- speculative-sampling verification.
 *
 * For i < K_b accept t_i iff u[b, i] < p_i(t_i) / q_i(t_i), i.e. with
 * probability min(1, p/q); stop at the first rejection n. If n < K_b draw
 * the correction from norm(max(0, p_n - q_n)); otherwise draw the bonus token
 * from p_{K_b} (spec-verify card, "Method"; llmstudio blog, sections 15-17
 * and 47). Both draws are inverse-CDF lookups with uniform u[b, K_b]: the
 * smallest x whose cumulative weight exceeds u * (total weight).
 *   - q_i(t_i) == 0 < p_i(t_i) accepts; p_i(t_i) == 0 rejects (even at u = 0).
 *   - The accept test is exact: it compares u * q < p in binary64.
 *   - Draw weights are summed in binary64, so rows need not be normalised
 *     (spec-verify card, "Correctness"); the accept ratio uses p and q as
 *     given, so distribution preservation assumes normalised rows warped
 *     identically (card, "Requirements and limits").
 *   - A residual with no positive mass (p_n == q_n) draws from max(0, p_n).
 *   - A final-draw row with no positive mass gives next_token = -1.
 * Only the gathered p_i(t_i), q_i(t_i) for i <= n and the one row (pair)
 * the final draw needs are read.
 *
 * target_probs [B, K+1, V] fp32, draft_probs [B, K, V] fp32, 4-byte aligned.
 * draft_tokens [B, K] int32 (may be NULL when K == 0), draft_lens [B] or NULL,
 * uniforms [B, K+1] fp32.
 * Result: ids and decisions agree exactly with an exact-arithmetic
 * evaluation except where u lies within ~1e-15 (relative) of a ratio or
 * cumulative-weight boundary.
 * Errors: SV_ERR_INVALID_ARG for null required pointers, B < 0, K < 0,
 * K > SV_MAX_K, V < 1 or V > INT32_MAX, misaligned pointers.
 */
sv_status sv_accept(const float* target_probs, const float* draft_probs, int32_t B, int32_t K,
                    int64_t V, const int32_t* draft_tokens, const int32_t* draft_lens,
                    const float* uniforms, int32_t* n_accepted, int32_t* next_token,
                    void* stream);

/*
 * sv_accept_logits -- speculative-sampling verification straight from logits.
 *
 * The result sv_accept gives on p = softmax(target_logits / T) and
 * q = softmax(draft_logits / T) (the verify compares the distributions after
 * the sampler's temperature step: llmstudio blog, sections 21-22 and 38;
 * spec-verify card, "Method"), without writing any probability row: each
 * position's target and draft rows are reduced to their softmax statistics
 * in one pass, p_i(t_i) and q_i(t_i) follow from the two logits at t_i, and
 * the correction or bonus row is re-derived from its logits for the draw.
 * Rows after a sequence's first rejection are never read, so a round reads
 * about (n_b + 2) row pairs per sequence instead of all of them twice.
 *
 * target_logits [B, K+1, V], draft_logits [B, K, V] of `dtype` (SV_F32 or
 * SV_BF16), element-aligned; draft_tokens, draft_lens, uniforms, outputs as
 * for sv_accept; temperature finite, > 0.
 * workspace    device memory of at least sv_accept_logits_workspace_bytes(B,
 *              K, V) bytes, 8-byte aligned, owned by the caller, contents
 *              irrelevant (initialised on `stream`): the slots in which the
 *              workgroups sharing a sequence's rows exchange partial
 *              statistics. With it each sequence's rows are split over
 *              several workgroups (a long chain of accepted positions runs on
 *              several compute units); NULL or 0 bytes (and any workspace
 *              when the query returns 0) selects one workgroup per sequence;
 *              fewer bytes than the query returns is SV_ERR_WORKSPACE.
 *              Results are identical either way up to the rounding of the
 *              partial sums.
 *              Calls that overlap in time must not share a workspace.
 * Accuracy: the row masses come from fp32 exponentials with fp64 sums
 * (relative error about 1e-7); the accept ratio p(t)/q(t) and every residual
 * weight p(x) * (1 - q(x)/p(x)) take q/p from the exact logit difference, so
 * both carry relative errors of a few 1e-7 and a cumulative weight carries
 * about 1e-7 of the target mass before it. Decisions and ids agree with an
 * exact evaluation except where u lies within ~1e-5 relative of a ratio or
 * cumulative-weight boundary. Bitwise identical run to run.
 * Errors: as sv_accept, plus SV_ERR_INVALID_ARG for a bad dtype or temperature.
 */
sv_status sv_accept_logits(const void* target_logits, const void* draft_logits, int dtype, int32_t B, int32_t K,
                           int64_t V, float temperature, const int32_t* draft_tokens, const int32_t* draft_lens,
                           const float* uniforms, int32_t* n_accepted, int32_t* next_token, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Workspace bytes sv_accept_logits and sv_accept_logits_lse use for these
 * sizes, the larger need of the two dtypes (0 when they use one workgroup per
 * sequence regardless: rows that fit one slice of 6144 fp32 or 12288 bf16
 * logits in either dtype, or need more than 64 slices in both). */
size_t sv_accept_logits_workspace_bytes(int32_t B, int32_t K, int64_t V);

/*
 * sv_accept_logits_lse -- sv_accept_logits with each draft row's distribution
 * given by its normaliser, for callers whose draft model has it already (it
 * computes the normaliser when it samples t_i from the row).
 *
 * The pages define q_i as the draft model's distribution at position i, the
 * one t_i was sampled from (spec-verify card, "Method"; llmstudio blog,
 * sections 15-17 and 21-22). Here it is
 *   q_i(x) = exp(draft_logits[b, i, x] / T - draft_lse[b, i]),
 * taken as given, in the accept ratio and in the residual alike. With the
 * row's true log-sum-exp, log sum_x exp(draft_logits[b, i, x] / T), the result
 * is sv_accept_logits' up to the rounding of the value passed in (relative
 * |lse| * 6e-8 on q); a different value scales q_i, and the verify follows
 * that scaled q_i. Only the target rows' statistics are computed: a draft row
 * is read at the accept test's one logit z_d,i(t_i) per examined position,
 * and whole only at the rejected position (for the residual), so a round
 * reads about (n_b + 1) target rows and one draft row per sequence.
 *
 * draft_lse    device fp32 [B, K], row-major (position i of sequence b at
 *              b * K + i), borrowed: the natural-log normaliser of draft row
 *              (b, i) at `temperature`. Entries past K_b are not read. Not
 *              finite: +inf (q_i = 0) and NaN (q_i NaN, not positive) accept
 *              t_i unless p_i(t_i) = 0; -inf (q_i = +inf) rejects it. A
 *              rejection at a position whose entry is not finite draws from
 *              max(0, p_n) (no residual mass).
 *              May be null only when B == 0 or K == 0. 4-byte aligned.
 * Every other argument, the workspace and the accuracy are as for
 * sv_accept_logits.
 * Errors: as sv_accept_logits, plus SV_ERR_INVALID_ARG for a null draft_lse
 * when K > 0.
 */
sv_status sv_accept_logits_lse(const void* target_logits, const void* draft_logits, int dtype, int32_t B, int32_t K,
                               int64_t V, float temperature, const float* draft_lse, const int32_t* draft_tokens,
                               const int32_t* draft_lens, const float* uniforms, int32_t* n_accepted,
                               int32_t* next_token, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sv_commit -- append one verify round to each sequence's token buffer on the
 * device: draft_tokens[b, :n] followed by next_token[b], n = n_accepted[b]
 * clamped to [0, K] (spec-verify card, "Usage": keep draft_tokens[:n_accepted],
 * append next_token). Lets a draft/verify loop keep its buffers in HBM.
 * seq       [B, cap] int32 token buffers; sequence b holds seq_len[b] tokens.
 * seq_len   [B] int32, updated.
 * done      [B] int32 flags, updated: a sequence is done once it reaches
 *           min(limit[b], cap) tokens, or right after committing `eos` (when
 *           eos >= 0); a done sequence is left unchanged by later calls.
 * limit     [B] int32 length limits, or NULL (cap for every sequence).
 * Tokens past the limit are dropped. All pointers are device memory.
 * Errors: SV_ERR_INVALID_ARG for B < 0, cap < 1, K not in [0, SV_MAX_K],
 * B*cap > INT32_MAX, null required pointers, misalignment.
 */
sv_status sv_commit(int32_t* seq, int32_t* seq_len, int32_t* done, int32_t B, int32_t cap,
                    const int32_t* draft_tokens, int32_t K, const int32_t* n_accepted,
                    const int32_t* next_token, const int32_t* limit, int32_t eos, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
