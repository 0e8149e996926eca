// api.hip -- the C ABI of libspecverify (declared in include/specverify.h):
// argument validation, device check, kernel dispatch and error reporting.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "specverify.h"

namespace {

thread_local char g_last_error[512] = "";

sv_status fail(sv_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

sv_status ok() {
    g_last_error[0] = '\0';
    return SV_OK;
}

// The kernels are built for gfx950 only; refuse any other device up front.
constexpr int kMaxDevices = 64;
std::once_flag g_arch_once[kMaxDevices];
bool g_arch_ok[kMaxDevices];

sv_status check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(SV_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
    std::call_once(g_arch_once[dev], [dev] {
        hipDeviceProp_t prop;
        g_arch_ok[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                         std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    });
    if (!g_arch_ok[dev]) return fail(SV_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return SV_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t dtype_bytes(int dtype) { return dtype == SV_BF16 ? 2 : 4; }

sv_status check_dtype(int dtype) {
    if (dtype != SV_F32 && dtype != SV_BF16) return fail(SV_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    return SV_OK;
}

sv_status check_sizes(const char* fn, int32_t B, int32_t K, int64_t V) {
    if (B < 0) return fail(SV_ERR_INVALID_ARG, "%s: B = %d < 0", fn, B);
    if (K < 0 || K > SV_MAX_K) return fail(SV_ERR_INVALID_ARG, "%s: K = %d not in [0, %d]", fn, K, SV_MAX_K);
    if (V < 1 || V > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: V = %lld not in [1, 2^31-1]", fn, (long long)V);
    return SV_OK;
}

// A workspace of workspace_bytes > 0 must hold at least `need` bytes and be
// 8-byte aligned; workspace_bytes == 0 (or a null pointer) means none.
sv_status check_workspace(const char* fn, const void* workspace, size_t workspace_bytes, size_t need) {
    if (workspace == nullptr || workspace_bytes == 0) return SV_OK;
    if (workspace_bytes < need)
        return fail(SV_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed (pass 0 bytes for none)", fn,
                    workspace_bytes, need);
    if (!aligned(workspace, 8)) return fail(SV_ERR_INVALID_ARG, "%s: workspace not 8-byte aligned", fn);
    return SV_OK;
}

sv_status launched(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(SV_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

sv_status greedy_common(const char* fn, const void* target, int dtype, int32_t B, int32_t K, int64_t V,
                        const int32_t* draft_tokens, const int32_t* draft_lens, int32_t* n_accepted,
                        int32_t* next_token, float* top2_margin, bool want_margin, void* workspace,
                        size_t workspace_bytes, void* stream) {
    sv_status st;
    if ((st = check_dtype(dtype)) != SV_OK) return st;
    if ((st = check_sizes(fn, B, K, V)) != SV_OK) return st;
    if (B == 0) return ok();
    if (!target || !n_accepted || !next_token || (K > 0 && !draft_tokens) || (want_margin && !top2_margin))
        return fail(SV_ERR_INVALID_ARG, "%s: null required pointer", fn);
    if (!aligned(target, dtype_bytes(dtype)) || !aligned(n_accepted, 4) || !aligned(next_token, 4) ||
        (draft_tokens && !aligned(draft_tokens, 4)) || (draft_lens && !aligned(draft_lens, 4)) ||
        (top2_margin && !aligned(top2_margin, 4)))
        return fail(SV_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if ((st = check_workspace(fn, workspace, workspace_bytes, sv::greedy_workspace_bytes(B, K, (int)V))) != SV_OK)
        return st;
    if ((st = check_device()) != SV_OK) return st;
    return launched(fn, sv::launch_greedy(target, dtype == SV_BF16, B, K, (int)V, draft_tokens, draft_lens, n_accepted,
                                          next_token, top2_margin, workspace, workspace_bytes, (hipStream_t)stream));
}

}  // namespace

static_assert(sizeof(sv_gate_params) == 48, "sv_gate_params layout: five doubles, an int32 and a float");
static_assert(sizeof(sv_penalties) == 64, "sv_penalties layout: pointers and two int32 strides");

extern "C" {

int sv_abi_version(void) { return SV_ABI_VERSION; }

const char* sv_status_string(int status) {
    switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_INVALID_ARG: return "SV_ERR_INVALID_ARG: an argument is out of range, null or misaligned";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED: the current device is not gfx950";
    case SV_ERR_HIP: return "SV_ERR_HIP: the HIP runtime reported an error";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE: the workspace is smaller than the call needs";
    default: return "unknown sv_status";
    }
}

const char* sv_last_error(void) { return g_last_error; }

size_t sv_softmax_warp_workspace_bytes(int32_t B, int32_t R, int64_t V) {
    if (B < 1 || R < 1 || V < 1 || V > INT32_MAX || (int64_t)B * R > INT32_MAX) return 0;
    return sv::warp_workspace_bytes(B, R, (int)V);
}

sv_status sv_set_wait_limit(int32_t polls) {
    if (polls < 0) return fail(SV_ERR_INVALID_ARG, "sv_set_wait_limit: polls = %d < 0", polls);
    sv::set_wait_limit(polls);
    return ok();
}

sv_status sv_set_greedy_lookahead(int32_t rows) {
    if (rows < 0 || rows > SV_MAX_K + 1)
        return fail(SV_ERR_INVALID_ARG, "sv_set_greedy_lookahead: rows = %d outside [0, %d]", rows, SV_MAX_K + 1);
    sv::set_greedy_lookahead(rows);
    return ok();
}

sv_status sv_softmax_warp(const void* logits, int dtype, int32_t B, int32_t R, int64_t V, const int32_t* draft_lens,
                          int32_t extra_rows, float temperature, float* probs, void* workspace, size_t workspace_bytes,
                          void* stream) {
    const char* fn = "sv_softmax_warp";
    sv_status st;
    if ((st = check_dtype(dtype)) != SV_OK) return st;
    if (B < 0) return fail(SV_ERR_INVALID_ARG, "%s: B = %d < 0", fn, B);
    if (R < 1) return fail(SV_ERR_INVALID_ARG, "%s: R = %d < 1", fn, R);
    if (extra_rows < 0 || extra_rows > R)
        return fail(SV_ERR_INVALID_ARG, "%s: extra_rows = %d not in [0, R]", fn, extra_rows);
    if (V < 1 || V > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: V = %lld not in [1, 2^31-1]", fn, (long long)V);
    if ((int64_t)B * R > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: B*R exceeds 2^31-1 rows", fn);
    if (!(temperature > 0.0f) || !std::isfinite(temperature))
        return fail(SV_ERR_INVALID_ARG, "%s: temperature %g must be finite and > 0", fn, (double)temperature);
    if (B == 0) return ok();
    if (!logits || !probs) return fail(SV_ERR_INVALID_ARG, "%s: null logits or probs", fn);
    if (!aligned(logits, dtype_bytes(dtype)) || !aligned(probs, 4) || (draft_lens && !aligned(draft_lens, 4)))
        return fail(SV_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if ((st = check_workspace(fn, workspace, workspace_bytes, sv::warp_workspace_bytes(B, R, (int)V))) != SV_OK)
        return st;
    if ((st = check_device()) != SV_OK) return st;
    return launched(fn, sv::launch_warp(logits, dtype == SV_BF16, B, R, (int)V, draft_lens, extra_rows, temperature,
                                        probs, workspace, workspace_bytes, (hipStream_t)stream));
}

sv_status sv_softmax_warp_noalloc(const void* logits, int dtype, int32_t B, int32_t R, int64_t V,
                                  const int32_t* draft_lens, int32_t extra_rows, float temperature, float* probs,
                                  void* stream) {
    static_assert(sv::kStaticScratchBytes == SV_NOALLOC_SCRATCH_BYTES, "header and library disagree on the scratch size");
    const char* fn = "sv_softmax_warp_noalloc";
    sv_status st;
    if ((st = check_dtype(dtype)) != SV_OK) return st;
    if (B < 0) return fail(SV_ERR_INVALID_ARG, "%s: B = %d < 0", fn, B);
    if (R < 1) return fail(SV_ERR_INVALID_ARG, "%s: R = %d < 1", fn, R);
    if (extra_rows < 0 || extra_rows > R)
        return fail(SV_ERR_INVALID_ARG, "%s: extra_rows = %d not in [0, R]", fn, extra_rows);
    if (V < 1 || V > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: V = %lld not in [1, 2^31-1]", fn, (long long)V);
    if ((int64_t)B * R > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: B*R exceeds 2^31-1 rows", fn);
    if (!(temperature > 0.0f) || !std::isfinite(temperature))
        return fail(SV_ERR_INVALID_ARG, "%s: temperature %g must be finite and > 0", fn, (double)temperature);
    if (B == 0) return ok();
    if (!logits || !probs) return fail(SV_ERR_INVALID_ARG, "%s: null logits or probs", fn);
    if (!aligned(logits, dtype_bytes(dtype)) || !aligned(probs, 4) || (draft_lens && !aligned(draft_lens, 4)))
        return fail(SV_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    const size_t need = sv::warp_workspace_bytes(B, R, (int)V);
    if (need > sv::kStaticScratchBytes)
        return fail(SV_ERR_WORKSPACE, "%s: %d x %d rows of %lld need %zu bytes of exchange slots; the static scratch "
                    "holds %zu (use sv_softmax_warp with a workspace)", fn, B, R, (long long)V, need,
                    sv::kStaticScratchBytes);
    if ((st = check_device()) != SV_OK) return st;
    void* scratch = nullptr;
    const hipError_t e = sv::static_scratch(&scratch);
    if (e != hipSuccess) return fail(SV_ERR_HIP, "%s: hipGetSymbolAddress: %s", fn, hipGetErrorString(e));
    return launched(fn, sv::launch_warp(logits, dtype == SV_BF16, B, R, (int)V, draft_lens, extra_rows, temperature,
                                        probs, scratch, sv::kStaticScratchBytes, (hipStream_t)stream));
}

sv_status sv_softmax_warp_filtered(const void* logits, int dtype, int32_t B, int32_t R, int64_t V,
                                   const int32_t* draft_lens, int32_t extra_rows, float temperature,
                                   const int32_t* top_k, const float* top_p, float* probs, void* stream) {
    const char* fn = "sv_softmax_warp_filtered";
    sv_status st;
    if ((st = check_dtype(dtype)) != SV_OK) return st;
    if (B < 0) return fail(SV_ERR_INVALID_ARG, "%s: B = %d < 0", fn, B);
    if (R < 1) return fail(SV_ERR_INVALID_ARG, "%s: R = %d < 1", fn, R);
    if (extra_rows < 0 || extra_rows > R)
        return fail(SV_ERR_INVALID_ARG, "%s: extra_rows = %d not in [0, R]", fn, extra_rows);
    if (V < 1 || V > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: V = %lld not in [1, 2^31-1]", fn, (long long)V);
    if ((int64_t)B * R > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: B*R exceeds 2^31-1 rows", fn);
    if (!(temperature > 0.0f) || !std::isfinite(temperature))
        return fail(SV_ERR_INVALID_ARG, "%s: temperature %g must be finite and > 0", fn, (double)temperature);
    if (B == 0) return ok();
    if (!logits || !probs) return fail(SV_ERR_INVALID_ARG, "%s: null logits or probs", fn);
    if (!aligned(logits, dtype_bytes(dtype)) || !aligned(probs, 4) || (draft_lens && !aligned(draft_lens, 4)) ||
        (top_k && !aligned(top_k, 4)) || (top_p && !aligned(top_p, 4)))
        return fail(SV_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if ((st = check_device()) != SV_OK) return st;
    return launched(fn, sv::launch_warp_filtered(logits, dtype == SV_BF16, B, R, (int)V, draft_lens, extra_rows,
                                                 temperature, top_k, top_p, probs, (hipStream_t)stream));
}

size_t sv_apply_penalties_workspace_bytes(int32_t B, int32_t cap) { return sv::penalty_workspace_bytes(B, cap); }

sv_status sv_apply_penalties(const void* logits, int dtype, int32_t B, int32_t R, int64_t V, const int32_t* draft_lens,
                             int32_t extra_rows, const sv_penalties* pen, float* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
    const char* fn = "sv_apply_penalties";
    sv_status st;
    if ((st = check_dtype(dtype)) != SV_OK) return st;
    if (B < 0) return fail(SV_ERR_INVALID_ARG, "%s: B = %d < 0", fn, B);
    if (R < 1) return fail(SV_ERR_INVALID_ARG, "%s: R = %d < 1", fn, R);
    if (extra_rows < 0 || extra_rows > R)
        return fail(SV_ERR_INVALID_ARG, "%s: extra_rows = %d not in [0, R]", fn, extra_rows);
    if (V < 1 || V > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: V = %lld not in [1, 2^31-1]", fn, (long long)V);
    if ((int64_t)B * R > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: B*R exceeds 2^31-1 rows", fn);
    if (!pen) return fail(SV_ERR_INVALID_ARG, "%s: null pen", fn);
    const sv_penalties& p = *pen;
    if (p.seq && !p.seq_len) return fail(SV_ERR_INVALID_ARG, "%s: seq without seq_len", fn);
    if (p.seq && p.cap < 1) return fail(SV_ERR_INVALID_ARG, "%s: cap = %d < 1", fn, p.cap);
    if (p.seq && (int64_t)B * p.cap > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: B*cap exceeds 2^31-1", fn);
    if (p.draft_tokens && (p.K < R - 1 || p.K > SV_MAX_K))
        return fail(SV_ERR_INVALID_ARG, "%s: K = %d must be in [R - 1, %d] with draft_tokens", fn, p.K, SV_MAX_K);
    if (B == 0) return ok();
    if (!logits || !out) return fail(SV_ERR_INVALID_ARG, "%s: null logits or out", fn);
    if (!aligned(logits, dtype_bytes(dtype)) || !aligned(out, 4) || (draft_lens && !aligned(draft_lens, 4)) ||
        (p.seq && !aligned(p.seq, 4)) || (p.seq_len && !aligned(p.seq_len, 4)) ||
        (p.draft_tokens && !aligned(p.draft_tokens, 4)) || (p.repetition && !aligned(p.repetition, 4)) ||
        (p.presence && !aligned(p.presence, 4)) || (p.frequency && !aligned(p.frequency, 4)))
        return fail(SV_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if (p.seq) {
        const size_t need = sv::penalty_workspace_bytes(B, p.cap);
        if (!workspace || workspace_bytes < need)
            return fail(SV_ERR_WORKSPACE, "%s: the history tables need %zu bytes of workspace, %zu given", fn, need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 4)) return fail(SV_ERR_INVALID_ARG, "%s: workspace not 4-byte aligned", fn);
    }
    if ((st = check_device()) != SV_OK) return st;
    return launched(fn, sv::launch_penalties(logits, dtype == SV_BF16, B, R, (int)V, draft_lens, extra_rows, p.seq,
                                             p.seq_len, p.cap, p.draft_tokens, p.K, p.repetition, p.presence,
                                             p.frequency, out, workspace, (hipStream_t)stream));
}

size_t sv_verify_greedy_workspace_bytes(int32_t B, int32_t K, int64_t V) {
    if (B < 1 || K < 0 || K > SV_MAX_K || V < 1 || V > INT32_MAX) return 0;
    return sv::greedy_workspace_bytes(B, K, (int)V);
}

sv_status sv_verify_greedy(const void* target, int dtype, int32_t B, int32_t K, int64_t V,
                           const int32_t* draft_tokens, const int32_t* draft_lens, int32_t* n_accepted,
                           int32_t* next_token, void* workspace, size_t workspace_bytes, void* stream) {
    return greedy_common("sv_verify_greedy", target, dtype, B, K, V, draft_tokens, draft_lens, n_accepted, next_token,
                         nullptr, false, workspace, workspace_bytes, stream);
}

sv_status sv_verify_greedy_margin(const void* target, int dtype, int32_t B, int32_t K, int64_t V,
                                  const int32_t* draft_tokens, const int32_t* draft_lens, int32_t* n_accepted,
                                  int32_t* next_token, float* top2_margin, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    return greedy_common("sv_verify_greedy_margin", target, dtype, B, K, V, draft_tokens, draft_lens, n_accepted,
                         next_token, top2_margin, true, workspace, workspace_bytes, stream);
}

sv_status sv_gate_update(double* hits, double* trials, int32_t B, int32_t NB, int32_t K, const int32_t* draft_lens,
                         const int32_t* n_accepted, const int32_t* buckets, double decay, void* stream) {
    const char* fn = "sv_gate_update";
    if (B < 0) return fail(SV_ERR_INVALID_ARG, "%s: B = %d < 0", fn, B);
    if (NB < 1) return fail(SV_ERR_INVALID_ARG, "%s: NB = %d < 1", fn, NB);
    if (K < 0 || K > SV_MAX_K) return fail(SV_ERR_INVALID_ARG, "%s: K = %d not in [0, %d]", fn, K, SV_MAX_K);
    if (!buckets && NB < K) return fail(SV_ERR_INVALID_ARG, "%s: NB = %d < K = %d with position buckets", fn, NB, K);
    if (!(decay >= 0.0 && decay <= 1.0)) return fail(SV_ERR_INVALID_ARG, "%s: decay %g not in [0, 1]", fn, decay);
    if ((int64_t)B * NB > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: B*NB exceeds 2^31-1", fn);
    if (B == 0) return ok();
    if (!hits || !trials || !n_accepted) return fail(SV_ERR_INVALID_ARG, "%s: null required pointer", fn);
    if (!aligned(hits, 8) || !aligned(trials, 8) || !aligned(n_accepted, 4) || (draft_lens && !aligned(draft_lens, 4)) ||
        (buckets && !aligned(buckets, 4)))
        return fail(SV_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    sv_status st;
    if ((st = check_device()) != SV_OK) return st;
    return launched(fn, sv::launch_gate_update(hits, trials, B, NB, K, draft_lens, n_accepted, buckets, decay,
                                               (hipStream_t)stream));
}

sv_status sv_gate_choose(const double* hits, const double* trials, int32_t B, int32_t NB, int32_t K,
                         const int32_t* buckets, const float* top2_margin, const sv_gate_params* params,
                         int32_t* next_lens, void* stream) {
    const char* fn = "sv_gate_choose";
    if (B < 0) return fail(SV_ERR_INVALID_ARG, "%s: B = %d < 0", fn, B);
    if (NB < 1) return fail(SV_ERR_INVALID_ARG, "%s: NB = %d < 1", fn, NB);
    if (K < 0 || K > SV_MAX_K) return fail(SV_ERR_INVALID_ARG, "%s: K = %d not in [0, %d]", fn, K, SV_MAX_K);
    if (!buckets && NB < K) return fail(SV_ERR_INVALID_ARG, "%s: NB = %d < K = %d with position buckets", fn, NB, K);
    if (!params) return fail(SV_ERR_INVALID_ARG, "%s: null params", fn);
    const sv_gate_params& p = *params;
    if (!(p.draft_ms >= 0.0 && p.verify_base_ms >= 0.0 && p.verify_slope_ms >= 0.0 && p.plain_ms > 0.0) ||
        !std::isfinite(p.draft_ms) || !std::isfinite(p.verify_base_ms) || !std::isfinite(p.verify_slope_ms) ||
        !std::isfinite(p.plain_ms) || !(p.draft_ms + p.verify_base_ms + p.verify_slope_ms > 0.0))
        return fail(SV_ERR_INVALID_ARG, "%s: costs must be finite, >= 0, plain_ms > 0 and a draft round > 0", fn);
    if (!(p.margin > 0.0) || !std::isfinite(p.margin)) return fail(SV_ERR_INVALID_ARG, "%s: margin %g", fn, p.margin);
    if (p.min_draft < 0) return fail(SV_ERR_INVALID_ARG, "%s: min_draft = %d < 0", fn, p.min_draft);
    if (!std::isfinite(p.margin_threshold))
        return fail(SV_ERR_INVALID_ARG, "%s: margin_threshold must be finite", fn);
    if ((int64_t)B * NB > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: B*NB exceeds 2^31-1", fn);
    if (B == 0) return ok();
    if (!hits || !trials || !next_lens) return fail(SV_ERR_INVALID_ARG, "%s: null required pointer", fn);
    if (!aligned(hits, 8) || !aligned(trials, 8) || !aligned(next_lens, 4) || (buckets && !aligned(buckets, 4)) ||
        (top2_margin && !aligned(top2_margin, 4)))
        return fail(SV_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    sv_status st;
    if ((st = check_device()) != SV_OK) return st;
    const sv::GateCosts g{p.draft_ms, p.verify_base_ms, p.verify_slope_ms, p.plain_ms,
                          p.margin,   p.min_draft,      (double)p.margin_threshold};
    return launched(fn, sv::launch_gate_choose(hits, trials, B, NB, K, buckets, top2_margin, g, next_lens,
                                               (hipStream_t)stream));
}

sv_status sv_commit(int32_t* seq, int32_t* seq_len, int32_t* done, int32_t B, int32_t cap, const int32_t* draft_tokens,
                    int32_t K, const int32_t* n_accepted, const int32_t* next_token, const int32_t* limit, int32_t eos,
                    void* stream) {
    const char* fn = "sv_commit";
    if (B < 0) return fail(SV_ERR_INVALID_ARG, "%s: B = %d < 0", fn, B);
    if (cap < 1) return fail(SV_ERR_INVALID_ARG, "%s: cap = %d < 1", fn, cap);
    if (K < 0 || K > SV_MAX_K) return fail(SV_ERR_INVALID_ARG, "%s: K = %d not in [0, %d]", fn, K, SV_MAX_K);
    if ((int64_t)B * cap > INT32_MAX) return fail(SV_ERR_INVALID_ARG, "%s: B*cap exceeds 2^31-1", fn);
    if (B == 0) return ok();
    if (!seq || !seq_len || !done || !n_accepted || !next_token || (K > 0 && !draft_tokens))
        return fail(SV_ERR_INVALID_ARG, "%s: null required pointer", fn);
    if (!aligned(seq, 4) || !aligned(seq_len, 4) || !aligned(done, 4) || !aligned(n_accepted, 4) ||
        !aligned(next_token, 4) || (draft_tokens && !aligned(draft_tokens, 4)) || (limit && !aligned(limit, 4)))
        return fail(SV_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    sv_status st;
    if ((st = check_device()) != SV_OK) return st;
    return launched(fn, sv::launch_commit(seq, seq_len, done, B, cap, draft_tokens, K, n_accepted, next_token, limit,
                                          eos, (hipStream_t)stream));
}

sv_status sv_accept(const float* target_probs, const float* draft_probs, int32_t B, int32_t K, int64_t V,
                    const int32_t* draft_tokens, const int32_t* draft_lens, const float* uniforms, int32_t* n_accepted,
                    int32_t* next_token, void* stream) {
    const char* fn = "sv_accept";
    sv_status st;
    if ((st = check_sizes(fn, B, K, V)) != SV_OK) return st;
    if (B == 0) return ok();
    if (!target_probs || !uniforms || !n_accepted || !next_token || (K > 0 && (!draft_probs || !draft_tokens)))
        return fail(SV_ERR_INVALID_ARG, "%s: null required pointer", fn);
    if (!aligned(target_probs, 4) || (draft_probs && !aligned(draft_probs, 4)) || !aligned(uniforms, 4) ||
        !aligned(n_accepted, 4) || !aligned(next_token, 4) || (draft_tokens && !aligned(draft_tokens, 4)) ||
        (draft_lens && !aligned(draft_lens, 4)))
        return fail(SV_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if ((st = check_device()) != SV_OK) return st;
    return launched(fn, sv::launch_accept(target_probs, draft_probs, B, K, (int)V, draft_tokens, draft_lens, uniforms,
                                          n_accepted, next_token, (hipStream_t)stream));
}

size_t sv_accept_logits_workspace_bytes(int32_t B, int32_t K, int64_t V) {
    if (B < 1 || K < 0 || K > SV_MAX_K || V < 1 || V > INT32_MAX) return 0;
    return sv::accept_logits_workspace_bytes(B, K, (int)V);
}

// The checks and launch shared by the two verify-from-logits entry points.
static sv_status accept_logits_common(const char* fn, const void* target_logits, const void* draft_logits, int dtype,
                               int32_t B, int32_t K, int64_t V, float temperature, const float* draft_lse,
                               bool lse_required, const int32_t* draft_tokens, const int32_t* draft_lens,
                               const float* uniforms, int32_t* n_accepted, int32_t* next_token, void* workspace,
                               size_t workspace_bytes, void* stream) {
    sv_status st;
    if ((st = check_dtype(dtype)) != SV_OK) return st;
    if ((st = check_sizes(fn, B, K, V)) != SV_OK) return st;
    if (!(temperature > 0.0f) || !std::isfinite(temperature))
        return fail(SV_ERR_INVALID_ARG, "%s: temperature %g must be finite and > 0", fn, (double)temperature);
    if (B == 0) return ok();
    if (!target_logits || !uniforms || !n_accepted || !next_token ||
        (K > 0 && (!draft_logits || !draft_tokens || (lse_required && !draft_lse))))
        return fail(SV_ERR_INVALID_ARG, "%s: null required pointer", fn);
    const size_t es = dtype_bytes(dtype);
    if (!aligned(target_logits, es) || (draft_logits && !aligned(draft_logits, es)) || !aligned(uniforms, 4) ||
        !aligned(n_accepted, 4) || !aligned(next_token, 4) || (draft_tokens && !aligned(draft_tokens, 4)) ||
        (draft_lens && !aligned(draft_lens, 4)) || (draft_lse && !aligned(draft_lse, 4)))
        return fail(SV_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
    if ((st = check_workspace(fn, workspace, workspace_bytes, sv::accept_logits_workspace_bytes(B, K, (int)V))) !=
        SV_OK)
        return st;
    if ((st = check_device()) != SV_OK) return st;
    return launched(fn, sv::launch_accept_logits(target_logits, draft_logits, dtype == SV_BF16, B, K, (int)V,
                                                 temperature, K > 0 ? draft_lse : nullptr, draft_tokens, draft_lens,
                                                 uniforms, n_accepted, next_token, workspace, workspace_bytes,
                                                 (hipStream_t)stream));
}

sv_status sv_accept_logits(const void* target_logits, const void* draft_logits, int dtype, int32_t B, int32_t K,
                           int64_t V, float temperature, const int32_t* draft_tokens, const int32_t* draft_lens,
                           const float* uniforms, int32_t* n_accepted, int32_t* next_token, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return accept_logits_common("sv_accept_logits", target_logits, draft_logits, dtype, B, K, V, temperature, nullptr,
                                false, draft_tokens, draft_lens, uniforms, n_accepted, next_token, workspace,
                                workspace_bytes, stream);
}

sv_status sv_accept_logits_lse(const void* target_logits, const void* draft_logits, int dtype, int32_t B, int32_t K,
                               int64_t V, float temperature, const float* draft_lse, const int32_t* draft_tokens,
                               const int32_t* draft_lens, const float* uniforms, int32_t* n_accepted,
                               int32_t* next_token, void* workspace, size_t workspace_bytes, void* stream) {
    return accept_logits_common("sv_accept_logits_lse", target_logits, draft_logits, dtype, B, K, V, temperature,
                                draft_lse, true, draft_tokens, draft_lens, uniforms, n_accepted, next_token,
                                workspace, workspace_bytes, stream);
}

}  // extern "C"
