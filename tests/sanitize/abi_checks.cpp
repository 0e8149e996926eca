// abi_checks.cpp -- drives the host side of libspecverify's C ABI under
// AddressSanitizer and UndefinedBehaviorSanitizer, with no GPU: every entry
// point with each kind of invalid argument its header documents (negative or
// oversized sizes, null required pointers, misalignment, bad dtypes and
// temperatures, undersized workspaces), which must be refused with the
// documented status before any device work, and the workspace-size queries
// over their whole argument range (the sizes that overflow 32-bit products
// included). Built host-only: the kernels' device code is not compiled, and
// nothing here reaches a launch. Exit status 0: every status was as
// documented and the sanitizers saw nothing. Test infrastructure only.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "specverify.h"

static int failures = 0;

static void expect(int got, int want, const char* what, int line) {
    const char* msg = sv_last_error();
    if (got != want) {
        std::fprintf(stderr, "line %d: %s returned %d (%s), expected %d\n", line, what, got, msg, want);
        ++failures;
    } else if (want != SV_OK && (msg == nullptr || std::strlen(msg) == 0 || std::strlen(msg) >= 512)) {
        std::fprintf(stderr, "line %d: %s: no message for status %d\n", line, what, got);
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

alignas(256) static unsigned char host_buf[1 << 16];  // stands in for device memory: never dereferenced

int main() {
    const int INV = SV_ERR_INVALID_ARG, WS = SV_ERR_WORKSPACE;
    void* a = host_buf;                 // aligned
    void* mis2 = host_buf + 1;          // misaligned for any element
    void* mis4 = host_buf + 2;          // 2-byte aligned only
    float* f = (float*)host_buf;
    int32_t* i32 = (int32_t*)host_buf;
    double* d = (double*)host_buf;
    const float nan = std::nanf("");

    if (sv_abi_version() != SV_ABI_VERSION) ++failures;
    for (int s = -1; s <= 5; ++s)
        if (sv_status_string(s) == nullptr) ++failures;

    // ---- workspace-size queries, whole range ----
    const int32_t Bs[] = {INT_MIN, -1, 0, 1, 7, 2048, 2049, 1 << 20, INT_MAX};
    const int32_t Ks[] = {INT_MIN, -1, 0, 1, 16, 64, 65, INT_MAX};
    const int64_t Vs[] = {INT64_MIN, -1, 0, 1, 4096, 32768, 32769, 256000, 2097152, INT32_MAX, (int64_t)INT32_MAX + 1,
                          INT64_MAX};
    size_t sink = 0;
    for (int32_t B : Bs)
        for (int32_t K : Ks)
            for (int64_t V : Vs) {
                sink += sv_softmax_warp_workspace_bytes(B, K, V);
                sink += sv_verify_greedy_workspace_bytes(B, K, V);
                sink += sv_accept_logits_workspace_bytes(B, K, V);
            }
    for (int32_t B : Bs)
        for (int32_t cap : Bs) sink += sv_apply_penalties_workspace_bytes(B, cap);
    if (sv_softmax_warp_workspace_bytes(-1, 2, 100) != 0 || sv_apply_penalties_workspace_bytes(0, 10) != 0) ++failures;

    // ---- sv_softmax_warp and its allocation-free form ----
    EXPECT(sv_softmax_warp(a, 7, 1, 1, 8, nullptr, 0, 1.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(a, SV_F32, -1, 1, 8, nullptr, 0, 1.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(a, SV_F32, 1, 0, 8, nullptr, 0, 1.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(a, SV_F32, 1, 2, 8, nullptr, 3, 1.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(a, SV_F32, 1, 2, 0, nullptr, 0, 1.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(a, SV_F32, 1, 2, (int64_t)INT32_MAX + 1, nullptr, 0, 1.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(a, SV_F32, INT_MAX, 2, 8, nullptr, 0, 1.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(a, SV_F32, 1, 1, 8, nullptr, 0, 0.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(a, SV_F32, 1, 1, 8, nullptr, 0, nan, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(a, SV_F32, 1, 1, 8, nullptr, 0, INFINITY, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(nullptr, SV_F32, 1, 1, 8, nullptr, 0, 1.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(mis4, SV_F32, 1, 1, 8, nullptr, 0, 1.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(mis2, SV_BF16, 1, 1, 8, nullptr, 0, 1.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(a, SV_F32, 1, 1, 8, (const int32_t*)mis4, 0, 1.0f, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_softmax_warp(a, SV_F32, 0, 1, 8, nullptr, 0, 1.0f, nullptr, nullptr, 0, nullptr), SV_OK);  // empty
    {
        const size_t need = sv_softmax_warp_workspace_bytes(64, 5, 256000);
        EXPECT(sv_softmax_warp(a, SV_BF16, 64, 5, 256000, nullptr, 1, 1.0f, f, a, need - 8, nullptr), WS);
        EXPECT(sv_softmax_warp(a, SV_BF16, 64, 5, 256000, nullptr, 1, 1.0f, f, mis4, need, nullptr), INV);
    }
    EXPECT(sv_softmax_warp_noalloc(a, SV_F32, 1, 1, 8, nullptr, 0, -1.0f, f, nullptr), INV);
    EXPECT(sv_softmax_warp_noalloc(nullptr, SV_F32, 1, 1, 8, nullptr, 0, 1.0f, f, nullptr), INV);
    EXPECT(sv_softmax_warp_noalloc(a, SV_BF16, 100000, 5, 256000, nullptr, 1, 1.0f, f, nullptr), WS);
    EXPECT(sv_set_wait_limit(-1), INV);

    // ---- sv_softmax_warp_filtered ----
    EXPECT(sv_softmax_warp_filtered(a, SV_F32, 1, 0, 8, nullptr, 0, 1.0f, i32, f, f, nullptr), INV);
    EXPECT(sv_softmax_warp_filtered(a, SV_F32, 1, 1, 8, nullptr, 0, 1.0f, (const int32_t*)mis4, f, f, nullptr), INV);
    EXPECT(sv_softmax_warp_filtered(a, SV_F32, 1, 1, 8, nullptr, 0, 1.0f, i32, (const float*)mis4, f, nullptr), INV);
    EXPECT(sv_softmax_warp_filtered(a, SV_F32, 1, 1, 8, nullptr, 0, 1.0f, i32, f, nullptr, nullptr), INV);

    // ---- sv_apply_penalties ----
    sv_penalties pen{};
    pen.seq = i32;
    pen.seq_len = i32;
    pen.cap = 16;
    pen.draft_tokens = i32;
    pen.K = 4;
    EXPECT(sv_apply_penalties(a, SV_F32, 1, 5, 8, nullptr, 1, nullptr, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_apply_penalties(a, 3, 1, 5, 8, nullptr, 1, &pen, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_apply_penalties(a, SV_F32, 1, 5, 8, nullptr, 6, &pen, f, nullptr, 0, nullptr), INV);
    EXPECT(sv_apply_penalties(a, SV_F32, 1, 5, 8, nullptr, 1, &pen, nullptr, nullptr, 0, nullptr), INV);
    {
        sv_penalties p2 = pen;
        p2.cap = 0;
        EXPECT(sv_apply_penalties(a, SV_F32, 1, 5, 8, nullptr, 1, &p2, f, a, 1 << 16, nullptr), INV);
        p2 = pen;
        p2.seq_len = nullptr;
        EXPECT(sv_apply_penalties(a, SV_F32, 1, 5, 8, nullptr, 1, &p2, f, a, 1 << 16, nullptr), INV);
        p2 = pen;
        p2.K = 3;  // fewer draft tokens than the rows' prefixes need (R - 1 = 4)
        EXPECT(sv_apply_penalties(a, SV_F32, 1, 5, 8, nullptr, 1, &p2, f, a, 1 << 16, nullptr), INV);
        p2 = pen;
        p2.K = 65;
        EXPECT(sv_apply_penalties(a, SV_F32, 1, 5, 8, nullptr, 1, &p2, f, a, 1 << 16, nullptr), INV);
        p2 = pen;
        p2.repetition = (const float*)mis4;
        EXPECT(sv_apply_penalties(a, SV_F32, 1, 5, 8, nullptr, 1, &p2, f, a, 1 << 16, nullptr), INV);
        const size_t need = sv_apply_penalties_workspace_bytes(1, 16);
        EXPECT(sv_apply_penalties(a, SV_F32, 1, 5, 8, nullptr, 1, &pen, f, a, need - 4, nullptr), WS);
    }

    // ---- greedy verify, with and without the margin ----
    EXPECT(sv_verify_greedy(a, SV_F32, -1, 4, 8, i32, nullptr, i32, i32, nullptr, 0, nullptr), INV);
    EXPECT(sv_verify_greedy(a, SV_F32, 1, 65, 8, i32, nullptr, i32, i32, nullptr, 0, nullptr), INV);
    EXPECT(sv_verify_greedy(a, SV_F32, 1, -1, 8, i32, nullptr, i32, i32, nullptr, 0, nullptr), INV);
    EXPECT(sv_verify_greedy(a, SV_F32, 1, 4, 0, i32, nullptr, i32, i32, nullptr, 0, nullptr), INV);
    EXPECT(sv_verify_greedy(a, 5, 1, 4, 8, i32, nullptr, i32, i32, nullptr, 0, nullptr), INV);
    EXPECT(sv_verify_greedy(a, SV_F32, 1, 4, 8, nullptr, nullptr, i32, i32, nullptr, 0, nullptr), INV);
    EXPECT(sv_verify_greedy(a, SV_F32, 1, 4, 8, i32, nullptr, nullptr, i32, nullptr, 0, nullptr), INV);
    EXPECT(sv_verify_greedy(mis4, SV_F32, 1, 4, 8, i32, nullptr, i32, i32, nullptr, 0, nullptr), INV);
    EXPECT(sv_verify_greedy(a, SV_F32, 1, 4, 8, i32, (const int32_t*)mis4, i32, i32, nullptr, 0, nullptr), INV);
    {
        const size_t need = sv_verify_greedy_workspace_bytes(8, 4, 256000);
        EXPECT(sv_verify_greedy(a, SV_F32, 8, 4, 256000, i32, nullptr, i32, i32, a, need - 8, nullptr), WS);
        EXPECT(sv_verify_greedy(a, SV_F32, 8, 4, 256000, i32, nullptr, i32, i32, mis4, need, nullptr), INV);
    }
    EXPECT(sv_verify_greedy_margin(a, SV_F32, 1, 4, 8, i32, nullptr, i32, i32, nullptr, nullptr, 0, nullptr), INV);
    EXPECT(sv_verify_greedy_margin(a, SV_F32, 1, 4, 8, i32, nullptr, i32, i32, (float*)mis4, nullptr, 0, nullptr),
           INV);

    // ---- sampled verify ----
    EXPECT(sv_accept(f, f, -1, 4, 8, i32, nullptr, f, i32, i32, nullptr), INV);
    EXPECT(sv_accept(f, f, 1, 65, 8, i32, nullptr, f, i32, i32, nullptr), INV);
    EXPECT(sv_accept(f, f, 1, 4, 0, i32, nullptr, f, i32, i32, nullptr), INV);
    EXPECT(sv_accept(nullptr, f, 1, 4, 8, i32, nullptr, f, i32, i32, nullptr), INV);
    EXPECT(sv_accept(f, nullptr, 1, 4, 8, i32, nullptr, f, i32, i32, nullptr), INV);
    EXPECT(sv_accept(f, f, 1, 4, 8, i32, nullptr, nullptr, i32, i32, nullptr), INV);
    EXPECT(sv_accept((const float*)mis4, f, 1, 4, 8, i32, nullptr, f, i32, i32, nullptr), INV);
    EXPECT(sv_accept_logits(a, a, SV_F32, 1, 4, 8, 0.0f, i32, nullptr, f, i32, i32, nullptr, 0, nullptr), INV);
    EXPECT(sv_accept_logits(a, a, 9, 1, 4, 8, 1.0f, i32, nullptr, f, i32, i32, nullptr, 0, nullptr), INV);
    EXPECT(sv_accept_logits(a, nullptr, SV_F32, 1, 4, 8, 1.0f, i32, nullptr, f, i32, i32, nullptr, 0, nullptr), INV);
    EXPECT(sv_accept_logits(mis2, a, SV_BF16, 1, 4, 8, 1.0f, i32, nullptr, f, i32, i32, nullptr, 0, nullptr), INV);
    {
        const size_t need = sv_accept_logits_workspace_bytes(64, 8, 152064);
        EXPECT(sv_accept_logits(a, a, SV_F32, 64, 8, 152064, 1.0f, i32, nullptr, f, i32, i32, a, need - 8, nullptr),
               WS);
        // the form with given draft normalisers: the same checks, plus its own argument
        EXPECT(sv_accept_logits_lse(a, a, SV_F32, 1, 4, 8, 0.0f, f, i32, nullptr, f, i32, i32, nullptr, 0, nullptr),
               INV);
        EXPECT(sv_accept_logits_lse(a, a, SV_F32, 1, 4, 8, 1.0f, nullptr, i32, nullptr, f, i32, i32, nullptr, 0,
                                    nullptr), INV);
        EXPECT(sv_accept_logits_lse(a, a, SV_F32, 1, 4, 8, 1.0f, (const float*)mis2, i32, nullptr, f, i32, i32,
                                    nullptr, 0, nullptr), INV);
        EXPECT(sv_accept_logits_lse(a, a, SV_F32, 64, 8, 152064, 1.0f, f, i32, nullptr, f, i32, i32, a, need - 8,
                                    nullptr), WS);
        EXPECT(sv_accept_logits_lse(nullptr, nullptr, SV_F32, 0, 4, 8, 1.0f, nullptr, nullptr, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, 0, nullptr), SV_OK);
    }

    // ---- draft-length gate ----
    sv_gate_params gp{};
    gp.draft_ms = 1.0;
    gp.verify_base_ms = 5.0;
    gp.verify_slope_ms = 0.1;
    gp.plain_ms = 4.0;
    gp.margin = 0.0;
    EXPECT(sv_gate_update(d, d, -1, 4, 4, nullptr, i32, nullptr, 0.9, nullptr), INV);
    EXPECT(sv_gate_update(d, d, 1, 0, 4, nullptr, i32, nullptr, 0.9, nullptr), INV);
    EXPECT(sv_gate_update(d, d, 1, 4, 65, nullptr, i32, nullptr, 0.9, nullptr), INV);
    EXPECT(sv_gate_update(d, d, 1, 4, 4, nullptr, i32, nullptr, 1.5, nullptr), INV);
    EXPECT(sv_gate_update(d, d, 1, 4, 4, nullptr, i32, nullptr, nan, nullptr), INV);
    EXPECT(sv_gate_update(nullptr, d, 1, 4, 4, nullptr, i32, nullptr, 0.9, nullptr), INV);
    EXPECT(sv_gate_update((double*)mis4, d, 1, 4, 4, nullptr, i32, nullptr, 0.9, nullptr), INV);
    EXPECT(sv_gate_choose(d, d, 1, 4, 4, nullptr, nullptr, nullptr, i32, nullptr), INV);
    {
        sv_gate_params bad = gp;
        bad.plain_ms = 0.0;
        EXPECT(sv_gate_choose(d, d, 1, 4, 4, nullptr, nullptr, &bad, i32, nullptr), INV);
        bad = gp;
        bad.verify_base_ms = nan;
        EXPECT(sv_gate_choose(d, d, 1, 4, 4, nullptr, nullptr, &bad, i32, nullptr), INV);
        bad = gp;
        bad.min_draft = 5;
        EXPECT(sv_gate_choose(d, d, 1, 4, 4, nullptr, nullptr, &bad, i32, nullptr), INV);
    }
    EXPECT(sv_gate_choose(d, d, 1, 4, 4, nullptr, nullptr, &gp, nullptr, nullptr), INV);

    // ---- commit ----
    EXPECT(sv_commit(i32, i32, i32, -1, 16, i32, 4, i32, i32, nullptr, -1, nullptr), INV);
    EXPECT(sv_commit(i32, i32, i32, 1, 0, i32, 4, i32, i32, nullptr, -1, nullptr), INV);
    EXPECT(sv_commit(i32, i32, i32, 1, 16, i32, 65, i32, i32, nullptr, -1, nullptr), INV);
    EXPECT(sv_commit(i32, i32, i32, INT_MAX, 16, i32, 4, i32, i32, nullptr, -1, nullptr), INV);
    EXPECT(sv_commit(nullptr, i32, i32, 1, 16, i32, 4, i32, i32, nullptr, -1, nullptr), INV);
    EXPECT(sv_commit(i32, i32, i32, 1, 16, i32, 4, i32, i32, (const int32_t*)mis4, -1, nullptr), INV);

    std::printf("abi host checks: %d failures (size sink %zu)\n", failures, sink);
    return failures ? 1 : 0;
}
