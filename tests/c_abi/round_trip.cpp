// round_trip.cpp -- a caller of libspecverify through its C ABI alone, with no
// Python in between: a seeded batch of fp32 logits, the greedy verify, the
// sampled round (sv_softmax_warp on the target and the draft rows, then
// sv_accept), the same round fused (sv_accept_logits) and fused with the draft
// rows' normalisers given (sv_accept_logits_lse, the normalisers computed here
// as the draft model's sampler would), each checked against the fp64 oracle
// (oracle/sv_oracle.h, linked here as test infrastructure), then timed back to
// back with HIP events.
//
// usage: round_trip B K V seed reps
// Prints one JSON line; exits 1 on a mismatch, 2 on a library or HIP error.
// The sampled check exempts what the oracle flags within 1e-7 (relative) of
// a boundary: a ratio flag the whole sequence, a CDF flag its drawn id.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "specverify.h"
#include "sv_oracle.h"

namespace {

#define HIP_OK(x)                                                                          \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                   \
            std::exit(2);                                                                  \
        }                                                                                  \
    } while (0)

#define SV_OK(x)                                                                           \
    do {                                                                                   \
        sv_status s_ = (x);                                                                \
        if (s_ != SV_OK) {                                                                 \
            std::fprintf(stderr, "%s: %s (%s)\n", #x, sv_status_string(s_), sv_last_error()); \
            std::exit(2);                                                                  \
        }                                                                                  \
    } while (0)

// splitmix64: uniform 64-bit words from a seed (Steele, Lea and Flood, 2014)
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    double uniform() { return (double)(next() >> 11) * 0x1.0p-53; }  // [0, 1)
    double normal() {                                                 // Box-Muller
        const double u1 = 1.0 - uniform(), u2 = uniform();
        return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
    }
};

template <class T>
T* to_device(const std::vector<T>& h) {
    T* d = nullptr;
    HIP_OK(hipMalloc(&d, h.size() * sizeof(T) + 16));
    if (!h.empty()) HIP_OK(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
    return d;
}

template <class T>
std::vector<T> to_host(const T* d, size_t n) {
    std::vector<T> h(n);
    HIP_OK(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
    return h;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 6) {
        std::fprintf(stderr, "usage: %s B K V seed reps\n", argv[0]);
        return 2;
    }
    const int B = std::atoi(argv[1]), K = std::atoi(argv[2]), reps = std::atoi(argv[5]);
    const int64_t V = std::atoll(argv[3]);
    Rng rng{(uint64_t)std::atoll(argv[4])};
    const float T = 1.0f;
    if (B < 1 || K < 1 || K > SV_MAX_K || V < 2 || reps < 1) {
        std::fprintf(stderr, "need B >= 1, 1 <= K <= %d, V >= 2, reps >= 1\n", SV_MAX_K);
        return 2;
    }

    // target logits ~ N(0, 3^2); draft = target + N(0, 1); half of the sequences
    // draft the target's argmax chain, the rest random ids; ragged lengths
    std::vector<float> zt((size_t)B * (K + 1) * V), zd((size_t)B * K * V), u((size_t)B * (K + 1));
    std::vector<int32_t> tok((size_t)B * K), lens(B);
    for (auto& x : zt) x = (float)(3.0 * rng.normal());
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < K; ++i)
            for (int64_t x = 0; x < V; ++x) {
                const size_t o = ((size_t)b * K + i) * V + x;
                zd[o] = (float)(zt[((size_t)b * (K + 1) + i) * V + x] + rng.normal());
            }
    for (int b = 0; b < B; ++b) {
        lens[b] = (int32_t)(rng.next() % (uint64_t)(K + 1));
        for (int i = 0; i < K; ++i) {
            const float* row = &zt[((size_t)b * (K + 1) + i) * V];
            int64_t am = 0;
            for (int64_t x = 1; x < V; ++x)
                if (row[x] > row[am]) am = x;
            tok[(size_t)b * K + i] = (b % 2 == 0) ? (int32_t)am : (int32_t)(rng.next() % (uint64_t)V);
        }
    }
    for (auto& x : u) x = (float)rng.uniform();
    // each draft row's normaliser log sum_x exp(z / T), in binary64 (what the draft
    // model's sampler computes when it draws from the row)
    std::vector<float> lse((size_t)B * K);
    for (size_t r = 0; r < lse.size(); ++r) {
        const float* row = &zd[r * V];
        double m = -INFINITY, s = 0.0;
        for (int64_t x = 0; x < V; ++x) m = std::fmax(m, (double)row[x] / T);
        for (int64_t x = 0; x < V; ++x) s += std::exp((double)row[x] / T - m);
        lse[r] = (float)(m + std::log(s));
    }

    float *d_zt = to_device(zt), *d_zd = to_device(zd), *d_u = to_device(u), *d_lse = to_device(lse);
    int32_t *d_tok = to_device(tok), *d_lens = to_device(lens);
    int32_t *d_n = nullptr, *d_nx = nullptr;
    HIP_OK(hipMalloc(&d_n, B * sizeof(int32_t)));
    HIP_OK(hipMalloc(&d_nx, B * sizeof(int32_t)));
    float *d_p = nullptr, *d_q = nullptr;
    HIP_OK(hipMalloc(&d_p, zt.size() * sizeof(float)));
    HIP_OK(hipMalloc(&d_q, zd.size() * sizeof(float)));
    const size_t ws_g = sv_verify_greedy_workspace_bytes(B, K, V);
    const size_t ws_w = sv_softmax_warp_workspace_bytes(B, K + 1, V);
    const size_t ws_f = sv_accept_logits_workspace_bytes(B, K, V);
    void *d_wg = nullptr, *d_ww = nullptr, *d_wf = nullptr;
    if (ws_g) {
        HIP_OK(hipMalloc(&d_wg, ws_g));
        HIP_OK(hipMemset(d_wg, 0, ws_g));  // the greedy workspace holds zeros before its first use
    }
    if (ws_w) HIP_OK(hipMalloc(&d_ww, ws_w));
    if (ws_f) HIP_OK(hipMalloc(&d_wf, ws_f));  // contents irrelevant: the call initialises its slots
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));

    auto greedy = [&]() {
        SV_OK(sv_verify_greedy(d_zt, SV_F32, B, K, V, d_tok, d_lens, d_n, d_nx, d_wg, ws_g, st));
    };
    auto sampled = [&]() {
        SV_OK(sv_softmax_warp(d_zt, SV_F32, B, K + 1, V, d_lens, 1, T, d_p, d_ww, ws_w, st));
        SV_OK(sv_softmax_warp(d_zd, SV_F32, B, K, V, d_lens, 0, T, d_q, d_ww, ws_w, st));
        SV_OK(sv_accept(d_p, d_q, B, K, V, d_tok, d_lens, d_u, d_n, d_nx, st));
    };
    auto fused = [&]() {
        SV_OK(sv_accept_logits(d_zt, d_zd, SV_F32, B, K, V, T, d_tok, d_lens, d_u, d_n, d_nx, d_wf, ws_f, st));
    };
    auto fused_lse = [&]() {
        SV_OK(sv_accept_logits_lse(d_zt, d_zd, SV_F32, B, K, V, T, d_lse, d_tok, d_lens, d_u, d_n, d_nx, d_wf, ws_f,
                                   st));
    };
    // sampled results against the oracle's (1e-7 flags): a ratio flag exempts the
    // whole sequence, a CDF flag its drawn id
    auto sampled_diff = [&](const std::vector<int32_t>& n, const std::vector<int32_t>& nx,
                            const std::vector<int32_t>& n_o, const std::vector<int32_t>& nx_o,
                            const std::vector<int32_t>& fl, int& flagged) {
        int diff = 0;
        flagged = 0;
        for (int b = 0; b < B; ++b) {
            const bool ratio = fl[b] & OR_FLAG_RATIO, cdf = fl[b] & OR_FLAG_CDF;
            flagged += ratio || cdf;
            if (!ratio && (n[b] != n_o[b] || (!cdf && nx[b] != nx_o[b]))) ++diff;
        }
        return diff;
    };

    // parity
    std::vector<int32_t> n_o(B), nx_o(B), fl(B);
    greedy();
    HIP_OK(hipStreamSynchronize(st));
    std::vector<int32_t> n = to_host(d_n, B), nx = to_host(d_nx, B);
    or_verify_greedy(zt.data(), OR_F32, B, K, V, tok.data(), lens.data(), n_o.data(), nx_o.data());
    int greedy_diff = 0;
    for (int b = 0; b < B; ++b) greedy_diff += (n[b] != n_o[b]) || (nx[b] != nx_o[b]);
    sampled();
    HIP_OK(hipStreamSynchronize(st));
    n = to_host(d_n, B);
    nx = to_host(d_nx, B);
    or_accept_logits(zt.data(), zd.data(), OR_F32, B, K, V, T, tok.data(), lens.data(), u.data(), OR_F32, 1e-7,
                     n_o.data(), nx_o.data(), fl.data());
    int flagged = 0, flagged_lse = 0, unused = 0;
    const int sampled_d = sampled_diff(n, nx, n_o, nx_o, fl, flagged);
    fused();
    HIP_OK(hipStreamSynchronize(st));
    const int fused_d = sampled_diff(to_host(d_n, B), to_host(d_nx, B), n_o, nx_o, fl, unused);
    fused_lse();
    HIP_OK(hipStreamSynchronize(st));
    std::vector<int32_t> n_l(B), nx_l(B), fl_l(B);
    or_accept_logits_lse(zt.data(), zd.data(), OR_F32, B, K, V, T, lse.data(), tok.data(), lens.data(), u.data(),
                         OR_F32, 1e-7, n_l.data(), nx_l.data(), fl_l.data());
    const int fused_lse_d = sampled_diff(to_host(d_n, B), to_host(d_nx, B), n_l, nx_l, fl_l, flagged_lse);

    // latency: rounds issued back to back from C
    hipEvent_t e0, e1;
    HIP_OK(hipEventCreate(&e0));
    HIP_OK(hipEventCreate(&e1));
    auto time_us = [&](auto&& round) {
        for (int i = 0; i < 3; ++i) round();
        HIP_OK(hipEventRecord(e0, st));
        for (int i = 0; i < reps; ++i) round();
        HIP_OK(hipEventRecord(e1, st));
        HIP_OK(hipEventSynchronize(e1));
        float ms = 0.f;
        HIP_OK(hipEventElapsedTime(&ms, e0, e1));
        return 1000.0 * ms / reps;
    };
    const double g_us = time_us(greedy), s_us = time_us(sampled), f_us = time_us(fused), l_us = time_us(fused_lse);
    std::printf("{\"B\": %d, \"K\": %d, \"V\": %lld, \"greedy_round_us\": %.2f, \"sampled_round_us\": %.2f, "
                "\"fused_round_us\": %.2f, \"fused_lse_round_us\": %.2f, \"greedy_mismatches\": %d, "
                "\"sampled_mismatches\": %d, \"fused_mismatches\": %d, \"fused_lse_mismatches\": %d, "
                "\"sampled_flagged\": %d, \"fused_lse_flagged\": %d}\n",
                B, K, (long long)V, g_us, s_us, f_us, l_us, greedy_diff, sampled_d, fused_d, fused_lse_d, flagged,
                flagged_lse);
    return greedy_diff || sampled_d || fused_d || fused_lse_d ? 1 : 0;
}
