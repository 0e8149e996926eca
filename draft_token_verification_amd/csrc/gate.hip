// gate.hip -- acceptance-driven draft-length gate, on the device so that a
// serving loop never copies n_accepted to the host between rounds.
//
// Policy (PocketLLM DSpark notes, "gating"): keep decayed per-bucket counts of
// observed acceptances (a bucket is a draft position, or a caller's confidence
// bucket of it); record only the positions a round observed -- 0 .. n_accepted,
// since positions after the first rejection were verified but their match is
// unknown (censored); choose the next draft length maximising expected tokens
// per unit of cost,
//   E(n) = 1 + sum_{i<n} prod_{j<=i} p_j,  cost(0) = plain,
//   cost(n) = draft + verify_base + verify_slope * n,
// take a truncation only if it beats the full draft by the margin factor,
// never draft fewer than min_draft, and skip the draft when the committed
// token's top1 - top2 logit margin is below margin_threshold (when > 0).
// A bucket with no trials counts as acceptance 1, so a cold gate drafts the
// full block and learns; ties go to the longer draft.
//
// One thread per sequence; the work is O(NB + K) scalar fp64 per sequence.
// Floating-point contraction is off so that every decision is the IEEE result
// of the expressions as written.
#include "common.hpp"
#include "launch.hpp"

namespace sv {
namespace {

constexpr int kBlock = 64;

__device__ __forceinline__ int bucket_at(const int32_t* buckets, int b, int K, int j, int NB) {
    const int c = buckets ? buckets[(int64_t)b * K + j] : j;
    return c < 0 ? 0 : (c >= NB ? NB - 1 : c);
}

__global__ __launch_bounds__(kBlock) void gate_update_kernel(double* __restrict__ hits, double* __restrict__ trials,
                                                             int B, int NB, int K, const int32_t* __restrict__ lens,
                                                             const int32_t* __restrict__ n_accepted,
                                                             const int32_t* __restrict__ buckets, double decay) {
#pragma clang fp contract(off)
    const int b = blockIdx.x * kBlock + threadIdx.x;
    if (b >= B) return;
    const int kb = clamp_len(lens, b, K);
    if (kb == 0) return;  // no draft: nothing observed, nothing forgotten
    double* h = hits + (int64_t)b * NB;
    double* t = trials + (int64_t)b * NB;
    for (int c = 0; c < NB; ++c) {
        h[c] *= decay;
        t[c] *= decay;
    }
    const int na = n_accepted[b];
    const int n = na < 0 ? 0 : (na > kb ? kb : na);
    const int last = n < kb ? n : kb - 1;
    for (int j = 0; j <= last; ++j) {
        const int c = bucket_at(buckets, b, K, j, NB);
        t[c] += 1.0;
        if (j < n) h[c] += 1.0;
    }
}

__global__ __launch_bounds__(kBlock) void gate_choose_kernel(const double* __restrict__ hits,
                                                             const double* __restrict__ trials, int B, int NB, int K,
                                                             const int32_t* __restrict__ buckets,
                                                             const float* __restrict__ top2_margin, GateCosts g,
                                                             int32_t* __restrict__ next_lens) {
#pragma clang fp contract(off)
    const int b = blockIdx.x * kBlock + threadIdx.x;
    if (b >= B) return;
    const double* h = hits + (int64_t)b * NB;
    const double* t = trials + (int64_t)b * NB;
    double E = 1.0, prod = 1.0;
    double best = E / g.plain_ms, full = best;
    int nstar = 0;
    for (int n = 1; n <= K; ++n) {
        const int c = bucket_at(buckets, b, K, n - 1, NB);
        const double tr = t[c];
        const double p = tr > 0.0 ? h[c] / tr : 1.0;
        prod *= p;
        E += prod;
        const double r = E / (g.draft_ms + g.verify_base_ms + g.verify_slope_ms * (double)n);
        if (r >= best) {
            best = r;
            nstar = n;
        }
        if (n == K) full = r;
    }
    int len = nstar;
    if (nstar < K && !(best >= g.margin * full)) len = K;
    if (len < g.min_draft) len = g.min_draft > K ? K : g.min_draft;
    if (g.margin_threshold > 0.0 && top2_margin && (double)top2_margin[b] < g.margin_threshold) len = 0;
    next_lens[b] = len;
}

}  // namespace

hipError_t launch_gate_update(double* hits, double* trials, int B, int NB, int K, const int32_t* lens,
                              const int32_t* n_accepted, const int32_t* buckets, double decay, hipStream_t stream) {
    hipLaunchKernelGGL(gate_update_kernel, dim3((B + kBlock - 1) / kBlock), dim3(kBlock), 0, stream, hits, trials, B,
                       NB, K, lens, n_accepted, buckets, decay);
    return hipGetLastError();
}

hipError_t launch_gate_choose(const double* hits, const double* trials, int B, int NB, int K, const int32_t* buckets,
                              const float* top2_margin, const GateCosts& g, int32_t* next_lens, hipStream_t stream) {
    hipLaunchKernelGGL(gate_choose_kernel, dim3((B + kBlock - 1) / kBlock), dim3(kBlock), 0, stream, hits, trials, B,
                       NB, K, buckets, top2_margin, g, next_lens);
    return hipGetLastError();
}

}  // namespace sv
