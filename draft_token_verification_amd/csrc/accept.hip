// accept.hip -- speculative-sampling verification for gfx950.
//
// Method (spec-verify card, "Method"; llmstudio blog "Как работает
// speculative decoding и MTP при инференсе LLM", sections 15-17 and 47):
// for i < K_b accept t_i with probability min(1, p_i(t_i)/q_i(t_i)), i.e. iff
// u[b,i] < p/q; stop at the first rejection n. If n < K_b draw the correction
// from norm(max(0, p_n - q_n)), else draw the bonus from p_{K_b}. The draw is
// the inverse CDF at u[b, K_b]: the smallest x whose cumulative weight
// exceeds u * S, S the total weight.
//
// Mapping: one workgroup (1024 lanes) per sequence.
//  1. Gather and decide (wavefront 0): lane i < K_b loads t_i, p_i(t_i),
//     q_i(t_i), u[b,i] and tests u*q < p in binary64 -- exact, since the
//     product of two binary32 values fits in binary64 -- so the ratio is never
//     rounded. A ballot over the lanes gives the first rejection n.
//  2. Segment sums (all 16 wavefronts): the one row pair the draw needs is
//     streamed once with 16-byte non-temporal loads; weights are formed and
//     summed in binary64 per 256*m-element segment (fixed DPP butterfly), and
//     the segment totals go to LDS.
//  3. Locate (wavefront 0): a carry-chained wave scan over the segment totals
//     finds the segment holding u*S; that single segment is re-read and
//     scanned in x order to find the id.
// Only the draw's row (pair) is read in full; gathers touch one value per
// tested position.
#include "common.hpp"
#include "launch.hpp"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 2;
constexpr int kSub = 4 * kWave;     // elements per sub-block: 4 per lane
constexpr int kMaxSeg = 7936;       // segment totals kept in LDS (62 KiB)

// The 4 elements x .. x+3 of p (and q): raw values, zero past V.
struct Raw4 {
    f32x4 p, q;
};

template <bool VEC>
__device__ __forceinline__ Raw4 load4(const float* p, const float* q, int64_t x, int V) {
    Raw4 r;
    r.q = f32x4{0.f, 0.f, 0.f, 0.f};
    if (VEC && x < V) {
        r.p = load_nt((const f32x4*)(p + x));
        if (q) r.q = load_nt((const f32x4*)(q + x));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r.p[j] = (x + j < V) ? p[x + j] : 0.f;
            if (q) r.q[j] = (x + j < V) ? q[x + j] : 0.f;
        }
    }
    return r;
}

// Weights of those elements, in binary64 (inputs widen exactly):
// q == nullptr: w = max(0, p) (bonus row); otherwise w = max(0, p - q) (residual).
__device__ __forceinline__ void weights4(const Raw4& r, bool resid, double w[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        double d = resid ? (double)r.p[j] - (double)r.q[j] : (double)r.p[j];
        w[j] = d > 0.0 ? d : 0.0;
    }
}

// Pass 2 of the draw: all wavefronts write seg[s] = sum of the weights of
// segment s (L = m * kSub elements). Returns the row's total weight S,
// identical in every lane (each wavefront sums seg[] in the same order).
template <bool VEC>
__device__ double segment_totals(const float* p, const float* q, int V, int m, int nseg, double* seg) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t L = (int64_t)m * kSub;
    for (int s0 = wave; s0 < nseg; s0 += kWaves * kUnroll) {
        double acc[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc[u] = 0.0;
        for (int k = 0; k < m; ++k) {
            Raw4 raw[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t x = (int64_t)(s0 + u * kWaves) * L + (int64_t)k * kSub + 4 * lane;
                raw[u] = load4<VEC>(p, q, x, V);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                double w[4];
                weights4(raw[u], q != nullptr, w);
                acc[u] += ((w[0] + w[1]) + w[2]) + w[3];
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const double tot = wave_sum_d(acc[u]);
            const int s = s0 + u * kWaves;
            if (lane == 0 && s < nseg) seg[s] = tot;
        }
    }
    __syncthreads();
    double part = 0.0;
    for (int s = lane; s < nseg; s += kWave) part += seg[s];
    return wave_sum_d(part);
}

// Smallest x with positive weight whose cumulative weight exceeds thr
// (wavefront 0 only). If rounding leaves no such x in the chosen segment,
// or u*S reaches S, the last positive-weight id is returned.
template <bool VEC>
__device__ int locate(const float* p, const float* q, int V, int m, int nseg, const double* seg, double thr) {
    const int lane = threadIdx.x & (kWave - 1);
    // segment level: first s with seg[s] > 0 and P(s) > thr
    double carry = 0.0, pexcl = 0.0;
    int sstar = -1, slast = -1;
    for (int c0 = 0; c0 < nseg; c0 += kWave) {
        const int s = c0 + lane;
        const double v = s < nseg ? seg[s] : 0.0;
        const double incl = wave_incl_scan_d(v, lane);
        double excl = __shfl_up(incl, 1, kWave);
        if (lane == 0) excl = 0.0;
        const uint64_t pos = __ballot(v > 0.0);
        if (pos) slast = c0 + 63 - __builtin_clzll(pos);
        const uint64_t hit = __ballot(v > 0.0 && carry + incl > thr);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            sstar = c0 + l;
            pexcl = carry + __shfl(excl, l, kWave);
            break;
        }
        carry = carry + readlane_d(incl, 63);
    }
    if (sstar < 0) {  // u*S at or beyond the total: last positive-weight id
        if (slast < 0) return -1;
        sstar = slast;
        thr = INFINITY;
    }
    // element level, in x order inside segment sstar
    const int64_t L = (int64_t)m * kSub;
    double cbase = pexcl;
    int last_pos = -1;
    for (int k = 0; k < m; ++k) {
        const int64_t x0 = (int64_t)sstar * L + (int64_t)k * kSub + 4 * lane;
        double w[4];
        weights4(load4<VEC>(p, q, x0, V), q != nullptr, w);
        const double p1 = w[0] + w[1], p2 = p1 + w[2], p3 = p2 + w[3];
        const double incl = wave_incl_scan_d(p3, lane);
        double excl = __shfl_up(incl, 1, kWave);
        if (lane == 0) excl = 0.0;
        const double base = cbase + excl;
        const double pref[4] = {w[0], p1, p2, p3};
        int cand = -1, lp = -1;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            if (w[j] > 0.0 && base + pref[j] > thr) cand = (int)(x0 + j);
            if (lp < 0 && w[j] > 0.0) lp = (int)(x0 + j);
        }
        const uint64_t hit = __ballot(cand >= 0);
        if (hit) return readlane_i(cand, __builtin_ctzll(hit));
        const uint64_t pos = __ballot(lp >= 0);
        if (pos) last_pos = readlane_i(lp, 63 - __builtin_clzll(pos));
        cbase = cbase + readlane_d(incl, 63);
    }
    return last_pos;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void accept_kernel(const float* __restrict__ p, const float* __restrict__ q,
                                                          int K, int V, int m, int nseg,
                                                          const int32_t* __restrict__ tokens,
                                                          const int32_t* __restrict__ lens,
                                                          const float* __restrict__ uniforms,
                                                          int32_t* __restrict__ n_accepted,
                                                          int32_t* __restrict__ next_token) {
    extern __shared__ double seg[];
    __shared__ int s_n;
    const int b = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int kb = clamp_len(lens, b, K);
    const int64_t Vl = V;

    // 1. gather p_i(t_i), q_i(t_i) and decide (lane i = position i)
    if (wave == 0) {
        bool rej = false;
        if (lane < kb) {
            const int t = tokens[(int64_t)b * K + lane];
            if (t < 0 || t >= V) {
                rej = true;  // out-of-range draft token: rejected, never dereferenced
            } else {
                const double pt = p[((int64_t)b * (K + 1) + lane) * Vl + t];
                const double qt = q[((int64_t)b * K + lane) * Vl + t];
                const double u = uniforms[(int64_t)b * (K + 1) + lane];
                rej = !(u * qt < pt);  // u < p/q without rounding the ratio
            }
        }
        const uint64_t mask = __ballot(rej);
        if (lane == 0) s_n = mask ? __builtin_ctzll(mask) : kb;
    }
    __syncthreads();
    const int n = s_n;

    // 2. the row (pair) of the final draw
    const float* prow;
    const float* qrow;
    if (n < kb) {
        prow = p + ((int64_t)b * (K + 1) + n) * Vl;
        qrow = q + ((int64_t)b * K + n) * Vl;
    } else {
        prow = p + ((int64_t)b * (K + 1) + kb) * Vl;
        qrow = nullptr;
    }
    double S = segment_totals<VEC>(prow, qrow, V, m, nseg, seg);
    if (!(S > 0.0) && qrow != nullptr) {
        // p_n == q_n leaves no residual mass: draw from max(0, p_n) instead
        __syncthreads();
        qrow = nullptr;
        S = segment_totals<VEC>(prow, qrow, V, m, nseg, seg);
    }
    if (wave != 0) return;

    // 3. inverse CDF at u[b, K_b]
    int next = -1;
    if (S > 0.0) {
        const double thr = (double)uniforms[(int64_t)b * (K + 1) + kb] * S;
        next = locate<VEC>(prow, qrow, V, m, nseg, seg, thr);
    }
    if (lane == 0) {
        n_accepted[b] = n;
        next_token[b] = next;
    }
}

}  // namespace

hipError_t launch_accept(const float* p, const float* q, int B, int K, int V, const int32_t* tokens,
                         const int32_t* lens, const float* uniforms, int32_t* n_accepted, int32_t* next_token,
                         hipStream_t stream) {
    // m sub-blocks per segment keep the segment count within the LDS table
    const int64_t per_seg_min = ((int64_t)V + kMaxSeg - 1) / kMaxSeg;
    const int m = (int)((per_seg_min + kSub - 1) / kSub);  // >= 1 since V >= 1
    const int64_t L = (int64_t)m * kSub;
    const int nseg = (int)(((int64_t)V + L - 1) / L);
    const size_t lds = (size_t)nseg * sizeof(double);
    const bool vec = (V % 4 == 0) && ((uintptr_t)p % 16 == 0) && ((uintptr_t)q % 16 == 0);
    if (vec)
        hipLaunchKernelGGL(accept_kernel<true>, dim3(B), dim3(kThreads), lds, stream, p, q, K, V, m, nseg, tokens, lens,
                           uniforms, n_accepted, next_token);
    else
        hipLaunchKernelGGL(accept_kernel<false>, dim3(B), dim3(kThreads), lds, stream, p, q, K, V, m, nseg, tokens,
                           lens, uniforms, n_accepted, next_token);
    return hipGetLastError();
}

}  // namespace sv
