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
// Two kernels, one workgroup (1024 lanes) per sequence, sharing the draw:
//
// accept_kernel -- p and q given as fp32 probability rows.
//  1. Gather and decide (wavefront 0): lane i < K_b loads t_i, p_i(t_i),
//     q_i(t_i), u[b,i] and tests u*q < p in binary64 -- exact, since the
//     product of two binary32 values fits in binary64 -- so the ratio is never
//     rounded. A ballot over the lanes gives the first rejection n.
//
// accept_logits_kernel -- p and q given as logits, warped on the fly: no
// probability row is ever written (the sampled verify needs the target
// distribution only at the positions it examines; blog, section 22).
//  1. For i = 0, 1, ... in order, one pass over target row i and draft row i
//     gives each row's log2-domain statistics (m, sum of 2^(y - m)), m an
//     integer at or above the row maximum (online, per lane, merged with DPP
//     and LDS); the ratio p_i(t_i)/q_i(t_i) follows from the difference of
//     the two logits at t_i and the two rows' statistics, and u < ratio is
//     tested in binary64. The loop stops at the first rejection, so rows
//     after it are never read. A residual weight is p(x) * (1 - q(x)/p(x))
//     with q(x)/p(x) again from the logit difference, so it keeps a small
//     relative error where the two rows nearly agree.
//
// The draw (both kernels):
//  2. Segment sums (all 16 wavefronts): the one row (pair) the draw needs is
//     streamed once; weights are formed and summed in binary64 per
//     256*m-element segment (fixed DPP butterfly) into an LDS table.
//  3. Locate (wavefront 0): a carry-chained wave scan over the segment totals
//     finds the segment holding u*S; that single segment is re-read and
//     scanned in x order to find the id.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kSub = 4 * kWave;     // elements per sub-block: 4 per lane
constexpr int kMaxSeg = 7936;       // segment totals kept in LDS (62 KiB)


__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- weight sources: 4 consecutive elements x .. x+3 per lane ------------
// load() issues the loads (zero / -inf past V, selected rather than branched
// on, so several loads stay in flight); weights() turns them into binary64
// draw weights.

// fp32 probability rows: w = max(0, p - q) (residual) or max(0, p) (q null).
template <bool VEC, bool D>
struct ProbSource {
    static constexpr int kUnroll = 2;  // segments in flight per wavefront (register budget)
    const float* p;
    const float* q;  // read only when D
    int V;
    struct Raw {
        f32x4 p, q;
    };
    // Loads are unconditional (from a clamped address) and the value is
    // selected afterwards, so no branch separates the loads in flight.
    __device__ Raw load(int64_t x) const {
        Raw r;
        r.q = f32x4{0.f, 0.f, 0.f, 0.f};
        if (VEC) {
            const bool in = x < V;
            const int64_t xs = in ? x : 0;
            const f32x4 zero{0.f, 0.f, 0.f, 0.f};
            const f32x4 a = load_nt((const f32x4*)(p + xs));
            r.p = in ? a : zero;
            if (D) {
                const f32x4 b = load_nt((const f32x4*)(q + xs));
                r.q = in ? b : zero;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool in = x + j < V;
                const int64_t xs = in ? x + j : 0;
                const float a = p[xs];
                r.p[j] = in ? a : 0.f;
                if (D) {
                    const float b = q[xs];
                    r.q[j] = in ? b : 0.f;
                }
            }
        }
        return r;
    }
    __device__ void weights(const Raw& r, double w[4]) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            double d = D ? (double)r.p[j] - (double)r.q[j] : (double)r.p[j];
            w[j] = d > 0.0 ? d : 0.0;
        }
    }
};

// Four consecutive logits: an 8-byte bf16 load or a 16-byte fp32 load.
template <bool BF16>
struct Logit4;

template <>
struct Logit4<true> {
    using Raw = u32x2;
    __device__ static Raw load(const void* row, int64_t x) { return *(const Raw*)((const uint16_t*)row + x); }
    __device__ static Raw neg_inf() { return Raw{0xFF80FF80u, 0xFF80FF80u}; }
    __device__ static void unpack(const Raw& r, float z[4]) {
        z[0] = bf16_lo(r[0]);
        z[1] = bf16_hi(r[0]);
        z[2] = bf16_lo(r[1]);
        z[3] = bf16_hi(r[1]);
    }
    __device__ static Raw pack(const float a[4]) {
        return Raw{(__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xFFFF0000u),
                   (__float_as_uint(a[2]) >> 16) | (__float_as_uint(a[3]) & 0xFFFF0000u)};
    }
    __device__ static float at(const void* row, int64_t i) { return bf16_at((const uint16_t*)row, i); }
};

template <>
struct Logit4<false> {
    using Raw = f32x4;
    __device__ static Raw load(const void* row, int64_t x) { return *(const Raw*)((const float*)row + x); }
    __device__ static Raw neg_inf() { return Raw{-INFINITY, -INFINITY, -INFINITY, -INFINITY}; }
    __device__ static void unpack(const Raw& r, float z[4]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) z[k] = r[k];
    }
    __device__ static Raw pack(const float a[4]) { return Raw{a[0], a[1], a[2], a[3]}; }
    __device__ static float at(const void* row, int64_t i) { return ((const float*)row)[i]; }
};

// Row statistics in the log2 domain: p(x) = 2^(z(x)*c - m) * inv, c = log2(e)/T.
struct RowStats {
    float m;
    double inv;
};

// The accept test u < p(t)/q(t) from the two logits at t. The ratio is formed
// from the logit difference rather than from p and q separately:
//   rho = 2^e * inv_t / inv_d,  e = (zt - zd) * c + m_d - m_t,
// with the difference of the two binary32 logits and its product with c
// taken in binary64 (exact up to one rounding) and the references m
// integral; 2^e is 2^(e - round(e)) in fp32 (within 2e-7 relative) scaled
// by an exact power of two. So rho carries about 2e-7 of relative error plus
// that of the two row masses S = 1/inv. A -inf target logit means p(t) = 0
// (reject); a -inf draft logit alone means q(t) = 0 < p(t) (accept).
__device__ __forceinline__ bool accepts(float zt, float zd, float c, const RowStats& st, const RowStats& sd,
                                        float u) {
    if (zt == -INFINITY) return false;
    if (zd == -INFINITY) return true;
    const double e = fma((double)zt - (double)zd, (double)c, (double)sd.m - (double)st.m);
    const double ei = rint(fmin(fmax(e, -4096.0), 4096.0));  // beyond the binary64 range either way
    const double two_e = __builtin_ldexp((double)ex2((float)(e - ei)), (int)ei);
    return (double)u < two_e * (st.inv / sd.inv);
}

// Statistics of a draft row given by its natural-log normaliser lse at
// temperature T (the draft model computes it when it samples from the row):
// in the kernels' log2 domain (y = z * c, c = log2(e) / T) the row's mass is
// 2^L with L = lse * log2(e), so m = ceil(L) and 1/inv = 2^(L - m). Finite
// lse only.
__device__ __forceinline__ RowStats given_stats(float lse) {
    const double L = (double)lse * 1.4426950408889634;
    const float m = (float)ceil(L);
    return RowStats{m, exp2((double)m - L)};
}

// The accept test with a given draft normaliser lse. Not finite: +inf makes
// q = 0 and NaN makes q NaN, neither positive, so the ratio is +inf (accept
// unless p(t) = 0); -inf makes q = +inf, so the ratio is 0 (reject).
__device__ __forceinline__ bool accepts_given(float zt, float zd, float c, const RowStats& st, float lse, float u) {
    if (lse == INFINITY || lse != lse) return zt != -INFINITY;
    if (lse == -INFINITY) return false;
    return accepts(zt, zd, c, st, given_stats(lse), u);
}

// 1 - 2^y for y < 0, with a relative error of a few 1e-7 everywhere: a
// series in t = y ln 2 near 0 (|t| <= 0.18, truncated after t^6 / 6!, whose
// remainder is below 1e-8 relative) and 1 - exp2(y) below, where the result
// is at least 0.16.
__device__ __forceinline__ float one_minus_exp2(float y) {
    const float t = y * 0.69314718f;
    float s = 1.0f / 720.0f;
    s = fmaf(s, t, 1.0f / 120.0f);
    s = fmaf(s, t, 1.0f / 24.0f);
    s = fmaf(s, t, 1.0f / 6.0f);
    s = fmaf(s, t, 0.5f);
    s = fmaf(s, t, 1.0f);
    const float near0 = -t * s;
    return y < -0.25f ? 1.0f - ex2(y) : near0;
}

// log2(q(x)/p(x)) - (zd(x) - zt(x)) * c = (m_t - m_d) + log2(inv_d / inv_t), one
// constant per row pair, split into an integral part ki and a fraction kf in
// [-0.5, 0.5] so that fp32 arithmetic keeps it to within 3e-8 (both exactly 0
// for two identical rows).
struct Shift {
    float ki, kf;
};

__device__ __forceinline__ Shift residual_shift(const RowStats& st, const RowStats& sd) {
    const double l = log2(sd.inv / st.inv);
    const double r = rint(l);
    return Shift{(float)(((double)st.m - (double)sd.m) + r), (float)(l - r)};
}

// Logits rows with their statistics: w = max(0, p - q) (residual, D) or
// max(0, p) (bonus or zero-residual fallback). The residual weight is formed
// as p(x) * (1 - q(x)/p(x)) with log2(q(x)/p(x)) = (zd(x) - zt(x)) * c + k0
// taken from the exact logit difference, so it keeps a small relative error
// where p and q nearly agree, instead of the absolute error of a difference of
// two separately rounded probabilities.
template <bool BF16, bool VEC, bool D>
struct LogitSource {
    // segments per wavefront step; with the next step's loads in flight too,
    // two fp32 pairs, or two bf16 pairs of element-wise loads, would not fit
    // the register budget
    static constexpr int kUnroll = BF16 && VEC ? 2 : 1;
    const void* zt;
    const void* zd;  // read only when D
    int V;
    float c;
    RowStats st, sd;
    Shift k;  // residual_shift(st, sd) when D
    using L = Logit4<BF16>;
    struct Raw {
        typename L::Raw t, d;
    };
    __device__ Raw load(int64_t x) const {
        Raw r;
        r.d = L::neg_inf();
        if (VEC) {
            const bool in = x < V;
            const int64_t xs = in ? x : 0;
            const typename L::Raw a = L::load(zt, xs);
            r.t = in ? a : L::neg_inf();
            if (D) {
                const typename L::Raw b = L::load(zd, xs);
                r.d = in ? b : L::neg_inf();
            }
        } else {
            float a[4], d[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool in = x + j < V;
                const int64_t xs = in ? x + j : 0;
                const float va = L::at(zt, xs);
                a[j] = in ? va : -INFINITY;
                if (D) {
                    const float vd = L::at(zd, xs);
                    d[j] = in ? vd : -INFINITY;
                } else {
                    d[j] = -INFINITY;
                }
            }
            r.t = L::pack(a);
            r.d = L::pack(d);
        }
        return r;
    }
    __device__ void weights(const Raw& r, double w[4]) const {
        float a[4], d[4];
        L::unpack(r.t, a);
        L::unpack(r.d, d);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float e = ex2(fmaf(a[j], c, -st.m));
            if (D) {
                // y = log2(q/p) (the logit difference is exact for bf16 logits);
                // q >= p (y >= 0), a NaN from two -inf logits or padding, and
                // p = 0 all give weight 0; q = 0 < p gives y = -inf, weight p
                const float y = fmaf(d[j] - a[j], c, k.ki) + k.kf;
                w[j] = y < 0.0f ? (double)(e * one_minus_exp2(y)) * st.inv : 0.0;
            } else {
                w[j] = fmax((double)e * st.inv, 0.0);  // a NaN gives 0
            }
        }
    }
};

// ---- the draw ---------------------------------------------------------------

// All NW wavefronts write seg[s] = sum of the weights of segment s
// (L = m * kSub elements). Returns the row's total weight S, identical in
// every lane (each wavefront sums seg[] in the same order).
template <int NW, class Src>
__device__ double segment_totals(const Src& src, int m, int nseg, double* seg) {
    constexpr int U = Src::kUnroll;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t L = (int64_t)m * kSub;
    // A wavefront takes its segments U at a time (s0 + u * NW) and walks their
    // sub-blocks k; the loads of the next (s0, k) step are issued before the
    // current step's weights are summed, across segment boundaries too (for
    // short rows m is 1 and each segment is a single step).
    using Raw = typename Src::Raw;
    auto fetch = [&](int s0, int k, Raw* r) {
#pragma unroll
        for (int u = 0; u < U; ++u) r[u] = src.load((int64_t)(s0 + u * NW) * L + (int64_t)k * kSub + 4 * lane);
    };
    Raw cur[U], nxt[U];
    double acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = 0.0;
    int s0 = wave, k = 0;
    if (s0 < nseg) fetch(s0, 0, cur);
    while (s0 < nseg) {
        int s1 = s0, k1 = k + 1;
        if (k1 == m) {
            k1 = 0;
            s1 = s0 + NW * U;
        }
        if (s1 < nseg) fetch(s1, k1, nxt);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            double w[4];
            src.weights(cur[u], w);
            acc[u] += ((w[0] + w[1]) + w[2]) + w[3];
        }
        if (k1 == 0) {  // the U segments are complete
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const double tot = wave_sum_d(acc[u]);
                const int s = s0 + u * NW;
                if (lane == 0 && s < nseg) seg[s] = tot;
                acc[u] = 0.0;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        s0 = s1;
        k = k1;
    }
    __syncthreads();
    double part = 0.0;
    for (int s = lane; s < nseg; s += kWave) part += seg[s];
    return wave_sum_d(part);
}

// Smallest x with positive weight whose cumulative weight exceeds thr
// (wavefront 0 only). If rounding leaves no such x in the chosen segment,
// or u*S reaches S, the last positive-weight id is returned.
template <class Src>
__device__ int locate(const Src& src, int m, int nseg, const double* seg, double thr) {
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
        src.weights(src.load(x0), w);
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

// After segment_totals: wavefront 0 locates the draw at u*S (-1 when the row
// has no positive weight). Only lane 0 of wavefront 0 may use the result.
template <class Src>
__device__ int draw(const Src& src, int m, int nseg, const double* seg, float u, double S) {
    if (threadIdx.x >= kWave) return -2;
    if (!(S > 0.0)) return -1;
    return locate(src, m, nseg, seg, (double)u * S);
}

// The final draw of a sequence: from the residual source `res` when
// `residual` (falling back to `bon`, the same target row alone, if the
// residual has no mass), else from the bonus source `bon`. Every lane of the
// workgroup calls it; the id is valid in lane 0.
template <class Res, class Bon>
__device__ int final_draw(const Res& res, const Bon& bon, bool residual, int m, int nseg, double* seg, float u) {
    if (residual) {
        const double S = segment_totals<kWaves>(res, m, nseg, seg);
        if (S > 0.0) return draw(res, m, nseg, seg, u, S);
        __syncthreads();  // p_n == q_n: no residual mass, draw from max(0, p_n)
    }
    const double S = segment_totals<kWaves>(bon, m, nseg, seg);
    return draw(bon, m, nseg, seg, u, S);
}

// ---- accept_kernel: probability rows ----------------------------------------

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

    // 2-3. the draw from the row (pair) it needs
    const bool residual = n < kb;
    const int prow = residual ? n : kb;
    ProbSource<VEC, true> res{p + ((int64_t)b * (K + 1) + prow) * Vl, residual ? q + ((int64_t)b * K + n) * Vl : nullptr,
                              V};
    ProbSource<VEC, false> bon{p + ((int64_t)b * (K + 1) + prow) * Vl, nullptr, V};
    const int next = final_draw(res, bon, residual, m, nseg, seg, uniforms[(int64_t)b * (K + 1) + kb]);
    if (threadIdx.x == 0) {
        n_accepted[b] = n;
        next_token[b] = next;
    }
}

// ---- accept_logits_kernel: logits rows, warped on the fly -------------------

// Online statistics of y = z*c: s = sum of 2^(y - m) over the elements seen,
// against a reference m that is an integer (the ceiling of the largest y so
// far) or kNoRef before the first finite y. Moving the reference therefore
// rescales s by an exact power of two, and every term 2^(y - m) is at most 1;
// -inf elements add exp2(-inf) = 0 and need no test. The 4-element fp32
// partials are summed in binary64.
struct Online {
    float m;
    double s;
};

constexpr float kNoRef = -3.40282347e38f;  // -FLT_MAX: below every finite y

// s * 2^(from - to) for integral from <= to (kNoRef included: shifts past
// the binary64 range give 0).
__device__ __forceinline__ double rescale(double s, float from, float to) {
    return __builtin_ldexp(s, (int)fmaxf(from - to, -1100.0f));
}

// Pairwise sum of N fp32 terms (a fixed tree: independent adds).
template <int N>
__device__ __forceinline__ float tree_sum(const float* e) {
    if constexpr (N == 1) {
        return e[0];
    } else {
        return tree_sum<N / 2>(e) + tree_sum<N - N / 2>(e + N / 2);
    }
}

// N elements at once: one max, at most one (exact) rescale, one fp32 partial
// sum and one binary64 add per N elements.
template <int N>
__device__ __forceinline__ void online_addn(const float* z, float c, Online& o) {
    const float zm = max_of<N>(z);
    const float r = max2f(o.m, ceilf(zm * c));
    o.s = rescale(o.s, o.m, r);  // exact; the identity when the reference stays
    o.m = r;
    float e[N];
#pragma unroll
    for (int k = 0; k < N; ++k) e[k] = ex2(fmaf(z[k], c, -o.m));
    o.s += (double)tree_sum<N>(e);
}

__device__ __forceinline__ void online_add4(const float z[4], float c, Online& o) { online_addn<4>(z, c, o); }

__device__ __forceinline__ void online_merge(Online& a, float m2, double s2) {
    const float mm = fmaxf(a.m, m2);
    a.s = rescale(a.s, a.m, mm) + rescale(s2, m2, mm);
    a.m = mm;
}

// Wave-wide merge (same butterfly as the other reductions); result uniform.
__device__ __forceinline__ void wave_online(Online& o) {
    online_merge(o, dpp_f<kDppQuadXor1>(o.m), dpp_d<kDppQuadXor1>(o.s));
    online_merge(o, dpp_f<kDppQuadXor2>(o.m), dpp_d<kDppQuadXor2>(o.s));
    online_merge(o, dpp_f<kDppRowHalfMirror>(o.m), dpp_d<kDppRowHalfMirror>(o.s));
    online_merge(o, dpp_f<kDppRowMirror>(o.m), dpp_d<kDppRowMirror>(o.s));
    online_merge(o, swz16_f(o.m), swz16_d(o.s));
    Online r{readlane_f(o.m, 0), readlane_d(o.s, 0)};
    online_merge(r, readlane_f(o.m, 32), readlane_d(o.s, 32));
    o = r;
}

struct StatsLds {
    float m[2][kWaves];
    double s[2][kWaves];
};

// Online statistics (m, s) of elements [x0, x0 + len) of target row zt and (D) draft
// row zd, merged over the NW wavefronts of the workgroup: rt and rd are
// uniform. For VEC, x0 and len are multiples of 4. Contains barriers.
template <bool BF16, bool VEC, bool D, int NW, int UD = 4>
__device__ void span_stats(const void* zt, const void* zd, int64_t x0, int len, float c, StatsLds* lds, Online& rt,
                           Online& rd) {
    using L = Logit4<BF16>;
    constexpr int NT = NW * kWave;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    Online ot{kNoRef, 0.0}, od{kNoRef, 0.0};
    if (VEC) {
        // Software-pipelined: the next U quads of the row(s) are in flight while
        // the current ones are consumed.
        constexpr int U = D ? UD : 2 * UD;
        constexpr int kStep = U * NT;
        const int nq = len / 4;
        const int nfull = nq / kStep;  // whole steps
        typename L::Raw ct[U], cd[U], nt[U], nd[U];
        auto fetch = [&](int base, typename L::Raw* t, typename L::Raw* d) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t x = x0 + 4 * (int64_t)(base + u * NT + tid);
                t[u] = L::load(zt, x);
                if (D) d[u] = L::load(zd, x);
            }
        };
        if (nfull > 0) fetch(0, nt, nd);
        for (int it = 0; it < nfull; ++it) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                ct[u] = nt[u];
                if (D) cd[u] = nd[u];
            }
            if (it + 1 < nfull) fetch((it + 1) * kStep, nt, nd);
            float a[4 * U];
#pragma unroll
            for (int u = 0; u < U; ++u) L::unpack(ct[u], a + 4 * u);
            online_addn<4 * U>(a, c, ot);
            if (D) {
#pragma unroll
                for (int u = 0; u < U; ++u) L::unpack(cd[u], a + 4 * u);
                online_addn<4 * U>(a, c, od);
            }
        }
        for (int j = nfull * kStep + tid; j < nq; j += NT) {
            float a[4];
            L::unpack(L::load(zt, x0 + 4 * (int64_t)j), a);
            online_add4(a, c, ot);
            if (D) {
                L::unpack(L::load(zd, x0 + 4 * (int64_t)j), a);
                online_add4(a, c, od);
            }
        }
    } else {
        for (int x = tid; x < len; x += NT) {
            const float a[4] = {L::at(zt, x0 + x), -INFINITY, -INFINITY, -INFINITY};
            online_add4(a, c, ot);
            if (D) {
                const float d[4] = {L::at(zd, x0 + x), -INFINITY, -INFINITY, -INFINITY};
                online_add4(d, c, od);
            }
        }
    }
    wave_online(ot);
    if (D) wave_online(od);
    __syncthreads();  // the LDS slots may still be read from the previous call
    if (lane == 0) {
        lds->m[0][wave] = ot.m;
        lds->s[0][wave] = ot.s;
        lds->m[1][wave] = od.m;
        lds->s[1][wave] = od.s;
    }
    __syncthreads();
    rt = Online{lane < NW ? lds->m[0][lane] : kNoRef, lane < NW ? lds->s[0][lane] : 0.0};
    wave_online(rt);
    if (D) {
        rd = Online{lane < NW ? lds->m[1][lane] : kNoRef, lane < NW ? lds->s[1][lane] : 0.0};
        wave_online(rd);
    }
}

// Statistics of whole rows (target, and draft when D), merged over the
// 1024-lane workgroup; every lane gets them. Contains barriers.
template <bool BF16, bool VEC, bool D>
__device__ void row_stats_pass(const void* zt, const void* zd, int V, float c, StatsLds* lds, RowStats& st,
                               RowStats& sd) {
    Online rt, rd;
    span_stats<BF16, VEC, D, kWaves, BF16 ? 2 : 1>(zt, zd, 0, V, c, lds, rt, rd);
    st = RowStats{rt.m, 1.0 / rt.s};
    if (D) sd = RowStats{rd.m, 1.0 / rd.s};
}

// LSE: the draft rows' normalisers are given (draft_lse [B, K]); a draft row
// is then read only at the rejected position, for the residual.
template <bool BF16, bool VEC, bool LSE>
__global__ __launch_bounds__(kThreads) void accept_logits_kernel(const void* __restrict__ zt,
                                                                 const void* __restrict__ zd, int K, int V, int m,
                                                                 int nseg, float c, const float* __restrict__ draft_lse,
                                                                 const int32_t* __restrict__ tokens,
                                                                 const int32_t* __restrict__ lens,
                                                                 const float* __restrict__ uniforms,
                                                                 int32_t* __restrict__ n_accepted,
                                                                 int32_t* __restrict__ next_token) {
    extern __shared__ double seg[];
    __shared__ StatsLds lds;
    using L = Logit4<BF16>;
    const int b = blockIdx.x;
    const int kb = clamp_len(lens, b, K);
    const size_t row_bytes = (size_t)V * (BF16 ? 2 : 4);
    const char* tbase = (const char*)zt + (size_t)b * (size_t)(K + 1) * row_bytes;
    const char* dbase = (const char*)zd + (size_t)b * (size_t)K * row_bytes;

    // 1. positions in order; stop at the first rejection
    int n = kb;
    bool have = false;  // statistics of row pair n are in st, sd
    RowStats st{0.f, 0.0}, sd{0.f, 0.0};
    for (int i = 0; i < kb; ++i) {
        const int t = tokens[(int64_t)b * K + i];
        if (t < 0 || t >= V) {  // out-of-range draft token: rejected, never dereferenced
            n = i;
            break;
        }
        const void* tr = tbase + (size_t)i * row_bytes;
        const void* dr = dbase + (size_t)i * row_bytes;
        const float u = uniforms[(int64_t)b * (K + 1) + i];
        row_stats_pass<BF16, VEC, !LSE>(tr, dr, V, c, &lds, st, sd);
        const bool ok = LSE ? accepts_given(L::at(tr, t), L::at(dr, t), c, st, draft_lse[(int64_t)b * K + i], u)
                            : accepts(L::at(tr, t), L::at(dr, t), c, st, sd, u);
        if (!ok) {
            n = i;
            have = true;
            break;
        }
    }

    // 2-3. the draw (LSE: a rejection whose normaliser is not finite has q = 0
    // or a residual of no mass, and draws from max(0, p_n))
    bool residual = n < kb;
    const float lse_n = LSE && residual ? draft_lse[(int64_t)b * K + n] : 0.0f;
    if (LSE && residual && !(lse_n > -INFINITY && lse_n < INFINITY)) residual = false;
    const void* zt_row = tbase + (size_t)(n < kb ? n : kb) * row_bytes;
    const void* zd_row = residual ? (const void*)(dbase + (size_t)n * row_bytes) : nullptr;
    if (!(n < kb && have)) {
        if (residual && !LSE)
            row_stats_pass<BF16, VEC, true>(zt_row, zd_row, V, c, &lds, st, sd);
        else
            row_stats_pass<BF16, VEC, false>(zt_row, nullptr, V, c, &lds, st, sd);
    }
    if (LSE && residual) sd = given_stats(lse_n);
    const LogitSource<BF16, VEC, true> res{zt_row, zd_row, V, c, st, sd,
                                           residual ? residual_shift(st, sd) : Shift{0.f, 0.f}};
    const LogitSource<BF16, VEC, false> bon{zt_row, nullptr, V, c, st, sd, Shift{0.f, 0.f}};
    const int next = final_draw(res, bon, residual, m, nseg, seg, uniforms[(int64_t)b * (K + 1) + kb]);
    if (threadIdx.x == 0) {
        n_accepted[b] = n;
        next_token[b] = next;
    }
}

// ---- accept_logits_sliced_kernel: each sequence over G workgroups ----------
//
// The procedure of accept_logits_kernel with the rows of a sequence split
// into G slices; workgroup (b, g) of 256 lanes owns slice g of every row of
// sequence b. A slice is kSliceVecs 16-byte vectors per lane and row (12288
// bf16 or 6144 fp32 logits), so at each examined position the workgroup
// issues its whole share of the target and draft rows as one batch of loads;
// the target share stays in registers and the draft share is parked in LDS.
// The kernel is bound by its arithmetic (two exponentials per element pair,
// and per position the reductions, the exchange and the accept test), not by
// memory: measured on MI355X at B = 512, K = 16, V = 256000 it runs about as
// fast with its slice loads removed. Six vectors per lane (G = 21 slices of
// 24 KB per row there) beat four by 4% and eight (which spills) by 30%.
// The slice's statistics, the accept test and the weights of the draw all
// come from those copies, so every byte the method needs is fetched once;
// the one exception is the slice the drawn id lies in, which the locating
// workgroup loads again (two slices of 24 KB per sequence). At each position
// the G workgroups publish their slices' statistics (m, s) of both rows into
// slots of the caller's workspace (filled with the empty marker before the
// launch) and each merges all G in one fixed order, so every slice takes the
// same decision. For the draw each publishes its slice's total weight and
// counts in; the others leave, and the last to arrive sums the totals,
// finds the slice holding u * S and locates the id there. Every wait is
// bounded: a workgroup that gives up loads the missing slices and computes
// their values itself with the same code and lane mapping, so results are
// bitwise identical either way.

constexpr int kSliceWaves = 4;
constexpr int kSliceThreads = kSliceWaves * kWave;
constexpr int kSliceVecs = 6;      // 16-byte vectors per lane and row: one batch of loads per position
constexpr int kMaxSlices = kWave;  // slice partials are merged across one wavefront
constexpr int kChunks = kSliceVecs * kSliceWaves;
constexpr uint32_t kBufferWord3 = 0x00020000u;  // gfx9 buffer descriptor: raw 32-bit data, no swizzle

// 16 bytes of a row: 8 bf16 or 4 fp32 logits.
template <bool BF16>
struct Vec16 {
    static constexpr int E = BF16 ? 8 : 4;
    __device__ static u32x4 neg_inf() {
        const uint32_t w = BF16 ? 0xFF80FF80u : 0xFF800000u;
        return u32x4{w, w, w, w};
    }
};

// Elements 4h .. 4h + 3 of a 16-byte vector (h < E / 4).
template <bool BF16>
__device__ __forceinline__ void quad_of(const u32x4& r, int h, float z[4]) {
    if (BF16) {
        z[0] = bf16_lo(r[2 * h]);
        z[1] = bf16_hi(r[2 * h]);
        z[2] = bf16_lo(r[2 * h + 1]);
        z[3] = bf16_hi(r[2 * h + 1]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) z[k] = __uint_as_float(r[k]);
    }
}

// The lane's share of elements [x0, x0 + len) of a row: vector u holds
// elements x0 + (u * 256 + lane) * E ... + E - 1 (lane = threadIdx.x), so
// each load instruction covers 4 KB of consecutive logits; vectors at or past
// x0 + len read as -inf (only a row's last slice is partial). VEC: buffer
// loads of 16 bytes (V a multiple of E, rows 16-byte aligned); otherwise
// element by element.
template <bool BF16, bool VEC>
__device__ __forceinline__ void load_slice(const char* row, int64_t x0, int len, u32x4 (&r)[kSliceVecs]) {
    using W = Vec16<BF16>;
    constexpr int E = W::E;
    constexpr int es = BF16 ? 2 : 4;
    const int tid = threadIdx.x;
    if (VEC) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(row) + x0 * es, 0, len * es, kBufferWord3);
#pragma unroll
        for (int u = 0; u < kSliceVecs; ++u)
            r[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, u * kSliceThreads * 16, 0);
        if (len < kSliceThreads * kSliceVecs * E) {  // the row's last slice: past its end reads -inf
#pragma unroll
            for (int u = 0; u < kSliceVecs; ++u)
                if ((u * kSliceThreads + tid) * E >= len) r[u] = W::neg_inf();
        }
    } else {
#pragma unroll
        for (int u = 0; u < kSliceVecs; ++u) {
            const int xi = (u * kSliceThreads + tid) * E;
            float z[E];
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const bool in = xi + j < len;
                const float v = Logit4<BF16>::at(row, x0 + (in ? xi + j : 0));
                z[j] = in ? v : -INFINITY;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                r[u][k] = BF16 ? (__float_as_uint(z[2 * k]) >> 16) | (__float_as_uint(z[2 * k + 1]) & 0xFFFF0000u)
                               : __float_as_uint(z[k]);
        }
    }
}

// Largest logit of the lane's share.
template <bool BF16>
__device__ __forceinline__ float lane_max(const u32x4 (&r)[kSliceVecs]) {
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kSliceVecs; ++u) {
#pragma unroll
        for (int h = 0; h < Vec16<BF16>::E / 4; ++h) {
            float z[4];
            quad_of<BF16>(r[u], h, z);
            mx = max3f(mx, max3f(z[0], z[1], z[2]), z[3]);
        }
    }
    return mx;
}

// Sum of 2^(z * c - m) over the lane's share: fp32 per vector, binary64
// across vectors (each vector unpacked afresh: no unpacked copy kept live).
template <bool BF16>
__device__ __forceinline__ double lane_expsum(const u32x4 (&r)[kSliceVecs], float c, float m) {
    constexpr int E = Vec16<BF16>::E;
    double s = 0.0;
#pragma unroll
    for (int u = 0; u < kSliceVecs; ++u) {
        u32x4 v = r[u];
        asm volatile("" : "+v"(v));
        float e[E];
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
            float z[4];
            quad_of<BF16>(v, h, z);
#pragma unroll
            for (int j = 0; j < 4; ++j) e[4 * h + j] = ex2(fmaf(z[j], c, -m));
        }
        s += (double)tree_sum<E>(e);
    }
    return s;
}

// Wave-wide maximum (fixed butterfly; result uniform).
__device__ __forceinline__ float wave_max_f(float x) {
    x = max2f(x, dpp_f<kDppQuadXor1>(x));
    x = max2f(x, dpp_f<kDppQuadXor2>(x));
    x = max2f(x, dpp_f<kDppRowHalfMirror>(x));
    x = max2f(x, dpp_f<kDppRowMirror>(x));
    x = max2f(x, swz16_f(x));
    return max2f(readlane_f(x, 0), readlane_f(x, 32));
}

// The N wave partials a[0 .. N) combined in a fixed pairwise order.
template <int N>
__device__ __forceinline__ float lds_max(const float* a) {
    if constexpr (N == 1) {
        return a[0];
    } else {
        return max2f(lds_max<N / 2>(a), lds_max<N - N / 2>(a + N / 2));
    }
}
template <int N>
__device__ __forceinline__ double lds_sum(const double* a) {
    if constexpr (N == 1) {
        return a[0];
    } else {
        return lds_sum<N / 2>(a) + lds_sum<N - N / 2>(a + N / 2);
    }
}

// Statistics (m, s) of the slice held in rt (and rd when D), over the
// workgroup: m is the ceiling of the slice's largest y = z * c (kNoRef if
// none is finite), shared by every lane, so the lanes' sums of 2^(y - m) add
// up without rescaling; the wave sums and the kSliceWaves wave partials are
// added in a fixed order. t and d are uniform. Contains barriers.
template <bool BF16, bool D>
__device__ void slice_stats(const u32x4 (&rt)[kSliceVecs], const u32x4 (&rd)[kSliceVecs], float c, StatsLds* lds,
                            Online& t, Online& d) {
    static_assert(kSliceWaves <= kWaves, "the wave partials live in StatsLds");
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    float xt = wave_max_f(lane_max<BF16>(rt)), xd = -INFINITY;
    if (D) xd = wave_max_f(lane_max<BF16>(rd));
    __syncthreads();  // the LDS slots may still be read from the previous call
    if (lane == 0) {
        lds->m[0][wave] = xt;
        if (D) lds->m[1][wave] = xd;
    }
    __syncthreads();
    t.m = max2f(kNoRef, ceilf(lds_max<kSliceWaves>(lds->m[0]) * c));
    const double st = wave_sum_d(lane_expsum<BF16>(rt, c, t.m));
    double sd = 0.0;
    if (D) {
        d.m = max2f(kNoRef, ceilf(lds_max<kSliceWaves>(lds->m[1]) * c));
        sd = wave_sum_d(lane_expsum<BF16>(rd, c, d.m));
    }
    if (lane == 0) {
        lds->s[0][wave] = st;
        if (D) lds->s[1][wave] = sd;
    }
    __syncthreads();
    t.s = lds_sum<kSliceWaves>(lds->s[0]);
    if (D) d.s = lds_sum<kSliceWaves>(lds->s[1]);
}

__device__ __forceinline__ unsigned long long pack_online(const Online& o) {
    return ((unsigned long long)__float_as_uint((float)o.s) << 32) | __float_as_uint(o.m);
}

// Shared state of a workgroup's exchanges.
struct SliceCtx {
    unsigned long long* s_words;  // LDS [2 * kMaxSlices]
    int* s_ready;
    u32x4* s_draft;  // LDS [kSliceVecs][256]: this slice of the current draft row
    int G, g, Ls, V, wait_limit;
    __device__ int len(int k) const { return (int)min((int64_t)Ls, (int64_t)V - (int64_t)k * Ls); }
    __device__ u32x4 draft(int u) const { return s_draft[u * kSliceThreads + threadIdx.x]; }
};

// Slice statistics of rows tr (and dr when D), loaded here: a fallback path.
template <bool BF16, bool VEC, bool D>
__device__ void other_slice_stats(const SliceCtx& x, int k, const char* tr, const char* dr, float c, StatsLds* lds,
                                  Online& t, Online& d) {
    u32x4 vt[kSliceVecs], vd[kSliceVecs];
    load_slice<BF16, VEC>(tr, (int64_t)k * x.Ls, x.len(k), vt);
    if (D) load_slice<BF16, VEC>(dr, (int64_t)k * x.Ls, x.len(k), vd);
    slice_stats<BF16, D>(vt, vd, c, lds, t, d);
}

// Position `pos`: load this slice of target row tr into rt (and of draft row
// dr into s_draft, when D), take the slice statistics, publish them into
// set[2g], set[2g + 1], gather all G and merge them in slice order into st
// (and sd). If the wait runs out every slice is loaded and computed here
// alike. Called by the whole workgroup.
template <bool BF16, bool VEC, bool D>
__device__ void position_stats(const SliceCtx& x, unsigned long long* set, const char* tr, const char* dr, float c,
                               u32x4 (&rt)[kSliceVecs], StatsLds* lds, RowStats& st, RowStats& sd) {
    const int64_t x0 = (int64_t)x.g * x.Ls;
    Online a, d{kNoRef, 0.0};
    u32x4 v[kSliceVecs];
    if (D) load_slice<BF16, VEC>(dr, x0, x.len(x.g), v);
    load_slice<BF16, VEC>(tr, x0, x.len(x.g), rt);
    slice_stats<BF16, D>(rt, v, c, lds, a, d);
    if (D) {
#pragma unroll
        for (int u = 0; u < kSliceVecs; ++u) x.s_draft[u * kSliceThreads + threadIdx.x] = v[u];  // own lanes only
    }
    publish_word(set + 2 * x.g, pack_online(a));
    publish_word(set + 2 * x.g + 1, D ? pack_online(d) : 0ull);  // both words: the gather waits for all 2G
    if (!gather_words(set, 2 * x.G, x.wait_limit, x.s_words, x.s_ready)) {
        for (int k = 0; k < x.G; ++k) {
            Online ak, dk{kNoRef, 0.0};
            other_slice_stats<BF16, VEC, D>(x, k, tr, dr, c, lds, ak, dk);
            if (threadIdx.x == 0) {
                x.s_words[2 * k] = pack_online(ak);
                x.s_words[2 * k + 1] = D ? pack_online(dk) : 0ull;
            }
        }
        load_slice<BF16, VEC>(tr, x0, x.len(x.g), rt);  // this slice again (its draft share is in LDS)
        __syncthreads();
    }
    // lane k holds slice k: the largest reference, then the slices' sums
    // scaled to it (exact powers of two) added in the fixed butterfly order
    const int lane = threadIdx.x & (kWave - 1);
    float mt = kNoRef, md = kNoRef;
    double s_t = 0.0, s_d = 0.0;
    if (lane < x.G) {
        const unsigned long long w = x.s_words[2 * lane];
        mt = __uint_as_float((unsigned)w);
        s_t = (double)__uint_as_float((unsigned)(w >> 32));
        if (D) {
            const unsigned long long w2 = x.s_words[2 * lane + 1];
            md = __uint_as_float((unsigned)w2);
            s_d = (double)__uint_as_float((unsigned)(w2 >> 32));
        }
    }
    const float Mt = wave_max_f(mt);
    st = RowStats{Mt, 1.0 / wave_sum_d(rescale(s_t, mt, Mt))};
    if (D) {
        const float Md = wave_max_f(md);
        sd = RowStats{Md, 1.0 / wave_sum_d(rescale(s_d, md, Md))};
    }
    __syncthreads();  // s_words is reused by the next exchange
}

// Draw weights of elements 4h .. 4h + 3 of a vector pair: max(0, p - q) (D;
// formed as in LogitSource) or max(0, p).
template <bool BF16, bool D>
__device__ __forceinline__ void quad_weights(const u32x4& vt, const u32x4& vd, int h, float c, const RowStats& st,
                                             const Shift& k, double w[4]) {
    float a[4], d[4];
    quad_of<BF16>(vt, h, a);
    if (D) quad_of<BF16>(vd, h, d);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float e = ex2(fmaf(a[j], c, -st.m));
        if (D) {
            const float y = fmaf(d[j] - a[j], c, k.ki) + k.kf;
            w[j] = y < 0.0f ? (double)(e * one_minus_exp2(y)) * st.inv : 0.0;
        } else {
            w[j] = fmax((double)e * st.inv, 0.0);  // a NaN gives 0
        }
    }
}

// Total draw weight of one vector pair, quad by quad in element order.
template <bool BF16, bool D>
__device__ __forceinline__ double vec_total(const u32x4& vt, const u32x4& vd, float c, const RowStats& st,
                                            const Shift& k) {
    double s = 0.0;
#pragma unroll
    for (int h = 0; h < Vec16<BF16>::E / 4; ++h) {
        double w[4];
        quad_weights<BF16, D>(vt, vd, h, c, st, k, w);
        s += ((w[0] + w[1]) + w[2]) + w[3];
    }
    return s;
}

// The slice's draw weights summed per chunk (vector u of wavefront w's 64
// lanes: 64 * E consecutive elements; chunk u * kSliceWaves + w, so chunks
// run in element order) into chunk[]; returns the slice total, the chunks
// summed in order (uniform). dvec(u) gives the draft vector u (D only).
// Contains barriers.
template <bool BF16, bool D, class DVec>
__device__ double slice_total(const u32x4 (&rt)[kSliceVecs], DVec dvec, float c, const RowStats& st,
                              const Shift& k, double* chunk) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    __syncthreads();  // chunk[] may still be read from the previous call
#pragma unroll
    for (int u = 0; u < kSliceVecs; ++u) {
        const double tot = wave_sum_d(vec_total<BF16, D>(rt[u], D ? dvec(u) : rt[u], c, st, k));
        if (lane == 0) chunk[u * kSliceWaves + wave] = tot;
    }
    __syncthreads();
    double S = 0.0;
#pragma unroll
    for (int q = 0; q < kChunks; ++q) S += chunk[q];
    return S;
}

// A total as a slot word: the sign bit flipped, so that no total is the empty
// marker (weights are never negative; a NaN keeps a NaN pattern).
__device__ __forceinline__ unsigned long long total_word(double S) {
    return (unsigned long long)__double_as_longlong(S) ^ 0x8000000000000000ull;
}
__device__ __forceinline__ double word_total(unsigned long long w) {
    return __longlong_as_double((long long)(w ^ 0x8000000000000000ull));
}

// The slices of a sequence count in on `counter` (filled with kEmptySlot
// before the launch, so the k-th arrival reads kEmptySlot + k); returns,
// uniform over the workgroup, whether this one was the last of the G.
__device__ __forceinline__ bool last_in(unsigned long long* counter, int G, int* s_flag) {
    if (threadIdx.x == 0) {
        const unsigned long long prev =
            __hip_atomic_fetch_add(counter, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = prev + 1ull == (unsigned long long)(G - 1);
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*s_flag) != 0;
}

// This workgroup's slice k of the draw rows: target slice into rt, and with
// D the draft slice into s_draft (each lane its own entries).
template <bool BF16, bool VEC, bool D>
__device__ void load_draw_slice(const SliceCtx& x, int k, const char* tr, const char* dr, u32x4 (&rt)[kSliceVecs]) {
    load_slice<BF16, VEC>(tr, (int64_t)k * x.Ls, x.len(k), rt);
    if (D) {
        u32x4 v[kSliceVecs];
        load_slice<BF16, VEC>(dr, (int64_t)k * x.Ls, x.len(k), v);
#pragma unroll
        for (int u = 0; u < kSliceVecs; ++u) x.s_draft[u * kSliceThreads + threadIdx.x] = v[u];
    }
}

// Element-level locate inside vector U of the calling wavefront's lanes:
// the lanes' vector totals scanned in lane order, then each lane's elements
// in order, quad by quad (weights formed again: no arrays kept). pre is the
// cumulative weight before the chunk. Returns the offset in the slice of the
// first positive-weight element whose cumulative weight exceeds thr, else
// the chunk's last positive-weight element (-1 if none), in every lane.
template <bool BF16, bool D, int U>
__device__ int locate_in_chunk(const SliceCtx& x, const u32x4 (&rt)[kSliceVecs], float c, const RowStats& st,
                               const Shift& k, double pre, double thr) {
    constexpr int E = Vec16<BF16>::E;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const u32x4 vt = rt[U];
    const u32x4 vd = D ? x.draft(U) : vt;
    const double incl = wave_incl_scan_d(vec_total<BF16, D>(vt, vd, c, st, k), lane);
    double excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = 0.0;
    double run = pre + excl;
    const int first = (U * kSliceThreads + wave * kWave + lane) * E;
    int cand = -1, lp = -1;
#pragma unroll
    for (int h = 0; h < E / 4; ++h) {
        double w[4];
        quad_weights<BF16, D>(vt, vd, h, c, st, k, w);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            run += w[j];
            if (cand < 0 && w[j] > 0.0 && run > thr) cand = first + 4 * h + j;
            if (w[j] > 0.0) lp = first + 4 * h + j;
        }
    }
    const uint64_t hit = __ballot(cand >= 0);
    if (hit) return readlane_i(cand, __builtin_ctzll(hit));
    const uint64_t pos = __ballot(lp >= 0);
    return pos ? readlane_i(lp, 63 - __builtin_clzll(pos)) : -1;
}

// locate_in_chunk for vector u, with u turned into a constant (registers are
// not indexable).
template <bool BF16, bool D, int U>
__device__ __forceinline__ int locate_dispatch(int u, const SliceCtx& x, const u32x4 (&rt)[kSliceVecs], float c,
                                               const RowStats& st, const Shift& k, double pre, double thr) {
    if constexpr (U + 1 == kSliceVecs) {
        return locate_in_chunk<BF16, D, U>(x, rt, c, st, k, pre, thr);
    } else {
        return u == U ? locate_in_chunk<BF16, D, U>(x, rt, c, st, k, pre, thr)
                      : locate_dispatch<BF16, D, U + 1>(u, x, rt, c, st, k, pre, thr);
    }
}

// Offset in the slice of the drawn id: the first element with positive
// weight whose cumulative weight (from the slice start) exceeds thr; if
// rounding leaves none, the last positive-weight element of the chunk the
// chunk totals point to (or of the slice, when thr is beyond them all).
// Only the wavefront holding that chunk returns it (in every lane); the
// others return -2.
template <bool BF16, bool D>
__device__ int locate_in_slice(const SliceCtx& x, const u32x4 (&rt)[kSliceVecs], float c, const RowStats& st,
                               const Shift& k, const double* chunk, double thr) {
    const int wave = threadIdx.x / kWave;
    double cum = 0.0, pre = 0.0;
    int qs = -1, qlast = -1;
    for (int q = 0; q < kChunks; ++q) {
        const double v = chunk[q];
        if (v > 0.0) {
            qlast = q;
            if (qs < 0 && cum + v > thr) {
                qs = q;
                pre = cum;
            }
        }
        cum += v;
    }
    if (qs < 0) {
        if (qlast < 0) return wave == 0 ? -1 : -2;
        qs = qlast;
        thr = INFINITY;
    }
    if (wave != qs % kSliceWaves) return -2;
    return locate_dispatch<BF16, D, 0>(qs / kSliceWaves, x, rt, c, st, k, pre, thr);
}

// Logit i of a row, the same for every lane, through the scalar unit: the
// aligned 32-bit word holding it, then its half for bf16 (a bf16 row may
// start at any even address, so the half follows from the address).
template <bool BF16>
__device__ __forceinline__ float uniform_logit(const char* row, int i) {
    if (BF16) {
        const uintptr_t a = (uintptr_t)row + (uintptr_t)i * 2;
        const uint32_t w = __builtin_amdgcn_readfirstlane(*(const uint32_t*)(a & ~(uintptr_t)3));
        return (a & 2) ? bf16_hi(w) : bf16_lo(w);
    }
    return __uint_as_float(__builtin_amdgcn_readfirstlane(*(const uint32_t*)(row + (size_t)i * 4)));
}

// LSE: the draft rows' normalisers are given (draft_lse [B, K]); only the
// target rows' statistics are exchanged, and a draft row is read only at the
// rejected position, for the residual.
template <bool BF16, bool VEC, bool LSE>
__global__ __launch_bounds__(kSliceThreads) void accept_logits_sliced_kernel(
    const void* __restrict__ zt, const void* __restrict__ zd, int K, int V, int G, int Ls, float c,
    const float* __restrict__ draft_lse, const int32_t* __restrict__ tokens, const int32_t* __restrict__ lens,
    const float* __restrict__ uniforms, int32_t* __restrict__ n_accepted, int32_t* __restrict__ next_token,
    unsigned long long* __restrict__ slots, int wait_limit, int last_locates) {
    __shared__ StatsLds lds;
    __shared__ u32x4 s_draft[kSliceVecs * kSliceThreads];
    __shared__ double chunk[kChunks];
    __shared__ unsigned long long s_words[2 * kMaxSlices];
    __shared__ double s_tot[kMaxSlices];
    __shared__ int s_ready;
    const int b = blockIdx.x / G, g = blockIdx.x - b * G;
    const int kb = clamp_len(lens, b, K);
    const size_t row_bytes = (size_t)V * (BF16 ? 2 : 4);
    const char* tbase = (const char*)zt + (size_t)b * (size_t)(K + 1) * row_bytes;
    const char* dbase = (const char*)zd + (size_t)b * (size_t)K * row_bytes;
    const SliceCtx x{s_words, &s_ready, s_draft, G, g, Ls, V, wait_limit};
    // per sequence: G words of draw totals (the residual's or the bonus's)
    // and the draw's arrival counter (in G words kept for it), then 2G words
    // per position
    unsigned long long* my = slots + (size_t)b * (size_t)(2 * G) * (size_t)(K + 2);
    unsigned long long* draw_sets = my;
    unsigned long long* pos_sets = my + 2 * G;

    // 1. positions in order; stop at the first rejection
    u32x4 rt[kSliceVecs];
    RowStats st{0.f, 0.0}, sd{0.f, 0.0};
    int n = 0;
    bool residual = false;
    for (; n < kb; ++n) {
        const char* tr = tbase + (size_t)n * row_bytes;
        const char* dr = dbase + (size_t)n * row_bytes;
        const int t = tokens[(int64_t)b * K + n];
        const bool valid = t >= 0 && t < V;  // an out-of-range draft token is rejected, never dereferenced
        const float zt_t = uniform_logit<BF16>(tr, valid ? t : 0), zd_t = uniform_logit<BF16>(dr, valid ? t : 0);
        const float u = uniforms[(int64_t)b * (K + 1) + n];
        position_stats<BF16, VEC, !LSE>(x, pos_sets + (size_t)n * 2 * G, tr, dr, c, rt, &lds, st, sd);
        const bool ok = LSE ? accepts_given(zt_t, zd_t, c, st, draft_lse[(int64_t)b * K + n], u)
                            : accepts(zt_t, zd_t, c, st, sd, u);
        if (!valid || !ok) {
            residual = true;
            break;
        }
    }
    const char* trow = tbase + (size_t)n * row_bytes;  // n == kb: the bonus row
    const char* drow = dbase + (size_t)n * row_bytes;  // read only for a residual
    if (!residual)
        position_stats<BF16, VEC, false>(x, pos_sets + (size_t)kb * 2 * G, trow, nullptr, c, rt, &lds, st, sd);
    if (LSE && residual) {
        // the given normaliser of row n: not finite means q = 0 or a residual of
        // no mass, so the draw takes max(0, p_n); otherwise this slice of draft
        // row n goes to LDS for the residual
        const float l = draft_lse[(int64_t)b * K + n];
        if (l > -INFINITY && l < INFINITY) {
            sd = given_stats(l);
            u32x4 v[kSliceVecs];
            load_slice<BF16, VEC>(drow, (int64_t)g * Ls, x.len(g), v);
#pragma unroll
            for (int u = 0; u < kSliceVecs; ++u) s_draft[u * kSliceThreads + threadIdx.x] = v[u];  // own lanes only
        } else {
            residual = false;
        }
    }

    if (g == 0 && threadIdx.x == 0) n_accepted[b] = n;

    // 2. this slice's total draw weight (its chunk sums stay in chunk[]) is
    // published. With last_locates (a launch many workgroups deep) the slices
    // count in and only the last to arrive goes on, so that the others free
    // their compute units: it sums the G totals in slice order and locates
    // the drawn id, in its own slice or in the one it loads again. Otherwise
    // every slice gathers the G totals and the one holding the id locates it
    // in its own copies.
    const Shift k0 = residual ? residual_shift(st, sd) : Shift{0.f, 0.f};
    auto own_draft = [&](int u) { return x.draft(u); };
    const double Sg = residual ? slice_total<BF16, true>(rt, own_draft, c, st, k0, chunk)
                               : slice_total<BF16, false>(rt, own_draft, c, st, k0, chunk);
    publish_word(draw_sets + g, total_word(Sg));
    if (last_locates && !last_in(draw_sets + G, G, &s_ready)) return;
    int held = g;  // the slice whose data (rt, s_draft) and chunk sums this workgroup holds
    if (gather_words(draw_sets, G, wait_limit, s_words, &s_ready)) {
        if (threadIdx.x < G) s_tot[threadIdx.x] = word_total(s_words[threadIdx.x]);
    } else {  // bounded wait ran out: every slice's total computed here alike
        for (int k = 0; k < G; ++k) {
            if (residual)
                load_draw_slice<BF16, VEC, true>(x, k, trow, drow, rt);
            else
                load_draw_slice<BF16, VEC, false>(x, k, trow, drow, rt);
            const double Sk = residual ? slice_total<BF16, true>(rt, own_draft, c, st, k0, chunk)
                                       : slice_total<BF16, false>(rt, own_draft, c, st, k0, chunk);
            if (threadIdx.x == 0) s_tot[k] = Sk;
        }
        held = G - 1;
    }
    __syncthreads();
    double S = 0.0;
    for (int k = 0; k < G; ++k) S += s_tot[k];
    bool bonus = !residual;
    if (residual && !(S > 0.0)) {
        // p_n == q_n: no residual mass, draw from max(0, p_n); every slice's
        // total computed here
        bonus = true;
        for (int k = 0; k < G; ++k) {
            load_draw_slice<BF16, VEC, false>(x, k, trow, nullptr, rt);
            const double Sk = slice_total<BF16, false>(rt, own_draft, c, st, k0, chunk);
            if (threadIdx.x == 0) s_tot[k] = Sk;
        }
        held = G - 1;
        __syncthreads();
        S = 0.0;
        for (int k = 0; k < G; ++k) S += s_tot[k];
    }
    if (!(S > 0.0)) {
        if (threadIdx.x == 0 && (last_locates || g == 0)) next_token[b] = -1;
        return;
    }

    // 3. the slice holding u * S: the first with positive total whose running
    // sum exceeds it; if rounding leaves none, the last with positive total.
    const double thr = (double)uniforms[(int64_t)b * (K + 1) + kb] * S;
    int ks = -1, klast = -1;
    double pre = 0.0, pre_ks = 0.0;
    for (int k = 0; k < G; ++k) {
        if (s_tot[k] > 0.0) {
            klast = k;
            if (ks < 0 && pre + s_tot[k] > thr) {
                ks = k;
                pre_ks = pre;
            }
        }
        pre += s_tot[k];
    }
    const double thr_local = ks < 0 ? INFINITY : thr - pre_ks;
    if (ks < 0) ks = klast;
    if (!last_locates && ks != g) return;
    if (ks != held) {  // that slice's data and chunk sums, again (the same values as its own workgroup's)
        if (bonus) {
            load_draw_slice<BF16, VEC, false>(x, ks, trow, nullptr, rt);
            slice_total<BF16, false>(rt, own_draft, c, st, k0, chunk);
        } else {
            load_draw_slice<BF16, VEC, true>(x, ks, trow, drow, rt);
            slice_total<BF16, true>(rt, own_draft, c, st, k0, chunk);
        }
    }
    const int xi = bonus ? locate_in_slice<BF16, false>(x, rt, c, st, k0, chunk, thr_local)
                         : locate_in_slice<BF16, true>(x, rt, c, st, k0, chunk, thr_local);
    if (xi != -2 && (threadIdx.x & (kWave - 1)) == 0) next_token[b] = xi < 0 ? -1 : (int)((int64_t)ks * Ls + xi);
}

__global__ void fill_empty(unsigned long long* __restrict__ p, int64_t n) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < n) p[i] = kEmptySlot;
}

// m sub-blocks per segment keep the segment count within the LDS table
void segment_shape(int V, int& m, int& nseg) {
    const int64_t per_seg_min = ((int64_t)V + kMaxSeg - 1) / kMaxSeg;
    m = (int)((per_seg_min + kSub - 1) / kSub);  // >= 1 since V >= 1
    const int64_t L = (int64_t)m * kSub;
    nseg = (int)(((int64_t)V + L - 1) / L);
}

}  // namespace

hipError_t launch_accept(const float* p, const float* q, int B, int K, int V, const int32_t* tokens,
                         const int32_t* lens, const float* uniforms, int32_t* n_accepted, int32_t* next_token,
                         hipStream_t stream) {
    int m, nseg;
    segment_shape(V, m, nseg);
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

hipError_t launch_fill_empty(unsigned long long* slots, int64_t words, hipStream_t stream) {
    if (words <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_empty, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream, slots, words);
    return hipGetLastError();
}

// Slices of the split fused verify: 256 lanes x kSliceVecs vectors x E
// elements (12288 bf16 or 6144 fp32 logits) each, G = ceil(V / Ls) of them.
// 0 when the rows are not split: rows of at most one slice, or of more than
// kMaxSlices slices (one workgroup per sequence reads those).
int fused_slices(int V, bool bf16, int& Ls) {
    Ls = kSliceThreads * kSliceVecs * (bf16 ? 8 : 4);
    const int64_t G = ((int64_t)V + Ls - 1) / Ls;
    return (G >= 2 && G <= kMaxSlices) ? (int)G : 0;
}

// B sequences x (K + 2) x 2G exchange words: 2G per position, 2G for the draw.
size_t fused_dtype_workspace_bytes(int B, int K, int V, bool bf16) {
    int Ls;
    const int G = fused_slices(V, bf16, Ls);
    if (G == 0 || (int64_t)B * G > INT32_MAX) return 0;  // the grid is B * G workgroups
    return (size_t)B * 2 * (size_t)G * (size_t)(K + 2) * sizeof(unsigned long long);
}

// The larger of the two dtypes' needs, so that one size serves either.
size_t accept_logits_workspace_bytes(int B, int K, int V) {
    const size_t a = fused_dtype_workspace_bytes(B, K, V, false), b = fused_dtype_workspace_bytes(B, K, V, true);
    return a > b ? a : b;
}

namespace {

// Whether the last slice of a sequence to arrive locates the drawn id (the
// others leave once they have published their totals) rather than the slice
// that holds it (all wait for every total). Leaving early frees compute units
// for the next sequences, which pays when the launch is many resident sets of
// workgroups deep (4 per compute unit fit at once); in a shallower launch the
// locating slice's second read is on the critical path instead. Measured on
// MI355X: B = 1024, V = 152064 fp32 (25 600 workgroups) 12% faster; B = 512,
// V = 256000 bf16 (10 752) 3% faster; B = 256, V = 128256 bf16 (2 816) 8% slower.
bool last_locates(int B, int G) {
    static std::atomic<int> cached[64];
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
        int n = cached[dev].load();
        if (n == 0) {
            if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
            cached[dev].store(n);
        }
        cus = n;
    }
    return (int64_t)B * G >= (int64_t)4 * 4 * cus;
}

// The launches of one dtype and one kind of draft input (LSE: normalisers given).
template <bool BF16, bool LSE>
hipError_t launch_accept_logits_t(const void* zt, const void* zd, int B, int K, int V, float c, const float* draft_lse,
                                  const int32_t* tokens, const int32_t* lens, const float* uniforms,
                                  int32_t* n_accepted, int32_t* next_token, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    const uintptr_t al = BF16 ? 8 : 16;
    const bool vec = (V % 4 == 0) && ((uintptr_t)zt % al == 0) && ((uintptr_t)zd % al == 0);
    const size_t need = fused_dtype_workspace_bytes(B, K, V, BF16);
    if (need > 0 && workspace && workspace_bytes >= need && (uintptr_t)workspace % 8 == 0) {
        int Ls;
        const int G = fused_slices(V, BF16, Ls);
        const bool vec16 = (V % (BF16 ? 8 : 4) == 0) && ((uintptr_t)zt % 16 == 0) && ((uintptr_t)zd % 16 == 0);
        const int64_t words = (int64_t)(need / sizeof(unsigned long long));
        unsigned long long* slots = (unsigned long long*)workspace;
        const hipError_t fe = launch_fill_empty(slots, words, stream);
        if (fe != hipSuccess) return fe;  // without the fill, stale slots would read as published
        const dim3 grid((unsigned)B * (unsigned)G), block(kSliceThreads);
        const int wl = get_wait_limit();
        const int ll = last_locates(B, G) ? 1 : 0;
        if (vec16)
            hipLaunchKernelGGL((accept_logits_sliced_kernel<BF16, true, LSE>), grid, block, 0, stream, zt, zd, K, V, G,
                               Ls, c, draft_lse, tokens, lens, uniforms, n_accepted, next_token, slots, wl, ll);
        else
            hipLaunchKernelGGL((accept_logits_sliced_kernel<BF16, false, LSE>), grid, block, 0, stream, zt, zd, K, V,
                               G, Ls, c, draft_lse, tokens, lens, uniforms, n_accepted, next_token, slots, wl, ll);
        return hipGetLastError();
    }
    int m, nseg;
    segment_shape(V, m, nseg);
    const size_t lds = (size_t)nseg * sizeof(double);
    if (vec)
        hipLaunchKernelGGL((accept_logits_kernel<BF16, true, LSE>), dim3(B), dim3(kThreads), lds, stream, zt, zd, K, V,
                           m, nseg, c, draft_lse, tokens, lens, uniforms, n_accepted, next_token);
    else
        hipLaunchKernelGGL((accept_logits_kernel<BF16, false, LSE>), dim3(B), dim3(kThreads), lds, stream, zt, zd, K,
                           V, m, nseg, c, draft_lse, tokens, lens, uniforms, n_accepted, next_token);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_accept_logits(const void* zt, const void* zd, bool bf16, int B, int K, int V, float temperature,
                                const float* draft_lse, const int32_t* tokens, const int32_t* lens,
                                const float* uniforms, int32_t* n_accepted, int32_t* next_token, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    const float c = 1.4426950408889634f / temperature;
    if (bf16)
        return draft_lse ? launch_accept_logits_t<true, true>(zt, zd, B, K, V, c, draft_lse, tokens, lens, uniforms,
                                                              n_accepted, next_token, workspace, workspace_bytes, stream)
                         : launch_accept_logits_t<true, false>(zt, zd, B, K, V, c, nullptr, tokens, lens, uniforms,
                                                               n_accepted, next_token, workspace, workspace_bytes,
                                                               stream);
    return draft_lse ? launch_accept_logits_t<false, true>(zt, zd, B, K, V, c, draft_lse, tokens, lens, uniforms,
                                                           n_accepted, next_token, workspace, workspace_bytes, stream)
                     : launch_accept_logits_t<false, false>(zt, zd, B, K, V, c, nullptr, tokens, lens, uniforms,
                                                            n_accepted, next_token, workspace, workspace_bytes, stream);
}

}  // namespace sv
