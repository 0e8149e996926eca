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

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void accept_logits_kernel(const void* __restrict__ zt,
                                                                 const void* __restrict__ zd, int K, int V, int m,
                                                                 int nseg, float c, const int32_t* __restrict__ tokens,
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
        row_stats_pass<BF16, VEC, true>(tr, dr, V, c, &lds, st, sd);
        if (!accepts(L::at(tr, t), L::at(dr, t), c, st, sd, uniforms[(int64_t)b * (K + 1) + i])) {
            n = i;
            have = true;
            break;
        }
    }

    // 2-3. the draw
    const bool residual = n < kb;
    const void* zt_row = tbase + (size_t)(residual ? n : kb) * row_bytes;
    const void* zd_row = residual ? (const void*)(dbase + (size_t)n * row_bytes) : nullptr;
    if (!(residual && have)) {
        if (residual)
            row_stats_pass<BF16, VEC, true>(zt_row, zd_row, V, c, &lds, st, sd);
        else
            row_stats_pass<BF16, VEC, false>(zt_row, nullptr, V, c, &lds, st, sd);
    }
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
// The same procedure as accept_logits_kernel, with the rows of a sequence
// split into G slices of Ls elements; workgroup (b, g) of 256 lanes owns
// slice g of every row of sequence b. At each examined position the G
// workgroups publish their slices' statistics (m, s) of the target and draft rows
// into sentinel-filled slots of the caller's workspace and merge all G in a
// fixed order, so every slice takes the same accept decision; for the draw
// each publishes its slice's total weight, all find the slice holding u * S,
// and that one locates the id inside it. A long chain of accepted positions
// thus runs on G compute units instead of one. Every wait is bounded: a
// workgroup that gives up recomputes the missing slices' values itself with
// the same code and lane mapping, so results are bitwise identical either way.

constexpr int kSliceWaves = 4;
constexpr int kSliceThreads = kSliceWaves * kWave;
constexpr int kMaxSlices = kMaxCoopSlices;
static_assert(kMaxSlices <= 8, "slice partials are merged by a butterfly over 8 lanes");

__device__ __forceinline__ unsigned long long pack_online(const Online& o) {
    return ((unsigned long long)__float_as_uint((float)o.s) << 32) | __float_as_uint(o.m);
}

__device__ __forceinline__ void merge_packed(Online& r, unsigned long long v) {
    online_merge(r, __uint_as_float((unsigned)v), (double)__uint_as_float((unsigned)(v >> 32)));
}

// Row statistics of the examined rows (target, and draft when D) from the G
// slices: publish this slice's partials into set[2g], set[2g + 1], gather all,
// merge in slice order. Called by the whole workgroup.
template <bool BF16, bool VEC, bool D>
__device__ void sliced_row_stats(unsigned long long* set, int G, int g, int Ls, int V, const void* zt, const void* zd,
                                 float c, StatsLds* lds, int wait_limit, unsigned long long* s_words, int* s_ready,
                                 RowStats& st, RowStats& sd) {
    const int64_t x0 = (int64_t)g * Ls;
    Online a, d;
    span_stats<BF16, VEC, D, kSliceWaves, BF16 ? 2 : 1>(zt, zd, x0, (int)min((int64_t)Ls, (int64_t)V - x0), c, lds, a, d);
    publish_word(set + 2 * g, pack_online(a));
    publish_word(set + 2 * g + 1, D ? pack_online(d) : 0ull);  // both words: the gather waits for all 2G
    if (!gather_words(set, 2 * G, wait_limit, s_words, s_ready)) {
        // bounded wait ran out: every slice's partials, recomputed here alike
        for (int k = 0; k < G; ++k) {
            const int64_t xk = (int64_t)k * Ls;
            Online ak, dk;
            span_stats<BF16, VEC, D, kSliceWaves, BF16 ? 2 : 1>(zt, zd, xk, (int)min((int64_t)Ls, (int64_t)V - xk), c, lds, ak,
                                                     dk);
            if (threadIdx.x == 0) {
                s_words[2 * k] = pack_online(ak);
                s_words[2 * k + 1] = D ? pack_online(dk) : 0ull;
            }
        }
        __syncthreads();
    }
    // merge the G <= 8 slices' partials in a fixed butterfly over lanes 0-7
    // of every wavefront (lane k holds slice k), then take lane 0's result
    const int lane = threadIdx.x & (kWave - 1);
    Online rt{kNoRef, 0.0}, rd{kNoRef, 0.0};
    if (lane < G) {
        merge_packed(rt, s_words[2 * lane]);
        if (D) merge_packed(rd, s_words[2 * lane + 1]);
    }
    online_merge(rt, dpp_f<kDppQuadXor1>(rt.m), dpp_d<kDppQuadXor1>(rt.s));
    online_merge(rt, dpp_f<kDppQuadXor2>(rt.m), dpp_d<kDppQuadXor2>(rt.s));
    online_merge(rt, dpp_f<kDppRowHalfMirror>(rt.m), dpp_d<kDppRowHalfMirror>(rt.s));
    st = RowStats{readlane_f(rt.m, 0), 1.0 / readlane_d(rt.s, 0)};
    if (D) {
        online_merge(rd, dpp_f<kDppQuadXor1>(rd.m), dpp_d<kDppQuadXor1>(rd.s));
        online_merge(rd, dpp_f<kDppQuadXor2>(rd.m), dpp_d<kDppQuadXor2>(rd.s));
        online_merge(rd, dpp_f<kDppRowHalfMirror>(rd.m), dpp_d<kDppRowHalfMirror>(rd.s));
        sd = RowStats{readlane_f(rd.m, 0), 1.0 / readlane_d(rd.s, 0)};
    }
    __syncthreads();  // s_words is reused by the next exchange
}

// Slice totals of the draw weights: this slice's table into seg (its total
// published into set[g]); all G totals into s_tot, in slice order.
template <class Src, class MakeSrc>
__device__ void sliced_totals(unsigned long long* set, int G, int g, int m, int nseg_max, int Ls, int V, double* seg,
                              int wait_limit, unsigned long long* s_words, int* s_ready, double* s_tot,
                              MakeSrc make) {
    const int64_t L = (int64_t)m * kSub;
    auto nseg_of = [&](int k) {
        const int64_t len = min((int64_t)Ls, (int64_t)V - (int64_t)k * Ls);
        return (int)((len + L - 1) / L);
    };
    const Src mine = make(g);
    const double Sg = segment_totals<kSliceWaves>(mine, m, nseg_of(g), seg);
    publish_word(set + g, (unsigned long long)__double_as_longlong(Sg));
    if (gather_words(set, G, wait_limit, s_words, s_ready)) {
        if (threadIdx.x < G) s_tot[threadIdx.x] = __longlong_as_double((long long)s_words[threadIdx.x]);
    } else {
        double* scratch = seg + nseg_max;  // keep this slice's table intact
        for (int k = 0; k < G; ++k) {
            const double Sk = segment_totals<kSliceWaves>(make(k), m, nseg_of(k), scratch);
            if (threadIdx.x == 0) s_tot[k] = Sk;
            __syncthreads();
        }
    }
    __syncthreads();
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kSliceThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void accept_logits_sliced_kernel(
    const void* __restrict__ zt, const void* __restrict__ zd, int K, int V, int G, int Ls, int m, int nseg_max, float c,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ lens, const float* __restrict__ uniforms,
    int32_t* __restrict__ n_accepted, int32_t* __restrict__ next_token, unsigned long long* __restrict__ slots,
    int wait_limit) {
    extern __shared__ double seg[];  // 2 * nseg_max: this slice's table, then a scratch table
    __shared__ StatsLds lds;
    __shared__ unsigned long long s_words[2 * kMaxSlices];
    __shared__ double s_tot[kMaxSlices];
    __shared__ int s_ready;
    using L = Logit4<BF16>;
    constexpr int kElem = BF16 ? 2 : 4;
    const int b = blockIdx.x / G, g = blockIdx.x - b * G;
    const int kb = clamp_len(lens, b, K);
    const size_t row_bytes = (size_t)V * kElem;
    const char* tbase = (const char*)zt + (size_t)b * (size_t)(K + 1) * row_bytes;
    const char* dbase = (const char*)zd + (size_t)b * (size_t)K * row_bytes;
    const int64_t x0 = (int64_t)g * Ls;
    const int len = (int)min((int64_t)Ls, (int64_t)V - x0);
    unsigned long long* my = slots + (size_t)b * (size_t)((K + 1) * 2 * G + 2 * G);
    unsigned long long* draw_sets = my + (size_t)(K + 1) * 2 * G;

    // 1. positions in order; stop at the first rejection
    int n = kb;
    bool have = false;
    RowStats st{0.f, 0.0}, sd{0.f, 0.0};
    for (int i = 0; i < kb; ++i) {
        const int t = tokens[(int64_t)b * K + i];
        if (t < 0 || t >= V) {  // out-of-range draft token: rejected, never dereferenced
            n = i;
            break;
        }
        const void* tr = tbase + (size_t)i * row_bytes;
        const void* dr = dbase + (size_t)i * row_bytes;
        sliced_row_stats<BF16, VEC, true>(my + (size_t)i * 2 * G, G, g, Ls, V, tr, dr, c, &lds, wait_limit, s_words,
                                          &s_ready, st, sd);
        if (!accepts(L::at(tr, t), L::at(dr, t), c, st, sd, uniforms[(int64_t)b * (K + 1) + i])) {
            n = i;
            have = true;
            break;
        }
    }

    // 2-3. the draw, slice by slice
    const bool residual = n < kb;
    const int pos = residual ? n : kb;
    const char* zt_row = tbase + (size_t)pos * row_bytes;
    const char* zd_row = residual ? dbase + (size_t)n * row_bytes : nullptr;
    if (!(residual && have)) {
        if (residual)
            sliced_row_stats<BF16, VEC, true>(my + (size_t)pos * 2 * G, G, g, Ls, V, zt_row, zd_row, c, &lds,
                                              wait_limit, s_words, &s_ready, st, sd);
        else
            sliced_row_stats<BF16, VEC, false>(my + (size_t)pos * 2 * G, G, g, Ls, V, zt_row, nullptr, c, &lds,
                                               wait_limit, s_words, &s_ready, st, sd);
    }
    using Res = LogitSource<BF16, VEC, true>;
    using Bon = LogitSource<BF16, VEC, false>;
    auto slice_len = [&](int k) { return (int)min((int64_t)Ls, (int64_t)V - (int64_t)k * Ls); };
    const Shift k0 = residual ? residual_shift(st, sd) : Shift{0.f, 0.f};
    auto make_res = [&](int k) {
        return Res{zt_row + (size_t)k * Ls * kElem, zd_row + (size_t)k * Ls * kElem, slice_len(k), c, st, sd, k0};
    };
    auto make_bon = [&](int k) {
        return Bon{zt_row + (size_t)k * Ls * kElem, nullptr, slice_len(k), c, st, sd, Shift{0.f, 0.f}};
    };
    bool use_bon = !residual;
    if (residual)
        sliced_totals<Res>(draw_sets, G, g, m, nseg_max, Ls, V, seg, wait_limit, s_words, &s_ready, s_tot, make_res);
    else
        sliced_totals<Bon>(draw_sets, G, g, m, nseg_max, Ls, V, seg, wait_limit, s_words, &s_ready, s_tot, make_bon);
    double S = 0.0;
    for (int k = 0; k < G; ++k) S += s_tot[k];
    if (residual && !(S > 0.0)) {
        // p_n == q_n: no residual mass, draw from max(0, p_n)
        use_bon = true;
        sliced_totals<Bon>(draw_sets + G, G, g, m, nseg_max, Ls, V, seg, wait_limit, s_words, &s_ready, s_tot,
                           make_bon);
        S = 0.0;
        for (int k = 0; k < G; ++k) S += s_tot[k];
    }
    if (g == 0 && threadIdx.x == 0) {
        n_accepted[b] = n;
        if (!(S > 0.0)) next_token[b] = -1;
    }
    if (!(S > 0.0)) return;
    // the slice holding u * S: the first with positive total whose running sum
    // exceeds it; if rounding leaves none, the last with positive total
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
    if (g != ks || threadIdx.x >= kWave) return;
    const int nseg = (len + (int)((int64_t)m * kSub) - 1) / (int)((int64_t)m * kSub);
    const int x = use_bon ? locate(make_bon(g), m, nseg, seg, thr_local) : locate(make_res(g), m, nseg, seg, thr_local);
    if (threadIdx.x == 0) next_token[b] = x < 0 ? -1 : (int)(x0 + x);
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

// Slices of the sliced verify kernels: at most 8, B * G <= 4096 workgroups of
// 256 lanes (twice what the chip holds at once; the dispatch order keeps a
// sequence's slices together), each slice at least 32768 elements (shorter
// slices spend more on the exchanges than they save); Ls is a multiple of 1024
// elements and every slice is non-empty. Measured on MI355X at B = 512,
// K = 16, V = 256000 for the fused sampled verify: G = 8 about 8% faster than
// G = 4 and 27% faster than G = 2.
void coop_slice_shape(int B, int V, int& G, int& Ls) {
    int g = 4096 / (B > 0 ? B : 1);
    g = g < 1 ? 1 : (g > kMaxSlices ? kMaxSlices : g);
    const int gv = (int)(((int64_t)V + 32767) / 32768);  // V may be INT32_MAX
    g = g < gv ? g : (gv > 1 ? gv : 1);
    int64_t ls = ((int64_t)V + g - 1) / g;
    ls = (ls + 1023) / 1024 * 1024;
    G = (int)(((int64_t)V + ls - 1) / ls);
    Ls = (int)ls;
}

hipError_t launch_fill_empty(unsigned long long* slots, int64_t words, hipStream_t stream) {
    if (words <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_empty, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream, slots, words);
    return hipGetLastError();
}

size_t accept_logits_workspace_bytes(int B, int K, int V) {
    int G, Ls;
    coop_slice_shape(B, V, G, Ls);
    if (G < 2) return 0;
    return (size_t)B * ((size_t)(K + 1) * 2 * G + 2 * (size_t)G) * sizeof(unsigned long long);
}

hipError_t launch_accept_logits(const void* zt, const void* zd, bool bf16, int B, int K, int V, float temperature,
                                const int32_t* tokens, const int32_t* lens, const float* uniforms,
                                int32_t* n_accepted, int32_t* next_token, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    const float c = 1.4426950408889634f / temperature;
    const uintptr_t al = bf16 ? 8 : 16;
    const bool vec = (V % 4 == 0) && ((uintptr_t)zt % al == 0) && ((uintptr_t)zd % al == 0);
    const size_t need = accept_logits_workspace_bytes(B, K, V);
    if (need > 0 && workspace && workspace_bytes >= need && (uintptr_t)workspace % 8 == 0) {
        int G, Ls, m, nseg;
        coop_slice_shape(B, V, G, Ls);
        segment_shape(Ls, m, nseg);
        const int64_t words = (int64_t)(need / sizeof(unsigned long long));
        unsigned long long* slots = (unsigned long long*)workspace;
        const hipError_t fe = launch_fill_empty(slots, words, stream);
        if (fe != hipSuccess) return fe;  // without the fill, stale slots would read as published
        const size_t lds = 2 * (size_t)nseg * sizeof(double);
        const dim3 grid((unsigned)B * (unsigned)G), block(kSliceThreads);
        const int wl = get_wait_limit();
        if (bf16) {
            if (vec)
                hipLaunchKernelGGL((accept_logits_sliced_kernel<true, true>), grid, block, lds, stream, zt, zd, K, V, G,
                                   Ls, m, nseg, c, tokens, lens, uniforms, n_accepted, next_token, slots, wl);
            else
                hipLaunchKernelGGL((accept_logits_sliced_kernel<true, false>), grid, block, lds, stream, zt, zd, K, V, G,
                                   Ls, m, nseg, c, tokens, lens, uniforms, n_accepted, next_token, slots, wl);
        } else {
            if (vec)
                hipLaunchKernelGGL((accept_logits_sliced_kernel<false, true>), grid, block, lds, stream, zt, zd, K, V, G,
                                   Ls, m, nseg, c, tokens, lens, uniforms, n_accepted, next_token, slots, wl);
            else
                hipLaunchKernelGGL((accept_logits_sliced_kernel<false, false>), grid, block, lds, stream, zt, zd, K, V,
                                   G, Ls, m, nseg, c, tokens, lens, uniforms, n_accepted, next_token, slots, wl);
        }
        return hipGetLastError();
    }
    int m, nseg;
    segment_shape(V, m, nseg);
    const size_t lds = (size_t)nseg * sizeof(double);
    if (bf16) {
        if (vec)
            hipLaunchKernelGGL((accept_logits_kernel<true, true>), dim3(B), dim3(kThreads), lds, stream, zt, zd, K, V,
                               m, nseg, c, tokens, lens, uniforms, n_accepted, next_token);
        else
            hipLaunchKernelGGL((accept_logits_kernel<true, false>), dim3(B), dim3(kThreads), lds, stream, zt, zd, K,
                               V, m, nseg, c, tokens, lens, uniforms, n_accepted, next_token);
    } else {
        if (vec)
            hipLaunchKernelGGL((accept_logits_kernel<false, true>), dim3(B), dim3(kThreads), lds, stream, zt, zd, K,
                               V, m, nseg, c, tokens, lens, uniforms, n_accepted, next_token);
        else
            hipLaunchKernelGGL((accept_logits_kernel<false, false>), dim3(B), dim3(kThreads), lds, stream, zt, zd, K,
                               V, m, nseg, c, tokens, lens, uniforms, n_accepted, next_token);
    }
    return hipGetLastError();
}

}  // namespace sv
