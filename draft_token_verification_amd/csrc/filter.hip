// filter.hip -- filtered warp for gfx950: temperature, top-k, top-p, then
// renormalisation, in the order of the sampler pipeline the llmstudio blog
// ("Как работает speculative decoding и MTP при инференсе LLM", section 38)
// lays out. Target and draft rows go through the same filters, so the
// sampled verify compares the distributions the sampler would draw from.
//
// Semantics (ids with probability 0 are filtered out):
//   top-k  keeps every id whose logit is at least the k-th largest logit
//          (ties at the boundary are all kept); k <= 0 or k >= V: off.
//   top-p  acts on the top-k survivors renormalised: an id is kept iff the
//          mass of the ids strictly more probable than it is below top_p
//          times the survivors' mass; equal logits share one decision; the
//          largest logit is always kept; top_p >= 1 or NaN: off.
//
// One workgroup of 1024 lanes per live row. The thresholds are found by a
// radix descent over order-preserving integer keys of the logits (16-bit keys
// for bf16, 32-bit for fp32; -0.0 is folded into +0.0 so that equal values
// have equal keys), one 8-bit digit per pass over the row:
//   top-k  counts per digit, among the keys that match the digits chosen so
//          far, give the digit of the k-th largest key;
//   top-p  masses per digit, 2^(z*c - M) (c = log2(e)/T, M = c * max z) in
//          fixed point (integers, 2^fxs per unit), give the digit of the last
//          kept value. Integer sums are exact and order-free, so the descent is
//          deterministic and a bin's mass equals the sum of its sub-bins.
// Counts and masses go into per-wavefront histograms in LDS (integer atomics)
// and are summed over the wavefronts between passes. The final pass writes
// 2^(z*c - M) / S_kept for kept ids and 0 elsewhere. Passes after the first
// re-read the row from the caches in front of HBM.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 256;
constexpr int kUnroll = 4;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order-preserving key of a logit: a < b  <=>  key(a) < key(b), equal
// values (including -0.0 and +0.0) give equal keys. bf16 values use the top
// 16 bits of the fp32 key (their low 16 bits carry no information).
template <bool BF16>
__device__ __forceinline__ uint32_t key_of(float z) {
    uint32_t u = __float_as_uint(z);
    u = (u == 0x80000000u) ? 0u : u;
    const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return BF16 ? (k >> 16) : k;
}

// round(e * 2^fxs) for 0 <= e <= ~1, exactly, without a 64-bit float convert.
__device__ __forceinline__ unsigned long long fixed_of(float e, int fxs) {
    const uint32_t b = __float_as_uint(e);
    const int E = (int)(b >> 23);
    if (E == 0) return 0ull;  // zero or below 2^-126
    const unsigned long long mant = (b & 0x7FFFFFu) | 0x800000u;  // e = mant * 2^(E - 150)
    const int sh = E - 150 + fxs;
    if (sh >= 0) return mant << sh;
    if (sh < -24) return 0ull;
    return (mant + (1ull << (-sh - 1))) >> (-sh);
}

// Element access: VEC rows are read 16 bytes per lane (8 bf16 or 4 fp32).
template <bool BF16>
struct Elems;

template <>
struct Elems<true> {
    static constexpr int N = 8;
    __device__ static void unpack(const u32x4& r, float z[8]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            z[2 * k] = bf16_lo(r[k]);
            z[2 * k + 1] = bf16_hi(r[k]);
        }
    }
    __device__ static float at(const void* row, int64_t i) { return bf16_at((const uint16_t*)row, i); }
};

template <>
struct Elems<false> {
    static constexpr int N = 4;
    __device__ static void unpack(const u32x4& r, float z[4]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) z[k] = __uint_as_float(r[k]);
    }
    __device__ static float at(const void* row, int64_t i) { return ((const float*)row)[i]; }
};

// Calls f(z, x) for every element of the row (each lane its own subset).
template <bool BF16, bool VEC, class F>
__device__ __forceinline__ void for_each(const void* row, int V, F&& f) {
    using E = Elems<BF16>;
    const int tid = threadIdx.x;
    if (VEC) {
        const u32x4* v = (const u32x4*)row;
        const int nv = V / E::N;
        int j = tid;
        for (; j + (kUnroll - 1) * kThreads < nv; j += kUnroll * kThreads) {
            u32x4 raw[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) raw[u] = v[j + u * kThreads];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float z[E::N];
                E::unpack(raw[u], z);
#pragma unroll
                for (int k = 0; k < E::N; ++k) f(z[k], (int64_t)(j + u * kThreads) * E::N + k);
            }
        }
        for (; j < nv; j += kThreads) {
            float z[E::N];
            E::unpack(v[j], z);
#pragma unroll
            for (int k = 0; k < E::N; ++k) f(z[k], (int64_t)j * E::N + k);
        }
    } else {
        for (int x = tid; x < V; x += kThreads) f(E::at(row, x), (int64_t)x);
    }
}

struct FilterLds {
    uint32_t cnt[kWaves][kBins];
    unsigned long long mass[kWaves][kBins];
    uint32_t tcnt[kBins];
    unsigned long long tmass[kBins];
    float wmax[kWaves];
};

// Sum the per-wavefront histograms into the totals and clear them for the
// next pass. Barrier before (the pass's atomics) and after (the totals).
__device__ __forceinline__ void reduce_hist(FilterLds* L, bool counts, bool masses) {
    __syncthreads();
    const int t = threadIdx.x;
    if (t < kBins) {
        uint32_t c = 0;
        unsigned long long m = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            if (counts) c += L->cnt[w][t];
            if (masses) m += L->mass[w][t];
        }
        L->tcnt[t] = c;
        L->tmass[t] = m;
    }
    // clearing: every (wave, bin) entry of the kind used, 4 per thread
    for (int i = t; i < kWaves * kBins; i += kThreads) {
        if (counts) (&L->cnt[0][0])[i] = 0u;
        if (masses) (&L->mass[0][0])[i] = 0ull;
    }
    __syncthreads();
}

__device__ __forceinline__ unsigned long long shfl_up_u64(unsigned long long v, int d) {
    const int lo = __shfl_up((int)(uint32_t)v, d, kWave), hi = __shfl_up((int)(uint32_t)(v >> 32), d, kWave);
    return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int l) {
    const uint32_t lo = (uint32_t)readlane_i((int)(uint32_t)v, l), hi = (uint32_t)readlane_i((int)(uint32_t)(v >> 32), l);
    return ((unsigned long long)hi << 32) | lo;
}

// Scan the 256 bin totals from the highest bin down (lane j holds bins
// 255-4j .. 252-4j) and return the first bin d whose cumulative value before
// it, C = base + sum of the bins above d, satisfies hit(C, C + bin[d]). Also
// returns that C. Executed by every wavefront alike; the result is uniform.
template <class Hit>
__device__ __forceinline__ int find_bin(const unsigned long long* tot, unsigned long long base, Hit hit,
                                        unsigned long long& before) {
    const int lane = threadIdx.x & (kWave - 1);
    unsigned long long v[4], run = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = tot[kBins - 1 - 4 * lane - i];
        run += v[i];
    }
    unsigned long long incl = run;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const unsigned long long y = shfl_up_u64(incl, d);
        if (lane >= d) incl += y;
    }
    unsigned long long c = base + (incl - run);
    int found = -1;
    unsigned long long cf = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (found < 0 && hit(c, c + v[i])) {
            found = i;
            cf = c;
        }
        c += v[i];
    }
    const unsigned long long ball = __ballot(found >= 0);
    if (ball == 0ull) {
        before = 0;
        return -1;
    }
    const int l = __builtin_ctzll(ball);
    const int i = readlane_i(found, l);
    before = readlane_u64(cf, l);
    return kBins - 1 - 4 * l - i;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void warp_filter_kernel(const void* __restrict__ logits, int R, int V,
                                                          const int32_t* __restrict__ lens, int extra_rows,
                                                          float c, const int32_t* __restrict__ top_k,
                                                          const float* __restrict__ top_p, int fxs,
                                                          float* __restrict__ probs) {
    constexpr int kBits = BF16 ? 16 : 32;
    constexpr int kLevels = kBits / 8;
    __shared__ FilterLds L;
    const int row = blockIdx.x;
    const int b = row / R, r = row - b * R;
    const int live = clamp_len(lens, b, R - extra_rows) + extra_rows;
    if (r >= live) return;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const char* zrow = (const char*)logits + (size_t)row * (size_t)V * (BF16 ? 2 : 4);
    float* prow = probs + (size_t)row * (size_t)V;

    const int k = top_k ? top_k[b] : 0;
    const bool kon = k > 0 && k < V;
    const float pp = top_p ? top_p[b] : 1.0f;
    const bool pon = pp < 1.0f;  // false for NaN

    for (int i = tid; i < kWaves * kBins; i += kThreads) {
        (&L.cnt[0][0])[i] = 0u;
        (&L.mass[0][0])[i] = 0ull;
    }
    __syncthreads();

    // pass 1: the row maximum, and the top digit's counts for top-k
    float zmax = -INFINITY;
    for_each<BF16, VEC>(zrow, V, [&](float z, int64_t) {
        zmax = fmaxf(zmax, z);
        if (kon) atomicAdd(&L.cnt[wave][key_of<BF16>(z) >> (kBits - 8)], 1u);
    });
    {
        float m = zmax;
        m = fmaxf(m, dpp_f<kDppQuadXor1>(m));
        m = fmaxf(m, dpp_f<kDppQuadXor2>(m));
        m = fmaxf(m, dpp_f<kDppRowHalfMirror>(m));
        m = fmaxf(m, dpp_f<kDppRowMirror>(m));
        m = fmaxf(m, swz16_f(m));
        m = fmaxf(readlane_f(m, 0), readlane_f(m, 32));
        if (lane == 0) L.wmax[wave] = m;
    }
    __syncthreads();
    {
        float m = lane < kWaves ? L.wmax[lane] : -INFINITY;
        m = fmaxf(m, dpp_f<kDppQuadXor1>(m));
        m = fmaxf(m, dpp_f<kDppQuadXor2>(m));
        m = fmaxf(m, dpp_f<kDppRowHalfMirror>(m));
        m = fmaxf(m, dpp_f<kDppRowMirror>(m));
        m = fmaxf(m, swz16_f(m));
        zmax = fmaxf(readlane_f(m, 0), readlane_f(m, 32));
    }
    const float Mc = zmax * c;

    // top-k: descend to the key of the k-th largest logit
    uint32_t tau_k = 0u;
    if (kon) {
        uint32_t prefix = 0u;
        unsigned long long need = (unsigned long long)k;
        for (int l = 0; l < kLevels; ++l) {
            const int sh = kBits - 8 * (l + 1);
            if (l > 0) {
                for_each<BF16, VEC>(zrow, V, [&](float z, int64_t) {
                    const uint32_t key = key_of<BF16>(z);
                    if ((key >> (sh + 8)) == prefix) atomicAdd(&L.cnt[wave][(key >> sh) & 0xFFu], 1u);
                });
            }
            reduce_hist(&L, true, false);
            // totals as 64-bit for the common scan
            unsigned long long* tot = L.tmass;
            if (tid < kBins) tot[tid] = L.tcnt[tid];
            __syncthreads();
            unsigned long long before;
            const int d = find_bin(tot, 0ull,
                                   [&](unsigned long long lo, unsigned long long hi) { return lo < need && need <= hi; },
                                   before);
            need -= before;
            prefix = (prefix << 8) | (uint32_t)(d < 0 ? 0 : d);
            __syncthreads();  // tot is rewritten by the next reduction
        }
        tau_k = prefix;
    }

    // masses of the survivors by top digit; top-p descends from there
    uint32_t tau = tau_k;
    unsigned long long s_kept = 0;
    {
        uint32_t prefix = 0u;
        unsigned long long base = 0;
        double target = 0.0;
        for (int l = 0; l < (pon ? kLevels : 1); ++l) {
            const int sh = kBits - 8 * (l + 1);
            for_each<BF16, VEC>(zrow, V, [&](float z, int64_t) {
                const uint32_t key = key_of<BF16>(z);
                if (key >= tau_k && (l == 0 || (key >> (sh + 8)) == prefix)) {
                    const unsigned long long f = fixed_of(ex2(fmaf(z, c, -Mc)), fxs);
                    if (f) atomicAdd(&L.mass[wave][(key >> sh) & 0xFFu], f);
                }
            });
            reduce_hist(&L, false, true);
            if (l == 0) {
                unsigned long long s = 0;
                for (int i = lane; i < kBins; i += kWave) s += L.tmass[i];
                // wave sum of 64-bit integers (exact, any order)
#pragma unroll
                for (int d = 1; d < kWave; d <<= 1) s += shfl_up_u64(s, d) * (lane >= d);
                s_kept = readlane_u64(s, kWave - 1);
                if (!pon) break;
                target = (double)pp * (double)s_kept;
                if (!(target > 0.0)) target = 0.5;  // top_p <= 0: keep the largest value only
            }
            unsigned long long before;
            const int d = find_bin(L.tmass, base,
                                   [&](unsigned long long lo, unsigned long long hi) {
                                       return (double)lo < target && target <= (double)hi;
                                   },
                                   before);
            base = before;
            prefix = (prefix << 8) | (uint32_t)(d < 0 ? 0 : d);  // d >= 0 by construction (finite logits)
            if (l == kLevels - 1) {
                tau = prefix;
                s_kept = before + L.tmass[d < 0 ? 0 : d];
            }
            __syncthreads();  // the totals are rewritten by the next reduction
        }
    }

    // final pass: normalised kept probabilities, zeros elsewhere
    const float inv = (float)(ldexp(1.0, fxs) / (double)s_kept);
    if (VEC) {
        using E = Elems<BF16>;
        const u32x4* v = (const u32x4*)zrow;
        f32x4* out = (f32x4*)prow;
        const int nv = V / E::N;
        for (int j = tid; j < nv; j += kThreads) {
            float z[E::N];
            E::unpack(v[j], z);
#pragma unroll
            for (int h = 0; h < E::N / 4; ++h) {
                f32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float zz = z[4 * h + q];
                    o[q] = key_of<BF16>(zz) >= tau ? ex2(fmaf(zz, c, -Mc)) * inv : 0.0f;
                }
                store_nt(out + (int64_t)j * (E::N / 4) + h, o);
            }
        }
    } else {
        for (int x = tid; x < V; x += kThreads) {
            const float zz = Elems<BF16>::at(zrow, x);
            prow[x] = key_of<BF16>(zz) >= tau ? ex2(fmaf(zz, c, -Mc)) * inv : 0.0f;
        }
    }
}

}  // namespace

// 2^fxs fixed-point units per unit of mass, so that V masses of at most ~1 sum
// below 2^62.
static int fixed_shift(int V) {
    int bits = 0;
    while ((1ll << bits) < (long long)V) ++bits;
    return 62 - bits;
}

hipError_t launch_warp_filtered(const void* logits, bool bf16, int B, int R, int V, const int32_t* lens,
                                int extra_rows, float temperature, const int32_t* top_k, const float* top_p,
                                float* probs, hipStream_t stream) {
    const float c = 1.4426950408889634f / temperature;
    const int fxs = fixed_shift(V);
    const dim3 grid((unsigned)B * (unsigned)R);
    const int n = bf16 ? 8 : 4;
    const bool vec = (V % n == 0) && ((uintptr_t)logits % 16 == 0) && ((uintptr_t)probs % 16 == 0);
    if (bf16) {
        if (vec)
            hipLaunchKernelGGL((warp_filter_kernel<true, true>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, c, top_k, top_p, fxs, probs);
        else
            hipLaunchKernelGGL((warp_filter_kernel<true, false>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, c, top_k, top_p, fxs, probs);
    } else {
        if (vec)
            hipLaunchKernelGGL((warp_filter_kernel<false, true>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, c, top_k, top_p, fxs, probs);
        else
            hipLaunchKernelGGL((warp_filter_kernel<false, false>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, c, top_k, top_p, fxs, probs);
    }
    return hipGetLastError();
}

}  // namespace sv
