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
// One workgroup of 1024 lanes per live row. The first pass over the row
// finds the row maximum M (logits in log2 units, y = z*c - M with
// c = log2(e)/T), the softmax sum when the row has no top-k (top-p needs it
// as the reference mass; top-k rows skip the exponentials), and, per
// wavefront, collects the keys of the logits within 20 log2 units of its
// running maximum into LDS.
//   common path  the k-th largest collected key comes from a bitwise search
//                with block-wide counts; for top-p, up to 64 top-k survivors
//                are sorted in a wavefront (bitonic network) and the nucleus
//                read off their prefix masses, one decision per group of
//                equal keys; with more, the nucleus's last key comes from a
//                bitwise search with block-wide masses instead. It
//                applies when the collected set holds at least k ids and
//                (top-p alone) the nucleus ends inside it; a wavefront whose
//                buffer overflows keeps only its largest keys (a key floor),
//                and the common path then needs k and the nucleus above the
//                highest floor.
//   general path a radix descent over order-preserving integer keys of the
//                logits (16-bit keys for bf16, 32-bit for fp32; -0.0 folded
//                into +0.0 so that equal values have equal keys), one 8-bit
//                digit per pass over the row: counts per digit among the keys
//                that match the digits chosen so far give the digit of the
//                k-th largest key; masses per digit, restricted to the top-k
//                survivors, give the digit of the last kept value. Counts and
//                masses go into per-wavefront histograms in LDS (integer
//                atomics), summed over the wavefronts between passes.
// Masses are 2^y in fixed point (integers, 2^fxs per unit) on both paths:
// integer sums are exact and order-free, so the thresholds are deterministic.
// The paths agree exactly except for top-p without top-k, where the common
// path takes the whole row's mass from the fp32 statistics (relative error
// ~1e-6) instead of an exact sum. The last pass writes 2^y / S_kept for kept
// ids and 0 elsewhere. When the common path decides, the candidates' element
// ids (kept beside their keys) mark the quads of four elements that hold a
// kept id in a bit map in LDS, and the last pass writes every other quad as
// zeros without reading it: the row is read from HBM once. The general path's
// passes, and the last pass without the map, re-read the row.
#include <math.h>

#include <type_traits>

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

// Online (max, sum) of y = z*c in log2 units over N elements (-inf skipped):
// m is the running max, s = sum 2^(y - m).
template <int N>
__device__ __forceinline__ void online_addf(const float* z, float c, float& m, float& s) {
    float zm = z[0];
#pragma unroll
    for (int k = 1; k < N; ++k) zm = fmaxf(zm, z[k]);
    const float ym = zm * c;
    if (ym > m) {
        s = (m == -INFINITY) ? 0.0f : s * ex2(m - ym);
        m = ym;
    }
    if (m == -INFINITY) return;
#pragma unroll
    for (int k = 0; k < N; ++k) s += ex2(fmaf(z[k], c, -m));
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
    uint32_t cnt[kWaves][kBins];             // also: the candidate keys (kCand of them)
    unsigned long long mass[kWaves][kBins];  // also: the candidates' exclusive prefix masses, then the
                                             // map of the quads that hold a kept id
    uint32_t ids[kWaves * kBins];            // the candidates' element ids, beside their keys
    uint32_t tcnt[kBins];
    unsigned long long tmass[kBins];
    unsigned long long wmass[2][kWaves];  // per-wavefront partials of the threshold searches
    int wnum[2][kWaves];
    float wmax[kWaves];
    float wsum_f[kWaves];
    int wcnt[kWaves];
};

constexpr int kCand = kWaves * kBins;  // candidates the sorted path holds (4096)
constexpr float kSpan = 20.0f;         // candidates: logits within 20 log2 units of the maximum

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

// Inverse of key_of: the logit a key stands for (+0.0 for the folded zeros).
template <bool BF16>
__device__ __forceinline__ float value_of(uint32_t key) {
    const uint32_t k = BF16 ? ((key << 16) | ((key & 0x8000u) ? 0u : 0xFFFFu)) : key;
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

constexpr int kWaveCap = kCand / kWaves;  // candidate slots per wavefront (256)

__device__ __forceinline__ float wave_max_f(float m) {
    m = fmaxf(m, dpp_f<kDppQuadXor1>(m));
    m = fmaxf(m, dpp_f<kDppQuadXor2>(m));
    m = fmaxf(m, dpp_f<kDppRowHalfMirror>(m));
    m = fmaxf(m, dpp_f<kDppRowMirror>(m));
    m = fmaxf(m, swz16_f(m));
    return fmaxf(readlane_f(m, 0), readlane_f(m, 32));
}

// Keep the entries of a wavefront's candidate buffer (keys in buf, element
// ids in ibuf) whose key is above fkey and whose logit lies within kSpan log2
// units of `run`, packed to the front. Wave-local and in place, 64 entries
// per step: a step's writes land below the entries of every later step, and
// the wavefront reads a step's entries before it writes any of them.
template <bool BF16>
__device__ __forceinline__ int wave_compact(uint32_t* buf, uint32_t* ibuf, int cnt, float c, float run,
                                            uint32_t fkey) {
    const int lane = threadIdx.x & (kWave - 1);
    int n = 0;
#pragma unroll
    for (int q = 0; q < kWaveCap / kWave; ++q) {
        const int i = q * kWave + lane;
        const uint32_t e = i < cnt ? buf[i] : 0u;
        const uint32_t id = i < cnt ? ibuf[i] : 0u;
        const bool keep = i < cnt && e > fkey && fmaf(value_of<BF16>(e), c, -run) > -kSpan;
        const uint64_t m = __ballot(keep);
        if (keep) {
            const int at = n + __popcll(m & ((1ull << lane) - 1ull));
            buf[at] = e;
            ibuf[at] = id;
        }
        n += __popcll(m);
    }
    return n;
}

// The smallest key f such that at most `room` entries have key > f, counting
// the buffer and the step's pending elements (z[e] where bit e of want is
// set); bitwise search over the key's bits. Wave-local, uniform result.
template <bool BF16, int N>
__device__ __forceinline__ uint32_t wave_floor(const uint32_t* buf, int cnt, int room, const float* z, uint32_t want) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t e[kWaveCap / kWave];
#pragma unroll
    for (int q = 0; q < kWaveCap / kWave; ++q) {
        const int i = q * kWave + lane;
        e[q] = i < cnt ? buf[i] : 0u;
    }
    uint32_t f = 0u;
#pragma unroll 1
    for (int bit = BF16 ? 15 : 31; bit >= 0; --bit) {
        const uint32_t t = f | ((1u << bit) - 1u);  // keep bit clear, all lower set
        int n = 0;
#pragma unroll
        for (int q = 0; q < kWaveCap / kWave; ++q) n += __popcll(__ballot(e[q] > t));
#pragma unroll
        for (int q = 0; q < N; ++q) n += __popcll(__ballot(((want >> q) & 1u) && key_of<BF16>(z[q]) > t));
        if (n > room) f |= 1u << bit;  // must go higher
    }
    return f;
}

// First pass over a row: the softmax statistics (y = z*c in log2 units;
// Mc = max y and, when `stats`, S = sum 2^(y - Mc) in fp32 as the plain warp;
// S = 0 otherwise) and, per wavefront, the keys of its logits that lie within
// kSpan log2 units of its running maximum and above its key floor. When a
// step's entries do not fit, the buffer is compacted; if that is not enough
// the floor rises so that at most 64 of the buffer's and the step's entries
// stay above it. Entries only ever leave for being below the row's window or
// the floor, so at the end the set {key > F, y > Mc - kSpan} (F: the highest
// floor) is complete: their keys are packed into cand[0 .. nc) (any order)
// and their element ids into ids[0 .. nc) in the same order.
// The per-element test is one float comparison against the larger of the
// window's lower end (rounded down by a safe margin, so the gather never
// misses an id the final set holds) and the value of the floor's key.
// Without `gather` (a row with neither filter) only the statistics are
// formed and the list stays empty.
template <bool BF16, bool VEC>
__device__ __forceinline__ void gather_pass(const void* zrow, int V, float c, bool stats, bool gather, FilterLds* L,
                                            float& Mc, float& S, int& nc) {
    using E = Elems<BF16>;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    uint32_t* buf = &L->cnt[0][0] + wave * kWaveCap;
    uint32_t* ibuf = L->ids + wave * kWaveCap;
    const float inv_c = 1.0f / c;
    float om = -INFINITY, os = 0.0f;  // this lane's online statistics
    float run = -INFINITY;            // the wavefront's running maximum (log2 units)
    uint32_t fkey = 0u;               // the wavefront's key floor
    float zf = -INFINITY;             // the logit of the floor's key (-inf: no floor)
    int cnt = 0;                      // entries in buf (wave-uniform)
    // The wavefronts' floors, published in LDS: a floor bounds the final set
    // (only keys above the highest floor remain), so each wavefront adopts
    // the highest published one before it takes elements. Reading a stale,
    // lower value only lets more elements in.
    uint32_t* floors = (uint32_t*)L->wcnt;
    if (lane == 0) floors[wave] = 0u;
    __syncthreads();
    auto adopt_floor = [&]() {
        uint32_t g = lane < kWaves ? __hip_atomic_load(&floors[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                                   : 0u;
        g = max(g, (uint32_t)dpp_i<kDppQuadXor1>((int)g));
        g = max(g, (uint32_t)dpp_i<kDppQuadXor2>((int)g));
        g = max(g, (uint32_t)dpp_i<kDppRowHalfMirror>((int)g));
        g = max(g, (uint32_t)dpp_i<kDppRowMirror>((int)g));  // lanes 0..15 hold the highest floor
        g = (uint32_t)readlane_i((int)g, 0);
        if (g > fkey) {
            fkey = g;
            zf = value_of<BF16>(g);
        }
    };
    // out-of-row elements come in as -inf: never above a threshold
    // running maximum first, so that the test in take() is as tight as possible
    float zlo = -INFINITY;  // the window's lower end for the current step
    auto update_run = [&](const float* z, auto n_const) {
        constexpr int n = decltype(n_const)::value;
        float smax = -INFINITY;
#pragma unroll
        for (int e = 0; e < n; ++e) smax = fmaxf(smax, z[e]);
        run = fmaxf(run, wave_max_f(smax) * c);
        zlo = (run - kSpan - 1e-3f) * inv_c;
        zlo = run == -INFINITY ? -INFINITY : zlo - fabsf(zlo) * 1e-6f;
    };
    auto take = [&](const float* z, auto n_const, int id0) {  // z[e] is element id0 + e
        constexpr int n = decltype(n_const)::value;
        float thr = fmaxf(zlo, zf);
        bool any = false;
#pragma unroll
        for (int e = 0; e < n; ++e) any |= z[e] > thr;
        if (__ballot(any) == 0ull) return;  // the common case: nothing near the maximum
        uint32_t want = 0u;  // bit e: element e goes into the buffer (lane masks would cost 2 SGPRs each)
        int need = 0;
#pragma unroll
        for (int e = 0; e < n; ++e) {
            const bool w = z[e] > thr;
            want |= (uint32_t)w << e;
            need += __popcll(__ballot(w));
        }
        if (cnt + need > kWaveCap) {  // rare: make room once for the whole step
            cnt = wave_compact<BF16>(buf, ibuf, cnt, c, run, fkey);
            if (cnt + need > kWaveCap) {
                // raise the floor so that at most 64 entries remain above it
                fkey = max(fkey, wave_floor<BF16, n>(buf, cnt, kWaveCap / 4, z, want));
                zf = value_of<BF16>(fkey);
                if (lane == 0) __hip_atomic_store(&floors[wave], fkey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                cnt = wave_compact<BF16>(buf, ibuf, cnt, c, run, fkey);
                thr = fmaxf(zlo, zf);
                want = 0u;
#pragma unroll
                for (int e = 0; e < n; ++e) want |= (uint32_t)(z[e] > thr) << e;
            }
        }
#pragma unroll
        for (int e = 0; e < n; ++e) {
            const bool w = (want >> e) & 1u;
            const uint64_t m = __ballot(w);
            if (w) {
                const int at = cnt + __popcll(m & ((1ull << lane) - 1ull));
                buf[at] = key_of<BF16>(z[e]);
                ibuf[at] = (uint32_t)(id0 + e);
            }
            cnt += __popcll(m);
        }
    };
    if (VEC) {
        constexpr int U = 2;  // 16 bf16 or 8 fp32 elements per lane per step
        constexpr int N = U * E::N;
        const u32x4* v = (const u32x4*)zrow;
        const int nv = V / E::N;
        // software-pipelined: the next step's loads are in flight while this
        // step is processed (clamped indexes, so the loads are unconditional)
        u32x4 nxt[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = u * kThreads + tid;
            nxt[u] = v[j < nv ? j : 0];
        }
        for (int j0 = 0; j0 < nv; j0 += U * kThreads) {
            float z[N];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool in = j0 + u * kThreads + tid < nv;
                E::unpack(nxt[u], z + u * E::N);
#pragma unroll
                for (int e = 0; e < E::N; ++e) z[u * E::N + e] = in ? z[u * E::N + e] : -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = j0 + (U + u) * kThreads + tid;
                nxt[u] = v[j < nv ? j : 0];
            }
            if (stats) {
#pragma unroll
                for (int u = 0; u < U; ++u) online_addf<E::N>(z + u * E::N, c, om, os);
            }
            if (!gather) continue;  // a row with neither filter needs only the statistics
            update_run(z, std::integral_constant<int, N>{});
            adopt_floor();
#pragma unroll
            for (int u = 0; u < U; ++u)
                take(z + u * E::N, std::integral_constant<int, E::N>{}, (j0 + u * kThreads + tid) * E::N);
        }
    } else {
        for (int x0 = 0; x0 < V; x0 += kThreads) {
            const bool in = x0 + tid < V;
            float z[1] = {in ? E::at(zrow, x0 + tid) : -INFINITY};
            if (stats) online_addf<1>(z, c, om, os);
            if (!gather) continue;
            update_run(z, std::integral_constant<int, 1>{});
            adopt_floor();
            take(z, std::integral_constant<int, 1>{}, x0 + tid);
        }
    }
    // the row's statistics (without `stats`, the maximum is the running one)
    if (stats) wave_lse(om, os);
    if (lane == 0) {
        L->wmax[wave] = stats ? om : run;
        L->wsum_f[wave] = os;
        __hip_atomic_store(&floors[wave], fkey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    om = lane < kWaves ? L->wmax[lane] : -INFINITY;
    os = lane < kWaves ? L->wsum_f[lane] : 0.0f;
    if (stats) {
        wave_lse(om, os);
    } else {
        om = wave_max_f(om);
        os = 0.0f;
    }
    Mc = om;
    S = os;
    uint32_t F = 0u;
    for (int w = 0; w < kWaves; ++w) F = max(F, (uint32_t)L->wcnt[w]);
    __syncthreads();  // wcnt is reused below
    // final filter against the row's window and the highest floor, then pack
    const int kept = wave_compact<BF16>(buf, ibuf, cnt, c, Mc, F);
    if (lane == 0) L->wcnt[wave] = kept;
    __syncthreads();
    int off = 0, total = 0;
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) off += L->wcnt[w];
        total += L->wcnt[w];
    }
    uint32_t e[kWaveCap / kWave], id[kWaveCap / kWave];
#pragma unroll
    for (int q = 0; q < kWaveCap / kWave; ++q) {
        const int i = q * kWave + lane;
        e[q] = i < kept ? buf[i] : 0u;
        id[q] = i < kept ? ibuf[i] : 0u;
    }
    __syncthreads();  // every wavefront holds its entries before any moves
    uint32_t* cand = &L->cnt[0][0];
#pragma unroll
    for (int q = 0; q < kWaveCap / kWave; ++q) {
        const int i = q * kWave + lane;
        if (i < kept) {
            cand[off + i] = e[q];
            L->ids[off + i] = id[q];
        }
    }
    __syncthreads();
    nc = total;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int lo = __shfl_xor((int)(uint32_t)v, d, kWave), hi = __shfl_xor((int)(uint32_t)(v >> 32), d, kWave);
        v += ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
    }
    return v;
}

constexpr int kMapWords = kWaves * kBins * 2;  // the kept-quad map: 32-bit words over the mass array

// The map of the quads (4 consecutive elements) that hold a kept id: bit q of
// map[] is set iff some candidate with key >= tau has its id in quad q. It
// covers the whole row when the candidates hold every kept id (the common
// path decided). `key`/`valid` are the caller's candidates (entry
// j * kThreads + tid), ids[] their element ids. Contains barriers; the map's
// memory (the mass array) must be free on entry.
template <int kPer>
__device__ __forceinline__ void mark_kept_quads(const uint32_t* key, const bool* valid, uint32_t tau,
                                                const uint32_t* ids, int nquads, uint32_t* map) {
    const int tid = threadIdx.x;
    const int nw = (nquads + 31) / 32;
    __syncthreads();
    for (int i = tid; i < nw; i += kThreads) map[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        if (valid[j] && key[j] >= tau) {
            const uint32_t q = ids[j * kThreads + tid] / 4u;
            atomicOr(&map[q / 32u], 1u << (q % 32u));
        }
    }
    __syncthreads();
}

// The k-th largest of the candidate keys held in registers (1 <= k <= their
// count): the largest t with at least k keys >= t, found digit by digit (8
// bits, from the top) with block-wide LDS histograms of the keys that match
// the digits chosen so far. Three histograms rotate: pass p fills number
// p % 3 and clears the next one, which pass p - 2 used and every lane had
// read before the barrier of pass p - 1; so a pass needs a single barrier.
// Every lane gets the result. Contains barriers.
template <int kPer, int kBits>
__device__ __forceinline__ uint32_t radix_kth(const uint32_t* key, const bool* valid, int k, FilterLds* L) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    uint32_t* hist[3] = {L->tcnt, (uint32_t*)L->tmass, (uint32_t*)L->tmass + kBins};
    if (tid < kBins) hist[0][tid] = 0u;
    __syncthreads();
    uint32_t prefix = 0u;
    int above = 0;  // keys whose digits so far exceed the chosen ones
    int p = 0;
#pragma unroll
    for (int shift = kBits - 8; shift >= 0; shift -= 8, ++p) {
        uint32_t* h = hist[p % 3];
        // the next pass's histogram: last read two passes ago, by every lane
        // before it reached the previous pass's barrier
        if (tid < kBins) hist[(p + 1) % 3][tid] = 0u;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (valid[j] && (shift + 8 >= kBits || (key[j] >> (shift + 8)) == (prefix >> (shift + 8))))
                atomicAdd(&h[(key[j] >> shift) & (kBins - 1)], 1u);
        __syncthreads();
        // lane l holds bins 255 - 4l .. 252 - 4l: the first bin, from the top,
        // at which the count of keys at or above reaches k
        uint32_t v[4], run = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = h[kBins - 1 - 4 * lane - i];
            run += v[i];
        }
        uint32_t incl = run;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const uint32_t y = (uint32_t)__shfl_up((int)incl, d, kWave);
            if (lane >= d) incl += y;
        }
        int c = above + (int)(incl - run), found = -1, cf = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (found < 0 && c + (int)v[i] >= k) {
                found = i;
                cf = c;
            }
            c += (int)v[i];
        }
        const uint64_t ball = __ballot(found >= 0);
        const int l = __builtin_ctzll(ball);  // never empty: at least k keys match the prefix
        above = readlane_i(cf, l);
        prefix |= (uint32_t)(kBins - 1 - 4 * l - readlane_i(found, l)) << shift;
    }
    return prefix;
}

// Thresholds from the nc candidates in cand[] (every key above the gather's
// cut): tau (smallest kept key) and s_kept (fixed-point mass of the kept
// ids). Each thread holds up to 4 candidates in registers.
//   top-k  the k-th largest key: the largest t with at least k candidate keys
//          >= t, by a bitwise search with block-wide counts.
//   top-p  among the survivors of top-k (keys >= that) an id is kept iff the
//          survivors strictly above it weigh less than the target, one
//          decision per group of equal keys: up to 64 survivors are sorted in
//          a wavefront and the rule read off their exclusive prefix masses;
//          more give the last kept key by a bitwise search on block-wide
//          masses (the same key).
// S_total is the row's mass in fixed-point units (the top-p reference without
// top-k). Returns false when the candidates cannot decide: fewer than k of
// them, or (top-p alone) a nucleus that keeps every candidate and may reach
// past them. When it decides and `map` is set (the row's quads fit the map),
// it also builds the kept-quad map in the mass array and sets `mapped`.
// Contains barriers.
template <bool BF16>
__device__ __forceinline__ bool select_thresholds(int nc, int V, float c, float Mc, int fxs, bool kon, int k, bool pon,
                                                  float pp, double S_total, FilterLds* L, bool map, uint32_t& tau,
                                                  double& s_kept, bool& mapped) {
    constexpr int kPer = kCand / kThreads;
    constexpr int kBits = BF16 ? 16 : 32;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    if (kon && nc < k) return false;
    uint32_t* cand = &L->cnt[0][0];
    uint32_t key[kPer];
    unsigned long long mass[kPer];
    bool valid[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = j * kThreads + tid;
        valid[j] = i < nc;
        key[j] = valid[j] ? cand[i] : 0u;
        mass[j] = valid[j] ? fixed_of(ex2(fmaf(value_of<BF16>(key[j]), c, -Mc)), fxs) : 0ull;
    }
    // block-wide sums: per-wavefront partials in alternating LDS halves, so a
    // half is rewritten only after every wavefront has passed the barrier
    // that follows its last read
    int half = 0;
    auto count_ge = [&](uint32_t t) {
        int n = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) n += __popcll(__ballot(valid[j] && key[j] >= t));
        if (lane == 0) L->wnum[half][wave] = n;
        __syncthreads();
        int tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += L->wnum[half][w];
        half ^= 1;
        return tot;
    };
    auto mass_ge = [&](uint32_t t) {
        unsigned long long m = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) m += valid[j] && key[j] >= t ? mass[j] : 0ull;
        m = wave_sum_u64(m);
        if (lane == 0) L->wmass[half][wave] = m;
        __syncthreads();
        unsigned long long tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += L->wmass[half][w];
        half ^= 1;
        return tot;
    };
    uint32_t kth = 0u;
    if (kon) kth = radix_kth<kPer, kBits>(key, valid, k, L);
    uint32_t* kmap = (uint32_t*)&L->mass[0][0];
    if (!pon) {
        tau = kth;
        s_kept = (double)mass_ge(kth);
        if (map && tau != 0u) {
            mark_kept_quads<kPer>(key, valid, tau, L->ids, V / 4, kmap);
            mapped = true;
        }
        return true;
    }
    // pack the survivors (keys >= kth) to the front of cand[], then sort them
    int ns = 0, off = 0;
    {
        int mine[kPer], wtot = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint64_t m = __ballot(valid[j] && key[j] >= kth);
            mine[j] = wtot + __popcll(m & ((1ull << lane) - 1ull));
            wtot += __popcll(m);
        }
        if (lane == 0) L->wnum[half][wave] = wtot;
        __syncthreads();  // also: every candidate has been read from cand[]
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int n = L->wnum[half][w];
            off += w < wave ? n : 0;
            ns += n;
        }
        half ^= 1;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (valid[j] && key[j] >= kth) cand[off + mine[j]] = key[j];
    }
    if (ns <= kWave) {
        // At most 64 survivors (k <= 64, or a short top-p list): every
        // wavefront sorts them in its lanes and reads the nucleus off a wave
        // scan, with no barrier. The same keys, masses and decision rule as
        // the block-wide path below, so the same thresholds.
        __syncthreads();  // the packed survivors are in cand[]
        uint32_t kk = lane < ns ? cand[lane] : 0u;  // 0 sorts last
        for (int size = 2; size <= kWave; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                const uint32_t other = (uint32_t)__shfl_xor((int)kk, stride, kWave);
                const bool larger_here = ((lane & stride) == 0) == ((lane & size) == 0);
                kk = larger_here ? max(kk, other) : min(kk, other);
            }
        }
        const unsigned long long mk = lane < ns ? fixed_of(ex2(fmaf(value_of<BF16>(kk), c, -Mc)), fxs) : 0ull;
        unsigned long long incl = mk;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) incl += shfl_up_u64(incl, d) * (lane >= d);
        const unsigned long long excl = incl - mk;
        const unsigned long long H0 = readlane_u64(incl, kWave - 1);  // the survivors' mass
        double target = (double)pp * (kon ? (double)H0 : S_total);
        if (!(target > 0.0)) target = 0.5;  // top_p <= 0: keep the largest value only
        const uint32_t prev = (uint32_t)__shfl_up((int)kk, 1, kWave);
        int last = (lane > 0 && lane < ns && kk != prev && (double)excl < target) ? lane : 0;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) last = max(last, __shfl_xor(last, d, kWave));
        tau = (uint32_t)readlane_i((int)kk, last);
        // every candidate at or above tau is a survivor, so both checks stay in the wavefront
        const unsigned long long at_or_above = __ballot(lane < ns && kk >= tau);
        if (!kon && nc < V && __popcll(at_or_above) == nc) return false;
        unsigned long long m = kk >= tau ? mk : 0ull;
        m = wave_sum_u64(m);
        s_kept = (double)m;
        if (map && tau != 0u) {
            mark_kept_quads<kPer>(key, valid, tau, L->ids, V / 4, (uint32_t*)&L->mass[0][0]);
            mapped = true;
        }
        return true;
    }
    // More survivors: no sort. The kept ids are those whose strictly larger
    // keys weigh less than the target, which is every key >= T for the
    // largest T whose mass at or above it still reaches the target (the
    // masses at or above t fall as t grows, and T is a key: the mass steps
    // down right after it). T comes from a bitwise search with block-wide
    // fixed-point sums; it is the key the sorted nucleus ends on, and the
    // largest key is always kept (its strictly larger mass is 0).
    const unsigned long long H0 = mass_ge(kth);  // the survivors' mass
    double target = (double)pp * (kon ? (double)H0 : S_total);
    if (!(target > 0.0)) target = 0.5;  // top_p <= 0: keep the largest value only
    uint32_t T = 0u;
    for (int bit = kBits - 1; bit >= 0; --bit) {
        const uint32_t t = T | (1u << bit);
        if ((double)mass_ge(t) >= target) T = t;
    }
    tau = T;
    // top-p alone: if no candidate is dropped, ids below the cut may belong
    if (!kon && nc < V && count_ge(tau) == nc) return false;
    s_kept = (double)mass_ge(tau);
    if (map && tau != 0u) {
        mark_kept_quads<kPer>(key, valid, tau, L->ids, V / 4, kmap);
        mapped = true;
    }
    return true;
}

// The general path (any row): radix descent with per-wavefront histograms.
template <bool BF16, bool VEC>
__device__ __forceinline__ void radix_thresholds(const void* zrow, int V, float c, float Mc, int fxs, bool kon, int k, bool pon,
                                 float pp, FilterLds* Lp, uint32_t& tau_out, unsigned long long& s_kept_out) {
    constexpr int kBits = BF16 ? 16 : 32;
    constexpr int kLevels = kBits / 8;
    FilterLds& L = *Lp;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    for (int i = tid; i < kWaves * kBins; i += kThreads) {
        (&L.cnt[0][0])[i] = 0u;
        (&L.mass[0][0])[i] = 0ull;
    }
    __syncthreads();
    // top-k: descend to the key of the k-th largest logit
    uint32_t tau_k = 0u;
    if (kon) {
        uint32_t prefix = 0u;
        unsigned long long need = (unsigned long long)k;
        for (int l = 0; l < kLevels; ++l) {
            const int sh = kBits - 8 * (l + 1);
            for_each<BF16, VEC>(zrow, V, [&](float z, int64_t) {
                const uint32_t key = key_of<BF16>(z);
                if (l == 0 || (key >> (sh + 8)) == prefix) atomicAdd(&L.cnt[wave][(key >> sh) & 0xFFu], 1u);
            });
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
    tau_out = tau;
    s_kept_out = s_kept;
}

// Final pass: normalised kept probabilities, zeros elsewhere. Kept means
// key >= tau, tested as z >= the logit of tau (keys order like the logits
// and equal logits have equal keys); a quad of four consecutive elements with
// nothing kept in the whole wavefront skips the exponentials. With the
// kept-quad map (VEC rows only), a quad whose bit is clear is written as
// zeros without being read, so the row is read again only where it keeps
// something. Each lane takes 4 consecutive elements, so every store
// instruction of a wavefront covers 1 KB of the output contiguously (no
// partially written lines).
template <bool BF16, bool VEC>
__device__ __forceinline__ void write_filtered(const void* zrow, float* prow, int V, float c, float Mc, int fxs,
                                               uint32_t tau, double s_kept, const uint32_t* map) {
    const int tid = threadIdx.x;
    const float inv = (float)(ldexp(1.0, fxs) / s_kept);
    const float zt = tau == 0u ? -INFINITY : value_of<BF16>(tau);
    auto prob = [&](float zz) { return zz >= zt ? ex2(fmaf(zz, c, -Mc)) * inv : 0.0f; };
    if (VEC) {
        constexpr int kU = BF16 ? 8 : 4;  // 64 bytes of logits per lane in flight
        using Raw = typename std::conditional<BF16, u32x2, f32x4>::type;  // native vectors: selects stay in registers
        f32x4* out = (f32x4*)prow;
        const Raw* in = (const Raw*)zrow;
        const int nq = V / 4;
        auto quad = [&](const Raw& r) {
            float z[4];
            if constexpr (BF16) {
                z[0] = bf16_lo(r.x);
                z[1] = bf16_hi(r.x);
                z[2] = bf16_lo(r.y);
                z[3] = bf16_hi(r.y);
            } else {
                z[0] = r.x;
                z[1] = r.y;
                z[2] = r.z;
                z[3] = r.w;
            }
            const bool any = (z[0] >= zt) | (z[1] >= zt) | (z[2] >= zt) | (z[3] >= zt);
            if (__ballot(any) == 0ull) return f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            return f32x4{prob(z[0]), prob(z[1]), prob(z[2]), prob(z[3])};
        };
        Raw none;  // -inf logits: nothing kept
        if constexpr (BF16) {
            none = u32x2{0xFF80FF80u, 0xFF80FF80u};
        } else {
            none = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
        auto fetch = [&](int q) {
            const bool hit = map == nullptr || ((map[q >> 5] >> (q & 31)) & 1u);
            return hit ? in[q] : none;
        };
        int j = tid;
        for (; j + (kU - 1) * kThreads < nq; j += kU * kThreads) {
            Raw r[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) r[u] = fetch(j + u * kThreads);
#pragma unroll
            for (int u = 0; u < kU; ++u) store_nt(out + j + u * kThreads, quad(r[u]));
        }
        for (; j < nq; j += kThreads) store_nt(out + j, quad(fetch(j)));
    } else {
        for (int x = tid; x < V; x += kThreads) prow[x] = prob(Elems<BF16>::at(zrow, x));
    }
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void warp_filter_kernel(const void* __restrict__ logits, int R, int V,
                                                          const int32_t* __restrict__ lens, int extra_rows,
                                                          float c, const int32_t* __restrict__ top_k,
                                                          const float* __restrict__ top_p, int fxs,
                                                          float* __restrict__ probs) {
    __shared__ FilterLds L;
    const int row = blockIdx.x;
    const int b = row / R, r = row - b * R;
    const int live = clamp_len(lens, b, R - extra_rows) + extra_rows;
    if (r >= live) return;
    const char* zrow = (const char*)logits + (size_t)row * (size_t)V * (BF16 ? 2 : 4);
    float* prow = probs + (size_t)row * (size_t)V;

    const int k = top_k ? top_k[b] : 0;
    const bool kon = k > 0 && k < V;
    const float pp = top_p ? top_p[b] : 1.0f;
    const bool pon = pp < 1.0f;  // false for NaN

    // pass 1: the statistics and the candidate ids
    float Mc, S;
    int nc;
    gather_pass<BF16, VEC>(zrow, V, c, !kon, kon || pon, &L, Mc, S, nc);  // top-k rows need no row sum
    uint32_t tau = 0u;
    double s_kept = 0.0;
    bool decided = false, mapped = false;
    if (!kon && !pon) {  // no filter: the plain softmax
        s_kept = (double)S * ldexp(1.0, fxs);
        decided = true;
    } else {
        const bool map = VEC && V / 4 <= kMapWords * 32;
        decided = select_thresholds<BF16>(nc, V, c, Mc, fxs, kon, k, pon, pp, (double)S * ldexp(1.0, fxs), &L, map,
                                          tau, s_kept, mapped);
    }
    if (!decided) {
        unsigned long long sk = 0;
        radix_thresholds<BF16, VEC>(zrow, V, c, Mc, fxs, kon, k, pon, pp, &L, tau, sk);
        s_kept = (double)sk;
    }
    write_filtered<BF16, VEC>(zrow, prow, V, c, Mc, fxs, tau, s_kept, mapped ? (const uint32_t*)&L.mass[0][0] : nullptr);
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
