// greedy.hip -- greedy verification (temperature 0) for gfx950.
//
// Method (spec-verify card, "Method"; llmstudio blog "Как работает
// speculative decoding и MTP при инференсе LLM", sections 13 and 48): accept
// draft token t_i while it equals argmax(target row i); at the first miss emit
// that row's argmax; if all K_b match emit argmax(target row K_b).
//
// Mapping, without a workspace: one workgroup (1024 lanes, 16 wavefronts)
// owns one sequence and walks its rows in order, so the early exit at the
// first miss is a plain loop exit: rows after the miss are never fetched and
// no workgroup waits on another. With a workspace (greedy_sliced_kernel
// below) the rows of a sequence are split over up to 64 workgroups of 32 KB
// slices that exchange their partial argmaxes at every position, so a long
// chain of matches is read by several compute units. Each row (or slice) is
// one streaming argmax:
//   - 16-byte coalesced non-temporal loads (8 bf16 or 4 fp32 per load),
//     UNROLL loads in flight per lane;
//   - per lane, a strict '>' keeps the first of equal maxima (each lane sees
//     its elements in increasing index order);
//   - wave64 merge with DPP quad permutes and row mirrors, a ds_swizzle and
//     two scalar lane reads; the 16 wave results meet in LDS and every
//     wavefront merges them again, so the row's argmax is uniform in all lanes.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "specverify.h"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 8;

// Argmax plus the runner-up value, for top1 - top2 margins: (v, i) merge as in
// argmax_merge; s is the largest value other than the winner's one
// occurrence, so a tied maximum leaves s == v (margin 0).
__device__ __forceinline__ void top2_merge(float& v, int& i, float& s, float w, int j, float t) {
    const bool take = (w > v) | ((w == v) & (j < i));
    s = fmaxf(fmaxf(s, t), take ? v : w);
    v = take ? w : v;
    i = take ? j : i;
}

__device__ __forceinline__ void wave_top2(float& v, int& i, float& s) {
    top2_merge(v, i, s, dpp_f<kDppQuadXor1>(v), dpp_i<kDppQuadXor1>(i), dpp_f<kDppQuadXor1>(s));
    top2_merge(v, i, s, dpp_f<kDppQuadXor2>(v), dpp_i<kDppQuadXor2>(i), dpp_f<kDppQuadXor2>(s));
    top2_merge(v, i, s, dpp_f<kDppRowHalfMirror>(v), dpp_i<kDppRowHalfMirror>(i), dpp_f<kDppRowHalfMirror>(s));
    top2_merge(v, i, s, dpp_f<kDppRowMirror>(v), dpp_i<kDppRowMirror>(i), dpp_f<kDppRowMirror>(s));
    top2_merge(v, i, s, swz16_f(v), swz16_i(i), swz16_f(s));
    float v0 = readlane_f(v, 0), s0 = readlane_f(s, 0);
    int i0 = readlane_i(i, 0);
    top2_merge(v0, i0, s0, readlane_f(v, 32), readlane_i(i, 32), readlane_f(s, 32));
    v = v0;
    i = i0;
    s = s0;
}

// One element in index order: the running (best, bidx) and, with M, the
// runner-up value `second`.
template <bool M>
__device__ __forceinline__ void take(float x, int idx, float& best, int& bidx, float& second) {
    if (x > best) {
        if (M) second = best;
        best = x;
        bidx = idx;
    } else if (M) {
        second = fmaxf(second, x);
    }
}

template <bool BF16>
struct RowReader;

// bf16 rows: 8 elements per 16-byte vector.
template <>
struct RowReader<true> {
    static constexpr int kPerVec = 8;
    using Vec = u32x4;
    __device__ static float at(const void* row, int64_t i) { return bf16_at((const uint16_t*)row, i); }
    template <bool M>
    __device__ static void scan(const Vec& w, int base, float& best, int& bidx, float& second) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            take<M>(bf16_lo(w[k]), base + 2 * k, best, bidx, second);
            take<M>(bf16_hi(w[k]), base + 2 * k + 1, best, bidx, second);
        }
    }
    // First vector of a lane: an element that only ties -inf must still be
    // taken when the lane holds nothing yet.
    template <bool M>
    __device__ static void scan_first(const Vec& w, int base, float& best, int& bidx, float& second) {
        const float lo0 = bf16_lo(w[0]);
        if (bidx == INT32_MAX) {
            best = lo0;
            bidx = base;
        } else {
            take<M>(lo0, base, best, bidx, second);
        }
        take<M>(bf16_hi(w[0]), base + 1, best, bidx, second);
#pragma unroll
        for (int k = 1; k < 4; ++k) {
            take<M>(bf16_lo(w[k]), base + 2 * k, best, bidx, second);
            take<M>(bf16_hi(w[k]), base + 2 * k + 1, best, bidx, second);
        }
    }
};

// fp32 rows: 4 elements per 16-byte vector.
template <>
struct RowReader<false> {
    static constexpr int kPerVec = 4;
    using Vec = f32x4;
    __device__ static float at(const void* row, int64_t i) { return ((const float*)row)[i]; }
    template <bool M>
    __device__ static void scan(const Vec& w, int base, float& best, int& bidx, float& second) {
#pragma unroll
        for (int k = 0; k < 4; ++k) take<M>(w[k], base + k, best, bidx, second);
    }
    template <bool M>
    __device__ static void scan_first(const Vec& w, int base, float& best, int& bidx, float& second) {
        if (bidx == INT32_MAX) {
            best = w[0];
            bidx = base;
        } else {
            take<M>(w[0], base, best, bidx, second);
        }
#pragma unroll
        for (int k = 1; k < 4; ++k) take<M>(w[k], base + k, best, bidx, second);
    }
};

// Merge of the lanes' (best, bidx, second) over a workgroup of NW wavefronts:
// the wave-wide merge, then the NW wave results through LDS buffer `slot`,
// merged again by every wavefront, so the result (index returned, maximum and
// runner-up in vmax / vsecond) is uniform. Contains one barrier.
template <bool M, int NW>
__device__ __forceinline__ int block_merge(float best, int bidx, float second, float (*lds_v)[NW], int (*lds_i)[NW],
                                           float (*lds_s)[NW], int slot, float& vmax, float& vsecond) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (M) {
        wave_top2(best, bidx, second);
    } else {
        wave_argmax(best, bidx);
    }
    if (lane == 0) {
        lds_v[slot][wave] = best;
        lds_i[slot][wave] = bidx;
        if (M) lds_s[slot][wave] = second;
    }
    __syncthreads();
    float v = lane < NW ? lds_v[slot][lane] : -INFINITY;
    int i = lane < NW ? lds_i[slot][lane] : INT32_MAX;
    if (M) {
        float s = lane < NW ? lds_s[slot][lane] : -INFINITY;
        wave_top2(v, i, s);
        vmax = v;
        vsecond = s;
    } else {
        wave_argmax(v, i);
        vmax = v;
    }
    return i;
}

// Argmax of elements [x0, x0 + len) of a row (len >= 1), over a workgroup of
// NW wavefronts. Returns the wave-uniform index (and, with M, the maximum and
// runner-up values in vmax / vsecond); every lane of the workgroup must call
// it (it contains one barrier). `slot` alternates between two LDS buffers so
// that consecutive calls never race on them.
template <bool BF16, bool M, int NW, int U = kUnroll>
__device__ __forceinline__ int span_argmax(const void* row, int x0, int len, float (*lds_v)[NW], int (*lds_i)[NW],
                                           float (*lds_s)[NW], int slot, float& vmax, float& vsecond) {
    using R = RowReader<BF16>;
    constexpr int E = R::kPerVec;
    constexpr int NT = NW * kWave;
    const int tid = threadIdx.x;
    const char* span = (const char*)row + (size_t)x0 * (BF16 ? 2 : 4);

    // Elements before the first 16-byte boundary, one per lane.
    const uintptr_t addr = (uintptr_t)span;
    int head = (int)(((16u - (addr & 15u)) & 15u) / (BF16 ? 2u : 4u));
    if (head > len) head = len;
    const int nvec = (len - head) / E;
    const int tail0 = head + nvec * E;

    float best = -INFINITY, second = -INFINITY;
    int bidx = INT32_MAX;
    if (tid < head) {
        best = R::at(span, tid);
        bidx = x0 + tid;
    }
    const typename R::Vec* vrow = (const typename R::Vec*)(span + head * (BF16 ? 2 : 4));
    const int base = x0 + head;
    // Batches of U vectors per lane, all U loads issued before any is
    // scanned, the last batch too (its loads past the span are skipped): a
    // span of n vectors takes ceil(n / (U * NT)) memory round trips. Vectors
    // are scanned in index order; scan_first also takes a -inf first element
    // when the lane holds nothing yet (the same as scan otherwise).
    for (int j = tid; j < nvec; j += U * NT) {
        typename R::Vec w[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (j + u * NT < nvec) w[u] = load_nt(vrow + j + u * NT);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (j + u * NT < nvec) R::template scan_first<M>(w[u], base + (j + u * NT) * E, best, bidx, second);
    }
    if (tail0 + tid < len) {
        const float v = R::at(span, tail0 + tid);
        if (bidx == INT32_MAX) {
            best = v;
            bidx = x0 + tail0 + tid;
        } else {
            take<M>(v, x0 + tail0 + tid, best, bidx, second);
        }
    }

    return block_merge<M, NW>(best, bidx, second, lds_v, lds_i, lds_s, slot, vmax, vsecond);
}

// M: also write top2_margin[b] = max - runner-up of the row next_token comes
// from (the committed token's row; 0 for a tied maximum, +inf when V == 1).
template <bool BF16, bool M>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void greedy_kernel(
    const void* __restrict__ target, int K, int V, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ lens, int32_t* __restrict__ n_accepted, int32_t* __restrict__ next_token,
    float* __restrict__ top2_margin) {
    __shared__ float lds_v[2][kWaves];
    __shared__ int lds_i[2][kWaves];
    __shared__ float lds_s[M ? 2 : 1][kWaves];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int kb = clamp_len(lens, b, K);
    // Draft token i sits in lane i (K <= 64); only positions < K_b are read.
    const int my_tok = lane < kb ? tokens[(int64_t)b * K + lane] : -1;
    const size_t row_bytes = (size_t)V * (BF16 ? 2 : 4);
    const char* base = (const char*)target + (size_t)b * (size_t)(K + 1) * row_bytes;

    int i = 0;
    for (;; ++i) {
        float vmax = 0.0f, vsecond = 0.0f;
        const int am = span_argmax<BF16, M, kWaves>(base + (size_t)i * row_bytes, 0, V, lds_v, lds_i, lds_s, i & 1,
                                                    vmax, vsecond);
        // a token outside [0, V) never equals an argmax: it is a miss
        if (i == kb || readlane_i(my_tok, i) != am) {
            if (threadIdx.x == 0) {
                n_accepted[b] = i;
                next_token[b] = am;
                if (M) top2_margin[b] = vmax - vsecond;
            }
            return;
        }
    }
}

// ---- greedy_sliced_kernel: each sequence over G workgroups -----------------
//
// The same walk with the rows of a sequence split into G slices of Ls
// elements; workgroup (b, g) of 256 lanes owns slice g of every row of
// sequence b and reads it in one batch of loads (a 32 KB slice: one memory
// round trip per position). At each position every slice publishes its
// (value, index) -- and, with M, its runner-up value -- into slots of the
// caller's workspace, and every workgroup decides the row from the slices'
// words alike. A row matches only when all G words are in and none beats the
// draft token; a miss is certain as soon as one word beats it, so at the
// miss (the last row of most sequences) a workgroup need not wait for the
// slowest slice. The row's argmax, the output, is then taken from all G
// words by the last of the sequence's workgroups to finish. A long chain of
// matches thus reads each row with G compute units instead of one. Every wait
// is bounded: a workgroup that gives up computes the missing slices itself,
// so the result is the same either way.
//
// Look-ahead (the depth L of the walk): a workgroup may read and scan its
// slices of rows i+1 .. i+L before it waits for the other slices of row i,
// so that the wait overlaps the next rows' loads. The scanned results wait
// in LDS; row r is published only once row r-1 has matched, so a workgroup
// never publishes a row it does not go on to gather. L = 0 is the exact
// walk; rows read ahead of a miss are read for nothing, which costs time
// whenever HBM is saturated. Results are the same for every L: a row is
// still decided only from the G slices of that row.
//
// The workspace needs no fill before a launch: an empty slot is a zero word
// (a published word never is: it carries index + 1, or a set low bit), and
// every launch leaves the workspace all zero again. When a workgroup is done
// with its sequence (every slot access finished) it counts itself out on the
// sequence's departure counter; the last of the G gathers the last row's
// words, writes the outputs, and clears every slot word the sequence used
// and the counter. So a workspace must hold zeros before its first use, and
// the next launch finds it so.
constexpr int kSliceWaves = 4;
constexpr int kSliceThreads = kSliceWaves * kWave;
constexpr int kSliceUnroll = 8;  // 128 bytes per lane in flight: a 32 KB slice in one batch
constexpr int kMarginUnroll = 6;  // with the runner-up values (8 would spill): the slice in two batches
constexpr int kMaxGreedySlices = kWave;  // slice results are merged across one wavefront

// Outcomes of the decision on one row.
constexpr int kWaitedOut = 0, kRowMatch = 1, kRowMiss = 2;

// Wavefront 0 polls the value words set[k * W] of the G slices of a row
// (bounded) until the row is decided against draft token tok, whose slice is
// gt (-1 when tok is outside [0, V): a miss). A row matches iff no element
// beats tok in the argmax order, i.e. iff no slice's best does. So the row is
// a miss as soon as one published word beats tok: the word of tok's own
// slice when its best is not tok, or another slice's when its value is above
// tok's logit (the best of tok's slice) or equal to it at a lower index. It
// matches once all G words are published and none beats tok. The decision
// also waits for this workgroup's own words (slice g), so that its publishes
// are visible before it can count itself out. Returns the outcome, uniform
// over the workgroup (kWaitedOut if the wait ran out first). Contains a
// barrier.
template <int W>
__device__ int decide_row(const unsigned long long* set, int G, int g, int tok, int gt, int wait_limit, int* s_flag) {
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        const unsigned long long all = G == kWave ? ~0ull : (1ull << G) - 1ull;
        int res = kWaitedOut;
        for (int tries = 0; tries <= wait_limit; ++tries) {
            unsigned long long w = 0ull;
            if (lane < G) w = __hip_atomic_load(set + lane * W, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            bool own = true;  // the runner-up word too, when there is one
            if (W > 1) own = __hip_atomic_load(set + g * W + W - 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0ull;
            const unsigned long long pres = __ballot(w != 0ull);
            if (own && ((pres >> g) & 1ull)) {
                if (gt < 0) {
                    res = kRowMiss;
                    break;
                }
                if ((pres >> gt) & 1ull) {
                    const float v = __uint_as_float((uint32_t)(w >> 32));
                    const int idx = (int)((uint32_t)w - 1u);
                    if (readlane_i(idx, gt) != tok) {
                        res = kRowMiss;
                        break;
                    }
                    const float z = readlane_f(v, gt);
                    if (__ballot((w != 0ull) & ((v > z) | ((v == z) & (idx < tok)))) != 0ull) {
                        res = kRowMiss;
                        break;
                    }
                    if (pres == all) {
                        res = kRowMatch;
                        break;
                    }
                }
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (lane == 0) *s_flag = res;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*s_flag);
}

// Wavefront 0 counts the workgroup out of its sequence once it has made its
// last slot access; returns (uniform) whether it was the last of the G. The
// count needs no fence in the common case: the workgroup has seen its own
// published words through the same device-coherent loads as the others use
// (`own_seen`), so they are visible before it counts itself out. Otherwise
// it polls them first (bounded), and one whose words it could not see, or
// that gave up waiting earlier (`waited_out`), releases first.
template <int W>
__device__ bool count_out(unsigned long long* counter, const unsigned long long* own, int G, bool own_seen,
                          bool waited_out, int wait_limit, int* s_flag) {
    if (threadIdx.x < kWave) {
        if (!own_seen && !waited_out) {
            bool seen = false;
            for (int tries = 0; tries <= wait_limit && !seen; ++tries) {
                unsigned long long w = 1ull;
                if (threadIdx.x < W) w = __hip_atomic_load(own + threadIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                seen = __ballot(w == 0ull) == 0ull;
                if (!seen) __builtin_amdgcn_s_sleep(2);
            }
            waited_out = !seen;
        }
        if (waited_out) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        unsigned long long prev = 0;
        if (threadIdx.x == 0) prev = __hip_atomic_fetch_add(counter, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (threadIdx.x == 0) *s_flag = prev == (unsigned long long)(G - 1);
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*s_flag) != 0;
}

// The last workgroup out returns the sequence's `nwords` slot words and its
// counter to zero (wavefront 0; every other workgroup has counted out, so no
// slot of the sequence is accessed again in this launch).
__device__ __forceinline__ void clear_sequence(unsigned long long* counter, unsigned long long* words, int nwords) {
    if (threadIdx.x >= kWave) return;
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));  // formed here: a copy kept from the kernel's start would be spilled
    for (int k = tid; k < nwords; k += kWave)
        __hip_atomic_store(words + k, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool BF16, bool M>
__global__ __launch_bounds__(kSliceThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void greedy_sliced_kernel(
    const void* __restrict__ target, int K, int V, int G, int Ls, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ lens, int32_t* __restrict__ n_accepted, int32_t* __restrict__ next_token,
    float* __restrict__ top2_margin, unsigned long long* __restrict__ departed, unsigned long long* __restrict__ slots,
    int wait_limit, int lookahead) {
    __shared__ float lds_v[2][kSliceWaves];
    __shared__ int lds_i[2][kSliceWaves];
    __shared__ float lds_s[M ? 2 : 1][kSliceWaves];
    __shared__ unsigned long long s_words[2 * kMaxGreedySlices];
    __shared__ unsigned long long s_ahead[SV_MAX_K + 1][M ? 2 : 1];  // this slice's scanned rows, not yet published
    __shared__ int s_ready;
    __shared__ int s_decided[2];  // alternate by position: a wavefront may still read the previous one
    __shared__ int s_last;
    constexpr int W = M ? 2 : 1;  // words per slice and position
    const int b = blockIdx.x / G, g = blockIdx.x - b * G;
    const int lane = threadIdx.x & (kWave - 1);
    const int kb = clamp_len(lens, b, K);
    const int my_tok = lane < kb ? tokens[(int64_t)b * K + lane] : -1;
    const size_t row_bytes = (size_t)V * (BF16 ? 2 : 4);
    const char* base = (const char*)target + (size_t)b * (size_t)(K + 1) * row_bytes;
    auto slice_len = [&](int k) { return (int)min((int64_t)Ls, (int64_t)V - (int64_t)k * Ls); };
    // never zero: the low half holds index + 1 (index < V <= INT32_MAX), or a set bit
    auto pack = [](float v, int i) {
        return ((unsigned long long)__float_as_uint(v) << 32) | (unsigned long long)((uint32_t)i + 1u);
    };
    auto pack2 = [](float s) { return ((unsigned long long)__float_as_uint(s) << 32) | 1ull; };
    auto slot_set = [&](int r) { return slots + ((size_t)b * (K + 1) + r) * (size_t)(G * W); };
    // this slice of row r, scanned into s_ahead[r] (thread 0 writes and later reads it)
    int parity = 0;
    auto scan_row = [&](int r) {
        float vr, sr = -INFINITY;
        const int ar = span_argmax<BF16, M, kSliceWaves, M ? kMarginUnroll : kSliceUnroll>(
            base + (size_t)r * row_bytes, g * Ls, slice_len(g), lds_v, lds_i, lds_s, parity, vr, sr);
        parity ^= 1;
        if (threadIdx.x == 0) {
            s_ahead[r][0] = pack(vr, ar);
            if (M) s_ahead[r][W - 1] = pack2(sr);
        }
    };
    // every slice's words of row `row`, computed here alike into s_words when
    // a bounded wait ran out (two vectors per lane in flight: a rare path,
    // kept small)
    auto compute_all = [&](const char* row) {
        for (int k = 0; k < G; ++k) {
            float vk, sk = -INFINITY;
            const int ik =
                span_argmax<BF16, M, kSliceWaves, 2>(row, k * Ls, slice_len(k), lds_v, lds_i, lds_s, parity, vk, sk);
            parity ^= 1;
            if (threadIdx.x == 0) {
                s_words[k * W] = pack(vk, ik);
                if (M) s_words[k * W + 1] = pack2(sk);
            }
        }
        __syncthreads();
    };
    // merge of the G <= 64 slices' words in s_words: lane k holds slice k, the
    // wave-wide merge (the (value, index) order is total and the runner-up is a
    // plain maximum, so every merge order gives the same result)
    float v, s = -INFINITY;
    int am;
    auto merge_words = [&]() {
        v = -INFINITY;
        am = INT32_MAX;
        s = -INFINITY;
        // the lane index formed here, on this rare path: a copy kept from the
        // kernel's start would be spilled
        int k = (int)threadIdx.x & (kWave - 1);
        asm volatile("" : "+v"(k));
        if (k < G) {
            v = __uint_as_float((uint32_t)(s_words[k * W] >> 32));
            am = (int)((uint32_t)s_words[k * W] - 1u);
            if (M) s = __uint_as_float((uint32_t)(s_words[k * W + 1] >> 32));
        }
        if (M)
            wave_top2(v, am, s);
        else
            wave_argmax(v, am);
    };
    int i = 0;
    int scanned = 0;  // rows 0 .. scanned-1 of this slice are scanned
    bool waited_out = false, own_seen = false;
    for (;; ++i) {
        unsigned long long* set = slot_set(i);
        if (scanned == i) scan_row(scanned++);
        if (threadIdx.x == 0) {
            publish_word(set + g * W, s_ahead[i][0]);
            if (M) publish_word(set + g * W + 1, s_ahead[i][W - 1]);
        }
        // rows up to i + L (at most K_b) read while the other slices of row i arrive
        for (const int last = min(kb, i + lookahead); scanned <= last;) scan_row(scanned++);
        // the last row has no draft token to test: its argmax is taken by the
        // last workgroup out
        if (i == kb) break;
        const int tok = readlane_i(my_tok, i);
        const int gt = (tok >= 0 && tok < V) ? tok / Ls : -1;  // outside [0, V): a miss
        const int r = decide_row<W>(set, G, g, tok, gt, wait_limit, &s_decided[i & 1]);
        if (r == kRowMatch) continue;
        if (r == kRowMiss) {
            own_seen = true;
            break;
        }
        waited_out = true;
        compute_all(base + (size_t)i * row_bytes);
        merge_words();
        __syncthreads();  // s_words is rewritten by the next position
        if (tok != am) break;
    }
    // row i is the sequence's last: the workgroups count out, and the last one
    // takes the row's argmax from all G slices, writes the outputs and clears
    // the sequence's slots
    unsigned long long* set = slot_set(i);
    if (!count_out<W>(departed + b, set + g * W, G, own_seen, waited_out, wait_limit, &s_last)) return;
    if (!gather_words(set, G * W, wait_limit, s_words, &s_ready, 0ull)) compute_all(base + (size_t)i * row_bytes);
    merge_words();
    if (threadIdx.x == 0) {
        n_accepted[b] = i;
        next_token[b] = am;
        if (M) top2_margin[b] = v - s;
    }
    clear_sequence(departed + b, slot_set(0), (i + 1) * G * W);
}

}  // namespace

// Slices of the split greedy verify: each 256-lane workgroup reads its slice
// of a row with one batch of kSliceUnroll 16-byte loads per lane (one memory
// round trip per position), so a row of V elements of s bytes takes
// G = V*s / (256 * 16 * kSliceUnroll) slices (24 KB each), at most 64 (longer
// rows get longer slices). Rows of at most 128 KB use one 1024-lane
// workgroup per sequence instead: that is one round trip too, without an
// exchange.
void greedy_slice_shape(int V, bool bf16, int& G, int& Ls) {
    const int64_t per = (int64_t)kSliceThreads * kSliceUnroll * (bf16 ? 8 : 4);
    const int64_t row_bytes = (int64_t)V * (bf16 ? 2 : 4);
    if (row_bytes <= 128 * 1024) {
        G = 1;
        Ls = V;
        return;
    }
    int64_t ls = per;
    if (((int64_t)V + ls - 1) / ls > kMaxGreedySlices) ls = ((int64_t)V + kMaxGreedySlices - 1) / kMaxGreedySlices;
    ls = (ls + 63) / 64 * 64;
    G = (int)(((int64_t)V + ls - 1) / ls);
    Ls = (int)ls;
}

// B departure counters, then 2 words per slice and position of every sequence.
size_t greedy_dtype_workspace_bytes(int B, int K, int V, bool bf16) {
    int G, Ls;
    greedy_slice_shape(V, bf16, G, Ls);
    if (G < 2) return 0;
    return ((size_t)B + (size_t)B * (size_t)(K + 1) * 2 * (size_t)G) * sizeof(unsigned long long);
}

namespace {
std::atomic<int> g_lookahead{SV_GREEDY_LOOKAHEAD};  // rows the split walk reads ahead of its decision
}  // namespace

void set_greedy_lookahead(int rows) { g_lookahead.store(rows); }

// The larger of the two dtypes' needs (fp32 rows are split into more slices),
// so that one size serves either.
size_t greedy_workspace_bytes(int B, int K, int V) { return greedy_dtype_workspace_bytes(B, K, V, false); }

hipError_t launch_greedy(const void* target, bool bf16, int B, int K, int V, const int32_t* tokens,
                         const int32_t* lens, int32_t* n_accepted, int32_t* next_token, float* top2_margin,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const size_t need = greedy_dtype_workspace_bytes(B, K, V, bf16);
    if (need > 0 && workspace && workspace_bytes >= need && (uintptr_t)workspace % 8 == 0) {
        int G, Ls;
        greedy_slice_shape(V, bf16, G, Ls);
        unsigned long long* departed = (unsigned long long*)workspace;  // zero between launches
        unsigned long long* slots = departed + B;
        const dim3 grid((unsigned)B * (unsigned)G), block(kSliceThreads);
        const int wl = get_wait_limit(), la = g_lookahead.load();
        if (top2_margin) {
            if (bf16)
                hipLaunchKernelGGL((greedy_sliced_kernel<true, true>), grid, block, 0, stream, target, K, V, G, Ls,
                                   tokens, lens, n_accepted, next_token, top2_margin, departed, slots, wl, la);
            else
                hipLaunchKernelGGL((greedy_sliced_kernel<false, true>), grid, block, 0, stream, target, K, V, G, Ls,
                                   tokens, lens, n_accepted, next_token, top2_margin, departed, slots, wl, la);
        } else {
            if (bf16)
                hipLaunchKernelGGL((greedy_sliced_kernel<true, false>), grid, block, 0, stream, target, K, V, G, Ls,
                                   tokens, lens, n_accepted, next_token, top2_margin, departed, slots, wl, la);
            else
                hipLaunchKernelGGL((greedy_sliced_kernel<false, false>), grid, block, 0, stream, target, K, V, G, Ls,
                                   tokens, lens, n_accepted, next_token, top2_margin, departed, slots, wl, la);
        }
        return hipGetLastError();
    }
    const dim3 grid(B), block(kThreads);
    if (top2_margin) {
        if (bf16)
            hipLaunchKernelGGL((greedy_kernel<true, true>), grid, block, 0, stream, target, K, V, tokens, lens,
                               n_accepted, next_token, top2_margin);
        else
            hipLaunchKernelGGL((greedy_kernel<false, true>), grid, block, 0, stream, target, K, V, tokens, lens,
                               n_accepted, next_token, top2_margin);
    } else {
        if (bf16)
            hipLaunchKernelGGL((greedy_kernel<true, false>), grid, block, 0, stream, target, K, V, tokens, lens,
                               n_accepted, next_token, top2_margin);
        else
            hipLaunchKernelGGL((greedy_kernel<false, false>), grid, block, 0, stream, target, K, V, tokens, lens,
                               n_accepted, next_token, top2_margin);
    }
    return hipGetLastError();
}

}  // namespace sv
