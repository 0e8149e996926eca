// penalty.hip -- the sampler's penalty stage for gfx950: repetition, presence
// and frequency penalties of the live logit rows, given each sequence's token
// history (llmstudio blog "Как работает speculative decoding и MTP при
// инференсе LLM", section 38: penalties are the first stage of the pipeline
// raw logits -> penalties -> temperature -> top-k -> top-p -> normalise;
// section 39: a stateful sampler's state must follow the speculative branch,
// so row r of a sequence sees the committed tokens and the draft tokens
// before position r).
//
// For an id with c > 0 occurrences in the row's history, in fp32 with one
// rounding per operation:
//   z1 = z < 0 ? z * theta : z / theta,   z' = z1 - fmaf(frequency, c, presence);
// other ids keep z. The output rows are fp32 (the penalised values are not
// bf16 values).
//
// Two kernels:
//  1. penalty_table_kernel, one 1024-lane workgroup per sequence: the
//     committed history seq[b, :seq_len[b]] is counted in an open-addressing
//     hash table in the workspace (capacity a power of two at least twice the
//     history buffer, so probing ends), then compacted into a list of
//     (id, count) pairs. The table is cleared by the same workgroup first,
//     so the workspace needs no preparation.
//  2. penalty_rows_kernel: each live row in slices of 32768 ids, one 1024-lane
//     workgroup per slice (as the warp's split path). A workgroup issues all
//     of its loads at once (32 ids per lane, 4 per load, so each lane's output
//     is one 16-byte store and a wave's stores are contiguous), marks in an LDS bitmap
//     the ids of the row's history (the committed list and the row's draft
//     prefix) that fall in its slice while they are in flight, with each
//     committed id's count in LDS (a byte; 255 and above are looked up in
//     the table), then writes each vector in fp32, patching in registers
//     those that hold marked ids (count = committed count + prefix
//     occurrences). A row is read once and written once. Rows whose length
//     (V not a multiple of 4) or alignment rules out vector access are copied
//     element by element by one workgroup and patched afterwards with
//     scattered stores.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxPrefix = kWave;  // draft prefixes are at most SV_MAX_K = 64 tokens
constexpr int kSlice = kThreads * 32;  // ids per workgroup in the 16-byte path: 32 per lane, loaded at once

// Table slot of an id: a multiplicative hash, then linear probing.
__device__ __forceinline__ uint32_t slot_of(int32_t id, uint32_t mask) {
    return ((uint32_t)id * 2654435761u) & mask;
}

// The penalised value of logit z seen c > 0 times (fp32; the quotient is
// formed in binary64 and rounded once, which is the correctly rounded fp32
// quotient: 53 >= 2 * 24 + 2 bits).
__device__ __forceinline__ float penalised(float z, int c, float theta, float presence, float frequency) {
#pragma clang fp contract(off)  // z * theta - d must round twice, as written
    const float z1 = z < 0.0f ? z * theta : (float)((double)z / (double)theta);
    const float d = __builtin_fmaf(frequency, (float)c, presence);
    return z1 - d;
}

struct TableView {
    int32_t* keys;    // [P]: id + 1, or 0 for an empty slot
    int32_t* counts;  // [P]
    int32_t* list;    // [2 * P]: (id, count) pairs of the occupied slots
    int32_t* n;       // [1]: pairs in the list
};

__device__ __forceinline__ TableView table_of(void* ws, int b, int P) {
    int32_t* base = (int32_t*)ws + (size_t)b * ((size_t)4 * P + 4);
    return TableView{base, base + P, base + 2 * P, base + 4 * P};
}

__global__ __launch_bounds__(kThreads) void penalty_table_kernel(const int32_t* __restrict__ seq,
                                                                  const int32_t* __restrict__ seq_len, int cap, int V,
                                                                  int P, void* __restrict__ ws) {
    __shared__ int s_n;
    const int b = blockIdx.x, tid = threadIdx.x;
    const TableView t = table_of(ws, b, P);
    const uint32_t mask = (uint32_t)P - 1u;
    for (int h = tid; h < P; h += kThreads) {
        t.keys[h] = 0;
        t.counts[h] = 0;
    }
    if (tid == 0) s_n = 0;
    __syncthreads();
    int n0 = seq_len[b];
    n0 = n0 < 0 ? 0 : (n0 > cap ? cap : n0);
    const int32_t* hist = seq + (size_t)b * cap;
    for (int j = tid; j < n0; j += kThreads) {
        const int32_t id = hist[j];
        if (id < 0 || id >= V) continue;  // outside the vocabulary: no logit to penalise
        uint32_t h = slot_of(id, mask);
        for (;;) {  // at most P - 1 other keys: the table is at most half full
            const int32_t k = atomicCAS(&t.keys[h], 0, id + 1);
            if (k == 0 || k == id + 1) {
                atomicAdd(&t.counts[h], 1);
                break;
            }
            h = (h + 1u) & mask;
        }
    }
    __syncthreads();
    for (int h = tid; h < P; h += kThreads) {
        // read past the first-level cache: the counts were formed by atomics
        const int32_t k = __hip_atomic_load(&t.keys[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (k != 0) {
            const int at = atomicAdd(&s_n, 1);
            t.list[2 * at] = k - 1;
            t.list[2 * at + 1] = __hip_atomic_load(&t.counts[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    __syncthreads();
    if (tid == 0) *t.n = s_n;
}

// Count of id in the committed history (0 when absent), by probing the table.
__device__ __forceinline__ int table_count(const TableView& t, int32_t id, uint32_t mask) {
    uint32_t h = slot_of(id, mask);
    for (;;) {
        const int32_t k = t.keys[h];
        if (k == 0) return 0;
        if (k == id + 1) return t.counts[h];
        h = (h + 1u) & mask;
    }
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void penalty_rows_kernel(
    const void* __restrict__ logits, int R, int V, int G, const int32_t* __restrict__ lens, int extra_rows,
    bool have_hist, int P, const void* __restrict__ ws, const int32_t* __restrict__ tokens, int K,
    const float* __restrict__ theta, const float* __restrict__ presence, const float* __restrict__ frequency,
    float* __restrict__ out) {
    __shared__ int32_t s_pre[kMaxPrefix];
    __shared__ uint32_t s_mark[kSlice / 32];   // VEC: committed ids of the slice, one bit each
    __shared__ uint32_t s_pmark[kSlice / 32];  // VEC: draft-prefix ids of the slice
    __shared__ uint8_t s_cnt[kSlice];          // VEC: committed count of each marked id (255: look it up)
    const int row = blockIdx.x / G, g = blockIdx.x - row * G;
    const int b = row / R, r = row - b * R;
    const int live = clamp_len(lens, b, R - extra_rows) + extra_rows;
    if (r >= live) return;
    const int tid = threadIdx.x;
    const size_t es = BF16 ? 2 : 4;
    const char* zrow = (const char*)logits + (size_t)row * (size_t)V * es;
    float* orow = out + (size_t)row * (size_t)V;
    auto at = [&](int64_t x) {
        return BF16 ? bf16_at((const uint16_t*)zrow, x) : ((const float*)zrow)[x];
    };
    // the draft prefix of this row: tokens[b, 0 .. r-1]
    const int np = tokens ? r : 0;
    if (tid < np) s_pre[tid] = tokens[(size_t)b * K + tid];
    const float th = theta ? theta[b] : 1.0f;
    const float pr = presence ? presence[b] : 0.0f;
    const float fr = frequency ? frequency[b] : 0.0f;
    auto prefix_count = [&](int32_t id, int upto) {
        int c = 0;
        for (int j = 0; j < upto; ++j) c += s_pre[j] == id;
        return c;
    };
    const uint32_t mask = (uint32_t)P - 1u;
    const TableView t = table_of(const_cast<void*>(ws), b, P);

    if (VEC) {
        // slice g of the row: kSlice ids, 4 per load (8 bytes of bf16 or 16 of
        // fp32) so that each lane's output is one 16-byte store and a wave's
        // stores are contiguous; all loads issued first, the marking below
        // runs while they are in flight
        constexpr int E = 4;
        constexpr int kVecs = kSlice / kThreads / E;
        const int x0 = g * kSlice;
        const int nv = (min(kSlice, V - x0)) / E;  // vectors in the slice
        using Raw = typename std::conditional<BF16, u32x2, u32x4>::type;
        const Raw* vin = (const Raw*)(zrow + (size_t)x0 * es);
        Raw w[kVecs];
#pragma unroll
        for (int u = 0; u < kVecs; ++u) w[u] = __builtin_nontemporal_load(vin + min(u * kThreads + tid, nv - 1));
        // 1. mark the history ids that fall in the slice: the committed ones
        // with their counts (each id is listed once), then the prefix's
        s_mark[tid] = 0u;
        s_pmark[tid] = 0u;
        __syncthreads();
        if (have_hist) {
            const int n = *t.n;
            for (int k = tid; k < n; k += kThreads) {
                const int o = t.list[2 * k] - x0;
                if (o >= 0 && o < kSlice) {
                    atomicOr(&s_mark[o >> 5], 1u << (o & 31));
                    s_cnt[o] = (uint8_t)min(t.list[2 * k + 1], 255);
                }
            }
        }
        if (tid < np) {
            const int o = s_pre[tid] - x0;
            if (o >= 0 && o < kSlice && s_pre[tid] < V) atomicOr(&s_pmark[o >> 5], 1u << (o & 31));
        }
        __syncthreads();
        // 2. each vector in fp32, patched in registers where it holds marked ids
#pragma unroll
        for (int u = 0; u < kVecs; ++u) {
            const int j = u * kThreads + tid;
            if (j >= nv) continue;
            float z[4];
            if constexpr (BF16) {
                z[0] = bf16_lo(w[u][0]);
                z[1] = bf16_hi(w[u][0]);
                z[2] = bf16_lo(w[u][1]);
                z[3] = bf16_hi(w[u][1]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) z[k] = __uint_as_float(w[u][k]);
            }
            const int o = j * E;
            const uint32_t cb = (s_mark[o >> 5] >> (o & 31)) & 0xFu, pb = (s_pmark[o >> 5] >> (o & 31)) & 0xFu;
            if (cb | pb) {  // rare: ids of the history
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    int c = 0;
                    if (cb & (1u << e)) {
                        c = s_cnt[o + e];
                        if (c == 255) c = table_count(t, x0 + o + e, mask);
                    }
                    if (pb & (1u << e)) c += prefix_count(x0 + o + e, np);
                    if (c > 0) z[e] = penalised(z[e], c, th, pr, fr);
                }
            }
            store_nt((f32x4*)(orow + (size_t)(x0 + o)), f32x4{z[0], z[1], z[2], z[3]});
        }
        return;
    }

    // element by element: the row in fp32, then the history's ids patched
    for (int x = tid; x < V; x += kThreads) orow[x] = at(x);
    __syncthreads();  // the prefix is in LDS and the copy's stores are complete before any patch overwrites one
    // ids of the committed history, with their prefix occurrences added
    if (have_hist) {
        const int n = *t.n;
        for (int k = tid; k < n; k += kThreads) {
            const int32_t id = t.list[2 * k];
            const int c = t.list[2 * k + 1] + prefix_count(id, np);
            orow[id] = penalised(at(id), c, th, pr, fr);
        }
    }
    // ids that only the prefix holds, patched once (at their first occurrence)
    if (tid < np) {
        const int32_t id = s_pre[tid];
        if (id >= 0 && id < V && prefix_count(id, tid) == 0) {
            const bool committed = have_hist && table_count(t, id, mask) > 0;
            if (!committed) orow[id] = penalised(at(id), prefix_count(id, np), th, pr, fr);
        }
    }
}

}  // namespace

// Table capacity for a history buffer of `cap` tokens: a power of two, at least
// 2 * cap (and 64).
int penalty_table_capacity(int cap) {
    int64_t p = 64;
    while (p < 2 * (int64_t)cap) p <<= 1;
    return (int)p;
}

size_t penalty_workspace_bytes(int B, int cap) {
    if (B < 1 || cap < 1) return 0;
    const size_t P = (size_t)penalty_table_capacity(cap);
    return (size_t)B * (4 * P + 4) * sizeof(int32_t);
}

hipError_t launch_penalties(const void* logits, bool bf16, int B, int R, int V, const int32_t* lens, int extra_rows,
                            const int32_t* seq, const int32_t* seq_len, int cap, const int32_t* tokens, int K,
                            const float* theta, const float* presence, const float* frequency, float* out,
                            void* workspace, hipStream_t stream) {
    const bool have_hist = seq != nullptr;
    const int P = have_hist ? penalty_table_capacity(cap) : 64;
    if (have_hist) {
        hipLaunchKernelGGL(penalty_table_kernel, dim3(B), dim3(kThreads), 0, stream, seq, seq_len, cap, V, P,
                           workspace);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t rows = (int64_t)B * R;
    const int64_t G = ((int64_t)V + kSlice - 1) / kSlice;
    const bool vec = (V % 4 == 0) && ((uintptr_t)logits % (bf16 ? 8 : 16) == 0) && ((uintptr_t)out % 16 == 0) &&
                     rows * G <= INT32_MAX;
    const int g = vec ? (int)G : 1;
    const dim3 grid((unsigned)(rows * g));
    if (bf16) {
        if (vec)
            hipLaunchKernelGGL((penalty_rows_kernel<true, true>), grid, dim3(kThreads), 0, stream, logits, R, V, g,
                               lens, extra_rows, have_hist, P, workspace, tokens, K, theta, presence, frequency, out);
        else
            hipLaunchKernelGGL((penalty_rows_kernel<true, false>), grid, dim3(kThreads), 0, stream, logits, R, V, g,
                               lens, extra_rows, have_hist, P, workspace, tokens, K, theta, presence, frequency, out);
    } else {
        if (vec)
            hipLaunchKernelGGL((penalty_rows_kernel<false, true>), grid, dim3(kThreads), 0, stream, logits, R, V, g,
                               lens, extra_rows, have_hist, P, workspace, tokens, K, theta, presence, frequency, out);
        else
            hipLaunchKernelGGL((penalty_rows_kernel<false, false>), grid, dim3(kThreads), 0, stream, logits, R, V, g,
                               lens, extra_rows, have_hist, P, workspace, tokens, K, theta, presence, frequency, out);
    }
    return hipGetLastError();
}

}  // namespace sv
