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
//  2. penalty_rows_kernel, one 1024-lane workgroup per live row: the row is
//     streamed to fp32 (16-byte loads and stores, four loads in flight per
//     lane), then only the history's
//     ids are patched: each listed id with its count plus its occurrences in
//     the row's draft prefix, and each prefix id absent from the committed
//     history (once, at its first occurrence in the prefix). A row reads and
//     writes V elements plus O(history) scattered ones.
#include "common.hpp"
#include "launch.hpp"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxPrefix = kWave;  // draft prefixes are at most SV_MAX_K = 64 tokens
constexpr int kCopyUnroll = 4;     // loads in flight per lane in the row copy

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
    const void* __restrict__ logits, int R, int V, const int32_t* __restrict__ lens, int extra_rows, bool have_hist,
    int P, const void* __restrict__ ws, const int32_t* __restrict__ tokens, int K, const float* __restrict__ theta,
    const float* __restrict__ presence, const float* __restrict__ frequency, float* __restrict__ out) {
    __shared__ int32_t s_pre[kMaxPrefix];
    const int row = blockIdx.x;
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

    // 1. the row in fp32, kCopyUnroll 16-byte loads in flight per lane
    if (VEC) {
        constexpr int E = BF16 ? 8 : 4;  // elements per 16-byte load
        const u32x4* vin = (const u32x4*)zrow;
        const int nv = V / E;
        auto put = [&](int j, const u32x4& w) {
            f32x4* o = (f32x4*)(orow + (size_t)j * E);
            if (BF16) {
                store_nt(o, f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])});
                store_nt(o + 1, f32x4{bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3])});
            } else {
                store_nt(o, f32x4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                                  __uint_as_float(w[3])});
            }
        };
        int j = tid;
        for (; j + (kCopyUnroll - 1) * kThreads < nv; j += kCopyUnroll * kThreads) {
            u32x4 w[kCopyUnroll];
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) w[u] = vin[j + u * kThreads];
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) put(j + u * kThreads, w[u]);
        }
        for (; j < nv; j += kThreads) put(j, vin[j]);
    } else {
        for (int x = tid; x < V; x += kThreads) orow[x] = at(x);
    }
    // the draft prefix of this row: tokens[b, 0 .. r-1]
    const int np = tokens ? r : 0;
    if (tid < np) s_pre[tid] = tokens[(size_t)b * K + tid];
    __syncthreads();  // the copy's stores are complete before any patch overwrites one

    const float th = theta ? theta[b] : 1.0f;
    const float pr = presence ? presence[b] : 0.0f;
    const float fr = frequency ? frequency[b] : 0.0f;
    auto prefix_count = [&](int32_t id, int upto) {
        int c = 0;
        for (int j = 0; j < upto; ++j) c += s_pre[j] == id;
        return c;
    };
    const uint32_t mask = (uint32_t)P - 1u;
    // 2. ids of the committed history, with their prefix occurrences added
    if (have_hist) {
        const TableView t = table_of(const_cast<void*>(ws), b, P);
        const int n = *t.n;
        for (int k = tid; k < n; k += kThreads) {
            const int32_t id = t.list[2 * k];
            const int c = t.list[2 * k + 1] + prefix_count(id, np);
            orow[id] = penalised(at(id), c, th, pr, fr);
        }
    }
    // 3. ids that only the prefix holds, patched once (at their first occurrence)
    if (tid < np) {
        const int32_t id = s_pre[tid];
        if (id >= 0 && id < V && prefix_count(id, tid) == 0) {
            const bool committed = have_hist && table_count(table_of(const_cast<void*>(ws), b, P), id, mask) > 0;
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
    const bool vec = (V % (bf16 ? 8 : 4) == 0) && ((uintptr_t)logits % 16 == 0) && ((uintptr_t)out % 16 == 0);
    const dim3 grid((unsigned)((int64_t)B * R));
    if (bf16) {
        if (vec)
            hipLaunchKernelGGL((penalty_rows_kernel<true, true>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, have_hist, P, workspace, tokens, K, theta, presence, frequency, out);
        else
            hipLaunchKernelGGL((penalty_rows_kernel<true, false>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, have_hist, P, workspace, tokens, K, theta, presence, frequency, out);
    } else {
        if (vec)
            hipLaunchKernelGGL((penalty_rows_kernel<false, true>), grid, dim3(kThreads), 0, stream, logits, R, V,
                               lens, extra_rows, have_hist, P, workspace, tokens, K, theta, presence, frequency, out);
        else
            hipLaunchKernelGGL((penalty_rows_kernel<false, false>), grid, dim3(kThreads), 0, stream, logits, R, V,
                               lens, extra_rows, have_hist, P, workspace, tokens, K, theta, presence, frequency, out);
    }
    return hipGetLastError();
}

}  // namespace sv
