// greedy.hip -- greedy verification (temperature 0) for gfx950.
//
// Method (spec-verify card, "Method"; llmstudio blog "Как работает
// speculative decoding и MTP при инференсе LLM", sections 13 and 48): accept
// draft token t_i while it equals argmax(target row i); at the first miss emit
// that row's argmax; if all K_b match emit argmax(target row K_b).
//
// Mapping: one workgroup (1024 lanes, 16 wavefronts) owns one sequence and
// walks its rows in order, so the early exit at the first miss is a plain
// loop exit: rows after the miss are never fetched and no workgroup waits on
// another. Each row is one streaming argmax over V elements:
//   - 16-byte coalesced non-temporal loads (8 bf16 or 4 fp32 per load),
//     UNROLL loads in flight per lane;
//   - per lane, a strict '>' keeps the first of equal maxima (each lane sees
//     its elements in increasing index order);
//   - wave64 merge with DPP quad permutes and row mirrors, a ds_swizzle and
//     two scalar lane reads; the 16 wave results meet in LDS and every
//     wavefront merges them again, so the row's argmax is uniform in all lanes.
#include "common.hpp"
#include "launch.hpp"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 8;

template <bool BF16>
struct RowReader;

// bf16 rows: 8 elements per 16-byte vector.
template <>
struct RowReader<true> {
    static constexpr int kPerVec = 8;
    using Vec = u32x4;
    __device__ static float at(const void* row, int64_t i) { return bf16_at((const uint16_t*)row, i); }
    __device__ static void scan(const Vec& w, int base, float& best, int& bidx) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float lo = bf16_lo(w[k]), hi = bf16_hi(w[k]);
            if (lo > best) { best = lo; bidx = base + 2 * k; }
            if (hi > best) { best = hi; bidx = base + 2 * k + 1; }
        }
    }
    // First vector of a lane: an element that only ties -inf must still be
    // taken when the lane holds nothing yet.
    __device__ static void scan_first(const Vec& w, int base, float& best, int& bidx) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float lo = bf16_lo(w[k]), hi = bf16_hi(w[k]);
            if (lo > best || bidx == INT32_MAX) { best = lo; bidx = base + 2 * k; }
            if (hi > best) { best = hi; bidx = base + 2 * k + 1; }
        }
    }
};

// fp32 rows: 4 elements per 16-byte vector.
template <>
struct RowReader<false> {
    static constexpr int kPerVec = 4;
    using Vec = f32x4;
    __device__ static float at(const void* row, int64_t i) { return ((const float*)row)[i]; }
    __device__ static void scan(const Vec& w, int base, float& best, int& bidx) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (w[k] > best) { best = w[k]; bidx = base + k; }
    }
    __device__ static void scan_first(const Vec& w, int base, float& best, int& bidx) {
        if (w[0] > best || bidx == INT32_MAX) { best = w[0]; bidx = base; }
#pragma unroll
        for (int k = 1; k < 4; ++k)
            if (w[k] > best) { best = w[k]; bidx = base + k; }
    }
};

// Argmax of one row of V elements. Returns the wave-uniform index; every lane
// of the workgroup must call it (it contains one barrier). `slot` alternates
// between two LDS buffers so that consecutive rows never race on them.
template <bool BF16>
__device__ int block_argmax(const void* row, int V, float (*lds_v)[kWaves], int (*lds_i)[kWaves], int slot) {
    using R = RowReader<BF16>;
    constexpr int E = R::kPerVec;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;

    // Elements before the first 16-byte boundary, one per lane.
    const uintptr_t addr = (uintptr_t)row;
    int head = (int)(((16u - (addr & 15u)) & 15u) / (BF16 ? 2u : 4u));
    if (head > V) head = V;
    const int nvec = (V - head) / E;
    const int tail0 = head + nvec * E;

    float best = -INFINITY;
    int bidx = INT32_MAX;
    if (tid < head) {
        best = R::at(row, tid);
        bidx = tid;
    }
    const typename R::Vec* vrow = (const typename R::Vec*)((const char*)row + head * (BF16 ? 2 : 4));
    int j = tid;
    if (j < nvec) {
        R::scan_first(load_nt(vrow + j), head + j * E, best, bidx);
        j += kThreads;
    }
    for (; j + (kUnroll - 1) * kThreads < nvec; j += kUnroll * kThreads) {
        typename R::Vec w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) w[u] = load_nt(vrow + j + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) R::scan(w[u], head + (j + u * kThreads) * E, best, bidx);
    }
    for (; j < nvec; j += kThreads) R::scan(load_nt(vrow + j), head + j * E, best, bidx);
    if (tail0 + tid < V) {
        float v = R::at(row, tail0 + tid);
        if (v > best || bidx == INT32_MAX) { best = v; bidx = tail0 + tid; }
    }

    wave_argmax(best, bidx);
    if (lane == 0) {
        lds_v[slot][wave] = best;
        lds_i[slot][wave] = bidx;
    }
    __syncthreads();
    float v = lane < kWaves ? lds_v[slot][lane] : -INFINITY;
    int i = lane < kWaves ? lds_i[slot][lane] : INT32_MAX;
    wave_argmax(v, i);
    return i;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void greedy_kernel(const void* __restrict__ target, int K, int V,
                                                          const int32_t* __restrict__ tokens,
                                                          const int32_t* __restrict__ lens,
                                                          int32_t* __restrict__ n_accepted,
                                                          int32_t* __restrict__ next_token) {
    __shared__ float lds_v[2][kWaves];
    __shared__ int lds_i[2][kWaves];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int kb = clamp_len(lens, b, K);
    // Draft token i sits in lane i (K <= 64); only positions < K_b are read.
    const int my_tok = lane < kb ? tokens[(int64_t)b * K + lane] : -1;
    const size_t row_bytes = (size_t)V * (BF16 ? 2 : 4);
    const char* base = (const char*)target + (size_t)b * (size_t)(K + 1) * row_bytes;

    int i = 0;
    for (;; ++i) {
        const int am = block_argmax<BF16>(base + (size_t)i * row_bytes, V, lds_v, lds_i, i & 1);
        // a token outside [0, V) never equals an argmax: it is a miss
        if (i == kb || readlane_i(my_tok, i) != am) {
            if (threadIdx.x == 0) {
                n_accepted[b] = i;
                next_token[b] = am;
            }
            return;
        }
    }
}

}  // namespace

hipError_t launch_greedy(const void* target, bool bf16, int B, int K, int V, const int32_t* tokens,
                         const int32_t* lens, int32_t* n_accepted, int32_t* next_token, hipStream_t stream) {
    if (bf16)
        hipLaunchKernelGGL(greedy_kernel<true>, dim3(B), dim3(kThreads), 0, stream, target, K, V, tokens, lens,
                           n_accepted, next_token);
    else
        hipLaunchKernelGGL(greedy_kernel<false>, dim3(B), dim3(kThreads), 0, stream, target, K, V, tokens, lens,
                           n_accepted, next_token);
    return hipGetLastError();
}

}  // namespace sv
