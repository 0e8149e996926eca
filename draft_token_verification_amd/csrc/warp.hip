// warp.hip -- temperature warp p = softmax(z / T) over rows, for gfx950.
//
// The sampled verify compares the distributions the sampler would draw from,
// after temperature, with target and draft warped the same way (llmstudio
// blog "Как работает speculative decoding и MTP при инференсе LLM", sections
// 21-22 and 38; spec-verify card, "Requirements and limits").
//
// Mapping: one workgroup (1024 lanes) per live row; rows past a sequence's
// live count exit at once. Work in the log2 domain: y = z * (log2(e) / T),
// p = 2^(y - M) / S with M = max y and S = sum 2^(y - M).
//   pass 1: plain (cacheable) loads, per-lane online (max, sum) with a
//           rescale only when a lane's running max grows; (max, sum) pairs
//           merge across the wavefront with DPP and a ds_swizzle, then across
//           wavefronts through LDS;
//   pass 2: the row is read again -- pass 1 left it in the caches in front of
//           HBM -- with non-temporal loads, and 2^(y - M) * (1/S) is written
//           as fp32 with non-temporal 16-byte stores.
// Every lane handles 4 consecutive elements per step (an 8-byte bf16 or
// 16-byte fp32 load), so each 16-byte store instruction covers a contiguous
// kilobyte across the wavefront: whole cache lines, no partial-line writes.
#include "common.hpp"
#include "launch.hpp"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 8;
constexpr float kLog2e = 1.4426950408889634f;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Four consecutive elements per lane: 8 bytes of bf16 or 16 bytes of fp32.
template <bool BF16>
struct Quad;

template <>
struct Quad<true> {
    using Raw = u32x2;
    __device__ static Raw load(const Raw* p) { return *p; }
    __device__ static Raw load_last(const Raw* p) { return __builtin_nontemporal_load(p); }
    __device__ static void unpack(const Raw& r, float z[4]) {
        z[0] = bf16_lo(r[0]);
        z[1] = bf16_hi(r[0]);
        z[2] = bf16_lo(r[1]);
        z[3] = bf16_hi(r[1]);
    }
    __device__ static float at(const void* row, int64_t i) { return bf16_at((const uint16_t*)row, i); }
};

template <>
struct Quad<false> {
    using Raw = f32x4;
    __device__ static Raw load(const Raw* p) { return *p; }
    __device__ static Raw load_last(const Raw* p) { return load_nt(p); }
    __device__ static void unpack(const Raw& r, float z[4]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) z[k] = r[k];
    }
    __device__ static float at(const void* row, int64_t i) { return ((const float*)row)[i]; }
};

template <int N>
__device__ __forceinline__ void online_add(const float z[N], float scale, float& m, float& s) {
    float zm = z[0];
#pragma unroll
    for (int k = 1; k < N; ++k) zm = fmaxf(zm, z[k]);
    const float ym = zm * scale;
    if (ym > m) {
        s = (m == -INFINITY) ? 0.0f : s * ex2(m - ym);
        m = ym;
    }
#pragma unroll
    for (int k = 0; k < N; ++k) s += ex2(fmaf(z[k], scale, -m));
}

__device__ __forceinline__ f32x4 normalised(const float z[4], float scale, float m, float inv) {
    f32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = ex2(fmaf(z[k], scale, -m)) * inv;
    return o;
}

// VEC: V is a multiple of 4 and rows start on load/store boundaries
// (checked by the launcher); otherwise one element per lane per step.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void warp_kernel(const void* __restrict__ logits, int R, int V,
                                                        const int32_t* __restrict__ lens, int extra_rows,
                                                        float scale, float* __restrict__ probs) {
    using Q = Quad<BF16>;
    __shared__ float lds_m[kWaves], lds_s[kWaves];
    const int row = blockIdx.x;
    const int b = row / R, r = row - b * R;
    const int live = clamp_len(lens, b, R - extra_rows) + extra_rows;
    if (r >= live) return;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const char* zrow = (const char*)logits + (size_t)row * (size_t)V * (BF16 ? 2 : 4);
    float* prow = probs + (size_t)row * (size_t)V;
    const typename Q::Raw* vz = (const typename Q::Raw*)zrow;
    const int nq = V / 4;

    // pass 1: online max / sum
    float m = -INFINITY, s = 0.0f;
    if (VEC) {
        int j = tid;
        for (; j + (kUnroll - 1) * kThreads < nq; j += kUnroll * kThreads) {
            typename Q::Raw raw[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) raw[u] = Q::load(vz + j + u * kThreads);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float z[4];
                Q::unpack(raw[u], z);
                online_add<4>(z, scale, m, s);
            }
        }
        for (; j < nq; j += kThreads) {
            float z[4];
            Q::unpack(Q::load(vz + j), z);
            online_add<4>(z, scale, m, s);
        }
    } else {
        for (int x = tid; x < V; x += kThreads) {
            float z[1] = {Q::at(zrow, x)};
            online_add<1>(z, scale, m, s);
        }
    }
    wave_lse(m, s);
    if (lane == 0) {
        lds_m[wave] = m;
        lds_s[wave] = s;
    }
    __syncthreads();
    m = lane < kWaves ? lds_m[lane] : -INFINITY;
    s = lane < kWaves ? lds_s[lane] : 0.0f;
    wave_lse(m, s);
    const float inv = 1.0f / s;

    // pass 2: normalised probabilities
    if (VEC) {
        f32x4* vp = (f32x4*)prow;
        int j = tid;
        for (; j + (kUnroll - 1) * kThreads < nq; j += kUnroll * kThreads) {
            typename Q::Raw raw[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) raw[u] = Q::load_last(vz + j + u * kThreads);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float z[4];
                Q::unpack(raw[u], z);
                store_nt(vp + j + u * kThreads, normalised(z, scale, m, inv));
            }
        }
        for (; j < nq; j += kThreads) {
            float z[4];
            Q::unpack(Q::load_last(vz + j), z);
            store_nt(vp + j, normalised(z, scale, m, inv));
        }
    } else {
        for (int x = tid; x < V; x += kThreads) prow[x] = ex2(fmaf(Q::at(zrow, x), scale, -m)) * inv;
    }
}

}  // namespace

hipError_t launch_warp(const void* logits, bool bf16, int B, int R, int V, const int32_t* lens, int extra_rows,
                       float temperature, float* probs, hipStream_t stream) {
    const float scale = kLog2e / temperature;
    const bool vec = (V % 4 == 0) && ((uintptr_t)logits % (bf16 ? 8 : 16) == 0) && ((uintptr_t)probs % 16 == 0);
    const dim3 grid((unsigned)B * (unsigned)R);
    if (bf16) {
        if (vec)
            hipLaunchKernelGGL((warp_kernel<true, true>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, scale, probs);
        else
            hipLaunchKernelGGL((warp_kernel<true, false>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, scale, probs);
    } else {
        if (vec)
            hipLaunchKernelGGL((warp_kernel<false, true>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, scale, probs);
        else
            hipLaunchKernelGGL((warp_kernel<false, false>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, scale, probs);
    }
    return hipGetLastError();
}

}  // namespace sv
