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
//   pass 1: 16-byte non-temporal loads, per-lane online (max, sum) with a
//           rescale only when a lane's running max grows; (max, sum) pairs
//           merge across the wavefront with DPP and a ds_swizzle, then across
//           wavefronts through LDS;
//   pass 2: the row is read again (recently touched, so mostly served by the
//           caches in front of HBM) and 2^(y - M) * (1/S) is written as fp32
//           with 16-byte non-temporal stores.
#include "common.hpp"
#include "launch.hpp"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 2;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 vectors carry 8 elements, fp32 vectors 4.
template <bool BF16>
struct Vec8;

template <>
struct Vec8<true> {
    static constexpr int kN = 8;
    using Raw = u32x4;
    __device__ static void unpack(const Raw& r, float z[8]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            z[2 * k] = bf16_lo(r[k]);
            z[2 * k + 1] = bf16_hi(r[k]);
        }
    }
    __device__ static float at(const void* row, int64_t i) { return bf16_at((const uint16_t*)row, i); }
};

template <>
struct Vec8<false> {
    static constexpr int kN = 4;
    using Raw = f32x4;
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

// Vector path: the row and output start on 16-byte boundaries and V is a
// multiple of the vector width (checked by the launcher).
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void warp_kernel(const void* __restrict__ logits, int R, int V,
                                                        const int32_t* __restrict__ lens, int extra_rows,
                                                        float scale, float* __restrict__ probs) {
    using W = Vec8<BF16>;
    constexpr int E = W::kN;
    __shared__ float lds_m[kWaves], lds_s[kWaves];
    const int row = blockIdx.x;
    const int b = row / R, r = row - b * R;
    const int live = clamp_len(lens, b, R - extra_rows) + extra_rows;
    if (r >= live) return;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const char* zrow = (const char*)logits + (size_t)row * (size_t)V * (BF16 ? 2 : 4);
    float* prow = probs + (size_t)row * (size_t)V;

    // pass 1: online max / sum
    float m = -INFINITY, s = 0.0f;
    if (VEC) {
        const typename W::Raw* vz = (const typename W::Raw*)zrow;
        const int nvec = V / E;
        int j = tid;
        for (; j + (kUnroll - 1) * kThreads < nvec; j += kUnroll * kThreads) {
            typename W::Raw raw[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) raw[u] = load_nt(vz + j + u * kThreads);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float z[E];
                W::unpack(raw[u], z);
                online_add<E>(z, scale, m, s);
            }
        }
        for (; j < nvec; j += kThreads) {
            float z[E];
            W::unpack(load_nt(vz + j), z);
            online_add<E>(z, scale, m, s);
        }
    } else {
        for (int x = tid; x < V; x += kThreads) {
            float z[1] = {W::at(zrow, x)};
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
        const typename W::Raw* vz = (const typename W::Raw*)zrow;
        f32x4* vp = (f32x4*)prow;
        const int nvec = V / E;
        for (int j = tid; j < nvec; j += kThreads) {
            float z[E];
            W::unpack(load_nt(vz + j), z);
#pragma unroll
            for (int h = 0; h < E / 4; ++h) {
                f32x4 o;
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = ex2(fmaf(z[4 * h + k], scale, -m)) * inv;
                store_nt(vp + (int64_t)j * (E / 4) + h, o);
            }
        }
    } else {
        for (int x = tid; x < V; x += kThreads) prow[x] = ex2(fmaf(W::at(zrow, x), scale, -m)) * inv;
    }
}

}  // namespace

hipError_t launch_warp(const void* logits, bool bf16, int B, int R, int V, const int32_t* lens, int extra_rows,
                       float temperature, float* probs, hipStream_t stream) {
    const float scale = kLog2e / temperature;
    const int width = bf16 ? 8 : 4;
    const bool vec = (V % width == 0) && ((uintptr_t)logits % 16 == 0) && ((uintptr_t)probs % 16 == 0);
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
