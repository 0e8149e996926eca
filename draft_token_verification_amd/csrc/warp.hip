// warp.hip -- temperature warp p = softmax(z / T) over rows, for gfx950.
//
// The sampled verify compares the distributions the sampler would draw from,
// after temperature, with target and draft warped the same way (llmstudio
// blog "Как работает speculative decoding и MTP при инференсе LLM", sections
// 21-22 and 38; spec-verify card, "Requirements and limits").
//
// Work in the log2 domain: y = z * (log2(e) / T), p = 2^(y - M) / S with
// M = max y and S = sum 2^(y - M). Two mappings:
//
// Cooperative (the fast path: V a multiple of 4, aligned rows, a workspace).
//   Each live row is split over G workgroups of 1024 lanes; lane t of slice g
//   holds 32 elements in registers, so the row is read from HBM exactly once.
//   Every workgroup reduces its slice to (m, s), publishes it as one 64-bit
//   word into the row's slot g (a relaxed device-scope atomic store into a slot
//   pre-filled with an all-ones sentinel -- the value is its own ready flag, so
//   no cache-wide release or acquire is needed), waits until the row's G slots
//   are filled, merges them in a fixed order, and writes its slice. Only about
//   (resident workgroups / G) rows are written at a time, which keeps the write
//   front compact: measured, that is what lets the fp32 stores stream at HBM
//   speed, where one-row-per-workgroup writes spread over hundreds of rows.
//   The wait is bounded. A workgroup that gives up recomputes all G slice
//   partials itself with the same code and the same lane mapping, so the result
//   is bitwise identical either way and the kernel can never hang.
// Per row (other layouts, or no workspace).
//   One workgroup per live row, two passes: online (max, sum) with cacheable
//   loads, then the normalised write reading the row again.
// Rows past a sequence's live count exit at once in both.
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCoopMaxG = 64;                       // slices per row the cooperative path accepts


__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Four consecutive elements per lane: 8 bytes of bf16 or 16 bytes of fp32.
template <bool BF16>
struct Quad;

template <>
struct Quad<true> {
    using Raw = u32x2;
    __device__ static Raw load(const Raw* p) { return *p; }
    __device__ static Raw load_last(const Raw* p) { return __builtin_nontemporal_load(p); }
    __device__ static Raw neg_inf() { return Raw{0xFF80FF80u, 0xFF80FF80u}; }
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
    __device__ static Raw neg_inf() { return Raw{-INFINITY, -INFINITY, -INFINITY, -INFINITY}; }
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
    if (m == -INFINITY) return;  // all -inf so far: nothing to add (and no -inf - -inf)
#pragma unroll
    for (int k = 0; k < N; ++k) s += ex2(fmaf(z[k], scale, -m));
}

__device__ __forceinline__ f32x4 normalised(const float z[4], float scale, float m, float inv) {
    f32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = ex2(fmaf(z[k], scale, -m)) * inv;
    return o;
}

constexpr int kCoopEpt = 32;                       // elements per lane in the cooperative path
constexpr int kCoopQuads = kCoopEpt / 4;
constexpr int kCoopSlice = kThreads * kCoopEpt;      // elements per workgroup slice
constexpr unsigned long long kEmpty = ~0ull;         // slot sentinel (a NaN pair: never a valid (m, s))

std::atomic<int> g_wait_limit{1 << 14};              // polls before a workgroup recomputes the row itself

__global__ void fill_slots(unsigned long long* __restrict__ slots, int64_t n) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < n) slots[i] = kEmpty;
}

__device__ __forceinline__ unsigned long long pack_ms(float m, float s) {
    return ((unsigned long long)__float_as_uint(s) << 32) | __float_as_uint(m);
}

// (m, s) of slice g of a row, reduced over the workgroup (uniform result;
// one barrier, so callers separate consecutive calls with another).
// KEEP: also leave the slice's 32 elements per lane in z (elements past V
// read as -inf). Both forms load and accumulate the same values in the same
// order, so they return bitwise identical partials.
template <bool BF16, bool KEEP>
__device__ __forceinline__ void slice_partial(const void* zrow, int nq, int g, float scale, float* z, float& m,
                                              float& s, float* lds_m, float* lds_s) {
    using Q = Quad<BF16>;
    const typename Q::Raw* vz = (const typename Q::Raw*)zrow;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int q0 = g * kThreads * kCoopQuads;
    m = -INFINITY;
    s = 0.0f;
    // All loads are issued before any is used (the select keeps them in
    // flight together); elements past V read as -inf.
    typename Q::Raw raw[kCoopQuads];
#pragma unroll
    for (int u = 0; u < kCoopQuads; ++u) {
        const int j = q0 + u * kThreads + tid;
        raw[u] = j < nq ? (KEEP ? Q::load_last(vz + j) : Q::load(vz + j)) : Q::neg_inf();
    }
    float t[kCoopEpt];
    float* zz = KEEP ? z : t;
#pragma unroll
    for (int u = 0; u < kCoopQuads; ++u) Q::unpack(raw[u], zz + 4 * u);
#pragma unroll
    for (int u = 0; u < kCoopQuads; ++u)
        if (q0 + u * kThreads + tid < nq) online_add<4>(zz + 4 * u, scale, m, s);
    wave_lse(m, s);
    if (lane == 0) {
        lds_m[wave] = m;
        lds_s[wave] = s;
    }
    __syncthreads();
    m = lane < kWaves ? lds_m[lane] : -INFINITY;
    s = lane < kWaves ? lds_s[lane] : 0.0f;
    wave_lse(m, s);
}

// Merge packed partials in a fixed order: lane k takes entries k, k+64, ...
// of vals[0..G), then the wavefront merges its lanes. Wavefront 0 only.
__device__ __forceinline__ void merge_lane(unsigned long long v, float& pm, float& ps) {
    lse_merge(pm, ps, __uint_as_float((unsigned)v), __uint_as_float((unsigned)(v >> 32)));
}

// Normalise and write slice g of a row from the 32 elements per lane in z.
__device__ __forceinline__ void write_slice(float* prow, int nq, int g, const float* z, float scale, float M,
                                            float inv) {
    f32x4* vp = (f32x4*)prow;
    const int q0 = g * kThreads * kCoopQuads;
#pragma unroll
    for (int u = 0; u < kCoopQuads; ++u) {
        const int j = q0 + u * kThreads + threadIdx.x;
        if (j < nq) store_nt(vp + j, normalised(z + 4 * u, scale, M, inv));
    }
}

// The bounded wait ran out: recompute every slice's partial exactly as its
// own workgroup did, merge them exactly as the waiting path does, then reload
// this workgroup's slice and write it. Called by the whole workgroup.
template <bool BF16>
__device__ __forceinline__ void coop_fallback(const void* zrow, float* prow, int nq, int G, int g,
                                                        float scale, float* lds_m, float* lds_s,
                                                        unsigned long long* lds_p, float* s_M, float* s_S) {
    const int tid = threadIdx.x;
    for (int k = 0; k < G; ++k) {
        float mk, sk;
        __syncthreads();  // lds_m / lds_s of the previous reduction are consumed
        slice_partial<BF16, false>(zrow, nq, k, scale, nullptr, mk, sk, lds_m, lds_s);
        if (tid == 0) lds_p[k] = pack_ms(mk, sk);
    }
    __syncthreads();
    if (tid < kWave) {
        float pm = -INFINITY, ps = 0.0f;
        for (int k = tid; k < G; k += kWave) merge_lane(lds_p[k], pm, ps);
        wave_lse(pm, ps);
        if (tid == 0) {
            *s_M = pm;
            *s_S = ps;
        }
    }
    __syncthreads();
    float z[kCoopEpt], m, s;
    slice_partial<BF16, true>(zrow, nq, g, scale, z, m, s, lds_m, lds_s);
    write_slice(prow, nq, g, z, scale, *s_M, 1.0f / *s_S);
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void warp_coop_kernel(const void* __restrict__ logits, int R, int V, int G,
                                                             const int32_t* __restrict__ lens, int extra_rows,
                                                             float scale, float* __restrict__ probs,
                                                             unsigned long long* __restrict__ slots, int wait_limit) {
    __shared__ float lds_m[kWaves], lds_s[kWaves];
    __shared__ unsigned long long lds_p[kCoopMaxG];
    __shared__ float s_M, s_S;
    __shared__ int s_ready;
    const int row = blockIdx.x / G, g = blockIdx.x - row * G;
    const int b = row / R, r = row - b * R;
    const int live = clamp_len(lens, b, R - extra_rows) + extra_rows;
    if (r >= live) return;
    const int tid = threadIdx.x;
    const int nq = V / 4;
    const char* zrow = (const char*)logits + (size_t)row * (size_t)V * (BF16 ? 2 : 4);
    float* prow = probs + (size_t)row * (size_t)V;
    unsigned long long* my_slots = slots + (size_t)row * G;

    float z[kCoopEpt], m, s;
    slice_partial<BF16, true>(zrow, nq, g, scale, z, m, s, lds_m, lds_s);
    if (tid == 0) __hip_atomic_store(my_slots + g, pack_ms(m, s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // Wavefront 0 polls the row's G slots (bounded) and merges them in
    // registers, lane k taking slots k, k+64, ... in order.
    if (tid < kWave) {
        bool ready = false;
        float pm = -INFINITY, ps = 0.0f;
        for (int tries = 0; tries <= wait_limit; ++tries) {
            bool mine = true;
            pm = -INFINITY;
            ps = 0.0f;
            for (int k = tid; k < G; k += kWave) {
                const unsigned long long v = __hip_atomic_load(my_slots + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v == kEmpty)
                    mine = false;
                else
                    merge_lane(v, pm, ps);
            }
            if (__ballot(!mine) == 0) {
                ready = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (ready) wave_lse(pm, ps);
        if (tid == 0) {
            s_ready = ready;
            s_M = pm;
            s_S = ps;
        }
    }
    __syncthreads();
    if (s_ready) {
        write_slice(prow, nq, g, z, scale, s_M, 1.0f / s_S);
        return;
    }
    coop_fallback<BF16>(zrow, prow, nq, G, g, scale, lds_m, lds_s, lds_p, &s_M, &s_S);
}

// VEC: V is a multiple of 4 and rows start on load/store boundaries
// (checked by the launcher); otherwise one element per lane per step.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void warp_rows_kernel(const void* __restrict__ logits, int R, int V,
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

int64_t warp_coop_slices(int V) { return ((int64_t)V + kCoopSlice - 1) / kCoopSlice; }

size_t warp_workspace_bytes(int B, int R, int V) {
    const int64_t G = warp_coop_slices(V);
    if (V % 4 != 0 || G > kCoopMaxG) return 0;
    return (size_t)B * (size_t)R * (size_t)G * sizeof(unsigned long long);
}

void set_wait_limit(int tries) { g_wait_limit.store(tries); }

hipError_t launch_warp(const void* logits, bool bf16, int B, int R, int V, const int32_t* lens, int extra_rows,
                       float temperature, float* probs, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const float scale = kLog2e / temperature;
    const bool vec = (V % 4 == 0) && ((uintptr_t)logits % (bf16 ? 8 : 16) == 0) && ((uintptr_t)probs % 16 == 0);
    const size_t need = warp_workspace_bytes(B, R, V);
    if (vec && need > 0 && workspace != nullptr && workspace_bytes >= need && ((uintptr_t)workspace % 8) == 0 &&
        (int64_t)B * R * warp_coop_slices(V) <= INT32_MAX) {
        const int G = (int)warp_coop_slices(V);
        const int64_t nslots = (int64_t)B * R * G;
        hipLaunchKernelGGL(fill_slots, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, stream,
                           (unsigned long long*)workspace, nslots);
        const hipError_t fe = hipGetLastError();
        if (fe != hipSuccess) return fe;  // without the fill, stale slots would read as published
        const dim3 grid((unsigned)((int64_t)B * R * G));
        if (bf16)
            hipLaunchKernelGGL((warp_coop_kernel<true>), grid, dim3(kThreads), 0, stream, logits, R, V, G, lens,
                               extra_rows, scale, probs, (unsigned long long*)workspace, g_wait_limit.load());
        else
            hipLaunchKernelGGL((warp_coop_kernel<false>), grid, dim3(kThreads), 0, stream, logits, R, V, G, lens,
                               extra_rows, scale, probs, (unsigned long long*)workspace, g_wait_limit.load());
        return hipGetLastError();
    }
    const dim3 grid((unsigned)B * (unsigned)R);
    if (bf16) {
        if (vec)
            hipLaunchKernelGGL((warp_rows_kernel<true, true>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, scale, probs);
        else
            hipLaunchKernelGGL((warp_rows_kernel<true, false>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, scale, probs);
    } else {
        if (vec)
            hipLaunchKernelGGL((warp_rows_kernel<false, true>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, scale, probs);
        else
            hipLaunchKernelGGL((warp_rows_kernel<false, false>), grid, dim3(kThreads), 0, stream, logits, R, V, lens,
                               extra_rows, scale, probs);
    }
    return hipGetLastError();
}

int get_wait_limit() { return g_wait_limit.load(); }

// ---- exchange slots without a caller's workspace ---------------------------
// The cooperative warp's slots in a fixed device array, for callers that
// cannot allocate: one copy per device, alive until the process ends, shared
// by every call on that device (so calls that overlap on one device race; the
// fill kernel resets the slots at the start of each call). In host code the
// array's name stands for a host shadow, never a device address: the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current.
static __device__ __align__(256) unsigned long long scratch[kStaticScratchBytes / sizeof(unsigned long long)];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];
}  // namespace

hipError_t static_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace sv
