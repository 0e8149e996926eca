// common.hpp -- device helpers shared by the libspecverify kernels (gfx950,
// wave64). Internal to the library; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- loads and stores ---------------------------------------------------
// Streamed rows are read once per pass; the non-temporal hint keeps them from
// displacing data that is reused.
__device__ __forceinline__ u32x4 load_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ f32x4 load_nt(const f32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_nt(f32x4* p, f32x4 v) { __builtin_nontemporal_store(v, p); }

// bf16 -> fp32 is exact: a bf16 is the upper half of the fp32 with the same bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p, int64_t i) { return __uint_as_float((uint32_t)p[i] << 16); }

// ---- cross-lane moves -----------------------------------------------------
// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane j <-> 7-j within each group of 8
constexpr int kDppRowMirror = 0x140;      // lane j <-> 15-j within each row of 16
// ds_swizzle bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10 -> lane ^ 16 within 32.
constexpr int kSwizzleXor16 = 0x401F;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
    int lo = __double2loint(x), hi = __double2hiint(x);
    return __hiloint2double(dpp_i<CTRL>(hi), dpp_i<CTRL>(lo));
}
__device__ __forceinline__ int swz16_i(int x) { return __builtin_amdgcn_ds_swizzle(x, kSwizzleXor16); }
__device__ __forceinline__ float swz16_f(float x) { return __int_as_float(swz16_i(__float_as_int(x))); }
__device__ __forceinline__ double swz16_d(double x) {
    return __hiloint2double(swz16_i(__double2hiint(x)), swz16_i(__double2loint(x)));
}
__device__ __forceinline__ int readlane_i(int x, int lane) { return __builtin_amdgcn_readlane(x, lane); }
__device__ __forceinline__ float readlane_f(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ double readlane_d(double x, int lane) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), lane),
                            __builtin_amdgcn_readlane(__double2loint(x), lane));
}

// ---- argmax with lowest-index ties ----------------------------------------
// (v, i) wins over (w, j) iff v > w, or v == w and i < j. This is a total
// order on (value, index) pairs of non-NaN values, so any combining order
// gives the same winner. IEEE == makes -0.0 and +0.0 tie.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float w, int j) {
    bool take = (w > v) | ((w == v) & (j < i));
    v = take ? w : v;
    i = take ? j : i;
}

// Wave-wide argmax: xor-1 and xor-2 quad permutes, half-row and row mirrors,
// a ds_swizzle across the two halves of each 32-lane group, and a final merge
// of lanes 0 and 32 through scalar reads. The result is wave-uniform.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    argmax_merge(v, i, dpp_f<kDppQuadXor1>(v), dpp_i<kDppQuadXor1>(i));
    argmax_merge(v, i, dpp_f<kDppQuadXor2>(v), dpp_i<kDppQuadXor2>(i));
    argmax_merge(v, i, dpp_f<kDppRowHalfMirror>(v), dpp_i<kDppRowHalfMirror>(i));
    argmax_merge(v, i, dpp_f<kDppRowMirror>(v), dpp_i<kDppRowMirror>(i));
    argmax_merge(v, i, swz16_f(v), swz16_i(i));
    float v0 = readlane_f(v, 0), v1 = readlane_f(v, 32);
    int i0 = readlane_i(i, 0), i1 = readlane_i(i, 32);
    argmax_merge(v0, i0, v1, i1);
    v = v0;
    i = i0;
}

// ---- fp64 wave sum (fixed butterfly order; result wave-uniform) ------------
__device__ __forceinline__ double wave_sum_d(double x) {
    x += dpp_d<kDppQuadXor1>(x);
    x += dpp_d<kDppQuadXor2>(x);
    x += dpp_d<kDppRowHalfMirror>(x);
    x += dpp_d<kDppRowMirror>(x);
    x += swz16_d(x);
    return readlane_d(x, 0) + readlane_d(x, 32);
}

// fp64 inclusive scan over the 64 lanes (Hillis-Steele, fixed order).
__device__ __forceinline__ double wave_incl_scan_d(double x, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        double y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    return x;
}

// The largest of three floats in one instruction. Written out because
// fmaxf on values that come from bit operations (unpacked bf16) or straight
// from memory makes the compiler quiet each operand with an extra max first.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ float max2f(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

template <int N>
__device__ __forceinline__ float max_of(const float* z) {
    static_assert(N >= 2, "");
    float r = max3f(z[0], z[1], N > 2 ? z[2] : z[1]);
#pragma unroll
    for (int k = 3; k < N; k += 2) r = max3f(r, z[k], z[k + 1 < N ? k + 1 : k]);
    return r;
}

// ---- softmax statistics in the log2 domain --------------------------------
// (m, s) describes sum_x 2^(y_x - m) = s. Merging keeps the larger m.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
    float mm = fmaxf(m, m2);
    float a = (m == -INFINITY) ? 0.0f : s * __builtin_amdgcn_exp2f(m - mm);
    float b = (m2 == -INFINITY) ? 0.0f : s2 * __builtin_amdgcn_exp2f(m2 - mm);
    m = mm;
    s = a + b;
}

__device__ __forceinline__ void wave_lse(float& m, float& s) {
    lse_merge(m, s, dpp_f<kDppQuadXor1>(m), dpp_f<kDppQuadXor1>(s));
    lse_merge(m, s, dpp_f<kDppQuadXor2>(m), dpp_f<kDppQuadXor2>(s));
    lse_merge(m, s, dpp_f<kDppRowHalfMirror>(m), dpp_f<kDppRowHalfMirror>(s));
    lse_merge(m, s, dpp_f<kDppRowMirror>(m), dpp_f<kDppRowMirror>(s));
    lse_merge(m, s, swz16_f(m), swz16_f(s));
    float m0 = readlane_f(m, 0), s0 = readlane_f(s, 0);
    lse_merge(m0, s0, readlane_f(m, 32), readlane_f(s, 32));
    m = m0;
    s = s0;
}

__device__ __forceinline__ int clamp_len(const int32_t* lens, int b, int K) {
    if (lens == nullptr) return K;
    int k = lens[b];
    return k < 0 ? 0 : (k > K ? K : k);
}

// ---- exchange between the workgroups that share a row or a sequence --------
// Slots are 64-bit words in a caller's workspace, filled with kEmptySlot
// before the launch; a workgroup publishes its partial result into its own
// slot with a relaxed agent-scope store and the others poll for it (bounded).
constexpr unsigned long long kEmptySlot = ~0ull;  // a NaN pattern: never a published value

// Wavefront 0 polls words set[0 .. nw) (bounded) and copies them to LDS;
// returns whether all were published (uniform after the barrier).
__device__ __forceinline__ bool gather_words(const unsigned long long* set, int nw, int wait_limit,
                                             unsigned long long* s_words, int* s_ready,
                                             unsigned long long empty = kEmptySlot) {
    const int tid = threadIdx.x;
    if (tid < kWave) {
        bool ready = false;
        for (int tries = 0; tries <= wait_limit; ++tries) {
            bool mine = true;
            for (int k = tid; k < nw; k += kWave) {
                const unsigned long long v = __hip_atomic_load(set + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v == empty)
                    mine = false;
                else
                    s_words[k] = v;
            }
            if (__ballot(!mine) == 0) {
                ready = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (tid == 0) *s_ready = ready;
    }
    __syncthreads();
    return *s_ready;
}

__device__ __forceinline__ void publish_word(unsigned long long* slot, unsigned long long v) {
    if (threadIdx.x == 0) __hip_atomic_store(slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sv
