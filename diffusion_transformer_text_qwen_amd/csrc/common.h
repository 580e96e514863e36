// Shared device helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxSeg = 16;

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float f) { return (__bf16)f; }
__device__ __forceinline__ float bf16r(float f) { return (float)(__bf16)f; }

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<__bf16>(__bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ __bf16 from_f<__bf16>(float v) { return (__bf16)v; }

// Round to the storage precision of the mode: identity for fp32, bf16 otherwise.
template <typename T> __device__ __forceinline__ float store_round(float v);
template <> __device__ __forceinline__ float store_round<float>(float v) { return v; }
template <> __device__ __forceinline__ float store_round<__bf16>(float v) { return bf16r(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Block-wide reduction over `nwaves` waves through a small LDS array.
template <int NWAVES, bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* red) {
    v = MAX ? wave_max(v) : wave_sum(v);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    __syncthreads();
    if (l == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < NWAVES; ++i) r = MAX ? fmaxf(r, red[i]) : r + red[i];
    return r;
}

// Row -> modulation set lookup.  Segments are consecutive ranges of the
// sequence; row r of a call sits at absolute position row_offset + r.
struct SegMap {
    int64_t end[kMaxSeg];   // absolute end position of each segment
    int32_t set[kMaxSeg];   // modulation set of each segment
    int32_t n;
    int64_t row_offset;
};

// Unrolled with static indices only, so the argument struct stays in
// registers / the kernel-argument segment (no private copy).
__device__ __forceinline__ int seg_set(const SegMap& sm, int64_t row) {
    const int64_t p = sm.row_offset + row;
    int set = sm.set[0];
#pragma unroll
    for (int s = 0; s < kMaxSeg - 1; ++s)
        if (s < sm.n - 1 && p >= sm.end[s]) set = sm.set[s + 1];
    return set;
}

// tanh-approximated GELU, 0.5 u (1 + tanh(k (u + 0.044715 u^3))) with
// k = sqrt(2/pi), evaluated as u * sigmoid(2 k (u + 0.044715 u^3)) (the same
// function: 0.5 (1 + tanh(x)) = 1 / (1 + exp(-2x))) with the hardware exp and
// reciprocal (a few ulp in fp32, far below the bf16 rounding that follows).
__device__ __forceinline__ float gelu_tanh_fast(float u) {
    const float z = 1.5957691216057308f * u * fmaf(0.044715f * u, u, 1.0f);
    const float e = __expf(-z);
    return u * __builtin_amdgcn_rcpf(1.0f + e);
}

// Symmetric int8 code of v for scale s (s == 0 -> 0); IEEE fp32 division,
// ties to even.
__device__ __forceinline__ int8_t quant_code(float v, float s) {
    if (s == 0.0f) return 0;
    float r = rintf(__fdiv_rn(v, s));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int8_t)(int)r;
}

}  // namespace dit
