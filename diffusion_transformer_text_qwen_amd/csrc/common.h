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

// Whole-wave reductions through DPP (no LDS): pairs and quads by quad_perm,
// rows of 16 by row rotations, then the four row results via readlane.  All
// 64 lanes must be active; every lane gets the same (wave-uniform) result.
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_allsum(float v) {
    v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_f<0x124>(v);   // row_ror:4
    v += dpp_f<0x128>(v);   // row_ror:8
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_allmax(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x128>(v));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
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
// k = sqrt(2/pi), evaluated as u / (1 + exp(-2k (u + 0.044715 u^3))) (the
// same function: 0.5 (1 + tanh(x)) = 1 / (1 + exp(-2x))), with the constants
// folded into one base-2 exponent and the hardware exp2 and reciprocal (a few
// ulp in fp32, far below the bf16 rounding that follows).  Large |u| saturate
// correctly: exp2 -> inf gives 0, exp2 -> 0 gives u.
__device__ __forceinline__ float gelu_tanh_fast(float u) {
    constexpr float A = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
    constexpr float B = A * 0.044715f;
    const float e = __builtin_amdgcn_exp2f(u * fmaf(B, u * u, A));
    return u * __builtin_amdgcn_rcpf(1.0f + e);
}

// Attention work order over one flat grid of nqb query blocks x H heads.
// Heads go in groups of hg, one group after the other; inside a group the head
// varies fastest and the query blocks with the longest key ranges come first.
// Workgroups are dealt round-robin to the 8 XCDs, so with hg a multiple of 8
// every query block of a head runs on the same XCD (its K/V stay in one L2).
// The host picks hg = H when the K/V of all heads fit well inside the
// memory-side cache, else 8, so that only about one group's K/V are live.
__device__ __forceinline__ void attn_block_order(unsigned b, int nqb, int H, int hg, int& qb, int& h) {
    const unsigned gsz = (unsigned)(hg * nqb);
    const int g = (int)(b / gsz), r = (int)(b % gsz);
    const int h0 = g * hg, cnt = H - h0 < hg ? H - h0 : hg;
    h = h0 + r % cnt;
    qb = nqb - 1 - r / cnt;
}
// Heads per group for K/V operands of kv_bytes in total.
inline int attn_head_group(int64_t kv_bytes, int H) {
    return kv_bytes <= ((int64_t)128 << 20) ? H : (H < 8 ? H : 8);
}

// Symmetric int8 code of v for scale s (s == 0 -> 0); IEEE fp32 division,
// ties to even.
__device__ __forceinline__ int8_t quant_code(float v, float s) {
    if (s == 0.0f) return 0;
    float r = rintf(__fdiv_rn(v, s));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int8_t)(int)r;
}

// Hides a value from the optimizer (no instruction): later unpacking of a
// packed row re-derives floats from it instead of keeping every float alive.
__device__ __forceinline__ void opaque(v4i& v) { asm volatile("" : "+v"(v)); }

// bf16 pair <-> two floats (low half first).
__device__ __forceinline__ float bf_lo(int w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(int w) { return __builtin_bit_cast(float, w & (int)0xFFFF0000); }
__device__ __forceinline__ int bf_pack(float lo, float hi) {
    v2bf p;
    p[0] = to_bf16(lo);
    p[1] = to_bf16(hi);
    return __builtin_bit_cast(int, p);
}

// Int8 codes of 8 values for scale s = fl(amax / 127) of a set containing
// them, identical to quant_code.  With inv = fl(1/s) and s normal,
// t = fl(v * inv) lies within 2.3e-5 of fl(v / s) and |t| < 127.00003, so
// both round to the same integer (no clamp needed) unless t is within that
// distance of a half-integer.  Rounding is t + 1.5*2^23, whose fp32 add rounds
// to nearest even and leaves the integer's two's-complement low byte in the
// low byte of the sum.  Chunks with any t closer than 1e-4 to a half-integer
// take the IEEE division (a wave-uniform branch, rare); fast == false (s tiny
// or zero) always divides.
__device__ __forceinline__ uint2 quant8(const float (&v)[8], float s, float inv, bool fast) {
    constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
    int b[8];
    float dev = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float t = v[e] * inv;
        const float m = t + kMagic;
        dev = fmaxf(dev, fabsf(t - (m - kMagic)));
        b[e] = __builtin_bit_cast(int, m);
    }
    if (__builtin_expect(__any(!fast || !(dev < 0.4999f)), 0)) {
        if (!fast || !(dev < 0.4999f)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = quant_code(v[e], s);
        }
    }
    // low bytes: [b0 b1 b2 b3], [b4 b5 b6 b7]
    const uint32_t p01 = __builtin_amdgcn_perm((uint32_t)b[1], (uint32_t)b[0], 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm((uint32_t)b[3], (uint32_t)b[2], 0x0c0c0400u);
    const uint32_t p45 = __builtin_amdgcn_perm((uint32_t)b[5], (uint32_t)b[4], 0x0c0c0400u);
    const uint32_t p67 = __builtin_amdgcn_perm((uint32_t)b[7], (uint32_t)b[6], 0x0c0c0400u);
    uint2 o;
    o.x = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
    o.y = __builtin_amdgcn_perm(p67, p45, 0x05040100u);
    return o;
}

// Asymmetric int8 code of x for scale s and zero point z:
// clamp(rint(x / s) + z, -128, 127) with an IEEE division, 0 when s == 0.
__device__ __forceinline__ int asym_code(float x, float s, int z) {
    if (s == 0.0f) return 0;
    const int r = (int)rintf(__fdiv_rn(x, s)) + z;
    return min(max(r, -128), 127);
}

// asym_code of 8 values of a row whose range [lo, hi] (containing 0) gave
// s = fl((hi - lo) / 255): |x / s| <= 255.01, so t = fl(x * inv) (inv = fl(1/s))
// lies within 5e-5 of fl(x / s) and rounds to the same integer unless it is
// that close to a half-integer; chunks with any t within 1e-4 of one, and
// fast == false (s tiny or zero), take the IEEE division.
__device__ __forceinline__ uint2 quant8_asym(const float (&v)[8], float s, float inv, int z, bool fast) {
    constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
    int b[8];
    float dev = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float t = v[e] * inv;
        const float m = t + kMagic;
        dev = fmaxf(dev, fabsf(t - (m - kMagic)));
        b[e] = min(max(__builtin_bit_cast(int, m) - 0x4B400000 + z, -128), 127);
    }
    if (__builtin_expect(__any(!fast || !(dev < 0.4999f)), 0)) {
        if (!fast || !(dev < 0.4999f)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = asym_code(v[e], s, z);
        }
    }
    const uint32_t p01 = __builtin_amdgcn_perm((uint32_t)b[1], (uint32_t)b[0], 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm((uint32_t)b[3], (uint32_t)b[2], 0x0c0c0400u);
    const uint32_t p45 = __builtin_amdgcn_perm((uint32_t)b[5], (uint32_t)b[4], 0x0c0c0400u);
    const uint32_t p67 = __builtin_amdgcn_perm((uint32_t)b[7], (uint32_t)b[6], 0x0c0c0400u);
    uint2 o;
    o.x = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
    o.y = __builtin_amdgcn_perm(p67, p45, 0x05040100u);
    return o;
}

// Raw buffer resource over `bytes` bytes at p: loads past the end read zero,
// stores past the end are dropped (bounds handled without branches).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
    return (v4i)__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(uint2 v, __amdgpu_buffer_rsrc_t r, int off) {
    typedef unsigned int v2u __attribute__((ext_vector_type(2)));
    v2u d;
    d[0] = v.x;
    d[1] = v.y;
    __builtin_amdgcn_raw_buffer_store_b64(d, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16(v4i v, __amdgpu_buffer_rsrc_t r, int off) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128((v4u)v, r, off, 0, 0);
}

}  // namespace dit
