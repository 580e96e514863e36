// Weight and activation formats of the gated block's linears: the W8A8 recipe
// of "Qwen-Image-2.1 W8A8 - FlagOS for Mac" (Quantization and validation:
// dynamic asymmetric per-token int8 activations, and the int8 weight column
// sums their zero points need) and MXFP4 weights (expanded to bf16 below).
//
// Asymmetric codes: the row's range widened to contain 0, lo = min(row, 0),
// hi = max(row, 0); s = fp32(hi - lo) / 255; zero point z = -128 - rint(lo / s)
// in [-128, 127]; q = clamp(rint(x / s) + z, -128, 127); IEEE fp32 divisions,
// ties to even; an all-zero row gives s = 0, z = 0, q = 0.  A GEMM over such
// codes subtracts z[m] * sum_k w[n, k] from its int32 sum.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
    if constexpr (std::is_same<T, __bf16>::value) {
        const v8bf x = *reinterpret_cast<const v8bf*>(p);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
    } else {
        const v4f a = *reinterpret_cast<const v4f*>(p), b = *reinterpret_cast<const v4f*>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = a[e];
            v[4 + e] = b[e];
        }
    }
}

// One workgroup per row; 8 consecutive values per thread and pass (K % 8 == 0).
template <typename T>
__global__ void __launch_bounds__(256) quant_asym_kernel(const T* __restrict__ x, int64_t ldx, int64_t K,
                                                         int8_t* __restrict__ q, float* __restrict__ scale,
                                                         int32_t* __restrict__ zero) {
    __shared__ float red[2][4];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const T* xr = x + row * ldx;
    float lo = 0.0f, hi = 0.0f;
    for (int64_t k = (int64_t)tid * 8; k < K; k += 256 * 8) {
        float v[8];
        load8(xr + k, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo = fminf(lo, v[e]);
            hi = fmaxf(hi, v[e]);
        }
    }
    hi = wave_allmax(hi);
    lo = -wave_allmax(-lo);
    if (lane == 0) {
        red[0][wave] = lo;
        red[1][wave] = hi;
    }
    __syncthreads();
    lo = fminf(fminf(red[0][0], red[0][1]), fminf(red[0][2], red[0][3]));
    hi = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    const float s = __fdiv_rn(hi - lo, 255.0f);
    const int z = s == 0.0f ? 0 : min(max(-128 - (int)rintf(__fdiv_rn(lo, s)), -128), 127);
    int8_t* qr = q + row * K;
    const float inv = __fdiv_rn(1.0f, s);
    const bool fast = s >= 0x1p-100f;
    for (int64_t k = (int64_t)tid * 8; k < K; k += 256 * 8) {
        float v[8];
        load8(xr + k, v);
        *reinterpret_cast<uint2*>(qr + k) = quant8_asym(v, s, inv, z, fast);
    }
    if (tid == 0) {
        scale[row] = s;
        zero[row] = z;
    }
}

// One wave per weight row: out[n] = sum_k w[n, k] (K % 16 == 0).
__global__ void __launch_bounds__(256) int8_colsum_kernel(const int8_t* __restrict__ w, int64_t N, int64_t K,
                                                          int32_t* __restrict__ out) {
    const int64_t n = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (n >= N) return;
    const int8_t* wr = w + n * K;
    int acc = 0;
    for (int64_t k = (int64_t)lane * 16; k < K; k += kWave * 16) {
        const v4i c = *reinterpret_cast<const v4i*>(wr + k);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int x = c[e];
            acc += (int)(int8_t)(x & 0xFF) + (int)(int8_t)((x >> 8) & 0xFF) + (int)(int8_t)((x >> 16) & 0xFF) +
                   (int)(int8_t)((x >> 24) & 0xFF);
        }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) acc += __shfl_xor(acc, m, kWave);
    if (lane == 0) out[n] = acc;
}

// MXFP4 ("Qwen_Image-2.1-MXFP4-Paiton", What was quantized): E2M1 codes packed
// low nibble first, one E8M0 scale per 32 input columns.  One thread per group:
// 16 code bytes and a scale byte -> 32 bf16 through the hardware fp4 -> bf16
// conversion with an fp32 scale (an E2M1 value times a power of two is exact in
// bf16 within its exponent range).
__global__ void __launch_bounds__(256) mxfp4_expand_kernel(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales, int64_t groups,
                                                           __bf16* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= groups) return;
    const v4i c = *reinterpret_cast<const v4i*>(codes + g * 16);
    const int e = scales[g];
    const float sc = e == 255 ? __builtin_nanf("") : ldexpf(1.0f, e - 127);
    v4i o[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // byte b of the word holds elements 2b (low nibble) and 2b + 1
        const uint32_t word = (uint32_t)c[w];
        o[w][0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0));
        o[w][1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1));
        o[w][2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2));
        o[w][3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3));
    }
    v4i* dst = reinterpret_cast<v4i*>(out + g * 32);
#pragma unroll
    for (int w = 0; w < 4; ++w) dst[w] = o[w];
}

}  // namespace

hipError_t launch_mxfp4_expand(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, void* out,
                               hipStream_t st) {
    const int64_t groups = N * (K / 32);
    if (groups == 0) return hipSuccess;
    mxfp4_expand_kernel<<<(unsigned)((groups + 255) / 256), 256, 0, st>>>(codes, scales, groups, (__bf16*)out);
    return hipGetLastError();
}

hipError_t launch_quantize_rows_asym(const void* x, bool bf16, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                     float* scale, int32_t* zero, hipStream_t st) {
    if (M == 0) return hipSuccess;
    if (bf16)
        quant_asym_kernel<__bf16><<<(unsigned)M, 256, 0, st>>>((const __bf16*)x, ldx, K, q, scale, zero);
    else
        quant_asym_kernel<float><<<(unsigned)M, 256, 0, st>>>((const float*)x, ldx, K, q, scale, zero);
    return hipGetLastError();
}

hipError_t launch_int8_colsum(const int8_t* w, int64_t N, int64_t K, int32_t* out, hipStream_t st) {
    if (N == 0) return hipSuccess;
    int8_colsum_kernel<<<(unsigned)((N + 3) / 4), 256, 0, st>>>(w, N, K, out);
    return hipGetLastError();
}

}  // namespace dit
