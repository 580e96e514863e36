// GEMMs of the block: y = A W^T with A [M, K] and W [N, K], both K-contiguous.
//  - int8 x int8 -> int32 on v_mfma_i32_16x16x64_i8 (W8A8 linears)
//  - bf16 x bf16 -> fp32 on v_mfma_f32_16x16x32_bf16 (bf16 linears)
//  - fp32 FMA tiles (fp32 mode)
// The two MFMA kernels share one byte-level tiling: a 16-byte operand slice per
// lane covers 16 int8 or 8 bf16 values of one row, so a 128-byte K step is two
// MFMA K steps for either type.
#include "common.h"
#include "kernels.h"

namespace dit {

__device__ __forceinline__ float gelu_tanh(float u) {
    const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * u * (1.0f + tanhf(k0 * (u + 0.044715f * u * u * u)));
}

// Apply the epilogue to one output element; v already holds acc*scales (+bias added here).
__device__ __forceinline__ void epilogue(const EpiParams& ep, int64_t m, int64_t n, float v,
                                         int32_t acc_i) {
    if (ep.bias) v += ep.bias[n];
    const bool rb = ep.act_bf16 != 0;
    if (ep.kind == EPI_STORE) {
        if (ep.y_bf16)
            reinterpret_cast<__bf16*>(ep.y)[m * ep.ldy + n] = to_bf16(v);
        else
            reinterpret_cast<float*>(ep.y)[m * ep.ldy + n] = v;
        if (ep.acc_out) ep.acc_out[m * ep.ldacc + n] = acc_i;
    } else if (ep.kind == EPI_GELU) {
        const float u = rb ? bf16r(v) : v;
        const float g = gelu_tanh(u);
        if (ep.y_bf16)
            reinterpret_cast<__bf16*>(ep.y)[m * ep.ldy + n] = to_bf16(g);
        else
            reinterpret_cast<float*>(ep.y)[m * ep.ldy + n] = g;
    } else {
        const int set = seg_set(ep.sm, m);
        const float gate = ep.gate[(int64_t)set * ep.gate_stride + n];
        if (rb) {
            __bf16* xp = reinterpret_cast<__bf16*>(ep.x) + m * ep.ldx + n;
            const float y = bf16r(v);
            *xp = to_bf16((float)*xp + gate * y);
        } else {
            float* xp = reinterpret_cast<float*>(ep.x) + m * ep.ldx + n;
            *xp = *xp + gate * v;
        }
    }
}

// ---------------------------------------------------------------- MFMA GEMM
constexpr int BM = 128, BN = 128, BKB = 128;   // tile rows, cols, K bytes
constexpr int LDS_STRIDE = BKB + 16;           // padded row (bytes): conflict-free 16-byte reads
constexpr int NTHREADS = 256;

template <bool I8>
__global__ void __launch_bounds__(NTHREADS, 2)
gemm_mfma_kernel(const uint8_t* __restrict__ A, int64_t lda_b, const uint8_t* __restrict__ W,
                 int64_t M, int64_t N, int64_t Kb, EpiParams ep) {
    __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * LDS_STRIDE];

    // Tile order: groups of 8 M-tiles sweep N so that neighbouring workgroups
    // share A rows and W rows in L2.
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const int bid = blockIdx.x;
    constexpr int GROUP = 8;
    const int per_group = GROUP * tiles_n;
    const int g = bid / per_group;
    const int first_m = g * GROUP;
    const int gsize = min(tiles_m - first_m, GROUP);
    const int tm = first_m + (bid % per_group) % gsize;
    const int tn = (bid % per_group) / gsize;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / 2, wn = wave % 2;

    // global -> register staging: 4 chunks of 16 bytes per operand per thread
    uint4 ra[4], rb[4];
    auto gload = [&](int64_t kb0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + i * NTHREADS;
            const int r = c / (BKB / 16), col = (c % (BKB / 16)) * 16;
            const int64_t gm = m0 + r, gn = n0 + r;
            ra[i] = gm < M ? *reinterpret_cast<const uint4*>(A + gm * lda_b + kb0 + col)
                           : make_uint4(0, 0, 0, 0);
            rb[i] = gn < N ? *reinterpret_cast<const uint4*>(W + gn * Kb + kb0 + col)
                           : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + i * NTHREADS;
            const int r = c / (BKB / 16), col = (c % (BKB / 16)) * 16;
            *reinterpret_cast<uint4*>(&As[buf][r * LDS_STRIDE + col]) = ra[i];
            *reinterpret_cast<uint4*>(&Bs[buf][r * LDS_STRIDE + col]) = rb[i];
        }
    };

    typedef typename std::conditional<I8, v4i, v4f>::type acc_t;
    acc_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

    const int nk = (int)(Kb / BKB);
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((int64_t)(kt + 1) * BKB);
#pragma unroll
        for (int ks = 0; ks < BKB / 64; ++ks) {
            uint4 af[4], bf[4];
            const int koff = ks * 64 + (lane / 16) * 16;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const uint4*>(
                    &As[buf][(wm * 64 + i * 16 + lane % 16) * LDS_STRIDE + koff]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const uint4*>(
                    &Bs[buf][(wn * 64 + j * 16 + lane % 16) * LDS_STRIDE + koff]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (I8) {
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                            *reinterpret_cast<v4i*>(&af[i]), *reinterpret_cast<v4i*>(&bf[j]),
                            acc[i][j], 0, 0, 0);
                    } else {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            *reinterpret_cast<v8bf*>(&af[i]), *reinterpret_cast<v8bf*>(&bf[j]),
                            acc[i][j], 0, 0, 0);
                    }
                }
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds rows (lane/16)*4 + r, column lane%16 of each 16x16 tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 64 + i * 16 + (lane / 16) * 4 + r;
                const int64_t n = n0 + wn * 64 + j * 16 + lane % 16;
                if (m < M && n < N) {
                    if constexpr (I8) {
                        const int32_t a = acc[i][j][r];
                        const float v = (float)a * ep.a_scale[m] * ep.w_scale[n];
                        epilogue(ep, m, n, v, a);
                    } else {
                        epilogue(ep, m, n, acc[i][j][r], 0);
                    }
                }
            }
}

static unsigned gemm_grid(int64_t M, int64_t N) {
    return (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
}

hipError_t launch_gemm_i8(const int8_t* a, const int8_t* w, int64_t M, int64_t N, int64_t K,
                          const EpiParams& ep, hipStream_t st) {
    if (M == 0) return hipSuccess;
    gemm_mfma_kernel<true><<<gemm_grid(M, N), NTHREADS, 0, st>>>(
        (const uint8_t*)a, K, (const uint8_t*)w, M, N, K, ep);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const void* a, int64_t lda, const void* w, int64_t M, int64_t N,
                            int64_t K, const EpiParams& ep, hipStream_t st) {
    if (M == 0) return hipSuccess;
    gemm_mfma_kernel<false><<<gemm_grid(M, N), NTHREADS, 0, st>>>(
        (const uint8_t*)a, lda * 2, (const uint8_t*)w, M, N, K * 2, ep);
    return hipGetLastError();
}

// ---------------------------------------------------------------- fp32 GEMM
// 64x64 tile, 256 threads, 4x4 outputs per thread, K step 16, plain FMA.
__global__ void __launch_bounds__(256) gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ W, int64_t M,
                                                       int64_t N, int64_t K, EpiParams ep) {
    __shared__ float As[16][64 + 4];
    __shared__ float Bs[16][64 + 4];
    const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    const int tid = threadIdx.x;
    const int tm = tid / 16, tn = tid % 16;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += 16) {
        // each thread loads 4 elements of A and 4 of W (64 rows x 16 k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * 256;
            const int r = e / 16, kk = e % 16;
            As[kk][r] = (m0 + r < M) ? A[(m0 + r) * lda + k0 + kk] : 0.0f;
            Bs[kk][r] = (n0 + r < N) ? W[(n0 + r) * K + k0 + kk] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][tm * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tn * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t m = m0 + tm * 4 + i, n = n0 + tn * 4 + j;
            if (m < M && n < N) epilogue(ep, m, n, acc[i][j], 0);
        }
}

hipError_t launch_gemm_f32(const float* a, int64_t lda, const float* w, int64_t M, int64_t N,
                           int64_t K, const EpiParams& ep, hipStream_t st) {
    if (M == 0) return hipSuccess;
    dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    gemm_f32_kernel<<<grid, 256, 0, st>>>(a, lda, w, M, N, K, ep);
    return hipGetLastError();
}

}  // namespace dit
