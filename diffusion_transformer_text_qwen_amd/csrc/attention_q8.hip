// Block-causal attention on int8 / fp8 operands ("Qwen_Image-2.1-MXFP4-Paiton",
// Runtime precision and quality: after the first denoising steps attention
// runs in int8/fp8).  Scores S^T = K Q^T on v_mfma_i32_32x32x32_i8, P V on the
// fp8 (e4m3) v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales: twice the bf16
// MFMA rate, and half the bytes per K/V tile.
//
// Quantization (a pass before the attention, over q and the K/V cache):
//   q: symmetric int8 per (token, head), scale amax/127;
//   k: symmetric int8 per (64-key tile, head), scale amax/127, so the tile's
//      scale is one number that folds into the softmax exponent;
//   v: e4m3 per (head, channel) over all keys, scale amax/448, applied to the
//      output;
//   P = 2^(score - running max) in (0, 2^8] (the lazy rescale bound) rounded to
//      e4m3 unscaled; the row sum adds the unrounded values.
// Codes use an IEEE fp32 division and round to nearest even.
//
// The pass writes K and V as LDS-ready tile images, so the attention kernel
// copies them into LDS with buffer loads that carry the lds bit:
//   K tile (8 KB): key r (row of 128 bytes), 16-byte chunk c (dims 16c..16c+15)
//     at chunk c ^ (r & 7): the eight key rows one ds_read_b128 phase reads hit
//     eight different bank groups;
//   V tile (8 KB): channel row ch of 64 bytes, position p = 32h + b holding the
//     key (b / 16) * 32 + (b % 4) + 8 ((b % 16) / 4) + 4h, the order in which the
//     S^T accumulator of lane half h hands P to the fp8 MFMA's B operand; 16-byte
//     chunk c of row ch at chunk c ^ ((ch >> 1) & 3).
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int QK_TILE = 64;        // keys per tile (the K scale granularity)
constexpr int TILE_IMG = 8192;     // bytes of one K or V tile image of one head
constexpr int Q8_QB = 128;         // queries per workgroup
constexpr int Q8_SLOTS = 4;        // LDS ring of (K, V) tile pairs
constexpr int Q8_SLOT = 2 * TILE_IMG;
constexpr float kFp8Max = 448.0f;
// Lazy rescale of the online softmax: P of a tile is formed against the
// running max as it stands, and the max is only raised (the tile's P formed
// again) when a lane's sum of P over the tile exceeds kRescaleMaxQ8, so every
// P that is rounded to e4m3 is at most 2^8 < 448 (no saturation).
constexpr float kRescaleMaxQ8 = 256.0f;

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

// key (within its tile) at V-image position p
__device__ __forceinline__ int vkey_of_pos(int p) {
    const int h = p / 32, b = p % 32;
    return (b / 16) * 32 + (b % 4) + 8 * ((b % 16) / 4) + 4 * h;
}

// e4m3 code of v / s (s == 0 -> 0): IEEE division, saturate to +-448, round to nearest even
__device__ __forceinline__ float fp8_arg(float v, float s) {
    if (s == 0.0f) return 0.0f;
    return fminf(fmaxf(__fdiv_rn(v, s), -kFp8Max), kFp8Max);
}
// The same argument through the reciprocal product t = v * inv (inv =
// fl(1 / s)): t lies within 3 ulps of fl(v / s), so both round to the same
// e4m3 value unless t is within a few ulps of an e4m3 rounding midpoint
// (normal range: the 20 fp32 mantissa bits below e4m3's 3 at 0x80000;
// subnormal range |t| < 2^-6: an odd multiple of 2^-10); those take the division.
__device__ __forceinline__ float fp8_arg_fast(float v, float s, float inv) {
    if (s == 0.0f) return 0.0f;
    const float t = v * inv;
    const float at = fabsf(t);
    bool near;
    if (at >= 0x1p-6f) {
        const int low = (int)(__builtin_bit_cast(uint32_t, at) & 0xFFFFFu);
        near = abs(low - 0x80000) <= 8;
    } else {
        const float u = at * 512.0f;
        near = fabsf(u - floorf(u) - 0.5f) < 0x1p-12f;
    }
    if (near) return fp8_arg(v, s);
    return fminf(fmaxf(t, -kFp8Max), kFp8Max);
}
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__global__ void __launch_bounds__(256) fill_u32_kernel(uint32_t* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// q: 16 lanes per (token, head) row, 8 values each.  The first nfill threads
// also clear the V channel amax words that the K kernel raises next.
__global__ void __launch_bounds__(256) attn_quant_q_kernel(const __bf16* __restrict__ q, int64_t ldq, int T_q,
                                                           int H, int8_t* __restrict__ q8,
                                                           float* __restrict__ sq, uint32_t* __restrict__ vamax,
                                                           int nfill) {
    {
        const int gi = blockIdx.x * 256 + threadIdx.x;
        if (gi < nfill) vamax[gi] = 0u;
    }
    const int64_t g = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
    const int sub = threadIdx.x % 16;
    const bool ok = g < (int64_t)T_q * H;
    const int64_t t = ok ? g / H : 0;
    const int h = ok ? (int)(g % H) : 0;
    float v[8] = {};
    if (ok) {
        const v8bf x = *reinterpret_cast<const v8bf*>(q + t * ldq + h * 128 + sub * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
    }
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[e]));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) a = fmaxf(a, __shfl_xor(a, m, kWave));
    const float s = __fdiv_rn(a, 127.0f);
    // codes of v / s (IEEE division, ties to even) through the reciprocal
    // product with a near-tie fallback, as for the per-token activations
    const uint2 o = quant8(v, s, __fdiv_rn(1.0f, s), s >= 0x1p-100f);
    if (!ok) return;
    *reinterpret_cast<uint2*>(q8 + ((int64_t)h * T_q + t) * 128 + sub * 8) = o;
    if (sub == 0) sq[(int64_t)h * T_q + t] = s;
}

// One (64-key tile, head) per workgroup: the K tile image and scale, and the
// per-channel amax of the V tile (atomicMax on the bits of non-negative floats).
__global__ void __launch_bounds__(256) attn_quant_k_kernel(const __bf16* __restrict__ k, int64_t ldk,
                                                           const __bf16* __restrict__ v, int64_t ldv, int T_k,
                                                           int nt, int8_t* __restrict__ k8,
                                                           float* __restrict__ sk, uint32_t* __restrict__ vamax) {
    __shared__ float red[4];
    __shared__ float vred[4][128];
    const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    // K: key r = tid / 4, dims (tid % 4) * 32 .. +32 (logical chunks 2 (tid % 4), +1)
    const int r = tid / 4, part = tid % 4;
    const int64_t key = (int64_t)t * QK_TILE + r;
    float kv[32] = {};
    if (key < T_k) {
        const __bf16* src = k + key * ldk + h * 128 + part * 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const v8bf x = *reinterpret_cast<const v8bf*>(src + c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) kv[c * 8 + e] = (float)x[e];
        }
    }
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) a = fmaxf(a, fabsf(kv[e]));
    a = wave_allmax(a);
    if (lane == 0) red[wave] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = __fdiv_rn(a, 127.0f);
    const float inv = __fdiv_rn(1.0f, s);
    const bool fast = s >= 0x1p-100f;
    int8_t* img = k8 + ((int64_t)h * nt + t) * TILE_IMG;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int c = part * 2 + half;
        float lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo[e] = kv[half * 16 + e];
            hi[e] = kv[half * 16 + 8 + e];
        }
        const uint2 a8 = quant8(lo, s, inv, fast), b8 = quant8(hi, s, inv, fast);
        const v4i o = {(int)a8.x, (int)a8.y, (int)b8.x, (int)b8.y};
        *reinterpret_cast<v4i*>(img + r * 128 + ((c ^ (r & 7)) << 4)) = o;
    }
    if (tid == 0) sk[(int64_t)h * nt + t] = s;
    // V channel amax: channels (tid % 16) * 8 .. +8, keys tid / 16 + 16 i
    const int cc = tid % 16, kr = tid / 16;
    float m[8] = {};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t kk = (int64_t)t * QK_TILE + kr + 16 * i;
        if (kk < T_k) {
            const v8bf x = *reinterpret_cast<const v8bf*>(v + kk * ldv + h * 128 + cc * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf((float)x[e]));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        m[e] = fmaxf(m[e], __shfl_xor(m[e], 16, kWave));
        m[e] = fmaxf(m[e], __shfl_xor(m[e], 32, kWave));
    }
    if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vred[wave][lane * 8 + e] = m[e];
    }
    __syncthreads();
    if (tid < 128) {
        const float mv = fmaxf(fmaxf(vred[0][tid], vred[1][tid]), fmaxf(vred[2][tid], vred[3][tid]));
        atomicMax(vamax + h * 128 + tid, __builtin_bit_cast(uint32_t, mv));
    }
}

// One (64-key tile, head) per workgroup: the V tile image; tile 0 also writes
// the channel scales.  The bf16 tile is staged in LDS so that each thread can
// read its channel of 32 keys.
__global__ void __launch_bounds__(256) attn_quant_v_kernel(const __bf16* __restrict__ v, int64_t ldv, int T_k,
                                                           int nt, const uint32_t* __restrict__ vamax,
                                                           uint8_t* __restrict__ v8, float* __restrict__ sv) {
    __shared__ __bf16 tile[QK_TILE][128 + 8];
    const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i;          // 1024 chunks of 8 values
        const int kr = idx / 16, cc = idx % 16;
        const int64_t kk = (int64_t)t * QK_TILE + kr;
        v8bf x = {};
        if (kk < T_k) x = *reinterpret_cast<const v8bf*>(v + kk * ldv + h * 128 + cc * 8);
        *reinterpret_cast<v8bf*>(&tile[kr][cc * 8]) = x;
    }
    __syncthreads();
    const int ch = tid / 2, ph = tid % 2;
    const float s = __fdiv_rn(__builtin_bit_cast(float, vamax[h * 128 + ch]), kFp8Max);
    const float inv = __fdiv_rn(1.0f, s);
    float r[32];
#pragma unroll
    for (int b = 0; b < 32; ++b) r[b] = fp8_arg_fast((float)tile[vkey_of_pos(ph * 32 + b)][ch], s, inv);
    uint8_t* row = v8 + ((int64_t)h * nt + t) * TILE_IMG + ch * 64;
    const int sw = (ch >> 1) & 3;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int c = ph * 2 + half;
        v4i o;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float* x = r + half * 16 + w * 4;
            o[w] = (int)fp8x4(x[0], x[1], x[2], x[3]);
        }
        *reinterpret_cast<v4i*>(row + ((c ^ sw) << 4)) = o;
    }
    if (t == 0 && ph == 0) sv[h * 128 + ch] = s;
}

// Attention: 128 queries of one head per workgroup, 4 waves x 32 queries; S^T
// and O^T per wave as in the bf16 kernel.  K/V tile images go straight into a
// 4-slot LDS ring, tile t+3 loaded while tile t is processed; one barrier per
// tile.  Lane l owns query l % 32 of its wave; its 32 scores of a tile are the
// keys of the two 32-key halves handed out by the 32x32 accumulator layout.
template <bool QBF16>
__global__ void __launch_bounds__(256, 2)
attn_q8_kernel(const int8_t* __restrict__ Q8, const float* __restrict__ SQ, const uint8_t* __restrict__ K8,
               const float* __restrict__ SK, const uint8_t* __restrict__ V8, const float* __restrict__ SV,
               __bf16* __restrict__ O, int T_q, int T_k, int nt, int ldo, AttnSegs sg, float c_log2,
               const __bf16* __restrict__ QB, int64_t ldqb, int H, int hg) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[Q8_SLOTS * Q8_SLOT];
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    typedef int v8i __attribute__((ext_vector_type(8)));

    const int nqb = (T_q + Q8_QB - 1) / Q8_QB;
    int qb, h;
    attn_block_order(blockIdx.x, nqb, H, hg, qb, h);
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int hh = lane / 32, lq = lane % 32;
    const int off = T_k - T_q;
    const int q_first = qb * Q8_QB;
    const int q_last = min(q_first + Q8_QB, T_q) - 1;
    const int kv_min = (int)kv_end_of(sg, off + q_first);
    const int kv_hi = (int)kv_end_of(sg, off + q_last);
    const int qi = q_first + wave * 32 + lq;
    const bool q_ok = qi < T_q;
    const int my_end = q_ok ? (int)kv_end_of(sg, off + qi) : T_k;

    // Q^T fragments (B operand): dims kb*32 + hh*16 .. +16 of this lane's query
    v4i qf[4];
    float cq;
    if constexpr (QBF16) {
        // the query row's int8 codes formed here from bf16 Q, exactly as
        // attn_quant_q_kernel forms them: amax over the row's 128 dims (this
        // lane's 64 and lane l^32's), s = amax / 127, codes of v / s
        float v[4][16];
        float a = 0.0f;
        {
            const __bf16* qrow = QB + (int64_t)(q_ok ? qi : 0) * ldqb + h * 128 + hh * 16;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const v8bf x0 = q_ok ? *reinterpret_cast<const v8bf*>(qrow + kb * 32) : v8bf{};
                const v8bf x1 = q_ok ? *reinterpret_cast<const v8bf*>(qrow + kb * 32 + 8) : v8bf{};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[kb][e] = (float)x0[e];
                    v[kb][8 + e] = (float)x1[e];
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) a = fmaxf(a, fabsf(v[kb][e]));
            }
        }
        a = fmaxf(a, __shfl_xor(a, 32, kWave));
        const float s = __fdiv_rn(a, 127.0f);
        const float inv = __fdiv_rn(1.0f, s);
        const bool fast = s >= 0x1p-100f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            float lo[8], hi[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                lo[e] = v[kb][e];
                hi[e] = v[kb][8 + e];
            }
            const uint2 c0 = quant8(lo, s, inv, fast), c1 = quant8(hi, s, inv, fast);
            qf[kb] = v4i{(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y};
        }
        cq = q_ok ? s * c_log2 : 0.0f;
    } else {
        const int8_t* qrow = Q8 + ((int64_t)h * T_q + (q_ok ? qi : 0)) * 128 + hh * 16;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) qf[kb] = q_ok ? *reinterpret_cast<const v4i*>(qrow + kb * 32) : v4i{};
        cq = q_ok ? SQ[(int64_t)h * T_q + qi] * c_log2 : 0.0f;
    }
    const float* skh = SK + (int64_t)h * nt;

    // tile images of this head; every load is inside [0, nt * 8 KB)
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(K8 + (int64_t)h * nt * TILE_IMG), 0, nt * TILE_IMG, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(V8 + (int64_t)h * nt * TILE_IMG), 0, nt * TILE_IMG, 0x00020000);
    const int wofs = __builtin_amdgcn_readfirstlane(wave * 2 * 1024);
    // loads of tile t into slot t % 4 (t clamped to the last tile: unused data): K first, then V
    auto dma = [&](int t) {
        const int td = min(t, nt - 1);
        uint8_t* s = lds + (t % Q8_SLOTS) * Q8_SLOT + wofs;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(s + i * 1024), 16, wofs + i * 1024 + lane * 16,
                                                     td * TILE_IMG, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(s + TILE_IMG + i * 1024), 16,
                                                     wofs + i * 1024 + lane * 16, td * TILE_IMG, 0, 0);
    };
    // K fragment (A operand): key kh*32 + lq, dims kb*32 + hh*16 .. +16
    int koff[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) koff[kb] = lq * 128 + (((2 * kb + hh) ^ (lq & 7)) << 4);
    // V^T fragment (A operand): channel dt*32 + lq, positions 32 hh .. +32
    const int vsw = (lq >> 1) & 3;
    const int voff0 = TILE_IMG + lq * 64 + (((2 * hh) ^ vsw) << 4);
    const int voff1 = TILE_IMG + lq * 64 + (((2 * hh + 1) ^ vsw) << 4);

    v16f oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = v16f{};
    float m_run = -INFINITY, l_run = 0.0f;

    auto scores = [&](const uint8_t* ks, v16i(&sacc)[2]) {
        sacc[0] = v16i{};
        sacc[1] = v16i{};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const v4i a = *reinterpret_cast<const v4i*>(ks + kh * 32 * 128 + koff[kb]);
                sacc[kh] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[kb], sacc[kh], 0, 0, 0);
            }
    };

    // Step t: softmax of tile t (scores in scur) with the scores of tile t+1
    // (into snxt) between its exponentials; P V of tile t with the loads of
    // tile t+3 between the MFMAs; then tile t+2's K and tile t+1's V must have
    // landed (this wave's later loads, 6, may stay in flight) and all waves meet.
    auto step = [&](int t, v16i(&scur)[2], v16i(&snxt)[2]) {
        const uint8_t* kn = lds + ((t + 1) % Q8_SLOTS) * Q8_SLOT;
        const uint8_t* vc = lds + (t % Q8_SLOTS) * Q8_SLOT;
        const int j0 = t * QK_TILE;
        float x[32];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int j = 0; j < 16; ++j) x[kh * 16 + j] = (float)scur[kh][j];
        if (j0 + QK_TILE > kv_min) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = j0 + kh * 32 + (j / 4) * 8 + hh * 4 + (j % 4);
                    if (key >= my_end) x[kh * 16 + j] = -INFINITY;
                }
        }
        // exponent scale of this tile (> 0, so that masked -inf stays -inf)
        const float ct = fmaxf(cq * skh[min(t, nt - 1)], 1e-30f);
        const float mb = m_run;
        snxt[0] = v16i{};
        snxt[1] = v16i{};
        v8i pk;
        float psum = 0.0f;
        v4i kf[8];
        kf[0] = *reinterpret_cast<const v4i*>(kn + koff[0]);
        kf[1] = *reinterpret_cast<const v4i*>(kn + 32 * 128 + koff[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // MFMA i: k-block i / 2, key half i % 2; fragment read two ahead
            if (i + 2 < 8) kf[i + 2] = *reinterpret_cast<const v4i*>(kn + ((i + 2) % 2) * 32 * 128 + koff[(i + 2) / 2]);
            snxt[i % 2] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[i], qf[i / 2], snxt[i % 2], 0, 0, 0);
            {
                // P of scores 4i .. 4i+3 -> one dword of the fp8 B operand
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p[e] = __builtin_amdgcn_exp2f(fmaf(x[4 * i + e], ct, -mb));
                    psum += p[e];
                }
                pk[i] = (int)fp8x4(p[0], p[1], p[2], p[3]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // P was formed against the running max.  When a lane's sum over this
        // tile exceeds kRescaleMaxQ8 (or is not finite), raise the running max
        // to the tile's max, rescale, and form P again (a wave-uniform branch,
        // taken on the first tile and on tiles whose scores climb well above
        // all earlier ones).
        if (__any(!(psum <= kRescaleMaxQ8))) {
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 32; ++e) mx = fmaxf(mx, x[e]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * ct;
            const float m_new = fmaxf(m_run, mx);
            if (m_new > m_run) {
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) oacc[dt][j] *= alpha;
                m_run = m_new;
            }
            // a row with no visible key so far keeps P = 0
            const float mb2 = m_run == -INFINITY ? 0.0f : m_run;
            psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p[e] = __builtin_amdgcn_exp2f(fmaf(x[4 * i + e], ct, -mb2));
                    psum += p[e];
                }
                pk[i] = (int)fp8x4(p[0], p[1], p[2], p[3]);
            }
        }
        l_run += psum;
        // O^T += V^T P^T: one fp8 MFMA per 32-channel block, loads of tile t+3 in between
        const int td3 = min(t + 3, nt - 1);
        uint8_t* s3 = lds + ((t + 3) % Q8_SLOTS) * Q8_SLOT + wofs;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            v8i va;
            const v4i lo = *reinterpret_cast<const v4i*>(vc + dt * 32 * 64 + voff0);
            const v4i hi = *reinterpret_cast<const v4i*>(vc + dt * 32 * 64 + voff1);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                va[w] = lo[w];
                va[4 + w] = hi[w];
            }
            oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pk, oacc[dt], 0, 0, 0, 127, 0, 127);
            if (dt < 2)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(s3 + dt * 1024), 16,
                                                         wofs + dt * 1024 + lane * 16, td3 * TILE_IMG, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(s3 + TILE_IMG + (dt - 2) * 1024), 16,
                                                         wofs + (dt - 2) * 1024 + lane * 16, td3 * TILE_IMG, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt vmcnt(6)\n\ts_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    const int ntiles = (kv_hi + QK_TILE - 1) / QK_TILE;
    // prologue: tiles 0, 1, 2 in flight; K(0), V(0), K(1) landed; scores of tile 0
    dma(0);
    dma(1);
    dma(2);
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    v16i sa[2], sb[2];
    scores(lds, sa);
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        step(t, sa, sb);
        step(t + 1, sb, sa);
    }
    if (t < ntiles) step(t, sa, sb);
    // the loads past the last tile must land before the workgroup exits
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
    if (!q_ok) return;
    const float inv = 1.0f / l_tot;
    __bf16* orow = O + (size_t)qi * ldo + h * 128;
    const float* svh = SV + h * 128;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c0 = dt * 32 + g * 8 + hh * 4;
            const v4f sc = *reinterpret_cast<const v4f*>(svh + c0);
            v4bf outv;
#pragma unroll
            for (int r = 0; r < 4; ++r) outv[r] = to_bf16(oacc[dt][g * 4 + r] * sc[r] * inv);
            *reinterpret_cast<v4bf*>(orow + c0) = outv;
        }
}

}  // namespace

AttnQ8Layout attn_q8_layout(int64_t T_q, int64_t T_k, int H) {
    AttnQ8Layout L{};
    L.nt = (T_k + QK_TILE - 1) / QK_TILE;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += up256(bytes);
        return at;
    };
    L.q8 = take((size_t)H * T_q * 128);
    L.sq = take((size_t)H * T_q * 4);
    L.k8 = take((size_t)H * L.nt * TILE_IMG);
    L.sk = take((size_t)H * L.nt * 4);
    L.v8 = take((size_t)H * L.nt * TILE_IMG);
    L.sv = take((size_t)H * 128 * 4);
    L.vamax = take((size_t)H * 128 * 4);
    L.total = off;
    return L;
}

hipError_t launch_attn_quantize(const void* q, const void* k, const void* v, int64_t T_q, int64_t T_k, int H,
                                int64_t ldq, int64_t ldk, int64_t ldv, void* buf, hipStream_t st, bool with_q) {
    const AttnQ8Layout L = attn_q8_layout(T_q, T_k, H);
    uint8_t* b = (uint8_t*)buf;
    uint32_t* vamax = (uint32_t*)(b + L.vamax);
    // the Q launch clears the V amax words when it has a thread for each
    if (!with_q) T_q = 0;
    const int64_t q_threads = (T_q * H + 15) / 16 * 256;
    const bool fold = T_q > 0 && q_threads >= (int64_t)H * 128;
    if (!fold) fill_u32_kernel<<<(unsigned)((H * 128 + 255) / 256), 256, 0, st>>>(vamax, H * 128);
    if (T_q > 0)
        attn_quant_q_kernel<<<(unsigned)((T_q * H + 15) / 16), 256, 0, st>>>(
            (const __bf16*)q, ldq, (int)T_q, H, (int8_t*)(b + L.q8), (float*)(b + L.sq), vamax,
            fold ? H * 128 : 0);
    if (L.nt > 0) {
        const dim3 grid((unsigned)L.nt, (unsigned)H);
        attn_quant_k_kernel<<<grid, 256, 0, st>>>((const __bf16*)k, ldk, (const __bf16*)v, ldv, (int)T_k,
                                                  (int)L.nt, (int8_t*)(b + L.k8), (float*)(b + L.sk), vamax);
        attn_quant_v_kernel<<<grid, 256, 0, st>>>((const __bf16*)v, ldv, (int)T_k, (int)L.nt, vamax,
                                                  (uint8_t*)(b + L.v8), (float*)(b + L.sv));
    }
    return hipGetLastError();
}

hipError_t launch_attention_q8(const void* buf, int64_t T_q, int64_t T_k, int H, void* o, int64_t ldo,
                               const AttnSegs& segs, float sm_scale, hipStream_t st, const void* q_bf16,
                               int64_t ldq) {
    if (T_q == 0) return hipSuccess;
    const AttnQ8Layout L = attn_q8_layout(T_q, T_k, H);
    const uint8_t* b = (const uint8_t*)buf;
    const float c = sm_scale * 1.4426950408889634f;
    const dim3 grid((unsigned)(((T_q + Q8_QB - 1) / Q8_QB) * H));
    const int hg = attn_head_group(2 * T_k * H * 128, H);   // int8 K, fp8 V
    if (q_bf16)
        attn_q8_kernel<true><<<grid, 256, 0, st>>>(nullptr, nullptr, (const uint8_t*)(b + L.k8),
                                                   (const float*)(b + L.sk), (const uint8_t*)(b + L.v8),
                                                   (const float*)(b + L.sv), (__bf16*)o, (int)T_q, (int)T_k,
                                                   (int)L.nt, (int)ldo, segs, c, (const __bf16*)q_bf16, ldq, H, hg);
    else
        attn_q8_kernel<false><<<grid, 256, 0, st>>>((const int8_t*)(b + L.q8), (const float*)(b + L.sq),
                                                    (const uint8_t*)(b + L.k8), (const float*)(b + L.sk),
                                                    (const uint8_t*)(b + L.v8), (const float*)(b + L.sv),
                                                    (__bf16*)o, (int)T_q, (int)T_k, (int)L.nt, (int)ldo, segs, c,
                                                    nullptr, 0, H, hg);
    return hipGetLastError();
}

}  // namespace dit
