// GEMMs of the block: y = A W^T with A [M, K] and W [N, K], both K-contiguous.
//  - int8 x int8 -> int32 on v_mfma_i32_16x16x64_i8 (W8A8 linears)
//  - bf16 x bf16 -> fp32 on v_mfma_f32_16x16x32_bf16 (bf16 linears)
//  - fp32 FMA tiles (fp32 mode)
// The two MFMA kernels share one byte-level tiling: a 16-byte operand slice per
// lane covers 16 int8 or 8 bf16 values of one row, so a 128-byte K step is two
// MFMA K steps for either type.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dit {

__device__ __forceinline__ float gelu_tanh(float u) { return gelu_tanh_fast(u); }

// Epilogue variants, fixed per kernel instantiation (keeps one path live).
enum EpiVariant : int { EV_STORE = 0, EV_STORE_ACC = 1, EV_GELU = 2, EV_RESID = 3, EV_QKV = 4 };

// EPI_QKV_ROPE, first half, on 16 consecutive columns n..n+15 of one row
// (bias already added): the bf16 rounding of the stored QKV output; returns
// the sum of squares of the rounded values (the row's RMSNorm statistic over
// its head is the sum over 8 such groups).
__device__ __forceinline__ float qkv_stat16(float (&v)[16]) {
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        v[e] = bf16r(v[e]);
        ss += v[e] * v[e];
    }
    return ss;
}
// The same, adding the column bias read from memory first.
__device__ __forceinline__ float qkv_prep16(const EpiParams& ep, int64_t n, float (&v)[16]) {
    if (ep.bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 b = *reinterpret_cast<const float4*>(ep.bias + n + 4 * q);
            v[4 * q] += b.x; v[4 * q + 1] += b.y; v[4 * q + 2] += b.z; v[4 * q + 3] += b.w;
        }
    }
    return qkv_stat16(v);
}

// Gains and RoPE factors of 16 consecutive columns n..n+15 of row m (loaded
// ahead of the statistic so their latency overlaps it).
struct QkvAux {
    float g[16], cs[8], sn[8];
};
__device__ __forceinline__ void qkv_gain16(const EpiParams& ep, int64_t n, QkvAux& a) {
    const int64_t D = ep.D;
    const int sec = (int)(n / D);
    const float* g = (sec == 0 ? ep.g_q : ep.g_k) + (n % 128);
    if (sec == 2) return;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 t = *reinterpret_cast<const float4*>(g + 4 * q);
        a.g[4 * q] = t.x; a.g[4 * q + 1] = t.y; a.g[4 * q + 2] = t.z; a.g[4 * q + 3] = t.w;
    }
}
__device__ __forceinline__ void qkv_rope16(const EpiParams& ep, int64_t m, int64_t n, QkvAux& a) {
    if (n / ep.D == 2) return;
    const int64_t p = m * 64 + (n % 128) / 2;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const float4 c = *reinterpret_cast<const float4*>(ep.cos_t + p + 4 * q);
        const float4 s = *reinterpret_cast<const float4*>(ep.sin_t + p + 4 * q);
        a.cs[4 * q] = c.x; a.cs[4 * q + 1] = c.y; a.cs[4 * q + 2] = c.z; a.cs[4 * q + 3] = c.w;
        a.sn[4 * q] = s.x; a.sn[4 * q + 1] = s.y; a.sn[4 * q + 2] = s.z; a.sn[4 * q + 3] = s.w;
    }
}

// Second half: v passes through; q and k get RMSNorm with the head's sum of
// squares, cast before the gain multiply, then RoPE on the interleaved pairs,
// each product rounded to bf16 (the order of the separate norm/RoPE kernel).
__device__ __forceinline__ void qkv_finish16(const EpiParams& ep, int64_t m, int64_t n, const float (&v)[16],
                                             float ss_head, const QkvAux& a) {
    const int64_t D = ep.D;
    const int sec = (int)(n / D);
    const int64_t c = n - (int64_t)sec * D;
    __bf16* dst = reinterpret_cast<__bf16*>(sec == 0 ? ep.q_out : sec == 1 ? ep.k_out : ep.v_out) + m * D + c;
    v8bf o0, o1;
    if (sec == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o0[e] = to_bf16(v[e]);
            o1[e] = to_bf16(v[8 + e]);
        }
    } else {
        const float r = 1.0f / sqrtf(ss_head * (1.0f / 128.0f) + ep.qk_eps);
        float out[16];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float na = bf16r(bf16r(v[2 * k] * r) * a.g[2 * k]);
            const float nb = bf16r(bf16r(v[2 * k + 1] * r) * a.g[2 * k + 1]);
            out[2 * k] = na * a.cs[k] - nb * a.sn[k];
            out[2 * k + 1] = na * a.sn[k] + nb * a.cs[k];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o0[e] = to_bf16(out[e]);
            o1[e] = to_bf16(out[8 + e]);
        }
    }
    reinterpret_cast<v8bf*>(dst)[0] = o0;
    reinterpret_cast<v8bf*>(dst)[1] = o1;
}

// Apply the epilogue to one output element; v already holds acc*scales (+bias added here).
template <int EV>
__device__ __forceinline__ void epilogue(const EpiParams& ep, int64_t m, int64_t n, float v,
                                         int32_t acc_i) {
    if (ep.bias) v += ep.bias[n];
    const bool rb = ep.act_bf16 != 0;
    if constexpr (EV == EV_STORE || EV == EV_STORE_ACC) {
        if (ep.y_bf16)
            reinterpret_cast<__bf16*>(ep.y)[m * ep.ldy + n] = to_bf16(v);
        else
            reinterpret_cast<float*>(ep.y)[m * ep.ldy + n] = v;
        if constexpr (EV == EV_STORE_ACC) ep.acc_out[m * ep.ldacc + n] = acc_i;
    } else if constexpr (EV == EV_GELU) {
        const float u = rb ? bf16r(v) : v;
        float g = gelu_tanh(u);
        if (ep.gmul) g *= (float)reinterpret_cast<const __bf16*>(ep.gmul)[m * ep.ldgm + n];
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

// Epilogue over 16 consecutive columns n0..n0+15 of row m (n0 % 16 == 0,
// 16-byte aligned rows).  v[] holds acc * scales (int8 GEMM) or the fp32 sums.
template <int EV>
__device__ __forceinline__ void epilogue16(const EpiParams& ep, int64_t m, int64_t n0, float (&v)[16],
                                           const int32_t (&acc)[16], bool add_bias = true) {
    if (add_bias && ep.bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 b = *reinterpret_cast<const float4*>(ep.bias + n0 + 4 * q);
            v[4 * q] += b.x; v[4 * q + 1] += b.y; v[4 * q + 2] += b.z; v[4 * q + 3] += b.w;
        }
    }
    const bool rb = ep.act_bf16 != 0;
    if constexpr (EV != EV_RESID) {
        if constexpr (EV == EV_GELU) {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = gelu_tanh(rb ? bf16r(v[e]) : v[e]);
            if (ep.gmul) {
                const v8bf* up = reinterpret_cast<const v8bf*>(reinterpret_cast<const __bf16*>(ep.gmul) +
                                                               m * ep.ldgm + n0);
                const v8bf u0 = up[0], u1 = up[1];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[e] *= (float)u0[e];
                    v[8 + e] *= (float)u1[e];
                }
            }
        }
        if (ep.y_bf16) {
            v8bf o0, o1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o0[e] = to_bf16(v[e]);
                o1[e] = to_bf16(v[8 + e]);
            }
            v8bf* yp = reinterpret_cast<v8bf*>(reinterpret_cast<__bf16*>(ep.y) + m * ep.ldy + n0);
            yp[0] = o0;
            yp[1] = o1;
        } else {
            float4* yp = reinterpret_cast<float4*>(reinterpret_cast<float*>(ep.y) + m * ep.ldy + n0);
#pragma unroll
            for (int q = 0; q < 4; ++q) yp[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
        if constexpr (EV == EV_STORE_ACC) {
            int4* ap = reinterpret_cast<int4*>(ep.acc_out + m * ep.ldacc + n0);
#pragma unroll
            for (int q = 0; q < 4; ++q) ap[q] = make_int4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
        }
    } else {
        const int set = seg_set(ep.sm, m);
        const float* gate = ep.gate + (int64_t)set * ep.gate_stride + n0;
        float gv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 gq = *reinterpret_cast<const float4*>(gate + 4 * q);
            gv[4 * q] = gq.x; gv[4 * q + 1] = gq.y; gv[4 * q + 2] = gq.z; gv[4 * q + 3] = gq.w;
        }
        if (rb) {
            v8bf* xp = reinterpret_cast<v8bf*>(reinterpret_cast<__bf16*>(ep.x) + m * ep.ldx + n0);
            v8bf x0 = xp[0], x1 = xp[1];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x0[e] = to_bf16((float)x0[e] + gv[e] * bf16r(v[e]));
                x1[e] = to_bf16((float)x1[e] + gv[8 + e] * bf16r(v[8 + e]));
            }
            xp[0] = x0;
            xp[1] = x1;
        } else {
            float4* xp = reinterpret_cast<float4*>(reinterpret_cast<float*>(ep.x) + m * ep.ldx + n0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4 xv = xp[q];
                xv.x += gv[4 * q] * v[4 * q];
                xv.y += gv[4 * q + 1] * v[4 * q + 1];
                xv.z += gv[4 * q + 2] * v[4 * q + 2];
                xv.w += gv[4 * q + 3] * v[4 * q + 3];
                xp[q] = xv;
            }
        }
    }
}

// ---------------------------------------------------------------- MFMA GEMM
constexpr int BM = 128, BN = 128, BKB = 128;   // tile rows, cols, K bytes
constexpr int LDS_STRIDE = BKB + 16;           // padded row (bytes): conflict-free 16-byte reads
constexpr int NTHREADS = 256;

template <bool I8, int EV>
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
    v4i ra[4], rb[4];
    auto gload = [&](int64_t kb0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + i * NTHREADS;
            const int r = c / (BKB / 16), col = (c % (BKB / 16)) * 16;
            const int64_t gm = m0 + r, gn = n0 + r;
            ra[i] = gm < M ? *reinterpret_cast<const v4i*>(A + gm * lda_b + kb0 + col) : v4i{0, 0, 0, 0};
            rb[i] = gn < N ? *reinterpret_cast<const v4i*>(W + gn * Kb + kb0 + col) : v4i{0, 0, 0, 0};
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + i * NTHREADS;
            const int r = c / (BKB / 16), col = (c % (BKB / 16)) * 16;
            *reinterpret_cast<v4i*>(&As[buf][r * LDS_STRIDE + col]) = ra[i];
            *reinterpret_cast<v4i*>(&Bs[buf][r * LDS_STRIDE + col]) = rb[i];
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
            v4i af[4], bf[4];
            const int koff = ks * 64 + (lane / 16) * 16;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const v4i*>(&As[buf][(wm * 64 + i * 16 + lane % 16) * LDS_STRIDE + koff]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const v4i*>(&Bs[buf][(wn * 64 + j * 16 + lane % 16) * LDS_STRIDE + koff]);
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
                        const int32_t a = acc[i][j][r] - (ep.a_zero ? ep.a_zero[m] * ep.w_sum[n] : 0);
                        const float v = (float)a * ep.a_scale[m] * ep.w_scale[n];
                        epilogue<EV>(ep, m, n, v, a);
                    } else {
                        epilogue<EV>(ep, m, n, acc[i][j][r], 0);
                    }
                }
            }
}

// ---------------------------------------------------------------- large-tile MFMA GEMM
// 256x256 workgroup tile, 8 waves (2 per SIMD) in a 2 x 4 grid, each wave
// owning a 128x64 sub-tile: 32 MFMA accumulator tiles of 16x16 held in VGPRs
// (built with -mllvm -amdgpu-mfma-vgpr-form=1; with accumulators in AGPRs the
// compiler rotates them through copies every iteration, and each copy waits
// for the MFMA pipe).  Two waves per SIMD let one wave's MFMAs run while the
// other waits on LDS.
// Software pipeline over K steps of 64 bytes (one MFMA K) grouped in stages of
// 128 bytes, with a 2-slot LDS ring (one stage per slot) filled by buffer
// loads straight into LDS (no register staging, no LDS write instructions).
// A stage row is one whole 128-byte line of A or W: loading only 64 bytes of
// each row per step measured half the L2-to-CU rate of whole lines (27 vs 52
// bytes per clock per CU with every CU loading), below the 32 bytes per clock
// the MFMAs consume.  While the MFMAs of step t run from registers, each wave
// reads the fragments of step t+1 from LDS; during the second step of stage s
// it also issues the loads of stage s+2 into the slot stage s used, which
// then have two steps to land.  One barrier per stage; the loop body is
// branch-free so the scheduler can interleave the three streams.
// LDS has 32 banks = 128 bytes, one stage row.  16-byte chunk c of row r sits
// at slot c ^ (r & 7), so the eight rows read together by one ds_read_b128
// phase hit eight different bank groups.
constexpr int L_BM = 256, L_BN = 256, L_BK = 64, L_SK = 128, L_SLOTS = 2, L_THREADS = 512;
constexpr int L_TILE_BYTES = L_BM * L_SK;               // one operand, one slot
constexpr int L_STAGE_BYTES = 2 * L_TILE_BYTES;
// Epilogue LDS: two slab buffers of 8 waves x 16 rows x (wave tile width + 4)
// words (at most 128 + 4 wide), then the tile's epilogue constants: weight
// scales [256], bias [256] and activation scales [256] (fp32), loaded into LDS
// with the operand prologue.
constexpr int L_CONST = 2 * 8 * 16 * (128 + 4) * 4;
constexpr int L_CONST_BYTES = 3 * 1024;


// Partial last round: with T tiles on C compute units, the C workgroups of one
// persistent launch each take floor(T/C) whole tiles; each of the r remaining
// tiles (all T when T < C) is split into S K ranges, one per workgroup, which
// stores its partial sums (int32 for int8 operands, fp32 for bf16).  A second
// launch adds the partials (int32: exact in any order; fp32: in K order) and
// applies the epilogue; the kernel boundary orders the partial stores before
// their reads.  On half the XCDs the K range runs before the whole tiles (its
// partial stores overlap them), on the other half after them.  For long K loops (more than 64 steps) two
// launches measured faster: whole tiles, then the K ranges (the same kernel
// with full = 0).
struct LargePlan {
    int32_t full;       // whole tiles of this launch: tile order [0, full)
    int32_t tail0;      // first split tile (tile order)
    int32_t r;          // split tiles [tail0, tail0 + r), S K ranges each (S = 0: none)
    int32_t S;
};

// Grouped tile order: groups of 8 M-tiles sweep N so that neighbouring tiles
// share rows of A and W.
__device__ __forceinline__ void tile_origin(int tau, int tiles_m, int tiles_n, int64_t& m0, int64_t& n0) {
    constexpr int GROUP = 8;
    const int per_group = GROUP * tiles_n;
    const int g = tau / per_group;
    const int first_m = g * GROUP;
    const int gsize = min(tiles_m - first_m, GROUP);
    m0 = (int64_t)(first_m + (tau % per_group) % gsize) * L_BM;
    n0 = (int64_t)((tau % per_group) / gsize) * L_BN;
}

// One 256 x 256 tile (TS = 1) or 128 x 128 sub-tile (TS = 2, whole K loop, no
// partial sums), K steps [ks0, ks0 + nk) (ks0 and nk even: whole stages), by
// the whole workgroup: with part == NULL the epilogue writes the outputs, else
// the int32 sums go to the 256 x 256 partial tile at part (fragment order).
// WN: waves along N (4: 2 x 4 waves of 128 x 64; 2: 4 x 2 waves of 64 x 128,
// so that one wave holds whole 128-column heads for the fused QKV epilogue).
// Either way a wave of a whole tile reads 12 fragments per step and issues 32
// MFMAs; on a sub-tile (WN = 4, waves of 64 x 32) 6 and 8.
// W4 (bf16 A only): W holds MXFP4 codes [N, K/2] (E2M1, element 2i in the low
// nibble of byte i) with E8M0 scales ep.w_mx_scale [N, K/32]; each stage's W
// tile is decoded to bf16 in registers (hardware fp4 -> bf16 conversion with
// the fp32 scale) and written to the LDS slot, so 4.25 bits per weight come
// from memory.  Thread t decodes 32 values: row t/2, K half t%2 of the stage.
template <bool I8, int EV, int WN, bool W4 = false, int TS = 1>
__device__ __forceinline__ void large_tile(const uint8_t* __restrict__ A, int64_t lda_b,
                                           const uint8_t* __restrict__ W, int64_t M, int64_t N, int64_t Kb,
                                           const EpiParams& ep, uint8_t* lds, int64_t m0, int64_t n0, int ks0,
                                           int nk, int32_t* part) {
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    static_assert(WN == 4 || WN == 2, "wave grid");
    static_assert(!(W4 && I8), "MXFP4 weights go with bf16 activations");
    static_assert(TS == 1 || (TS == 2 && !W4), "128 x 128 sub-tiles, no MXFP4");
    constexpr int T_BM = L_BM / TS, T_BN = L_BN / TS;       // tile
    constexpr int A_BYTES = T_BM * L_SK, STAGE_BYTES = (T_BM + T_BN) * L_SK;
    constexpr int NLD = 4 / TS;                             // 1 KB loads per wave, operand and stage
    constexpr int WTM = T_BM / (8 / WN), WTN = T_BN / WN;   // wave tile
    static_assert(EV != EV_QKV || WTN == 128, "the fused QKV epilogue needs whole heads per wave");
    constexpr int MF = WTM / 16, NF = WTN / 16;             // 16 x 16 accumulator tiles
    const int wm = wave / WN, wn = wave % WN;

    // Operands go from memory straight into the LDS ring (buffer loads with the
    // lds bit: lane l of a wave's load lands at its M0 base + 16 l).  Wave w's
    // load i covers 16-byte positions p = (4w + i)*64 + lane of a 256 x 128-byte
    // stage, i.e. slot p % 8 of row p / 8; the swizzle is applied by choosing
    // the source chunk (p % 8) ^ (row & 7).  Each group of 8 lanes thus reads
    // one whole 128-byte line.  Rows beyond M or N are clamped: their products
    // only reach outputs that are never stored.  32-bit offsets; the K offset
    // of a stage is the scalar soffset.
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, (int)(M * lda_b), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc((void*)W, 0, (int)(W4 ? N * (Kb / 4) : N * Kb), 0x00020000);
    int aoff[4], boff[4];   // entries [0, NLD)
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int p = (wave * NLD + i) * 64 + lane, r = p >> 3, c = (p & 7) ^ (r & 7);
        aoff[i] = (int)(min(m0 + r, M - 1) * lda_b) + c * 16;
        boff[i] = (int)(min(n0 + r, N - 1) * Kb) + c * 16;
    }
    // MXFP4 W: code and scale offsets of this thread's row and K half; LDS
    // byte offset of its row in the W part of a slot
    const __amdgpu_buffer_rsrc_t rs_s4 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)ep.w_mx_scale, 0, W4 ? (int)(N * (Kb / 64)) : 0, 0x00020000);
    int w4_off = 0, s4_off = 0, w4_lds = 0, w4_sw = 0;
    v4i w4_codes = {0, 0, 0, 0};
    uint32_t w4_scale = 0;
    if constexpr (W4) {
        const int row = tid >> 1, half = tid & 1;
        const int64_t gr = min(n0 + row, N - 1);
        w4_off = (int)(gr * (Kb / 4)) + half * 16;
        s4_off = (int)(gr * (Kb / 64)) + half;
        w4_lds = A_BYTES + row * L_SK;
        w4_sw = (row & 7) | (half << 5);   // chunk c = 4 half + j sits at slot c ^ (row & 7)
        (void)boff;
    }
    const int wbase = __builtin_amdgcn_readfirstlane(wave * NLD * 1024);
    typedef typename std::conditional<I8, v4i, v4f>::type acc_t;
    typedef typename std::conditional<I8, v4i, v8bf>::type frag_t;
    // fragment reads: lane reads chunk (4h + lane / 16) of rows base + lane % 16
    // (+16 i) in step half h; rows are 16-aligned, so row & 7 = lane & 7
    const int sw = lane & 7, chunk = lane / 16;
    const int arow = wm * WTM + lane % 16, brow = wn * WTN + lane % 16;
    const int aswz0 = arow * L_SK + ((chunk ^ sw) << 4), aswz1 = arow * L_SK + (((4 + chunk) ^ sw) << 4);
    const int bswz0 = A_BYTES + brow * L_SK + ((chunk ^ sw) << 4);
    const int bswz1 = A_BYTES + brow * L_SK + (((4 + chunk) ^ sw) << 4);
    const int nst = nk / 2;   // stages (nk is even)

#define LG_DMA(stage)                                                                         \
    do {                                                                                      \
        const int kb0 = ks0 * L_BK + (stage) * L_SK;                                          \
        uint8_t* sl = lds + ((stage) % L_SLOTS) * STAGE_BYTES + wbase;                         \
        _Pragma("unroll") for (int i = 0; i < NLD; ++i) {                                     \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_ptr_t)(sl + i * 1024), 16, aoff[i], kb0, 0, 0); \
            if constexpr (!W4)                                                                \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, (lds_ptr_t)(sl + A_BYTES + i * 1024), 16, \
                                                         boff[i], kb0, 0, 0);                 \
        }                                                                                     \
    } while (0)
// MXFP4 W: codes and scale of a stage into registers (issued one stage before
// they are decoded), then decoded into the stage's slot
#define W4_LOAD(stage)                                                                        \
    do {                                                                                      \
        const int kb0 = ks0 * L_BK + (stage) * L_SK;                                          \
        w4_codes = (v4i)__builtin_amdgcn_raw_buffer_load_b128(rs_w, w4_off, kb0 / 4, 0);       \
        w4_scale = __builtin_amdgcn_raw_buffer_load_b8(rs_s4, s4_off, kb0 / 64, 0);            \
    } while (0)
#define W4_STORE(stage)                                                                       \
    do {                                                                                      \
        uint8_t* sl = lds + ((stage) % L_SLOTS) * STAGE_BYTES + w4_lds;                        \
        const float sc = w4_scale == 255u ? __builtin_nanf("") : ldexpf(1.0f, (int)w4_scale - 127); \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                       \
            const uint32_t word = (uint32_t)w4_codes[j];                                      \
            v4i o;                                                                            \
            o[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0)); \
            o[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1)); \
            o[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2)); \
            o[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3)); \
            const int chunk = ((w4_sw >> 5) * 4 + j) ^ (w4_sw & 7);                          \
            *reinterpret_cast<v4i*>(sl + (chunk << 4)) = o;                                   \
        }                                                                                     \
    } while (0)
// fragments of step half H of the stage in slot (stage % 2)
#define LG_FRAGS(stage, H, fa, fb)                                                      \
    do {                                                                                \
        const uint8_t* src = lds + ((stage) % L_SLOTS) * STAGE_BYTES;                   \
        _Pragma("unroll") for (int j = 0; j < NF; ++j)                                  \
            fb[j] = *reinterpret_cast<const frag_t*>(src + ((H) ? bswz1 : bswz0) + j * 16 * L_SK); \
        _Pragma("unroll") for (int i = 0; i < MF; ++i)                                  \
            fa[i] = *reinterpret_cast<const frag_t*>(src + ((H) ? aswz1 : aswz0) + i * 16 * L_SK); \
    } while (0)
// End of a step: this wave's loads issued since the last stage boundary may
// stay in flight (VM: 8 per thread, or 0); everything older has landed in LDS.
// Then all waves meet.  The scheduling fences keep each step's MFMAs on their
// side of the barrier.
#define LG_BARRIER(VM)                                                                  \
    do {                                                                                \
        __builtin_amdgcn_sched_barrier(0);                                              \
        asm volatile("s_waitcnt vmcnt(" #VM ")\n\ts_waitcnt lgkmcnt(0)" ::: "memory");  \
        __builtin_amdgcn_s_barrier();                                                   \
        __builtin_amdgcn_sched_barrier(0);                                              \
    } while (0)
#define LG_MFMA(fa, fb)                                                                           \
    _Pragma("unroll") for (int i = 0; i < MF; ++i)                                                \
        _Pragma("unroll") for (int j = 0; j < NF; ++j) {                                          \
            if constexpr (I8)                                                                     \
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0); \
            else                                                                                  \
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0); \
        }
// interleave: per 8 MFMAs, 3 fragment reads (and 2 loads into LDS when the
// step issues a stage)
#define LG_SCHEDULE(LOADS)                                                 \
    if constexpr (TS == 1) {                                               \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) {                    \
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);             \
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);             \
            if (LOADS) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  \
        }                                                                  \
    }
// stage s: step 2s (fragments of step 2s+1), then step 2s+1 (loads of stage
// s+2 when LOADS, fragments of step 2s+2).  One barrier per stage, after step
// 2s: stage s+1 has landed for every wave and every read of slot s (stage s)
// is done, so step 2s+1 may refill slot s and read slot s+1.  Nothing needs a
// barrier after step 2s+1: the next refill of slot s+1 waits for the barrier
// after step 2s+2.
// With MXFP4 W the barrier also covers the codes of stage s+2 (loaded one stage
// earlier); they are decoded into the freed slot, and the codes of stage s+3
// are loaded (W4_NEXT).
#define LG_PAIR(s, LOADS, W4_NEXT)                              \
    do {                                                        \
        LG_FRAGS(s, 1, fa1, fb1);                               \
        LG_MFMA(fa0, fb0);                                      \
        LG_SCHEDULE(false);                                     \
        LG_BARRIER(0);                                          \
        if constexpr (W4) {                                     \
            if (LOADS) W4_STORE((s) + 2);                       \
            if (W4_NEXT) W4_LOAD((s) + 3);                      \
        }                                                       \
        if (LOADS) LG_DMA((s) + 2);                             \
        LG_FRAGS((s) + 1, 0, fa0, fb0);                         \
        LG_MFMA(fa1, fb1);                                      \
        LG_SCHEDULE(LOADS);                                     \
        __builtin_amdgcn_sched_barrier(0);                      \
    } while (0)

    acc_t acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
    if constexpr (I8) {
        // Zero points of asymmetric activation codes: the wanted integer sum is
        // sum_k (q - z) w = sum_k q w - z sum_k w, so the accumulators start at
        // -z[m] * wsum[n] (lane l holds column l % 16 and rows 4 (l / 16) + r of
        // each 16 x 16 tile).  |z| <= 128 and |wsum| <= 2^23 for K <= 65536: a
        // 24-bit product, exact in int32.  K-split partial tiles leave the
        // correction to their reduce.
        if (ep.a_zero != nullptr && part == nullptr) {
            int wsj[NF];
#pragma unroll
            for (int j = 0; j < NF; ++j) {
                const int64_t nn = n0 + wn * WTN + j * 16 + lane % 16;
                wsj[j] = nn < N ? ep.w_sum[nn] : 0;
            }
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t mm = m0 + wm * WTM + i * 16 + (lane / 16) * 4 + r;
                    const int z = mm < M ? ep.a_zero[mm] : 0;
#pragma unroll
                    for (int j = 0; j < NF; ++j) acc[i][j][r] = -__mul24(z, wsj[j]);
                }
        }
    }

    // the epilogue's column and row constants of a whole tile go to LDS ahead of
    // the operands (wave 0; the prologue's first wait covers them: loads land
    // in issue order); columns or rows past N or M read as zero
    if (part == nullptr && __builtin_amdgcn_readfirstlane(wave) == 0) {
        if constexpr (I8) {
            const auto rw = __builtin_amdgcn_make_buffer_rsrc((void*)ep.w_scale, 0, (int)(N * 4), 0x00020000);
            const auto ra = __builtin_amdgcn_make_buffer_rsrc((void*)ep.a_scale, 0, (int)(M * 4), 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(lds + L_CONST), 16, (int)(n0 * 4) + lane * 16,
                                                     0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(lds + L_CONST + 2048), 16,
                                                     (int)(m0 * 4) + lane * 16, 0, 0, 0);
        }
        if (ep.bias != nullptr) {
            const auto rb = __builtin_amdgcn_make_buffer_rsrc((void*)ep.bias, 0, (int)(N * 4), 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(lds + L_CONST + 1024), 16,
                                                     (int)(n0 * 4) + lane * 16, 0, 0, 0);
        }
    }
    // prologue: stages 0 and 1 in flight, wait for 0, fragments of step 0
    if constexpr (W4) {
        // codes of stages 0 and 1 decoded before the first barrier, those of
        // stage 2 in flight (two loads per thread and stage)
        W4_LOAD(0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        W4_STORE(0);
        if (nst > 1) {
            W4_LOAD(1);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            W4_STORE(1);
        }
        LG_DMA(0);
        if (nst > 1) LG_DMA(1);
        if (nst > 2) {
            W4_LOAD(2);
            LG_BARRIER(6);
        } else if (nst > 1) {
            LG_BARRIER(4);
        } else {
            LG_BARRIER(0);
        }
    } else {
        LG_DMA(0);
        if (nst > 1) {
            // this wave's loads of stage 1 (2 NLD) may stay in flight
            LG_DMA(1);
            if constexpr (TS == 1)
                LG_BARRIER(8);
            else
                LG_BARRIER(4);
        } else {
            LG_BARRIER(0);
        }
    }
    frag_t fa0[MF], fb0[NF], fa1[MF], fb1[NF];
    LG_FRAGS(0, 0, fa0, fb0);

    // Stages that load stage s+2, then the last two without loads.  The step
    // after the last reads fragments of a slot nobody uses (harmless).
    int s = 0;
    if constexpr (W4) {
        for (; s + 3 < nst; ++s) LG_PAIR(s, true, true);
        if (s + 2 < nst) {
            LG_PAIR(s, true, false);
            ++s;
        }
    } else {
        for (; s + 2 < nst; ++s) LG_PAIR(s, true, false);
    }
    for (; s < nst; ++s) LG_PAIR(s, false, false);
    // every load has landed (the last barrier waited for all); the epilogue
    // reuses LDS once every wave's fragment reads are done
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#undef LG_DMA
#undef W4_LOAD
#undef W4_STORE
#undef LG_FRAGS
#undef LG_BARRIER
#undef LG_MFMA
#undef LG_SCHEDULE
#undef LG_PAIR

    if (TS == 1 && part != nullptr) {
        // K-split partial sums go straight from the accumulators, in fragment
        // order: 16-byte piece ((((wm MF + i) WN + wn) NF + j) 64 + lane) holds
        // acc[i][j], so each store of a wave is 1 KB contiguous and the 16 KB
        // of tile rows [16 b, 16 b + 16) are contiguous (WN NF = 16).  Row
        // blocks at or past M are not stored (their reduce returns first).
#pragma unroll
        for (int i = 0; i < MF; ++i) {
            if (m0 + wm * WTM + i * 16 >= M) break;
#pragma unroll
            for (int j = 0; j < NF; ++j)
                reinterpret_cast<acc_t*>(part)[((((wm * MF + i) * WN + wn) * NF + j) << 6) + lane] = acc[i][j];
        }
        return;
    }

    // Epilogue: for each 16-row slab i, every wave parks its 16 x WTN slab of
    // accumulators in its own LDS region (two buffers: slab i+1 is parked
    // while slab i is finished), then each lane finishes 16 consecutive
    // columns of one row (LPR lanes per row, RPP rows per pass).
    constexpr int EP_STRIDE = WTN + 4;   // words per slab row (padded)
    constexpr int LPR = WTN / 16, RPP = kWave / LPR;
    // rows of a slab per pass: RPP (lanes of rows past the slab's 16 idle)
    constexpr int PASSES = RPP >= 16 ? 1 : 16 / RPP;
    static_assert(2 * 8 * 16 * EP_STRIDE * 4 <= L_CONST, "slab buffers");
    float* const slab_buf[2] = {reinterpret_cast<float*>(lds) + wave * 16 * EP_STRIDE,
                                reinterpret_cast<float*>(lds) + (8 + wave) * 16 * EP_STRIDE};
    const int er0 = lane / LPR, ec = (lane % LPR) * 16;
    const int64_t n = n0 + wn * WTN + ec;
    QkvAux aux;
    if constexpr (EV == EV_QKV) {
        qkv_gain16(ep, n, aux);
    }
    // column constants (weight scales, bias) from the tile's LDS copy
    const float* cl = reinterpret_cast<const float*>(lds + L_CONST);
    float colw[16], colb[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const v4f w4 = I8 ? *reinterpret_cast<const v4f*>(cl + wn * WTN + ec + 4 * q) : v4f{1.f, 1.f, 1.f, 1.f};
        const v4f b4 = ep.bias != nullptr ? *reinterpret_cast<const v4f*>(cl + 256 + wn * WTN + ec + 4 * q)
                                          : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            colw[4 * q + e] = w4[e];
            colb[4 * q + e] = b4[e];
        }
    }
    auto park = [&](int i) {
        float* sl = slab_buf[i & 1];
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (I8)
                    reinterpret_cast<int32_t*>(sl)[((lane / 16) * 4 + r) * EP_STRIDE + j * 16 + lane % 16] =
                        acc[i][j][r];
                else
                    sl[((lane / 16) * 4 + r) * EP_STRIDE + j * 16 + lane % 16] = acc[i][j][r];
            }
    };
    park(0);
#pragma unroll
    for (int i = 0; i < MF; ++i) {
        const float* slab = slab_buf[i & 1];
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            const int er = min(pass * RPP + er0, 15);
            const int64_t m = m0 + wm * WTM + i * 16 + er;
            // this row's 16 accumulators (and its activation scale) first, then
            // slab i+1 is parked while they are finished: a wave's LDS accesses
            // execute in order, so the writes wait behind these reads only, and
            // slab i's buffer is parked again only after its last reads
            acc_t t[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) t[q] = *reinterpret_cast<const acc_t*>(slab + er * EP_STRIDE + ec + 4 * q);
            const float sa = I8 ? cl[512 + wm * WTM + i * 16 + er] : 1.0f;
            if (pass == 0 && i + 1 < MF) {
                asm volatile("" ::: "memory");
                park(i + 1);
            }
            float v[16];
            int32_t ai[16];
            const bool ok = pass * RPP + er0 < 16 && m < M && n < N;
            if (ok) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (I8) {
                            // (zero-point correction, if any, is already in the accumulators)
                            ai[4 * q + e] = t[q][e];
                            v[4 * q + e] = (float)t[q][e] * sa * colw[4 * q + e];
                        } else {
                            ai[4 * q + e] = 0;
                            v[4 * q + e] = t[q][e];
                        }
                    }
            }
            if constexpr (EV == EV_QKV) {
                // a head's 128 columns are this wave's 8 lanes of the row
                float ss = 0.0f;
                if (ok) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) v[e] += colb[e];
                    ss = qkv_stat16(v);
                }
                ss += dpp_f<0xB1>(ss);
                ss += dpp_f<0x4E>(ss);
                ss += __shfl_xor(ss, 4, kWave);
                if (ok) {
                    qkv_rope16(ep, m, n, aux);
                    qkv_finish16(ep, m, n, v, ss, aux);
                }
            } else {
                if (ok) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) v[e] += colb[e];
                    epilogue16<EV>(ep, m, n, v, ai, false);
                }
            }
        }
        asm volatile("" ::: "memory");
    }
    // the next tile's loads reuse the LDS of this epilogue; its global stores
    // may stay in flight
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// SUB > 0: the r tiles of the last round are not split along K but into
// SUB x SUB sub-tiles of (256 / SUB)^2 with the whole K loop each (S = SUB^2
// jobs per tile): no partial sums and no reduce, at the price of smaller
// tiles (more operand bytes and fragment reads per product) for that round.
template <bool I8, int EV, int WN, bool W4 = false, int SUB = 0>
__global__ void __launch_bounds__(L_THREADS, 1)
gemm_large_kernel(const uint8_t* __restrict__ A, int64_t lda_b, const uint8_t* __restrict__ W,
                  int64_t M, int64_t N, int64_t Kb, EpiParams ep, LargePlan lp) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tiles_m = (int)((M + L_BM - 1) / L_BM);
    const int tiles_n = (int)((N + L_BN - 1) / L_BN);
    const int nk_all = (int)(Kb / L_BK);
    const int G = gridDim.x, b = blockIdx.x;
    // Jobs: one K range of a split tile (job cj) and whole tiles, one round of
    // G per job.  Workgroups are dealt round-robin to the 8 XCDs; with full a
    // multiple of G, XCD x takes the contiguous tile range [x full/8,
    // (x+1) full/8) so that tiles sharing rows of A or W share an L2.  One call
    // site keeps one copy of the tile code.  The even XCDs take their K range
    // first and the odd ones last, so the two halves of the chip run their
    // whole tiles a K range out of phase: the epilogues' output stores, which
    // saturate the write path when every CU stores its tile at once, come in
    // two bursts of half the size.
    const bool chunk = lp.S > 0 && b < lp.r * lp.S;
    const bool xcd = G % 8 == 0 && lp.full % G == 0;
    const int jobs = (lp.full + G - 1) / G;
    const int cj = chunk ? ((b & 1) ? jobs : 0) : -1;   // job index of the K range
    for (int j = 0; j < jobs + (chunk ? 1 : 0); ++j) {
        // keep the epilogue's parameter loads inside the loop (hoisting them
        // would hold them in registers across the main loop)
        asm volatile("" ::: "memory");
        int tau, ks0 = 0, nk = nk_all;
        int32_t* part = nullptr;
        const int jw = (chunk && j > cj) ? j - 1 : j;            // whole-tile round
        if (j == cj) {
            // split job J of workgroup b: XCD x = b % 8 takes the contiguous
            // job range [x q + min(x, rem), ...) (q = rS / 8, rem = rS % 8), i.e.
            // all K ranges of neighbouring tiles, so their A and W slices are
            // fetched into one L2 and shared there
            const int rS = lp.r * lp.S, x = b % 8, q = rS / 8, rem = rS % 8;
            const int J = x * q + min(x, rem) + b / 8;
            const int t = J / lp.S, k = J % lp.S;
            if constexpr (SUB > 0) {
                // sub-tile k of tile t: rows (k / SUB) 256/SUB.., columns (k % SUB) 256/SUB..
                int64_t m0, n0;
                tile_origin(lp.tail0 + t, tiles_m, tiles_n, m0, n0);
                m0 += (int64_t)(k / SUB) * (L_BM / SUB);
                n0 += (int64_t)(k % SUB) * (L_BN / SUB);
                large_tile<I8, EV, 4, false, SUB>(A, lda_b, W, M, N, Kb, ep, lds, m0, n0, 0, nk_all, nullptr);
                continue;
            }
            // whole 128-byte stages
            ks0 = 2 * (int)((int64_t)k * (nk_all / 2) / lp.S);
            nk = 2 * (int)((int64_t)(k + 1) * (nk_all / 2) / lp.S) - ks0;
            tau = lp.tail0 + t;
            part = ep.split_partial + ((int64_t)t * lp.S + k) * (L_BM * L_BN);
        } else {
            tau = xcd ? (b % 8) * (lp.full / 8) + jw * (G / 8) + b / 8 : jw * G + b;
            if (tau >= lp.full) continue;
        }
        int64_t m0, n0;
        tile_origin(tau, tiles_m, tiles_n, m0, n0);
        large_tile<I8, EV, WN, W4>(A, lda_b, W, M, N, Kb, ep, lds, m0, n0, ks0, nk, part);
    }
}

constexpr int kNumCU = 256;
constexpr size_t L_LDS = (size_t)std::max(L_SLOTS * L_STAGE_BYTES, L_CONST + L_CONST_BYTES);
static_assert(L_LDS <= 160 * 1024, "LDS per workgroup");

// The 256 x 256 persistent kernel takes a shape when its tiles, or their K-split
// ranges, occupy at least three quarters of the compute units; smaller shapes
// go to the 128 x 128 kernel.
static bool use_large(int64_t M, int64_t N, int nk, bool can_split) {
    const int64_t tiles = ((M + L_BM - 1) / L_BM) * ((N + L_BN - 1) / L_BN);
    if (tiles >= kNumCU) return true;
    int64_t jobs = tiles;
    if (can_split) {
        const int64_t S = std::min<int64_t>(std::min<int64_t>(kNumCU / tiles, 16), nk / 8);
        if (S >= 2) jobs = tiles * S;
    }
    return 4 * jobs >= 3 * kNumCU;
}

static unsigned large_grid(int64_t M, int64_t N) {
    return (unsigned)(((M + L_BM - 1) / L_BM) * ((N + L_BN - 1) / L_BN));
}

static unsigned gemm_grid(int64_t M, int64_t N) {
    return (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
}

static int variant(const EpiParams& ep) {
    if (ep.kind == EPI_QKV_ROPE) return EV_QKV;
    if (ep.kind == EPI_GELU) return EV_GELU;
    if (ep.kind == EPI_RESID) return EV_RESID;
    return ep.acc_out ? EV_STORE_ACC : EV_STORE;
}

static int num_cus() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n = v;
        else
            n = kNumCU;
    }
    return n;
}

// Split plan for T tiles of nk K steps: split only the r tiles of the last,
// partial round (every tile when T < C) into S <= C / r ranges of at least 8
// steps each.
static int plan_split(int64_t tiles, int nk, const EpiParams& ep, int64_t* full) {
    *full = tiles;
    if (!ep.split_partial) return 0;
    const int C = num_cus();
    const int64_t R = tiles / C, r = tiles - R * C;
    if (r == 0) return 0;
    int S = (int)std::min<int64_t>(C / r, 16);
    S = std::min(S, nk / 8);
    // a smaller scratch takes fewer K ranges per tile
    S = (int)std::min<int64_t>(S, ep.split_bytes / (r * (int64_t)L_BM * L_BN * 4));
    if (S < 2) return 0;
    *full = R * C;
    return S;
}

// Sum of the S partial tiles of each split tile, then the epilogue.  One
// workgroup per 16 rows of a tile: it adds the 16 KB fragment-order block of
// those rows from each partial (1024 coalesced 16-byte pieces; piece p of the
// block holds rows 4 ((p % 64) / 16) + e, e < 4, of column 16 (p / 64) + p % 16),
// transposes the sums through LDS, and thread t finishes 16 consecutive columns
// of row t / 16.  int8: int32 partials (exact in any order), then the
// zero-point correction and the scales; bf16: fp32 partials added in K order.
template <bool I8, int EV>
__global__ void __launch_bounds__(256) split_reduce_kernel(int64_t M, int64_t N, EpiParams ep, int32_t tau0,
                                                           int32_t S) {
    constexpr int RS = L_BN + 4;   // LDS row stride (words): the 4 rows of a piece hit distinct banks
    typedef typename std::conditional<I8, int32_t, float>::type elt_t;
    typedef typename std::conditional<I8, v4i, v4f>::type part_t;
    __shared__ __attribute__((aligned(16))) elt_t red[16 * RS];
    const int tiles_m = (int)((M + L_BM - 1) / L_BM);
    const int tiles_n = (int)((N + L_BN - 1) / L_BN);
    const int local = blockIdx.x / 16, rb = blockIdx.x % 16;
    int64_t tm0, tn0;
    tile_origin(tau0 + local, tiles_m, tiles_n, tm0, tn0);
    if (tm0 + rb * 16 >= M) return;   // row block not stored (whole workgroup)
    const int t = threadIdx.x;
    const int32_t* blk = ep.split_partial + (int64_t)local * S * (L_BM * L_BN) + rb * 16 * L_BN;
    part_t sum4[4] = {};
    for (int s2 = 0; s2 < S; ++s2)
#pragma unroll
        for (int u = 0; u < 4; ++u)
            sum4[u] += reinterpret_cast<const part_t*>(blk + (int64_t)s2 * (L_BM * L_BN))[t + 256 * u];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int pc = t + 256 * u, ln = pc & 63;
        const int col = (pc >> 6) * 16 + (ln & 15), row = (ln >> 4) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(row + e) * RS + col] = sum4[u][e];
    }
    __syncthreads();
    const int row = rb * 16 + t / 16, col = (t % 16) * 16;
    const int64_t m = tm0 + row, n = tn0 + col;
    if (m >= M || n >= N) return;
    const elt_t* lr = red + (t / 16) * RS + col;
    QkvAux aux;
    if constexpr (EV == EV_QKV) {
        qkv_gain16(ep, n, aux);
        qkv_rope16(ep, m, n, aux);
    }
    float v[16];
    int32_t ai[16] = {};
    if constexpr (I8) {
        v4i sum[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) sum[q] = *reinterpret_cast<const v4i*>(lr + 4 * q);
        if (ep.a_zero) {
            const int za = ep.a_zero[m];
#pragma unroll
            for (int q = 0; q < 4; ++q) sum[q] -= za * *reinterpret_cast<const v4i*>(ep.w_sum + n + 4 * q);
        }
        const float sa = ep.a_scale[m];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const v4f sw = *reinterpret_cast<const v4f*>(ep.w_scale + n + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ai[4 * q + e] = sum[q][e];
                v[4 * q + e] = (float)sum[q][e] * sa * sw[e];
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const v4f f = *reinterpret_cast<const v4f*>(lr + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = f[e];
        }
    }
    if constexpr (EV == EV_QKV) {
        // 16 threads per row; a head's 128 columns are 8 neighbouring lanes
        float ss = qkv_prep16(ep, n, v);
        ss += __shfl_xor(ss, 1, kWave);
        ss += __shfl_xor(ss, 2, kWave);
        ss += __shfl_xor(ss, 4, kWave);
        qkv_finish16(ep, m, n, v, ss, aux);
    } else {
        epilogue16<EV>(ep, m, n, v, ai);
    }
}

// The large kernel addresses each operand with 32-bit buffer offsets.
static bool takes_large(int64_t M, int64_t N, int64_t lda_b, int64_t Kb, bool can_split) {
    return use_large(M, N, (int)(Kb / L_BK), can_split) && lda_b % 16 == 0 && Kb % L_SK == 0 &&
           M * lda_b < ((int64_t)1 << 31) && N * Kb < ((int64_t)1 << 31);
}

bool gemm_bf16_direct_mxfp4(int64_t M, int64_t N, int64_t K, int64_t lda, bool can_split) {
    return takes_large(M, N, lda * 2, K * 2, can_split);
}

// One persistent launch (two for long K loops with a split remainder) of the
// 256 x 256 kernel: full whole tiles, then r remainder tiles as S jobs each
// (K ranges with SUB == 0, sub-tiles otherwise).
template <bool I8, int EV, bool W4, int SUB>
static void launch_large(const uint8_t* a, int64_t lda_b, const uint8_t* w, int64_t M, int64_t N, int64_t Kb,
                         const EpiParams& ep, hipStream_t st, int64_t tiles, int64_t full, int32_t r, int S) {
    constexpr int kWN = EV == EV_QKV ? 2 : 4;
    static bool lds_set = false;   // allow 128 KB of dynamic LDS (once per instantiation)
    if (!lds_set) {
        (void)hipFuncSetAttribute((const void*)gemm_large_kernel<I8, EV, kWN, W4, SUB>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)L_LDS);
        lds_set = true;
    }
    const int C = num_cus();
    if (S && Kb / L_BK > 64) {
        // long K loops: whole tiles, then the jobs of the remainder tiles
        if (full > 0)
            gemm_large_kernel<I8, EV, kWN, W4, SUB><<<(unsigned)std::min<int64_t>(C, full), L_THREADS, L_LDS, st>>>(
                a, lda_b, w, M, N, Kb, ep, LargePlan{(int32_t)full, (int32_t)full, 0, 0});
        gemm_large_kernel<I8, EV, kWN, W4, SUB><<<(unsigned)(r * S), L_THREADS, L_LDS, st>>>(
            a, lda_b, w, M, N, Kb, ep, LargePlan{0, (int32_t)full, r, S});
    } else {
        // persistent: at most one workgroup per compute unit, and one for
        // each remainder job (r * S <= C)
        const int64_t G = std::min<int64_t>(C, std::max<int64_t>(full > 0 ? tiles : 0, (int64_t)r * S));
        gemm_large_kernel<I8, EV, kWN, W4, SUB><<<(unsigned)(G > 0 ? G : std::min<int64_t>(C, tiles)), L_THREADS,
                                                  L_LDS, st>>>(a, lda_b, w, M, N, Kb, ep,
                                                               LargePlan{(int32_t)full, (int32_t)full, r, S});
    }
    if (SUB == 0 && S) split_reduce_kernel<I8, EV><<<(unsigned)(r * 16), 256, 0, st>>>(M, N, ep, (int32_t)full, S);
}

// Sub-tiles for the r tiles of a partial last round after at least one whole
// round: 128 x 128 (4 jobs per tile) when that gives between C/2 and C jobs,
// else 0 (K-split, or a plain partial round).  Measured on the 1024px block
// (same-process A/B against the K-split): MLP up (r = 64) 253.7 -> 244.1 us;
// 64 x 64 sub-tiles for out / down (r = 16) were 12 and 34 us slower, and the
// QKV epilogue's 8 x 1 wave grid on 128 x 128 sub-tiles 13 us slower (one A
// and eight B fragment reads per eight MFMAs).
static int remainder_subtiles(int64_t tiles, int ev, bool w4) {
    const int64_t C = num_cus(), R = tiles / C, r = tiles - R * C;
    if (w4 || ev == EV_QKV || R < 1 || r == 0) return 0;
    return 4 * r <= C && 8 * r >= C ? 2 : 0;
}

template <bool I8, int EV, bool W4 = false>
static void launch_mfma(const uint8_t* a, int64_t lda_b, const uint8_t* w, int64_t M, int64_t N, int64_t Kb,
                        const EpiParams& ep, hipStream_t st) {
    if (W4 || takes_large(M, N, lda_b, Kb, ep.split_partial != nullptr)) {
        const int64_t tiles = large_grid(M, N);
        const int sub = remainder_subtiles(tiles, EV, W4);
        if constexpr (!W4) {
            if constexpr (EV != EV_QKV) {
                if (sub) {
                    const int64_t full = tiles / num_cus() * num_cus();
                    launch_large<I8, EV, W4, 2>(a, lda_b, w, M, N, Kb, ep, st, tiles, full, (int32_t)(tiles - full),
                                                4);
                    return;
                }
            }
        }
        int64_t full = tiles;
        const int S = plan_split(tiles, (int)(Kb / L_BK), ep, &full);
        const int32_t r = S ? (int32_t)(tiles - full) : 0;
        launch_large<I8, EV, W4, 0>(a, lda_b, w, M, N, Kb, ep, st, tiles, full, r, S);
    }
    else if constexpr (EV == EV_QKV) {
        // store the QKV output, then the separate norm/RoPE kernel
        EpiParams e = ep;
        e.kind = EPI_STORE;
        e.y_bf16 = 1;
        gemm_mfma_kernel<I8, EV_STORE><<<gemm_grid(M, N), NTHREADS, 0, st>>>(a, lda_b, w, M, N, Kb, e);
        (void)launch_qk_norm_rope(ep.y, true, M, (int)(ep.D / 128), ep.g_q, ep.g_k, ep.cos_t, ep.sin_t, ep.qk_eps,
                                  ep.q_out, ep.k_out, ep.D, ep.v_out, ep.D, st);
    } else
        gemm_mfma_kernel<I8, EV><<<gemm_grid(M, N), NTHREADS, 0, st>>>(a, lda_b, w, M, N, Kb, ep);
}

template <bool I8>
static void launch_mfma_any(const uint8_t* a, int64_t lda_b, const uint8_t* w, int64_t M, int64_t N, int64_t Kb,
                            const EpiParams& ep, hipStream_t st) {
    if constexpr (!I8) {
        if (ep.w_mx_scale != nullptr) {
            switch (variant(ep)) {
                case EV_GELU: launch_mfma<false, EV_GELU, true>(a, lda_b, w, M, N, Kb, ep, st); break;
                case EV_QKV: launch_mfma<false, EV_QKV, true>(a, lda_b, w, M, N, Kb, ep, st); break;
                case EV_RESID: launch_mfma<false, EV_RESID, true>(a, lda_b, w, M, N, Kb, ep, st); break;
                default: launch_mfma<false, EV_STORE, true>(a, lda_b, w, M, N, Kb, ep, st); break;
            }
            return;
        }
    }
    switch (variant(ep)) {
        case EV_STORE: launch_mfma<I8, EV_STORE>(a, lda_b, w, M, N, Kb, ep, st); break;
        case EV_STORE_ACC: launch_mfma<I8, EV_STORE_ACC>(a, lda_b, w, M, N, Kb, ep, st); break;
        case EV_GELU: launch_mfma<I8, EV_GELU>(a, lda_b, w, M, N, Kb, ep, st); break;
        case EV_QKV: launch_mfma<I8, EV_QKV>(a, lda_b, w, M, N, Kb, ep, st); break;
        default: launch_mfma<I8, EV_RESID>(a, lda_b, w, M, N, Kb, ep, st); break;
    }
}

hipError_t launch_gemm_i8(const int8_t* a, const int8_t* w, int64_t M, int64_t N, int64_t K,
                          const EpiParams& ep, hipStream_t st) {
    if (M == 0) return hipSuccess;
    launch_mfma_any<true>((const uint8_t*)a, K, (const uint8_t*)w, M, N, K, ep, st);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const void* a, int64_t lda, const void* w, int64_t M, int64_t N,
                            int64_t K, const EpiParams& ep, hipStream_t st) {
    if (M == 0) return hipSuccess;
    launch_mfma_any<false>((const uint8_t*)a, lda * 2, (const uint8_t*)w, M, N, K * 2, ep, st);
    return hipGetLastError();
}

// ---------------------------------------------------------------- fp32 GEMM
// 64x64 tile, 256 threads, 4x4 outputs per thread, K step 16, plain FMA.
template <int EV>
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
            if (m < M && n < N) epilogue<EV>(ep, m, n, acc[i][j], 0);
        }
}

hipError_t launch_gemm_f32(const float* a, int64_t lda, const float* w, int64_t M, int64_t N,
                           int64_t K, const EpiParams& ep, hipStream_t st) {
    if (M == 0) return hipSuccess;
    dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    switch (variant(ep)) {
        case EV_GELU: gemm_f32_kernel<EV_GELU><<<grid, 256, 0, st>>>(a, lda, w, M, N, K, ep); break;
        case EV_RESID: gemm_f32_kernel<EV_RESID><<<grid, 256, 0, st>>>(a, lda, w, M, N, K, ep); break;
        default: gemm_f32_kernel<EV_STORE><<<grid, 256, 0, st>>>(a, lda, w, M, N, K, ep); break;
    }
    return hipGetLastError();
}

}  // namespace dit
