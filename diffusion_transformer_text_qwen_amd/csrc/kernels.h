// Internal launchers (host side) of the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "common.h"

namespace dit {

enum EpiKind : int32_t { EPI_STORE = 0, EPI_GELU = 1, EPI_RESID = 2, EPI_QKV_ROPE = 3 };

// What the GEMM does with each output element v = acc (fp32 or bf16 GEMM) or
// v = acc * a_scale[m] * w_scale[n] (int8 GEMM), after adding bias[n]:
//   EPI_STORE: y[m, n] = v (bf16-rounded if y_bf16); acc_out[m, n] = int32 acc.
//   EPI_GELU:  u = round(v); y[m, n] = round(GELU_tanh(u)).
//   EPI_RESID: y = round(v); x[m, n] = round(x[m, n] + gate[set(m)][n] * y).
//   EPI_QKV_ROPE (bf16 storage; N = 3 D, D % 256 == 0): y = round(v) is the
//     [q | k | v] row of the QKV linear; per 128-wide head of q and k:
//     RMSNorm, cast, gain, cast, RoPE (cos/sin row m), cast; then q -> q_out,
//     k -> k_out, v -> v_out (row stride D).  Shapes the large-tile kernel does
//     not take store y to the y scratch and run the separate norm/RoPE kernel.
// round() is bf16 rounding when act_bf16, identity in fp32 mode.
struct EpiParams {
    int32_t kind;
    int32_t act_bf16;      // bf16 storage semantics for rounding and x
    int32_t y_bf16;        // output dtype of EPI_STORE / EPI_GELU
    const float* a_scale;  // int8 GEMM only
    const float* w_scale;
    const float* bias;     // may be NULL
    void* y;
    int64_t ldy;
    int32_t* acc_out;      // may be NULL
    int64_t ldacc;
    void* x;               // EPI_RESID
    int64_t ldx;
    const float* gate;     // gate row of modulation set 0; set s at gate + s * gate_stride
    int64_t gate_stride;
    SegMap sm;
    // Remainder split-K scratch (int8 GEMM only; NULL = no split): int32
    // partial tiles of the split launch, read back by the reduce launch.
    int32_t* split_partial;
    int64_t split_bytes;   // capacity of split_partial in bytes
    // EPI_QKV_ROPE
    void* q_out;
    void* k_out;
    void* v_out;
    const float* g_q;
    const float* g_k;
    const float* cos_t;    // [M, 64]
    const float* sin_t;
    float qk_eps;
    int64_t D;
    // Asymmetric int8 activations (NULL = symmetric): the int32 sum becomes
    // acc - a_zero[m] * w_sum[n] before scaling.
    const int32_t* a_zero;
    const int32_t* w_sum;
    // EPI_GELU only (NULL = none): multiply GELU(v) by this bf16 [M, ldgm]
    // tensor (the gated MLP's proj output).
    const void* gmul;
    int64_t ldgm;
    // bf16 GEMM only (NULL = bf16 weights): W holds MXFP4 codes [N, K/2] and
    // these are its E8M0 scales [N, K/32], decoded in the operand staging.
    // Only shapes that gemm_bf16_direct_mxfp4 accepts.
    const uint8_t* w_mx_scale;
};

// Bytes of split scratch the int8 GEMM may use for any shape: at most C tiles x
// 256 x 256 int32 (r * S <= C with C = 256 compute units).
constexpr int64_t kSplitPartialBytes = (int64_t)256 * 256 * 256 * 4;

hipError_t launch_gemm_i8(const int8_t* a, const int8_t* w, int64_t M, int64_t N, int64_t K,
                          const EpiParams& ep, hipStream_t st);
hipError_t launch_gemm_bf16(const void* a, int64_t lda, const void* w, int64_t M, int64_t N,
                            int64_t K, const EpiParams& ep, hipStream_t st);
// Whether the bf16 GEMM of this shape runs on the large-tile kernel, which can
// decode MXFP4 weights in its operand staging (ep.w_mx_scale).
bool gemm_bf16_direct_mxfp4(int64_t M, int64_t N, int64_t K, int64_t lda, bool can_split);
hipError_t launch_gemm_f32(const float* a, int64_t lda, const float* w, int64_t M, int64_t N,
                           int64_t K, const EpiParams& ep, hipStream_t st);

hipError_t launch_quantize_rows(const void* x, bool bf16, int64_t M, int64_t K, int64_t ldx,
                                int8_t* q, float* scale, hipStream_t st);
hipError_t launch_quantize_rows_asym(const void* x, bool bf16, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                     float* scale, int32_t* zero, hipStream_t st);
hipError_t launch_mxfp4_expand(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, void* out,
                               hipStream_t st);
hipError_t launch_int8_colsum(const int8_t* w, int64_t N, int64_t K, int32_t* out, hipStream_t st);
// g = bf16(GELU_tanh(u)) of bf16 u [M, K] (row stride ldu, 0 = K), quantized per
// row; g_out (bf16 [M, K], row stride K) also receives g when not NULL (K <= 16384).
hipError_t launch_gelu_quantize_rows(const void* u, int64_t M, int64_t K, int8_t* q, float* scale,
                                     hipStream_t st, int64_t ldu = 0, void* g_out = nullptr);
// h (if not NULL) and/or the int8 codes of h (qo, qs; if qo is not NULL).
hipError_t launch_adaln(const void* x, bool bf16, int64_t M, int64_t D, const float* shift,
                        const float* scale, int64_t mod_stride, const SegMap& sm, float eps, void* h, int8_t* qo,
                        float* qs, hipStream_t st);
// bf16 x, D <= 4096: h (if not NULL) and the asymmetric int8 codes of h
// (qo, qs, zero points qz), as launch_quantize_rows_asym would form them from h.
bool adaln_fuses_asym(int64_t D, int64_t mod_stride, const void* x, const void* shift, const void* scale,
                      const void* h, const void* qo);
hipError_t launch_adaln_asym(const void* x, int64_t M, int64_t D, const float* shift, const float* scale,
                             int64_t mod_stride, const SegMap& sm, float eps, void* h, int8_t* qo, float* qs,
                             int32_t* qz, hipStream_t st);
hipError_t launch_adaln_small(const void* x, bool bf16, int64_t M, int64_t D, const float* shift,
                              const float* scale, int64_t mod_stride, const SegMap& sm, float eps, void* h, int8_t* qo,
                              float* qs, hipStream_t st);
hipError_t launch_qk_norm_rope(const void* qkv, bool bf16, int64_t T, int H, const float* g_q,
                               const float* g_k, const float* cos_t, const float* sin_t, float eps,
                               void* q_out, void* k_out, int64_t ldk, void* v_out, int64_t ldv,
                               hipStream_t st);
hipError_t launch_rope_tables(int32_t text_len, const int32_t* grids, int32_t n_img, int64_t row0,
                              int64_t T_rows, float theta, float* cos_out, float* sin_out,
                              hipStream_t st);
hipError_t launch_cast(const void* x, bool x_bf16, void* y, bool y_bf16, int64_t n, hipStream_t st);
hipError_t launch_euler(float* x, const void* v, bool bf16, int64_t n, float sigma, float sigma_next,
                        hipStream_t st);

// Attention: kv_end[s] = end position of segment s (keys [0, kv_end[seg]) are
// visible to a query of segment seg).
struct AttnSegs {
    int64_t end[kMaxSeg];
    int32_t n;
};
// Keys visible to a query at absolute position pos: [0, end of its segment).
// Static indices only (keeps the argument struct out of private memory).
__device__ __forceinline__ int64_t kv_end_of(const AttnSegs& sg, int64_t pos) {
    int64_t e = sg.end[0];
#pragma unroll
    for (int s = 0; s < kMaxSeg - 1; ++s)
        if (s < sg.n - 1 && pos >= sg.end[s]) e = sg.end[s + 1];
    return e;
}
hipError_t launch_attention_bf16(const void* q, const void* k, const void* v, void* o, int64_t T_q,
                                 int64_t T_k, int H, int64_t ldq, int64_t ldk, int64_t ldv,
                                 int64_t ldo, const AttnSegs& segs, float sm_scale, hipStream_t st);
hipError_t launch_attention_f32(const float* q, const float* k, const float* v, float* o, int64_t T_q,
                                int64_t T_k, int H, int64_t ldq, int64_t ldk, int64_t ldv,
                                int64_t ldo, const AttnSegs& segs, float sm_scale, hipStream_t st);

// Int8 / fp8 attention operands: one buffer holding, at the offsets below,
// q8 [H][T_q][128] int8, q_scale [H][T_q] f32, k8 [H][nt][64 x 128] int8 tile
// images, k_scale [H][nt] f32, v8 [H][nt][128 x 64] e4m3 tile images,
// v_scale [H][128] f32 and v_amax [H][128] u32 (scratch); nt = ceil(T_k/64).
struct AttnQ8Layout {
    size_t q8, sq, k8, sk, v8, sv, vamax, total;
    int64_t nt;
};
AttnQ8Layout attn_q8_layout(int64_t T_q, int64_t T_k, int H);
// with_q = false leaves the Q parts of the buffer unwritten (the attention
// kernel then quantizes bf16 Q itself: launch_attention_q8 with q_bf16).
hipError_t launch_attn_quantize(const void* q, const void* k, const void* v, int64_t T_q, int64_t T_k, int H,
                                int64_t ldq, int64_t ldk, int64_t ldv, void* buf, hipStream_t st,
                                bool with_q = true);
// q_bf16 != NULL: Q is read as bf16 [T_q, H, 128] (row stride ldq) and
// quantized in the kernel exactly as the buffer's Q codes would be.
hipError_t launch_attention_q8(const void* buf, int64_t T_q, int64_t T_k, int H, void* o, int64_t ldo,
                               const AttnSegs& segs, float sm_scale, hipStream_t st,
                               const void* q_bf16 = nullptr, int64_t ldq = 0);

}  // namespace dit
