/*
 * dit.h - C ABI of the MI355X (gfx950) single-stream DiT block library.
 *
 * The block is the one every denoise step of Qwen-Image-2.1 runs 32 times: a
 * 4096-wide single-stream DiT block over a [text | reference | target] token
 * sequence ("RGBA-Image-2.1 - Core AI port of Qwen-Image-2.1", intro and Graph
 * contracts; "qwen-image-mnn", What runs where).
 *
 * Conventions shared by every entry point
 *  - Device pointers are plain device addresses (hipMalloc'd or torch tensors);
 *    "host" arguments are ordinary host memory.  The caller owns every buffer.
 *  - Matrices are row-major.  Weights are [N, K] with K contiguous (one output
 *    channel per row).  bf16 data is IEEE bfloat16 (uint16 storage).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *    work on it: no allocation, no synchronization, so they can be captured
 *    into a HIP graph.
 *  - Every argument is checked before the first HIP call; an invalid call
 *    returns a DIT_E_* code and launches nothing ("Qwen_Image-2.1-MXFP4-Paiton",
 *    Tested operating limits: unsupported settings are rejected before GPU
 *    execution).  DIT_E_HIP reports a failed launch.  dit_last_error() gives a
 *    thread-local description of the last failure.  Nothing throws or aborts.
 *  - Results are deterministic: the same inputs give bitwise-equal outputs.
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIT_ABI_VERSION 5

typedef enum {
    DIT_OK = 0,
    DIT_E_NULL = 1,         /* a required pointer is NULL */
    DIT_E_SHAPE = 2,        /* inconsistent or out-of-range sizes */
    DIT_E_DTYPE = 3,        /* dtype or mode not accepted here */
    DIT_E_ALIGN = 4,        /* pointer or stride not 16-byte aligned */
    DIT_E_UNSUPPORTED = 5,  /* valid, but outside the supported set */
    DIT_E_WORKSPACE = 6,    /* workspace NULL or too small */
    DIT_E_HIP = 7           /* a HIP launch failed */
} dit_status_t;

typedef enum { DIT_F32 = 0, DIT_BF16 = 1, DIT_I8 = 2, DIT_I32 = 3 } dit_dtype_t;

typedef enum {
    DIT_MODE_F32 = 0,   /* everything fp32 */
    DIT_MODE_BF16 = 1,  /* bf16 tensors, fp32 statistics/accumulators/softmax */
    DIT_MODE_W8A8 = 2   /* bf16 mode with the four linears W8A8 */
} dit_mode_t;

int dit_abi_version(void);
const char* dit_status_string(int status);
const char* dit_last_error(void);

/*
 * Symmetric per-row int8 quantization ("Qwen-Image-2.1 W8A8 - FlagOS for Mac",
 * Quantization and validation: dynamic per-token activations, per-output-channel
 * weights, fp32 scales, zero point 0).  For each row m of x [M, K] (row stride ldx
 * elements, dtype DIT_BF16 or DIT_F32): s = amax/127 (fp32), q = clamp(rint(x/s),
 * -127, 127) with IEEE fp32 division and ties to even; an all-zero row gives s = 0
 * and q = 0.  q [M, K] int8 (row stride K), scale [M] fp32.
 * Supported: 1 <= K <= 32768 (bf16) or 16384 (f32), K % 8 == 0, ldx % 8 == 0,
 * 16-byte aligned x and q.
 */
int dit_quantize_rows(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                      int8_t* q, float* scale, void* stream);

/*
 * GELU fused into the per-row quantization of the MLP activation (the W8A8
 * block's MLP-down input).  g = bf16(GELU_tanh(u)) with the tanh form
 * 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))) evaluated in fp32
 * ("qwen-image-mnn" and the Core AI port name a GELU MLP; the tanh form is the
 * workloads' choice), then the codes of g exactly as dit_quantize_rows.
 * u [M, K] bf16 (row stride ldu elements); q [M, K] int8 (row stride K); scale
 * [M] fp32; g_out (NULL or bf16 [M, K], row stride K) also receives g, the
 * values the codes are taken from.  Supported: K % 8 == 0, ldu % 8 == 0,
 * K <= 16384, 16-byte aligned u, q and g_out.
 */
int dit_gelu_quantize_rows(const void* u, int64_t M, int64_t K, int64_t ldu, int8_t* q, float* scale,
                           void* g_out, void* stream);

/*
 * W8A8 linear ("Qwen-Image-2.1 W8A8 - FlagOS for Mac", Quantization and
 * validation: int8 x int8 with int32 accumulation, fp32 scaling, bf16 output).
 *   y[m, n] = float(sum_k a[m,k] * w[n,k]) * a_scale[m] * w_scale[n] + bias[n]
 * a [M, K] int8 (row stride K), w [N, K] int8 (row stride K), a_scale [M],
 * w_scale [N], bias [N] fp32 or NULL.  y [M, N] with row stride ldy, dtype
 * DIT_BF16 (rounded to nearest even) or DIT_F32.  If acc_out is not NULL the
 * exact int32 sums are also stored there ([M, N], row stride N).
 * workspace (device, may be NULL): scratch of workspace_bytes >=
 * w8a8_linear_workspace_bytes() lets the kernel split the K range of the tiles
 * of a partially filled last round across workgroups (exact: int32 partial
 * sums); its contents need not be initialized and are left unspecified.
 * Supported: K % 128 == 0, N % 16 == 0, K <= 133144 (so K*127^2 < 2^31).
 */
size_t w8a8_linear_workspace_bytes(void);
int w8a8_linear(const int8_t* a, const float* a_scale, int64_t M, int64_t K,
                const int8_t* w, const float* w_scale, const float* bias, int64_t N,
                void* y, int y_dtype, int64_t ldy, int32_t* acc_out, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * w8a8_linear for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same linear, the
 * same arguments without the workspace, bitwise-equal results.  The K-split
 * partial sums go to the library's own device scratch, a static array of
 * 32 MiB per GPU (held until the process ends); a launch whose split would
 * need more takes fewer K ranges.  The scratch is fully written before it is
 * read, so it needs no clearing; it is shared by every call on one GPU, so
 * calls that overlap on one GPU (different streams or threads) race.  The
 * first call on each device looks up the scratch address (no allocation,
 * library call or memset otherwise).  Errors as w8a8_linear.
 */
int w8a8_linear_noalloc(const int8_t* a, const float* a_scale, int64_t M, int64_t K,
                        const int8_t* w, const float* w_scale, const float* bias, int64_t N,
                        void* y, int y_dtype, int64_t ldy, int32_t* acc_out, void* stream);

/*
 * Asymmetric per-row int8 quantization ("Qwen-Image-2.1 W8A8 - FlagOS for Mac",
 * Quantization and validation: dynamic asymmetric INT8 activations per token,
 * fp32 scales).  The page gives no formula; reading: the row's range widened to
 * contain 0, lo = min(row, 0), hi = max(row, 0); scale = fp32(hi - lo) / 255,
 * zero point z = -128 - rint(lo / scale) (in [-128, 127]),
 * q = clamp(rint(x / scale) + z, -128, 127), IEEE fp32 divisions, ties to even;
 * a code stands for (q - z) * scale; an all-zero row gives scale 0, z 0, q 0.
 * x [M, K] bf16|f32 (row stride ldx); q [M, K] int8 (row stride K); scale [M]
 * fp32; zero [M] int32.  Supported: K % 8 == 0, ldx % 8 == 0, 16-byte aligned x, q.
 */
int dit_quantize_rows_asym(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                           float* scale, int32_t* zero, void* stream);

/* out[n] = sum_k w[n, k] for int8 w [N, K] (row stride K): the row sums a GEMM
 * over zero-point activation codes subtracts (z[m] * out[n]).  K % 16 == 0. */
int dit_int8_colsum(const int8_t* w, int64_t N, int64_t K, int32_t* out, void* stream);

/*
 * w8a8_linear over asymmetric activation codes (dit_quantize_rows_asym):
 *   y[m, n] = float(sum_k a[m,k] w[n,k] - a_zero[m] * w_sum[n]) * a_scale[m] * w_scale[n] + bias[n]
 * with w_sum from dit_int8_colsum (16-byte aligned).  a_zero == NULL is
 * w8a8_linear.  Supported as w8a8_linear, with K <= 65536 (255*127*K < 2^31).
 */
int w8a8_linear_asym(const int8_t* a, const float* a_scale, const int32_t* a_zero, int64_t M, int64_t K,
                     const int8_t* w, const float* w_scale, const int32_t* w_sum, const float* bias, int64_t N,
                     void* y, int y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/*
 * bf16 linear for the non-quantized linears ("Qwen-Image-2.1 W8A8 - FlagOS for
 * Mac", Quantization and validation: the linears outside the W8A8 set stay
 * BF16; "qwen-image-mnn", Install / run: no fp16 arithmetic on this path):
 * y = a w^T + bias with fp32 accumulation.  a [M, K] bf16 (row stride lda), w [N, K] bf16 (row stride K),
 * bias [N] fp32 or NULL, y [M, N] bf16 or fp32 (row stride ldy).
 * Supported: K % 64 == 0, N % 16 == 0, lda % 8 == 0.
 */
int bf16_linear(const void* a, int64_t M, int64_t K, int64_t lda, const void* w,
                const float* bias, int64_t N, void* y, int y_dtype, int64_t ldy, void* stream);

/*
 * fp32 linear, the fp32 mode's linears ("Qwen Image 2.1 native qualification",
 * Numerical checks: the fp32 re-implementation checked against the reference
 * at fine tolerances): y = a w^T + bias, fp32 throughout.  a [M, K] f32
 * (row stride lda), w [N, K] f32, y [M, N] f32 (row stride ldy).
 * Supported: K % 16 == 0, N % 16 == 0.
 */
int f32_linear(const float* a, int64_t M, int64_t K, int64_t lda, const float* w,
               const float* bias, int64_t N, float* y, int64_t ldy, void* stream);

/*
 * The block's QKV linear with its fused epilogue (the path dit_block_forward
 * runs in the bf16 and W8A8 modes): [q | k | v] = a w^T + bias, rounded to
 * bf16; per token and 128-wide head of q and k the RMSNorm of
 * dit_qk_norm_rope with the cast to bf16 before the gain multiply ("Qwen Image
 * 2.1 native qualification", Numerical checks), then the interleaved RoPE
 * rotation by cos_t/sin_t [T, 64] ("RGBA-Image-2.1 - Core AI port", Graph
 * contracts), rounded to bf16; v passes through.
 * mode DIT_MODE_W8A8: a int8 codes [T, D] with a_scale [T], w int8 [3D, D] with
 * w_scale [3D] (the linear of w8a8_linear); mode DIT_MODE_BF16: a bf16 [T, D],
 * w bf16 [3D, D], scales unused.  D = H*128.  bias [3D] fp32 or NULL; g_q, g_k
 * [128] fp32.  q_out, k_out, v_out: bf16 [T, D] each (row stride D; k_out and
 * v_out may be the rows [T_k - T, T_k) of a [T_k, H, 128] K/V cache).
 * workspace: dit_qkv_linear_workspace_bytes(T, H) bytes of device scratch
 * (K-split partial sums, and the [q|k|v] rows of the launches that store them
 * before a separate norm/RoPE pass); contents need not be initialized.
 * Supported: D % 256 == 0, D <= 8192, T * 3D < 2^31; every pointer 16-byte
 * aligned.
 */
size_t dit_qkv_linear_workspace_bytes(int64_t T, int32_t H);
int dit_qkv_linear(int mode, const void* a, const float* a_scale, int64_t T, int32_t H, const void* w,
                   const float* w_scale, const float* bias, const float* g_q, const float* g_k, const float* cos_t,
                   const float* sin_t, float eps, void* q_out, void* k_out, void* v_out, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Block-causal attention ("RGBA-Image-2.1 - Core AI port", intro; "qwen-image-mnn",
 * What runs where).  Keys are split into n_seg consecutive segments of lengths
 * seg_len[] (host array, sum = T_k).  Query row i sits at absolute position
 * T_k - T_q + i (so the first T_k - T_q keys may come from a prefix cache) and may
 * attend key j iff segment(j) <= segment(T_k - T_q + i): each segment sees itself
 * and every earlier one.  Per head h:
 *   o[i, h, :] = sum_j softmax_j(sm_scale * q[i,h,:].k[j,h,:]) v[j,h,:]
 * q [T_q, H, d], k and v [T_k, H, d], o [T_q, H, d]; ldq/ldk/ldv/ldo are row
 * strides in elements between consecutive tokens (>= H*d).  dtype DIT_BF16
 * (fp32 softmax, bf16 P for the PV product, bf16 output) or DIT_F32.
 * sm_scale <= 0 means 1/sqrt(d).  Supported: d == 128, 1 <= T_q <= T_k,
 * 1 <= n_seg <= 16, strides % 8 == 0.
 */
int block_causal_attention(const void* q, const void* k, const void* v, void* o, int dtype,
                           int64_t T_q, int64_t T_k, int32_t H, int32_t d, int64_t ldq,
                           int64_t ldk, int64_t ldv, int64_t ldo, const int32_t* seg_len,
                           int32_t n_seg, float sm_scale, void* stream);

/*
 * Int8 / fp8 attention ("Qwen_Image-2.1-MXFP4-Paiton", Runtime precision and
 * quality: after the first denoising steps the runtime runs attention in
 * int8/fp8; the page names only the formats).  Reading:
 *   q: int8 symmetric per (token, head), scale amax/127;
 *   k: int8 symmetric per (tile of 64 consecutive keys, head), scale amax/127;
 *   v: e4m3 per (head, channel) over all T_k keys, scale amax/448;
 *   codes by an IEEE fp32 division, round half to even (v saturates at 448);
 *   scores = exact int32 dot products times sm_scale and the q and k scales;
 *   P = exp of the score minus a running row maximum, raised lazily so that
 *   every P is at most 2^8 when formed (earlier sums are rescaled when it
 *   rises), rounded to e4m3 for the P V product; the softmax normalizer sums
 *   the unrounded P; o is bf16.
 *
 * dit_attn_q8_bytes: size of the operand buffer for (T_q, T_k, H); if
 * offsets != NULL writes the byte offsets of its 7 parts (256-aligned):
 *   [0] q8      int8 [H][T_q][128]
 *   [1] q_scale f32  [H][T_q]
 *   [2] k8      int8 [H][nt][64][128], nt = ceil(T_k / 64): per (head, tile) an
 *               8 KB image, key r's 16-byte chunk c (dims 16c..16c+15) at byte
 *               r*128 + 16*(c ^ (r & 7)); keys past T_k are 0
 *   [3] k_scale f32  [H][nt]
 *   [4] v8      e4m3 [H][nt][128][64]: per (head, tile) an 8 KB image, channel
 *               row ch at byte ch*64; position p = 32*g + b (g = 0, 1;
 *               b = 0..31) holds key (b/16)*32 + (b%4) + 8*((b%16)/4) + 4*g of
 *               the tile, and 16-byte chunk c of the row sits at chunk
 *               c ^ ((ch >> 1) & 3); keys past T_k are 0
 *   [5] v_scale f32  [H][128]
 *   [6] scratch u32  [H][128] (channel amax)
 *
 * dit_attn_quantize: fills the buffer from bf16 q [T_q, H, 128] and the bf16
 * K/V cache [T_k, H, 128] (row strides ldq/ldk/ldv in elements, % 8 == 0,
 * 16-byte aligned); buf_bytes >= dit_attn_q8_bytes.  Enqueued on `stream`
 * (no allocation, no memset).
 *
 * block_causal_attention_q8: o [T_q, H, 128] bf16 (row stride ldo) from the
 * buffer, block-causal over seg_len as block_causal_attention.  sm_scale <= 0
 * means 1/sqrt(128).  Supported: 1 <= H <= 65535, 0 <= T_q <= T_k < 2^31,
 * H * nt * 8192 < 2^31, 1 <= n_seg <= 16.
 */
size_t dit_attn_q8_bytes(int64_t T_q, int64_t T_k, int32_t H, int64_t* offsets);
int dit_attn_quantize(const void* q, const void* k, const void* v, int64_t T_q, int64_t T_k, int32_t H,
                      int64_t ldq, int64_t ldk, int64_t ldv, void* buf, size_t buf_bytes, void* stream);
int block_causal_attention_q8(const void* buf, int64_t T_q, int64_t T_k, int32_t H, void* o, int64_t ldo,
                              const int32_t* seg_len, int32_t n_seg, float sm_scale, void* stream);

/*
 * 3-axis RoPE tables ("RGBA-Image-2.1 - Core AI port", Graph contracts, RoPE).
 * Sequence = [text (text_len tokens) | image 0 | image 1 | ...]; image k is a
 * grids[2k] x grids[2k+1] (h x w) latent grid in raster order (host array).
 * Positions: text token i -> (i, i, i); image k token (y, x) -> (text_len + k,
 * y - (h - h/2), x - (w - w/2)) with integer halving.  Head-dim pairs 0..15 use
 * the frame position, 16..39 the height, 40..63 the width; pair j of an axis
 * with dim d_a (32, 48, 48) turns by pos * theta^(-2j/d_a).  Writes
 * cos/sin [T_rows, 64] fp32 for sequence rows [row0, row0 + T_rows) (angles in
 * fp64, rounded once to fp32).  Supported: n_img <= 15.
 */
int dit_rope_tables(int32_t text_len, const int32_t* grids, int32_t n_img, int64_t row0,
                    int64_t T_rows, float theta, float* cos_out, float* sin_out, void* stream);

/*
 * Q/K RMSNorm + RoPE, the QKV epilogue of the block ("Qwen Image 2.1 native
 * qualification", Numerical checks: the normalized value is cast to the gain's
 * dtype before the gain multiply).  qkv [T, 3*H*128] (row stride 3*H*128) holds
 * the linear output [q | k | v].  Per token and head:
 *   n = t / sqrt(mean(t^2) + eps); bf16 mode: n -> bf16, n*g -> bf16; then the
 *   interleaved pair rotation by cos/sin [T, 64]; bf16 mode rounds once more.
 * Writes q_out [T, H*128], k_out and v_out (row strides ldk, ldv, e.g. rows of a
 * K/V cache).  dtype DIT_BF16 or DIT_F32 for all tensors; g_q, g_k [128] fp32.
 */
int dit_qk_norm_rope(const void* qkv, int dtype, int64_t T, int32_t H, const float* g_q,
                     const float* g_k, const float* cos_t, const float* sin_t, float eps,
                     void* q_out, void* k_out, int64_t ldk, void* v_out, int64_t ldv,
                     void* stream);

/*
 * adaLN prologue ("qwen-image-mnn", What runs where: timestep modulation rows
 * shift and scale the normalized tokens): h = LayerNorm(x) * (1 + scale) + shift
 * (no affine, biased variance, fp32 statistics) with one (shift, scale) pair [D]
 * fp32 for all rows.  x [M, D] bf16 or f32 (row stride D).  Outputs (at least
 * one): h [M, D] when h_out is not NULL (h_dtype must equal x_dtype; bf16
 * rounds once), and, when q_out is not NULL, that same h (bf16-rounded in bf16)
 * quantized per row as in dit_quantize_rows (q_out [M, D] int8, q_scale [M]).
 * Supported: D % 256 == 0, D <= 8192; x, h_out and q_out 16-byte aligned.
 */
int dit_adaln_modulate(const void* x, int x_dtype, int64_t M, int64_t D, const float* shift,
                       const float* scale, float eps, void* h_out, int h_dtype, int8_t* q_out,
                       float* q_scale, void* stream);

/*
 * The adaLN prologue with the activation codes of the W8A8 recipe ("Qwen-Image-2.1
 * W8A8 - FlagOS for Mac", Quantization and validation: dynamic asymmetric
 * per-token int8 activations): h as in dit_adaln_modulate (bf16 x, bf16 h),
 * written to h_out when it is not NULL, and h quantized per row exactly as
 * dit_quantize_rows_asym quantizes it (q_out [M, D] int8, q_scale [M] fp32,
 * q_zero [M] int32), in one pass over x.  Supported: D % 256 == 0, D <= 4096;
 * x and h_out 16-byte aligned, q_out 8-byte aligned; else DIT_E_UNSUPPORTED or
 * DIT_E_ALIGN before any launch.
 */
int dit_adaln_modulate_asym(const void* x, int64_t M, int64_t D, const float* shift, const float* scale,
                            float eps, void* h_out, int8_t* q_out, float* q_scale, int32_t* q_zero,
                            void* stream);

/* FlowMatch Euler update ("RGBA-Image-2.1 - Core AI port", Graph contracts,
 * Sampler): x[i] += (sigma_next - sigma) * v[i] in fp32; x fp32, v bf16 or f32. */
int dit_euler_step(float* x, const void* v, int v_dtype, int64_t n, float sigma,
                   float sigma_next, void* stream);

/* Element-wise dtype conversion (fp32 <-> bf16, round to nearest even), e.g. the
 * fp32 sampler latent entering a bf16 DiT ("RGBA-Image-2.1 - Core AI port",
 * Graph contracts: fp32 graph inputs and outputs around bf16 compute).
 * x and y may not overlap. */
int dit_cast(const void* x, int x_dtype, void* y, int y_dtype, int64_t n, void* stream);

/* ------------------------------------------------------------------ the block */

typedef struct {
    int32_t mode;       /* dit_mode_t */
    int32_t D;          /* width; D == H * head_dim */
    int32_t H;          /* heads */
    int32_t head_dim;   /* must be 128 */
    int32_t F;          /* MLP width */
    float ln_eps;       /* adaLN LayerNorm eps (1e-6) */
    float qk_eps;       /* Q/K RMSNorm eps (1e-6) */
    int32_t attn_quant; /* 0: bf16/fp32 attention; 1: int8 Q K^T and fp8 P V
                           (block_causal_attention_q8; bf16 and W8A8 modes) */
} dit_block_config;

typedef struct {
    /* [N, K] row-major: int8 codes (W8A8), bf16 (BF16) or f32 (F32).
       w_qkv [3D, D] (q | k | v rows), w_o [D, D], w_1 [F, D], w_2 [D, F]. */
    const void *w_qkv, *w_o, *w_1, *w_2;
    /* per-output-channel fp32 scales (W8A8 only, else NULL) */
    const float *s_qkv, *s_o, *s_1, *s_2;
    /* fp32 biases [3D], [D], [F], [D] */
    const float *b_qkv, *b_o, *b_1, *b_2;
    /* Q/K RMSNorm gains [128] fp32, shared by all heads */
    const float *g_q, *g_k;
} dit_block_weights;

typedef struct {
    void* x;                    /* [T_q, D] in/out, bf16 (f32 in F32 mode) */
    const float* mod;           /* [n_mod, 6, D]: shift1, scale1, gate1, shift2, scale2, gate2 */
    int32_t n_mod;
    const int32_t* mod_of_seg;  /* host [n_seg]: modulation set of each segment */
    const float* cos_t;         /* [T_q, 64] RoPE tables of the computed rows */
    const float* sin_t;
    const int32_t* seg_len;     /* host [n_seg], sum = T_k */
    int32_t n_seg;
    int64_t T_q;                /* rows computed (the last T_q rows of the sequence) */
    int64_t T_k;                /* sequence length */
    void* k_cache;              /* [T_k, H, 128] K (post-norm, post-RoPE); rows [0, T_k-T_q) */
    void* v_cache;              /*   are read, rows [T_k-T_q, T_k) are written by the call */
} dit_block_io;

/*
 * Workspace the block needs for T_q computed rows (bytes, 256-aligned pieces):
 * the intermediate activations, and in the bf16 and W8A8 modes also one region
 * of w8a8_linear_workspace_bytes() for K-split partial sums of the linears
 * (int32 for W8A8, fp32 for bf16).  Contents need not be initialized.
 */
size_t dit_block_workspace_bytes(const dit_block_config* cfg, int64_t T_q, int64_t T_k);

/*
 * One single-stream DiT block ("RGBA-Image-2.1 - Core AI port of Qwen-Image-2.1",
 * intro and Graph contracts: one stream over [text | image] with block-causal
 * attention; "qwen-image-mnn", What runs where: 3-axis RoPE, Q/K RMSNorm and
 * the timestep modulation rows; "Qwen-Image-2.1 W8A8 - FlagOS for Mac",
 * Quantization and validation: the W8A8 linears) on the last T_q rows of a
 * T_k-token sequence:
 *   h  = LN(x)(1+scale1)+shift1;  [q|k|v] = h Wqkv^T + b_qkv
 *   q, k <- RoPE(RMSNorm(q, k) * g);  K/V rows -> cache
 *   o  = block-causal attention(q, K cache, V cache)   (int8/fp8 if cfg->attn_quant)
 *   x1 = x + gate1 * (o Wo^T + b_o)
 *   x  = x1 + gate2 * (GELU_tanh((LN(x1)(1+scale2)+shift2) W1^T + b1) W2^T + b2)
 * Each row uses the modulation set of its segment.  In W8A8 mode the inputs of
 * the four linears are quantized per token (dit_quantize_rows) and the weights
 * are int8 codes with per-output-channel scales.  Supported: head_dim == 128,
 * D == H*128, D % 256 == 0, F % 256 == 0, D <= 8192, 1 <= n_seg <= 16.
 */
int dit_block_forward(const dit_block_config* cfg, const dit_block_weights* w,
                      const dit_block_io* io, void* workspace, size_t workspace_bytes,
                      void* stream);

/* The same block applied n_blocks times in order (one denoise step's stack);
 * weights[b] is block b.  io->x is updated in place; k_cache/v_cache (if not
 * NULL) are arrays of n_blocks per-block caches. */
int dit_stack_forward(const dit_block_config* cfg, const dit_block_weights* weights,
                      int32_t n_blocks, const dit_block_io* io, void* const* k_caches,
                      void* const* v_caches, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * MXFP4 weights ("Qwen_Image-2.1-MXFP4-Paiton", What was quantized and Runtime
 * precision and quality): E2M1 values packed two per byte, element 2i in the
 * low nibble of byte i of its row, and one E8M0 scale per group of 32 input
 * columns: w[n, k] = e2m1(code[n, k]) * 2^(scales[n, k / 32] - 127) (E8M0 255 is
 * NaN).  The runtime reconstructs the weights and computes in bf16; the
 * reconstruction is exact in bf16 while the scaled values stay in its normal
 * range.
 * dit_mxfp4_expand: codes [N, K/2] uint8, scales [N, K/32] uint8 -> w_bf16 [N, K]
 * (row stride K).  K % 32 == 0; codes and w_bf16 16-byte aligned.
 * mxfp4_linear: y = a w^T + bias with w given as MXFP4; a [M, K] bf16 (row
 * stride lda), y bf16|f32 (row stride ldy).  Shapes that fill the GPU with
 * 256 x 256 tiles decode the codes to bf16 in the GEMM's operand staging (the
 * weights cross HBM at 4.25 bits per value; the workspace is not touched);
 * smaller shapes expand the weights into the workspace,
 * mxfp4_linear_workspace_bytes(N, K) bytes, then run the bf16 linear.  Both
 * give bitwise the bf16 linear on the decoded weights.  K % 64 == 0.
 */
int dit_mxfp4_expand(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, void* w_bf16,
                     void* stream);
size_t mxfp4_linear_workspace_bytes(int64_t N, int64_t K);
int mxfp4_linear(const void* a, int64_t M, int64_t K, int64_t lda, const uint8_t* codes, const uint8_t* scales,
                 const float* bias, int64_t N, void* y, int y_dtype, int64_t ldy, void* workspace,
                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ gated-MLP block, per-linear W8A8 */

/*
 * One linear of the gated block ("Qwen-Image-2.1 W8A8 - FlagOS for Mac",
 * Quantization and validation: a mixed W8A8/BF16 transformer in which only some
 * linears run W8A8).  s != NULL: w holds int8 codes [N, K] (symmetric per
 * output channel, scales s [N]) and wsum [N] their row sums (dit_int8_colsum);
 * the activation is quantized asymmetrically per token (dit_quantize_rows_asym).
 * mx_scale != NULL: MXFP4 weights (see dit_mxfp4_expand), decoded in the
 * GEMM's operand staging (or, for shapes too small for the large-tile GEMM,
 * expanded to bf16 in the workspace for the call).  Otherwise w is bf16 [N, K]
 * and wsum is ignored.
 * b: fp32 bias [N] or NULL.
 */
typedef struct {
    const void* w;
    const float* s;
    const int32_t* wsum;
    const float* b;
    const uint8_t* mx_scale;   /* != NULL: w holds MXFP4 codes [N, K/2] and these
                                  E8M0 scales [N, K/32] (dit_mxfp4_expand); s must
                                  be NULL */
} dit_linear;

/*
 * Weights of the gated-MLP block.  The page names Q/K and MLP proj/gate
 * modules, and its checkpoint size implies a gated MLP; reading of the MLP:
 *   u = h2 W_proj^T + b_proj;  t = h2 W_gate^T + b_gate  (each stored bf16)
 *   g = u * GELU_tanh(t)  (stored bf16);  y2 = g W_down^T + b_down
 * qk [2D, D] (q rows, then k rows), v [D, D], o [D, D], proj/gate [F, D],
 * down [D, F]; g_q, g_k [128] fp32 (16-byte aligned).
 */
typedef struct {
    dit_linear qk, v, o, proj, gate, down;
    const float *g_q, *g_k;
} dit_gated_block_weights;

/* Workspace of dit_block_forward_gated (bytes). */
size_t dit_gated_block_workspace_bytes(const dit_block_config* cfg, int64_t T_q, int64_t T_k);

/*
 * The block of dit_block_forward with the gated MLP above and a per-linear
 * choice of W8A8 (the page's recipe: Q/K, proj and gate W8A8 in blocks 2..29
 * of 32, zero-based, everything else bf16; the caller picks per block by
 * passing int8 or bf16 weights).  cfg->mode must be DIT_MODE_BF16 (bf16
 * activations); cfg->F is the gated width; cfg->attn_quant selects the
 * int8/fp8 attention.  io as for dit_block_forward (cos_t, sin_t 16-byte
 * aligned).  Errors before any launch as dit_block_forward.
 */
int dit_block_forward_gated(const dit_block_config* cfg, const dit_gated_block_weights* w, const dit_block_io* io,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ one velocity evaluation */

/*
 * DiT head and tail ([Core AI port, graph contracts]: the DiT maps the packed
 * latent [N, 64] and the text features [L, 4096] to a velocity [N, 64]).  The
 * pages give only these shapes; reading used here: txt_in = Linear(C_txt -> D),
 * img_in = Linear(C_lat -> D), tail = LayerNorm (no affine) of the target rows
 * modulated by (shift, scale) = mod_final, then proj_out = Linear(D -> C_lat).
 * Weights are [out, in] row-major in the activation dtype (bf16 in the bf16
 * and W8A8 modes, f32 in the f32 mode); biases are fp32 (NULL = none).
 * Caller-owned device memory; not modified.
 */
typedef struct {
    const void* w_txt_in;       /* [D, C_txt] */
    const float* b_txt_in;      /* [D] */
    const void* w_img_in;       /* [D, C_lat] */
    const float* b_img_in;      /* [D] */
    const void* w_proj_out;     /* [C_lat, D] */
    const float* b_proj_out;    /* [C_lat] */
    int32_t C_txt;              /* multiple of 64 */
    int32_t C_lat;              /* multiple of 64 */
} dit_head_weights;

/*
 * The sequence is [text (L_txt) | reference image (R) | target image (N)],
 * T_k = L_txt + R + N = sum(seg_len).  Either all T_k rows are computed
 * (T_q == T_k: text rows from txt_feats, reference rows from ref_latent) or
 * only the target rows (T_q == N), the text and reference K/V then being read
 * from rows [0, T_k - N) of each block's cache, written by an earlier call with
 * the same prefix inputs (the prefix rows use a modulation set that does not
 * change between steps, so both give the same result).  Device pointers unless
 * noted; caller-owned.
 */
typedef struct {
    const void* txt_feats;      /* [L_txt, C_txt] activation dtype; read only when T_q == T_k */
    const float* ref_latent;    /* [R, C_lat] fp32; read only when T_q == T_k and R > 0 */
    const float* latent;        /* [N, C_lat] fp32 target latent (not modified) */
    int64_t L_txt, R, N;
    const float* mod;           /* [n_mod, 6, D] modulation sets, as in dit_block_io */
    int32_t n_mod;
    const int32_t* mod_of_seg;  /* host [n_seg] */
    const float* mod_final;     /* [2, D] shift, scale of the tail's adaLN */
    const float* cos_t;         /* [T_q, 64] RoPE tables of the computed rows */
    const float* sin_t;
    const int32_t* seg_len;     /* host [n_seg] */
    int32_t n_seg;
    int64_t T_q;                /* T_k or N */
    void* const* k_caches;      /* host array of n_blocks device caches [T_k, H, 128] */
    void* const* v_caches;
    void* vel;                  /* [N, C_lat] activation dtype: the velocity */
} dit_velocity_io;

/* Workspace of dit_velocity_forward (bytes); T_k = L_txt + R + N.  After a
 * call the workspace begins with the block stack's output rows x [T_q, D]
 * (activation dtype, row stride D), the input of the tail. */
size_t dit_velocity_workspace_bytes(const dit_block_config* cfg, int64_t T_q, int64_t T_k, int64_t N,
                                    int32_t C_lat);

/*
 * One evaluation of the DiT: head -> n_blocks blocks (dit_stack_forward) ->
 * tail, writing io->vel.  The denoise loop then applies dit_euler_step to the
 * target latent ([Core AI port, graph contracts]: one Euler update per step).
 * Enqueues work on `stream` only (no allocation, no synchronization), so one
 * call can be captured in a HIP graph and replayed with new contents of the
 * same buffers.  Errors: DIT_E_NULL / DIT_E_SHAPE / DIT_E_UNSUPPORTED /
 * DIT_E_WORKSPACE / DIT_E_ALIGN before any launch; DIT_E_HIP on launch failure.
 */
int dit_velocity_forward(const dit_block_config* cfg, const dit_block_weights* blocks, int32_t n_blocks,
                         const dit_head_weights* head, const dit_velocity_io* io, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ tracing */

/* Launch sites of the block, in launch order. */
typedef enum {
    DIT_SITE_ADALN1 = 0, DIT_SITE_QKV_GEMM, DIT_SITE_QK_NORM_ROPE, DIT_SITE_ATTENTION,
    DIT_SITE_QUANT_O, DIT_SITE_OUT_GEMM, DIT_SITE_ADALN2, DIT_SITE_UP_GEMM, DIT_SITE_QUANT_G,
    DIT_SITE_DOWN_GEMM, DIT_SITE_ATTN_QUANT, DIT_N_SITES
} dit_site_t;

/*
 * Per-launch kernel timing with HIP events (measurement only).  dit_profile_begin
 * creates `capacity` event pairs (this allocates; call it outside any timed or
 * captured region); while active, every kernel that dit_block_forward or
 * dit_stack_forward launches records a start and an end event on its stream
 * (at most `capacity` launches are recorded; later ones are counted in nothing).
 * dit_profile_end waits for the recorded events, writes per site the summed
 * milliseconds (ms_out[n_sites]) and launch counts (count_out[n_sites]), frees
 * the events and stops recording.  Not for use from several threads at once.
 */
int dit_profile_begin(int32_t capacity);
int dit_profile_end(double* ms_out, int64_t* count_out, int32_t n_sites);
const char* dit_site_name(int32_t site);

#ifdef __cplusplus
}
#endif
#endif /* DIT_H */
