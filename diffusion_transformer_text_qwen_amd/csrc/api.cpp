// C ABI of the block library: argument checks (before any HIP call), the
// block's workspace plan and the launch sequence of one block.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/dit.h"
#include "kernels.h"

using namespace dit;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return DIT_OK;
    return fail(DIT_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define CHECK(cond, code, ...)                  \
    do {                                        \
        if (!(cond)) return fail(code, __VA_ARGS__); \
    } while (0)

#define RUN(expr, what)                          \
    do {                                         \
        int _s = hip_status((expr), what);       \
        if (_s != DIT_OK) return _s;             \
    } while (0)

hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int64_t kMaxK8 = 133144;   // K * 127^2 < 2^31

int check_segs(const int32_t* seg_len, int32_t n_seg, int64_t T_k) {
    CHECK(seg_len != nullptr, DIT_E_NULL, "seg_len is NULL");
    CHECK(n_seg >= 1 && n_seg <= kMaxSeg, DIT_E_UNSUPPORTED, "n_seg=%d outside [1, %d]", n_seg, kMaxSeg);
    int64_t sum = 0;
    for (int i = 0; i < n_seg; ++i) {
        CHECK(seg_len[i] >= 0, DIT_E_SHAPE, "seg_len[%d]=%d < 0", i, seg_len[i]);
        sum += seg_len[i];
    }
    CHECK(sum == T_k, DIT_E_SHAPE, "sum(seg_len)=%lld != T_k=%lld", (long long)sum, (long long)T_k);
    return DIT_OK;
}

AttnSegs make_attn_segs(const int32_t* seg_len, int32_t n_seg) {
    AttnSegs a{};
    int64_t acc = 0;
    for (int i = 0; i < n_seg; ++i) {
        acc += seg_len[i];
        a.end[i] = acc;
    }
    a.n = n_seg;
    return a;
}

SegMap make_segmap(const int32_t* seg_len, const int32_t* mod_of_seg, int32_t n_seg, int64_t row_offset) {
    SegMap m{};
    int64_t acc = 0;
    for (int i = 0; i < n_seg; ++i) {
        acc += seg_len[i];
        m.end[i] = acc;
        m.set[i] = mod_of_seg ? mod_of_seg[i] : 0;
    }
    m.n = n_seg;
    m.row_offset = row_offset;
    return m;
}

// ---- launch timing (measurement only)
struct Profiler {
    bool on = false;
    int cap = 0, used = 0;
    std::vector<hipEvent_t> ev;
    std::vector<int> site;
} g_prof;

struct ProfScope {
    int idx = -1;
    hipStream_t st;
    ProfScope(int site, hipStream_t s) : st(s) {
        if (g_prof.on && g_prof.used < g_prof.cap) {
            idx = g_prof.used++;
            g_prof.site[idx] = site;
            (void)hipEventRecord(g_prof.ev[2 * idx], st);
        }
    }
    ~ProfScope() {
        if (idx >= 0) (void)hipEventRecord(g_prof.ev[2 * idx + 1], st);
    }
};

EpiParams store_epi(void* y, int64_t ldy, bool y_bf16, const float* bias) {
    EpiParams ep{};
    ep.kind = EPI_STORE;
    ep.act_bf16 = y_bf16;
    ep.y_bf16 = y_bf16;
    ep.bias = bias;
    ep.y = y;
    ep.ldy = ldy;
    return ep;
}

// ---- device scratch of w8a8_linear_noalloc (for callers that cannot allocate)
// The K-split partial sums of w8a8_linear_noalloc live in this array, one copy
// per GPU, held until the process ends.  Host code never passes the array's
// name to a kernel (in host code it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and is kept in scratch_ptr[].
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

int noalloc_scratch(void** out) {
    int dev = -1;
    RUN(hipGetDevice(&dev), "hipGetDevice");
    CHECK(dev >= 0 && dev < kMaxDevices, DIT_E_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        RUN(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        CHECK(p != nullptr && aligned16(p), DIT_E_HIP, "scratch symbol address invalid");
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return DIT_OK;
}

}  // namespace

extern "C" {

int dit_abi_version(void) { return DIT_ABI_VERSION; }

const char* dit_status_string(int s) {
    switch (s) {
        case DIT_OK: return "ok";
        case DIT_E_NULL: return "null pointer";
        case DIT_E_SHAPE: return "bad shape";
        case DIT_E_DTYPE: return "bad dtype or mode";
        case DIT_E_ALIGN: return "misaligned pointer or stride";
        case DIT_E_UNSUPPORTED: return "unsupported size";
        case DIT_E_WORKSPACE: return "workspace missing or too small";
        case DIT_E_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

const char* dit_last_error(void) { return g_err; }

int dit_quantize_rows(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                      float* scale, void* stream) {
    CHECK(x_dtype == DIT_BF16 || x_dtype == DIT_F32, DIT_E_DTYPE, "x_dtype must be bf16 or f32");
    CHECK(M >= 0 && K >= 1 && ldx >= K, DIT_E_SHAPE, "need M>=0, K>=1, ldx>=K");
    CHECK(K % 8 == 0 && ldx % 8 == 0, DIT_E_UNSUPPORTED, "K and ldx must be multiples of 8");
    CHECK(K <= (x_dtype == DIT_BF16 ? 32768 : 16384), DIT_E_UNSUPPORTED, "K=%lld too large", (long long)K);
    CHECK(M <= 0x7fffffff, DIT_E_UNSUPPORTED, "M too large");
    if (M == 0) return DIT_OK;
    CHECK(x && q && scale, DIT_E_NULL, "x, q and scale must be non-NULL");
    CHECK(aligned16(x) && aligned16(q), DIT_E_ALIGN, "x and q must be 16-byte aligned");
    RUN(launch_quantize_rows(x, x_dtype == DIT_BF16, M, K, ldx, q, scale, S(stream)), "quantize_rows");
    return DIT_OK;
}

int dit_gelu_quantize_rows(const void* u, int64_t M, int64_t K, int64_t ldu, int8_t* q, float* scale,
                           void* g_out, void* stream) {
    CHECK(M >= 0 && K >= 1 && ldu >= K, DIT_E_SHAPE, "need M>=0, K>=1, ldu>=K");
    CHECK(K % 8 == 0 && ldu % 8 == 0, DIT_E_UNSUPPORTED, "K and ldu must be multiples of 8");
    CHECK(K <= 16384, DIT_E_UNSUPPORTED, "K=%lld above 16384", (long long)K);
    CHECK(M <= 0x7fffffff, DIT_E_UNSUPPORTED, "M too large");
    CHECK(ldu * 2 * (M ? M : 1) < ((int64_t)1 << 62), DIT_E_UNSUPPORTED, "u too large");
    if (M == 0) return DIT_OK;
    CHECK(u && q && scale, DIT_E_NULL, "u, q and scale must be non-NULL");
    CHECK(aligned16(u) && aligned16(q) && (!g_out || aligned16(g_out)), DIT_E_ALIGN,
          "u, q and g_out must be 16-byte aligned");
    RUN(launch_gelu_quantize_rows(u, M, K, q, scale, S(stream), ldu, g_out), "gelu_quantize_rows");
    return DIT_OK;
}

size_t w8a8_linear_workspace_bytes(void) { return (size_t)kSplitPartialBytes; }

static int check_w8a8_args(const int8_t* a, const float* a_scale, int64_t M, int64_t K, const int8_t* w,
                           const float* w_scale, int64_t N, const void* y, int y_dtype, int64_t ldy) {
    CHECK(y_dtype == DIT_BF16 || y_dtype == DIT_F32, DIT_E_DTYPE, "y_dtype must be bf16 or f32");
    CHECK(M >= 0 && K >= 1 && N >= 1 && ldy >= N, DIT_E_SHAPE, "need M>=0, K>=1, N>=1, ldy>=N");
    CHECK(K % 128 == 0, DIT_E_UNSUPPORTED, "K=%lld must be a multiple of 128", (long long)K);
    CHECK(N % 16 == 0, DIT_E_UNSUPPORTED, "N=%lld must be a multiple of 16", (long long)N);
    CHECK(K <= kMaxK8, DIT_E_UNSUPPORTED, "K=%lld beyond the int32-safe bound", (long long)K);
    CHECK(((M + 127) / 128) * ((N + 127) / 128) < 0x7fffffff, DIT_E_UNSUPPORTED, "too many tiles");
    CHECK(M * K < ((int64_t)1 << 31) && N * K < ((int64_t)1 << 31), DIT_E_UNSUPPORTED,
          "operands must be below 2 GiB");
    if (M == 0) return DIT_OK;
    CHECK(a && a_scale && w && w_scale && y, DIT_E_NULL, "a, a_scale, w, w_scale and y must be non-NULL");
    CHECK(aligned16(a) && aligned16(w), DIT_E_ALIGN, "a and w must be 16-byte aligned");
    return DIT_OK;
}

int w8a8_linear(const int8_t* a, const float* a_scale, int64_t M, int64_t K, const int8_t* w,
                const float* w_scale, const float* bias, int64_t N, void* y, int y_dtype, int64_t ldy,
                int32_t* acc_out, void* workspace, size_t workspace_bytes, void* stream) {
    int s = check_w8a8_args(a, a_scale, M, K, w, w_scale, N, y, y_dtype, ldy);
    if (s) return s;
    CHECK(workspace == nullptr || workspace_bytes >= w8a8_linear_workspace_bytes(), DIT_E_WORKSPACE,
          "workspace needs %zu bytes", w8a8_linear_workspace_bytes());
    if (M == 0) return DIT_OK;
    CHECK(workspace == nullptr || aligned16(workspace), DIT_E_ALIGN, "workspace must be 16-byte aligned");
    EpiParams ep = store_epi(y, ldy, y_dtype == DIT_BF16, bias);
    ep.a_scale = a_scale;
    ep.w_scale = w_scale;
    ep.acc_out = acc_out;
    ep.ldacc = N;
    if (workspace) {
        ep.split_partial = (int32_t*)workspace;
        ep.split_bytes = kSplitPartialBytes;
    }
    RUN(launch_gemm_i8(a, w, M, N, K, ep, S(stream)), "w8a8_linear");
    return DIT_OK;
}

int w8a8_linear_noalloc(const int8_t* a, const float* a_scale, int64_t M, int64_t K, const int8_t* w,
                        const float* w_scale, const float* bias, int64_t N, void* y, int y_dtype, int64_t ldy,
                        int32_t* acc_out, void* stream) {
    int s = check_w8a8_args(a, a_scale, M, K, w, w_scale, N, y, y_dtype, ldy);
    if (s) return s;
    if (M == 0) return DIT_OK;
    void* part = nullptr;
    s = noalloc_scratch(&part);
    if (s) return s;
    EpiParams ep = store_epi(y, ldy, y_dtype == DIT_BF16, bias);
    ep.a_scale = a_scale;
    ep.w_scale = w_scale;
    ep.acc_out = acc_out;
    ep.ldacc = N;
    ep.split_partial = (int32_t*)part;
    ep.split_bytes = (int64_t)kNoAllocScratchBytes;
    RUN(launch_gemm_i8(a, w, M, N, K, ep, S(stream)), "w8a8_linear_noalloc");
    return DIT_OK;
}

int dit_quantize_rows_asym(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                           float* scale, int32_t* zero, void* stream) {
    CHECK(x_dtype == DIT_BF16 || x_dtype == DIT_F32, DIT_E_DTYPE, "x_dtype must be bf16 or f32");
    CHECK(M >= 0 && K >= 1 && ldx >= K, DIT_E_SHAPE, "need M>=0, K>=1, ldx>=K");
    CHECK(K % 8 == 0 && ldx % 8 == 0, DIT_E_UNSUPPORTED, "K and ldx must be multiples of 8");
    CHECK(M <= 0x7fffffff, DIT_E_UNSUPPORTED, "M too large");
    if (M == 0) return DIT_OK;
    CHECK(x && q && scale && zero, DIT_E_NULL, "x, q, scale and zero must be non-NULL");
    CHECK(aligned16(x) && aligned16(q), DIT_E_ALIGN, "x and q must be 16-byte aligned");
    RUN(launch_quantize_rows_asym(x, x_dtype == DIT_BF16, M, K, ldx, q, scale, zero, S(stream)),
        "quantize_rows_asym");
    return DIT_OK;
}

int dit_int8_colsum(const int8_t* w, int64_t N, int64_t K, int32_t* out, void* stream) {
    CHECK(N >= 0 && K >= 1, DIT_E_SHAPE, "need N>=0, K>=1");
    CHECK(K % 16 == 0, DIT_E_UNSUPPORTED, "K must be a multiple of 16");
    CHECK(N <= ((int64_t)1 << 32), DIT_E_UNSUPPORTED, "N too large");
    if (N == 0) return DIT_OK;
    CHECK(w && out, DIT_E_NULL, "w and out must be non-NULL");
    CHECK(aligned16(w), DIT_E_ALIGN, "w must be 16-byte aligned");
    RUN(launch_int8_colsum(w, N, K, out, S(stream)), "int8_colsum");
    return DIT_OK;
}

int dit_mxfp4_expand(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, void* w_bf16,
                     void* stream) {
    CHECK(N >= 0 && K >= 1, DIT_E_SHAPE, "need N>=0, K>=1");
    CHECK(K % 32 == 0, DIT_E_UNSUPPORTED, "K must be a multiple of 32");
    CHECK(N * (K / 32) < ((int64_t)1 << 31) * 256, DIT_E_UNSUPPORTED, "too many groups");
    if (N == 0) return DIT_OK;
    CHECK(codes && scales && w_bf16, DIT_E_NULL, "codes, scales and w_bf16 must be non-NULL");
    CHECK(aligned16(codes) && aligned16(w_bf16), DIT_E_ALIGN, "codes and w_bf16 must be 16-byte aligned");
    RUN(launch_mxfp4_expand(codes, scales, N, K, w_bf16, S(stream)), "mxfp4_expand");
    return DIT_OK;
}

size_t mxfp4_linear_workspace_bytes(int64_t N, int64_t K) {
    return (N < 0 || K < 0) ? 0 : (size_t)N * (size_t)K * 2;
}

int mxfp4_linear(const void* a, int64_t M, int64_t K, int64_t lda, const uint8_t* codes, const uint8_t* scales,
                 const float* bias, int64_t N, void* y, int y_dtype, int64_t ldy, void* workspace,
                 size_t workspace_bytes, void* stream) {
    CHECK(y_dtype == DIT_BF16 || y_dtype == DIT_F32, DIT_E_DTYPE, "y_dtype must be bf16 or f32");
    CHECK(M >= 0 && K >= 1 && N >= 1 && lda >= K && ldy >= N, DIT_E_SHAPE, "bad sizes or strides");
    CHECK(K % 64 == 0 && lda % 8 == 0, DIT_E_UNSUPPORTED, "K must be a multiple of 64, lda of 8");
    CHECK(N % 16 == 0, DIT_E_UNSUPPORTED, "N must be a multiple of 16");
    CHECK(workspace != nullptr && workspace_bytes >= mxfp4_linear_workspace_bytes(N, K), DIT_E_WORKSPACE,
          "workspace needs %zu bytes", mxfp4_linear_workspace_bytes(N, K));
    if (M == 0) return DIT_OK;
    CHECK(a && codes && scales && y, DIT_E_NULL, "a, codes, scales and y must be non-NULL");
    CHECK(aligned16(a) && aligned16(codes) && aligned16(workspace), DIT_E_ALIGN,
          "a, codes and workspace must be 16-byte aligned");
    hipStream_t st = S(stream);
    EpiParams ep = store_epi(y, ldy, y_dtype == DIT_BF16, bias);
    if (gemm_bf16_direct_mxfp4(M, N, K, lda, false) && N * (K / 2) < ((int64_t)1 << 31)) {
        // the large-tile GEMM decodes the codes in its operand staging
        ep.w_mx_scale = scales;
        RUN(launch_gemm_bf16(a, lda, codes, M, N, K, ep, st), "mxfp4_linear");
        return DIT_OK;
    }
    RUN(launch_mxfp4_expand(codes, scales, N, K, workspace, st), "mxfp4_expand");
    RUN(launch_gemm_bf16(a, lda, workspace, M, N, K, ep, st), "mxfp4_linear");
    return DIT_OK;
}

int w8a8_linear_asym(const int8_t* a, const float* a_scale, const int32_t* a_zero, int64_t M, int64_t K,
                     const int8_t* w, const float* w_scale, const int32_t* w_sum, const float* bias, int64_t N,
                     void* y, int y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
    CHECK(a_zero == nullptr || w_sum != nullptr || M == 0, DIT_E_NULL, "a_zero needs w_sum");
    CHECK(w_sum == nullptr || aligned16(w_sum), DIT_E_ALIGN, "w_sum must be 16-byte aligned");
    if (a_zero == nullptr)
        return w8a8_linear(a, a_scale, M, K, w, w_scale, bias, N, y, y_dtype, ldy, nullptr, workspace,
                           workspace_bytes, stream);
    CHECK(y_dtype == DIT_BF16 || y_dtype == DIT_F32, DIT_E_DTYPE, "y_dtype must be bf16 or f32");
    CHECK(M >= 0 && K >= 1 && N >= 1 && ldy >= N, DIT_E_SHAPE, "need M>=0, K>=1, N>=1, ldy>=N");
    CHECK(K % 128 == 0, DIT_E_UNSUPPORTED, "K=%lld must be a multiple of 128", (long long)K);
    CHECK(N % 16 == 0, DIT_E_UNSUPPORTED, "N=%lld must be a multiple of 16", (long long)N);
    CHECK(K <= 65536, DIT_E_UNSUPPORTED, "K=%lld beyond the int32-safe bound (255 * 127 * K < 2^31)", (long long)K);
    CHECK(M * K < ((int64_t)1 << 31) && N * K < ((int64_t)1 << 31), DIT_E_UNSUPPORTED,
          "operands must be below 2 GiB");
    CHECK(workspace == nullptr || workspace_bytes >= w8a8_linear_workspace_bytes(), DIT_E_WORKSPACE,
          "workspace needs %zu bytes", w8a8_linear_workspace_bytes());
    if (M == 0) return DIT_OK;
    CHECK(a && a_scale && w && w_scale && y, DIT_E_NULL, "a, a_scale, w, w_scale and y must be non-NULL");
    CHECK(aligned16(a) && aligned16(w), DIT_E_ALIGN, "a and w must be 16-byte aligned");
    CHECK(workspace == nullptr || aligned16(workspace), DIT_E_ALIGN, "workspace must be 16-byte aligned");
    EpiParams ep = store_epi(y, ldy, y_dtype == DIT_BF16, bias);
    ep.a_scale = a_scale;
    ep.w_scale = w_scale;
    ep.a_zero = a_zero;
    ep.w_sum = w_sum;
    if (workspace) {
        ep.split_partial = (int32_t*)workspace;
        ep.split_bytes = kSplitPartialBytes;
    }
    RUN(launch_gemm_i8(a, w, M, N, K, ep, S(stream)), "w8a8_linear_asym");
    return DIT_OK;
}

int bf16_linear(const void* a, int64_t M, int64_t K, int64_t lda, const void* w, const float* bias,
                int64_t N, void* y, int y_dtype, int64_t ldy, void* stream) {
    CHECK(y_dtype == DIT_BF16 || y_dtype == DIT_F32, DIT_E_DTYPE, "y_dtype must be bf16 or f32");
    CHECK(M >= 0 && K >= 1 && N >= 1 && lda >= K && ldy >= N, DIT_E_SHAPE, "bad sizes or strides");
    CHECK(K % 64 == 0 && lda % 8 == 0, DIT_E_UNSUPPORTED, "K must be a multiple of 64, lda of 8");
    CHECK(N % 16 == 0, DIT_E_UNSUPPORTED, "N must be a multiple of 16");
    CHECK(((M + 127) / 128) * ((N + 127) / 128) < 0x7fffffff, DIT_E_UNSUPPORTED, "too many tiles");
    if (M == 0) return DIT_OK;
    CHECK(a && w && y, DIT_E_NULL, "a, w and y must be non-NULL");
    CHECK(aligned16(a) && aligned16(w), DIT_E_ALIGN, "a and w must be 16-byte aligned");
    EpiParams ep = store_epi(y, ldy, y_dtype == DIT_BF16, bias);
    RUN(launch_gemm_bf16(a, lda, w, M, N, K, ep, S(stream)), "bf16_linear");
    return DIT_OK;
}

int f32_linear(const float* a, int64_t M, int64_t K, int64_t lda, const float* w, const float* bias,
               int64_t N, float* y, int64_t ldy, void* stream) {
    CHECK(M >= 0 && K >= 1 && N >= 1 && lda >= K && ldy >= N, DIT_E_SHAPE, "bad sizes or strides");
    CHECK(K % 16 == 0 && N % 16 == 0, DIT_E_UNSUPPORTED, "K and N must be multiples of 16");
    CHECK((M + 63) / 64 < 65536, DIT_E_UNSUPPORTED, "M too large for the fp32 kernel");
    if (M == 0) return DIT_OK;
    CHECK(a && w && y, DIT_E_NULL, "a, w and y must be non-NULL");
    EpiParams ep = store_epi(y, ldy, false, bias);
    RUN(launch_gemm_f32(a, lda, w, M, N, K, ep, S(stream)), "f32_linear");
    return DIT_OK;
}

size_t dit_qkv_linear_workspace_bytes(int64_t T, int32_t H) {
    if (T < 0 || H < 1) return 0;
    return (size_t)kSplitPartialBytes + (((size_t)T * 3 * H * 128 * 2 + 255) & ~(size_t)255);
}

int dit_qkv_linear(int mode, const void* a, const float* a_scale, int64_t T, int32_t H, const void* w,
                   const float* w_scale, const float* bias, const float* g_q, const float* g_k, const float* cos_t,
                   const float* sin_t, float eps, void* q_out, void* k_out, void* v_out, void* workspace,
                   size_t workspace_bytes, void* stream) {
    CHECK(mode == DIT_MODE_BF16 || mode == DIT_MODE_W8A8, DIT_E_DTYPE, "mode must be BF16 or W8A8");
    CHECK(T >= 0 && H >= 1, DIT_E_SHAPE, "need T>=0, H>=1");
    const int64_t D = (int64_t)H * 128;
    CHECK(D % 256 == 0 && D <= 8192, DIT_E_UNSUPPORTED, "H*128 must be a multiple of 256, <= 8192");
    CHECK(T * 3 * D < ((int64_t)1 << 31), DIT_E_UNSUPPORTED, "T * 3 * H * 128 must be below 2^31");
    CHECK(eps >= 0.0f, DIT_E_SHAPE, "eps must be >= 0");
    CHECK(workspace != nullptr && workspace_bytes >= dit_qkv_linear_workspace_bytes(T, H), DIT_E_WORKSPACE,
          "workspace needs %zu bytes", dit_qkv_linear_workspace_bytes(T, H));
    if (T == 0) return DIT_OK;
    CHECK(a && w && g_q && g_k && cos_t && sin_t && q_out && k_out && v_out, DIT_E_NULL, "NULL argument");
    CHECK(mode != DIT_MODE_W8A8 || (a_scale && w_scale), DIT_E_NULL, "W8A8 needs a_scale and w_scale");
    CHECK(aligned16(a) && aligned16(w) && aligned16(g_q) && aligned16(g_k) && aligned16(cos_t) &&
              aligned16(sin_t) && aligned16(q_out) && aligned16(k_out) && aligned16(v_out) &&
              aligned16(workspace) && (!bias || aligned16(bias)),
          DIT_E_ALIGN, "pointers must be 16-byte aligned");
    EpiParams ep = store_epi((uint8_t*)workspace + kSplitPartialBytes, 3 * D, true, bias);
    ep.kind = EPI_QKV_ROPE;
    ep.q_out = q_out;
    ep.k_out = k_out;
    ep.v_out = v_out;
    ep.g_q = g_q;
    ep.g_k = g_k;
    ep.cos_t = cos_t;
    ep.sin_t = sin_t;
    ep.qk_eps = eps;
    ep.D = D;
    ep.split_partial = (int32_t*)workspace;
    ep.split_bytes = kSplitPartialBytes;
    if (mode == DIT_MODE_W8A8) {
        ep.a_scale = a_scale;
        ep.w_scale = w_scale;
        RUN(launch_gemm_i8((const int8_t*)a, (const int8_t*)w, T, 3 * D, D, ep, S(stream)), "qkv_linear");
    } else {
        RUN(launch_gemm_bf16(a, D, w, T, 3 * D, D, ep, S(stream)), "qkv_linear");
    }
    return DIT_OK;
}

int block_causal_attention(const void* q, const void* k, const void* v, void* o, int dtype, int64_t T_q,
                           int64_t T_k, int32_t H, int32_t d, int64_t ldq, int64_t ldk, int64_t ldv,
                           int64_t ldo, const int32_t* seg_len, int32_t n_seg, float sm_scale,
                           void* stream) {
    CHECK(dtype == DIT_BF16 || dtype == DIT_F32, DIT_E_DTYPE, "dtype must be bf16 or f32");
    CHECK(d == 128, DIT_E_UNSUPPORTED, "only head_dim 128 is supported (got %d)", d);
    CHECK(H >= 1 && H <= 65535, DIT_E_SHAPE, "H=%d outside [1, 65535]", H);
    CHECK(T_q >= 0 && T_q <= T_k, DIT_E_SHAPE, "need 0 <= T_q <= T_k");
    const int64_t row = (int64_t)H * d;
    CHECK(ldq >= row && ldk >= row && ldv >= row && ldo >= row, DIT_E_SHAPE, "row strides must be >= H*d");
    CHECK(ldq % 8 == 0 && ldk % 8 == 0 && ldv % 8 == 0 && ldo % 8 == 0, DIT_E_ALIGN,
          "row strides must be multiples of 8 elements");
    CHECK(T_k < ((int64_t)1 << 40), DIT_E_UNSUPPORTED, "T_k too large");
    int s = check_segs(seg_len, n_seg, T_k);
    if (s) return s;
    if (T_q == 0) return DIT_OK;
    CHECK(q && k && v && o, DIT_E_NULL, "q, k, v and o must be non-NULL");
    CHECK(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o), DIT_E_ALIGN,
          "q, k, v and o must be 16-byte aligned");
    if (sm_scale <= 0.0f) sm_scale = 1.0f / std::sqrt((float)d);
    const AttnSegs segs = make_attn_segs(seg_len, n_seg);
    if (dtype == DIT_BF16) {
        CHECK(T_k < ((int64_t)1 << 31) && ldq < ((int64_t)1 << 31) && ldk < ((int64_t)1 << 31) &&
                  ldv < ((int64_t)1 << 31) && ldo < ((int64_t)1 << 31),
              DIT_E_UNSUPPORTED, "bf16 attention needs T_k and strides below 2^31");
        RUN(launch_attention_bf16(q, k, v, o, T_q, T_k, H, ldq, ldk, ldv, ldo, segs, sm_scale, S(stream)),
            "attention_bf16");
    } else {
        CHECK((T_q * H + 3) / 4 < 0x7fffffff, DIT_E_UNSUPPORTED, "T_q*H too large");
        RUN(launch_attention_f32((const float*)q, (const float*)k, (const float*)v, (float*)o, T_q, T_k, H,
                                 ldq, ldk, ldv, ldo, segs, sm_scale, S(stream)),
            "attention_f32");
    }
    return DIT_OK;
}

int dit_rope_tables(int32_t text_len, const int32_t* grids, int32_t n_img, int64_t row0, int64_t T_rows,
                    float theta, float* cos_out, float* sin_out, void* stream) {
    CHECK(text_len >= 0 && n_img >= 0 && n_img <= 15, DIT_E_UNSUPPORTED, "need text_len>=0, 0<=n_img<=15");
    CHECK(n_img == 0 || grids != nullptr, DIT_E_NULL, "grids is NULL");
    CHECK(theta > 0.0f, DIT_E_SHAPE, "theta must be positive");
    int64_t total = text_len;
    for (int k = 0; k < n_img; ++k) {
        CHECK(grids[2 * k] >= 1 && grids[2 * k + 1] >= 1, DIT_E_SHAPE, "grid %d has a zero side", k);
        total += (int64_t)grids[2 * k] * grids[2 * k + 1];
    }
    CHECK(row0 >= 0 && T_rows >= 0 && row0 + T_rows <= total, DIT_E_SHAPE, "rows outside the sequence");
    CHECK(T_rows * 64 / 256 < 0x7fffffff, DIT_E_UNSUPPORTED, "too many rows");
    if (T_rows == 0) return DIT_OK;
    CHECK(cos_out && sin_out, DIT_E_NULL, "cos_out and sin_out must be non-NULL");
    RUN(launch_rope_tables(text_len, grids, n_img, row0, T_rows, theta, cos_out, sin_out, S(stream)),
        "rope_tables");
    return DIT_OK;
}

int dit_qk_norm_rope(const void* qkv, int dtype, int64_t T, int32_t H, const float* g_q, const float* g_k,
                     const float* cos_t, const float* sin_t, float eps, void* q_out, void* k_out,
                     int64_t ldk, void* v_out, int64_t ldv, void* stream) {
    CHECK(dtype == DIT_BF16 || dtype == DIT_F32, DIT_E_DTYPE, "dtype must be bf16 or f32");
    CHECK(T >= 0 && H >= 1, DIT_E_SHAPE, "need T>=0, H>=1");
    CHECK(ldk >= (int64_t)H * 128 && ldv >= (int64_t)H * 128, DIT_E_SHAPE, "ldk, ldv must be >= H*128");
    CHECK(ldk % 2 == 0 && ldv % 2 == 0, DIT_E_ALIGN, "ldk, ldv must be even");
    CHECK((T * H + 3) / 4 < 0x7fffffff, DIT_E_UNSUPPORTED, "T*H too large");
    if (T == 0) return DIT_OK;
    CHECK(qkv && g_q && g_k && cos_t && sin_t && q_out && k_out && v_out, DIT_E_NULL, "NULL argument");
    RUN(launch_qk_norm_rope(qkv, dtype == DIT_BF16, T, H, g_q, g_k, cos_t, sin_t, eps, q_out, k_out, ldk,
                            v_out, ldv, S(stream)),
        "qk_norm_rope");
    return DIT_OK;
}

int dit_adaln_modulate(const void* x, int x_dtype, int64_t M, int64_t D, const float* shift,
                       const float* scale, float eps, void* h_out, int h_dtype, int8_t* q_out,
                       float* q_scale, void* stream) {
    CHECK(x_dtype == DIT_BF16 || x_dtype == DIT_F32, DIT_E_DTYPE, "x_dtype must be bf16 or f32");
    CHECK(h_out == nullptr || h_dtype == x_dtype, DIT_E_DTYPE, "h_dtype must equal x_dtype");
    CHECK(M >= 0 && D >= 256, DIT_E_SHAPE, "need M>=0, D>=256");
    CHECK(D % 256 == 0 && D <= 8192, DIT_E_UNSUPPORTED, "D must be a multiple of 256, <= 8192");
    CHECK(M <= 0x7fffffff, DIT_E_UNSUPPORTED, "M too large");
    if (M == 0) return DIT_OK;
    CHECK(x && shift && scale, DIT_E_NULL, "x, shift and scale must be non-NULL");
    CHECK(h_out != nullptr || q_out != nullptr, DIT_E_NULL, "h_out and q_out are both NULL");
    CHECK(q_out == nullptr || q_scale != nullptr, DIT_E_NULL, "q_scale is NULL");
    CHECK(aligned16(x) && (!q_out || aligned16(q_out)) && (!h_out || aligned16(h_out)), DIT_E_ALIGN,
          "x, h_out and q_out must be 16-byte aligned");
    SegMap sm{};
    sm.end[0] = M;
    sm.set[0] = 0;
    sm.n = 1;
    RUN(launch_adaln(x, x_dtype == DIT_BF16, M, D, shift, scale, 0, sm, eps, h_out, q_out, q_scale, S(stream)),
        "adaln");
    return DIT_OK;
}

int dit_adaln_modulate_asym(const void* x, int64_t M, int64_t D, const float* shift, const float* scale,
                            float eps, void* h_out, int8_t* q_out, float* q_scale, int32_t* q_zero,
                            void* stream) {
    CHECK(M >= 0 && D >= 256, DIT_E_SHAPE, "need M>=0, D>=256");
    CHECK(D % 256 == 0 && D <= 4096, DIT_E_UNSUPPORTED, "D must be a multiple of 256, <= 4096");
    CHECK(M <= 0x7fffffff, DIT_E_UNSUPPORTED, "M too large");
    if (M == 0) return DIT_OK;
    CHECK(x && shift && scale && q_out && q_scale && q_zero, DIT_E_NULL,
          "x, shift, scale, q_out, q_scale and q_zero must be non-NULL");
    CHECK(aligned16(x) && aligned16(shift) && aligned16(scale) && (!h_out || aligned16(h_out)) &&
              ((uintptr_t)q_out & 7) == 0,
          DIT_E_ALIGN, "x, shift, scale and h_out must be 16-byte aligned, q_out 8-byte aligned");
    SegMap sm{};
    sm.end[0] = M;
    sm.set[0] = 0;
    sm.n = 1;
    RUN(launch_adaln_asym(x, M, D, shift, scale, 0, sm, eps, h_out, q_out, q_scale, q_zero, S(stream)),
        "adaln_asym");
    return DIT_OK;
}

int dit_euler_step(float* x, const void* v, int v_dtype, int64_t n, float sigma, float sigma_next,
                   void* stream) {
    CHECK(v_dtype == DIT_BF16 || v_dtype == DIT_F32, DIT_E_DTYPE, "v_dtype must be bf16 or f32");
    CHECK(n >= 0 && (n + 255) / 256 < 0x7fffffff, DIT_E_SHAPE, "bad n");
    if (n == 0) return DIT_OK;
    CHECK(x && v, DIT_E_NULL, "x and v must be non-NULL");
    RUN(launch_euler(x, v, v_dtype == DIT_BF16, n, sigma, sigma_next, S(stream)), "euler");
    return DIT_OK;
}

int dit_cast(const void* x, int x_dtype, void* y, int y_dtype, int64_t n, void* stream) {
    CHECK((x_dtype == DIT_BF16 || x_dtype == DIT_F32) && (y_dtype == DIT_BF16 || y_dtype == DIT_F32), DIT_E_DTYPE,
          "dtypes must be bf16 or f32");
    CHECK(n >= 0 && (n + 255) / 256 < 0x7fffffff, DIT_E_SHAPE, "bad n");
    if (n == 0) return DIT_OK;
    CHECK(x && y, DIT_E_NULL, "x and y must be non-NULL");
    RUN(launch_cast(x, x_dtype == DIT_BF16, y, y_dtype == DIT_BF16, n, S(stream)), "cast");
    return DIT_OK;
}

// ------------------------------------------------------------------ block

size_t dit_attn_q8_bytes(int64_t T_q, int64_t T_k, int32_t H, int64_t* offsets) {
    if (T_q < 0 || T_k < T_q || H < 1) return 0;
    const AttnQ8Layout L = attn_q8_layout(T_q, T_k, H);
    if (offsets) {
        const size_t o[7] = {L.q8, L.sq, L.k8, L.sk, L.v8, L.sv, L.vamax};
        for (int i = 0; i < 7; ++i) offsets[i] = (int64_t)o[i];
    }
    return L.total;
}

static int check_q8_shape(int64_t T_q, int64_t T_k, int32_t H) {
    CHECK(H >= 1 && H <= 65535, DIT_E_SHAPE, "H=%d outside [1, 65535]", H);
    CHECK(T_q >= 0 && T_q <= T_k, DIT_E_SHAPE, "need 0 <= T_q <= T_k");
    CHECK(T_k < ((int64_t)1 << 31), DIT_E_UNSUPPORTED, "T_k must be below 2^31");
    CHECK((int64_t)H * ((T_k + 63) / 64) * 8192 < ((int64_t)1 << 31), DIT_E_UNSUPPORTED,
          "H * ceil(T_k/64) * 8192 must be below 2^31");
    return DIT_OK;
}

int dit_attn_quantize(const void* q, const void* k, const void* v, int64_t T_q, int64_t T_k, int32_t H,
                      int64_t ldq, int64_t ldk, int64_t ldv, void* buf, size_t buf_bytes, void* stream) {
    int s = check_q8_shape(T_q, T_k, H);
    if (s) return s;
    const int64_t row = (int64_t)H * 128;
    CHECK(ldq >= row && ldk >= row && ldv >= row, DIT_E_SHAPE, "row strides must be >= H*128");
    CHECK(ldq % 8 == 0 && ldk % 8 == 0 && ldv % 8 == 0, DIT_E_ALIGN, "row strides must be multiples of 8");
    CHECK(buf != nullptr && buf_bytes >= dit_attn_q8_bytes(T_q, T_k, H, nullptr), DIT_E_WORKSPACE,
          "buf needs %zu bytes", dit_attn_q8_bytes(T_q, T_k, H, nullptr));
    CHECK((T_q == 0 || q) && (T_k == 0 || (k && v)), DIT_E_NULL, "q, k and v must be non-NULL");
    CHECK(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(buf), DIT_E_ALIGN,
          "q, k, v and buf must be 16-byte aligned");
    RUN(launch_attn_quantize(q, k, v, T_q, T_k, H, ldq, ldk, ldv, buf, S(stream)), "attn_quantize");
    return DIT_OK;
}

int block_causal_attention_q8(const void* buf, int64_t T_q, int64_t T_k, int32_t H, void* o, int64_t ldo,
                              const int32_t* seg_len, int32_t n_seg, float sm_scale, void* stream) {
    int s = check_q8_shape(T_q, T_k, H);
    if (s) return s;
    CHECK(ldo >= (int64_t)H * 128 && ldo % 8 == 0 && ldo < ((int64_t)1 << 31), DIT_E_SHAPE,
          "ldo must be >= H*128, a multiple of 8 and below 2^31");
    s = check_segs(seg_len, n_seg, T_k);
    if (s) return s;
    if (T_q == 0) return DIT_OK;
    CHECK(buf && o, DIT_E_NULL, "buf and o must be non-NULL");
    CHECK(aligned16(buf) && aligned16(o), DIT_E_ALIGN, "buf and o must be 16-byte aligned");
    if (sm_scale <= 0.0f) sm_scale = 1.0f / std::sqrt(128.0f);
    RUN(launch_attention_q8(buf, T_q, T_k, H, o, ldo, make_attn_segs(seg_len, n_seg), sm_scale, S(stream)),
        "attention_q8");
    return DIT_OK;
}

namespace {

struct Plan {
    size_t h, a8, sa, qkv, q, o, o8, so, g, g8, sg, split, aq, total;
};

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

Plan plan(const dit_block_config* cfg, int64_t T, int64_t T_k) {
    const size_t act = cfg->mode == DIT_MODE_F32 ? 4 : 2;
    const size_t D = cfg->D, F = cfg->F;
    const bool q8 = cfg->mode == DIT_MODE_W8A8;
    Plan p{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += up256(bytes);
        return at;
    };
    p.h = take(q8 ? 0 : T * D * act);
    p.a8 = take(q8 ? T * D : 0);
    p.sa = take(q8 ? T * 4 : 0);
    p.qkv = take(T * 3 * D * act);
    p.q = take(T * D * act);
    p.o = take(T * D * act);
    p.o8 = take(q8 ? T * D : 0);
    p.so = take(q8 ? T * 4 : 0);
    p.g = take(T * F * act);
    p.g8 = take(q8 ? T * F : 0);
    p.sg = take(q8 ? T * 4 : 0);
    // K-split partial sums of the MFMA GEMMs (int32 for W8A8, fp32 for bf16)
    p.split = take(cfg->mode != DIT_MODE_F32 ? (size_t)kSplitPartialBytes : 0);
    p.aq = take(cfg->attn_quant ? attn_q8_layout(T, T_k, cfg->H).total : 0);
    p.total = off;
    return p;
}

int check_cfg(const dit_block_config* cfg) {
    CHECK(cfg != nullptr, DIT_E_NULL, "cfg is NULL");
    CHECK(cfg->mode >= DIT_MODE_F32 && cfg->mode <= DIT_MODE_W8A8, DIT_E_DTYPE, "unknown mode %d", cfg->mode);
    CHECK(cfg->head_dim == 128, DIT_E_UNSUPPORTED, "head_dim must be 128");
    CHECK(cfg->H >= 1 && (int64_t)cfg->D == (int64_t)cfg->H * 128, DIT_E_SHAPE, "D must equal H*128");
    CHECK(cfg->D % 256 == 0 && cfg->D <= 8192, DIT_E_UNSUPPORTED, "D must be a multiple of 256, <= 8192");
    CHECK(cfg->F >= 256 && cfg->F % 256 == 0 && cfg->F <= 16384, DIT_E_UNSUPPORTED,
          "F must be a multiple of 256 in [256, 16384]");
    CHECK(cfg->ln_eps >= 0.0f && cfg->qk_eps >= 0.0f, DIT_E_SHAPE, "eps must be >= 0");
    CHECK(cfg->attn_quant == 0 || cfg->attn_quant == 1, DIT_E_SHAPE, "attn_quant must be 0 or 1");
    CHECK(cfg->attn_quant == 0 || cfg->mode != DIT_MODE_F32, DIT_E_DTYPE,
          "int8/fp8 attention needs the bf16 or W8A8 mode");
    return DIT_OK;
}

int check_weights(const dit_block_config* cfg, const dit_block_weights* w) {
    CHECK(w != nullptr, DIT_E_NULL, "weights is NULL");
    CHECK(w->w_qkv && w->w_o && w->w_1 && w->w_2, DIT_E_NULL, "a weight matrix is NULL");
    CHECK(w->b_qkv && w->b_o && w->b_1 && w->b_2, DIT_E_NULL, "a bias is NULL");
    CHECK(w->g_q && w->g_k, DIT_E_NULL, "g_q or g_k is NULL");
    if (cfg->mode == DIT_MODE_W8A8)
        CHECK(w->s_qkv && w->s_o && w->s_1 && w->s_2, DIT_E_NULL, "W8A8 needs the weight scales");
    CHECK(aligned16(w->w_qkv) && aligned16(w->w_o) && aligned16(w->w_1) && aligned16(w->w_2), DIT_E_ALIGN,
          "weights must be 16-byte aligned");
    return DIT_OK;
}

int check_io(const dit_block_config* cfg, const dit_block_io* io) {
    CHECK(io != nullptr, DIT_E_NULL, "io is NULL");
    CHECK(io->T_q >= 0 && io->T_q <= io->T_k, DIT_E_SHAPE, "need 0 <= T_q <= T_k");
    CHECK(io->T_k < ((int64_t)1 << 31), DIT_E_UNSUPPORTED, "T_k must be below 2^31");
    int s = check_segs(io->seg_len, io->n_seg, io->T_k);
    if (s) return s;
    if (cfg->attn_quant) {
        s = check_q8_shape(io->T_q, io->T_k, cfg->H);
        if (s) return s;
    }
    CHECK(io->n_mod >= 1, DIT_E_SHAPE, "n_mod must be >= 1");
    CHECK(io->mod_of_seg != nullptr, DIT_E_NULL, "mod_of_seg is NULL");
    for (int i = 0; i < io->n_seg; ++i)
        CHECK(io->mod_of_seg[i] >= 0 && io->mod_of_seg[i] < io->n_mod, DIT_E_SHAPE,
              "mod_of_seg[%d]=%d outside [0, n_mod)", i, io->mod_of_seg[i]);
    if (io->T_q == 0) return DIT_OK;
    CHECK(io->x && io->mod && io->cos_t && io->sin_t && io->k_cache && io->v_cache, DIT_E_NULL,
          "x, mod, cos_t, sin_t, k_cache and v_cache must be non-NULL");
    CHECK(aligned16(io->x) && aligned16(io->k_cache) && aligned16(io->v_cache), DIT_E_ALIGN,
          "x and the caches must be 16-byte aligned");
    return DIT_OK;
}

int block_impl(const dit_block_config* cfg, const dit_block_weights* w, const dit_block_io* io,
               void* k_cache, void* v_cache, uint8_t* ws, hipStream_t st) {
    const int64_t T = io->T_q, D = cfg->D, F = cfg->F;
    const int H = cfg->H;
    const int mode = cfg->mode;
    const bool f32 = mode == DIT_MODE_F32, q8 = mode == DIT_MODE_W8A8;
    const bool bf = !f32;
    const size_t act = f32 ? 4 : 2;
    const Plan p = plan(cfg, T, io->T_k);
    const int64_t row_off = io->T_k - io->T_q;
    const SegMap sm = make_segmap(io->seg_len, io->mod_of_seg, io->n_seg, row_off);
    const AttnSegs segs = make_attn_segs(io->seg_len, io->n_seg);
    const int64_t mstride = 6 * D;
    void* x = io->x;
    void* h = ws + p.h;
    int8_t* a8 = (int8_t*)(ws + p.a8);
    float* sa = (float*)(ws + p.sa);
    void* qkv = ws + p.qkv;
    void* qb = ws + p.q;
    void* ob = ws + p.o;
    int8_t* o8 = (int8_t*)(ws + p.o8);
    float* so = (float*)(ws + p.so);
    void* gb = ws + p.g;
    int8_t* g8 = (int8_t*)(ws + p.g8);
    float* sg = (float*)(ws + p.sg);
    uint8_t* kc = (uint8_t*)k_cache + (size_t)row_off * D * act;
    uint8_t* vc = (uint8_t*)v_cache + (size_t)row_off * D * act;

    int32_t* split_partial = (int32_t*)(ws + p.split);
    auto gemm = [&](const void* A, const int8_t* A8, const float* As, const void* Wt, const float* Ws,
                    int64_t N, int64_t K, const EpiParams& ep) -> hipError_t {
        if (q8) {
            EpiParams e = ep;
            e.a_scale = As;
            e.w_scale = Ws;
            e.split_partial = split_partial;
            e.split_bytes = kSplitPartialBytes;
            return launch_gemm_i8(A8, (const int8_t*)Wt, T, N, K, e, st);
        }
        if (bf) {
            EpiParams e = ep;
            e.split_partial = split_partial;
            e.split_bytes = kSplitPartialBytes;
            return launch_gemm_bf16(A, K, Wt, T, N, K, e, st);
        }
        return launch_gemm_f32((const float*)A, K, (const float*)Wt, T, N, K, ep, st);
    };

    // S1: adaLN prologue 1 (fused per-token quantization in W8A8 mode)
    {
    ProfScope ps(DIT_SITE_ADALN1, st);
    RUN(launch_adaln(x, bf, T, D, io->mod + 0 * D, io->mod + 1 * D, mstride, sm, cfg->ln_eps, q8 ? nullptr : h,
                     q8 ? a8 : nullptr, sa, st),
        "adaln1");
    }
    // S2 + S3: QKV linear; Q/K RMSNorm + RoPE and the K/V cache rows.  In the
    // bf16 modes the norm/RoPE runs in the GEMM's epilogue (the [q|k|v] tile
    // never goes to memory); fp32 mode stores qkv and runs the separate kernel.
    const bool fused = bf && aligned16(w->g_q) && aligned16(w->g_k) && aligned16(io->cos_t) && aligned16(io->sin_t);
    {
        EpiParams ep = store_epi(qkv, 3 * D, bf, w->b_qkv);
        if (fused) {
            ep.kind = EPI_QKV_ROPE;
            ep.q_out = qb;
            ep.k_out = kc;
            ep.v_out = vc;
            ep.g_q = w->g_q;
            ep.g_k = w->g_k;
            ep.cos_t = io->cos_t;
            ep.sin_t = io->sin_t;
            ep.qk_eps = cfg->qk_eps;
            ep.D = D;
        }
        ProfScope ps(DIT_SITE_QKV_GEMM, st);
        RUN(gemm(h, a8, sa, w->w_qkv, w->s_qkv, 3 * D, D, ep), "qkv_gemm");
    }
    if (!fused) {
        ProfScope ps(DIT_SITE_QK_NORM_ROPE, st);
        RUN(launch_qk_norm_rope(qkv, bf, T, H, w->g_q, w->g_k, io->cos_t, io->sin_t, cfg->qk_eps, qb, kc, D, vc,
                                D, st),
            "qk_norm_rope");
    }
    // S4: block-causal attention over the whole cache
    const float scale = 1.0f / std::sqrt(128.0f);
    if (cfg->attn_quant) {
        {
            ProfScope ps(DIT_SITE_ATTN_QUANT, st);
            RUN(launch_attn_quantize(qb, k_cache, v_cache, T, io->T_k, H, D, D, D, ws + p.aq, st, false),
                "attn_quantize");
        }
        ProfScope ps(DIT_SITE_ATTENTION, st);
        RUN(launch_attention_q8(ws + p.aq, T, io->T_k, H, ob, D, segs, scale, st, qb, D), "attention_q8");
    } else {
    ProfScope ps(DIT_SITE_ATTENTION, st);
    if (bf)
        RUN(launch_attention_bf16(qb, k_cache, v_cache, ob, T, io->T_k, H, D, D, D, D, segs, scale, st),
            "attention");
    else
        RUN(launch_attention_f32((const float*)qb, (const float*)k_cache, (const float*)v_cache, (float*)ob, T,
                                 io->T_k, H, D, D, D, D, segs, scale, st),
            "attention");
    }
    // S5 + S6: quantize o, out-projection with gated residual into x
    if (q8) {
        ProfScope ps(DIT_SITE_QUANT_O, st);
        RUN(launch_quantize_rows(ob, true, T, D, D, o8, so, st), "quantize_o");
    }
    {
        EpiParams ep{};
        ep.kind = EPI_RESID;
        ep.act_bf16 = bf;
        ep.bias = w->b_o;
        ep.x = x;
        ep.ldx = D;
        ep.gate = io->mod + 2 * D;
        ep.gate_stride = mstride;
        ep.sm = sm;
        ProfScope ps(DIT_SITE_OUT_GEMM, st);
        RUN(gemm(ob, o8, so, w->w_o, w->s_o, D, D, ep), "out_gemm");
    }
    // S7: adaLN prologue 2
    {
    ProfScope ps(DIT_SITE_ADALN2, st);
    RUN(launch_adaln(x, bf, T, D, io->mod + 3 * D, io->mod + 4 * D, mstride, sm, cfg->ln_eps, q8 ? nullptr : h,
                     q8 ? a8 : nullptr, sa, st),
        "adaln2");
    }
    // S8: MLP up + GELU.  W8A8: the up GEMM stores u (bf16) and the GELU is
    // applied in the HBM-bound quantization pass of S9, which has spare ALU;
    // otherwise the GELU runs in the GEMM epilogue.
    {
        EpiParams ep{};
        ep.kind = q8 ? EPI_STORE : EPI_GELU;
        ep.act_bf16 = bf;
        ep.y_bf16 = bf;
        ep.bias = w->b_1;
        ep.y = gb;
        ep.ldy = F;
        ProfScope ps(DIT_SITE_UP_GEMM, st);
        RUN(gemm(h, a8, sa, w->w_1, w->s_1, F, D, ep), "up_gemm");
    }
    // S9 + S10: (GELU +) quantize g, MLP down with gated residual into x
    if (q8) {
        ProfScope ps(DIT_SITE_QUANT_G, st);
        RUN(launch_gelu_quantize_rows(gb, T, F, g8, sg, st), "gelu_quantize_g");
    }
    {
        EpiParams ep{};
        ep.kind = EPI_RESID;
        ep.act_bf16 = bf;
        ep.bias = w->b_2;
        ep.x = x;
        ep.ldx = D;
        ep.gate = io->mod + 5 * D;
        ep.gate_stride = mstride;
        ep.sm = sm;
        ProfScope ps(DIT_SITE_DOWN_GEMM, st);
        RUN(gemm(gb, g8, sg, w->w_2, w->s_2, D, F, ep), "down_gemm");
    }
    return DIT_OK;
}

struct GatedPlan {
    size_t h, a8, sa, za, qkv, q, o, u, g, split, aq, wx, total;
};

GatedPlan gated_plan(const dit_block_config* cfg, int64_t T, int64_t T_k) {
    const size_t D = cfg->D, F = cfg->F;
    GatedPlan p{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += up256(bytes);
        return at;
    };
    p.h = take(T * D * 2);
    p.a8 = take(T * std::max(D, F));
    p.sa = take(T * 4);
    p.za = take(T * 4);
    p.qkv = take(T * 3 * D * 2);   // only used when the fused QK epilogue is not available
    p.q = take(T * D * 2);
    p.o = take(T * D * 2);
    p.u = take(T * F * 2);
    p.g = take(T * F * 2);
    p.split = take((size_t)kSplitPartialBytes);
    p.aq = take(cfg->attn_quant ? attn_q8_layout(T, T_k, cfg->H).total : 0);
    p.wx = take(std::max(2 * D * D, F * D) * 2);   // MXFP4 weights expanded for one linear
    p.total = off;
    return p;
}

int check_linear(const dit_linear& L, const char* name) {
    CHECK(L.w != nullptr, DIT_E_NULL, "linear %s: w is NULL", name);
    CHECK(aligned16(L.w), DIT_E_ALIGN, "linear %s: w must be 16-byte aligned", name);
    if (L.s) CHECK(L.wsum && aligned16(L.wsum), DIT_E_NULL, "linear %s: int8 needs a 16-byte aligned wsum", name);
    CHECK(!(L.s && L.mx_scale), DIT_E_SHAPE, "linear %s: int8 and MXFP4 at once", name);
    return DIT_OK;
}

int gated_impl(const dit_block_config* cfg, const dit_gated_block_weights* w, const dit_block_io* io,
               uint8_t* ws, hipStream_t st) {
    const int64_t T = io->T_q, D = cfg->D, F = cfg->F;
    const int H = cfg->H;
    const GatedPlan p = gated_plan(cfg, T, io->T_k);
    const int64_t row_off = io->T_k - io->T_q;
    const SegMap sm = make_segmap(io->seg_len, io->mod_of_seg, io->n_seg, row_off);
    const AttnSegs segs = make_attn_segs(io->seg_len, io->n_seg);
    const int64_t mstride = 6 * D;
    void* x = io->x;
    void* h = ws + p.h;
    int8_t* a8 = (int8_t*)(ws + p.a8);
    float* sa = (float*)(ws + p.sa);
    int32_t* za = (int32_t*)(ws + p.za);
    void* qb = ws + p.q;
    void* ob = ws + p.o;
    void* ub = ws + p.u;
    void* gb = ws + p.g;
    uint8_t* kc = (uint8_t*)io->k_cache + (size_t)row_off * D * 2;
    uint8_t* vc = (uint8_t*)io->v_cache + (size_t)row_off * D * 2;
    int32_t* split_partial = (int32_t*)(ws + p.split);
    // one linear: int8 codes of the activation (already in a8/sa/za) if the
    // linear is W8A8, else the bf16 activation A
    auto lin = [&](const dit_linear& L, const void* A, int64_t N, int64_t K, const EpiParams& ep) -> hipError_t {
        EpiParams e = ep;
        e.split_partial = split_partial;
        e.split_bytes = kSplitPartialBytes;
        if (L.mx_scale) {
            if (gemm_bf16_direct_mxfp4(T, N, K, K, true)) {
                // decoded in the GEMM's operand staging
                e.w_mx_scale = L.mx_scale;
                return launch_gemm_bf16(A, K, L.w, T, N, K, e, st);
            }
            const hipError_t x = launch_mxfp4_expand((const uint8_t*)L.w, L.mx_scale, N, K, ws + p.wx, st);
            if (x != hipSuccess) return x;
            return launch_gemm_bf16(A, K, ws + p.wx, T, N, K, e, st);
        }
        if (!L.s) return launch_gemm_bf16(A, K, L.w, T, N, K, e, st);
        e.a_scale = sa;
        e.a_zero = za;
        e.w_scale = L.s;
        e.w_sum = L.wsum;
        return launch_gemm_i8(a8, (const int8_t*)L.w, T, N, K, e, st);
    };
    auto quant = [&](const void* A, int64_t K) -> hipError_t {
        return launch_quantize_rows_asym(A, true, T, K, K, a8, sa, za, st);
    };
    // adaLN prologue: h (bf16) when a bf16 or MXFP4 linear reads it, and the
    // asymmetric codes of h when an int8 linear does (fused into the adaLN
    // pass where its kernel takes the shape, else a second pass over h)
    auto prologue = [&](const float* shift, const float* scale, const dit_linear& l1,
                        const dit_linear& l2) -> hipError_t {
        const bool need_q = l1.s || l2.s, need_h = !l1.s || !l2.s;
        void* ho = need_h ? h : nullptr;
        if (need_q && adaln_fuses_asym(D, mstride, x, shift, scale, ho, a8))
            return launch_adaln_asym(x, T, D, shift, scale, mstride, sm, cfg->ln_eps, ho, a8, sa, za, st);
        const hipError_t e = launch_adaln(x, true, T, D, shift, scale, mstride, sm, cfg->ln_eps, h, nullptr,
                                          nullptr, st);
        if (e != hipSuccess || !need_q) return e;
        return quant(h, D);
    };

    {
        ProfScope ps(DIT_SITE_ADALN1, st);
        RUN(prologue(io->mod + 0 * D, io->mod + 1 * D, w->qk, w->v), "adaln1");
    }
    {
        // Q/K: RMSNorm + RoPE in the GEMM epilogue (columns [0, D) q, [D, 2D) k)
        EpiParams ep = store_epi(ws + p.qkv, 3 * D, true, w->qk.b);
        ep.kind = EPI_QKV_ROPE;
        ep.q_out = qb;
        ep.k_out = kc;
        ep.v_out = ob;   // unused columns of the unfused fallback land in o (overwritten by S4)
        ep.g_q = w->g_q;
        ep.g_k = w->g_k;
        ep.cos_t = io->cos_t;
        ep.sin_t = io->sin_t;
        ep.qk_eps = cfg->qk_eps;
        ep.D = D;
        ProfScope ps(DIT_SITE_QKV_GEMM, st);
        RUN(lin(w->qk, h, 2 * D, D, ep), "qk_gemm");
        RUN(lin(w->v, h, D, D, store_epi(vc, D, true, w->v.b)), "v_gemm");
    }
    const float scale = 1.0f / std::sqrt(128.0f);
    if (cfg->attn_quant) {
        {
            ProfScope ps(DIT_SITE_ATTN_QUANT, st);
            RUN(launch_attn_quantize(qb, io->k_cache, io->v_cache, T, io->T_k, H, D, D, D, ws + p.aq, st, false),
                "attn_quantize");
        }
        ProfScope ps(DIT_SITE_ATTENTION, st);
        RUN(launch_attention_q8(ws + p.aq, T, io->T_k, H, ob, D, segs, scale, st, qb, D), "attention_q8");
    } else {
        ProfScope ps(DIT_SITE_ATTENTION, st);
        RUN(launch_attention_bf16(qb, io->k_cache, io->v_cache, ob, T, io->T_k, H, D, D, D, D, segs, scale, st),
            "attention");
    }
    EpiParams resid{};
    resid.kind = EPI_RESID;
    resid.act_bf16 = 1;
    resid.x = x;
    resid.ldx = D;
    resid.gate_stride = mstride;
    resid.sm = sm;
    {
        if (w->o.s) {
            ProfScope pq(DIT_SITE_QUANT_O, st);
            RUN(quant(ob, D), "quantize o");
        }
        EpiParams ep = resid;
        ep.bias = w->o.b;
        ep.gate = io->mod + 2 * D;
        ProfScope ps(DIT_SITE_OUT_GEMM, st);
        RUN(lin(w->o, ob, D, D, ep), "out_gemm");
    }
    {
        ProfScope ps(DIT_SITE_ADALN2, st);
        RUN(prologue(io->mod + 3 * D, io->mod + 4 * D, w->proj, w->gate), "adaln2");
    }
    {
        // gated MLP: u = proj(h2) (bf16), then g = u * GELU(gate(h2)) in the gate GEMM's epilogue
        ProfScope ps(DIT_SITE_UP_GEMM, st);
        RUN(lin(w->proj, h, F, D, store_epi(ub, F, true, w->proj.b)), "proj_gemm");
        EpiParams ep = store_epi(gb, F, true, w->gate.b);
        ep.kind = EPI_GELU;
        ep.gmul = ub;
        ep.ldgm = F;
        RUN(lin(w->gate, h, F, D, ep), "gate_gemm");
    }
    {
        if (w->down.s) {
            ProfScope pq(DIT_SITE_QUANT_G, st);
            RUN(quant(gb, F), "quantize g");
        }
        EpiParams ep = resid;
        ep.bias = w->down.b;
        ep.gate = io->mod + 5 * D;
        ProfScope ps(DIT_SITE_DOWN_GEMM, st);
        RUN(lin(w->down, gb, D, F, ep), "down_gemm");
    }
    return DIT_OK;
}

}  // namespace

size_t dit_block_workspace_bytes(const dit_block_config* cfg, int64_t T_q, int64_t T_k) {
    if (!cfg || T_q < 0 || T_k < T_q) return 0;
    return plan(cfg, T_q, T_k).total;
}

int dit_block_forward(const dit_block_config* cfg, const dit_block_weights* w, const dit_block_io* io,
                      void* workspace, size_t workspace_bytes, void* stream) {
    int s = check_cfg(cfg);
    if (s) return s;
    s = check_weights(cfg, w);
    if (s) return s;
    s = check_io(cfg, io);
    if (s) return s;
    if (io->T_q == 0) return DIT_OK;
    const size_t need = plan(cfg, io->T_q, io->T_k).total;
    CHECK(workspace != nullptr && workspace_bytes >= need, DIT_E_WORKSPACE, "workspace needs %zu bytes", need);
    CHECK(aligned16(workspace), DIT_E_ALIGN, "workspace must be 16-byte aligned");
    return block_impl(cfg, w, io, io->k_cache, io->v_cache, (uint8_t*)workspace, S(stream));
}

int dit_stack_forward(const dit_block_config* cfg, const dit_block_weights* weights, int32_t n_blocks,
                      const dit_block_io* io, void* const* k_caches, void* const* v_caches, void* workspace,
                      size_t workspace_bytes, void* stream) {
    int s = check_cfg(cfg);
    if (s) return s;
    CHECK(n_blocks >= 0 && (n_blocks == 0 || weights != nullptr), DIT_E_NULL, "weights is NULL");
    CHECK(k_caches != nullptr && v_caches != nullptr, DIT_E_NULL, "cache arrays are NULL");
    for (int b = 0; b < n_blocks; ++b) {
        s = check_weights(cfg, &weights[b]);
        if (s) return s;
        CHECK(k_caches[b] && v_caches[b], DIT_E_NULL, "cache of block %d is NULL", b);
        CHECK(aligned16(k_caches[b]) && aligned16(v_caches[b]), DIT_E_ALIGN, "caches must be 16-byte aligned");
    }
    dit_block_io one = *io;
    one.k_cache = n_blocks ? k_caches[0] : io->k_cache;
    one.v_cache = n_blocks ? v_caches[0] : io->v_cache;
    s = check_io(cfg, &one);
    if (s) return s;
    if (io->T_q == 0 || n_blocks == 0) return DIT_OK;
    const size_t need = plan(cfg, io->T_q, io->T_k).total;
    CHECK(workspace != nullptr && workspace_bytes >= need, DIT_E_WORKSPACE, "workspace needs %zu bytes", need);
    CHECK(aligned16(workspace), DIT_E_ALIGN, "workspace must be 16-byte aligned");
    for (int b = 0; b < n_blocks; ++b) {
        s = block_impl(cfg, &weights[b], io, k_caches[b], v_caches[b], (uint8_t*)workspace, S(stream));
        if (s) return s;
    }
    return DIT_OK;
}

size_t dit_gated_block_workspace_bytes(const dit_block_config* cfg, int64_t T_q, int64_t T_k) {
    if (!cfg || T_q < 0 || T_k < T_q) return 0;
    return gated_plan(cfg, T_q, T_k).total;
}

int dit_block_forward_gated(const dit_block_config* cfg, const dit_gated_block_weights* w, const dit_block_io* io,
                            void* workspace, size_t workspace_bytes, void* stream) {
    int s = check_cfg(cfg);
    if (s) return s;
    CHECK(cfg->mode == DIT_MODE_BF16, DIT_E_DTYPE, "the gated block takes bf16 activations (mode BF16)");
    CHECK(w != nullptr, DIT_E_NULL, "weights is NULL");
    const dit_linear* all[6] = {&w->qk, &w->v, &w->o, &w->proj, &w->gate, &w->down};
    const char* names[6] = {"qk", "v", "o", "proj", "gate", "down"};
    for (int i = 0; i < 6; ++i) {
        s = check_linear(*all[i], names[i]);
        if (s) return s;
    }
    CHECK(w->g_q && w->g_k && aligned16(w->g_q) && aligned16(w->g_k), DIT_E_ALIGN,
          "g_q and g_k must be non-NULL and 16-byte aligned");
    CHECK(w->qk.b == nullptr || aligned16(w->qk.b), DIT_E_ALIGN, "qk bias must be 16-byte aligned");
    s = check_io(cfg, io);
    if (s) return s;
    if (io->T_q == 0) return DIT_OK;
    CHECK(aligned16(io->cos_t) && aligned16(io->sin_t), DIT_E_ALIGN, "cos_t and sin_t must be 16-byte aligned");
    const size_t need = gated_plan(cfg, io->T_q, io->T_k).total;
    CHECK(workspace != nullptr && workspace_bytes >= need, DIT_E_WORKSPACE, "workspace needs %zu bytes", need);
    CHECK(aligned16(workspace), DIT_E_ALIGN, "workspace must be 16-byte aligned");
    return gated_impl(cfg, w, io, (uint8_t*)workspace, S(stream));
}

size_t dit_velocity_workspace_bytes(const dit_block_config* cfg, int64_t T_q, int64_t T_k, int64_t N,
                                    int32_t C_lat) {
    if (!cfg || T_q < 0 || T_k < T_q || N < 0 || C_lat < 0) return 0;
    const size_t es = cfg->mode == DIT_MODE_F32 ? 4 : 2;
    return up256((size_t)T_q * cfg->D * es) + up256((size_t)T_q * C_lat * es) + up256((size_t)N * cfg->D * es) +
           plan(cfg, T_q, T_k).total;
}

int dit_velocity_forward(const dit_block_config* cfg, const dit_block_weights* blocks, int32_t n_blocks,
                         const dit_head_weights* head, const dit_velocity_io* io, void* workspace,
                         size_t workspace_bytes, void* stream) {
    int s = check_cfg(cfg);
    if (s) return s;
    CHECK(head != nullptr && io != nullptr, DIT_E_NULL, "head and io must be non-NULL");
    CHECK(n_blocks >= 0 && (n_blocks == 0 || blocks != nullptr), DIT_E_NULL, "blocks is NULL");
    CHECK(head->w_img_in && head->w_proj_out, DIT_E_NULL, "w_img_in and w_proj_out must be non-NULL");
    CHECK(head->C_lat >= 64 && head->C_lat % 64 == 0, DIT_E_UNSUPPORTED, "C_lat must be a positive multiple of 64");
    CHECK(io->L_txt >= 0 && io->R >= 0 && io->N >= 1, DIT_E_SHAPE, "need L_txt >= 0, R >= 0, N >= 1");
    const int64_t T_k = io->L_txt + io->R + io->N;
    CHECK(io->T_q == T_k || io->T_q == io->N, DIT_E_SHAPE, "T_q must be L_txt + R + N or N");
    const bool full = io->T_q == T_k;
    if (full && io->L_txt > 0) {
        CHECK(head->w_txt_in && io->txt_feats, DIT_E_NULL, "text rows need w_txt_in and txt_feats");
        CHECK(head->C_txt >= 64 && head->C_txt % 64 == 0, DIT_E_UNSUPPORTED, "C_txt must be a positive multiple of 64");
        CHECK(aligned16(io->txt_feats) && aligned16(head->w_txt_in), DIT_E_ALIGN, "txt_feats/w_txt_in misaligned");
    }
    if (full && io->R > 0) CHECK(io->ref_latent != nullptr, DIT_E_NULL, "reference rows need ref_latent");
    CHECK(io->latent && io->vel && io->mod_final, DIT_E_NULL, "latent, vel and mod_final must be non-NULL");
    CHECK(aligned16(io->latent) && aligned16(io->vel) && (!io->ref_latent || aligned16(io->ref_latent)) &&
              aligned16(head->w_img_in) && aligned16(head->w_proj_out) && aligned16(io->mod_final),
          DIT_E_ALIGN, "latents, vel, head weights and mod_final must be 16-byte aligned");
    CHECK(io->k_caches && io->v_caches, DIT_E_NULL, "cache arrays are NULL");
    dit_block_io bio{};
    bio.mod = io->mod;
    bio.n_mod = io->n_mod;
    bio.mod_of_seg = io->mod_of_seg;
    bio.cos_t = io->cos_t;
    bio.sin_t = io->sin_t;
    bio.seg_len = io->seg_len;
    bio.n_seg = io->n_seg;
    bio.T_q = io->T_q;
    bio.T_k = T_k;
    for (int b = 0; b < n_blocks; ++b) {
        s = check_weights(cfg, &blocks[b]);
        if (s) return s;
        CHECK(io->k_caches[b] && io->v_caches[b], DIT_E_NULL, "cache of block %d is NULL", b);
        CHECK(aligned16(io->k_caches[b]) && aligned16(io->v_caches[b]), DIT_E_ALIGN, "caches must be 16-byte aligned");
    }
    const size_t need = dit_velocity_workspace_bytes(cfg, io->T_q, T_k, io->N, head->C_lat);
    CHECK(workspace != nullptr && workspace_bytes >= need, DIT_E_WORKSPACE, "workspace needs %zu bytes", need);
    CHECK(aligned16(workspace), DIT_E_ALIGN, "workspace must be 16-byte aligned");
    uint8_t* ws = (uint8_t*)workspace;
    const int64_t D = cfg->D, C = head->C_lat, T_q = io->T_q, N = io->N;
    const bool f32 = cfg->mode == DIT_MODE_F32;
    const size_t es = f32 ? 4 : 2;
    uint8_t* x = ws;
    uint8_t* latc = x + up256((size_t)T_q * D * es);
    uint8_t* hf = latc + up256((size_t)T_q * C * es);
    uint8_t* blk = hf + up256((size_t)N * D * es);
    bio.x = x;
    bio.k_cache = n_blocks ? io->k_caches[0] : latc;   // checked below only when blocks run
    bio.v_cache = n_blocks ? io->v_caches[0] : latc;
    s = check_io(cfg, &bio);
    if (s) return s;
    hipStream_t st = S(stream);
    // y[M, Nn] = a[M, K] w[Nn, K]^T + b in the activation dtype.  The bf16
    // linears of the head and tail use the blocks' K-split region (free
    // outside the blocks), so launches with few tiles (txt_in on the text
    // rows, proj_out's 64 columns) split along K instead of running on a few CUs.
    int32_t* head_split = f32 ? nullptr : (int32_t*)(blk + plan(cfg, T_q, T_k).split);
    auto linear = [&](const void* a, int64_t M, int64_t K, const void* w, const float* b, void* y,
                      int64_t Nn) -> hipError_t {
        if (M == 0) return hipSuccess;
        EpiParams ep = store_epi(y, Nn, !f32, b);
        if (f32) return launch_gemm_f32((const float*)a, K, (const float*)w, M, Nn, K, ep, st);
        ep.split_partial = head_split;
        ep.split_bytes = kSplitPartialBytes;
        return launch_gemm_bf16(a, K, w, M, Nn, K, ep, st);
    };
    // latent rows -> activation dtype (the fp32 mode reads the fp32 latent directly)
    auto lat_rows = [&](const float* src, int64_t rows, uint8_t* dst) -> const void* {
        if (f32) return src;
        (void)launch_cast(src, false, dst, true, rows * C, st);
        return dst;
    };
    const int64_t tgt = T_q - N;   // first target row among the computed rows
    if (full) {
        if (io->L_txt > 0)
            RUN(linear(io->txt_feats, io->L_txt, head->C_txt, head->w_txt_in, head->b_txt_in, x, D), "txt_in");
        if (io->R > 0) {
            const void* a = lat_rows(io->ref_latent, io->R, latc);
            RUN(hipGetLastError(), "cast ref_latent");
            RUN(linear(a, io->R, C, head->w_img_in, head->b_img_in, x + (size_t)io->L_txt * D * es, D), "img_in ref");
        }
    }
    {
        const void* a = lat_rows(io->latent, N, latc + (size_t)(full ? io->R : 0) * C * es);
        RUN(hipGetLastError(), "cast latent");
        RUN(linear(a, N, C, head->w_img_in, head->b_img_in, x + (size_t)tgt * D * es, D), "img_in");
    }
    for (int b = 0; b < n_blocks; ++b) {
        s = block_impl(cfg, &blocks[b], &bio, io->k_caches[b], io->v_caches[b], blk, st);
        if (s) return s;
    }
    SegMap sm{};
    sm.end[0] = N;
    sm.set[0] = 0;
    sm.n = 1;
    RUN(launch_adaln(x + (size_t)tgt * D * es, !f32, N, D, io->mod_final, io->mod_final + D, 0, sm, cfg->ln_eps,
                     hf, nullptr, nullptr, st),
        "final adaln");
    RUN(linear(hf, N, D, head->w_proj_out, head->b_proj_out, io->vel, C), "proj_out");
    return DIT_OK;
}

int dit_profile_begin(int32_t capacity) {
    CHECK(!g_prof.on, DIT_E_UNSUPPORTED, "profiling already active");
    CHECK(capacity >= 1 && capacity <= (1 << 20), DIT_E_SHAPE, "capacity outside [1, 2^20]");
    g_prof.ev.assign(2 * (size_t)capacity, nullptr);
    g_prof.site.assign((size_t)capacity, 0);
    for (auto& e : g_prof.ev) {
        hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) {
            for (auto& f : g_prof.ev)
                if (f) (void)hipEventDestroy(f);
            g_prof.ev.clear();
            return hip_status(r, "hipEventCreate");
        }
    }
    g_prof.cap = capacity;
    g_prof.used = 0;
    g_prof.on = true;
    return DIT_OK;
}

int dit_profile_end(double* ms_out, int64_t* count_out, int32_t n_sites) {
    CHECK(g_prof.on, DIT_E_UNSUPPORTED, "profiling not active");
    CHECK(ms_out && count_out, DIT_E_NULL, "ms_out and count_out must be non-NULL");
    CHECK(n_sites >= 1, DIT_E_SHAPE, "n_sites must be >= 1");
    for (int i = 0; i < n_sites; ++i) {
        ms_out[i] = 0.0;
        count_out[i] = 0;
    }
    int status = DIT_OK;
    for (int i = 0; i < g_prof.used; ++i) {
        float ms = 0.0f;
        hipError_t r = hipEventSynchronize(g_prof.ev[2 * i + 1]);
        if (r == hipSuccess) r = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
        if (r != hipSuccess) {
            status = hip_status(r, "hipEventElapsedTime");
            break;
        }
        const int s = g_prof.site[i];
        if (s < n_sites) {
            ms_out[s] += ms;
            count_out[s] += 1;
        }
    }
    for (auto& e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.on = false;
    g_prof.used = g_prof.cap = 0;
    return status;
}

const char* dit_site_name(int32_t site) {
    static const char* names[DIT_N_SITES] = {"adaln1", "qkv_gemm", "qk_norm_rope", "attention", "quant_o",
                                             "out_gemm", "adaln2", "up_gemm", "quant_g", "down_gemm",
                                             "attn_quant"};
    return (site >= 0 && site < DIT_N_SITES) ? names[site] : "unknown";
}

}  // extern "C"
