// Block-causal flash attention, head dim 128.
//
// Block-causal structure: segments are consecutive key ranges and a query of
// segment s sees segments 0..s, i.e. exactly the key prefix [0, end(s)).  A
// workgroup of 128 queries therefore loops over keys [0, end of its last
// query's segment) and masks only the tiles that cross the first query's
// segment end; fully masked tiles are never visited.
//
// bf16 kernel (gfx950 MFMA 32x32x16 bf16): 4 waves x 32 queries.  Each wave
// computes S^T = K Q^T so that every lane owns one query column: the row max
// and row sum of the online softmax are lane-local except for one exchange
// between lane l and lane l^32.  O^T = V^T P^T accumulates in 64 fp32
// registers per lane.  K tiles sit in LDS key-major, V tiles transposed
// (d-major), both padded for conflict-free reads.  The PV product uses a
// fixed permutation of the 16 keys of each MFMA step (the order in which the
// S^T accumulator hands them to a lane), applied to both operands.
#include "common.h"
#include "kernels.h"

namespace dit {

constexpr int AQ = 128;                 // queries per workgroup
constexpr int AK = 64;                  // keys per tile
constexpr int KS_STRIDE = 128 * 2 + 16; // bytes per key row of the K tile (272 = 16 mod 128:
                                        // eight rows read together hit eight bank groups)
constexpr int VT_STRIDE = AK * 2 + 16;  // bytes per d row of the transposed V tile (144 = 16
                                        // mod 128, same reason)
constexpr int KS_BYTES = AK * KS_STRIDE;
constexpr int VT_BYTES = 128 * VT_STRIDE;
// Lazy rescale of the online softmax: P of a tile is formed against the
// running max as it stands, and the max is only raised (the tile's P formed
// again) when a lane's sum of P over the tile exceeds kRescaleMax, so every P
// that enters the PV product is at most 2^8.  No per-tile max is computed on
// the common path.
constexpr float kRescaleMax = 256.0f;

// Transposed V tile.  Keys are stored in the order the S^T accumulator hands
// them to a lane for the PV product: within each 16-key block, key k sits at
// position (k % 4) + 4*((k / 8) % 2) + 8*((k / 4) % 2), so the 8 keys one
// lane contributes to an MFMA step are 8 consecutive positions (one 16-byte
// read at a constant offset from a per-lane base).  With 144-byte rows the
// operand reads (8 lanes, consecutive d) and the transposing 8-byte writes
// (16 lanes, 16 different key groups of one d row) are both conflict-free.

// Raw buffer resource over the rows [j0, T_k) of one head of K or V: rows at
// or past T_k lie beyond num_records and read as zero.  Rebased per tile, so
// the 32-bit offsets only span one tile.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t kv_rsrc(const __bf16* base, int j0, int T_k, int ld) {
    const int64_t bytes = (int64_t)(T_k - j0 - 1) * ld * 2 + 256;
    const int nrec = bytes <= 0 ? 0 : bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)j0 * ld), 0, nrec, 0x00020000);
}

// Software pipeline over key tiles.  K and V have separate double buffers, K
// one tile ahead: while the MFMA pipe computes the scores of tile t+1, the
// VALU turns the first half of tile t's scores into P (and tile t+2's K goes
// from registers to LDS, tile t+3's K is loaded); then P V of tile t runs,
// its first half beside P of the second key half, its second half while tile
// t+1's V goes from registers to LDS; tile t+2's V is loaded last.  One
// barrier per tile.
__global__ void __launch_bounds__(256, 2)
attn_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ Kg,
                 const __bf16* __restrict__ Vg, __bf16* __restrict__ O, int T_q, int T_k,
                 int ldq, int ldk, int ldv, int ldo, AttnSegs sg, float c_log2, int H, int hg) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * KS_BYTES + 2 * VT_BYTES];
    uint8_t* const kbuf0 = lds;
    uint8_t* const kbuf1 = lds + KS_BYTES;
    uint8_t* const vbuf0 = lds + 2 * KS_BYTES;
    uint8_t* const vbuf1 = lds + 2 * KS_BYTES + VT_BYTES;

    const int nqb = (T_q + AQ - 1) / AQ;
    int qb, h;
    attn_block_order(blockIdx.x, nqb, H, hg, qb, h);
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int hh = lane / 32, lq = lane % 32;
    const int off = T_k - T_q;

    const int q_first = qb * AQ;
    const int q_last = min(q_first + AQ, T_q) - 1;
    const int kv_min = (int)kv_end_of(sg, off + q_first);
    const int kv_hi = (int)kv_end_of(sg, off + q_last);

    const int qi = q_first + wave * 32 + lq;   // this lane's query
    const bool q_ok = qi < T_q;
    const int my_end = q_ok ? (int)kv_end_of(sg, off + qi) : T_k;

    // Q^T fragments (B operand): Q[qi][kb*16 + hh*8 .. +7]
    v8bf qf[8];
    {
        const __bf16* qrow = Q + (size_t)(q_ok ? qi : 0) * ldq + h * 128 + hh * 8;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) qf[kb] = q_ok ? *reinterpret_cast<const v8bf*>(qrow + kb * 16) : v8bf{};
    }

    // global -> register staging.  K: keys kkey + 16 i, chunk kch; V: keys
    // 4*kg .. 4*kg+3, d-chunk dc.  Keys past T_k read as zero: their scores
    // are masked and their P is exactly 0.
    const int kkey = tid / 16, kch = tid % 16;
    const int kg = tid % 16, dc = tid / 16;
    const __bf16* kbase = Kg + h * 128;
    const __bf16* vbase = Vg + h * 128;
    const int koff = kkey * ldk * 2 + kch * 16;
    const int voff = kg * 4 * ldv * 2 + dc * 16;
    // LDS position of this thread's first V key (its 4 keys are consecutive)
    const int vpos = 16 * (kg / 4) + ((kg % 4) == 1 ? 8 : (kg % 4) == 2 ? 4 : (kg % 4) == 3 ? 12 : 0);
    v4i rk[4], rv[4];
    auto gload_k = [&](int j0) {
        const __amdgpu_buffer_rsrc_t r = kv_rsrc(kbase, j0, T_k, ldk);
#pragma unroll
        for (int i = 0; i < 4; ++i) rk[i] = (v4i)__builtin_amdgcn_raw_buffer_load_b128(r, koff, i * 16 * ldk * 2, 0);
    };
    auto gload_v = [&](int j0) {
        const __amdgpu_buffer_rsrc_t r = kv_rsrc(vbase, j0, T_k, ldv);
#pragma unroll
        for (int i = 0; i < 4; ++i) rv[i] = (v4i)__builtin_amdgcn_raw_buffer_load_b128(r, voff, i * ldv * 2, 0);
    };
    auto sstore_k = [&](uint8_t* ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<v4i*>(ks + (kkey + 16 * i) * KS_STRIDE + kch * 16) = rk[i];
    };
    auto sstore_v = [&](uint8_t* vt) {
        // transpose: 4 keys x 8 dims -> 8 rows (d) of 4 keys
        uint8_t* vdst = vt + dc * 8 * VT_STRIDE + vpos * 2;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int w = r / 2;
            const uint32_t sel = (r % 2) ? 0x07060302u : 0x05040100u;
            uint2 packed;
            packed.x = __builtin_amdgcn_perm((uint32_t)rv[1][w], (uint32_t)rv[0][w], sel);
            packed.y = __builtin_amdgcn_perm((uint32_t)rv[3][w], (uint32_t)rv[2][w], sel);
            *reinterpret_cast<uint2*>(vdst + r * VT_STRIDE) = packed;
        }
    };
    // S^T = K Q^T for one tile: two 32-key halves
    auto scores = [&](const uint8_t* ks, v16f(&sacc)[2]) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) sacc[kh] = v16f{};
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const v8bf a = *reinterpret_cast<const v8bf*>(ks + (kh * 32 + lq) * KS_STRIDE + kb * 32 + hh * 16);
                sacc[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kb], sacc[kh], 0, 0, 0);
            }
    };
    // V^T operand reads: chunk (2b + hh) of row d = dt*32 + lq
    const int vrd = lq * VT_STRIDE + hh * 16;

    v16f oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = v16f{};
    const v2bf kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    // One pipeline step: softmax of tile t (scores in scur) overlapped with
    // the scores of tile t+1 (into snxt, from knext) and P V of tile t from
    // vcur; stores K(t+2) into kfree and V(t+1) into vnext; loads K(t+3),
    // V(t+2).  Buffers past the last tile hold zeros or unused keys.
    auto step = [&](int t, v16f(&scur)[2], v16f(&snxt)[2], const uint8_t* knext, const uint8_t* vcur,
                    uint8_t* kfree, uint8_t* vnext) {
        const int j0 = t * AK;
        // mask keys beyond this query's visible prefix (only tiles that cross it)
        if (j0 + AK > kv_min) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = j0 + kh * 32 + (j / 4) * 8 + hh * 4 + (j % 4);
                    if (key >= my_end) scur[kh][j] = -INFINITY;
                }
        }
        // P of scores e, e+1 (bf16, as the PV MFMA takes them) against the
        // reference mref; the row sum adds the same rounded values with one dot2
        v8bf pb[4];
        auto p_pair = [&](int e, float mref, float& ps) {
            v2bf p2;
            p2[0] = to_bf16(__builtin_amdgcn_exp2f(fmaf(scur[e / 16][e % 16], c_log2, -mref)));
            p2[1] = to_bf16(__builtin_amdgcn_exp2f(fmaf(scur[e / 16][e % 16 + 1], c_log2, -mref)));
            pb[e / 8][e % 8] = p2[0];
            pb[e / 8][e % 8 + 1] = p2[1];
            ps = __builtin_amdgcn_fdot2_f32_bf16(p2, kOnes2, ps, false);
        };
        // P of one key half was formed against the running max.  When a
        // lane's sum over the half exceeds kRescaleMax (or is not finite),
        // raise the running max to the half's max, rescale, and form that
        // half's P again (a wave-uniform branch, taken on the first tile and
        // on tiles whose scores climb well above all earlier ones).  O and l
        // already hold the earlier P against the old max, so both are scaled.
        auto settle = [&](int kh, float& ps) {
            if (__any(!(ps <= kRescaleMax))) {
                float mx = -INFINITY;
#pragma unroll
                for (int j = 0; j < 16; ++j) mx = fmaxf(mx, scur[kh][j]);
                mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
                const float m_new = fmaxf(m_run, mx);
                if (m_new > m_run) {
                    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c_log2);
                    l_run *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int j = 0; j < 16; ++j) oacc[dt][j] *= alpha;
                    m_run = m_new;
                }
                // a row with no visible key so far keeps P = 0
                const float mb2 = m_run == -INFINITY ? 0.0f : m_run * c_log2;
                ps = 0.0f;
#pragma unroll
                for (int e = 16 * kh; e < 16 * kh + 16; e += 2) p_pair(e, mb2, ps);
            }
            l_run += ps;
        };
        // Scores of tile t+1 interleaved with P of key half 0 of tile t (one
        // score per MFMA), the LDS stores of K(t+2) and the loads of K(t+3):
        // MFMA i (key half i % 2, k-block i / 2) with its operand read four
        // ahead; sched_barrier keeps each group where it is written.
        auto kfrag = [&](int i) {
            return *reinterpret_cast<const v8bf*>(knext + ((i % 2) * 32 + lq) * KS_STRIDE + (i / 2) * 32 + hh * 16);
        };
        v8bf kf[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[i] = kfrag(i);
        const __amdgpu_buffer_rsrc_t krs = kv_rsrc(kbase, j0 + 3 * AK, T_k, ldk);
        snxt[0] = v16f{};
        snxt[1] = v16f{};
        float mb = m_run * c_log2;
        float ps0 = 0.0f, ps1 = 0.0f;
        float pe = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + 4 < 16) kf[i + 4] = kfrag(i + 4);
            snxt[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i / 2], snxt[i % 2], 0, 0, 0);
            const float p = __builtin_amdgcn_exp2f(fmaf(scur[0][i], c_log2, -mb));
            if (i % 2 == 0) {
                pe = p;
            } else {
                v2bf p2;
                p2[0] = to_bf16(pe);
                p2[1] = to_bf16(p);
                pb[i / 8][i % 8 - 1] = p2[0];
                pb[i / 8][i % 8] = p2[1];
                ps0 = __builtin_amdgcn_fdot2_f32_bf16(p2, kOnes2, ps0, false);
            }
            if (i % 4 == 1)
                *reinterpret_cast<v4i*>(kfree + (kkey + 16 * (i / 4)) * KS_STRIDE + kch * 16) = rk[i / 4];
            if (i % 4 == 2)
                rk[i / 4] = (v4i)__builtin_amdgcn_raw_buffer_load_b128(krs, koff, (i / 4) * 16 * ldk * 2, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        settle(0, ps0);
        // O^T += V^T P^T (16 keys per MFMA in the S^T lane order; MFMA i: key
        // block i / 4, d tile i % 4), operands read four ahead.  MFMAs 0-7
        // (key half 0) run beside P of key half 1, two scores each; MFMAs 8-15
        // beside the transposing LDS stores of V(t+1); the loads of V(t+2)
        // follow.
        auto vfrag = [&](int i) {
            return *reinterpret_cast<const v8bf*>(vcur + vrd + (i % 4) * 32 * VT_STRIDE + (i / 4) * 32);
        };
        v8bf vf[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) vf[i] = vfrag(i);
        const __amdgpu_buffer_rsrc_t vrs = kv_rsrc(vbase, j0 + 2 * AK, T_k, ldv);
        uint8_t* vdst = vnext + dc * 8 * VT_STRIDE + vpos * 2;
        mb = m_run * c_log2;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i + 4 < 16) vf[i + 4] = vfrag(i + 4);
            oacc[i % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pb[i / 4], oacc[i % 4], 0, 0, 0);
            p_pair(16 + 2 * i, mb, ps1);
            __builtin_amdgcn_sched_barrier(0);
        }
        settle(1, ps1);
#pragma unroll
        for (int i = 8; i < 16; ++i) {
            if (i + 4 < 16) vf[i + 4] = vfrag(i + 4);
            oacc[i % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pb[i / 4], oacc[i % 4], 0, 0, 0);
            {
                // transpose: 4 keys x 8 dims -> row d = dc*8 + r of 4 keys
                const int r = i - 8, w = r / 2;
                const uint32_t sel = (r % 2) ? 0x07060302u : 0x05040100u;
                uint2 packed;
                packed.x = __builtin_amdgcn_perm((uint32_t)rv[1][w], (uint32_t)rv[0][w], sel);
                packed.y = __builtin_amdgcn_perm((uint32_t)rv[3][w], (uint32_t)rv[2][w], sel);
                *reinterpret_cast<uint2*>(vdst + r * VT_STRIDE) = packed;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) rv[q] = (v4i)__builtin_amdgcn_raw_buffer_load_b128(vrs, voff, q * ldv * 2, 0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
    };

    const int ntiles = (kv_hi + AK - 1) / AK;
    // prologue: K(0), V(0), K(1) in LDS; K(2), V(1) in registers; scores of tile 0
    gload_k(0);
    gload_v(0);
    sstore_k(kbuf0);
    sstore_v(vbuf0);
    gload_k(AK);
    sstore_k(kbuf1);
    gload_k(2 * AK);
    gload_v(AK);
    __syncthreads();
    v16f sa[2], sb[2];
    scores(kbuf0, sa);
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        step(t, sa, sb, kbuf1, vbuf0, kbuf0, vbuf1);
        step(t + 1, sb, sa, kbuf0, vbuf1, kbuf1, vbuf0);
    }
    if (t < ntiles) step(t, sa, sb, kbuf1, vbuf0, kbuf0, vbuf1);

    const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
    if (!q_ok) return;
    const float inv = 1.0f / l_tot;
    __bf16* orow = O + (size_t)qi * ldo + h * 128;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            v4bf outv;
#pragma unroll
            for (int r = 0; r < 4; ++r) outv[r] = to_bf16(oacc[dt][g * 4 + r] * inv);
            *reinterpret_cast<v4bf*>(orow + dt * 32 + g * 8 + hh * 4) = outv;
        }
}

hipError_t launch_attention_bf16(const void* q, const void* k, const void* v, void* o, int64_t T_q,
                                 int64_t T_k, int H, int64_t ldq, int64_t ldk, int64_t ldv,
                                 int64_t ldo, const AttnSegs& segs, float sm_scale, hipStream_t st) {
    if (T_q == 0) return hipSuccess;
    const float c = sm_scale * 1.4426950408889634f;
    const dim3 grid((unsigned)(((T_q + AQ - 1) / AQ) * H));
    attn_bf16_kernel<<<grid, 256, 0, st>>>((const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                                           (__bf16*)o, (int)T_q, (int)T_k, (int)ldq, (int)ldk, (int)ldv,
                                           (int)ldo, segs, c, H, attn_head_group(2 * T_k * H * 128 * 2, H));
    return hipGetLastError();
}

// ---------------------------------------------------------------- fp32 (fp32 mode)
// One wave per (query, head); lane l holds dims 2l, 2l+1.  Plain online softmax
// over the visible key prefix.
__global__ void __launch_bounds__(256) attn_f32_kernel(const float* __restrict__ Q,
                                                       const float* __restrict__ Kg,
                                                       const float* __restrict__ Vg,
                                                       float* __restrict__ O, int64_t T_q,
                                                       int64_t T_k, int H, int64_t ldq, int64_t ldk,
                                                       int64_t ldv, int64_t ldo, AttnSegs sg,
                                                       float scale) {
    const int64_t item = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (item >= T_q * H) return;
    const int lane = threadIdx.x % kWave;
    const int64_t i = item / H;
    const int h = (int)(item % H);
    const int64_t end = kv_end_of(sg, T_k - T_q + i);
    const float q0 = Q[i * ldq + h * 128 + 2 * lane], q1 = Q[i * ldq + h * 128 + 2 * lane + 1];
    float m = -INFINITY, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int64_t j = 0; j < end; ++j) {
        const float* kr = Kg + j * ldk + h * 128 + 2 * lane;
        const float s = wave_sum(q0 * kr[0] + q1 * kr[1]) * scale;
        const float m_new = fmaxf(m, s);
        const float a = expf(m - m_new), p = expf(s - m_new);
        const float* vr = Vg + j * ldv + h * 128 + 2 * lane;
        o0 = o0 * a + p * vr[0];
        o1 = o1 * a + p * vr[1];
        l = l * a + p;
        m = m_new;
    }
    O[i * ldo + h * 128 + 2 * lane] = o0 / l;
    O[i * ldo + h * 128 + 2 * lane + 1] = o1 / l;
}

hipError_t launch_attention_f32(const float* q, const float* k, const float* v, float* o, int64_t T_q,
                                int64_t T_k, int H, int64_t ldq, int64_t ldk, int64_t ldv,
                                int64_t ldo, const AttnSegs& segs, float sm_scale, hipStream_t st) {
    const int64_t items = T_q * H;
    if (items == 0) return hipSuccess;
    attn_f32_kernel<<<(unsigned)((items + 3) / 4), 256, 0, st>>>(q, k, v, o, T_q, T_k, H, ldq, ldk, ldv,
                                                                 ldo, segs, sm_scale);
    return hipGetLastError();
}

}  // namespace dit
