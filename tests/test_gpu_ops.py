"""GPU op-level parity against the oracle (through the C ABI)."""
import math

import numpy as np
import pytest
import torch

import ditsynth
import oracle
import diffusion_transformer_text_qwen_amd as dq
from gpu_helpers import DEV, bf16_ulp, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu


# bf16 widths: up to 16384 columns the row's chunks are dealt once over 4 waves
# (K <= 4096) or 8 (widths that are not whole multiples leave chunks past K);
# above that one 256-thread workgroup per row strides over the row.
@pytest.mark.parametrize("M,K,bf16,zero_rows", [
    (1, 64, True, ()), (9, 2056, True, ()), (37, 4096, True, (3, 36)), (33, 4104, True, (5,)),
    (20, 12288, True, ()), (300, 16384, True, (0,)), (6, 24576, True, (2,)), (5, 512, False, ()),
    (64, 16384, False, (1,))])
def test_quantize_rows_bit_exact(M, K, bf16, zero_rows):
    say("quantize", M, K, bf16)
    x = ditsynth.rows(M, K, seed=M + K, scale=3.0, bf16=bf16, zero_rows=zero_rows)
    if not bf16:
        x[0, :10] *= 8.0      # outlier-like entries
    q = torch.empty((M, K), dtype=torch.int8, device=DEV)
    s = torch.empty(M, dtype=torch.float32, device=DEV)
    dq.quantize_rows(dev(x, torch.bfloat16 if bf16 else torch.float32), q, s)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(x.astype(np.float64))
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("K", [4096, 12296])
def test_quantize_rows_strided_bit_exact(K):
    """Rows read with a stride larger than K (a column slice of a wider matrix)."""
    say("quantize strided", K)
    M = 11
    wide = ditsynth.rows(M, K + 64, seed=K + 7, scale=2.0, bf16=True, zero_rows=())
    x = dev(wide, torch.bfloat16)[:, :K]
    assert x.stride(0) == K + 64
    q = torch.empty((M, K), dtype=torch.int8, device=DEV)
    s = torch.empty(M, dtype=torch.float32, device=DEV)
    dq.quantize_rows(x, q, s)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(wide[:, :K].astype(np.float64))
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_quantize_outlier_weights_bit_exact():
    w = ditsynth.workload(2)
    ws = ditsynth.block_weights(ditsynth.custom("wq", 512, 4, 2048, 4, [(2, 2)], "w8a8", 21, outliers=True))
    for name in ("w_qkv", "w_2"):
        a = ws[name]
        q = torch.empty(a.shape, dtype=torch.int8, device=DEV)
        s = torch.empty(a.shape[0], dtype=torch.float32, device=DEV)
        dq.quantize_rows(dev(a), q, s)
        torch.cuda.synchronize()
        q_ref, s_ref = oracle.quantize_rows(a)
        assert np.array_equal(s.cpu().numpy(), s_ref) and np.array_equal(q.cpu().numpy(), q_ref), name
    assert w.outliers


@pytest.mark.parametrize("M,N,K,ws", [(1, 16, 128, False), (77, 272, 384, False), (300, 512, 4096, True),
                                      (129, 128, 16384, False), (4429, 4144, 256, False), (4096, 4096, 640, False),
                                      (4352, 4096, 1024, True), (4429, 4144, 2048, True),
                                      (1024, 15360, 256, False), (1152, 3072, 4096, True),
                                      (1152, 1536, 8192, True), (320, 12288, 4096, True),
                                      (320, 4096, 16384, True), (4352, 16384, 256, True)])
def test_w8a8_linear_exact_accumulators(M, N, K, ws):
    """ws=True passes a workspace: tiles of a partial last round (272 tiles on 256
    CUs), or every tile of a launch with fewer tiles than CUs (60 and 30 tiles, the
    second with a long K loop), are split along K and their partial int32 sums
    added by a reduce launch; 240 tiles without a workspace run as one partial round.
    A last round of 32..64 tiles (306 tiles at 4429 x 4144 with ragged edges, 1088
    at 4352 x 16384) runs as 128 x 128 sub-tiles with the whole K loop instead.
    At M = 320 the second row of tiles holds 64 rows (its partial sums store only
    those), with a short (96 tiles) and a long (32 tiles) K loop."""
    say("w8a8", M, N, K, ws)
    a, b, sa, sb, bias = ditsynth.int8_operands(M, N, K, seed=M * 7 + N)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    yf = torch.empty((M, N), dtype=torch.float32, device=DEV)
    work = torch.full((dq.w8a8_linear_workspace_bytes(),), 0x5A, dtype=torch.uint8, device=DEV) if ws else None
    args = (dev(a, torch.int8), dev(sa), dev(b, torch.int8), dev(sb), dev(bias))
    dq.w8a8_linear(*args, y, acc_out=acc, workspace=work)
    dq.w8a8_linear(*args, yf, workspace=work)
    torch.cuda.synchronize()
    acc_ref = oracle.int8_matmul_exact(a, b)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    ref = oracle.w8a8_linear(a, sa, b, sb, bias)
    # fp32 epilogue: float(acc), two products and the bias add, each rounded once
    f32_err = 4 * 2.0 ** -24 * (np.abs(ref - bias[None, :]) + np.abs(bias)[None, :])
    assert np.all(np.abs(host(yf) - ref) <= f32_err)
    assert np.all(np.abs(host(y) - ref) <= bf16_ulp(ref) / 2 + f32_err)


def test_w8a8_linear_full_shapes_sampled():
    """The four W8A8 shapes of the 1024^2 workload (M = 4352), sampled entries exact."""
    rng = np.random.default_rng(0)
    for N, K in ((12288, 4096), (4096, 4096), (16384, 4096), (4096, 16384)):
        M = 4352
        say("w8a8 full", M, N, K)
        a, b, sa, sb, bias = ditsynth.int8_operands(M, N, K, seed=N + K)
        acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        work = torch.empty((dq.w8a8_linear_workspace_bytes(),), dtype=torch.uint8, device=DEV)
        dq.w8a8_linear(dev(a, torch.int8), dev(sa), dev(b, torch.int8), dev(sb), dev(bias), y, acc_out=acc,
                       workspace=work)
        torch.cuda.synchronize()
        ms = rng.integers(0, M, 256)
        ns = rng.integers(0, N, 256)
        ms[:4] = [0, M - 1, 0, M - 1]
        ns[:4] = [0, N - 1, N - 1, 0]
        got = acc.cpu().numpy()[ms, ns].astype(np.int64)
        ref = np.array([int(a[m].astype(np.int64) @ b[n].astype(np.int64)) for m, n in zip(ms, ns)])
        assert np.array_equal(got, ref)
        prod = ref * sa[ms].astype(np.float64) * sb[ns].astype(np.float64)
        yref = prod + bias[ns]
        f32_err = 4 * 2.0 ** -24 * (np.abs(prod) + np.abs(bias[ns]))
        assert np.all(np.abs(host(y)[ms, ns] - yref) <= bf16_ulp(yref) / 2 + f32_err)


@pytest.mark.parametrize("M,N,K", [(5, 64, 64), (100, 272, 640), (320, 4096, 4096), (4429, 4144, 192)])
def test_bf16_linear(M, N, K):
    say("bf16 linear", M, N, K)
    rng = np.random.default_rng(M + N)
    a = ditsynth.to_bf16_grid(rng.standard_normal((M, K)).astype(np.float32))
    w = ditsynth.to_bf16_grid((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    bias = ditsynth.to_bf16_grid((rng.standard_normal(N) * 0.02).astype(np.float32))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    yf = torch.empty((M, N), dtype=torch.float32, device=DEV)
    dq.bf16_linear(dev(a, torch.bfloat16), dev(w, torch.bfloat16), dev(bias), y)
    dq.bf16_linear(dev(a, torch.bfloat16), dev(w, torch.bfloat16), dev(bias), yf)
    torch.cuda.synchronize()
    ref = oracle.linear(a, w, bias)
    # fp32 accumulation: |err| <= K * 2^-24 * sum|a w| (bound), then one bf16 rounding
    acc_bound = K * 2.0 ** -24 * (np.abs(a.astype(np.float64)) @ np.abs(w.astype(np.float64)).T)
    assert np.all(np.abs(host(yf) - ref) <= acc_bound + 1e-30)
    assert np.all(np.abs(host(y) - ref) <= bf16_ulp(ref) / 2 + acc_bound + 1e-30)


def test_f32_linear():
    rng = np.random.default_rng(5)
    M, N, K = 80, 1536, 512
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bias = (rng.standard_normal(N) * 0.02).astype(np.float32)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    dq.f32_linear(dev(a), dev(w), dev(bias), y)
    torch.cuda.synchronize()
    ref = oracle.linear(a, w, bias)
    bound = K * 2.0 ** -24 * (np.abs(a.astype(np.float64)) @ np.abs(w.astype(np.float64)).T) + np.abs(ref) * 2 ** -24
    assert np.all(np.abs(host(y) - ref) <= bound)


ATTN_CASES = [
    # seg_len, T_q, H
    ([16, 64], 80, 4),
    ([64, 256], 320, 2),
    ([1, 7, 120], 128, 2),
    ([128, 1024], 1152, 2),
    ([40, 90, 333], 333, 3),          # cached step: queries are the last segment
    ([256, 1024, 700], 1980, 1),
    ([300], 300, 2),                  # one segment: plain full attention
    ([100, 37], 1, 2),                # a single query (the last row) against a cached prefix
    ([5, 17, 1, 64, 3, 40, 9, 70, 2, 33, 11, 8, 60, 1, 25, 30], 379, 1),   # the maximum of 16 segments
]


@pytest.mark.parametrize("seg_len,T_q,H", ATTN_CASES)
def test_attention_bf16(seg_len, T_q, H):
    say("attn bf16", seg_len, T_q, H)
    T_k = sum(seg_len)
    q, k, v = ditsynth.attention_inputs(T_q, T_k, H, seed=T_k + H)
    o = torch.empty((T_q, H, 128), dtype=torch.bfloat16, device=DEV)
    dq.block_causal_attention(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), o, seg_len)
    torch.cuda.synchronize()
    ref = oracle.attention(q, k, v, seg_len)
    got = host(o)
    # bf16 P (8 significant bits) and one bf16 output rounding
    assert rel_l2(got, ref) < 1e-2
    assert np.max(np.abs(got - ref)) < 0.05


def test_attention_bf16_special_cases():
    seg_len = [1, 63, 200]
    T = 264
    q, k, v = ditsynth.attention_inputs(T, T, 2, seed=3)
    o = torch.empty((T, 2, 128), dtype=torch.bfloat16, device=DEV)
    dq.block_causal_attention(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), o, seg_len)
    o0 = torch.empty_like(o)
    dq.block_causal_attention(torch.zeros_like(o), dev(k, torch.bfloat16), dev(v, torch.bfloat16), o0, seg_len)
    torch.cuda.synchronize()
    # a query with one visible key returns that value exactly
    assert np.array_equal(host(o)[0], v[0].astype(np.float64))
    # q = 0: mean of the visible values
    got0 = host(o0)
    for i, n in ((5, 64), (100, 264)):
        ref = v[:n].astype(np.float64).mean(axis=0)
        assert np.all(np.abs(got0[i] - ref) <= bf16_ulp(ref) + 2e-3 * np.abs(ref).max())


def test_attention_bf16_running_max_raised_mid_sequence():
    """Key norms grow tile by tile and spike late, so the running max is raised
    (and a tile's P formed again) many times after the first tile."""
    T, H = 704, 2
    q, k, v = ditsynth.attention_inputs(T, T, H, seed=9)
    growth = 1.0 + 0.6 * (np.arange(T) // 64)
    k = k * growth[:, None, None]
    k[600:606] *= 3.0
    k = ditsynth.to_bf16_grid(k)
    for seg_len in ([T], [100, 604]):
        say("attn bf16 rising scores", seg_len)
        o = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
        dq.block_causal_attention(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), o,
                                  seg_len)
        torch.cuda.synchronize()
        ref = oracle.attention(q, k, v, seg_len)
        got = host(o)
        assert np.all(np.isfinite(got))
        assert rel_l2(got, ref) < 1e-2
        assert np.max(np.abs(got - ref)) < 0.05


def test_attention_bf16_causal_invariance_and_determinism():
    seg_len = [64, 300, 500]
    T = sum(seg_len)
    q, k, v = ditsynth.attention_inputs(T, T, 2, seed=4)
    qd, kd, vd = dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16)
    o1 = torch.empty((T, 2, 128), dtype=torch.bfloat16, device=DEV)
    o2 = torch.empty_like(o1)
    o3 = torch.empty_like(o1)
    dq.block_causal_attention(qd, kd, vd, o1, seg_len)
    dq.block_causal_attention(qd, kd, vd, o2, seg_len)
    kd2, vd2 = kd.clone(), vd.clone()
    kd2[364:] = -kd2[364:]
    vd2[364:] = vd2[364:] * 3
    dq.block_causal_attention(qd, kd2, vd2, o3, seg_len)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(o1[:364], o3[:364])
    assert not torch.equal(o1[364:], o3[364:])


def test_attention_bf16_full_size_sampled():
    """2048^2 edit workload: 16,384 target queries over 17,664 keys, 32 heads,
    and the uncached call with all 17,664 queries."""
    seg_len = [256, 1024, 16384]
    T_k, T_q, H = 17664, 16384, 32
    say("attn full", T_q, T_k, H)
    q, k, v = ditsynth.attention_inputs(T_k, T_k, H, seed=44)
    kd, vd = dev(k, torch.bfloat16), dev(v, torch.bfloat16)
    o = torch.empty((T_q, H, 128), dtype=torch.bfloat16, device=DEV)
    dq.block_causal_attention(dev(q[T_k - T_q:], torch.bfloat16), kd, vd, o, seg_len)
    of = torch.empty((T_k, H, 128), dtype=torch.bfloat16, device=DEV)
    dq.block_causal_attention(dev(q, torch.bfloat16), kd, vd, of, seg_len)
    torch.cuda.synchronize()
    # target rows see every key: the oracle's last-rows convention applies directly
    rows = np.array([0, 1, 127, 128, 5000, 9999, 16383])
    ref = oracle.attention(q[T_k - T_q + rows], k, v, seg_len)
    assert rel_l2(host(o)[rows], ref) < 1e-2
    # cached and uncached calls agree bit for bit on the target rows
    assert torch.equal(o, of[T_k - T_q:])
    # text rows see the text keys only; reference rows see text + reference
    ref_t = oracle.attention(q[:4], k[:256], v[:256], [256])
    assert rel_l2(host(of)[:4], ref_t) < 1e-2
    r_rows = np.array([256, 700, 1279])
    ref_r = oracle.attention(q[r_rows], k[:1280], v[:1280], [256, 1024])
    assert rel_l2(host(of)[r_rows], ref_r) < 1e-2


def test_attention_f32():
    seg_len = [16, 64]
    q, k, v = ditsynth.attention_inputs(80, 80, 4, seed=6, bf16=False)
    o = torch.empty((80, 4, 128), dtype=torch.float32, device=DEV)
    dq.block_causal_attention(dev(q), dev(k), dev(v), o, seg_len)
    torch.cuda.synchronize()
    assert rel_l2(host(o), oracle.attention(q, k, v, seg_len)) < 1e-5


def test_rope_tables():
    for text, grids in ((16, [(8, 8)]), (256, [(32, 32), (128, 128)]), (3, [(3, 5), (2, 2)])):
        T = text + sum(h * w for h, w in grids)
        c = torch.empty((T, 64), dtype=torch.float32, device=DEV)
        s = torch.empty((T, 64), dtype=torch.float32, device=DEV)
        dq.rope_tables(text, grids, 0, T, c, s)
        torch.cuda.synchronize()
        cr, sr = oracle.rope_tables(oracle.rope_positions(text, grids))
        assert np.max(np.abs(c.cpu().numpy() - cr)) <= 6e-8
        assert np.max(np.abs(s.cpu().numpy() - sr)) <= 6e-8
        # a row window
        c2 = torch.empty((5, 64), dtype=torch.float32, device=DEV)
        s2 = torch.empty((5, 64), dtype=torch.float32, device=DEV)
        dq.rope_tables(text, grids, T - 5, 5, c2, s2)
        torch.cuda.synchronize()
        assert torch.equal(c2, c[T - 5:]) and torch.equal(s2, s[T - 5:])


def _qkv_case(T, H, seed):
    rng = np.random.default_rng(seed)
    qkv = ditsynth.to_bf16_grid((rng.standard_normal((T, 3 * H * 128)) * 2).astype(np.float32))
    g_q = ditsynth.to_bf16_grid((1 + 0.02 * rng.standard_normal(128)).astype(np.float32))
    g_k = ditsynth.to_bf16_grid((1 + 0.02 * rng.standard_normal(128)).astype(np.float32))
    pos = rng.integers(-64, 300, size=(T, 3))
    c, s = oracle.rope_tables(pos)
    return qkv, g_q, g_k, c.astype(np.float32), s.astype(np.float32)


def test_qk_norm_rope_bf16_cast_order():
    T, H = 300, 4
    qkv, g_q, g_k, c, s = _qkv_case(T, H, 8)
    D = H * 128
    qo = torch.empty((T, D), dtype=torch.bfloat16, device=DEV)
    ko = torch.empty((T, D), dtype=torch.bfloat16, device=DEV)
    vo = torch.empty((T, D), dtype=torch.bfloat16, device=DEV)
    dq.qk_norm_rope(dev(qkv, torch.bfloat16), dev(g_q), dev(g_k), dev(c), dev(s), qo, ko, vo)
    torch.cuda.synchronize()
    q_in = qkv[:, :D].reshape(T, H, 128).astype(np.float64)
    ref = oracle.round_bf16(oracle.apply_rope(oracle.qk_rmsnorm(q_in, g_q, "bf16"), c, s)).reshape(T, D)
    got = host(qo)
    assert np.all(np.abs(got - ref) <= bf16_ulp(ref) + 1e-30)
    match = np.mean(got == ref)
    # the other order (gain, then one rounding) is measurably further away
    n = q_in / np.sqrt((q_in ** 2).mean(-1, keepdims=True) + 1e-6)
    wrong = oracle.round_bf16(oracle.apply_rope(oracle.round_bf16(n * g_q), c, s)).reshape(T, D)
    assert match > 0.99
    assert np.mean(got == wrong) < match - 0.005
    assert np.array_equal(host(vo), qkv[:, 2 * D:])
    k_ref = oracle.round_bf16(oracle.apply_rope(oracle.qk_rmsnorm(qkv[:, D:2 * D].reshape(T, H, 128), g_k, "bf16"),
                                                c, s)).reshape(T, D)
    assert np.all(np.abs(host(ko) - k_ref) <= bf16_ulp(k_ref) + 1e-30)


def test_qk_norm_rope_f32():
    T, H = 80, 4
    qkv, g_q, g_k, c, s = _qkv_case(T, H, 9)
    D = H * 128
    outs = [torch.empty((T, D), dtype=torch.float32, device=DEV) for _ in range(3)]
    dq.qk_norm_rope(dev(qkv), dev(g_q), dev(g_k), dev(c), dev(s), *outs)
    torch.cuda.synchronize()
    ref = oracle.apply_rope(oracle.qk_rmsnorm(qkv[:, :D].reshape(T, H, 128), g_q, "f32"), c, s).reshape(T, D)
    assert rel_l2(host(outs[0]), ref) < 1e-6


def test_adaln_bf16_and_fused_quant():
    rng = np.random.default_rng(10)
    M, D = 100, 4096
    x = ditsynth.to_bf16_grid((rng.standard_normal((M, D)) * 2 + 0.5).astype(np.float32))
    shift = (rng.standard_normal(D) * 0.7).astype(np.float32)
    scale = (rng.standard_normal(D) * 0.7).astype(np.float32)
    h = torch.empty((M, D), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((M, D), dtype=torch.int8, device=DEV)
    qs = torch.empty(M, dtype=torch.float32, device=DEV)
    xd = dev(x, torch.bfloat16)
    dq.adaln_modulate(xd, dev(shift), dev(scale), h_out=h)
    dq.adaln_modulate(xd, dev(shift), dev(scale), q_out=q, q_scale=qs)
    torch.cuda.synchronize()
    ref = oracle.adaln_modulate(x, shift, scale)
    ref_b = oracle.round_bf16(ref)
    got = host(h)
    assert np.all(np.abs(got - ref) <= bf16_ulp(ref) + 1e-6)
    assert np.mean(got == ref_b) > 0.99
    s = qs.cpu().numpy().astype(np.float64)
    amax = np.abs(ref_b).max(axis=1)
    assert np.all(np.abs(s * 127 - amax) <= bf16_ulp(amax))
    deq = q.cpu().numpy().astype(np.float64) * s[:, None]
    assert np.all(np.abs(deq - ref) <= s[:, None] * 0.5 + bf16_ulp(ref) + 1e-6)


def test_adaln_f32_small_width():
    rng = np.random.default_rng(11)
    M, D = 80, 512
    x = rng.standard_normal((M, D)).astype(np.float32)
    shift = rng.standard_normal(D).astype(np.float32)
    scale = rng.standard_normal(D).astype(np.float32)
    h = torch.empty((M, D), dtype=torch.float32, device=DEV)
    dq.adaln_modulate(dev(x), dev(shift), dev(scale), h_out=h)
    torch.cuda.synchronize()
    assert rel_l2(host(h), oracle.adaln_modulate(x, shift, scale)) < 1e-6


def test_euler():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4096, 64)).astype(np.float32)
    v = ditsynth.to_bf16_grid(rng.standard_normal((4096, 64)).astype(np.float32))
    xd = dev(x)
    dq.euler_step(xd, dev(v, torch.bfloat16), 1.0, 1.0 - 0.98 / 39)
    torch.cuda.synchronize()
    ref = oracle.euler_update(x, v, 1.0, np.float64(np.float32(1.0 - 0.98 / 39)))
    assert np.all(np.abs(host(xd) - ref) <= 2 * 2.0 ** -24 * np.abs(ref) + 2.0 ** -30)
    xd2 = dev(x)
    dq.euler_step(xd2, dev(v, torch.bfloat16), 0.5, 0.5)
    torch.cuda.synchronize()
    assert np.array_equal(xd2.cpu().numpy(), x)
