"""Op-level parity of the fused paths the block runs (through the C ABI):

* the QKV linear with its Q/K RMSNorm + RoPE epilogue (dit_qkv_linear), on the
  persistent large-tile kernel, its K-split reduce and the small-shape path,
  with the cast order of "Qwen Image 2.1 native qualification", Numerical
  checks (normalized value cast to bf16 before the gain multiply);
* the adaLN prologue with its fused per-token int8 codes: codes and scales
  bit-identical to the oracle's quantization of the kernel's own bf16 h;
* the GELU fused into the quantization of g: g within 1 bf16 ulp of the oracle
  and the codes bit-identical to the oracle's quantization of the kernel's g.
"""
import numpy as np
import pytest
import torch

import ditsynth
import oracle
import diffusion_transformer_text_qwen_amd as dq
from gpu_helpers import DEV, bf16_ulp, dev, host, say

pytestmark = pytest.mark.gpu


def _qkv_inputs(T, D, mode, seed):
    """Activation and QKV weights of the block's recipe (adaLN-like rows, N(0, 0.02)
    weights, gains 1 + N(0, 0.02)), RoPE tables of a [text | image] sequence."""
    rng = np.random.default_rng(seed)
    h = ditsynth.to_bf16_grid((rng.standard_normal((T, D)) * 0.8).astype(np.float32))
    w = rng.standard_normal((3 * D, D)).astype(np.float32) * np.float32(0.02)
    b = ditsynth.to_bf16_grid((rng.standard_normal(3 * D) * 0.02).astype(np.float32))
    g_q = ditsynth.to_bf16_grid((1 + 0.02 * rng.standard_normal(128)).astype(np.float32))
    g_k = ditsynth.to_bf16_grid((1 + 0.02 * rng.standard_normal(128)).astype(np.float32))
    text = min(64, T // 4)
    side = int(np.ceil(np.sqrt(T - text)))
    pos = oracle.rope_positions(text, [(side, side)])[:T]
    c, s = oracle.rope_tables(pos)
    if mode == "bf16":
        w = ditsynth.to_bf16_grid(w)
    return h, w, b, g_q, g_k, c.astype(np.float32), s.astype(np.float32)


def _norm_rope_ref(y, g, c, s, right_order=True):
    """RMSNorm + gain + RoPE of the rounded linear output y [R, H, 128] (bf16
    storage); right_order=False takes the gain before the one rounding."""
    if right_order:
        return oracle.round_bf16(oracle.apply_rope(oracle.qk_rmsnorm(y, g, "bf16"), c, s))
    n = y / np.sqrt((y ** 2).mean(-1, keepdims=True) + 1e-6)
    return oracle.round_bf16(oracle.apply_rope(oracle.round_bf16(n * g), c, s))


@pytest.mark.parametrize("T,D,mode", [
    (4352, 4096, "w8a8"),   # 816 tiles: three whole rounds + 48 tiles split along K (reduce path)
    (300, 4096, "w8a8"),    # 96 tiles, every tile split (all rows through the reduce)
    (4352, 4096, "bf16"),
    (80, 512, "w8a8"),      # small shape: GEMM stores [q|k|v], then the norm/RoPE kernel
])
def test_qkv_linear_fused_epilogue(T, D, mode):
    say("qkv linear", T, D, mode)
    H = D // 128
    h, w, b, g_q, g_k, c, s = _qkv_inputs(T, D, mode, seed=T + D)
    q_out, k_out, v_out = (torch.empty((T, D), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    ws = torch.empty(dq.qkv_linear_workspace_bytes(T, H), dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(T)
    rows = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 192)]))
    if mode == "w8a8":
        qa, sa = oracle.quantize_rows(h)
        qw, sw = oracle.quantize_rows(w)
        args = dict(a_scale=dev(sa), w_scale=dev(sw))
        dq.qkv_linear(dev(qa, torch.int8), dev(qw, torch.int8), dev(b), dev(g_q), dev(g_k), dev(c), dev(s),
                      q_out, k_out, v_out, ws, **args)
        # the accumulators of these rows, from the plain linear (pinned bit-exact elsewhere)
        acc = torch.empty((T, 3 * D), dtype=torch.int32, device=DEV)
        y_tmp = torch.empty((T, 3 * D), dtype=torch.float32, device=DEV)
        dq.w8a8_linear(dev(qa, torch.int8), dev(sa), dev(qw, torch.int8), dev(sw), dev(b), y_tmp, acc_out=acc)
        torch.cuda.synchronize()
        acc_r = acc.cpu().numpy()[rows].astype(np.int64)
        assert np.array_equal(acc_r, oracle.int8_matmul_exact(qa[rows], qw))
        y = acc_r.astype(np.float64) * sa[rows, None].astype(np.float64) * sw[None, :].astype(np.float64) + b
    else:
        dq.qkv_linear(dev(h, torch.bfloat16), dev(w, torch.bfloat16), dev(b), dev(g_q), dev(g_k), dev(c), dev(s),
                      q_out, k_out, v_out, ws)
        torch.cuda.synchronize()
        y = oracle.linear(h[rows], w, b)
    y = oracle.round_bf16(y)
    R = len(rows)
    cr, sr = c[rows].astype(np.float64), s[rows].astype(np.float64)
    q_ref = _norm_rope_ref(y[:, :D].reshape(R, H, 128), g_q, cr, sr).reshape(R, D)
    k_ref = _norm_rope_ref(y[:, D:2 * D].reshape(R, H, 128), g_k, cr, sr).reshape(R, D)
    q_got, k_got, v_got = (host(t)[rows] for t in (q_out, k_out, v_out))
    # one bf16 ulp (fp32 statistics and products vs fp64)
    for got, ref, name in ((q_got, q_ref, "q"), (k_got, k_ref, "k")):
        bad = np.abs(got - ref) > bf16_ulp(ref) + 1e-30
        assert not bad.any(), (name, np.argwhere(bad)[:5])
    match = np.mean(q_got == q_ref)
    wrong = _norm_rope_ref(y[:, :D].reshape(R, H, 128), g_q, cr, sr, right_order=False).reshape(R, D)
    match_wrong = np.mean(q_got == wrong)
    exact_bar = 0.99 if mode == "w8a8" else 0.98   # bf16 mode: fp32 vs fp64 sums of 4096 products
    say(f"  q exact {match:.4f} (other cast order {match_wrong:.4f}), k exact {np.mean(k_got == k_ref):.4f}")
    assert match > exact_bar and np.mean(k_got == k_ref) > exact_bar
    assert match_wrong < match - 0.005
    # v passes through the rounding only
    v_ref = y[:, 2 * D:]
    assert np.all(np.abs(v_got - v_ref) <= bf16_ulp(v_ref) + 1e-30)
    assert np.mean(v_got == v_ref) > exact_bar


@pytest.mark.parametrize("M,D", [(100, 4096), (4352, 4096), (37, 512), (6, 8192)])
def test_adaln_fused_codes_bit_exact(M, D):
    """One launch writes h and its codes; the codes and scales equal the oracle's
    quantization of that h bit for bit, and h is the oracle's adaLN within one
    bf16 rounding."""
    say("adaln fused codes", M, D)
    rng = np.random.default_rng(M + D)
    x = ditsynth.to_bf16_grid((rng.standard_normal((M, D)) * 2 + 0.5).astype(np.float32))
    x[M // 2] *= 40.0                                   # a large-amplitude row
    shift = (rng.standard_normal(D) * 0.7).astype(np.float32)
    scale = (rng.standard_normal(D) * 0.7).astype(np.float32)
    h = torch.empty((M, D), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((M, D), dtype=torch.int8, device=DEV)
    qs = torch.empty(M, dtype=torch.float32, device=DEV)
    dq.adaln_modulate(dev(x, torch.bfloat16), dev(shift), dev(scale), h_out=h, q_out=q, q_scale=qs)
    torch.cuda.synchronize()
    hg = host(h)
    q_ref, s_ref = oracle.quantize_rows(hg)
    assert np.array_equal(qs.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    ref = oracle.adaln_modulate(x, shift, scale)
    assert np.all(np.abs(hg - ref) <= bf16_ulp(ref) + 1e-6)
    assert np.mean(hg == oracle.round_bf16(ref)) > 0.99


@pytest.mark.parametrize("M,K", [(300, 16384), (97, 4096), (33, 12288), (5, 1032)])
def test_gelu_quantize_bit_exact(M, K):
    """g = bf16(GELU_tanh(u)) within one bf16 ulp of the oracle (>= 99.9% equal),
    and the codes and scales equal the oracle's quantization of the kernel's g."""
    say("gelu quantize", M, K)
    rng = np.random.default_rng(M * K)
    u = ditsynth.to_bf16_grid((rng.standard_normal((M, K)) * 1.5).astype(np.float32))
    u[0, :8] = [0.0, -0.0, 30.0, -30.0, 9.5, -9.5, 1e-3, -1e-3]     # zero, saturation, tiny
    q = torch.empty((M, K), dtype=torch.int8, device=DEV)
    s = torch.empty(M, dtype=torch.float32, device=DEV)
    g = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    dq.gelu_quantize_rows(dev(u, torch.bfloat16), q, s, g_out=g)
    torch.cuda.synchronize()
    gg = host(g)
    ref = oracle.gelu_tanh(u.astype(np.float64))
    bad = np.abs(gg - ref) > bf16_ulp(ref) + 1e-30
    assert not bad.any(), np.argwhere(bad)[:5]
    match = np.mean(gg == oracle.round_bf16(ref))
    say(f"  g exact {match:.5f}")
    assert match >= 0.999
    q_ref, s_ref = oracle.quantize_rows(gg)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    # without g_out the codes are the same
    q2 = torch.empty_like(q)
    s2 = torch.empty_like(s)
    dq.gelu_quantize_rows(dev(u, torch.bfloat16), q2, s2)
    torch.cuda.synchronize()
    assert torch.equal(q2, q) and torch.equal(s2, s)
