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


def _norm_rope_ref(y, g, c, s, right_order=True, pre=False):
    """RMSNorm + gain + RoPE of the rounded linear output y [R, H, 128] (bf16
    storage); right_order=False takes the gain before the one rounding.
    pre=True also returns the rotation's inputs."""
    if right_order:
        n = oracle.qk_rmsnorm(y, g, "bf16")
    else:
        n = oracle.round_bf16(y / np.sqrt((y ** 2).mean(-1, keepdims=True) + 1e-6) * g)
    out = oracle.round_bf16(oracle.apply_rope(n, c, s))
    return (out, n) if pre else out


def _rotation_bound(n, c, s):
    """|change of a rotated pair| when each input of the pair moves by up to
    three bf16 ulps: a one-ulp change of the rounded linear output (fp32 against
    fp64 sums or dequantization, at a rounding boundary) moves the rounded
    normalized value by up to two of its ulps (their binades need not match) and
    the rounded gain product by one more.  The rotation mixes the pair, so this
    can be many ulps of an output whose two terms nearly cancel."""
    R, H, _ = n.shape
    u = bf16_ulp(n).reshape(R, H, 64, 2)
    m = np.maximum(np.abs(c), np.abs(s))[:, None, :]
    per_pair = 3 * (u[..., 0] + u[..., 1]) * m
    return np.repeat(per_pair, 2, axis=-1).reshape(R, H * 128)


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
    y_gpu = None
    if mode == "w8a8":
        qa, sa = oracle.quantize_rows(h)
        qw, sw = oracle.quantize_rows(w)
        args = dict(a_scale=dev(sa), w_scale=dev(sw))
        dq.qkv_linear(dev(qa, torch.int8), dev(qw, torch.int8), dev(b), dev(g_q), dev(g_k), dev(c), dev(s),
                      q_out, k_out, v_out, ws, **args)
        # the same linear stored as bf16 (same launch plan: same shape and a
        # workspace), with its int32 sums
        acc = torch.empty((T, 3 * D), dtype=torch.int32, device=DEV)
        y_st = torch.empty((T, 3 * D), dtype=torch.bfloat16, device=DEV)
        work = torch.empty((dq.w8a8_linear_workspace_bytes(),), dtype=torch.uint8, device=DEV)
        dq.w8a8_linear(dev(qa, torch.int8), dev(sa), dev(qw, torch.int8), dev(sw), dev(b), y_st, acc_out=acc,
                       workspace=work)
        torch.cuda.synchronize()
        acc_r = acc.cpu().numpy()[rows].astype(np.int64)
        assert np.array_equal(acc_r, oracle.int8_matmul_exact(qa[rows], qw))
        y = acc_r.astype(np.float64) * sa[rows, None].astype(np.float64) * sw[None, :].astype(np.float64) + b
        y_gpu = host(y_st)[rows]
    else:
        dq.qkv_linear(dev(h, torch.bfloat16), dev(w, torch.bfloat16), dev(b), dev(g_q), dev(g_k), dev(c), dev(s),
                      q_out, k_out, v_out, ws)
        torch.cuda.synchronize()
        y = oracle.linear(h[rows], w, b)
    y = oracle.round_bf16(y)
    R = len(rows)
    cr, sr = c[rows].astype(np.float64), s[rows].astype(np.float64)
    q_ref, n_q = _norm_rope_ref(y[:, :D].reshape(R, H, 128), g_q, cr, sr, pre=True)
    k_ref, n_k = _norm_rope_ref(y[:, D:2 * D].reshape(R, H, 128), g_k, cr, sr, pre=True)
    q_ref, k_ref = q_ref.reshape(R, D), k_ref.reshape(R, D)
    q_got, k_got, v_got = (host(t)[rows] for t in (q_out, k_out, v_out))
    exact_bar = 0.99 if mode == "w8a8" else 0.98   # bf16 mode: fp32 vs fp64 sums of 4096 products
    for got, ref, n, name in ((q_got, q_ref, n_q, "q"), (k_got, k_ref, n_k, "k")):
        err = np.abs(got - ref)
        one_ulp = err <= bf16_ulp(ref) + 1e-30
        say(f"  {name}: exact {np.mean(got == ref):.5f}, within 1 ulp {np.mean(one_ulp):.5f}")
        assert np.mean(one_ulp) >= 0.999 and np.mean(got == ref) > exact_bar
        if mode == "w8a8":
            # exact sums: every element within the rotated input bound
            bad = err > bf16_ulp(ref) + _rotation_bound(n, cr, sr) + 1e-30
            assert not bad.any(), (name, np.argwhere(bad)[:5])
        else:
            # fp32 sums of 4096 products: their error moves tiny outputs by more
            # than an ulp; the tensor as a whole stays at bf16 rounding level
            assert np.linalg.norm(got - ref) <= 2.0 ** -8 * np.linalg.norm(ref)
    match = np.mean(q_got == q_ref)
    wrong = _norm_rope_ref(y[:, :D].reshape(R, H, 128), g_q, cr, sr, right_order=False).reshape(R, D)
    match_wrong = np.mean(q_got == wrong)
    say(f"  q exact {match:.4f} (other cast order {match_wrong:.4f})")
    assert match_wrong < match - 0.005
    if y_gpu is not None:
        # from the GPU's own rounded output of the plain linear (a separate
        # kernel instantiation: its fp32 dequantization may contract the
        # products differently, so a few rounded values may differ by an ulp)
        for got, sec, g, name in ((q_got, 0, g_q, "q"), (k_got, 1, g_k, "k")):
            ref2, n2 = _norm_rope_ref(y_gpu[:, sec * D:(sec + 1) * D].reshape(R, H, 128), g, cr, sr, pre=True)
            ref2 = ref2.reshape(R, D)
            err = np.abs(got - ref2)
            assert not (err > bf16_ulp(ref2) + _rotation_bound(n2, cr, sr) + 1e-30).any(), name
            say(f"  {name} from the GPU's linear output: exact {np.mean(got == ref2):.5f}, "
                f"within 1 ulp {np.mean(err <= bf16_ulp(ref2) + 1e-30):.5f}")
            assert np.mean(err <= bf16_ulp(ref2) + 1e-30) >= 0.9999 and np.mean(got == ref2) > 0.99
        v_st = y_gpu[:, 2 * D:]
        assert np.all(np.abs(v_got - v_st) <= bf16_ulp(v_st) + 1e-30) and np.mean(v_got == v_st) >= 0.9999
    # v passes through the rounding only (bf16: plus the fp32 summation error
    # of 4096 products, at most K 2^-24 sum|h w| for any order)
    v_ref = y[:, 2 * D:]
    acc_err = 0.0 if mode == "w8a8" else D * 2.0 ** -24 * (np.abs(h[rows]).astype(np.float64) @
                                                         np.abs(w[2 * D:]).astype(np.float64).T)
    assert np.all(np.abs(v_got - v_ref) <= bf16_ulp(v_ref) + acc_err + 1e-30)
    assert np.mean(v_got == v_ref) > exact_bar


@pytest.mark.parametrize("M,D", [(100, 4096), (4352, 4096), (37, 512), (6, 8192)])
def test_adaln_fused_codes_bit_exact(M, D):
    """One launch writes h and its codes; the codes and scales equal the oracle's
    quantization of that h bit for bit, and h is the oracle's adaLN within one
    bf16 rounding."""
    say("adaln fused codes", M, D)
    rng = np.random.default_rng(M + D)
    x = (rng.standard_normal((M, D)) * 2 + 0.5).astype(np.float32)
    x[M // 2] *= 40.0                                   # a large-amplitude row
    x = ditsynth.to_bf16_grid(x)
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


@pytest.mark.parametrize("M,D", [(100, 4096), (4352, 4096), (37, 512), (29, 1024)])
def test_adaln_fused_asym_codes_bit_exact(M, D):
    """The adaLN pass with the W8A8 recipe's asymmetric activation codes: codes,
    scales and zero points equal the oracle's asymmetric quantization of the
    kernel's own h bit for bit, h is the oracle's adaLN within one bf16 rounding,
    and the launch without h_out writes the same codes."""
    say("adaln fused asym codes", M, D)
    rng = np.random.default_rng(M * 3 + D)
    x = (rng.standard_normal((M, D)) * 2 + 0.5).astype(np.float32)
    x[M // 2] *= 40.0                                   # a large-amplitude row
    x[M // 3] = 1.5                                     # a constant row: h = shift
    x = ditsynth.to_bf16_grid(x)
    shift = (rng.standard_normal(D) * 0.7).astype(np.float32)
    scale = (rng.standard_normal(D) * 0.7).astype(np.float32)
    args = (dev(x, torch.bfloat16), dev(shift), dev(scale))
    h = torch.empty((M, D), dtype=torch.bfloat16, device=DEV)
    out = []
    for h_out in (h, None):
        q = torch.full((M, D), 99, dtype=torch.int8, device=DEV)
        qs = torch.empty(M, dtype=torch.float32, device=DEV)
        qz = torch.empty(M, dtype=torch.int32, device=DEV)
        dq.adaln_modulate_asym(*args, q, qs, qz, h_out=h_out)
        out.append((q, qs, qz))
    torch.cuda.synchronize()
    hg = host(h)
    q_ref, s_ref, z_ref = oracle.quantize_rows_asym(hg)
    for q, qs, qz in out:
        assert np.array_equal(qs.cpu().numpy(), s_ref)
        assert np.array_equal(qz.cpu().numpy(), z_ref)
        assert np.array_equal(q.cpu().numpy(), q_ref)
    ref = oracle.adaln_modulate(x, shift, scale)
    assert np.all(np.abs(hg - ref) <= bf16_ulp(ref) + 1e-6)
    assert np.mean(hg == oracle.round_bf16(ref)) > 0.99
    # the codes span the int8 range: the row minimum maps to -128
    assert (q_ref.min(axis=1) == -128).mean() > 0.9


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
