"""Pins of the oracle's LayerNorm/adaLN, Q/K RMSNorm, RoPE and GELU (CPU only)."""
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as Fn

import ditsynth
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_layernorm_closed_form_and_library():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 512)) * 3.0 + 0.7
    h = oracle.adaln_modulate(x, 0.0, 0.0, eps=1e-6)
    assert np.allclose(h.mean(axis=1), 0.0, atol=1e-12)
    var = x.var(axis=1)
    assert np.allclose(h.var(axis=1), var / (var + 1e-6), rtol=1e-12)
    ref = Fn.layer_norm(torch.from_numpy(x), (512,), eps=1e-6).numpy()
    assert np.allclose(h, ref, rtol=1e-12, atol=1e-12)
    # modulation: scale 1, shift 2 -> 2*xhat + 2 ; per-column scale/shift broadcast
    assert np.allclose(oracle.adaln_modulate(x, 2.0, 1.0), 2 * ref + 2, atol=1e-12)
    sc = rng.standard_normal(512)
    sh = rng.standard_normal(512)
    assert np.allclose(oracle.adaln_modulate(x, sh, sc), ref * (1 + sc) + sh, atol=1e-12)


def test_rmsnorm_unit_rms_and_gain():
    rng = np.random.default_rng(2)
    t = rng.standard_normal((5, 3, 128)) * 4.0
    n = oracle.qk_rmsnorm(t, np.ones(128), "f32", eps=0.0)
    assert np.allclose(np.sqrt((n ** 2).mean(axis=-1)), 1.0, rtol=1e-13)
    g = 1.0 + 0.02 * rng.standard_normal(128)
    assert np.allclose(oracle.qk_rmsnorm(t, g, "f32", eps=0.0), n * g, rtol=1e-13)


def test_rmsnorm_bf16_matches_library_cast_order():
    """Library bf16 ops, normalize in fp32 -> cast to gain dtype -> multiply (the order the
    qualification page records); the opposite order disagrees on a measurable fraction."""
    rng = np.random.default_rng(3)
    t = oracle.round_bf16(rng.standard_normal((64, 4, 128)) * 2.0)
    g = oracle.round_bf16(1.0 + 0.02 * rng.standard_normal(128))
    tt = torch.from_numpy(t).to(torch.float32)
    gb = torch.from_numpy(g).to(torch.bfloat16)
    n32 = tt * torch.rsqrt(tt.pow(2).mean(-1, keepdim=True) + 1e-6)
    ref = (n32.to(torch.bfloat16) * gb).to(torch.float64).numpy()
    wrong = (n32 * gb.to(torch.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.qk_rmsnorm(t, g, "bf16")
    # fp32 normalization in the library vs fp64 in the oracle: rare one-ulp differences only
    ulp = np.abs(ref) * 2.0 ** -7
    assert np.all(np.abs(got - ref) <= ulp + 1e-30)
    mism_right = np.mean(got != ref)
    mism_wrong = np.mean(got != wrong)
    assert mism_right < 0.01
    assert mism_wrong > 5 * mism_right + 0.01


def test_positions_golden():
    gold = json.load(open(os.path.join(GOLD, "positions.json")))
    for case in gold["cases"]:
        pos = oracle.rope_positions(case["text_len"], [tuple(g) for g in case["grids"]])
        assert pos.shape[0] == case["text_len"] + sum(h * w for h, w in case["grids"])
        for row, expect in case["rows"].items():
            assert pos[int(row)].tolist() == expect, (case, row)


def test_token_counts_and_table_range_golden():
    gold = json.load(open(os.path.join(GOLD, "token_counts.json")))
    pos_gold = json.load(open(os.path.join(GOLD, "positions.json")))
    for side, n in gold["tokens_per_square_side"].items():
        g = int(side) // gold["pixels_per_token_side"]
        pos = oracle.rope_positions(512, [(g, g)])
        assert pos.shape[0] - 512 == n
        assert pos.min() >= pos_gold["table_min"] and pos.max() <= pos_gold["table_max"]
    w = ditsynth.workload(4)
    assert w.seg_len == [256, 1024, 16384]


def test_rope_closed_forms():
    pos = np.array([[0, 0, 0], [3, -2, 5]])
    c, s = oracle.rope_tables(pos)
    assert c.shape == (2, 64)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)        # position 0 -> identity
    # pair 0 of every axis has omega = 1: angle = the position itself
    assert np.isclose(c[1, 0], math.cos(3)) and np.isclose(c[1, 16], math.cos(-2)) and np.isclose(c[1, 40], math.cos(5))
    # pair 1 of the frame axis (32 dims): omega = 10000^(-2/32)
    assert np.isclose(s[1, 1], math.sin(3 * 10000 ** (-1 / 16)))
    # pair 1 of the height axis (48 dims): omega = 10000^(-2/48)
    assert np.isclose(s[1, 17], math.sin(-2 * 10000 ** (-1 / 24)))
    # last width pair: j = 23 of 24
    assert np.isclose(c[1, 63], math.cos(5 * 10000 ** (-46 / 48)))
    t = np.arange(2 * 1 * 128, dtype=np.float64).reshape(2, 1, 128)
    r = oracle.apply_rope(t, c, s)
    assert np.array_equal(r[0], t[0])
    # first pair rotated by angle 3: (x0 cos - x1 sin, x0 sin + x1 cos)
    x0, x1 = t[1, 0, 0], t[1, 0, 1]
    assert np.isclose(r[1, 0, 0], x0 * math.cos(3) - x1 * math.sin(3))
    assert np.isclose(r[1, 0, 1], x0 * math.sin(3) + x1 * math.cos(3))


def test_rope_norm_preservation_and_relative_position():
    rng = np.random.default_rng(5)
    pos = rng.integers(-100, 300, size=(20, 3))
    c, s = oracle.rope_tables(pos)
    q = rng.standard_normal((20, 2, 128))
    k = rng.standard_normal((20, 2, 128))
    rq = oracle.apply_rope(q, c, s)
    pair_norm = lambda t: t[..., 0::2] ** 2 + t[..., 1::2] ** 2
    assert np.allclose(pair_norm(rq), pair_norm(q), rtol=1e-12)
    shift = np.array([7, -13, 29])
    c2, s2 = oracle.rope_tables(pos + shift)
    rq2 = oracle.apply_rope(q, c2, s2)
    rk = oracle.apply_rope(k, c, s)
    rk2 = oracle.apply_rope(k, c2, s2)
    d1 = np.einsum("ihd,jhd->hij", rq, rk)
    d2 = np.einsum("ihd,jhd->hij", rq2, rk2)
    assert np.allclose(d1, d2, rtol=1e-9, atol=1e-9)
    # and it does depend on the relative position
    c3, s3 = oracle.rope_tables(pos * 2)
    d3 = np.einsum("ihd,jhd->hij", oracle.apply_rope(q, c3, s3), oracle.apply_rope(k, c3, s3))
    assert not np.allclose(d1, d3, atol=1e-3)


def test_gelu_closed_forms_and_library():
    u = np.linspace(-8, 8, 4001)
    g = oracle.gelu_tanh(u)
    ref = Fn.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    assert np.allclose(g, ref, rtol=1e-14, atol=1e-15)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.allclose(g - oracle.gelu_tanh(-u), u, atol=1e-13)         # odd part is x/2
    assert np.isclose(oracle.gelu_tanh(np.array([1.0]))[0],
                      0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * 1.044715)))


def _gelu_decimal(u: float) -> float:
    """0.5 u (1 + tanh(x)) in 120-digit decimal arithmetic, tanh from its
    exponential definition (textbook formula, no cancellation at this precision)."""
    import decimal
    with decimal.localcontext() as ctx:
        ctx.prec = 120
        U = decimal.Decimal(u)
        k = (decimal.Decimal(2) / decimal.Decimal(math.pi)).sqrt()
        X = k * (U + decimal.Decimal("0.044715") * U ** 3)
        e2 = (2 * X).exp()
        tanh = (e2 - 1) / (e2 + 1)
        return float(decimal.Decimal("0.5") * U * (1 + tanh))


def test_gelu_matches_high_precision_definition_in_the_negative_tail():
    """Relative error below 1e-12 against the tanh definition evaluated to 120
    digits (1 + tanh keeps 70 of them at u = -11), including u far enough below zero that fp64 1 + tanh(x) cancels
    (pi enters through fp64 math.pi in both, so the constant is the same)."""
    us = [-11.0, -9.5, -8.0, -6.5, -5.0, -3.0, -1.0, -0.25, 0.0, 0.3, 1.7, 4.0, 9.0]
    got = oracle.gelu_tanh(np.array(us))
    for u, g in zip(us, got):
        ref = _gelu_decimal(u)
        assert abs(g - ref) <= 1e-12 * abs(ref) + 1e-300, (u, g, ref)
    # the naive fp64 evaluation loses the tail (what the rewritten form avoids)
    naive = 0.5 * -8.0 * (1.0 + math.tanh(math.sqrt(2 / math.pi) * (-8.0 + 0.044715 * -512.0)))
    assert naive == 0.0 and _gelu_decimal(-8.0) < 0.0
