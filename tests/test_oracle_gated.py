"""Pins of the oracle's asymmetric activation quantization, the zero-point W8A8
linear and the gated-MLP block (CPU only)."""
import numpy as np
import pytest

import ditsynth
import oracle


def _rows(seed, M=40, K=300):
    assert M > 6
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K)).astype(np.float32) * np.exp(rng.standard_normal((M, 1))).astype(np.float32)
    a[3] = np.abs(a[3])          # all >= 0: zero point -128
    a[4] = -np.abs(a[4])         # all <= 0: zero point 127
    a[5] = 0.0                   # all zero
    a[6] += 5.0                  # far from zero, one-signed
    return oracle.round_bf16(a)


def test_asym_codes_properties():
    a = _rows(1)
    q, s, z = oracle.quantize_rows_asym(a)
    assert q.dtype == np.int8 and s.dtype == np.float32 and z.dtype == np.int32
    assert s[5] == 0 and z[5] == 0 and np.all(q[5] == 0)
    assert z[3] == -128 and z[4] == 127
    ok = s > 0
    qi = q.astype(np.int64)
    rec = (qi - z[:, None]) * s[:, None].astype(np.float64)
    # every value is within half a step of its reconstruction (+ fp32 rounding of s and a/s)
    assert np.all(np.abs(rec - a)[ok] <= (s[:, None] * (0.5 + 1e-4) * np.ones_like(a))[ok])
    # zero is exact: a code equal to z stands for 0, and the range ends map to -128 / 127
    # the range is widened to contain 0: its ends min(row, 0) and max(row, 0) map to -128 and (about) 127
    lo, hi = np.minimum(a.min(axis=1), 0), np.maximum(a.max(axis=1), 0)
    code_lo = np.rint(lo / np.where(ok, s, 1)) + z
    code_hi = np.rint(hi / np.where(ok, s, 1)) + z
    assert np.all(np.abs(code_lo[ok] + 128) <= 1) and np.all(np.abs(code_hi[ok] - 127) <= 1)
    neg = ok & (a.min(axis=1) < 0)
    assert np.all(np.min(qi, axis=1)[neg] == -128)
    zero_at = np.where(a[0] == 0)[0]
    assert np.all(q[0, zero_at] == z[0])


def test_asym_codes_brute_force_tiny():
    """Each code is the nearest grid point (q - z) s of the affine int8 grid (ties
    aside), found by exhaustive search over all 256 codes."""
    a = _rows(2, M=8, K=50)
    q, s, z = oracle.quantize_rows_asym(a)
    for m in range(a.shape[0]):
        if s[m] == 0:
            continue
        grid = (np.arange(-128, 128) - int(z[m])) * np.float64(s[m])
        for kk in range(a.shape[1]):
            d = np.abs(grid - a[m, kk])
            best = np.min(d)
            assert d[int(q[m, kk]) + 128] <= best + 1e-6 * s[m]


def test_w8a8_asym_equals_dequantized_product():
    rng = np.random.default_rng(3)
    a = _rows(3, M=30, K=256)
    w = oracle.round_bf16(rng.standard_normal((48, 256)) * 0.02)
    b = oracle.round_bf16(rng.standard_normal(48) * 0.02)
    qa, sa, za = oracle.quantize_rows_asym(a)
    qw, sw = oracle.quantize_rows(w)
    got = oracle.w8a8_linear_asym(qa, sa, za, qw, sw, b)
    deq_a = (qa.astype(np.float64) - za[:, None]) * sa[:, None]
    deq_w = qw.astype(np.float64) * sw[:, None]
    np.testing.assert_allclose(got, deq_a @ deq_w.T + b, rtol=1e-12, atol=1e-12)
    # and it approximates the unquantized product to int8 accuracy
    ref = a.astype(np.float64) @ w.T.astype(np.float64) + b
    assert oracle.rel_l2(got, ref) < 2e-2


def _gated_as_plain(w, wg):
    """Plain-block weights equal to a gated block whose proj is 0 with bias 1."""
    D = w.D
    return {"w_qkv": np.concatenate([wg["w_qk"], wg["w_v"]]), "b_qkv": np.concatenate([wg["b_qk"], wg["b_v"]]),
            "g_q": wg["g_q"], "g_k": wg["g_k"], "w_o": wg["w_o"], "b_o": wg["b_o"],
            "w_1": wg["w_gate"], "b_1": wg["b_gate"], "w_2": wg["w_down"], "b_2": wg["b_down"]}


def test_gated_block_reduces_to_plain_block():
    """proj = 0 with bias 1 makes g = GELU(gate): the gated block is then the plain
    block with W_1 = W_gate, and [W_qk; W_v] = W_qkv (all bf16)."""
    w = ditsynth.custom("g", 256, 2, 768, 16, [(4, 6)], "bf16", 50)
    wg = ditsynth.gated_block_weights(w)
    wg["w_proj"][:] = 0.0
    wg["b_proj"][:] = 1.0
    inp = ditsynth.block_inputs(w)
    c, s = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    got = oracle.block_forward_gated(inp["x"], inp["mod"], inp["mod_of_seg"], inp["seg_len"], c, s, wg)
    ref = oracle.block_forward(inp["x"], inp["mod"], inp["mod_of_seg"], inp["seg_len"], c, s, _gated_as_plain(w, wg),
                               "bf16")
    np.testing.assert_array_equal(got["x_out"], ref["x_out"])


def test_gated_block_int8_scope():
    """W8A8 on Q/K and proj/gate moves the output by int8-level amounts; an
    all-int8 block moves it further."""
    w = ditsynth.custom("g", 256, 2, 768, 16, [(4, 6)], "bf16", 51)
    wg = ditsynth.gated_block_weights(w)
    inp = ditsynth.block_inputs(w)
    c, s = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    args = (inp["x"], inp["mod"], inp["mod_of_seg"], inp["seg_len"], c, s, wg)
    x = inp["x"].astype(np.float64)
    base = oracle.block_forward_gated(*args)["x_out"] - x
    rec = oracle.block_forward_gated(*args, int8=("w_qk", "w_proj", "w_gate"))["x_out"] - x
    full = oracle.block_forward_gated(*args, int8=oracle.GATED_LINEARS)["x_out"] - x
    e_rec, e_full = oracle.rel_l2(rec, base), oracle.rel_l2(full, base)
    assert 1e-4 < e_rec < 0.15 and e_rec < e_full
