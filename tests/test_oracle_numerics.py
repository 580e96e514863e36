"""Pins of the oracle's rounding, quantization and integer GEMM (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import ditsynth
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_round_bf16_matches_library_rne_on_fp32_inputs():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # include exact ties: low 16 bits = 0x8000
    u = x.view(np.uint32).copy()
    u[::7] = (u[::7] & 0xFFFF0000) | 0x8000
    x = u.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_subnormal_range_matches_library():
    """fp32 inputs around and below bf16's smallest normal 2^-126 (fp32
    subnormals included), against torch's fp32 -> bf16 rounding."""
    rng = np.random.default_rng(12)
    e = rng.uniform(-152.0, -120.0, 100_000)
    x = (np.sign(rng.standard_normal(e.size)) * 2.0 ** e).astype(np.float32)
    u = x.view(np.uint32).copy()
    u[::5] = (u[::5] & 0xFFFF0000) | 0x8000            # ties
    x = u.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_round_bf16_hand_values():
    r = oracle.round_bf16
    assert r(1.0) == 1.0
    assert r(1 + 2 ** -8) == 1.0                   # tie -> even mantissa
    assert r(1 + 3 * 2 ** -8) == 1 + 2 ** -6       # tie -> even mantissa (up)
    assert r(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7
    assert r(-1.5) == -1.5
    assert r(3.0e38) == 2.9908525e38 or abs(r(3.0e38) - 3.0e38) / 3.0e38 < 2 ** -8


def test_gain_after_cast_golden():
    g = json.load(open(os.path.join(GOLD, "rmsnorm_cast_order.json")))
    assert oracle.apply_gain(np.array([g["n"]]), np.array([g["g"]]), "bf16")[0] == g["cast_then_gain"]
    # the other order, worked by hand, differs
    assert oracle.round_bf16(g["n"] * g["g"]) == g["gain_then_cast"]
    assert g["cast_then_gain"] != g["gain_then_cast"]


def test_quantize_integer_rows_are_lossless():
    a = np.array([[127, -3, 0, 64, -127], [1, 2, 3, 4, 5]], dtype=np.float64)
    a[1] *= 127 / 5          # amax 127 after scaling: row 1 = 25.4*[1..5]
    q, s = oracle.quantize_rows(a[:1])
    assert s[0] == np.float32(1.0)
    assert np.array_equal(q[0], np.array([127, -3, 0, 64, -127], dtype=np.int8))


def test_quantize_zero_row_and_power_of_two_round_trip():
    a = np.zeros((3, 16))
    codes = np.array([127, -5, 3, 0, 100, -127, 1, 2, 7, 9, -9, 11, 12, 13, 14, 15])
    a[1] = codes * 0.25          # scale 0.25 = amax/127 exactly
    a[2] = -codes * 2.0 ** -10
    q, s = oracle.quantize_rows(a)
    assert s[0] == 0 and np.all(q[0] == 0)
    assert s[1] == np.float32(0.25) and np.array_equal(q[1], codes.astype(np.int8))
    assert s[2] == np.float32(2.0 ** -10) and np.array_equal(q[2], (-codes).astype(np.int8))


def test_quantize_error_bound_symmetry_and_range():
    a = ditsynth.rows(64, 4096, seed=5, scale=2.0, bf16=True)
    q, s = oracle.quantize_rows(a)
    assert q.min() >= -127 and q.max() <= 127
    assert np.all(np.abs(q).max(axis=1) == 127)
    err = np.abs(a.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    # half a step, plus the rounding of the fp32 division and scale
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    qn, sn = oracle.quantize_rows(-a)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)


def test_quantize_uses_fp32_division():
    # For a row whose amax is 127*2^e the scale is a power of two; elsewhere the fp32
    # scale is amax/127 rounded once, the code is rint of an fp32 quotient.
    a = np.array([[1.0, 0.5, 0.1, -0.3]], dtype=np.float32).astype(np.float64)
    q, s = oracle.quantize_rows(a)
    s32 = np.float32(np.float32(1.0) / np.float32(127.0))
    assert s[0] == s32
    expect = [int(np.rint(np.float32(np.float32(v) / s32))) for v in a[0]]
    assert q[0].tolist() == expect == [127, 64, 13, -38]


def test_int8_matmul_exact_brute_force_tiny():
    rng = np.random.default_rng(3)
    qa = rng.integers(-127, 128, size=(5, 67), dtype=np.int8)
    qw = rng.integers(-127, 128, size=(7, 67), dtype=np.int8)
    acc = oracle.int8_matmul_exact(qa, qw)
    for m in range(5):
        for n in range(7):
            assert acc[m, n] == sum(int(qa[m, k]) * int(qw[n, k]) for k in range(67))


def test_int8_matmul_exact_at_full_depth():
    rng = np.random.default_rng(4)
    qa = np.full((3, 16384), 127, dtype=np.int8)
    qa[1] = -127
    qa[2] = rng.integers(-127, 128, size=16384, dtype=np.int8)
    qw = rng.integers(-127, 128, size=(9, 16384), dtype=np.int8)
    qw[0] = 127
    acc = oracle.int8_matmul_exact(qa, qw)
    ref = qa.astype(np.int64) @ qw.astype(np.int64).T
    assert np.array_equal(acc, ref)
    assert acc[0, 0] == 16384 * 127 * 127


def test_w8a8_linear_dequant():
    qa = np.array([[1, -2, 3]], dtype=np.int8)
    qw = np.array([[4, 5, 6], [-1, 0, 1]], dtype=np.int8)
    y = oracle.w8a8_linear(qa, np.array([0.5], np.float32), qw, np.array([2.0, 0.25], np.float32),
                           np.array([1.0, -1.0]))
    assert y.tolist() == [[(4 - 10 + 18) * 0.5 * 2.0 + 1.0, (-1 + 0 + 3) * 0.5 * 0.25 - 1.0]]


def test_weight_quantization_per_output_channel():
    w = ditsynth.workload(2)
    ws = ditsynth.block_weights(ditsynth.custom("q", 256, 2, 512, 4, [(2, 2)], "w8a8", 9, outliers=True))
    q, s = oracle.quantize_rows(ws["w_o"])
    assert q.shape == ws["w_o"].shape and s.shape == (ws["w_o"].shape[0],)
    deq = q.astype(np.float64) * s[:, None]
    assert np.all(np.abs(deq - ws["w_o"]) <= s[:, None] * (0.5 + 1e-5))
    assert w.outliers
