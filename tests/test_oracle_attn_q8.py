"""Pins of the oracle's quantized (int8 Q K^T, fp8 P V) attention (CPU only).

The e4m3 rounding is checked against torch's float8_e4m3fn conversion (an
independent implementation of the same format), the quantizers against their
defining properties, and attention_q8 against the oracle's plain attention in
the special case where every quantization step is exact, plus a two-key case
worked out by hand.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_fp8_rounding_matches_torch_in_range():
    rng = np.random.default_rng(3)
    grid = oracle.decode_fp8_e4m3(np.arange(256, dtype=np.uint8))
    grid = grid[np.isfinite(grid)]
    mids = (np.sort(grid)[1:] + np.sort(grid)[:-1]) / 2          # ties: round half to even
    rand = np.concatenate([rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 9, 20000),
                           rng.uniform(-448, 448, 5000)])
    x = np.concatenate([grid, mids, rand]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    np.testing.assert_array_equal(oracle.round_fp8_e4m3(x), _torch_e4m3(x))


def test_fp8_codes_match_torch_bit_patterns():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_fp8_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(mine[ok], ref[ok])
    # encode is the inverse on the finite codes (0x80, the negative zero, encodes as 0x00)
    finite = codes[ok & (codes != 0x80)]
    np.testing.assert_array_equal(oracle.encode_fp8_e4m3(oracle.decode_fp8_e4m3(finite)), finite)


def test_fp8_grid_facts():
    r = oracle.round_fp8_e4m3
    assert r(448.0) == 448.0 and r(500.0) == 448.0 and r(-1e6) == -448.0   # saturation (reading)
    assert r(2.0 ** -9) == 2.0 ** -9                                        # smallest subnormal
    assert r(2.0 ** -10) == 0.0                                             # tie to even (zero)
    assert r(1.0625) == 1.0 and r(1.1875) == 1.25                           # ties to even mantissa
    assert r(0.9048) == 0.875                                               # spacing 1/16 below 1
    assert oracle.encode_fp8_e4m3(np.array([1.0]))[0] == 0x38


def test_quantize_attn_q_k_properties():
    rng = np.random.default_rng(5)
    T, H, d = 150, 3, 128
    x = oracle.round_bf16(rng.standard_normal((T, H, d)) * np.exp(rng.standard_normal((T, H, 1))))
    q8, sq = oracle.quantize_attn_q(x)
    assert q8.shape == (T, H, d) and sq.shape == (T, H)
    assert np.all(np.abs(q8.astype(int)) <= 127)
    # the largest magnitude of each (token, head) maps to +-127, and the error is at most half a step
    assert np.all(np.max(np.abs(q8.astype(int)), axis=2) == 127)
    err = np.abs(q8 * sq[..., None].astype(np.float64) - x)
    assert np.all(err <= sq[..., None] * (0.5 + 1e-4))   # + fp32 rounding of s and x/s
    k8, sk = oracle.quantize_attn_k(x)
    nt = (T + 63) // 64
    assert sk.shape == (nt, H)
    for t in range(nt):
        blk = x[t * 64:(t + 1) * 64]
        for h in range(H):
            assert sk[t, h] == np.float32(np.max(np.abs(blk[:, h, :]).astype(np.float32)) / np.float32(127))
            assert np.max(np.abs(k8[t * 64:(t + 1) * 64, h].astype(int))) == 127
    # tiles are independent: changing the keys of tile 1 leaves tile 0's codes alone
    y = x.copy()
    y[70:80] *= 4.0
    k8b, skb = oracle.quantize_attn_k(y)
    np.testing.assert_array_equal(k8b[:64], k8[:64])
    assert np.all(skb[0] == sk[0]) and not np.all(skb[1] == sk[1])


def test_quantize_attn_v_properties():
    rng = np.random.default_rng(6)
    T, H, d = 90, 2, 128
    v = oracle.round_bf16(rng.standard_normal((T, H, d)) * 3.0)
    v[:, 1, 5] = 0.0                                          # an all-zero channel
    v8, sv = oracle.quantize_attn_v(v)
    assert sv.shape == (H, d) and sv[1, 5] == 0 and np.all(v8[:, 1, 5] == 0)
    assert np.all(np.abs(v8) <= 448)
    np.testing.assert_array_equal(oracle.round_fp8_e4m3(v8), v8)          # on the grid
    ok = sv > 0
    assert np.all(np.max(np.abs(v8), axis=0)[ok] == 448.0)                # amax -> 448
    rec = v8 * sv[None].astype(np.float64)
    big = (np.abs(v) >= 2.0 ** -6 * sv[None]) & (sv[None] > 0) & (v != 0)   # normal range of the codes
    rel = np.abs(rec - v)[big] / np.abs(v)[big]
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-5)                            # half of e4m3's 2^-3 spacing


def test_attention_q8_equals_plain_attention_when_exact():
    """Integer q/k codes with amax 127 (scale 1), V on the e4m3 grid with channel
    amax 448 (scale 1), scale = ln 2 and score gaps of at most 8: every P = 2^-n
    is an e4m3 value, so no step rounds and the result is plain attention."""
    rng = np.random.default_rng(7)
    T_q, T_k, H, d = 12, 40, 2, 128
    seg_len = [10, 14, 16]
    q = np.zeros((T_k, H, d))
    k = np.zeros((T_k, H, d))
    q[:, :, 0] = 127.0                                 # q.k = 127 * k[:, 0] + small integer terms
    k[:, :, 0] = 1.0
    k[:, :, 1] = rng.integers(-4, 5, (T_k, H))        # score = 127 + q1 * k1 with q1 = 1
    q[:, :, 1] = 1.0
    q[:, :, 2] = -127.0                                # k8 tile amax 127 needs a 127 somewhere
    k[:, :, 2] = 0.0
    k[0, :, 3] = 127.0
    q = q[T_k - T_q:]
    v = oracle.round_fp8_e4m3(rng.standard_normal((T_k, H, d)) * 40.0)
    v[0] = 448.0                                       # channel amax 448 -> scale 1
    q8, sq = oracle.quantize_attn_q(q)
    k8, sk = oracle.quantize_attn_k(k)
    v8, sv = oracle.quantize_attn_v(v)
    assert np.all(sq == 1.0) and np.all(sk == 1.0) and np.all(sv == 1.0)
    np.testing.assert_array_equal(v8, v)
    got = oracle.attention_q8(q8, sq, k8, sk, v8, sv, seg_len, scale=math.log(2.0))
    ref = oracle.attention(q, k, v, seg_len, scale=math.log(2.0))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-9)


def test_attention_q8_two_keys_by_hand():
    """One query, two keys with scores 0 and -0.1: P = (1, e^-0.1); e^-0.1 = 0.9048
    rounds to 0.875 on e4m3 (spacing 1/16 in [0.5, 1)), while the normalizer adds
    the unrounded 1 + e^-0.1."""
    d = 128
    q8 = np.zeros((1, 1, d), np.int8)
    k8 = np.zeros((2, 1, d), np.int8)
    q8[0, 0, 0] = 1
    k8[1, 0, 0] = -1
    sq = np.ones((1, 1), np.float32)
    sk = np.ones((1, 1), np.float32)
    v8 = np.zeros((2, 1, d))
    v8[0, 0, :] = 2.0
    v8[1, 0, :] = -3.0
    sv = np.full((1, d), 0.5, np.float32)
    got = oracle.attention_q8(q8, sq, k8, sk, v8, sv, [2], scale=0.1)
    expect = (1.0 * 1.0 + 0.875 * -1.5) / (1.0 + math.exp(-0.1))
    np.testing.assert_allclose(got[0, 0], expect, rtol=1e-14)


def test_attention_quantized_close_to_plain():
    """On bf16-like data the quantized attention stays within a few percent of fp64 attention."""
    rng = np.random.default_rng(8)
    T, H, d = 96, 2, 128
    q = oracle.round_bf16(rng.standard_normal((T, H, d)))
    k = oracle.round_bf16(rng.standard_normal((T, H, d)))
    v = oracle.round_bf16(rng.standard_normal((T, H, d)))
    got = oracle.attention_quantized(q, k, v, [32, 64])
    ref = oracle.attention(q, k, v, [32, 64])
    assert oracle.rel_l2(got, ref) < 5e-2


@pytest.mark.parametrize("flip", ["sk_tile", "sv_channel"])
def test_attention_q8_sees_scales(flip):
    """A plausible indexing mistake (tile scale of the wrong tile, channel scale of
    the wrong channel) changes the result."""
    rng = np.random.default_rng(9)
    T, H, d = 130, 1, 128
    q = oracle.round_bf16(rng.standard_normal((T, H, d)))
    k = oracle.round_bf16(rng.standard_normal((T, H, d)) * np.repeat([1.0, 3.0, 0.5], [64, 64, 2])[:, None, None])
    v = oracle.round_bf16(rng.standard_normal((T, H, d)) * np.linspace(0.1, 4, d))
    q8, sq = oracle.quantize_attn_q(q)
    k8, sk = oracle.quantize_attn_k(k)
    v8, sv = oracle.quantize_attn_v(v)
    base = oracle.attention_q8(q8, sq, k8, sk, v8, sv, [T])
    if flip == "sk_tile":
        sk = sk[::-1].copy()
    else:
        sv = sv[:, ::-1].copy()
    assert oracle.rel_l2(oracle.attention_q8(q8, sq, k8, sk, v8, sv, [T]), base) > 1e-2


def test_attention_q8_bound_covers_any_rounding_reference():
    """The bound holds for the exact-max rounding and for P rounded after scaling by
    2^delta (delta in [0, 8], what a running maximum below the final one gives),
    and it is not vacuous (the rounding error reaches a sizeable part of it)."""
    rng = np.random.default_rng(10)
    T, H, d = 160, 2, 128
    seg_len = [40, 120]
    q = oracle.round_bf16(rng.standard_normal((T, H, d)) * 1.5)
    k = oracle.round_bf16(rng.standard_normal((T, H, d)))
    v = oracle.round_bf16(rng.standard_normal((T, H, d)))
    q8, sq = oracle.quantize_attn_q(q)
    k8, sk = oracle.quantize_attn_k(k)
    v8, sv = oracle.quantize_attn_v(v)
    exact = oracle.attention_q8(q8, sq, k8, sk, v8, sv, seg_len, round_p=False)
    rounded = oracle.attention_q8(q8, sq, k8, sk, v8, sv, seg_len)
    bound = oracle.attention_q8_bound(q8, sq, k8, sk, v8, sv, seg_len)
    assert np.all(np.abs(rounded - exact) <= bound * (1 + 1e-9))
    assert np.max(np.abs(rounded - exact) / bound) > 0.2
    # P rounded relative to a stale maximum: P' = P 2^delta, rounded, scaled back
    allowed = oracle.allowed_mask(seg_len, T)
    for h in range(H):
        key_scale = sk[np.arange(T) // 64, h].astype(np.float64)
        s = (q8[:, h].astype(np.float64) @ k8[:, h].astype(np.float64).T) * sq[:, h, None] * key_scale / math.sqrt(d)
        s = np.where(allowed, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        delta = rng.uniform(0, 8 * math.log(2), (T, 1))
        p8 = oracle.round_fp8_e4m3(p * np.exp(delta)) / np.exp(delta)
        vd = v8[:, h] * sv[h][None].astype(np.float64)
        stale = (p8 @ vd) / p.sum(axis=1, keepdims=True)
        assert np.all(np.abs(stale - exact[:, h]) <= bound[:, h] * (1 + 1e-9))
