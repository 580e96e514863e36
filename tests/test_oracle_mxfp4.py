"""Pins of the oracle's MXFP4 weight decoding (CPU only)."""
import numpy as np
import torch

import ditsynth
import oracle


def test_e8m0_scales_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    packed = np.zeros((256, 16), np.uint8)
    packed[:, 0] = 0x02                                 # element 0 = +1.0
    got = oracle.mxfp4_decode(packed, codes[:, None])[:, 0]
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_e2m1_codes_from_the_bit_fields():
    """Every 4-bit code against sign * 2^(e-1) * (1 + m/2) (e > 0) or sign * m/2 (e = 0)."""
    nib = np.arange(16, dtype=np.uint8)
    packed = np.zeros((16, 16), np.uint8)
    packed[:, 0] = nib                                  # low nibble: element 0
    got = oracle.mxfp4_decode(packed, np.full((16, 1), 127, np.uint8))[:, 0]
    for c in range(16):
        sign = -1.0 if c & 8 else 1.0
        e, m = (c >> 1) & 3, c & 1
        ref = sign * (2.0 ** (e - 1) * (1 + m / 2) if e else m / 2)
        assert got[c] == ref, c


def test_low_nibble_first_packing():
    vals = np.array([0.5, -6.0, 3.0, 0.0, 1.5, -1.0] + [2.0] * 26, np.float64)        # one row, K = 32
    code = {v: i for i, v in enumerate(oracle.E2M1_VALUES)}
    nib = np.array([code[abs(v)] | (8 if v < 0 else 0) for v in vals], np.uint8)
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None, :]
    got = oracle.mxfp4_decode(packed, np.array([[130]], np.uint8))
    np.testing.assert_array_equal(got[0], vals * 8.0)


def test_decoded_weights_are_exact_in_bf16():
    codes, scales = ditsynth.mxfp4_weights(64, 256, seed=3)
    w = oracle.mxfp4_decode(codes, scales)
    assert np.all(np.isfinite(w))
    np.testing.assert_array_equal(oracle.round_bf16(w), w)


def test_gated_block_with_mxfp4_equals_block_on_decoded_weights():
    w = ditsynth.custom("mx", 256, 2, 768, 16, [(4, 6)], "bf16", 52)
    wg = ditsynth.gated_block_weights(w)
    mx = {}
    for name, (N, K) in (("w_qk", (512, 256)), ("w_down", (256, 768)), ("w_gate", (768, 256))):
        mx[name] = ditsynth.mxfp4_weights(N, K, seed=len(mx) + 7)
    inp = ditsynth.block_inputs(w)
    c, s = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    args = (inp["x"], inp["mod"], inp["mod_of_seg"], inp["seg_len"], c, s)
    got = oracle.block_forward_gated(*args, wg, mx=mx)["x_out"]
    plain = dict(wg)
    for name, (codes, scales) in mx.items():
        plain[name] = oracle.mxfp4_decode(codes, scales)
    ref = oracle.block_forward_gated(*args, plain)["x_out"]
    np.testing.assert_array_equal(got, ref)
