"""Int8 / fp8 attention on the GPU (through the C ABI) against the oracle.

The quantization pass is bit-exact (codes and scales) against the oracle's
quantizers.  The attention kernel rounds P to e4m3 relative to a running row
maximum (up to 2^8 below the final one) where the oracle rounds relative to the
exact maximum; for zero-mean random values the output is a small average, so
two independent e4m3 roundings of P (3.6% rms each) differ by a few percent of
|o|.  The check is therefore element-wise against the rigorous envelope of
e4m3 rounding of P around the unrounded-P result (oracle.attention_q8_bound,
valid for any rounding reference), plus bf16 rounding of the output; with
exactly representable P (integer scores with sm_scale = ln 2) the kernel
matches the oracle key by key.
"""
import math

import numpy as np
import pytest
import torch

import ditsynth
import oracle
import diffusion_transformer_text_qwen_amd as dq
from gpu_helpers import DEV, GpuBlock, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu


def _check_envelope(got, c, seg_len, T_k, scale=None, rows=None, q_rows=None):
    """|got - attention with unrounded P| <= e4m3 envelope + bf16 rounding, element-wise."""
    q8, sq = c["q8"], c["sq"]
    if q_rows is not None:
        q8, sq = q8[q_rows], sq[q_rows]
    args = (q8, sq, c["k8"][:T_k], c["sk"], oracle.decode_fp8_e4m3(c["v8"][:T_k]), c["sv"], seg_len)
    exact = oracle.attention_q8(*args, scale=scale, round_p=False)
    bound = oracle.attention_q8_bound(*args, scale=scale)
    rounded = oracle.attention_q8(*args, scale=scale)
    if rows is not None:
        got = got[rows]
        exact, bound, rounded = exact[rows], bound[rows], rounded[rows]
    slack = bound * 1.01 + 2.0 ** -8 * np.abs(exact) + 1e-6
    worst = float(np.max(np.abs(got - exact) / slack))
    e = rel_l2(got, rounded)
    say(f"  envelope use {worst:.3f}; rel_l2 vs oracle (exact-max rounding) {e:.3e}")
    assert np.all(np.isfinite(got))
    assert worst <= 1.0
    assert e <= 0.1


def _decode(buf, T_q, T_k, H):
    """The operand buffer's parts, per the layout documented with dit_attn_q8_bytes."""
    _, off = dq.attn_q8_layout(T_q, T_k, H)
    b = buf.cpu().numpy()
    nt = (T_k + 63) // 64
    q8 = b[off["q8"]:off["q8"] + H * T_q * 128].view(np.int8).reshape(H, T_q, 128).transpose(1, 0, 2)
    sq = b[off["q_scale"]:off["q_scale"] + H * T_q * 4].view(np.float32).reshape(H, T_q).T
    kimg = b[off["k8"]:off["k8"] + H * nt * 8192].view(np.int8).reshape(H, nt, 64, 8, 16)
    k8 = np.empty((H, nt, 64, 8, 16), np.int8)
    for r in range(64):
        for c in range(8):
            k8[:, :, r, c] = kimg[:, :, r, c ^ (r & 7)]
    k8 = k8.reshape(H, nt * 64, 128).transpose(1, 0, 2)
    sk = b[off["k_scale"]:off["k_scale"] + H * nt * 4].view(np.float32).reshape(H, nt).T
    vimg = b[off["v8"]:off["v8"] + H * nt * 8192].reshape(H, nt, 128, 4, 16)
    vrow = np.empty((H, nt, 128, 64), np.uint8)
    for ch in range(128):
        for c in range(4):
            vrow[:, :, ch, c * 16:(c + 1) * 16] = vimg[:, :, ch, c ^ ((ch >> 1) & 3)]
    v8 = np.empty((H, nt, 64, 128), np.uint8)
    for p in range(64):
        g, bb = p // 32, p % 32
        key = (bb // 16) * 32 + (bb % 4) + 8 * ((bb % 16) // 4) + 4 * g
        v8[:, :, key, :] = vrow[:, :, :, p]
    v8 = v8.reshape(H, nt * 64, 128).transpose(1, 0, 2)
    sv = b[off["v_scale"]:off["v_scale"] + H * 128 * 4].view(np.float32).reshape(H, 128)
    return {"q8": q8, "sq": sq, "k8": k8, "sk": sk, "v8": v8, "sv": sv}


def _quantize_on_gpu(q, k, v):
    T_q, H, _ = q.shape
    T_k = k.shape[0]
    n, _ = dq.attn_q8_layout(T_q, T_k, H)
    buf = torch.empty(n, dtype=torch.uint8, device=DEV)
    buf.fill_(0xA5)   # every byte the layout covers must be written
    dq.attn_quantize(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), buf)
    torch.cuda.synchronize()
    return buf


@pytest.mark.parametrize("T_q,T_k,H,scale", [(200, 330, 3, 1.0), (64, 64, 1, 1.0), (130, 130, 2, 37.0),
                                             (1, 65, 2, 0.01)])
def test_quantize_bit_exact(T_q, T_k, H, scale):
    say("attn quantize", T_q, T_k, H, scale)
    q, k, v = ditsynth.attention_inputs(T_q, T_k, H, seed=T_k + 7 * H)
    q, k, v = (ditsynth.to_bf16_grid(a * scale) for a in (q, k, v))
    if T_k >= 70:
        k[64:70] = 0.0             # rows of zeros inside a tile
        v[:, 0, 3] = 0.0           # an all-zero value channel
    buf = _quantize_on_gpu(q, k, v)
    got = _decode(buf, T_q, T_k, H)
    q8, sq = oracle.quantize_attn_q(q)
    k8, sk = oracle.quantize_attn_k(k)
    v8, sv = oracle.quantize_attn_v(v)
    np.testing.assert_array_equal(got["q8"], q8)
    np.testing.assert_array_equal(got["sq"], sq)
    np.testing.assert_array_equal(got["k8"][:T_k], k8)
    assert np.all(got["k8"][T_k:] == 0)
    np.testing.assert_array_equal(got["sk"], sk)
    np.testing.assert_array_equal(oracle.decode_fp8_e4m3(got["v8"][:T_k]), v8)
    assert np.all(oracle.decode_fp8_e4m3(got["v8"][T_k:]) == 0)
    np.testing.assert_array_equal(got["sv"], sv)


ATTN_CASES = [
    # seg_len, T_q, H, input scale
    ([16, 64], 80, 2, 1.0),
    ([1, 7, 120], 128, 2, 1.0),
    ([40, 90, 333], 333, 3, 1.0),        # cached step: queries are the last segment
    ([64, 256, 700], 1020, 1, 1.0),
    ([300], 300, 2, 3.0),                # peaked scores: exercises the running-max rescale
    ([200], 200, 1, 0.05),               # nearly uniform attention
    ([100, 37], 1, 2, 1.0),              # a single query (the last row) against a cached prefix
    ([5, 17, 1, 64, 3, 40, 9, 70, 2, 33, 11, 8, 60, 1, 25, 30], 379, 1, 1.0),   # 16 segments
]


@pytest.mark.parametrize("seg_len,T_q,H,scale", ATTN_CASES)
def test_attention_q8_matches_oracle(seg_len, T_q, H, scale):
    say("attn q8", seg_len, T_q, H, scale)
    T_k = sum(seg_len)
    q, k, v = ditsynth.attention_inputs(T_q, T_k, H, seed=T_k + H + 1)
    q, k = ditsynth.to_bf16_grid(q * scale), ditsynth.to_bf16_grid(k * scale)
    buf = _quantize_on_gpu(q, k, v)
    o = torch.empty((T_q, H, 128), dtype=torch.bfloat16, device=DEV)
    dq.block_causal_attention_q8(buf, T_q, T_k, H, o, seg_len)
    torch.cuda.synchronize()
    c = _decode(buf, T_q, T_k, H)
    got = host(o)
    say(f"  rel_l2 vs unquantized attention {rel_l2(got, oracle.attention(q, k, v, seg_len)):.3e}")
    _check_envelope(got, c, seg_len, T_k)


def test_attention_q8_running_max_raised_mid_sequence():
    """Key norms grow tile by tile and spike late: the running max is raised
    (and a tile's P formed again) many times after the first tile; every P
    that is rounded to e4m3 stays below its saturation."""
    T, H = 704, 2
    q, k, v = ditsynth.attention_inputs(T, T, H, seed=10)
    growth = 1.0 + 0.6 * (np.arange(T) // 64)
    k = k * growth[:, None, None]
    k[600:606] *= 3.0
    q, k = ditsynth.to_bf16_grid(q), ditsynth.to_bf16_grid(k)
    buf = _quantize_on_gpu(q, k, v)
    c = _decode(buf, T, T, H)
    for seg_len in ([T], [100, 604]):
        say("attn q8 rising scores", seg_len)
        o = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
        dq.block_causal_attention_q8(buf, T, T, H, o, seg_len)
        torch.cuda.synchronize()
        _check_envelope(host(o), c, seg_len, T)


def test_attention_q8_exact_weights():
    """Integer scores (q/k codes with scale 1) and sm_scale = ln 2 make every P a
    power of two that e4m3 holds exactly; with V one-hot (448, scale 1) on a
    window of 128 keys, o[i, c] is key c's softmax weight times 448, which the
    kernel must reproduce for every key and query up to bf16 rounding."""
    seg_len = [40, 90, 333]
    T_k, T_q = sum(seg_len), 333
    rng = np.random.default_rng(1)
    q = np.zeros((T_q, 1, 128))
    k = np.zeros((T_k, 1, 128))
    q[:, :, 0] = 127
    q[:, :, 1] = 1
    k[:, :, 1] = rng.integers(0, 7, (T_k, 1))     # scores 0..6 (log2 units)
    k[:, :, 2] = 127                               # every K tile has amax 127
    for w0 in range(0, T_k, 128):
        v = np.zeros((T_k, 1, 128))
        n = min(128, T_k - w0)
        v[w0 + np.arange(n), 0, np.arange(n)] = 448.0
        buf = _quantize_on_gpu(q, k, v)
        o = torch.empty((T_q, 1, 128), dtype=torch.bfloat16, device=DEV)
        dq.block_causal_attention_q8(buf, T_q, T_k, 1, o, seg_len, math.log(2.0))
        torch.cuda.synchronize()
        c = _decode(buf, T_q, T_k, 1)
        assert np.all(c["sq"] == 1) and np.all(c["sk"] == 1) and np.all(c["sv"][0, :n] == 1)
        ref = oracle.attention_q8(c["q8"], c["sq"], c["k8"][:T_k], c["sk"], oracle.decode_fp8_e4m3(c["v8"][:T_k]),
                                  c["sv"], seg_len, scale=math.log(2.0))
        # fp32 arithmetic then one bf16 rounding: within one bf16 step of the exact value
        np.testing.assert_allclose(host(o), ref, rtol=2.0 ** -8, atol=1e-30)


def test_attention_q8_special_cases():
    """A query with one visible key returns that key's dequantized value; the
    result does not depend on keys a query cannot see; repeated calls agree."""
    seg_len = [1, 63, 200]
    T = sum(seg_len)
    q, k, v = ditsynth.attention_inputs(T, T, 2, seed=11)
    buf = _quantize_on_gpu(q, k, v)
    o = torch.empty((T, 2, 128), dtype=torch.bfloat16, device=DEV)
    o2 = torch.empty_like(o)
    dq.block_causal_attention_q8(buf, T, T, 2, o, seg_len)
    dq.block_causal_attention_q8(buf, T, T, 2, o2, seg_len)
    k2, v2 = k.copy(), v.copy()
    k2[64:] = -k2[64:]
    v2[64:] = v2[64:] * 0.5
    buf2 = _quantize_on_gpu(q, k2, v2)
    o3 = torch.empty_like(o)
    dq.block_causal_attention_q8(buf2, T, T, 2, o3, seg_len)
    torch.cuda.synchronize()
    c = _decode(buf, T, T, 2)
    v0 = oracle.decode_fp8_e4m3(c["v8"][0]) * c["sv"]            # [H, 128]
    got0 = host(o)[0]
    assert np.all(np.abs(got0 - v0) <= 2.0 ** -8 * np.abs(v0) + 1e-30)   # P = 1: only fp32/bf16 rounding
    assert torch.equal(o, o2)
    # keys 64.. changed: the rows that cannot see them keep their values up to the
    # V channel scales (which cover all keys); every row stays inside the envelope
    _check_envelope(host(o3), _decode(buf2, T, T, 2), seg_len, T)
    assert not torch.equal(o[64:], o3[64:])


def test_attention_q8_full_size_sampled():
    """2048^2 edit workload: 16,384 target queries over 17,664 keys, 32 heads."""
    seg_len = [256, 1024, 16384]
    T_k, T_q, H = 17664, 16384, 32
    say("attn q8 full", T_q, T_k, H)
    q, k, v = ditsynth.attention_inputs(T_q, T_k, H, seed=45)
    n, _ = dq.attn_q8_layout(T_q, T_k, H)
    buf = torch.empty(n, dtype=torch.uint8, device=DEV)
    dq.attn_quantize(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), buf)
    o = torch.empty((T_q, H, 128), dtype=torch.bfloat16, device=DEV)
    dq.block_causal_attention_q8(buf, T_q, T_k, H, o, seg_len)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 5000, 16383])
    q8, sq = oracle.quantize_attn_q(q[rows])
    k8, sk = oracle.quantize_attn_k(k)
    v8, sv = oracle.quantize_attn_v(v)
    c = {"q8": q8, "sq": sq, "k8": k8, "sk": sk, "v8": oracle.encode_fp8_e4m3(v8), "sv": sv}
    _check_envelope(host(o)[rows], c, [T_k], T_k)                  # target rows see every key


@pytest.mark.parametrize("mode", ["bf16", "w8a8"])
def test_block_with_quantized_attention(mode):
    w = ditsynth.custom("bq", 512, 4, 2048, 40, [(1, 3), (10, 12)], mode, 36)
    say("block attn_quant", mode, w.T)
    wt = ditsynth.block_weights(w)
    inp = ditsynth.block_inputs(w)
    gb = GpuBlock(w, wt, attn_quant=True)
    got = host(gb.run(inp["x"], inp["mod"], inp["mod_of_seg"]))
    c, s = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    ref = oracle.block_forward(inp["x"], inp["mod"], inp["mod_of_seg"], inp["seg_len"], c, s, wt, mode,
                               attn_quant=True)["x_out"]
    x = inp["x"].astype(np.float64)
    e_out, e_delta = rel_l2(got, ref), rel_l2(got - x, ref - x)
    say(f"  rel_l2 out {e_out:.3e} delta {e_delta:.3e}")
    assert e_out <= 2e-2 and e_delta <= 5e-2


def test_f32_mode_rejects_quantized_attention():
    w = ditsynth.custom("bqf", 512, 4, 2048, 16, [(8, 8)], "f32", 37)
    inp = ditsynth.block_inputs(w)
    gb = GpuBlock(w, attn_quant=True)
    with pytest.raises(dq.DitError):
        gb.run(inp["x"], inp["mod"], inp["mod_of_seg"])
