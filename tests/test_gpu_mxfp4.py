"""MXFP4 weights on the GPU (through the C ABI): the expansion to bf16 is exact
against the oracle's decoding, the MXFP4 linear is the bf16 linear on the
decoded weights, and the gated block with MXFP4 linears matches the oracle."""
import numpy as np
import pytest
import torch

import ditsynth
import oracle
import diffusion_transformer_text_qwen_amd as dq
from gpu_helpers import DEV, bf16_ulp, dev, host, rel_l2, say
from test_gpu_gated import GatedSetup

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K,lo,hi", [(37, 96, 100, 140), (4096, 4096, 115, 125), (3, 64, 1, 250)])
def test_mxfp4_expand_exact(N, K, lo, hi):
    """Every code and scales across the normal bf16 range; scales near the range ends
    keep the products normal (2^(e-127) * 0.5 >= 2^-126 needs e >= 1)."""
    say("mxfp4 expand", N, K)
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    codes[0, :8] = np.arange(0, 256, 32, dtype=np.uint8) | np.arange(8, dtype=np.uint8)   # all low / high nibbles
    scales = rng.integers(lo, hi + 1, (N, K // 32)).astype(np.uint8)
    if lo <= 2:
        scales[:, 0] = 2                      # smallest product 0.5 * 2^-125 = 2^-126: normal
    out = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    dq.mxfp4_expand(dev(codes, torch.uint8), dev(scales, torch.uint8), out)
    torch.cuda.synchronize()
    ref = oracle.mxfp4_decode(codes, scales)
    np.testing.assert_array_equal(host(out), ref)


@pytest.mark.parametrize("M,N,K", [(100, 272, 640), (4352, 4096, 4096)])
def test_mxfp4_linear(M, N, K):
    say("mxfp4 linear", M, N, K)
    rng = np.random.default_rng(M + N)
    a = ditsynth.to_bf16_grid(rng.standard_normal((M, K)).astype(np.float32))
    codes, scales = ditsynth.mxfp4_weights(N, K, seed=M)
    bias = ditsynth.to_bf16_grid((rng.standard_normal(N) * 0.02).astype(np.float32))
    ws = torch.empty(dq.lib().mxfp4_linear_workspace_bytes(N, K), dtype=torch.uint8, device=DEV)
    yf = torch.empty((M, N), dtype=torch.float32, device=DEV)
    dq.mxfp4_linear(dev(a, torch.bfloat16), dev(codes, torch.uint8), dev(scales, torch.uint8), dev(bias), yf, ws)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 512 else np.concatenate([np.arange(8), rng.integers(0, M, 56)])
    w = oracle.mxfp4_decode(codes, scales)
    ref = oracle.linear(a[rows], w, bias)
    # fp32 accumulation of exact bf16 products: |err| <= K * 2^-24 * sum|a w|
    acc_bound = K * 2.0 ** -24 * (np.abs(a[rows].astype(np.float64)) @ np.abs(w).T)
    assert np.all(np.abs(host(yf)[rows] - ref) <= acc_bound + 1e-30)


@pytest.mark.parametrize("M,N,K", [(4352, 4096, 4096), (4429, 4144, 2048), (1024, 12288, 4096)])
def test_mxfp4_linear_decoded_in_staging_equals_expanded(M, N, K):
    """Shapes on the large-tile GEMM decode the MXFP4 codes in its operand
    staging: bitwise the bf16 linear on the expanded weights (same tiles, same
    MFMA order), including ragged M and N."""
    say("mxfp4 direct", M, N, K)
    rng = np.random.default_rng(M + N + K)
    a = ditsynth.to_bf16_grid(rng.standard_normal((M, K)).astype(np.float32))
    codes, scales = ditsynth.mxfp4_weights(N, K, seed=K)
    bias = ditsynth.to_bf16_grid((rng.standard_normal(N) * 0.02).astype(np.float32))
    ad, cd, sd, bd = dev(a, torch.bfloat16), dev(codes, torch.uint8), dev(scales, torch.uint8), dev(bias)
    ws = torch.full((dq.lib().mxfp4_linear_workspace_bytes(N, K),), 0x7F, dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    dq.mxfp4_linear(ad, cd, sd, bd, y, ws)
    w_exp = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    dq.mxfp4_expand(cd, sd, w_exp)
    y2 = torch.empty_like(y)
    dq.bf16_linear(ad, w_exp, bd, y2)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    # the workspace (the expansion target of small shapes) is not touched
    assert bool((ws == 0x7F).all())
    np.testing.assert_array_equal(host(w_exp)[::97], oracle.mxfp4_decode(codes[::97], scales[::97]))


@pytest.mark.parametrize("attn_quant", [False, True])
def test_gated_block_with_mxfp4_linears(attn_quant):
    """All six linears MXFP4 (the page's checkpoint quantizes every main matrix)."""
    st = GatedSetup("gmx", 512, 4, 1536, 40, [(1, 3), (10, 12)], 62)
    D, F = 512, 1536
    shapes = {"qk": (2 * D, D), "v": (D, D), "o": (D, D), "proj": (F, D), "gate": (F, D), "down": (D, F)}
    mx = {n: ditsynth.mxfp4_weights(*shp, seed=70 + i) for i, (n, shp) in enumerate(shapes.items())}
    say("gated block mxfp4", attn_quant)
    w = st.w
    cfg = dq.block_config("bf16", w.D, w.H, w.F, attn_quant=attn_quant)
    x = dev(st.inp["x"], torch.bfloat16)
    k = torch.zeros((w.T, w.H, 128), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    ws = torch.empty(dq.gated_workspace_bytes(cfg, w.T, w.T), dtype=torch.uint8, device=DEV)
    gw = dq.GatedBlockWeights(st.wts[0], mx=mx)
    dq.block_forward_gated(cfg, gw, x, dev(st.inp["mod"]), st.inp["mod_of_seg"], st.cos, st.sin, w.seg_len, k, v, ws)
    torch.cuda.synchronize()
    got = host(x)
    ref = oracle.block_forward_gated(st.inp["x"], st.inp["mod"], st.inp["mod_of_seg"], st.inp["seg_len"], st.cos_h,
                                     st.sin_h, st.wts[0], attn_quant=attn_quant,
                                     mx={"w_" + n: cs for n, cs in mx.items()})["x_out"]
    x0 = st.inp["x"].astype(np.float64)
    e_out, e_delta = rel_l2(got, ref), rel_l2(got - x0, ref - x0)
    say(f"  rel_l2 out {e_out:.3e} delta {e_delta:.3e}")
    assert np.all(np.isfinite(got))
    assert e_out <= 2e-2 and e_delta <= 5e-2
