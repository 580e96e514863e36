"""The W8A8 recipe of the FlagOS page on the GPU (through the C ABI): asymmetric
per-token activation codes, zero-point W8A8 linears and the gated-MLP block with
a per-linear W8A8 choice, against the oracle."""
import numpy as np
import pytest
import torch

import ditsynth
import oracle
import diffusion_transformer_text_qwen_amd as dq
from gpu_helpers import DEV, bf16_ulp, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu


def _rows(M, K, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K)).astype(np.float32) * np.exp(rng.standard_normal((M, 1))).astype(np.float32)
    a[0] = np.abs(a[0])
    if M > 2:
        a[1] = -np.abs(a[1])
        a[2] = 0.0
    if M > 3:
        a[3] += 3.0
    return oracle.round_bf16(a)


@pytest.mark.parametrize("M,K", [(37, 520), (5, 4096), (300, 16384)])
def test_quantize_rows_asym_bit_exact(M, K):
    say("asym quant", M, K)
    a = _rows(M, K, M + K)
    q = torch.empty((M, K), dtype=torch.int8, device=DEV)
    s = torch.empty(M, dtype=torch.float32, device=DEV)
    z = torch.empty(M, dtype=torch.int32, device=DEV)
    dq.quantize_rows_asym(dev(a, torch.bfloat16), q, s, z)
    torch.cuda.synchronize()
    q_ref, s_ref, z_ref = oracle.quantize_rows_asym(a)
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(z.cpu().numpy(), z_ref)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


def test_int8_colsum_exact():
    rng = np.random.default_rng(3)
    w = rng.integers(-127, 128, (300, 1040)).astype(np.int8)
    out = torch.empty(300, dtype=torch.int32, device=DEV)
    dq.int8_colsum(dev(w, torch.int8), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), w.astype(np.int64).sum(axis=1))


def _asym_case(M, N, K, seed):
    a = _rows(M, K, seed)
    rng = np.random.default_rng(seed + 1)
    w = oracle.round_bf16(rng.standard_normal((N, K)) * 0.02)
    bias = oracle.round_bf16(rng.standard_normal(N) * 0.02)
    qa, sa, za = oracle.quantize_rows_asym(a)
    qw, sw = oracle.quantize_rows(w)
    return qa, sa, za, qw, sw, bias


@pytest.mark.parametrize("M,N,K,ws", [(70, 96, 256, False), (300, 1024, 1024, True)])
def test_w8a8_linear_asym_small(M, N, K, ws):
    say("w8a8 asym", M, N, K, ws)
    qa, sa, za, qw, sw, bias = _asym_case(M, N, K, M + N)
    wsum = torch.empty(N, dtype=torch.int32, device=DEV)
    qw_d = dev(qw, torch.int8)
    dq.int8_colsum(qw_d, wsum)
    yf = torch.empty((M, N), dtype=torch.float32, device=DEV)
    work = torch.empty((dq.w8a8_linear_workspace_bytes(),), dtype=torch.uint8, device=DEV) if ws else None
    dq.w8a8_linear_asym(dev(qa, torch.int8), dev(sa), dev(za, torch.int32), qw_d, dev(sw), wsum, dev(bias), yf,
                        workspace=work)
    torch.cuda.synchronize()
    ref = oracle.w8a8_linear_asym(qa, sa, za, qw, sw, bias)
    # fp32 epilogue: float(acc), two products and the bias add, each rounded once
    f32_err = 4 * 2.0 ** -24 * (np.abs(ref - bias[None, :]) + np.abs(bias)[None, :])
    assert np.all(np.abs(host(yf) - ref) <= f32_err)


def test_w8a8_linear_asym_full_shapes_sampled():
    """Large-tile kernel shapes (M = 4352): the zero-point correction in the
    persistent kernel's epilogue and in the K-split reduce."""
    rng = np.random.default_rng(1)
    for N, K in ((12288, 4096), (4096, 16384)):
        M = 4352
        say("w8a8 asym full", M, N, K)
        qa, sa, za, qw, sw, bias = _asym_case(M, N, K, N + K)
        wsum = torch.empty(N, dtype=torch.int32, device=DEV)
        qw_d = dev(qw, torch.int8)
        dq.int8_colsum(qw_d, wsum)
        yf = torch.empty((M, N), dtype=torch.float32, device=DEV)
        work = torch.empty((dq.w8a8_linear_workspace_bytes(),), dtype=torch.uint8, device=DEV)
        dq.w8a8_linear_asym(dev(qa, torch.int8), dev(sa), dev(za, torch.int32), qw_d, dev(sw), wsum, dev(bias), yf,
                            workspace=work)
        torch.cuda.synchronize()
        ms = rng.integers(0, M, 64)
        ms[:2] = [0, M - 1]
        ref = oracle.w8a8_linear_asym(qa[ms], sa[ms], za[ms], qw, sw, bias)
        f32_err = 4 * 2.0 ** -24 * (np.abs(ref - bias[None, :]) + np.abs(bias)[None, :])
        assert np.all(np.abs(host(yf)[ms] - ref) <= f32_err)
        del yf


class GatedSetup:
    def __init__(self, name, D, H, F, text, images, seed, n_blocks=1):
        self.w = ditsynth.custom(name, D, H, F, text, list(images), "bf16", seed, n_blocks=n_blocks)
        self.inp = ditsynth.block_inputs(self.w)
        self.wts = [ditsynth.gated_block_weights(self.w, b) for b in range(n_blocks)]
        T = self.w.T
        self.cos = torch.empty((T, 64), dtype=torch.float32, device=DEV)
        self.sin = torch.empty((T, 64), dtype=torch.float32, device=DEV)
        dq.rope_tables(self.w.text, self.w.images, 0, T, self.cos, self.sin)
        c, s = oracle.rope_tables(oracle.rope_positions(self.w.text, self.w.images))
        self.cos_h, self.sin_h = c, s

    def gpu(self, int8_per_block, attn_quant=False):
        w = self.w
        cfg = dq.block_config("bf16", w.D, w.H, w.F, attn_quant=attn_quant)
        T = w.T
        x = dev(self.inp["x"], torch.bfloat16)
        k = torch.zeros((T, w.H, 128), dtype=torch.bfloat16, device=DEV)
        v = torch.zeros_like(k)
        ws = torch.empty(dq.gated_workspace_bytes(cfg, T, T), dtype=torch.uint8, device=DEV)
        for b, arrays in enumerate(self.wts):
            gw = dq.GatedBlockWeights(arrays, int8_per_block[b])
            dq.block_forward_gated(cfg, gw, x, dev(self.inp["mod"]), self.inp["mod_of_seg"], self.cos, self.sin,
                                   w.seg_len, k, v, ws)
        torch.cuda.synchronize()
        return host(x)

    def oracle(self, int8_per_block, attn_quant=False):
        x = self.inp["x"]
        for b, arrays in enumerate(self.wts):
            names = tuple("w_" + n for n in int8_per_block[b])
            x = oracle.block_forward_gated(x, self.inp["mod"], self.inp["mod_of_seg"], self.inp["seg_len"],
                                           self.cos_h, self.sin_h, arrays, int8=names,
                                           attn_quant=attn_quant)["x_out"]
        return x


@pytest.mark.parametrize("int8,attn_quant", [((), False), (("qk", "proj", "gate"), False),
                                             (dq.GATED_LINEARS, False), (("qk", "proj", "gate"), True)])
def test_gated_block_matches_oracle(int8, attn_quant):
    # [40 | 1x3 | 10x12] = 163 rows: two 128-row query blocks with a ragged tail, three segments
    st = GatedSetup("gated", 512, 4, 1536, 40, [(1, 3), (10, 12)], 60)
    say("gated block", int8, attn_quant, st.w.T)
    got = st.gpu([int8], attn_quant)
    ref = st.oracle([int8], attn_quant)
    x = st.inp["x"].astype(np.float64)
    e_out, e_delta = rel_l2(got, ref), rel_l2(got - x, ref - x)
    say(f"  rel_l2 out {e_out:.3e} delta {e_delta:.3e}")
    assert np.all(np.isfinite(got))
    assert e_out <= 2e-2 and e_delta <= 5e-2


def test_gated_stack_with_the_pages_scope():
    """Six blocks, W8A8 on Q/K, proj and gate in blocks 2..3 (the page's 2..29 of 32,
    scaled to six blocks), bf16 elsewhere."""
    st = GatedSetup("gstack", 512, 4, 1536, 24, [(8, 8)], 61, n_blocks=6)
    scope = [dq.recipe_int8_linears(b, 6) for b in range(6)]
    assert scope[2] and scope[3] and not (scope[0] or scope[1] or scope[4] or scope[5])
    got = st.gpu(scope)
    ref = st.oracle(scope)
    x = st.inp["x"].astype(np.float64)
    e_out, e_delta = rel_l2(got, ref), rel_l2(got - x, ref - x)
    say(f"  gated stack rel_l2 out {e_out:.3e} delta {e_delta:.3e}")
    assert e_out <= 2e-2 and e_delta <= 5e-2
