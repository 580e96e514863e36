"""GPU block-level parity against the oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import ditsynth
import oracle
import diffusion_transformer_text_qwen_amd as dq
from gpu_helpers import DEV, GpuBlock, act_dtype, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "w8a8": 2e-2}


def _oracle_block(w, wt, inp, qweights=None):
    c, s = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    return oracle.block_forward(inp["x"], inp["mod"], inp["mod_of_seg"], inp["seg_len"], c, s, wt, w.mode,
                                qweights=qweights)


def _check_block(w, label):
    say("block", label, w.name, w.mode, w.T)
    wt = ditsynth.block_weights(w)
    inp = ditsynth.block_inputs(w)
    gb = GpuBlock(w, wt)
    got = host(gb.run(inp["x"], inp["mod"], inp["mod_of_seg"]))
    ref = _oracle_block(w, wt, inp)["x_out"]
    x = inp["x"].astype(np.float64)
    e_out, e_delta = rel_l2(got, ref), rel_l2(got - x, ref - x)
    say(f"  rel_l2 out {e_out:.3e} delta {e_delta:.3e}")
    assert np.all(np.isfinite(got))
    assert e_out <= TOL[w.mode]
    assert e_delta <= TOL[w.mode] * (1 if w.mode == "f32" else 2.5)
    return gb, got


def test_block_tiny_fp32():
    _check_block(ditsynth.workload(0), "c0")


def test_block_bf16_256px():
    _check_block(ditsynth.workload(1), "c1")


def test_block_w8a8_512px_outliers():
    _check_block(ditsynth.workload(2), "c2")


@pytest.mark.parametrize("mode", ["f32", "bf16", "w8a8"])
def test_block_ragged_small(mode):
    # 40 + 10x12 = 160 rows: two 128-row tiles with a ragged tail, three segments incl. a short one
    w = ditsynth.custom("ragged", 512, 4, 2048, 40, [(1, 3), (10, 12)], mode, 30)
    _check_block(w, "ragged")


def test_zero_gates_identity():
    for mode in ("f32", "bf16", "w8a8"):
        w = ditsynth.custom("zg", 512, 4, 2048, 16, [(8, 8)], mode, 31)
        inp = ditsynth.block_inputs(w)
        inp["mod"][:, 2, :] = 0.0
        inp["mod"][:, 5, :] = 0.0
        gb = GpuBlock(w)
        got = gb.run(inp["x"], inp["mod"], inp["mod_of_seg"])
        assert torch.equal(got, dev(inp["x"], act_dtype(mode))), mode


def test_causal_invariance_and_determinism():
    w = ditsynth.custom("ci", 512, 4, 2048, 24, [(6, 6), (12, 12)], "w8a8", 32)
    inp = ditsynth.block_inputs(w)
    gb = GpuBlock(w)
    a = gb.run(inp["x"], inp["mod"], inp["mod_of_seg"]).clone()
    b = gb.run(inp["x"], inp["mod"], inp["mod_of_seg"]).clone()
    assert torch.equal(a, b)
    x2 = inp["x"].copy()
    P = w.prefix_len
    x2[P:] = ditsynth.to_bf16_grid(x2[P:] * 1.5 - 0.25)
    c = gb.run(x2, inp["mod"], inp["mod_of_seg"])
    assert torch.equal(a[:P], c[:P])
    assert not torch.equal(a[P:], c[P:])


@pytest.mark.parametrize("mode", ["bf16", "w8a8"])
def test_prefix_cache_two_steps(mode):
    """[text | ref | target]: step 1 fills the cache; step 2 on the target rows only
    equals step 2 computed uncached, bit for bit, and matches the oracle."""
    w = ditsynth.custom("edit", 512, 4, 2048, 32, [(8, 8), (16, 16)], mode, 33, steps=2)
    wt = ditsynth.block_weights(w)
    P = w.prefix_len
    s1 = ditsynth.block_inputs(w, step=0)
    s2 = ditsynth.block_inputs(w, step=1)
    cached = GpuBlock(w, wt)
    cached.run(s1["x"], s1["mod"], s1["mod_of_seg"])                        # uncached step 1
    out_c = cached.run(s2["x"][P:], s2["mod"], s2["mod_of_seg"])             # cached step 2
    fresh = GpuBlock(w, wt)
    out_u = fresh.run(s2["x"], s2["mod"], s2["mod_of_seg"])                  # uncached step 2
    assert torch.equal(out_c, out_u[P:])
    assert torch.equal(cached.k[:P], fresh.k[:P]) and torch.equal(cached.v[:P], fresh.v[:P])
    ref = _oracle_block(w, wt, s2)["x_out"][P:]
    x = s2["x"][P:].astype(np.float64)
    got = host(out_c)
    assert rel_l2(got, ref) <= TOL[mode]
    assert rel_l2(got - x, ref - x) <= 2.5 * TOL[mode]


@pytest.mark.parametrize("mode", ["bf16", "w8a8"])
def test_stack_step_with_head_tail_euler(mode):
    """Two blocks + DiT head/tail + Euler, every step through the C ABI."""
    w = ditsynth.custom("step", 512, 4, 2048, 24, [(8, 8)], mode, 34, n_blocks=2)
    st = ditsynth.step_inputs(w)
    inp = ditsynth.block_inputs(w)
    wts = [ditsynth.block_weights(w, b) for b in range(2)]
    D, L, N = w.D, w.text, 64
    bws = [dq.BlockWeights(a, mode) for a in wts]
    cfg = dq.block_config(mode, D, w.H, w.F)
    T = w.T
    cos = torch.empty((T, 64), dtype=torch.float32, device=DEV)
    sin = torch.empty((T, 64), dtype=torch.float32, device=DEV)
    dq.rope_tables(L, w.images, 0, T, cos, sin)
    lat = dev(st["latent"])
    lat_b = torch.empty((N, 64), dtype=torch.bfloat16, device=DEV)
    dq.cast(lat, lat_b)
    x = torch.empty((T, D), dtype=torch.bfloat16, device=DEV)
    dq.bf16_linear(dev(st["txt_feats"], torch.bfloat16), dev(st["w_txt_in"], torch.bfloat16), dev(st["b_txt_in"]), x[:L])
    dq.bf16_linear(lat_b, dev(st["w_img_in"], torch.bfloat16), dev(st["b_img_in"]), x[L:])
    kc = [torch.empty((T, w.H, 128), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    vc = [torch.empty((T, w.H, 128), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    ws = torch.empty(dq.workspace_bytes(cfg, T, T), dtype=torch.uint8, device=DEV)
    dq.stack_forward(cfg, bws, x, dev(inp["mod"]), inp["mod_of_seg"], cos, sin, w.seg_len, kc, vc, ws)
    hf = torch.empty((N, D), dtype=torch.bfloat16, device=DEV)
    mf = dev(st["mod_final"][0])
    dq.adaln_modulate(x[L:], mf[0], mf[1], h_out=hf)
    vel = torch.empty((N, 64), dtype=torch.bfloat16, device=DEV)
    dq.bf16_linear(hf, dev(st["w_proj_out"], torch.bfloat16), dev(st["b_proj_out"]), vel)
    dq.euler_step(lat, vel, float(st["sigma"]), float(st["sigma_next"]))
    torch.cuda.synchronize()
    c, s = oracle.rope_tables(oracle.rope_positions(L, w.images))
    ref = oracle.dit_step(st, [(a, None) for a in wts], inp["mod"], inp["mod_of_seg"], inp["seg_len"], c, s, mode)
    e_v = rel_l2(host(vel), ref["vel"])
    e_x = rel_l2(host(x), ref["x_blocks"])
    dlat = host(lat) - st["latent"]
    e_lat = rel_l2(dlat, ref["latent_next"] - st["latent"])
    say(f"  step {mode}: vel {e_v:.3e} x {e_x:.3e} dlat {e_lat:.3e}")
    assert e_x <= TOL[mode] and e_v <= 2.5 * TOL[mode] and e_lat <= 2.5 * TOL[mode]


def _sampled_rows_check(w, wt, inp, gpu_out, rows, k_prefix=None, v_prefix=None, cos_sin=None):
    c, s = cos_sin
    ref = oracle.block_forward_rows(inp["x"], inp["mod"], inp["mod_of_seg"], inp["seg_len"], c, s, wt, w.mode,
                                    rows, k_prefix=k_prefix, v_prefix=v_prefix)
    got = host(gpu_out)[rows]
    x = inp["x"][rows].astype(np.float64)
    e_out, e_delta = rel_l2(got, ref["x_out"]), rel_l2(got - x, ref["x_out"] - x)
    say(f"  sampled rows: rel_l2 out {e_out:.3e} delta {e_delta:.3e}")
    assert e_out <= TOL[w.mode] and e_delta <= 2.5 * TOL[w.mode]
    return ref


def test_block_w8a8_1024px_full_size_sampled():
    w = ditsynth.workload(3)
    say("c3 block 0 full size", w.T)
    wt = ditsynth.block_weights(w, 0)
    inp = ditsynth.block_inputs(w)
    gb = GpuBlock(w, wt)
    out = gb.run(inp["x"], inp["mod"], inp["mod_of_seg"])
    rows = np.array([0, 100, 255, 256, 257, 1000, 2222, 3333, 4351])
    cs = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    _sampled_rows_check(w, wt, inp, out, rows, cos_sin=cs)


def test_block_bf16_1024px_full_size_sampled():
    """bf16 mode at 4352 rows (large-tile GEMM path for every epilogue)."""
    w = ditsynth.custom("bf16_1024", 4096, 32, 16384, 256, [(64, 64)], "bf16", 35)
    wt = ditsynth.block_weights(w, 0)
    inp = ditsynth.block_inputs(w)
    gb = GpuBlock(w, wt)
    out = gb.run(inp["x"], inp["mod"], inp["mod_of_seg"])
    rows = np.array([0, 255, 256, 3000, 4351])
    cs = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    _sampled_rows_check(w, wt, inp, out, rows, cos_sin=cs)


def test_block_w8a8_2048px_edit_two_steps_sampled():
    """Prefix K/V written by the uncached step 1 and reused by the cached step 2."""
    w = ditsynth.workload(4)
    say("c4 two steps", w.T)
    wt = ditsynth.block_weights(w, 0)
    P = w.prefix_len
    s1 = ditsynth.block_inputs(w, step=0)
    s2 = ditsynth.block_inputs(w, step=1)
    gb = GpuBlock(w, wt)
    gb.run(s1["x"], s1["mod"], s1["mod_of_seg"])
    out = gb.run(s2["x"][P:], s2["mod"], s2["mod_of_seg"])
    c, s = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    qw = oracle.quantize_block_weights(wt)
    # oracle prefix K/V from step 1's prefix rows (prefix rows only see the prefix)
    pre = {k: (v[:P] if k == "x" else v) for k, v in s1.items()}
    pre["seg_len"] = np.array(w.seg_len[:-1], dtype=np.int32)
    pre["mod_of_seg"] = s1["mod_of_seg"][:-1]
    pref = oracle.block_forward_rows(pre["x"], pre["mod"], pre["mod_of_seg"], pre["seg_len"], c[:P], s[:P], wt,
                                     "w8a8", [0], qweights=qw)
    tgt = {"x": s2["x"][P:], "mod": s2["mod"], "mod_of_seg": s2["mod_of_seg"], "seg_len": s2["seg_len"]}
    rows = np.array([0, 1, 4095, 8000, 16383])
    ref = oracle.block_forward_rows(tgt["x"], tgt["mod"], tgt["mod_of_seg"], tgt["seg_len"], c[P:], s[P:], wt,
                                    "w8a8", rows, k_prefix=pref["k"], v_prefix=pref["v"], qweights=qw)
    got = host(out)[rows]
    x = tgt["x"][rows].astype(np.float64)
    e_out, e_delta = rel_l2(got, ref["x_out"]), rel_l2(got - x, ref["x_out"] - x)
    say(f"  c4 cached step: rel_l2 out {e_out:.3e} delta {e_delta:.3e}")
    assert e_out <= 2e-2 and e_delta <= 5e-2
    # the cache holds the prefix K of step 1 (post-norm, post-RoPE)
    kp = host(gb.k[:P]).reshape(P, w.H, 128)
    assert rel_l2(kp, pref["k"]) <= 2e-2
