"""Compositions at the workloads' full sizes against the oracle (through the C ABI).

* One DiT evaluation of the 1024^2 step (256 text + 4096 image tokens, width
  4096, W8A8) through dit_velocity_forward with four blocks of distinct
  weights, against oracle.dit_step: the velocity and the block stack's output
  rows ("RGBA-Image-2.1 - Core AI port of Qwen-Image-2.1", Graph contracts).
* The gated-MLP block of the FlagOS recipe at its own width (F = 12288) and
  the 1024^2 token count, with the page's W8A8 scope and with every linear
  W8A8 ("Qwen-Image-2.1 W8A8 - FlagOS for Mac", Quantization and validation).

These run the oracle at 4352 rows (about 10 s of host time per block).
"""
import numpy as np
import pytest
import torch

import ditsynth
import oracle
import diffusion_transformer_text_qwen_amd as dq
from gpu_helpers import DEV, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu

# Block output tolerance (the block's bar); a stack of n blocks adds the
# independent rounding and code-flip errors of each block, so its bar scales
# with sqrt(n).
TOL_BLOCK = 2e-2


@pytest.mark.timeout(1200)
def test_velocity_forward_1024px_four_blocks():
    n_blocks = 4
    w = ditsynth.custom("step1024x4", 4096, 32, 16384, 256, [(64, 64)], "w8a8", 3, n_blocks=n_blocks)
    say("velocity 1024px", n_blocks, "blocks", w.T)
    st = ditsynth.step_inputs(w)
    inp = ditsynth.block_inputs(w)
    D, L, N, T = w.D, w.text, w.seg_len[-1], w.T
    cfg = dq.block_config("w8a8", D, w.H, w.F)
    bws, blocks = [], []
    for b in range(n_blocks):
        arrays = ditsynth.block_weights(w, b)
        bws.append(dq.BlockWeights(arrays, "w8a8"))
        blocks.append((arrays, None))
    head = dq.HeadWeights({
        "w_txt_in": dev(st["w_txt_in"], torch.bfloat16), "b_txt_in": dev(st["b_txt_in"]),
        "w_img_in": dev(st["w_img_in"], torch.bfloat16), "b_img_in": dev(st["b_img_in"]),
        "w_proj_out": dev(st["w_proj_out"], torch.bfloat16), "b_proj_out": dev(st["b_proj_out"])})
    cos = torch.empty((T, 64), dtype=torch.float32, device=DEV)
    sin = torch.empty((T, 64), dtype=torch.float32, device=DEV)
    dq.rope_tables(L, w.images, 0, T, cos, sin)
    kc = [torch.empty((T, w.H, 128), dtype=torch.bfloat16, device=DEV) for _ in range(n_blocks)]
    vc = [torch.empty_like(k) for k in kc]
    ws = torch.empty(dq.velocity_workspace_bytes(cfg, T, N, 64), dtype=torch.uint8, device=DEV)
    vel = torch.empty((N, 64), dtype=torch.bfloat16, device=DEV)
    dq.velocity_forward(cfg, bws, head, dev(st["latent"]), vel, dev(inp["mod"]), inp["mod_of_seg"],
                        dev(st["mod_final"][0]), cos, sin, w.seg_len, kc, vc, ws,
                        txt_feats=dev(st["txt_feats"], torch.bfloat16), L_txt=L)
    torch.cuda.synchronize()
    x_blocks = host(ws[:T * D * 2].view(torch.bfloat16).view(T, D))
    got_vel = host(vel)
    assert np.all(np.isfinite(got_vel)) and np.all(np.isfinite(x_blocks))
    del bws
    torch.cuda.empty_cache()
    c, s = oracle.rope_tables(oracle.rope_positions(L, w.images))
    ref = oracle.dit_step(st, blocks, inp["mod"], inp["mod_of_seg"], inp["seg_len"], c, s, "w8a8")
    # the stack input: the head's rows (txt_in, img_in of the bf16 latent), computed by the oracle
    x0 = np.concatenate([
        oracle.round_bf16(oracle.linear(st["txt_feats"], st["w_txt_in"], st["b_txt_in"])),
        oracle.round_bf16(oracle.linear(oracle.round_bf16(st["latent"]), st["w_img_in"], st["b_img_in"]))])
    e_x = rel_l2(x_blocks, ref["x_blocks"])
    e_dx = rel_l2(x_blocks - x0, ref["x_blocks"] - x0)
    e_v = rel_l2(got_vel, ref["vel"])
    say(f"  4 blocks: x rel_l2 {e_x:.3e} (delta {e_dx:.3e}), vel {e_v:.3e}")
    bar = TOL_BLOCK * np.sqrt(n_blocks)
    assert e_x <= bar and e_dx <= 2.5 * bar and e_v <= 2.5 * bar
    # the Euler update of the step on this velocity
    lat = dev(st["latent"])
    dq.euler_step(lat, vel, float(st["sigma"]), float(st["sigma_next"]))
    torch.cuda.synchronize()
    want = oracle.euler_update(st["latent"], got_vel, float(st["sigma"]), float(np.float32(st["sigma_next"])))
    assert np.all(np.abs(host(lat) - want) <= 4 * 2.0 ** -24 * (np.abs(want) + 1.0))


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("scope", ["page", "all", "mxfp4"])
def test_gated_block_1024px_full_width(scope):
    """scope: the page's W8A8 linears, every linear W8A8, or every linear
    MXFP4 (decoded in the GEMM's operand staging at this size)."""
    w = ditsynth.custom("gated1024", 4096, 32, 12288, 256, [(64, 64)], "bf16", 62)
    T = w.T
    say("gated block 1024px F=12288", scope, T)
    arrays = ditsynth.gated_block_weights(w, 0)
    inp = ditsynth.block_inputs(w)
    int8 = {"page": ("qk", "proj", "gate"), "all": dq.GATED_LINEARS, "mxfp4": ()}[scope]
    mx = None
    if scope == "mxfp4":
        D, F = w.D, w.F
        shapes = {"qk": (2 * D, D), "v": (D, D), "o": (D, D), "proj": (F, D), "gate": (F, D), "down": (D, F)}
        mx = {n: ditsynth.mxfp4_weights(*shp, seed=80 + i) for i, (n, shp) in enumerate(shapes.items())}
    cfg = dq.block_config("bf16", w.D, w.H, w.F)
    cos = torch.empty((T, 64), dtype=torch.float32, device=DEV)
    sin = torch.empty((T, 64), dtype=torch.float32, device=DEV)
    dq.rope_tables(w.text, w.images, 0, T, cos, sin)
    x = dev(inp["x"], torch.bfloat16)
    k = torch.zeros((T, w.H, 128), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    ws = torch.empty(dq.gated_workspace_bytes(cfg, T, T), dtype=torch.uint8, device=DEV)
    gw = dq.GatedBlockWeights(arrays, int8, mx=mx)
    dq.block_forward_gated(cfg, gw, x, dev(inp["mod"]), inp["mod_of_seg"], cos, sin, w.seg_len, k, v, ws)
    torch.cuda.synchronize()
    got = host(x)
    del gw, ws
    torch.cuda.empty_cache()
    c, s = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    ref = oracle.block_forward_gated(inp["x"], inp["mod"], inp["mod_of_seg"], inp["seg_len"], c, s, arrays,
                                     int8=tuple("w_" + n for n in int8),
                                     mx={"w_" + n: cs for n, cs in mx.items()} if mx else None)["x_out"]
    x0 = inp["x"].astype(np.float64)
    e_out, e_delta = rel_l2(got, ref), rel_l2(got - x0, ref - x0)
    say(f"  gated {scope}: rel_l2 out {e_out:.3e} delta {e_delta:.3e}")
    assert np.all(np.isfinite(got))
    assert e_out <= TOL_BLOCK and e_delta <= 2.5 * TOL_BLOCK
