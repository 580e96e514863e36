"""Denoise loop through dit_velocity_forward + dit_euler_step (GPU).

Parity: the loop's latent change against the oracle's loop (which recomputes
every row at every step).  Invariants: the cached-prefix loop equals the
recomputing loop bit for bit when the prefix is a whole number of 128-row
query blocks; graph replay equals eager execution bit for bit at every step,
with the loop's own eager copies, Euler launches and synchronizations between
the replays.
"""
import numpy as np
import pytest
import torch

import ditsynth
import oracle
import diffusion_transformer_text_qwen_amd as dq
from diffusion_transformer_text_qwen_amd.loop import DenoiseLoop
from gpu_helpers import DEV, act_dtype, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "w8a8": 2e-2}


class Setup:
    def __init__(self, mode, text, images, steps, n_blocks=2, seed=41):
        w = ditsynth.custom("loop", 512, 4, 2048, text, list(images), mode, seed, n_blocks=n_blocks)
        self.w, self.mode = w, mode
        self.li = ditsynth.loop_inputs(w, steps)
        self.wts = [ditsynth.block_weights(w, b) for b in range(n_blocks)]
        act = act_dtype(mode)
        self.blocks = [dq.BlockWeights(a, mode) for a in self.wts]
        self.cfg = dq.block_config(mode, w.D, w.H, w.F)
        li = self.li
        self.head = dq.HeadWeights({
            "w_txt_in": dev(li["w_txt_in"], act), "b_txt_in": dev(li["b_txt_in"]),
            "w_img_in": dev(li["w_img_in"], act), "b_img_in": dev(li["b_img_in"]),
            "w_proj_out": dev(li["w_proj_out"], act), "b_proj_out": dev(li["b_proj_out"])})
        T = w.T
        self.cos = torch.empty((T, 64), dtype=torch.float32, device=DEV)
        self.sin = torch.empty((T, 64), dtype=torch.float32, device=DEV)
        dq.rope_tables(w.text, w.images, 0, T, self.cos, self.sin)
        self.txt = dev(li["txt_feats"], act)
        self.ref = dev(li["ref_latent"]) if li["ref_latent"].shape[0] else None
        self.mods = dev(li["mods"])
        self.finals = dev(li["mod_finals"])

    def loop(self):
        return DenoiseLoop(self.cfg, self.blocks, self.head, self.w.seg_len, self.li["mod_of_seg"], self.w.text,
                           self.cos, self.sin, n_mod=self.li["mods"].shape[1])

    def run(self, cache_prefix, graph=False, per_step=False, quant_attn_from=None):
        lat = dev(self.li["latent"])
        steps = []
        on_step = (lambda i: (torch.cuda.synchronize(), steps.append(lat.clone()))) if per_step else None
        self.loop().run(lat, self.txt, self.ref, self.mods, self.finals, self.li["sigmas"],
                        cache_prefix=cache_prefix, graph=graph, on_step=on_step, quant_attn_from=quant_attn_from)
        torch.cuda.synchronize()
        return lat, steps

    def oracle(self, cache_prefix=False, quant_attn_from=None):
        c, s = oracle.rope_tables(oracle.rope_positions(self.w.text, self.w.images))
        return oracle.denoise_loop(self.li, [(a, None) for a in self.wts], self.li["mod_of_seg"], self.w.seg_len,
                                   c, s, self.mode, cache_prefix=cache_prefix, quant_attn_from=quant_attn_from)


@pytest.mark.parametrize("mode", ["w8a8", "bf16"])
def test_edit_loop_matches_oracle(mode):
    """[text 64 | reference 8x8 | target 16x16], 3 steps, prefix cached after step 0."""
    say("edit loop", mode)
    st = Setup(mode, 64, ((8, 8), (16, 16)), steps=3)
    lat, _ = st.run(cache_prefix=True)
    ref = st.oracle()
    lat0 = st.li["latent"].astype(np.float64)
    e = rel_l2(host(lat) - lat0, ref["latent"] - lat0)
    say(f"  latent change rel_l2 {e:.3e}")
    assert e <= 2.5 * TOL[mode]


def test_t2i_loop_f32_matches_oracle():
    say("t2i loop f32")
    st = Setup("f32", 16, ((8, 8),), steps=2)
    lat, _ = st.run(cache_prefix=False)
    ref = st.oracle()
    lat0 = st.li["latent"].astype(np.float64)
    e = rel_l2(host(lat) - lat0, ref["latent"] - lat0)
    say(f"  latent change rel_l2 {e:.3e}")
    assert e <= TOL["f32"]


def test_cached_prefix_equals_recompute_bitwise():
    """Prefix 64 + 64 = 128 rows: the target rows form the same query blocks in
    both loops, so every kernel sees the same operands."""
    say("cached == recompute")
    st = Setup("w8a8", 64, ((8, 8), (16, 16)), steps=3)
    a, _ = st.run(cache_prefix=True)
    b, _ = st.run(cache_prefix=False)
    assert torch.equal(a, b)


@pytest.mark.parametrize("cache_prefix,images,text", [(False, ((8, 8),), 16), (True, ((8, 8), (16, 16)), 64)])
def test_graph_replay_equals_eager_every_step(cache_prefix, images, text):
    say("graph replay", cache_prefix)
    st = Setup("w8a8", text, images, steps=5)
    _, eager = st.run(cache_prefix=cache_prefix, per_step=True)
    _, graphed = st.run(cache_prefix=cache_prefix, graph=True, per_step=True)
    assert len(eager) == len(graphed) == 5
    for i, (x, y) in enumerate(zip(eager, graphed)):
        assert torch.equal(x, y), f"step {i}"
    assert not torch.equal(eager[0], eager[-1])


@pytest.mark.parametrize("mode", ["w8a8", "bf16"])
def test_loop_with_quantized_attention_schedule(mode):
    """Step 0 with bf16 attention, steps 1-2 with int8/fp8 attention ([text | ref | target],
    prefix cached after step 0), against the oracle loop with the same schedule."""
    say("loop attn schedule", mode)
    st = Setup(mode, 64, ((8, 8), (16, 16)), steps=3)
    lat, _ = st.run(cache_prefix=True, quant_attn_from=1)
    ref = st.oracle(cache_prefix=True, quant_attn_from=1)
    lat0 = st.li["latent"].astype(np.float64)
    e = rel_l2(host(lat) - lat0, ref["latent"] - lat0)
    say(f"  latent change rel_l2 {e:.3e}")
    assert e <= 2.5 * TOL[mode]
    # the schedule changes the result (the quantized steps really ran)
    plain, _ = st.run(cache_prefix=True)
    assert not torch.equal(plain, lat)


def test_graph_replay_equals_eager_with_attention_schedule():
    st = Setup("w8a8", 64, ((8, 8), (16, 16)), steps=5)
    _, eager = st.run(cache_prefix=True, per_step=True, quant_attn_from=2)
    _, graphed = st.run(cache_prefix=True, graph=True, per_step=True, quant_attn_from=2)
    for i, (x, y) in enumerate(zip(eager, graphed)):
        assert torch.equal(x, y), f"step {i}"
