"""Pins of the oracle's denoise loop (CPU only).

The loop is [CoreAI, Graph contracts]: velocity from the DiT, then one Euler
update of the target latent per step.  Pinned by closed forms of the Euler
recursion, by the prefix-cache invariance, and by agreement with dit_step.
"""
import numpy as np
import pytest

import ditsynth
import oracle


def _setup(mode, images=((4, 4), (8, 8)), steps=3, n_blocks=1, seed=31):
    w = ditsynth.custom("loop", 512, 4, 2048, 16, list(images), mode, seed, n_blocks=n_blocks)
    li = ditsynth.loop_inputs(w, steps)
    blocks = [(ditsynth.block_weights(w, b), None) for b in range(n_blocks)]
    pos = oracle.rope_positions(w.text, w.images)
    cos, sin = oracle.rope_tables(pos)
    return w, li, blocks, cos, sin


def test_constant_velocity_closed_form():
    """proj_out = 0 with bias c makes every step's velocity c, so the Euler
    recursion telescopes: latent_S = latent_0 + (sigma_S - sigma_0) c."""
    w, li, blocks, cos, sin = _setup("bf16")
    c = ditsynth.to_bf16_grid(np.linspace(-1.5, 2.0, 64).astype(np.float32))
    li["w_proj_out"] = np.zeros_like(li["w_proj_out"])
    li["b_proj_out"] = c
    out = oracle.denoise_loop(li, blocks, li["mod_of_seg"], w.seg_len, cos, sin, "bf16")
    sig = li["sigmas"].astype(np.float64)
    want = li["latent"].astype(np.float64) + (sig[-1] - sig[0]) * c.astype(np.float64)[None, :]
    assert np.allclose(out["latent"], want, rtol=0, atol=1e-12)
    assert np.array_equal(out["vel"], np.broadcast_to(c.astype(np.float64), out["vel"].shape))


def test_constant_sigma_is_identity():
    w, li, blocks, cos, sin = _setup("f32", images=((8, 8),), steps=2)
    li["sigmas"] = np.full_like(li["sigmas"], 0.5)
    out = oracle.denoise_loop(li, blocks, li["mod_of_seg"], w.seg_len, cos, sin, "f32")
    assert np.array_equal(out["latent"], li["latent"].astype(np.float64))


def test_prefix_cache_matches_recompute():
    """Editing: text and reference rows use the step-independent set 0, so
    reusing their step-0 K/V gives the recomputed values (f32: no rounding
    points, so equal to BLAS summation order)."""
    w, li, blocks, cos, sin = _setup("f32", steps=3, n_blocks=2)
    full = oracle.denoise_loop(li, blocks, li["mod_of_seg"], w.seg_len, cos, sin, "f32")
    cached = oracle.denoise_loop(li, blocks, li["mod_of_seg"], w.seg_len, cos, sin, "f32", cache_prefix=True)
    assert np.allclose(cached["latent"], full["latent"], rtol=0, atol=1e-10)
    # a wrong prefix (the step's own target set for the prefix) must change the result
    li2 = dict(li)
    li2["mods"] = li["mods"][:, ::-1].copy()
    other = oracle.denoise_loop(li2, blocks, li["mod_of_seg"], w.seg_len, cos, sin, "f32", cache_prefix=True)
    assert not np.allclose(other["latent"], full["latent"], rtol=0, atol=1e-6)


def test_one_step_matches_dit_step():
    w, li, blocks, cos, sin = _setup("bf16", images=((8, 8),), steps=1, n_blocks=2)
    out = oracle.denoise_loop(li, blocks, li["mod_of_seg"], w.seg_len, cos, sin, "bf16")
    step_in = dict(li)
    step_in["mod_final"] = li["mod_finals"][:1]
    step_in["sigma"], step_in["sigma_next"] = li["sigmas"][0], li["sigmas"][1]
    ref = oracle.dit_step(step_in, blocks, li["mods"][0], li["mod_of_seg"], w.seg_len, cos, sin, "bf16")
    assert np.array_equal(out["latent"], ref["latent_next"])
    assert np.array_equal(out["vel"], ref["vel"])


def test_loop_sigmas_schedule():
    s = ditsynth.loop_sigmas(40)
    assert s.shape == (41,) and s[0] == 1.0 and s[-1] == 0.0
    assert abs(float(s[39]) - 0.02) < 1e-6 and abs(float(s[1]) - (1 - 0.98 / 39)) < 1e-7
    assert np.all(np.diff(s) < 0)
