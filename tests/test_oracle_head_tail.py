"""Pins of the oracle's DiT head and tail (dit_step, denoise_loop), CPU only.

"RGBA-Image-2.1 - Core AI port of Qwen-Image-2.1", Graph contracts: the DiT
maps the packed latent [N, 64] and the text features [L, D] to a velocity
[N, 64] over the sequence [text | image]; one Euler update follows.

With every block's gates at zero a block is the identity (pinned in
test_oracle_block), so the step reduces to the head and the tail alone:
    vel = proj_out(LN(img_in(latent)) * (1 + scale_f) + shift_f)
on the image rows only.  That closed form is computed here with torch's
layer_norm and linear in fp64 (library routines, not the oracle's code), and
the order of the text and image rows inside the stack is pinned by the
block-causal invariant: the text rows of the stack output depend on the text
features only, and equal the stack run on the text rows alone.

Each pin is also run against mutated copies of the oracle's functions (shift
and scale swapped, the tail reading text rows, the text and image rows swapped
in the sequence); every mutant must fail at least one pin.
"""
import inspect
import textwrap

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import ditsynth
import oracle
from oracle import dit_oracle


def _zero_gates(wt, mod):
    mod = np.array(mod, copy=True)
    mod[..., 2, :] = 0.0
    mod[..., 5, :] = 0.0
    return mod


def _t(a):
    return torch.as_tensor(np.asarray(a, np.float64))


def _tail_closed_form(x_img, mf, w_out, b_out, round_bf16=False):
    """proj_out(LN(x_img)(1 + scale) + shift) with torch fp64 (bf16 rounding of
    the stored tensors by torch's own conversion when asked)."""
    def st(t):
        return t.to(torch.bfloat16).to(torch.float64) if round_bf16 else t
    x = _t(x_img)
    h = F.layer_norm(x, (x.shape[-1],), eps=1e-6) * (1.0 + _t(mf[1])) + _t(mf[0])
    h = st(h)
    return st(F.linear(h, _t(w_out), _t(b_out))).numpy()


def _head_closed_form(lat, w, b, round_bf16=False):
    def st(t):
        return t.to(torch.bfloat16).to(torch.float64) if round_bf16 else t
    return st(F.linear(st(_t(lat)), _t(w), _t(b))).numpy()


def _setup_step(mode, text=6, grid=(3, 5), n_blocks=2, seed=11):
    w = ditsynth.custom("ht", 256, 2, 512, text, [grid], mode, seed, n_blocks=n_blocks)
    st = ditsynth.step_inputs(w)
    inp = ditsynth.block_inputs(w)
    cos, sin = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    blocks = [(ditsynth.block_weights(w, b), None) for b in range(n_blocks)]
    return w, st, inp, cos, sin, blocks


def _check_step(step_fn, mode="f32"):
    """All head/tail pins of one dit_step implementation; returns a list of the
    failed pins' names (empty when every pin holds)."""
    failed = []
    w, st, inp, cos, sin, blocks = _setup_step(mode)
    L = w.text
    rb = mode != "f32"
    tol = 1e-10 if mode == "f32" else 0.0
    # 1. zero gates: velocity is the head/tail closed form on the image rows
    mod0 = _zero_gates(None, inp["mod"])
    r = step_fn(st, blocks, mod0, inp["mod_of_seg"], inp["seg_len"], cos, sin, mode)
    x_img = _head_closed_form(st["latent"], st["w_img_in"], st["b_img_in"], rb)
    x_txt = _head_closed_form(st["txt_feats"], st["w_txt_in"], st["b_txt_in"], rb)
    vel = _tail_closed_form(x_img, st["mod_final"][0], st["w_proj_out"], st["b_proj_out"], rb)
    if mode == "f32":
        ok = np.allclose(r["vel"], vel, rtol=1e-10, atol=1e-12)
    else:
        # torch and NumPy sum in different orders; a bf16 rounding may land on
        # the other side of a tie-free boundary for a few values.
        ok = np.mean(r["vel"] == vel) > 0.97 and np.allclose(r["vel"], vel, rtol=2 ** -7, atol=1e-6)
    if not ok:
        failed.append("zero-gate velocity")
    if not np.allclose(r["x_blocks"], np.concatenate([x_txt, x_img]), rtol=tol, atol=tol + 1e-12):
        failed.append("zero-gate stack rows")
    want_next = st["latent"].astype(np.float64) + (float(st["sigma_next"]) - float(st["sigma"])) * vel
    if not np.allclose(r["latent_next"], want_next, rtol=1e-6, atol=1e-6):
        failed.append("euler")
    # 2. live blocks: the text rows of the stack see only the text rows
    r1 = step_fn(st, blocks, inp["mod"], inp["mod_of_seg"], inp["seg_len"], cos, sin, mode)
    st2 = dict(st)
    st2["latent"] = st["latent"] + np.float32(0.5)
    r2 = step_fn(st2, blocks, inp["mod"], inp["mod_of_seg"], inp["seg_len"], cos, sin, mode)
    if not np.array_equal(r1["x_blocks"][:L], r2["x_blocks"][:L]):
        failed.append("text rows independent of the latent")
    if np.allclose(r1["x_blocks"][L:], r2["x_blocks"][L:]):
        failed.append("image rows follow the latent")
    # the text rows equal the stack on the text segment alone
    xt = x_txt.copy()
    for wts, q in blocks:
        xt = oracle.block_forward(xt, inp["mod"], inp["mod_of_seg"][:1], np.array([L], np.int32),
                                  cos[:L], sin[:L], wts, mode, qweights=q)["x_out"]
    if not np.allclose(r1["x_blocks"][:L], xt, rtol=1e-9, atol=1e-9):
        failed.append("text rows equal the text-only stack")
    return failed


def _mutant(fn, old, new):
    """A copy of oracle function ``fn`` with one source substring replaced,
    compiled in the oracle module's namespace (a planted mistake, CPU only)."""
    src = textwrap.dedent(inspect.getsource(fn))
    assert src.count(old) == 1, (fn.__name__, old)
    ns = dict(vars(dit_oracle))
    exec(compile(src.replace(old, new), f"<mutant {fn.__name__}>", "exec"), ns)
    return ns[fn.__name__]


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_dit_step_head_tail_pins_hold(mode):
    assert _check_step(oracle.dit_step, mode) == []


STEP_MUTANTS = [
    ("mf[0], mf[1])", "mf[1], mf[0])"),                               # shift and scale swapped
    ("x[L:]", "x[:x.shape[0] - L]"),                                   # tail reads the first rows
    ("np.concatenate([x_txt, x_img]", "np.concatenate([x_img, x_txt]"),   # image rows first
    ("linear(_store(lat, mode), step_in[\"w_img_in\"]", "linear(_store(lat, mode) * 0.5, step_in[\"w_img_in\"]"),
]


@pytest.mark.parametrize("old,new", STEP_MUTANTS)
def test_dit_step_pins_catch_mutants(old, new):
    bad = _mutant(oracle.dit_step, old, new)
    assert _check_step(bad, "f32") != []


# ------------------------------------------------------------------ denoise loop

def _setup_loop(mode, steps=2):
    w = ditsynth.custom("htl", 256, 2, 512, 5, [(2, 3), (3, 4)], mode, 13, n_blocks=2)
    li = ditsynth.loop_inputs(w, steps)
    blocks = [(ditsynth.block_weights(w, b), None) for b in range(2)]
    cos, sin = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    return w, li, blocks, cos, sin


def _check_loop(loop_fn, cache_prefix=False):
    failed = []
    w, li, blocks, cos, sin = _setup_loop("f32")
    L, R = w.text, w.seg_len[1]
    li0 = dict(li)
    li0["mods"] = _zero_gates(None, li["mods"])
    out = loop_fn(li0, blocks, li["mod_of_seg"], w.seg_len, cos, sin, "f32", cache_prefix=cache_prefix)
    lat = li["latent"].astype(np.float64)
    sig = li["sigmas"].astype(np.float64)
    for i in range(len(sig) - 1):
        x_img = _head_closed_form(lat, li["w_img_in"], li["b_img_in"])
        vel = _tail_closed_form(x_img, li["mod_finals"][i], li["w_proj_out"], li["b_proj_out"])
        lat = lat + (sig[i + 1] - sig[i]) * vel
    if not (np.allclose(out["latent"], lat, rtol=1e-9, atol=1e-10) and
            np.allclose(out["vel"], vel, rtol=1e-9, atol=1e-10)):
        failed.append("zero-gate loop closed form")
    # live blocks: the target's velocity depends on the text and the reference
    base = loop_fn(li, blocks, li["mod_of_seg"], w.seg_len, cos, sin, "f32", cache_prefix=cache_prefix)
    for key in ("txt_feats", "ref_latent"):
        li2 = dict(li)
        li2[key] = li[key] + np.float32(0.25)
        o2 = loop_fn(li2, blocks, li["mod_of_seg"], w.seg_len, cos, sin, "f32", cache_prefix=cache_prefix)
        if np.allclose(o2["vel"], base["vel"], rtol=0, atol=1e-9):
            failed.append(f"velocity depends on {key}")
    # the reference and target rows go through img_in: with img_in's weight
    # doubled and both latents halved (constant sigmas, so the latent stays
    # put) every row of the sequence is the same and so is the velocity
    lic = dict(li)
    lic["sigmas"] = np.full_like(li["sigmas"], 0.5)
    basec = loop_fn(lic, blocks, li["mod_of_seg"], w.seg_len, cos, sin, "f32", cache_prefix=cache_prefix)
    li3 = dict(lic)
    li3["ref_latent"] = li["ref_latent"] * np.float32(0.5)
    li3["w_img_in"] = li["w_img_in"] * np.float32(2.0)
    li3["latent"] = li["latent"] * np.float32(0.5)
    o3 = loop_fn(li3, blocks, li["mod_of_seg"], w.seg_len, cos, sin, "f32", cache_prefix=cache_prefix)
    if not np.allclose(o3["vel"], basec["vel"], rtol=1e-9, atol=1e-10):
        failed.append("reference rows use img_in")
    return failed


@pytest.mark.parametrize("cache_prefix", [False, True])
def test_denoise_loop_head_tail_pins_hold(cache_prefix):
    assert _check_loop(oracle.denoise_loop, cache_prefix) == []


LOOP_MUTANTS = [
    ("mf[0], mf[1])", "mf[1], mf[0])"),
    ("x[x.shape[0] - N:]", "x[:N]"),
    ("parts + [x_tgt]", "[x_tgt] + parts"),
    ("linear(_store(ref, mode), loop_in[\"w_img_in\"]", "linear(_store(ref, mode), loop_in[\"w_txt_in\"][:, :64]"),
]


@pytest.mark.parametrize("old,new", LOOP_MUTANTS)
def test_denoise_loop_pins_catch_mutants(old, new):
    bad = _mutant(oracle.denoise_loop, old, new)
    assert _check_loop(bad) != []
