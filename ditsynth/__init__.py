"""Seeded synthetic inputs for the single-stream DiT block.

This module is shared by the CPU oracle (``oracle/``) and the HIP path
(``diffusion_transformer_text_qwen_amd``).  It only draws random numbers and
arranges them into the shapes of the five workloads below; it contains none of
the block's arithmetic.  The one computation it performs on the draws is the
synthesis of adaLN modulation rows from a random timestep embedding
(``mod = SiLU(temb) @ W_mod.T + b_mod``): the pages never describe the
timestep embedder, so it is treated as part of input synthesis, not of the
block (the block consumes ``mod`` as an input).

Workloads (token counts: one token per 16x16 pixel tile, no 2x2 packing, as in
the Core AI port of Qwen-Image-2.1, section "Graph contracts"):

  0 tiny_fp32        D=512,  H=4,  F=2048,  [text 16  | image 8x8]            fp32, seed 0
  1 block_bf16_256   D=4096, H=32, F=16384, [text 64  | image 16x16]          bf16, seed 1
  2 block_w8a8_512   D=4096, H=32, F=16384, [text 128 | image 32x32]          W8A8 + 0.1% x8 outliers, seed 2
  3 stack_w8a8_1024  32 blocks, [text 256 | image 64x64], W8A8, head/tail + Euler, seed 3
  4 edit_w8a8_2048   [text 256 | ref 32x32 | target 128x128], W8A8, 2 steps with prefix K/V, seed 4

Distributions: weights and biases N(0, 0.02); RMSNorm gains 1 + N(0, 0.02);
activations, latents, text features and timestep embeddings N(0, 1).  In the
bf16 and W8A8 workloads every bf16 tensor (activations, bf16 weights, biases,
gains) is drawn in fp32 and stored on the bf16 grid (round to nearest even);
W8A8 weight masters stay fp32 (they are quantized to int8 at load time by
each side independently).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    idx: int
    name: str
    D: int
    H: int
    F: int
    text: int
    images: Tuple[Tuple[int, int], ...]   # (h, w) latent grids in sequence order
    mode: str                             # "f32" | "bf16" | "w8a8"
    seed: int
    n_blocks: int = 1
    outliers: bool = False
    steps: int = 1                        # >1: prefix K/V reused across steps

    @property
    def seg_len(self) -> List[int]:
        return [self.text] + [h * w for h, w in self.images]

    @property
    def T(self) -> int:
        return sum(self.seg_len)

    @property
    def prefix_len(self) -> int:
        """Rows before the last (target) segment."""
        return self.T - self.seg_len[-1]


WORKLOADS = [
    Workload(0, "tiny_fp32", 512, 4, 2048, 16, ((8, 8),), "f32", 0),
    Workload(1, "block_bf16_256px", 4096, 32, 16384, 64, ((16, 16),), "bf16", 1),
    Workload(2, "block_w8a8_512px", 4096, 32, 16384, 128, ((32, 32),), "w8a8", 2, outliers=True),
    Workload(3, "stack_w8a8_1024px", 4096, 32, 16384, 256, ((64, 64),), "w8a8", 3, n_blocks=32),
    Workload(4, "edit_w8a8_2048px", 4096, 32, 16384, 256, ((32, 32), (128, 128)), "w8a8", 4, steps=2),
]


def workload(idx_or_name) -> Workload:
    for w in WORKLOADS:
        if w.idx == idx_or_name or w.name == idx_or_name:
            return w
    raise KeyError(idx_or_name)


def custom(name: str, D: int, H: int, F: int, text: int, images, mode: str, seed: int, **kw) -> Workload:
    """A workload with the same recipe at another size (used for small parity cases)."""
    return Workload(-1, name, D, H, F, text, tuple(tuple(g) for g in images), mode, seed, **kw)


# --------------------------------------------------------------------------- helpers

def to_bf16_grid(a: np.ndarray) -> np.ndarray:
    """Store fp32 draws on the bf16 grid (nearest, ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that already lie on the bf16 grid."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _streams(w: Workload, n: int) -> List[np.random.Generator]:
    return [np.random.default_rng(s) for s in np.random.SeedSequence(w.seed).spawn(n)]


def _normal(rng, shape, std=1.0) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _store(w: Workload, a: np.ndarray) -> np.ndarray:
    return a if w.mode == "f32" else to_bf16_grid(a)


# Stream layout of one workload's SeedSequence: 0 activations, 1 modulation,
# 2 DiT head/tail, 3.. one stream per block.
_S_ACT, _S_MOD, _S_HEAD, _S_BLOCK0 = 0, 1, 2, 3


def block_weights(w: Workload, block: int = 0) -> Dict[str, np.ndarray]:
    """Weights of block ``block``: fp32 arrays ([N, K] row-major, K contiguous).

    bf16 workload: every tensor on the bf16 grid.  W8A8 workloads: the four
    linear matrices are fp32 masters; biases and gains on the bf16 grid.
    """
    rng = _streams(w, _S_BLOCK0 + w.n_blocks)[_S_BLOCK0 + block]
    D, F = w.D, w.F
    out = {}
    for name, shape in (("w_qkv", (3 * D, D)), ("b_qkv", (3 * D,)), ("g_q", (HEAD_DIM,)),
                        ("g_k", (HEAD_DIM,)), ("w_o", (D, D)), ("b_o", (D,)),
                        ("w_1", (F, D)), ("b_1", (F,)), ("w_2", (D, F)), ("b_2", (D,))):
        a = _normal(rng, shape, 0.02)
        if name.startswith("g_"):
            a = (a + np.float32(1.0)).astype(np.float32)
        if w.outliers and name.startswith("w_"):
            n_out = int(0.001 * a.size)
            idx = rng.choice(a.size, size=n_out, replace=False)
            a.reshape(-1)[idx] *= np.float32(8.0)
        if w.mode == "bf16" or (w.mode == "w8a8" and not name.startswith("w_")):
            a = to_bf16_grid(a)
        out[name] = a
    return out


def gated_block_weights(w: Workload, block: int = 0) -> Dict[str, np.ndarray]:
    """Weights of block ``block`` of the gated-MLP form: w_qk [2D, D], w_v [D, D],
    w_o [D, D], w_proj [F, D], w_gate [F, D], w_down [D, F] and biases, N(0, 0.02),
    gains g_q, g_k 1 + N(0, 0.02); every tensor on the bf16 grid (linears that
    run W8A8 are quantized from these values at load time by each side)."""
    rng = _streams(w, _S_BLOCK0 + w.n_blocks)[_S_BLOCK0 + block]
    D, F = w.D, w.F
    out = {}
    for name, shape in (("w_qk", (2 * D, D)), ("b_qk", (2 * D,)), ("w_v", (D, D)), ("b_v", (D,)),
                        ("g_q", (HEAD_DIM,)), ("g_k", (HEAD_DIM,)), ("w_o", (D, D)), ("b_o", (D,)),
                        ("w_proj", (F, D)), ("b_proj", (F,)), ("w_gate", (F, D)), ("b_gate", (F,)),
                        ("w_down", (D, F)), ("b_down", (D,))):
        a = _normal(rng, shape, 0.02)
        if name.startswith("g_"):
            a = (a + np.float32(1.0)).astype(np.float32)
        out[name] = to_bf16_grid(a)
    return out


def mxfp4_weights(N: int, K: int, seed: int, scale_exp: int = 121):
    """A synthetic MXFP4 checkpoint matrix [N, K]: uniform random 4-bit E2M1 codes
    packed two per byte ([N, K/2] uint8) and E8M0 group scales ([N, K/32] uint8)
    drawn around 2^(scale_exp - 127) (x2^-1..x2^1), so weights have magnitudes
    near those of the N(0, 0.02) draws.  Codes are drawn directly: no encoder."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = (scale_exp + rng.integers(-1, 2, (N, K // 32))).astype(np.uint8)
    return codes, scales


def _modulation_sets(w: Workload, n_sets: int, rows: int = 6) -> np.ndarray:
    """[n_sets, rows, D] modulation rows, each set from its own timestep embedding."""
    rng = _streams(w, _S_BLOCK0)[_S_MOD]
    D = w.D
    w_mod = _normal(rng, (rows * D, D), 0.02).astype(np.float64)
    b_mod = _normal(rng, (rows * D,), 0.02).astype(np.float64)
    sets = []
    for _ in range(n_sets):
        temb = _normal(rng, (D,), 1.0).astype(np.float64)
        silu = temb / (1.0 + np.exp(-temb))
        sets.append((w_mod @ silu + b_mod).reshape(rows, D))
    return np.stack(sets).astype(np.float32)


def block_inputs(w: Workload, step: int = 0) -> Dict[str, np.ndarray]:
    """Activations of one block call.

    Returns x [T, D] (all rows of the sequence, the step's target rows last),
    mod [n_sets, 6, D] fp32, mod_of_seg [n_seg] int32, seg_len [n_seg] int32.
    With ``w.steps > 1`` the prefix rows (text, reference) and the prefix
    modulation set (set 0) are the same for every step; the target rows and
    the target modulation set (set 1 + step) change per step.
    """
    rngs = _streams(w, _S_BLOCK0)
    rng = rngs[_S_ACT]
    T, D = w.T, w.D
    x_prefix = _normal(rng, (w.prefix_len, D))
    targets = [_normal(rng, (w.seg_len[-1], D)) for _ in range(w.steps)]
    x = _store(w, np.concatenate([x_prefix, targets[step]], axis=0))
    n_seg = len(w.seg_len)
    if w.steps > 1:
        mod = _modulation_sets(w, 1 + w.steps)
        mod_of_seg = np.array([0] * (n_seg - 1) + [1 + step], dtype=np.int32)
    else:
        mod = _modulation_sets(w, 1)
        mod_of_seg = np.zeros(n_seg, dtype=np.int32)
    assert x.shape == (T, D)
    return {"x": x, "mod": mod, "mod_of_seg": mod_of_seg,
            "seg_len": np.array(w.seg_len, dtype=np.int32)}


def step_inputs(w: Workload) -> Dict[str, np.ndarray]:
    """Inputs around the block stack of one denoise step (DiT head and tail).

    latent [N, 64] fp32 (the sampler's packed latent), txt_feats [L, D] (text
    encoder features, bf16 grid), img_in Linear(64 -> D), txt_in Linear(D -> D),
    final modulation [1, 2, D] (shift, scale), proj_out Linear(D -> 64), and the
    two sigmas of the Euler update.
    """
    rng = _streams(w, _S_BLOCK0)[_S_HEAD]
    D, L = w.D, w.text
    N = w.seg_len[-1]
    out = {
        "latent": _normal(rng, (N, 64)),
        "txt_feats": _store(w, _normal(rng, (L, D))),
        "w_img_in": _store(w, _normal(rng, (D, 64), 0.02)),
        "b_img_in": _store(w, _normal(rng, (D,), 0.02)),
        "w_txt_in": _store(w, _normal(rng, (D, D), 0.02)),
        "b_txt_in": _store(w, _normal(rng, (D,), 0.02)),
        "w_proj_out": _store(w, _normal(rng, (64, D), 0.02)),
        "b_proj_out": _store(w, _normal(rng, (64,), 0.02)),
    }
    w_mod = _normal(rng, (2 * D, D), 0.02).astype(np.float64)
    b_mod = _normal(rng, (2 * D,), 0.02).astype(np.float64)
    temb = _normal(rng, (D,), 1.0).astype(np.float64)
    silu = temb / (1.0 + np.exp(-temb))
    out["mod_final"] = (w_mod @ silu + b_mod).reshape(1, 2, D).astype(np.float32)
    out["sigma"] = np.float32(1.0)
    out["sigma_next"] = np.float32(1.0 - 0.98 / 39.0)
    return out


def loop_sigmas(steps: int, total: int = 40) -> np.ndarray:
    """Sigmas of the first ``steps`` Euler steps of a ``total``-step loop: the
    linear schedule 1 -> 0.02 over ``total`` values, then 0 (fp32 values, so
    both sides take the same numbers)."""
    sched = [1.0 - 0.98 * i / (total - 1) for i in range(total)] + [0.0]
    return np.asarray(sched[:steps + 1], dtype=np.float32)


def loop_inputs(w: Workload, steps: int) -> Dict[str, np.ndarray]:
    """Inputs of a ``steps``-step denoise loop: step_inputs (target latent, text
    features, head/tail weights) plus reference latents [R, 64] for every image
    segment but the last (editing), the modulation of each step mods
    [S, n_mod, 6, D] with mod_of_seg, the tail modulation of each step
    mod_finals [S, 2, D], and sigmas [S + 1].

    One image segment (text-to-image): one modulation set per step for every
    token, from that step's timestep embedding.  Several (editing): set 0 is the
    prefix set (text and references, the same at every step), set 1 the
    target's set of the step (the same sets as block_inputs(w, step))."""
    si = step_inputs(w)
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 2000]))
    D = w.D
    R = int(sum(h * ww for h, ww in w.images[:-1]))
    edit = len(w.images) > 1
    out = dict(si)
    out["ref_latent"] = _normal(rng, (R, 64)) if R else np.zeros((0, 64), np.float32)
    if edit:
        sets = _modulation_sets(w, 1 + steps)
        out["mods"] = np.stack([sets[[0, 1 + i]] for i in range(steps)])
        out["mod_of_seg"] = np.asarray([0] * (len(w.seg_len) - 1) + [1], np.int32)
    else:
        out["mods"] = _modulation_sets(w, steps)[:, None]
        out["mod_of_seg"] = np.zeros(len(w.seg_len), np.int32)
    w_mf = _normal(rng, (2 * D, D), 0.02).astype(np.float64)
    b_mf = _normal(rng, (2 * D,), 0.02).astype(np.float64)
    finals = []
    for _ in range(steps):
        temb = _normal(rng, (D,), 1.0).astype(np.float64)
        finals.append((w_mf @ (temb / (1.0 + np.exp(-temb))) + b_mf).reshape(2, D))
    out["mod_finals"] = np.stack(finals).astype(np.float32)
    out["sigmas"] = loop_sigmas(steps)
    out["seg_len"] = np.asarray(w.seg_len, np.int32)
    return out


def attention_inputs(T_q: int, T_k: int, H: int, seed: int, bf16: bool = True):
    """q [T_q,H,128], k/v [T_k,H,128] N(0,1) draws for attention-only cases."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (T_q, H, HEAD_DIM))
    k = _normal(rng, (T_k, H, HEAD_DIM))
    v = _normal(rng, (T_k, H, HEAD_DIM))
    if bf16:
        q, k, v = to_bf16_grid(q), to_bf16_grid(k), to_bf16_grid(v)
    return q, k, v


def int8_operands(M: int, N: int, K: int, seed: int):
    """Uniform int8 codes in [-127, 127] with fp32 scales, for GEMM-only cases."""
    rng = np.random.default_rng(seed)
    a = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    b = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    sa = (rng.random(M, dtype=np.float32) * np.float32(0.02) + np.float32(0.001)).astype(np.float32)
    sb = (rng.random(N, dtype=np.float32) * np.float32(0.002) + np.float32(1e-4)).astype(np.float32)
    bias = to_bf16_grid(_normal(rng, (N,), 0.02))
    return a, b, sa, sb, bias


def rows(M: int, K: int, seed: int, scale: float = 1.0, bf16: bool = True, zero_rows=()):
    """[M, K] N(0, scale) rows (optionally some rows all zero) for quantizer cases."""
    rng = np.random.default_rng(seed)
    a = _normal(rng, (M, K), scale)
    for r in zero_rows:
        a[r] = 0.0
    return to_bf16_grid(a) if bf16 else a


# --------------------------------------------------------------------------- device-side draws
# The same distributions drawn with torch's device generator, for workloads too
# large to draw on the host (the 32-block stack).  Different random numbers
# than the host draws, same recipe.

def _torch():
    import torch
    return torch


def device_normal(shape, std, gen, device="cuda", bf16_grid=False):
    torch = _torch()
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std
    if bf16_grid:
        t = t.to(torch.bfloat16).to(torch.float32)
    return t


def device_generator(w: Workload, stream: int, device="cuda"):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([w.seed, stream]).generate_state(1)[0]))
    return g


def device_gated_block_weights(w: Workload, block: int, F: int, device="cuda"):
    """Device draws of gated_block_weights (width F), every tensor on the bf16 grid."""
    g = device_generator(w, 2000 + block, device)
    D = w.D
    out = {}
    for name, shape in (("w_qk", (2 * D, D)), ("b_qk", (2 * D,)), ("w_v", (D, D)), ("b_v", (D,)),
                        ("g_q", (HEAD_DIM,)), ("g_k", (HEAD_DIM,)), ("w_o", (D, D)), ("b_o", (D,)),
                        ("w_proj", (F, D)), ("b_proj", (F,)), ("w_gate", (F, D)), ("b_gate", (F,)),
                        ("w_down", (D, F)), ("b_down", (D,))):
        t = device_normal(shape, 0.02, g, device)
        if name.startswith("g_"):
            t = t + 1.0
        out[name] = t.to(_torch().bfloat16).to(_torch().float32)
    return out


def device_block_weights(w: Workload, block: int, device="cuda"):
    """Yields (name, fp32 device tensor) for one block, masters first (see block_weights)."""
    g = device_generator(w, 1000 + block, device)
    D, F = w.D, w.F
    for name, shape in (("w_qkv", (3 * D, D)), ("b_qkv", (3 * D,)), ("g_q", (HEAD_DIM,)),
                        ("g_k", (HEAD_DIM,)), ("w_o", (D, D)), ("b_o", (D,)),
                        ("w_1", (F, D)), ("b_1", (F,)), ("w_2", (D, F)), ("b_2", (D,))):
        is_w = name.startswith("w_")
        t = device_normal(shape, 0.02, g, device, bf16_grid=(w.mode == "bf16" or not is_w))
        if name.startswith("g_"):
            t = (t + 1.0).to(_torch().bfloat16).to(_torch().float32)
        yield name, t


def device_step_inputs(w: Workload, device="cuda"):
    """Device versions of block_inputs (step 0) and step_inputs."""
    torch = _torch()
    g = device_generator(w, 1, device)
    D, L, N = w.D, w.text, w.seg_len[-1]
    out = {
        "latent": device_normal((N, 64), 1.0, g, device),
        "txt_feats": device_normal((L, D), 1.0, g, device, True),
        "w_img_in": device_normal((D, 64), 0.02, g, device, True),
        "b_img_in": device_normal((D,), 0.02, g, device, True),
        "w_txt_in": device_normal((D, D), 0.02, g, device, True),
        "b_txt_in": device_normal((D,), 0.02, g, device, True),
        "w_proj_out": device_normal((64, D), 0.02, g, device, True),
        "b_proj_out": device_normal((64,), 0.02, g, device, True),
    }
    for name, rows, n_sets in (("mod", 6, 1 + (w.steps if w.steps > 1 else 0)), ("mod_final", 2, 1)):
        w_mod = device_normal((rows * D, D), 0.02, g, device)
        b_mod = device_normal((rows * D,), 0.02, g, device)
        sets = []
        for _ in range(max(n_sets, 1)):
            temb = device_normal((D,), 1.0, g, device)
            silu = temb / (1.0 + torch.exp(-temb))
            sets.append((w_mod @ silu + b_mod).reshape(rows, D))
        out[name] = torch.stack(sets).contiguous()
        del w_mod
    out["x_target"] = [device_normal((N, D), 1.0, g, device, True) for _ in range(w.steps)]
    out["x_prefix"] = device_normal((w.prefix_len, D), 1.0, g, device, True)
    return out


def device_loop_inputs(w: Workload, steps: int, device="cuda"):
    """Device modulation of a ``steps``-step loop (the loop_inputs layout, drawn
    with the device generator): mods [S, n_mod, 6, D], mod_finals [S, 2, D],
    mod_of_seg, sigmas (host floats)."""
    torch = _torch()
    g = device_generator(w, 2000, device)
    D = w.D
    edit = len(w.images) > 1
    out = {}
    for name, rows, n_sets in (("mods", 6, steps + (1 if edit else 0)), ("mod_finals", 2, steps)):
        w_mod = device_normal((rows * D, D), 0.02, g, device)
        b_mod = device_normal((rows * D,), 0.02, g, device)
        sets = []
        for _ in range(n_sets):
            temb = device_normal((D,), 1.0, g, device)
            sets.append((w_mod @ (temb / (1.0 + torch.exp(-temb))) + b_mod).reshape(rows, D))
        out[name] = torch.stack(sets).contiguous()
        del w_mod
    if edit:
        out["mods"] = torch.stack([out["mods"][[0, 1 + i]] for i in range(steps)]).contiguous()
        out["mod_of_seg"] = [0] * (len(w.seg_len) - 1) + [1]
    else:
        out["mods"] = out["mods"][:, None].contiguous()
        out["mod_of_seg"] = [0] * len(w.seg_len)
    out["sigmas"] = [float(v) for v in loop_sigmas(steps)]
    return out
