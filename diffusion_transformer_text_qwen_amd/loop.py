"""Denoise loop over dit_velocity_forward: per step the DiT maps the target latent
(with the text features, and for editing the reference latents) to a velocity,
then one Euler update moves the latent from sigma_i to sigma_{i+1} ("RGBA-Image-2.1 -
Core AI port of Qwen-Image-2.1", Graph contracts).

Step 0 computes every row of [text | references | target] and fills the per-block
K/V caches.  With ``cache_prefix`` the later steps compute only the target rows
and attend to the cached prefix K/V ("Qwen_Image-2.1-MXFP4-Paiton", prefix reuse;
valid when the prefix rows use a modulation set that does not change between
steps).  With ``graph`` one velocity evaluation of the repeated shape is captured
in a HIP graph (torch.cuda.CUDAGraph on the library's stream) and replayed; the
step's modulation is copied into the captured buffers before each replay and the
Euler update, whose sigmas change per step, runs after it.  With
``quant_attn_from`` the steps from that index on run the attention on int8/fp8
operands ("Qwen_Image-2.1-MXFP4-Paiton", Runtime precision and quality: the
first steps keep the original precision).
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import (BlockConfig, BlockWeights, HeadWeights, euler_step, velocity_forward,
               velocity_workspace_bytes, MODES)


class DenoiseLoop:
    """Buffers of one loop: per-block K/V caches, workspace, velocity and the
    modulation buffers the captured step reads.

    cfg/blocks: the block stack; head: HeadWeights; seg_len: [text, refs..., target]
    lengths (text may be 0); mod_of_seg: modulation set of each segment;
    cos/sin: [T_k, 64] RoPE tables of all rows; n_mod: modulation sets per step.
    """

    def __init__(self, cfg: BlockConfig, blocks: Sequence[BlockWeights], head: HeadWeights,
                 seg_len: Sequence[int], mod_of_seg: Sequence[int], L_txt: int, cos: torch.Tensor,
                 sin: torch.Tensor, n_mod: int, device="cuda"):
        self.cfg = BlockConfig(cfg.mode, cfg.D, cfg.H, cfg.head_dim, cfg.F, cfg.ln_eps, cfg.qk_eps, cfg.attn_quant)
        self.blocks, self.head = list(blocks), head
        self.seg_len = [int(v) for v in seg_len]
        self.mod_of_seg = [int(v) for v in mod_of_seg]
        self.T_k = sum(self.seg_len)
        self.L = int(L_txt)
        self.N = self.seg_len[-1]
        self.R = self.T_k - self.L - self.N
        self.cos, self.sin = cos, sin
        act = torch.float32 if cfg.mode == 0 else torch.bfloat16
        C = head.t["w_img_in"].shape[1]
        self.k_caches = [torch.empty((self.T_k, cfg.H, 128), dtype=act, device=device) for _ in self.blocks]
        self.v_caches = [torch.empty((self.T_k, cfg.H, 128), dtype=act, device=device) for _ in self.blocks]
        # sized for the int8/fp8 attention buffers too (bf16 and W8A8 modes)
        sizing = BlockConfig(cfg.mode, cfg.D, cfg.H, cfg.head_dim, cfg.F, cfg.ln_eps, cfg.qk_eps,
                             int(cfg.mode != MODES["f32"]))
        self.ws = torch.empty(velocity_workspace_bytes(sizing, self.T_k, self.N, C), dtype=torch.uint8, device=device)
        self.vel = torch.empty((self.N, C), dtype=act, device=device)
        self.mod = torch.empty((n_mod, 6, cfg.D), dtype=torch.float32, device=device)
        self.mod_final = torch.empty((2, cfg.D), dtype=torch.float32, device=device)
        self.graph: Optional[torch.cuda.CUDAGraph] = None

    def velocity(self, latent, txt_feats=None, ref_latent=None, cached: bool = False, quant: bool = False) -> None:
        """self.vel from the current contents of latent, self.mod, self.mod_final;
        quant: int8/fp8 attention."""
        self.cfg.attn_quant = int(quant)
        T_q = self.N if cached else self.T_k
        r0 = self.T_k - T_q
        velocity_forward(self.cfg, self.blocks, self.head, latent, self.vel, self.mod, self.mod_of_seg,
                         self.mod_final, self.cos[r0:], self.sin[r0:], self.seg_len, self.k_caches,
                         self.v_caches, self.ws, txt_feats=txt_feats, ref_latent=ref_latent, L_txt=self.L,
                         R=self.R, T_q=T_q)

    def run(self, latent: torch.Tensor, txt_feats, ref_latent, mods, mod_finals, sigmas: Sequence[float],
            cache_prefix: bool = False, graph: bool = False, on_step=None,
            quant_attn_from: Optional[int] = None) -> torch.Tensor:
        """Runs len(sigmas) - 1 steps on latent [N, C] (fp32, updated in place).

        mods [S, n_mod, 6, D] and mod_finals [S, 2, D] are device tensors; on_step(i)
        is called after step i's Euler update (tests use it to inspect each step);
        steps i >= quant_attn_from (if given) use the int8/fp8 attention."""
        sig = [float(v) for v in sigmas]
        captured = None
        seen = set()
        for i in range(len(sig) - 1):
            self.mod.copy_(mods[i])
            self.mod_final.copy_(mod_finals[i])
            cached = cache_prefix and i > 0
            quant = quant_attn_from is not None and i >= quant_attn_from
            key = (cached, quant)
            # the first call of each variant runs eagerly (it also sets the kernels' attributes)
            if graph and key in seen:
                if self.graph is None or captured != key:
                    self.graph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(self.graph):
                        self.velocity(latent, txt_feats, ref_latent, cached, quant)
                    captured = key
                self.graph.replay()
            else:
                self.velocity(latent, txt_feats, ref_latent, cached, quant)
                seen.add(key)
            euler_step(latent, self.vel, sig[i], sig[i + 1])
            if on_step is not None:
                on_step(i)
        return latent
