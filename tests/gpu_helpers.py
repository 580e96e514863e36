"""Shared helpers of the GPU parity tests: device upload and comparisons.

Inputs come from ``ditsynth``; expected values only from ``oracle``.
"""
import sys

import numpy as np
import torch

import ditsynth
import diffusion_transformer_text_qwen_amd as dq

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=torch.float32):
    return torch.as_tensor(np.ascontiguousarray(a)).to(DEV).to(dtype).contiguous()


def act_dtype(mode):
    return torch.float32 if mode == "f32" else torch.bfloat16


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.int8 else t.cpu().numpy()


def bf16_ulp(ref):
    """Spacing of bf16 at |ref| (2^(e-7)); the smallest normal spacing for zeros."""
    a = np.abs(np.asarray(ref, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


class GpuBlock:
    """One block of a workload on the GPU: weights, caches, workspace, RoPE tables."""

    def __init__(self, w, weights=None, block=0, attn_quant=False):
        self.w = w
        self.mode = w.mode
        arrays = weights if weights is not None else ditsynth.block_weights(w, block)
        self.weights = dq.BlockWeights(arrays, w.mode)
        self.cfg = dq.block_config(w.mode, w.D, w.H, w.F, attn_quant=attn_quant)
        T = w.T
        self.cos = torch.empty((T, 64), dtype=torch.float32, device=DEV)
        self.sin = torch.empty((T, 64), dtype=torch.float32, device=DEV)
        dq.rope_tables(w.text, w.images, 0, T, self.cos, self.sin)
        self.k = torch.zeros((T, w.H, 128), dtype=act_dtype(w.mode), device=DEV)
        self.v = torch.zeros((T, w.H, 128), dtype=act_dtype(w.mode), device=DEV)
        self.ws = torch.empty(dq.workspace_bytes(self.cfg, T, T), dtype=torch.uint8, device=DEV)

    def run(self, x_np, mod, mod_of_seg, T_q=None):
        """Run on the last T_q rows of the sequence (x_np holds exactly those rows)."""
        w = self.w
        T_q = x_np.shape[0] if T_q is None else T_q
        x = dev(x_np, act_dtype(self.mode))
        r0 = w.T - T_q
        dq.block_forward(self.cfg, self.weights, x, dev(mod), mod_of_seg, self.cos[r0:], self.sin[r0:],
                         w.seg_len, self.k, self.v, self.ws)
        torch.cuda.synchronize()
        return x
