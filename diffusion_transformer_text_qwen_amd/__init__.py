"""Python binding of the gfx950 single-stream DiT block library (libditblock.so).

Argument marshalling only: every function passes torch tensor addresses and
the current HIP stream to the C ABI declared in ``include/dit.h``; all
arithmetic runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libditblock.so")

F32, BF16, I8, I32 = 0, 1, 2, 3
MODE_F32, MODE_BF16, MODE_W8A8 = 0, 1, 2
MODES = {"f32": MODE_F32, "bf16": MODE_BF16, "w8a8": MODE_W8A8}

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_fp = ctypes.c_float


class DitError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name} failed with status {status}: {detail}")
        self.status = status


class BlockConfig(ctypes.Structure):
    _fields_ = [("mode", _c_i32), ("D", _c_i32), ("H", _c_i32), ("head_dim", _c_i32), ("F", _c_i32),
                ("ln_eps", _fp), ("qk_eps", _fp), ("attn_quant", _c_i32)]


class BlockWeightsC(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_qkv", "w_o", "w_1", "w_2", "s_qkv", "s_o", "s_1", "s_2",
                                   "b_qkv", "b_o", "b_1", "b_2", "g_q", "g_k")]


class LinearC(ctypes.Structure):
    _fields_ = [("w", _vp), ("s", _vp), ("wsum", _vp), ("b", _vp), ("mx_scale", _vp)]


class GatedBlockWeightsC(ctypes.Structure):
    _fields_ = [(n, LinearC) for n in ("qk", "v", "o", "proj", "gate", "down")] + [("g_q", _vp), ("g_k", _vp)]


class BlockIO(ctypes.Structure):
    _fields_ = [("x", _vp), ("mod", _vp), ("n_mod", _c_i32), ("mod_of_seg", _vp), ("cos_t", _vp),
                ("sin_t", _vp), ("seg_len", _vp), ("n_seg", _c_i32), ("T_q", _c_i64), ("T_k", _c_i64),
                ("k_cache", _vp), ("v_cache", _vp)]


class HeadWeightsC(ctypes.Structure):
    _fields_ = [("w_txt_in", _vp), ("b_txt_in", _vp), ("w_img_in", _vp), ("b_img_in", _vp),
                ("w_proj_out", _vp), ("b_proj_out", _vp), ("C_txt", _c_i32), ("C_lat", _c_i32)]


class VelocityIO(ctypes.Structure):
    _fields_ = [("txt_feats", _vp), ("ref_latent", _vp), ("latent", _vp), ("L_txt", _c_i64), ("R", _c_i64),
                ("N", _c_i64), ("mod", _vp), ("n_mod", _c_i32), ("mod_of_seg", _vp), ("mod_final", _vp),
                ("cos_t", _vp), ("sin_t", _vp), ("seg_len", _vp), ("n_seg", _c_i32), ("T_q", _c_i64),
                ("k_caches", _vp), ("v_caches", _vp), ("vel", _vp)]


_SIGS = {
    "dit_abi_version": ([], ctypes.c_int),
    "dit_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "dit_last_error": ([], ctypes.c_char_p),
    "dit_quantize_rows": ([_vp, ctypes.c_int, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp], ctypes.c_int),
    "dit_gelu_quantize_rows": ([_vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _vp], ctypes.c_int),
    "dit_qkv_linear_workspace_bytes": ([_c_i64, _c_i32], ctypes.c_size_t),
    "dit_qkv_linear": ([ctypes.c_int, _vp, _vp, _c_i64, _c_i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _fp, _vp, _vp,
                        _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "w8a8_linear_workspace_bytes": ([], ctypes.c_size_t),
    "w8a8_linear": ([_vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp, _c_i64, _vp, ctypes.c_int, _c_i64, _vp, _vp,
                     ctypes.c_size_t, _vp], ctypes.c_int),
    "w8a8_linear_noalloc": ([_vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp, _c_i64, _vp, ctypes.c_int, _c_i64, _vp,
                             _vp], ctypes.c_int),
    "bf16_linear": ([_vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_i64, _vp, ctypes.c_int, _c_i64, _vp],
                    ctypes.c_int),
    "f32_linear": ([_vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_i64, _vp, _c_i64, _vp], ctypes.c_int),
    "block_causal_attention": ([_vp, _vp, _vp, _vp, ctypes.c_int, _c_i64, _c_i64, _c_i32, _c_i32, _c_i64,
                                _c_i64, _c_i64, _c_i64, _vp, _c_i32, _fp, _vp], ctypes.c_int),
    "dit_quantize_rows_asym": ([_vp, ctypes.c_int, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _vp], ctypes.c_int),
    "dit_int8_colsum": ([_vp, _c_i64, _c_i64, _vp, _vp], ctypes.c_int),
    "w8a8_linear_asym": ([_vp, _vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _c_i64, _vp, ctypes.c_int, _c_i64,
                          _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "dit_mxfp4_expand": ([_vp, _vp, _c_i64, _c_i64, _vp, _vp], ctypes.c_int),
    "mxfp4_linear_workspace_bytes": ([_c_i64, _c_i64], ctypes.c_size_t),
    "mxfp4_linear": ([_vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _c_i64, _vp, ctypes.c_int, _c_i64, _vp,
                      ctypes.c_size_t, _vp], ctypes.c_int),
    "dit_gated_block_workspace_bytes": ([ctypes.POINTER(BlockConfig), _c_i64, _c_i64], ctypes.c_size_t),
    "dit_block_forward_gated": ([ctypes.POINTER(BlockConfig), ctypes.POINTER(GatedBlockWeightsC),
                                 ctypes.POINTER(BlockIO), _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "dit_attn_q8_bytes": ([_c_i64, _c_i64, _c_i32, _vp], ctypes.c_size_t),
    "dit_attn_quantize": ([_vp, _vp, _vp, _c_i64, _c_i64, _c_i32, _c_i64, _c_i64, _c_i64, _vp, ctypes.c_size_t,
                           _vp], ctypes.c_int),
    "block_causal_attention_q8": ([_vp, _c_i64, _c_i64, _c_i32, _vp, _c_i64, _vp, _c_i32, _fp, _vp], ctypes.c_int),
    "dit_rope_tables": ([_c_i32, _vp, _c_i32, _c_i64, _c_i64, _fp, _vp, _vp, _vp], ctypes.c_int),
    "dit_qk_norm_rope": ([_vp, ctypes.c_int, _c_i64, _c_i32, _vp, _vp, _vp, _vp, _fp, _vp, _vp, _c_i64, _vp,
                          _c_i64, _vp], ctypes.c_int),
    "dit_adaln_modulate": ([_vp, ctypes.c_int, _c_i64, _c_i64, _vp, _vp, _fp, _vp, ctypes.c_int, _vp, _vp,
                            _vp], ctypes.c_int),
    "dit_adaln_modulate_asym": ([_vp, _c_i64, _c_i64, _vp, _vp, _fp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "dit_euler_step": ([_vp, _vp, ctypes.c_int, _c_i64, _fp, _fp, _vp], ctypes.c_int),
    "dit_cast": ([_vp, ctypes.c_int, _vp, ctypes.c_int, _c_i64, _vp], ctypes.c_int),
    "dit_profile_begin": ([_c_i32], ctypes.c_int),
    "dit_profile_end": ([_vp, _vp, _c_i32], ctypes.c_int),
    "dit_site_name": ([_c_i32], ctypes.c_char_p),
    "dit_block_workspace_bytes": ([ctypes.POINTER(BlockConfig), _c_i64, _c_i64], ctypes.c_size_t),
    "dit_block_forward": ([ctypes.POINTER(BlockConfig), ctypes.POINTER(BlockWeightsC), ctypes.POINTER(BlockIO),
                           _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "dit_stack_forward": ([ctypes.POINTER(BlockConfig), ctypes.POINTER(BlockWeightsC), _c_i32,
                           ctypes.POINTER(BlockIO), _vp, _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "dit_velocity_workspace_bytes": ([ctypes.POINTER(BlockConfig), _c_i64, _c_i64, _c_i64, _c_i32],
                                     ctypes.c_size_t),
    "dit_velocity_forward": ([ctypes.POINTER(BlockConfig), ctypes.POINTER(BlockWeightsC), _c_i32,
                              ctypes.POINTER(HeadWeightsC), ctypes.POINTER(VelocityIO), _vp, ctypes.c_size_t,
                              _vp], ctypes.c_int),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libditblock.so (built by ``build.py``); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run diffusion_transformer_text_qwen_amd/build.py")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(l, name)
            f.argtypes = args
            f.restype = res
        _lib = l
    return _lib


def exported_symbols() -> List[str]:
    return list(_SIGS)


def _check(status: int, name: str) -> None:
    if status != 0:
        raise DitError(status, name, lib().dit_last_error().decode())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dt(t: torch.Tensor) -> int:
    return {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8, torch.int32: I32}[t.dtype]


def _host_i32(seq) -> ctypes.Array:
    arr = (ctypes.c_int32 * len(seq))(*[int(v) for v in seq])
    return arr


# ---------------------------------------------------------------- op-level calls

def quantize_rows(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, stream=None) -> None:
    M, K = x.shape
    _check(lib().dit_quantize_rows(_p(x), _dt(x), M, K, x.stride(0), _p(q), _p(scale), _stream(stream)),
           "dit_quantize_rows")


def gelu_quantize_rows(u, q, scale, g_out=None, stream=None) -> None:
    """Codes of g = bf16(GELU_tanh(u)) per row (u bf16 [M, K]); g_out receives g if given."""
    M, K = u.shape
    _check(lib().dit_gelu_quantize_rows(_p(u), M, K, u.stride(0), _p(q), _p(scale), _p(g_out), _stream(stream)),
           "dit_gelu_quantize_rows")


def qkv_linear_workspace_bytes(T: int, H: int) -> int:
    return int(lib().dit_qkv_linear_workspace_bytes(T, H))


def qkv_linear(a, w, bias, g_q, g_k, cos_t, sin_t, q_out, k_out, v_out, workspace, a_scale=None, w_scale=None,
               eps: float = 1e-6, stream=None) -> None:
    """The block's QKV linear with the fused Q/K RMSNorm + RoPE epilogue: a [T, D]
    int8 codes (with a_scale, w int8 + w_scale) or bf16; q/k/v_out bf16 [T, D]."""
    T, D = a.shape
    mode = MODE_W8A8 if a.dtype == torch.int8 else MODE_BF16
    _check(lib().dit_qkv_linear(mode, _p(a), _p(a_scale), T, D // 128, _p(w), _p(w_scale), _p(bias), _p(g_q),
                                _p(g_k), _p(cos_t), _p(sin_t), eps, _p(q_out), _p(k_out), _p(v_out),
                                _p(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "dit_qkv_linear")


def quantize_rows_asym(x, q, scale, zero, stream=None) -> None:
    """Asymmetric per-row int8 codes of x [M, K] (bf16/f32): q int8, scale f32 [M], zero int32 [M]."""
    M, K = x.shape
    _check(lib().dit_quantize_rows_asym(_p(x), _dt(x), M, K, x.stride(0), _p(q), _p(scale), _p(zero),
                                        _stream(stream)), "dit_quantize_rows_asym")


def int8_colsum(w, out, stream=None) -> None:
    """out[n] = sum_k w[n, k] (int8 [N, K] -> int32 [N])."""
    N, K = w.shape
    _check(lib().dit_int8_colsum(_p(w), N, K, _p(out), _stream(stream)), "dit_int8_colsum")


def w8a8_linear_asym(a, a_scale, a_zero, w, w_scale, w_sum, bias, y, workspace=None, stream=None) -> None:
    M, K = a.shape
    N = w.shape[0]
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().w8a8_linear_asym(_p(a), _p(a_scale), _p(a_zero), M, K, _p(w), _p(w_scale), _p(w_sum), _p(bias), N,
                                  _p(y), _dt(y), y.stride(0), _p(workspace), wsb, _stream(stream)),
           "w8a8_linear_asym")


def mxfp4_expand(codes, scales, w_bf16, stream=None) -> None:
    """MXFP4 codes [N, K/2] uint8 + E8M0 scales [N, K/32] uint8 -> w_bf16 [N, K]."""
    N, K = w_bf16.shape
    _check(lib().dit_mxfp4_expand(_p(codes), _p(scales), N, K, _p(w_bf16), _stream(stream)), "dit_mxfp4_expand")


def mxfp4_linear(a, codes, scales, bias, y, workspace, stream=None) -> None:
    M, K = a.shape
    N = codes.shape[0]
    _check(lib().mxfp4_linear(_p(a), M, K, a.stride(0), _p(codes), _p(scales), _p(bias), N, _p(y), _dt(y),
                              y.stride(0), _p(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)), "mxfp4_linear")


def w8a8_linear_workspace_bytes() -> int:
    return int(lib().w8a8_linear_workspace_bytes())


def w8a8_linear(a, a_scale, w, w_scale, bias, y, acc_out=None, workspace=None, stream=None) -> None:
    M, K = a.shape
    N = w.shape[0]
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().w8a8_linear(_p(a), _p(a_scale), M, K, _p(w), _p(w_scale), _p(bias), N, _p(y), _dt(y),
                             y.stride(0), _p(acc_out), _p(workspace), wsb, _stream(stream)), "w8a8_linear")


def w8a8_linear_noalloc(a, a_scale, w, w_scale, bias, y, acc_out=None, stream=None) -> None:
    """w8a8_linear with the K-split partials in the library's static device scratch."""
    M, K = a.shape
    N = w.shape[0]
    _check(lib().w8a8_linear_noalloc(_p(a), _p(a_scale), M, K, _p(w), _p(w_scale), _p(bias), N, _p(y), _dt(y),
                                     y.stride(0), _p(acc_out), _stream(stream)), "w8a8_linear_noalloc")


def bf16_linear(a, w, bias, y, stream=None) -> None:
    M, K = a.shape
    N = w.shape[0]
    _check(lib().bf16_linear(_p(a), M, K, a.stride(0), _p(w), _p(bias), N, _p(y), _dt(y), y.stride(0),
                             _stream(stream)), "bf16_linear")


def f32_linear(a, w, bias, y, stream=None) -> None:
    M, K = a.shape
    N = w.shape[0]
    _check(lib().f32_linear(_p(a), M, K, a.stride(0), _p(w), _p(bias), N, _p(y), y.stride(0),
                            _stream(stream)), "f32_linear")


def block_causal_attention(q, k, v, o, seg_len: Sequence[int], sm_scale: float = 0.0, stream=None) -> None:
    """q [T_q, H, 128], k/v [T_k, H, 128], o [T_q, H, 128] (row-contiguous per token)."""
    T_q, H, d = q.shape
    T_k = k.shape[0]
    segs = _host_i32(seg_len)
    _check(lib().block_causal_attention(_p(q), _p(k), _p(v), _p(o), _dt(q), T_q, T_k, H, d, q.stride(0),
                                        k.stride(0), v.stride(0), o.stride(0), ctypes.cast(segs, _vp),
                                        len(seg_len), sm_scale, _stream(stream)), "block_causal_attention")


Q8_PARTS = ("q8", "q_scale", "k8", "k_scale", "v8", "v_scale", "v_amax")


def attn_q8_layout(T_q: int, T_k: int, H: int) -> Tuple[int, Dict[str, int]]:
    """(bytes, {part: byte offset}) of the int8/fp8 attention operand buffer."""
    offs = (ctypes.c_int64 * 7)()
    n = int(lib().dit_attn_q8_bytes(T_q, T_k, H, ctypes.cast(offs, _vp)))
    return n, dict(zip(Q8_PARTS, [int(v) for v in offs]))


def attn_quantize(q, k, v, buf, stream=None) -> None:
    """q [T_q, H, 128], k/v [T_k, H, 128] bf16 -> the operand buffer (uint8 device tensor)."""
    T_q, H, _ = q.shape
    T_k = k.shape[0]
    _check(lib().dit_attn_quantize(_p(q), _p(k), _p(v), T_q, T_k, H, q.stride(0), k.stride(0), v.stride(0),
                                   _p(buf), buf.numel() * buf.element_size(), _stream(stream)), "dit_attn_quantize")


def block_causal_attention_q8(buf, T_q: int, T_k: int, H: int, o, seg_len: Sequence[int], sm_scale: float = 0.0,
                              stream=None) -> None:
    """o [T_q, H, 128] bf16 from an operand buffer filled by attn_quantize."""
    segs = _host_i32(seg_len)
    _check(lib().block_causal_attention_q8(_p(buf), T_q, T_k, H, _p(o), o.stride(0), ctypes.cast(segs, _vp),
                                           len(seg_len), sm_scale, _stream(stream)), "block_causal_attention_q8")


def rope_tables(text_len: int, grids, row0: int, T_rows: int, cos_out, sin_out, theta: float = 10000.0,
                stream=None) -> None:
    flat = [int(v) for g in grids for v in g]
    arr = _host_i32(flat) if flat else None
    _check(lib().dit_rope_tables(text_len, ctypes.cast(arr, _vp) if arr is not None else None, len(grids),
                                 row0, T_rows, theta, _p(cos_out), _p(sin_out), _stream(stream)),
           "dit_rope_tables")


def qk_norm_rope(qkv, g_q, g_k, cos_t, sin_t, q_out, k_out, v_out, eps: float = 1e-6, stream=None) -> None:
    T = qkv.shape[0]
    H = qkv.shape[1] // (3 * 128)
    _check(lib().dit_qk_norm_rope(_p(qkv), _dt(qkv), T, H, _p(g_q), _p(g_k), _p(cos_t), _p(sin_t), eps,
                                  _p(q_out), _p(k_out), k_out.stride(0), _p(v_out), v_out.stride(0),
                                  _stream(stream)), "dit_qk_norm_rope")


def adaln_modulate(x, shift, scale, h_out=None, q_out=None, q_scale=None, eps: float = 1e-6,
                   stream=None) -> None:
    M, D = x.shape
    hdt = _dt(h_out) if h_out is not None else _dt(x)
    _check(lib().dit_adaln_modulate(_p(x), _dt(x), M, D, _p(shift), _p(scale), eps, _p(h_out), hdt,
                                    _p(q_out), _p(q_scale), _stream(stream)), "dit_adaln_modulate")


def adaln_modulate_asym(x, shift, scale, q_out, q_scale, q_zero, h_out=None, eps: float = 1e-6,
                        stream=None) -> None:
    M, D = x.shape
    _check(lib().dit_adaln_modulate_asym(_p(x), M, D, _p(shift), _p(scale), eps, _p(h_out), _p(q_out),
                                         _p(q_scale), _p(q_zero), _stream(stream)), "dit_adaln_modulate_asym")


def euler_step(x, v, sigma: float, sigma_next: float, stream=None) -> None:
    _check(lib().dit_euler_step(_p(x), _p(v), _dt(v), x.numel(), sigma, sigma_next, _stream(stream)),
           "dit_euler_step")


def cast(x, y, stream=None) -> None:
    _check(lib().dit_cast(_p(x), _dt(x), _p(y), _dt(y), x.numel(), _stream(stream)), "dit_cast")


N_SITES = 11


def profile_begin(capacity: int) -> None:
    _check(lib().dit_profile_begin(capacity), "dit_profile_begin")


def profile_end() -> Dict[str, Dict[str, float]]:
    """{site name: {"ms": summed ms, "count": launches}} of the launches recorded since begin."""
    ms = (ctypes.c_double * N_SITES)()
    cnt = (ctypes.c_int64 * N_SITES)()
    _check(lib().dit_profile_end(ctypes.cast(ms, _vp), ctypes.cast(cnt, _vp), N_SITES), "dit_profile_end")
    return {lib().dit_site_name(i).decode(): {"ms": ms[i], "count": cnt[i]} for i in range(N_SITES)}


# ---------------------------------------------------------------- the block

def block_config(mode: str, D: int, H: int, F: int, ln_eps: float = 1e-6, qk_eps: float = 1e-6,
                 attn_quant: bool = False) -> BlockConfig:
    return BlockConfig(MODES[mode], D, H, 128, F, ln_eps, qk_eps, int(bool(attn_quant)))


class BlockWeights:
    """Device-resident weights of one block in the layout the library reads.

    From fp32 host arrays ``w_*`` ([N, K]), ``b_*``, ``g_q``, ``g_k``: in W8A8
    mode the matrices are uploaded as fp32 masters and quantized per output
    channel on the GPU (``dit_quantize_rows``), then the masters are freed.
    """

    def __init__(self, arrays: Dict, mode: str, device="cuda"):
        self.mode = mode
        self.t: Dict[str, torch.Tensor] = {}
        for name in ("w_qkv", "w_o", "w_1", "w_2"):
            a = torch.as_tensor(arrays[name])
            if mode == "w8a8":
                master = a.to(device=device, dtype=torch.float32).contiguous()
                q = torch.empty(master.shape, dtype=torch.int8, device=device)
                s = torch.empty(master.shape[0], dtype=torch.float32, device=device)
                quantize_rows(master, q, s)
                self.t[name] = q
                self.t["s" + name[1:]] = s
                del master
            elif mode == "bf16":
                self.t[name] = a.to(device=device, dtype=torch.float32).to(torch.bfloat16).contiguous()
            else:
                self.t[name] = a.to(device=device, dtype=torch.float32).contiguous()
        for name in ("b_qkv", "b_o", "b_1", "b_2", "g_q", "g_k"):
            self.t[name] = torch.as_tensor(arrays[name]).to(device=device, dtype=torch.float32).contiguous()
        self.c = BlockWeightsC(**{n: (self.t[n].data_ptr() if n in self.t else None)
                                  for n, _ in BlockWeightsC._fields_})

    @classmethod
    def from_device(cls, tensors: Dict[str, torch.Tensor], mode: str) -> "BlockWeights":
        obj = cls.__new__(cls)
        obj.mode = mode
        obj.t = dict(tensors)
        obj.c = BlockWeightsC(**{n: (obj.t[n].data_ptr() if n in obj.t else None) for n, _ in BlockWeightsC._fields_})
        return obj


def workspace_bytes(cfg: BlockConfig, T_q: int, T_k: int) -> int:
    return int(lib().dit_block_workspace_bytes(ctypes.byref(cfg), T_q, T_k))


def _io(x, mod, mod_of_seg, cos_t, sin_t, seg_len, T_k, k_cache, v_cache):
    mos = _host_i32(mod_of_seg)
    segs = _host_i32(seg_len)
    io = BlockIO(x=_p(x), mod=_p(mod), n_mod=mod.shape[0], mod_of_seg=ctypes.cast(mos, _vp), cos_t=_p(cos_t),
                 sin_t=_p(sin_t), seg_len=ctypes.cast(segs, _vp), n_seg=len(seg_len), T_q=x.shape[0], T_k=T_k,
                 k_cache=_p(k_cache), v_cache=_p(v_cache))
    return io, (mos, segs)


def block_forward(cfg: BlockConfig, w: BlockWeights, x, mod, mod_of_seg, cos_t, sin_t, seg_len, k_cache, v_cache,
                  workspace, stream=None) -> None:
    """x [T_q, D] updated in place; k_cache/v_cache [T_k, H, 128]."""
    T_k = int(sum(seg_len))
    io, keep = _io(x, mod, mod_of_seg, cos_t, sin_t, seg_len, T_k, k_cache, v_cache)
    _check(lib().dit_block_forward(ctypes.byref(cfg), ctypes.byref(w.c), ctypes.byref(io), _p(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "dit_block_forward")
    del keep


def stack_forward(cfg: BlockConfig, ws: Sequence[BlockWeights], x, mod, mod_of_seg, cos_t, sin_t, seg_len,
                  k_caches, v_caches, workspace, stream=None) -> None:
    T_k = int(sum(seg_len))
    n = len(ws)
    arr = (BlockWeightsC * n)(*[w.c for w in ws])
    kc = (_vp * n)(*[_p(t) for t in k_caches])
    vc = (_vp * n)(*[_p(t) for t in v_caches])
    io, keep = _io(x, mod, mod_of_seg, cos_t, sin_t, seg_len, T_k, None, None)
    _check(lib().dit_stack_forward(ctypes.byref(cfg), arr, n, ctypes.byref(io), ctypes.cast(kc, _vp),
                                   ctypes.cast(vc, _vp), _p(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "dit_stack_forward")
    del keep


class HeadWeights:
    """Device tensors of the DiT head/tail (dit_head_weights): w_txt_in [D, C_txt],
    w_img_in [D, C_lat], w_proj_out [C_lat, D] in the activation dtype and fp32
    biases b_txt_in, b_img_in, b_proj_out."""

    def __init__(self, t: dict):
        self.t = t
        self.c = HeadWeightsC(
            w_txt_in=_p(t.get("w_txt_in")), b_txt_in=_p(t.get("b_txt_in")), w_img_in=_p(t["w_img_in"]),
            b_img_in=_p(t.get("b_img_in")), w_proj_out=_p(t["w_proj_out"]), b_proj_out=_p(t.get("b_proj_out")),
            C_txt=t["w_txt_in"].shape[1] if t.get("w_txt_in") is not None else 0, C_lat=t["w_img_in"].shape[1])


def velocity_workspace_bytes(cfg: BlockConfig, T_q: int, N: int, C_lat: int, T_k: Optional[int] = None) -> int:
    """T_k = L_txt + R + N (defaults to T_q, the whole sequence)."""
    T_k = T_q if T_k is None else T_k
    return int(lib().dit_velocity_workspace_bytes(ctypes.byref(cfg), T_q, T_k, N, C_lat))


def velocity_forward(cfg: BlockConfig, ws: Sequence[BlockWeights], head: HeadWeights, latent, vel, mod,
                     mod_of_seg, mod_final, cos_t, sin_t, seg_len, k_caches, v_caches, workspace,
                     txt_feats=None, ref_latent=None, L_txt: int = 0, R: int = 0, T_q: Optional[int] = None,
                     stream=None) -> None:
    """dit_velocity_forward: vel [N, C_lat] from the target latent [N, C_lat] (fp32);
    T_q = L_txt + R + N computes every row, T_q = N only the target rows."""
    N = latent.shape[0]
    T_k = int(sum(seg_len))
    if T_q is None:
        T_q = T_k
    n = len(ws)
    arr = (BlockWeightsC * max(n, 1))(*[w.c for w in ws])
    kc = (_vp * max(n, 1))(*[_p(t) for t in k_caches])
    vc = (_vp * max(n, 1))(*[_p(t) for t in v_caches])
    mos = _host_i32(mod_of_seg)
    segs = _host_i32(seg_len)
    io = VelocityIO(txt_feats=_p(txt_feats), ref_latent=_p(ref_latent), latent=_p(latent), L_txt=L_txt, R=R, N=N,
                    mod=_p(mod), n_mod=mod.shape[0], mod_of_seg=ctypes.cast(mos, _vp), mod_final=_p(mod_final),
                    cos_t=_p(cos_t), sin_t=_p(sin_t), seg_len=ctypes.cast(segs, _vp), n_seg=len(seg_len), T_q=T_q,
                    k_caches=ctypes.cast(kc, _vp), v_caches=ctypes.cast(vc, _vp), vel=_p(vel))
    _check(lib().dit_velocity_forward(ctypes.byref(cfg), arr, n, ctypes.byref(head.c), ctypes.byref(io),
                                      _p(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "dit_velocity_forward")
    del mos, segs, kc, vc, arr


# ---------------------------------------------------------------- gated-MLP block (per-linear W8A8)

GATED_LINEARS = ("qk", "v", "o", "proj", "gate", "down")


def recipe_int8_linears(block: int, n_blocks: int) -> Tuple[str, ...]:
    """The page's W8A8 scope ("Qwen-Image-2.1 W8A8 - FlagOS for Mac", Quantization
    and validation): Q/K and the MLP proj/gate linears in blocks 2..n-3 (2..29 of 32)."""
    return ("qk", "proj", "gate") if 2 <= block <= n_blocks - 3 else ()


class GatedBlockWeights:
    """Device weights of one gated block: arrays w_qk, w_v, w_o, w_proj, w_gate,
    w_down ([N, K]) with biases b_* and gains g_q, g_k; the linears named in
    ``int8`` are quantized per output channel on the GPU (codes, scales and the
    codes' row sums); ``mx`` maps linears to MXFP4 (codes [N, K/2], E8M0 scales
    [N, K/32]) uploaded as they are; the others uploaded as bf16."""

    def __init__(self, arrays: Dict, int8: Sequence[str] = (), device="cuda", mx: Optional[Dict] = None):
        self.t: Dict[str, torch.Tensor] = {}
        self.int8 = tuple(int8)
        mx = mx or {}
        lin = {}
        for name in GATED_LINEARS:
            b = torch.as_tensor(arrays["b_" + name]).to(device=device, dtype=torch.float32).contiguous()
            self.t["b_" + name] = b
            if name in mx:
                codes, scales = (torch.as_tensor(v).to(device=device, dtype=torch.uint8).contiguous() for v in mx[name])
                self.t.update({"mx_" + name: codes, "mxs_" + name: scales})
                lin[name] = LinearC(w=_p(codes), s=None, wsum=None, b=_p(b), mx_scale=_p(scales))
                continue
            a = torch.as_tensor(arrays["w_" + name])
            if name in self.int8:
                master = a.to(device=device, dtype=torch.float32).contiguous()
                q = torch.empty(master.shape, dtype=torch.int8, device=device)
                sc = torch.empty(master.shape[0], dtype=torch.float32, device=device)
                quantize_rows(master, q, sc)
                ws = torch.empty(master.shape[0], dtype=torch.int32, device=device)
                int8_colsum(q, ws)
                del master
                self.t.update({"w_" + name: q, "s_" + name: sc, "wsum_" + name: ws})
                lin[name] = LinearC(w=_p(q), s=_p(sc), wsum=_p(ws), b=_p(b))
            else:
                wt = a.to(device=device, dtype=torch.float32).to(torch.bfloat16).contiguous()
                self.t["w_" + name] = wt
                lin[name] = LinearC(w=_p(wt), s=None, wsum=None, b=_p(b))
        for name in ("g_q", "g_k"):
            self.t[name] = torch.as_tensor(arrays[name]).to(device=device, dtype=torch.float32).contiguous()
        self.c = GatedBlockWeightsC(**lin, g_q=_p(self.t["g_q"]), g_k=_p(self.t["g_k"]))


def gated_workspace_bytes(cfg: BlockConfig, T_q: int, T_k: int) -> int:
    return int(lib().dit_gated_block_workspace_bytes(ctypes.byref(cfg), T_q, T_k))


def block_forward_gated(cfg: BlockConfig, w: GatedBlockWeights, x, mod, mod_of_seg, cos_t, sin_t, seg_len, k_cache,
                        v_cache, workspace, stream=None) -> None:
    """x [T_q, D] bf16 updated in place; k_cache/v_cache [T_k, H, 128] bf16."""
    T_k = int(sum(seg_len))
    io, keep = _io(x, mod, mod_of_seg, cos_t, sin_t, seg_len, T_k, k_cache, v_cache)
    _check(lib().dit_block_forward_gated(ctypes.byref(cfg), ctypes.byref(w.c), ctypes.byref(io), _p(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)),
           "dit_block_forward_gated")
    del keep
