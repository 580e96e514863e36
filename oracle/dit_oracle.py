"""Oracle for one single-stream DiT block, its ops, and one denoise step.

Sources (page title, section):
  [FlagOS]   "Qwen-Image-2.1 W8A8 - FlagOS for Mac", Quantization and validation
  [mere]     "Qwen Image 2.1 native qualification", Numerical checks
  [CoreAI]   "RGBA-Image-2.1 - Core AI port of Qwen-Image-2.1", intro and Graph contracts
  [MNN]      "qwen-image-mnn" package description, What runs where / Install, run
  [Paiton]   "Qwen_Image-2.1-MXFP4-Paiton", Runtime precision and quality / Tested operating limits

Where the pages leave a step open, the reading taken is stated at the function.

Precision modes of ``block_forward``:
  "f32":  every value kept in fp64 (the reference for a GPU that computes in fp32).
  "bf16": fp64 arithmetic, with each tensor the block stores rounded to bf16 at the
          point where it is stored (activations, linear outputs, q/k/v, attention
          output, GELU output, residual stream); statistics, softmax, accumulators and
          modulation stay fp64.
  "w8a8": "bf16" with the inputs of the four linears quantized to int8 per token and
          the weights int8 per output channel (int32-exact accumulation).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "round_bf16", "quantize_rows", "int8_matmul_exact", "w8a8_linear", "linear",
    "adaln_modulate", "qk_rmsnorm", "apply_gain", "block_forward_rows", "rope_positions", "rope_tables", "apply_rope",
    "segment_ids", "allowed_mask", "attention", "gelu_tanh", "block_forward",
    "quantize_block_weights", "dit_step", "denoise_loop", "euler_update", "rel_l2", "HEAD_DIM",
    "ROPE_AXES", "ROPE_THETA", "LN_EPS", "QK_EPS",
    "round_fp8_e4m3", "encode_fp8_e4m3", "decode_fp8_e4m3", "quantize_attn_q", "quantize_attn_k",
    "quantize_attn_v", "attention_q8", "attention_q8_bound", "attention_quantized", "ATTN_KEY_TILE", "FP8_MAX",
    "quantize_rows_asym", "w8a8_linear_asym", "block_forward_gated", "GATED_LINEARS", "mxfp4_decode",
    "E2M1_VALUES",
]

HEAD_DIM = 128
ROPE_AXES = (32, 48, 48)   # frame, height, width share of the head dim
ROPE_THETA = 10000.0
LN_EPS = 1e-6
QK_EPS = 1e-6


# ----------------------------------------------------------------------------- rounding

def round_bf16(a) -> np.ndarray:
    """Nearest bfloat16 value of each element (ties to even), as float64.

    bf16 keeps 7 of fp64's 52 explicit mantissa bits; in bf16's normal range
    (|a| >= 2^-126) the low 45 bits are rounded off on the integer view.  Below
    it bf16 is subnormal with a fixed step of 2^-133 (fp32's exponent range, 7
    fraction bits), so the value is rounded to a multiple of that step (values
    under half a step go to a signed zero).  Valid for finite values below
    bf16's largest finite value.
    """
    a = np.ascontiguousarray(a, dtype=np.float64)
    bits = a.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    bits = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    out = bits.view(np.float64)
    tiny = np.abs(a) < 2.0 ** -126
    if np.any(tiny):
        out = out.copy()
        sub = np.rint(a[tiny] * 2.0 ** 133) * 2.0 ** -133   # exact scaling, ties to even
        out[tiny] = np.copysign(sub, a[tiny])
    return out


def _store(a, mode: str):
    return a if mode == "f32" else round_bf16(a)


# ----------------------------------------------------------------------------- W8A8

def quantize_rows(a) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric per-row int8 quantization with fp32 scales.

    [FlagOS, Quantization and validation]: int8 weights are symmetric per
    output channel with zero point 0 and fp32 scales; activations are
    quantized dynamically per token.  Reading: the activation side uses the
    same symmetric rule (the workloads ask for symmetric activations), with
    s = amax/127 in fp32, q = clamp(round_half_even(a/s), -127, 127) using an
    IEEE fp32 division, and an all-zero row giving s = 0 and q = 0.  The values
    must be exactly representable in fp32 (they are bf16 or fp32 tensors).
    Returns (q int8 [..., K], s float32 [...]).
    """
    a64 = np.asarray(a, dtype=np.float64)
    a32 = a64.astype(np.float32)
    if not np.array_equal(a32.astype(np.float64), a64):
        raise ValueError("quantize_rows: input not representable in fp32")
    amax = np.max(np.abs(a32), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    r = (a32 / safe[..., None]).astype(np.float32)
    q = np.clip(np.rint(r), -127, 127)
    q[s == 0] = 0
    return q.astype(np.int8), s


def int8_matmul_exact(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k qa[m, k] * qw[n, k] exactly, as int64.

    [FlagOS, Quantization and validation]: int32 accumulation.  With codes in
    [-127, 127] every partial sum is an integer below K*127^2 < 2^53, so fp64
    BLAS returns it exactly whatever its summation order.
    """
    K = qa.shape[-1]
    assert qw.shape[-1] == K
    assert K * 127 * 127 < 2 ** 53
    if K <= 1024:
        return np.rint(qa.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64)
    # Same exactness argument in fp32 for chunks of 1024: |partial sums| <= 1024*127^2 < 2^24.
    acc = np.zeros((qa.shape[0], qw.shape[0]), dtype=np.int64)
    for k0 in range(0, K, 1024):
        part = qa[:, k0:k0 + 1024].astype(np.float32) @ qw[:, k0:k0 + 1024].astype(np.float32).T
        acc += np.rint(part).astype(np.int64)
    return acc


def quantize_rows_asym(a) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Asymmetric per-row int8 quantization with fp32 scales and int32 zero points.

    [FlagOS, Quantization and validation]: activations are quantized dynamically,
    asymmetric int8 per token/row, fp32 scales.  Reading (the page gives no
    formula): the range is widened to contain 0, lo = min(row, 0), hi = max(row, 0);
    s = fp32(hi - lo) / 255 in fp32; zero point z = -128 - rint(lo / s), which
    lies in [-128, 127]; q = clamp(rint(a / s) + z, -128, 127); IEEE fp32
    divisions, ties to even; the value a code stands for is (q - z) * s.  An
    all-zero row gives s = 0, z = 0, q = 0.  Returns (q int8, s float32, z int32).
    """
    a64 = np.asarray(a, dtype=np.float64)
    a32 = a64.astype(np.float32)
    if not np.array_equal(a32.astype(np.float64), a64):
        raise ValueError("quantize_rows_asym: input not representable in fp32")
    lo = np.minimum(np.min(a32, axis=-1), np.float32(0))
    hi = np.maximum(np.max(a32, axis=-1), np.float32(0))
    s = ((hi - lo).astype(np.float32) / np.float32(255.0)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    z = (-128 - np.rint((lo / safe).astype(np.float32))).astype(np.int64)
    z = np.clip(z, -128, 127)
    r = np.rint((a32 / safe[..., None]).astype(np.float32)).astype(np.int64) + z[..., None]
    q = np.clip(r, -128, 127)
    q[s == 0] = 0
    z[s == 0] = 0
    return q.astype(np.int8), s, z.astype(np.int32)


def w8a8_linear_asym(qa, sa, za, qw, sw, bias) -> np.ndarray:
    """y = (sum_k (qa[m,k] - za[m]) qw[n,k]) * sa[m] * sw[n] + bias[n], fp64.

    The integer sum is the exact int32 product minus the zero point times the
    weight codes' row sum (both exact integers)."""
    acc = int8_matmul_exact(qa, qw) - np.asarray(za, np.int64)[:, None] * \
        np.asarray(qw, np.int64).sum(axis=1)[None, :]
    y = acc.astype(np.float64) * np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y


# [Paiton, What was quantized]: MXFP4 storage, E2M1 values packed low nibble
# first, one E8M0 scale per group of 32 input columns.  E2M1 (OCP MX): sign,
# 2 exponent bits (bias 1), 1 mantissa bit -> 0, 0.5, 1, 1.5, 2, 3, 4, 6; E8M0:
# the power of two 2^(e - 127) (e = 255 is NaN).
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def mxfp4_decode(codes, scales) -> np.ndarray:
    """Weights [N, K] (fp64) from packed codes [N, K/2] (uint8, element 2i in the
    low nibble of byte i) and E8M0 scales [N, K/32] (uint8).  [Paiton, Runtime
    precision and quality / What was quantized]: the runtime reconstructs these
    weights and computes in bf16; every E2M1 value times a power of two is
    exact in bf16 inside bf16's exponent range."""
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.uint8)
    N, half = codes.shape
    K = 2 * half
    if scales.shape != (N, K // 32):
        raise ValueError("mxfp4_decode: scales must be [N, K/32]")
    nib = np.empty((N, K), np.uint8)
    nib[:, 0::2] = codes & 0x0F
    nib[:, 1::2] = codes >> 4
    mag = np.asarray(E2M1_VALUES, np.float64)[nib & 7]
    val = np.where(nib & 8, -mag, mag)
    e = scales.astype(np.int64)
    pw = np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))
    return val * np.repeat(pw, 32, axis=1)


def w8a8_linear(qa, sa, qw, sw, bias) -> np.ndarray:
    """y = acc * s_a[m] * s_w[n] + b[n] in fp64 ([FlagOS]: fp32 scaling after int32 accumulation)."""
    acc = int8_matmul_exact(qa, qw).astype(np.float64)
    y = acc * np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y


def linear(a, w, bias) -> np.ndarray:
    """y = a @ w.T + b in fp64; w is [N, K]."""
    y = np.asarray(a, np.float64) @ np.asarray(w, np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y


def quantize_block_weights(weights: Dict[str, np.ndarray]) -> Dict[str, Tuple[np.ndarray, np.ndarray]]:
    """Per-output-channel int8 codes and fp32 scales of the four linear matrices."""
    return {k: quantize_rows(weights[k]) for k in ("w_qkv", "w_o", "w_1", "w_2")}


# ----------------------------------------------------------------------------- norms

def adaln_modulate(x, shift, scale, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm without affine (biased variance) followed by x_hat*(1+scale)+shift.

    [MNN, What runs where] names the per-block modulation rows; the reading is
    the plain adaLN form with (shift, scale) rows broadcast per token.
    """
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    xhat = (x - mu) / np.sqrt(var + eps)
    return xhat * (1.0 + np.asarray(scale, np.float64)) + np.asarray(shift, np.float64)


def qk_rmsnorm(t, g, mode: str, eps: float = QK_EPS) -> np.ndarray:
    """Per-head RMSNorm over the 128 head dims, with a learned gain g [128].

    [mere, Numerical checks]: the normalized activation is cast to the gain's
    dtype (bf16 in the bf16 modes) before it is multiplied by the gain; the
    product is a bf16 tensor again.
    """
    t = np.asarray(t, np.float64)
    n = t / np.sqrt((t * t).mean(axis=-1, keepdims=True) + eps)
    return apply_gain(n, g, mode)


def apply_gain(n, g, mode: str) -> np.ndarray:
    """Gain step of the Q/K RMSNorm: in the bf16 modes, round n to bf16, multiply, round again."""
    if mode == "f32":
        return np.asarray(n, np.float64) * np.asarray(g, np.float64)
    return round_bf16(round_bf16(n) * np.asarray(g, np.float64))


# ----------------------------------------------------------------------------- RoPE

def rope_positions(text_len: int, grids: Sequence[Tuple[int, int]]) -> np.ndarray:
    """(frame, height, width) position of every token of [text | image_0 | image_1 ...].

    [CoreAI, Graph contracts]: text token i sits at (i, i, i); image token (y, x)
    of an h x w grid, in raster order, sits at (L, y - (h - h//2), x - (w - w//2))
    with L the text length.  Reading for a second image segment: the k-th image
    segment (0-based) takes frame L + k.
    """
    pos = [(i, i, i) for i in range(text_len)]
    for k, (h, w) in enumerate(grids):
        for y in range(h):
            for x in range(w):
                pos.append((text_len + k, y - (h - h // 2), x - (w - w // 2)))
    return np.array(pos, dtype=np.int64).reshape(-1, 3)


def rope_tables(pos: np.ndarray, theta: float = ROPE_THETA, axes=ROPE_AXES):
    """cos/sin [T, 64], one angle per interleaved pair of head dims.

    [CoreAI, Graph contracts] passes per-token cos/sin of width 64 per stream;
    [MNN, What runs where] names the 3-axis RoPE.  Axis a owns axes[a] head dims,
    i.e. axes[a]/2 pairs; pair j of axis a rotates by pos_a * theta^(-2j/axes[a]).
    Pairs are ordered frame, height, width.
    """
    angles = []
    for a, dim in enumerate(axes):
        j = np.arange(dim // 2, dtype=np.float64)
        omega = theta ** (-2.0 * j / dim)
        angles.append(pos[:, a:a + 1].astype(np.float64) * omega[None, :])
    phi = np.concatenate(angles, axis=1)
    return np.cos(phi), np.sin(phi)


def apply_rope(t, cos, sin) -> np.ndarray:
    """Rotate interleaved pairs (t[2m], t[2m+1]) of each head by the token's angle m."""
    t = np.asarray(t, np.float64)
    c = np.asarray(cos, np.float64)[:, None, :]
    s = np.asarray(sin, np.float64)[:, None, :]
    ev, od = t[..., 0::2], t[..., 1::2]
    out = np.empty_like(t)
    out[..., 0::2] = ev * c - od * s
    out[..., 1::2] = ev * s + od * c
    return out


# ----------------------------------------------------------------------------- attention

def segment_ids(seg_len: Sequence[int]) -> np.ndarray:
    return np.repeat(np.arange(len(seg_len)), np.asarray(seg_len, dtype=np.int64))


def allowed_mask(seg_len: Sequence[int], T_q: int) -> np.ndarray:
    """allowed[i, j]: query row i (absolute position T_k - T_q + i) may attend key j.

    [CoreAI, intro] and [MNN, What runs where]: the single-stream DiT attends
    block-causally over its segments.  Reading: every segment sees itself
    bidirectionally and all earlier segments.
    """
    seg = segment_ids(seg_len)
    T_k = seg.shape[0]
    sq = seg[T_k - T_q:]
    return seg[None, :] <= sq[:, None]


def attention(q, k, v, seg_len: Sequence[int], scale: Optional[float] = None) -> np.ndarray:
    """Block-causal softmax attention per head, fp64.

    q [T_q, H, d], k and v [T_k, H, d]; query row i is at absolute position
    T_k - T_q + i, so a prefix of keys may come from a cache.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T_q, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    allowed = allowed_mask(seg_len, T_q)
    out = np.empty_like(q)
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h, :]
    return out


# ----------------------------------------------------------------------------- quantized attention

# [Paiton, Runtime precision and quality]: after the first denoising steps the
# runtime switches to int8 activations and int8/fp8 attention.  The page names
# the number formats only.  Reading taken here (SageAttention-style):
#   * Q K^T in int8: Q symmetric per (token, head), K symmetric per (tile of
#     ATTN_KEY_TILE consecutive keys, head); scales amax/127 in fp32, codes by
#     an IEEE fp32 division and round-half-even (the rule of quantize_rows);
#   * P V in fp8 e4m3: V symmetric per (head, channel) over all keys, scale
#     amax/448; P = exp(S - rowmax) in [0, 1] rounded to e4m3 unscaled;
#   * O = (sum_j fp8(P_ij) * V_j) / (sum_j P_ij): the normalizer adds the
#     unrounded probabilities.
ATTN_KEY_TILE = 64
FP8_MAX = 448.0


def round_fp8_e4m3(x) -> np.ndarray:
    """Nearest e4m3 value (ties to even), saturating at +-448.

    e4m3 (OCP FP8, "fn" variant): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
    normal values 2^(e-7) * (1 + m/8) for e = 1..15 (the top code 0x7F is NaN,
    so 448 = 2^8 * 1.75 is the largest), subnormals 2^-6 * m/8.  On the grid
    the spacing is 2^(E-3) for |x| in [2^E, 2^(E+1)), E >= -6, and 2^-9 below
    2^-6.  Saturation above 448 is the reading for out-of-range inputs.
    """
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    E = np.maximum(ex.astype(np.int64) - 1, -6)
    step = np.ldexp(1.0, E - 3)
    r = np.rint(a / step) * step              # power-of-two division: exact; rint ties to even
    r = np.minimum(r, FP8_MAX)
    return np.copysign(r, x)


def encode_fp8_e4m3(v) -> np.ndarray:
    """Byte codes of values already on the e4m3 grid (|v| <= 448)."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    sign = (np.signbit(v) & (a > 0)).astype(np.uint8) << 7
    _, ex = np.frexp(a)
    E = ex.astype(np.int64) - 1
    normal = a >= 2.0 ** -6
    e_field = np.where(normal, E + 7, 0)
    mant = np.where(normal, a / np.ldexp(1.0, np.where(normal, E, 0)) - 1.0, a / 2.0 ** -6) * 8.0
    if not np.all(mant == np.rint(mant)) or np.any(a > FP8_MAX):
        raise ValueError("encode_fp8_e4m3: value not on the e4m3 grid")
    return (sign | (e_field.astype(np.uint8) << 3) | np.rint(mant).astype(np.uint8)).astype(np.uint8)


def decode_fp8_e4m3(c) -> np.ndarray:
    """Values of e4m3 byte codes (0x7F and 0xFF are NaN)."""
    c = np.asarray(c, np.uint8).astype(np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def quantize_attn_q(q) -> Tuple[np.ndarray, np.ndarray]:
    """q [T, H, d] -> int8 codes [T, H, d] and fp32 scales [T, H] (per token and head)."""
    return quantize_rows(q)


def quantize_attn_k(k, tile: int = ATTN_KEY_TILE) -> Tuple[np.ndarray, np.ndarray]:
    """k [T_k, H, d] -> int8 codes [T_k, H, d] and fp32 scales [ceil(T_k / tile), H].

    One scale per (tile of consecutive keys, head): amax over the tile's keys and
    the head's d channels, with the rule of quantize_rows."""
    k = np.asarray(k, np.float64)
    T_k, H, d = k.shape
    nt = (T_k + tile - 1) // tile
    codes = np.zeros((T_k, H, d), np.int8)
    scales = np.zeros((nt, H), np.float32)
    for t in range(nt):
        blk = k[t * tile:(t + 1) * tile]                     # [n, H, d]
        flat = np.transpose(blk, (1, 0, 2)).reshape(H, -1)   # per head: all values of the tile
        qf, sf = quantize_rows(flat)
        codes[t * tile:(t + 1) * tile] = np.transpose(qf.reshape(H, blk.shape[0], d), (1, 0, 2))
        scales[t] = sf
    return codes, scales


def quantize_attn_v(v) -> Tuple[np.ndarray, np.ndarray]:
    """v [T_k, H, d] -> e4m3 values [T_k, H, d] (float64 on the e4m3 grid) and fp32
    scales [H, d]: s = amax over all keys / 448 per (head, channel), values
    round_fp8_e4m3(fp32(v / s)) with an IEEE fp32 division; s = 0 gives 0."""
    v64 = np.asarray(v, np.float64)
    v32 = v64.astype(np.float32)
    if not np.array_equal(v32.astype(np.float64), v64):
        raise ValueError("quantize_attn_v: input not representable in fp32")
    amax = np.max(np.abs(v32), axis=0)                       # [H, d]
    s = (amax / np.float32(FP8_MAX)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    r = (v32 / safe[None]).astype(np.float32)
    vals = round_fp8_e4m3(r)
    vals[:, s == 0] = 0.0
    return vals, s


def _q8_probs(q8, sq, k8, sk, seg_len, scale, tile, h):
    """P = exp(S - rowmax) [T_q, T_k] of head h on the quantized operands (0 where masked)."""
    q8 = np.asarray(q8, np.float64)
    k8 = np.asarray(k8, np.float64)
    T_q, _, d = q8.shape
    T_k = k8.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    allowed = allowed_mask(seg_len, T_q)
    key_scale = np.asarray(sk, np.float64)[np.arange(T_k) // tile, h]
    acc = q8[:, h, :] @ k8[:, h, :].T                      # integers below 2^53: exact
    s = acc * np.asarray(sq, np.float64)[:, h, None] * key_scale[None, :] * scale
    s = np.where(allowed, s, -np.inf)
    return np.exp(s - s.max(axis=1, keepdims=True))


def attention_q8(q8, sq, k8, sk, v8, sv, seg_len: Sequence[int], scale: Optional[float] = None,
                 tile: int = ATTN_KEY_TILE, round_p: bool = True) -> np.ndarray:
    """Block-causal attention on quantized operands (the reading above), fp64.

    q8 [T_q, H, d] int8 with sq [T_q, H]; k8 [T_k, H, d] int8 with sk
    [ceil(T_k/tile), H]; v8 [T_k, H, d] e4m3 values with sv [H, d].  Scores are
    exact integer dot products times the scales; the softmax is fp64.
    round_p=False keeps P unrounded (the reference for attention_q8_bound)."""
    v8 = np.asarray(v8, np.float64)
    T_q, H, d = np.asarray(q8).shape
    out = np.empty((T_q, H, d))
    for h in range(H):
        p = _q8_probs(q8, sq, k8, sk, seg_len, scale, tile, h)
        p8 = round_fp8_e4m3(p) if round_p else p
        vd = v8[:, h, :] * np.asarray(sv, np.float64)[h][None, :]
        out[:, h, :] = (p8 @ vd) / p.sum(axis=1, keepdims=True)
    return out


def attention_q8_bound(q8, sq, k8, sk, v8, sv, seg_len: Sequence[int], scale: Optional[float] = None,
                       tile: int = ATTN_KEY_TILE) -> np.ndarray:
    """Element-wise bound on |attention_q8(round_p=True) - attention_q8(round_p=False)|
    for any rounding reference: if P is rounded to e4m3 after scaling by any
    2^delta >= 1 (a running maximum below the final one), each rounded value is
    within 2^-4 of it relatively (half of e4m3's 2^-3 mantissa step) or 2^-10
    absolutely (half the subnormal step 2^-9), and dividing back by 2^delta
    only shrinks the absolute part.  Hence
        |err[i, c]| <= (2^-4 sum_j P_ij |v_jc| + 2^-10 sum_j |v_jc|) / sum_j P_ij
    with the sums over the keys query i sees."""
    v8 = np.asarray(v8, np.float64)
    T_q, H, d = np.asarray(q8).shape
    out = np.empty((T_q, H, d))
    for h in range(H):
        p = _q8_probs(q8, sq, k8, sk, seg_len, scale, tile, h)
        vabs = np.abs(v8[:, h, :] * np.asarray(sv, np.float64)[h][None, :])
        seen = (p > 0).astype(np.float64)
        out[:, h, :] = (2.0 ** -4 * (p @ vabs) + 2.0 ** -10 * (seen @ vabs)) / p.sum(axis=1, keepdims=True)
    return out


def attention_quantized(q, k, v, seg_len: Sequence[int], scale: Optional[float] = None) -> np.ndarray:
    """Quantize q, k, v (bf16 or fp32 tensors) as above, then attention_q8."""
    q8, sq = quantize_attn_q(q)
    k8, sk = quantize_attn_k(k)
    v8, sv = quantize_attn_v(v)
    return attention_q8(q8, sq, k8, sk, v8, sv, seg_len, scale)


# ----------------------------------------------------------------------------- MLP

def gelu_tanh(u) -> np.ndarray:
    """tanh-approximated GELU (the workloads' MLP activation):
    0.5 u (1 + tanh(x)) with x = sqrt(2/pi) (u + 0.044715 u^3).

    For x < 0 the factor 1 + tanh(x) is taken as 2 e^{2x} / (1 + e^{2x}), the
    same number written without the cancellation that leaves fp64's
    1 + tanh(x) at zero or rounding noise once x < -19 (u below about -6).
    """
    u = np.asarray(u, np.float64)
    x = math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)
    e = np.exp(2.0 * np.minimum(x, 0.0))
    one_plus_tanh = np.where(x >= 0.0, 1.0 + np.tanh(np.maximum(x, 0.0)), 2.0 * e / (1.0 + e))
    return 0.5 * u * one_plus_tanh


# ----------------------------------------------------------------------------- block

def _row_mod(mod, mod_of_seg, seg_len, T_q) -> np.ndarray:
    """[T_q, 6, D] modulation rows of each computed token (by its segment's set)."""
    seg = segment_ids(seg_len)
    rows_seg = seg[seg.shape[0] - T_q:]
    return np.asarray(mod, np.float64)[np.asarray(mod_of_seg)[rows_seg]]


def _lin(a, name, weights, qweights, mode):
    if mode == "w8a8":
        qa, sa = quantize_rows(a)
        qw, sw = qweights[name]
        return w8a8_linear(qa, sa, qw, sw, weights["b" + name[1:]])
    return linear(a, weights[name], weights["b" + name[1:]])


def block_forward(x, mod, mod_of_seg, seg_len, cos, sin, weights, mode: str,
                  k_prefix=None, v_prefix=None, qweights=None,
                  ln_eps: float = LN_EPS, qk_eps: float = QK_EPS,
                  attn_quant: bool = False) -> Dict[str, np.ndarray]:
    """Forward of one single-stream DiT block on the last T_q rows of the sequence.

    x [T_q, D]: the rows computed by this call (the whole sequence, or the target
    rows when the prefix K/V come from a cache).  mod [n_sets, 6, D] holds rows
    (shift1, scale1, gate1, shift2, scale2, gate2); mod_of_seg maps each segment
    to its set.  cos/sin [T_q, 64] belong to the computed rows.  k_prefix/v_prefix
    [T_k - T_q, H, 128] are the cached K/V of the earlier rows (post-norm,
    post-RoPE K and plain V).

    Order (reading: pre-norm adaLN with gated residuals, the arrangement that uses
    six modulation rows and a gated residual):
      h  = LN(x)(1+scale1)+shift1;  [q|k|v] = h Wqkv^T + b
      q, k <- RoPE(RMSNorm_head(q, k) * g)   (cast before gain [mere])
      o  = block-causal attention(q, [k_prefix; k], [v_prefix; v])
      x1 = x + gate1 * (o Wo^T + bo)
      h2 = LN(x1)(1+scale2)+shift2
      x2 = x1 + gate2 * (GELU_tanh(h2 W1^T + b1) W2^T + b2)
    attn_quant: the attention runs on int8/fp8 operands (``attention_quantized``).
    Returns x_out and the new K/V rows plus intermediates.
    """
    x = np.asarray(x, np.float64)
    T_q, D = x.shape
    H = D // HEAD_DIM
    if mode == "w8a8" and qweights is None:
        qweights = quantize_block_weights(weights)
    m = _row_mod(mod, mod_of_seg, seg_len, T_q)
    shift1, scale1, gate1, shift2, scale2, gate2 = (m[:, i, :] for i in range(6))

    h = _store(adaln_modulate(x, shift1, scale1, ln_eps), mode)
    qkv = _store(_lin(h, "w_qkv", weights, qweights, mode), mode)
    q = qkv[:, :D].reshape(T_q, H, HEAD_DIM)
    k = qkv[:, D:2 * D].reshape(T_q, H, HEAD_DIM)
    v = qkv[:, 2 * D:].reshape(T_q, H, HEAD_DIM)
    q = _store(apply_rope(qk_rmsnorm(q, weights["g_q"], mode, qk_eps), cos, sin), mode)
    k = _store(apply_rope(qk_rmsnorm(k, weights["g_k"], mode, qk_eps), cos, sin), mode)
    if k_prefix is not None and len(k_prefix):
        k_all = np.concatenate([np.asarray(k_prefix, np.float64), k], axis=0)
        v_all = np.concatenate([np.asarray(v_prefix, np.float64), v], axis=0)
    else:
        k_all, v_all = k, v
    attend = attention_quantized if attn_quant else attention
    o = _store(attend(q, k_all, v_all, seg_len), mode).reshape(T_q, D)
    y = _store(_lin(o, "w_o", weights, qweights, mode), mode)
    x1 = _store(x + gate1 * y, mode)
    h2 = _store(adaln_modulate(x1, shift2, scale2, ln_eps), mode)
    u = _store(_lin(h2, "w_1", weights, qweights, mode), mode)
    g = _store(gelu_tanh(u), mode)
    y2 = _store(_lin(g, "w_2", weights, qweights, mode), mode)
    x2 = _store(x1 + gate2 * y2, mode)
    return {"x_out": x2, "k": k, "v": v, "q": q, "h": h, "qkv": qkv, "o": o,
            "x1": x1, "h2": h2, "u": u, "g": g}


GATED_LINEARS = ("w_qk", "w_v", "w_o", "w_proj", "w_gate", "w_down")


def block_forward_gated(x, mod, mod_of_seg, seg_len, cos, sin, weights, int8=(), attn_quant: bool = False,
                        k_prefix=None, v_prefix=None, ln_eps: float = LN_EPS,
                        qk_eps: float = QK_EPS, mx=None) -> Dict[str, np.ndarray]:
    """The block with a gated MLP and a per-linear choice of W8A8 ([FlagOS,
    Quantization and validation]: Q/K and the MLP proj/gate linears of the middle
    blocks run W8A8 with asymmetric per-token activations, the rest bf16).

    weights: w_qk [2D, D] (q rows, then k rows), w_v [D, D], w_o [D, D],
    w_proj [F, D], w_gate [F, D], w_down [D, F] (fp32 masters on the bf16 grid),
    their biases b_*, and g_q, g_k.  int8: names of the linears that run W8A8
    (weights quantized symmetric per output channel, activations asymmetric per
    token, w8a8_linear_asym); mx: {name: (codes, scales)} for linears stored as
    MXFP4 ([Paiton]: reconstructed weights, bf16 arithmetic; the reconstruction
    rounded to bf16 is exact in range); every other linear is bf16.  bf16
    storage semantics throughout (mode "bf16").

    Reading for the MLP (the page names a proj and a gate module; the other
    block structure of block_forward is kept):
      u = h2 W_proj^T + b_proj;  t = h2 W_gate^T + b_gate  (both stored bf16)
      g = u * GELU_tanh(t)  (stored bf16);  y2 = g W_down^T + b_down
    """
    mode = "bf16"
    mx = mx or {}
    x = np.asarray(x, np.float64)
    T_q, D = x.shape
    H = D // HEAD_DIM
    m = _row_mod(mod, mod_of_seg, seg_len, T_q)
    shift1, scale1, gate1, shift2, scale2, gate2 = (m[:, i, :] for i in range(6))

    def lin(a, name):
        b = weights["b" + name[1:]]
        if name in mx:
            codes, scales = mx[name]
            return linear(a, round_bf16(mxfp4_decode(codes, scales)), b)
        if name in int8:
            qa, sa, za = quantize_rows_asym(a)
            qw, sw = quantize_rows(weights[name])
            return w8a8_linear_asym(qa, sa, za, qw, sw, b)
        return linear(a, weights[name], b)

    h = _store(adaln_modulate(x, shift1, scale1, ln_eps), mode)
    qk = _store(lin(h, "w_qk"), mode)
    v = _store(lin(h, "w_v"), mode).reshape(T_q, H, HEAD_DIM)
    q = qk[:, :D].reshape(T_q, H, HEAD_DIM)
    k = qk[:, D:].reshape(T_q, H, HEAD_DIM)
    q = _store(apply_rope(qk_rmsnorm(q, weights["g_q"], mode, qk_eps), cos, sin), mode)
    k = _store(apply_rope(qk_rmsnorm(k, weights["g_k"], mode, qk_eps), cos, sin), mode)
    if k_prefix is not None and len(k_prefix):
        k_all = np.concatenate([np.asarray(k_prefix, np.float64), k], axis=0)
        v_all = np.concatenate([np.asarray(v_prefix, np.float64), v], axis=0)
    else:
        k_all, v_all = k, v
    attend = attention_quantized if attn_quant else attention
    o = _store(attend(q, k_all, v_all, seg_len), mode).reshape(T_q, D)
    y = _store(lin(o, "w_o"), mode)
    x1 = _store(x + gate1 * y, mode)
    h2 = _store(adaln_modulate(x1, shift2, scale2, ln_eps), mode)
    u = _store(lin(h2, "w_proj"), mode)
    t = _store(lin(h2, "w_gate"), mode)
    g = _store(u * gelu_tanh(t), mode)
    y2 = _store(lin(g, "w_down"), mode)
    x2 = _store(x1 + gate2 * y2, mode)
    return {"x_out": x2, "k": k, "v": v, "q": q, "o": o, "u": u, "g": g, "x1": x1}


def block_forward_rows(x, mod, mod_of_seg, seg_len, cos, sin, weights, mode: str, rows,
                       k_prefix=None, v_prefix=None, qweights=None,
                       ln_eps: float = LN_EPS, qk_eps: float = QK_EPS) -> Dict[str, np.ndarray]:
    """``block_forward`` restricted to the output rows ``rows`` (indices into x).

    Keys and values are needed for every row, so the adaLN prologue and the QKV
    linear run on all rows; every later step runs on the requested rows only.
    Row-local steps give the same values as the full computation.
    """
    x = np.asarray(x, np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    T_q, D = x.shape
    H = D // HEAD_DIM
    if mode == "w8a8" and qweights is None:
        qweights = quantize_block_weights(weights)
    m = _row_mod(mod, mod_of_seg, seg_len, T_q)
    shift1, scale1, gate1, shift2, scale2, gate2 = (m[:, i, :] for i in range(6))
    h = _store(adaln_modulate(x, shift1, scale1, ln_eps), mode)
    kv = _store(_lin_cols(h, weights, qweights, mode, D, 3 * D), mode)
    k = _store(apply_rope(qk_rmsnorm(kv[:, :D].reshape(T_q, H, HEAD_DIM), weights["g_k"], mode, qk_eps),
                          cos, sin), mode)
    v = kv[:, D:].reshape(T_q, H, HEAD_DIM)
    qr = _store(_lin_cols(h[rows], weights, qweights, mode, 0, D), mode).reshape(len(rows), H, HEAD_DIM)
    qr = _store(apply_rope(qk_rmsnorm(qr, weights["g_q"], mode, qk_eps), cos[rows], sin[rows]), mode)
    if k_prefix is not None and len(k_prefix):
        k_all = np.concatenate([np.asarray(k_prefix, np.float64), k], axis=0)
        v_all = np.concatenate([np.asarray(v_prefix, np.float64), v], axis=0)
    else:
        k_all, v_all = k, v
    T_k = k_all.shape[0]
    allowed = allowed_mask(seg_len, T_q)[rows]
    scale = 1.0 / math.sqrt(HEAD_DIM)
    o = np.empty((len(rows), H, HEAD_DIM))
    for hd in range(H):
        sc = (qr[:, hd, :] @ k_all[:, hd, :].T) * scale
        sc = np.where(allowed, sc, -np.inf)
        sc = sc - sc.max(axis=1, keepdims=True)
        p = np.exp(sc)
        o[:, hd, :] = (p / p.sum(axis=1, keepdims=True)) @ v_all[:, hd, :]
    assert T_k == allowed.shape[1]
    o = _store(o, mode).reshape(len(rows), D)
    xr = x[rows]
    y = _store(_lin(o, "w_o", weights, qweights, mode), mode)
    x1 = _store(xr + gate1[rows] * y, mode)
    h2 = _store(adaln_modulate(x1, shift2[rows], scale2[rows], ln_eps), mode)
    u = _store(_lin(h2, "w_1", weights, qweights, mode), mode)
    g = _store(gelu_tanh(u), mode)
    y2 = _store(_lin(g, "w_2", weights, qweights, mode), mode)
    x2 = _store(x1 + gate2[rows] * y2, mode)
    return {"x_out": x2, "k": k, "v": v, "q": qr, "o": o}


def _lin_cols(a, weights, qweights, mode, c0, c1):
    """Columns [c0, c1) of the QKV linear."""
    b = weights["b_qkv"][c0:c1]
    if mode == "w8a8":
        qa, sa = quantize_rows(a)
        qw, sw = qweights["w_qkv"]
        return w8a8_linear(qa, sa, qw[c0:c1], sw[c0:c1], b)
    return linear(a, weights["w_qkv"][c0:c1], b)


# ----------------------------------------------------------------------------- one denoise step

def euler_update(latent, v, sigma: float, sigma_next: float) -> np.ndarray:
    """FlowMatch Euler step x + (sigma_next - sigma) * v  ([CoreAI, Graph contracts])."""
    return np.asarray(latent, np.float64) + (float(sigma_next) - float(sigma)) * np.asarray(v, np.float64)


def dit_step(step_in: Dict[str, np.ndarray], blocks, mod, mod_of_seg, seg_len, cos, sin, mode: str):
    """One denoise step: DiT head, the block stack, DiT tail, Euler update.

    [CoreAI, Graph contracts]: the DiT takes the packed latent [N, 64] and text
    features [L, D] and returns a velocity [N, 64]; the sampler then makes one
    Euler update.  Reading for the head and tail, which the pages do not spell
    out: img_in = Linear(64 -> D), txt_in = Linear(D -> D); tail = LN with a
    (shift, scale) modulation pair, then proj_out = Linear(D -> 64) on the image
    rows.  ``blocks`` yields (weights, qweights-or-None) per block.
    """
    lat = np.asarray(step_in["latent"], np.float64)
    x_img = _store(linear(_store(lat, mode), step_in["w_img_in"], step_in["b_img_in"]), mode)
    x_txt = _store(linear(step_in["txt_feats"], step_in["w_txt_in"], step_in["b_txt_in"]), mode)
    x = np.concatenate([x_txt, x_img], axis=0)
    for weights, qweights in blocks:
        x = block_forward(x, mod, mod_of_seg, seg_len, cos, sin, weights, mode, qweights=qweights)["x_out"]
    L = x_txt.shape[0]
    mf = np.asarray(step_in["mod_final"], np.float64)[0]
    hf = _store(adaln_modulate(x[L:], mf[0], mf[1]), mode)
    vel = _store(linear(hf, step_in["w_proj_out"], step_in["b_proj_out"]), mode)
    return {"latent_next": euler_update(lat, vel, step_in["sigma"], step_in["sigma_next"]),
            "vel": vel, "x_blocks": x}


def denoise_loop(loop_in: Dict[str, np.ndarray], blocks, mod_of_seg, seg_len, cos, sin, mode: str,
                 cache_prefix: bool = False, quant_attn_from: Optional[int] = None) -> Dict[str, np.ndarray]:
    """The sampling loop around the DiT ([CoreAI], Graph contracts): each step
    maps the target latent (with the text features, and for editing the
    reference latents) to a velocity and makes one Euler update of the target
    latent, sigma_i -> sigma_{i+1}.

    loop_in: latent [N, C] fp32 (target), txt_feats [L, C_txt], ref_latent
    [R, C] (R may be 0), the head/tail weights of ``dit_step``, mods
    [S, n_mod, 6, D], mod_finals [S, 2, D], sigmas [S + 1].  The sequence is
    [text | references | target]; seg_len covers it and cos/sin [T_k, 64] are
    the tables of all its rows.  ``blocks`` yields (weights, qweights-or-None).

    cache_prefix: steps after the first compute only the target rows and take
    the text/reference K/V kept from the first step ([Paiton], prefix reuse).
    When the prefix segments use a modulation set that is the same at every
    step this changes nothing (prefix rows never attend to target rows); the
    default recomputes every row at every step.

    quant_attn_from: steps with index >= this run the attention on int8/fp8
    operands ([Paiton, Runtime precision and quality]: the first steps keep the
    original precision); None keeps every step unquantized.
    """
    lat = np.asarray(loop_in["latent"], np.float64).copy()
    txt = np.asarray(loop_in["txt_feats"], np.float64)
    ref = np.asarray(loop_in["ref_latent"], np.float64)
    L, R, N = txt.shape[0], ref.shape[0], lat.shape[0]
    T_k = L + R + N
    sig = [float(v) for v in loop_in["sigmas"]]
    blocks = list(blocks)
    caches = None
    vel = None
    for i in range(len(sig) - 1):
        mod = loop_in["mods"][i]
        full = not (cache_prefix and caches is not None)
        x_tgt = _store(linear(_store(lat, mode), loop_in["w_img_in"], loop_in["b_img_in"]), mode)
        if full:
            parts = []
            if L:
                parts.append(_store(linear(txt, loop_in["w_txt_in"], loop_in["b_txt_in"]), mode))
            if R:
                parts.append(_store(linear(_store(ref, mode), loop_in["w_img_in"], loop_in["b_img_in"]), mode))
            x = np.concatenate(parts + [x_tgt], axis=0)
            c, s = cos, sin
        else:
            x = x_tgt
            c, s = cos[T_k - N:], sin[T_k - N:]
        kept = []
        for b, (weights, qweights) in enumerate(blocks):
            kp, vp = (None, None) if full else caches[b]
            out = block_forward(x, mod, mod_of_seg, seg_len, c, s, weights, mode,
                                k_prefix=kp, v_prefix=vp, qweights=qweights,
                                attn_quant=quant_attn_from is not None and i >= quant_attn_from)
            if full:
                kept.append((out["k"][:T_k - N], out["v"][:T_k - N]))
            x = out["x_out"]
        if full:
            caches = kept
        mf = np.asarray(loop_in["mod_finals"][i], np.float64)
        hf = _store(adaln_modulate(x[x.shape[0] - N:], mf[0], mf[1]), mode)
        vel = _store(linear(hf, loop_in["w_proj_out"], loop_in["b_proj_out"]), mode)
        lat = euler_update(lat, vel, sig[i], sig[i + 1])
    return {"latent": lat, "vel": vel}


def rel_l2(y, y_ref) -> float:
    """||y - y_ref||_2 / ||y_ref||_2 over the whole tensor, in fp64."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    return float(np.linalg.norm((y - y_ref).ravel()) / np.linalg.norm(y_ref.ravel()))
