"""The C-ABI library loads, exports every symbol of include/dit.h, and rejects
invalid calls before any HIP call (CPU only: no compute is launched)."""
import ctypes
import os
import re

import pytest

import diffusion_transformer_text_qwen_amd as dq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "dit.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = dq.lib()
    names = _header_functions()
    assert len(names) >= 15, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dq.exported_symbols())
    assert lib.dit_abi_version() == 5


def test_status_strings():
    lib = dq.lib()
    for s in range(8):
        assert lib.dit_status_string(s)
    assert lib.dit_status_string(99) == b"unknown status"


NULL = None
S = None  # default stream; never used since every call below fails validation


def _err(code):
    return code, dq.lib().dit_last_error().decode()


def test_quantize_rows_validation():
    lib = dq.lib()
    assert lib.dit_quantize_rows(NULL, 7, 4, 64, 64, NULL, NULL, S) == 3          # dtype
    assert lib.dit_quantize_rows(NULL, dq.BF16, 4, 64, 32, NULL, NULL, S) == 2    # ldx < K
    assert lib.dit_quantize_rows(NULL, dq.BF16, 4, 60, 64, NULL, NULL, S) == 5    # K % 8
    assert lib.dit_quantize_rows(NULL, dq.BF16, 4, 65536, 65536, NULL, NULL, S) == 5
    assert lib.dit_quantize_rows(NULL, dq.BF16, 4, 64, 64, NULL, NULL, S) == 1    # NULL
    assert lib.dit_quantize_rows(16, dq.BF16, 4, 64, 64, 24, 32, S) == 4          # misaligned q
    assert lib.dit_quantize_rows(NULL, dq.BF16, 0, 64, 64, NULL, NULL, S) == 0    # empty: no-op


def test_linear_validation():
    lib = dq.lib()
    W = (NULL, 0)   # no workspace
    assert lib.w8a8_linear(16, 16, 4, 100, 16, 16, NULL, 64, 16, dq.BF16, 64, NULL, *W, S) == 5     # K % 128
    assert lib.w8a8_linear(16, 16, 4, 128, 16, 16, NULL, 60, 16, dq.BF16, 64, NULL, *W, S) == 5     # N % 16
    assert lib.w8a8_linear(16, 16, 4, 133248, 16, 16, NULL, 64, 16, dq.BF16, 64, NULL, *W, S) == 5  # int32 bound
    assert lib.w8a8_linear(16, 16, 4, 128, 16, 16, NULL, 64, 16, dq.I8, 64, NULL, *W, S) == 3
    assert lib.w8a8_linear(NULL, 16, 4, 128, 16, 16, NULL, 64, 16, dq.BF16, 64, NULL, *W, S) == 1
    assert lib.w8a8_linear(17, 16, 4, 128, 16, 16, NULL, 64, 16, dq.BF16, 64, NULL, *W, S) == 4
    assert lib.w8a8_linear(16, 16, 4, 128, 16, 16, NULL, 64, 16, dq.BF16, 32, NULL, *W, S) == 2     # ldy < N
    assert lib.w8a8_linear(16, 16, 4, 128, 16, 16, NULL, 64, 16, dq.BF16, 64, NULL, 256, 1024, S) == 6  # small ws
    assert lib.w8a8_linear(NULL, NULL, 0, 128, NULL, NULL, NULL, 64, NULL, dq.BF16, 64, NULL, *W, S) == 0
    assert lib.w8a8_linear_workspace_bytes() >= 64 << 20
    assert lib.bf16_linear(16, 4, 96, 96, 16, NULL, 64, 16, dq.BF16, 64, S) == 5
    assert lib.bf16_linear(16, 4, 64, 60, 16, NULL, 64, 16, dq.BF16, 64, S) == 2
    assert lib.f32_linear(16, 4, 20, 20, 16, NULL, 64, 16, 64, S) == 5


def _attn(dtype=dq.BF16, T_q=8, T_k=8, H=2, d=128, ld=256, segs=(3, 5), ptr=16):
    arr = (ctypes.c_int32 * len(segs))(*segs) if segs is not None else None
    return dq.lib().block_causal_attention(ptr, ptr, ptr, ptr, dtype, T_q, T_k, H, d, ld, ld, ld, ld,
                                           ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None,
                                           len(segs) if segs is not None else 1, 0.0, S)


def test_attention_validation():
    assert _attn(d=64) == 5
    assert _attn(dtype=dq.I8) == 3
    assert _attn(T_q=9) == 2                     # T_q > T_k
    assert _attn(segs=(3, 4)) == 2               # sum != T_k
    assert _attn(segs=None) == 1
    assert _attn(segs=tuple([1] * 8) + (0,) * 9, T_k=8) == 5   # 17 segments
    assert _attn(ld=200) == 2
    assert _attn(ld=260) == 4
    assert _attn(ptr=NULL) == 1
    assert _attn(ptr=24) == 4
    assert _attn(T_q=0, ptr=NULL) == 0           # empty query set: no-op


def test_rope_and_misc_validation():
    lib = dq.lib()
    g = (ctypes.c_int32 * 2)(8, 8)
    gp = ctypes.cast(g, ctypes.c_void_p)
    assert lib.dit_rope_tables(16, gp, 1, 0, 81, 10000.0, 16, 16, S) == 2      # past the end
    assert lib.dit_rope_tables(16, gp, 16, 0, 8, 10000.0, 16, 16, S) == 5
    assert lib.dit_rope_tables(16, None, 1, 0, 8, 10000.0, 16, 16, S) == 1
    assert lib.dit_rope_tables(16, gp, 1, 0, 8, 10000.0, NULL, NULL, S) == 1
    assert lib.dit_qk_norm_rope(16, dq.BF16, 4, 2, 16, 16, 16, 16, 1e-6, 16, 16, 100, 16, 256, S) == 2
    assert lib.dit_adaln_modulate(16, dq.BF16, 4, 300, 16, 16, 1e-6, 16, dq.BF16, NULL, NULL, S) == 5
    assert lib.dit_adaln_modulate(16, dq.BF16, 4, 512, 16, 16, 1e-6, 16, dq.F32, NULL, NULL, S) == 3
    assert lib.dit_euler_step(NULL, NULL, dq.F32, 10, 1.0, 0.5, S) == 1
    # h and codes together; neither is an error; misaligned h
    assert lib.dit_adaln_modulate(16, dq.BF16, 4, 512, 16, 16, 1e-6, NULL, dq.BF16, NULL, NULL, S) == 1
    assert lib.dit_adaln_modulate(16, dq.BF16, 4, 512, 16, 16, 1e-6, 24, dq.BF16, 16, 16, S) == 4
    assert lib.dit_adaln_modulate(16, dq.BF16, 4, 512, 16, 16, 1e-6, 16, dq.BF16, 16, NULL, S) == 1
    # adaLN with asymmetric codes: D range, NULL outputs, alignment of h and q
    assert lib.dit_adaln_modulate_asym(16, 4, 8192, 16, 16, 1e-6, 16, 16, 16, 16, S) == 5
    assert lib.dit_adaln_modulate_asym(16, 4, 300, 16, 16, 1e-6, 16, 16, 16, 16, S) == 5
    assert lib.dit_adaln_modulate_asym(16, 4, 512, 16, 16, 1e-6, 16, 16, 16, NULL, S) == 1
    assert lib.dit_adaln_modulate_asym(16, 4, 512, 16, 16, 1e-6, 24, 16, 16, 16, S) == 4
    assert lib.dit_adaln_modulate_asym(16, 4, 512, 16, 16, 1e-6, NULL, 20, 16, 16, S) == 4


def test_gelu_quantize_validation():
    lib = dq.lib()
    assert lib.dit_gelu_quantize_rows(16, 4, 64, 32, 16, 16, NULL, S) == 2       # ldu < K
    assert lib.dit_gelu_quantize_rows(16, 4, 60, 64, 16, 16, NULL, S) == 5       # K % 8
    assert lib.dit_gelu_quantize_rows(16, 4, 16392, 16392, 16, 16, NULL, S) == 5  # K > 16384
    assert lib.dit_gelu_quantize_rows(16, 4, 64, 64, NULL, 16, NULL, S) == 1
    assert lib.dit_gelu_quantize_rows(16, 4, 64, 64, 16, 16, 24, S) == 4         # misaligned g_out
    assert lib.dit_gelu_quantize_rows(NULL, 0, 64, 64, NULL, NULL, NULL, S) == 0


def test_qkv_linear_validation():
    lib = dq.lib()
    need = lib.dit_qkv_linear_workspace_bytes(4352, 32)
    assert need >= lib.w8a8_linear_workspace_bytes() + 4352 * 3 * 4096 * 2

    def call(mode=dq.MODE_W8A8, T=8, H=4, ws=256, wsb=1 << 40, ptr=256, scale=256):
        return lib.dit_qkv_linear(mode, ptr, scale, T, H, ptr, scale, NULL, ptr, ptr, ptr, ptr, 1e-6, ptr, ptr, ptr,
                                  ws, wsb, S)
    assert call(mode=dq.MODE_F32) == 3
    assert call(H=3) == 5                              # D % 256
    assert call(H=128) == 5                            # D > 8192
    assert call(ws=NULL) == 6
    assert call(wsb=1024) == 6
    assert call(ptr=NULL) == 1
    assert call(scale=NULL) == 1                       # W8A8 needs scales
    assert call(mode=dq.MODE_BF16, scale=NULL, ptr=264) == 4
    assert call(T=0) == 0


def _block_args(mode=dq.MODE_W8A8, D=512, H=4, F=2048, segs=(16, 64), T_q=80, mos=(0, 0), n_mod=1):
    cfg = dq.BlockConfig(mode, D, H, 128, F, 1e-6, 1e-6)
    w = dq.BlockWeightsC(**{n: 256 for n, _ in dq.BlockWeightsC._fields_})
    sarr = (ctypes.c_int32 * len(segs))(*segs)
    marr = (ctypes.c_int32 * len(mos))(*mos)
    io = dq.BlockIO(x=256, mod=256, n_mod=n_mod, mod_of_seg=ctypes.cast(marr, ctypes.c_void_p), cos_t=256,
                    sin_t=256, seg_len=ctypes.cast(sarr, ctypes.c_void_p), n_seg=len(segs), T_q=T_q,
                    T_k=sum(segs), k_cache=256, v_cache=256)
    return cfg, w, io, (sarr, marr)


def test_block_validation():
    lib = dq.lib()
    need = lib.dit_block_workspace_bytes(ctypes.byref(dq.BlockConfig(2, 4096, 32, 128, 16384, 1e-6, 1e-6)),
                                         17664, 17664)
    assert need > 17664 * (4096 * 6 + 16384 * 3)

    def call(cfg, w, io, ws=256, wsb=1 << 40):
        return lib.dit_block_forward(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(io), ws, wsb, S)

    cfg, w, io, keep = _block_args()
    cfg.head_dim = 64
    assert call(cfg, w, io) == 5
    cfg, w, io, keep = _block_args(D=640, H=4)
    assert call(cfg, w, io) == 2                       # D != H*128
    cfg, w, io, keep = _block_args(mode=7)
    assert call(cfg, w, io) == 3
    cfg, w, io, keep = _block_args(F=1000)
    assert call(cfg, w, io) == 5
    cfg, w, io, keep = _block_args(segs=(16, 60))
    assert call(cfg, w, io) == 2                       # T_q > T_k
    cfg, w, io, keep = _block_args(mos=(0, 1))
    assert call(cfg, w, io) == 2                       # mod set out of range
    cfg, w, io, keep = _block_args()
    w.s_o = None
    assert call(cfg, w, io) == 1                       # W8A8 without scales
    cfg, w, io, keep = _block_args()
    io.k_cache = None
    assert call(cfg, w, io) == 1
    cfg, w, io, keep = _block_args()
    assert call(cfg, w, io, ws=256, wsb=1024) == 6     # workspace too small
    # the kernels take T_k as a 32-bit count
    cfg, w, io, keep = _block_args(segs=(16, (1 << 31) - 16), T_q=80)
    assert call(cfg, w, io) == 5
    # int8/fp8 attention: H * ceil(T_k / 64) * 8192 (the K and V operand images)
    # must stay below 2^31 bytes (H = 32: T_k < 524288)
    cfg, w, io, keep = _block_args(D=4096, H=32, F=16384, segs=(16, 600000 - 16), T_q=80)
    cfg.attn_quant = 1
    assert call(cfg, w, io) == 5
    cfg, w, io, keep = _block_args()
    io.x = 264
    assert call(cfg, w, io) == 4
    cfg, w, io, keep = _block_args(T_q=0)
    assert call(cfg, w, io, ws=None, wsb=0) == 0       # nothing to compute


def _velocity_args(segs=(16, 16, 64), T_q=96, L_txt=16, R=16, N=64, mos=(0, 0, 1), n_mod=2):
    cfg = dq.BlockConfig(dq.MODE_W8A8, 512, 4, 128, 2048, 1e-6, 1e-6)
    w = dq.BlockWeightsC(**{n: 256 for n, _ in dq.BlockWeightsC._fields_})
    head = dq.HeadWeightsC(w_txt_in=256, b_txt_in=256, w_img_in=256, b_img_in=256, w_proj_out=256,
                           b_proj_out=256, C_txt=512, C_lat=64)
    sarr = (ctypes.c_int32 * len(segs))(*segs)
    marr = (ctypes.c_int32 * len(mos))(*mos)
    kc = (ctypes.c_void_p * 1)(256)
    vc = (ctypes.c_void_p * 1)(256)
    io = dq.VelocityIO(txt_feats=256, ref_latent=256, latent=256, L_txt=L_txt, R=R, N=N, mod=256, n_mod=n_mod,
                       mod_of_seg=ctypes.cast(marr, ctypes.c_void_p), mod_final=256, cos_t=256, sin_t=256,
                       seg_len=ctypes.cast(sarr, ctypes.c_void_p), n_seg=len(segs), T_q=T_q,
                       k_caches=ctypes.cast(kc, ctypes.c_void_p), v_caches=ctypes.cast(vc, ctypes.c_void_p), vel=256)
    return cfg, w, head, io, (sarr, marr, kc, vc)


def test_velocity_validation():
    """dit_velocity_forward rejects bad arguments before any HIP call."""
    lib = dq.lib()
    cfg = dq.BlockConfig(dq.MODE_W8A8, 512, 4, 128, 2048, 1e-6, 1e-6)
    need = lib.dit_velocity_workspace_bytes(ctypes.byref(cfg), 96, 96, 64, 64)
    assert need > lib.dit_block_workspace_bytes(ctypes.byref(cfg), 96, 96) + 96 * 512 * 2

    def call(cfg, w, head, io, ws=256, wsb=1 << 40):
        return lib.dit_velocity_forward(ctypes.byref(cfg), ctypes.byref(w), 1, ctypes.byref(head),
                                        ctypes.byref(io), ws, wsb, S)

    a = _velocity_args(T_q=80)
    assert call(*a[:4]) == 2                               # T_q neither T_k nor N
    a = _velocity_args(segs=(16, 16, 60))
    assert call(*a[:4]) == 2                               # seg_len does not add up to L_txt + R + N
    a = _velocity_args()
    a[2].C_lat = 48
    assert call(*a[:4]) == 5                               # C_lat not a multiple of 64
    a = _velocity_args()
    a[3].txt_feats = None
    assert call(*a[:4]) == 1                               # text rows without features
    a = _velocity_args(T_q=64)
    a[3].txt_feats = None
    a[3].ref_latent = None
    assert call(*a[:4], ws=256, wsb=16) == 6               # cached step: prefix inputs not needed, workspace small
    a = _velocity_args()
    a[3].vel = 264
    assert call(*a[:4]) == 4                               # misaligned output
    a = _velocity_args(mos=(0, 0, 2))
    assert call(*a[:4]) == 2                               # modulation set out of range


def test_attn_q8_validation():
    """Layout of the int8/fp8 attention buffer and the argument checks (no HIP call)."""
    lib = dq.lib()
    n, off = dq.attn_q8_layout(200, 330, 3)
    nt = (330 + 63) // 64
    sizes = {"q8": 3 * 200 * 128, "q_scale": 3 * 200 * 4, "k8": 3 * nt * 8192, "k_scale": 3 * nt * 4,
             "v8": 3 * nt * 8192, "v_scale": 3 * 128 * 4, "v_amax": 3 * 128 * 4}
    order = list(dq.Q8_PARTS)
    for i, name in enumerate(order):
        assert off[name] % 256 == 0
        end = off[name] + sizes[name]
        assert end <= (off[order[i + 1]] if i + 1 < len(order) else n)
    assert lib.dit_attn_q8_bytes(5, 4, 1, None) == 0          # T_q > T_k
    assert lib.dit_attn_q8_bytes(4, 4, 0, None) == 0          # H < 1
    q = 256
    assert lib.dit_attn_quantize(q, q, q, 10, 20, 0, 128, 128, 128, q, 1 << 30, S) == 2      # H
    assert lib.dit_attn_quantize(q, q, q, 10, 20, 1, 64, 128, 128, q, 1 << 30, S) == 2       # ldq < H*128
    assert lib.dit_attn_quantize(q, q, q, 10, 20, 1, 132, 128, 128, q, 1 << 30, S) == 4      # ldq % 8
    assert lib.dit_attn_quantize(q, q, q, 10, 20, 1, 128, 128, 128, q, 16, S) == 6           # buffer small
    assert lib.dit_attn_quantize(q, q, q, 10, 20, 1, 128, 128, 128, None, 1 << 30, S) == 6   # buffer NULL
    assert lib.dit_attn_quantize(q, q, 264, 10, 20, 1, 128, 128, 128, q, 1 << 30, S) == 4    # v misaligned
    segs = (ctypes.c_int32 * 2)(8, 12)
    sp = ctypes.cast(segs, ctypes.c_void_p)
    assert lib.block_causal_attention_q8(q, 10, 21, 1, q, 128, sp, 2, 0.0, S) == 2          # seg sum != T_k
    assert lib.block_causal_attention_q8(q, 10, 20, 1, q, 120, sp, 2, 0.0, S) == 2          # ldo < H*128
    assert lib.block_causal_attention_q8(None, 10, 20, 1, q, 128, sp, 2, 0.0, S) == 1       # buffer NULL
    assert lib.block_causal_attention_q8(q, 0, 20, 1, None, 128, sp, 2, 0.0, S) == 0        # T_q == 0: no-op
    cfg = dq.BlockConfig(dq.MODE_F32, 512, 4, 128, 2048, 1e-6, 1e-6, 1)
    assert lib.dit_block_workspace_bytes(ctypes.byref(cfg), 96, 96) > 0


def test_gated_validation():
    """Asymmetric quantization, column sums, the zero-point linear and the gated
    block reject bad arguments before any HIP call."""
    lib = dq.lib()
    p = 256
    assert lib.dit_quantize_rows_asym(p, 9, 4, 64, 64, p, p, p, S) == 3              # dtype
    assert lib.dit_quantize_rows_asym(p, 1, 4, 60, 64, p, p, p, S) == 5              # K % 8
    assert lib.dit_quantize_rows_asym(p, 1, 4, 64, 64, p, p, None, S) == 1           # zero NULL
    assert lib.dit_quantize_rows_asym(p, 1, 0, 64, 64, None, None, None, S) == 0     # M == 0: no-op
    assert lib.dit_int8_colsum(p, 8, 40, p, S) == 5                                  # K % 16
    assert lib.dit_int8_colsum(264, 8, 64, p, S) == 4                                # misaligned w
    assert lib.w8a8_linear_asym(p, p, p, 4, 128, p, p, None, None, 16, p, 1, 16, None, 0, S) == 1   # no w_sum
    assert lib.w8a8_linear_asym(p, p, p, 4, 128 * 1024, p, p, p, None, 16, p, 1, 16, None, 0, S) == 5  # K bound
    cfg = dq.BlockConfig(dq.MODE_W8A8, 512, 4, 128, 1536, 1e-6, 1e-6, 0)
    lin = dq.LinearC(w=p, s=None, wsum=None, b=p)
    w = dq.GatedBlockWeightsC(qk=lin, v=lin, o=lin, proj=lin, gate=lin, down=lin, g_q=p, g_k=p)
    segs = (ctypes.c_int32 * 2)(24, 64)
    mos = (ctypes.c_int32 * 2)(0, 0)
    io = dq.BlockIO(x=p, mod=p, n_mod=1, mod_of_seg=ctypes.cast(mos, ctypes.c_void_p), cos_t=p, sin_t=p,
                    seg_len=ctypes.cast(segs, ctypes.c_void_p), n_seg=2, T_q=88, T_k=88, k_cache=p, v_cache=p)
    call = lambda c, ww, wsb=1 << 40: lib.dit_block_forward_gated(ctypes.byref(c), ctypes.byref(ww), ctypes.byref(io),
                                                                 p, wsb, S)
    assert call(cfg, w) == 3                                       # activations must be bf16 (mode BF16)
    cfg.mode = dq.MODE_BF16
    w.proj = dq.LinearC(w=p, s=p, wsum=None, b=p)
    assert call(cfg, w) == 1                                       # int8 linear without its row sums
    w.proj = dq.LinearC(w=264, s=None, wsum=None, b=p)
    assert call(cfg, w) == 4                                       # misaligned weights
    w.proj = lin
    assert call(cfg, w, wsb=64) == 6                               # workspace too small
    assert lib.dit_gated_block_workspace_bytes(ctypes.byref(cfg), 88, 88) > 0


def test_mxfp4_validation():
    lib = dq.lib()
    p = 256
    assert lib.dit_mxfp4_expand(p, p, 4, 48, p, S) == 5                      # K % 32
    assert lib.dit_mxfp4_expand(p, None, 4, 64, p, S) == 1                   # scales NULL
    assert lib.dit_mxfp4_expand(264, p, 4, 64, p, S) == 4                    # codes misaligned
    assert lib.dit_mxfp4_expand(p, p, 0, 64, p, S) == 0                      # N == 0: no-op
    assert lib.mxfp4_linear_workspace_bytes(16, 64) == 16 * 64 * 2
    assert lib.mxfp4_linear(p, 8, 64, 64, p, p, None, 16, p, 1, 16, p, 16, S) == 6      # workspace small
    assert lib.mxfp4_linear(p, 8, 96, 96, p, p, None, 16, p, 1, 16, p, 1 << 20, S) == 5  # K % 64
    assert lib.mxfp4_linear(p, 8, 64, 64, p, p, None, 16, p, 7, 16, p, 1 << 20, S) == 3  # y dtype
