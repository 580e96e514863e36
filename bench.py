"""Throughput of the single-stream DiT block path on one MI355X.

Default workload (timed step): one denoise step of the 1024x1024 generation,
i.e. 32 W8A8 blocks over [256 text | 4096 image] tokens (D 4096, 32 heads x 128,
MLP 16384) plus the DiT head (img_in, txt_in), tail (final adaLN, proj_out) and
the FlowMatch Euler update of the 4096 x 64 latent.  Reported value: DiT-block
tokens/s = 32 * 4352 block rows / step time.

Also measured (reported under "denoise_loop_1024px"): the whole 40-step loop of
the same generation, eager and with one DiT evaluation captured in a HIP graph
and replayed (Euler updates between replays).

Also measured (reported under "edit_2048px"): one block of the 2048x2048 edit
workload, [256 text | 1024 reference | 16384 target], uncached step (17,664
rows) and the cached step that reuses the prefix K/V (16,384 rows), the latter
also with the int8/fp8 attention.

Also measured (reported under "gated_recipe_1024px"): one gated-MLP block
(F 12288) over the same tokens, all-bf16, with the FlagOS page's W8A8 scope
(Q/K, proj and gate int8 with asymmetric per-token activations), and with all
six linears stored as MXFP4 (decoded to bf16 in the GEMM's operand staging,
bf16 arithmetic).

Also measured (reported under "small_blocks"): one block of the 256x256
generation in bf16 ([64 text | 256 image] tokens) and one of the 512x512
generation in W8A8 ([128 text | 1024 image] tokens).

Also measured (reported under "attn_int8_fp8_1024px"): the same step as the
timed one with the int8 Q K^T / fp8 P V attention (the pages' later denoising
steps), and the 40-step loop with the first 7 steps bf16 attention, the rest
int8/fp8 ("denoise_loop_1024px", key "graph_sched_ms").

Inputs are seeded synthetic tensors (ditsynth); the path runs entirely in the
HIP library through its C ABI.  value / ms_per_step come from K timed steps
without instrumentation; per-launch kernel times (roofline, kernels) from HIP
events the library records around each launch during K more timed steps
(ms_per_step_profiled: their step time).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-edit]
  python bench.py --copy-probe MIB   # plain bf16 copy of MIB MiB, for HBM counter calibration

roofline.traffic: bytes per int8 GEMM launch site from rocprofv3 FETCH_SIZE and
WRITE_SIZE passes over this script, each divided by what the same counter reads
per byte of the --copy-probe copy (profiles/gemm_w8a8_1024px_traffic.json).
These counters count L2 misses to the data fabric (part of which the memory-side
cache serves), so the figure bounds HBM bytes from above.  It is null when
gemm.hip no longer matches the hash recorded with the counters.  The adaLN and
quantization kernels' entries in "kernels" carry the same counters' bytes
(profiles/hbm_kernels_1024px_traffic.json) next to their algorithmic bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DiT-block tokens/s at 4096/16384 img tokens; int8 GEMM & attn % of MFMA peak"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, published (5.0 POP/s)
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 (and int8) MFMA, published (5.0 PFLOP/s)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published (8 TB/s)
GEMM_SITES = ("qkv_gemm", "out_gemm", "up_gemm", "down_gemm")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_ops(T, D, F):
    """Algorithmic int8 ops of the four linears of one block: 2*T*(3D*D + D*D + F*D + D*F)."""
    return {"qkv_gemm": 2 * T * 3 * D * D, "out_gemm": 2 * T * D * D, "up_gemm": 2 * T * F * D,
            "down_gemm": 2 * T * D * F}


def attn_pairs(seg_len, T_q):
    """Allowed (query, key) pairs: a query of segment s sees keys [0, end(s))."""
    ends, acc = [], 0
    for n in seg_len:
        acc += n
        ends.append(acc)
    T_k = acc
    pairs, start = 0, 0
    for n, e in zip(seg_len, ends):
        lo = max(start, T_k - T_q)
        if e > lo:
            pairs += (e - lo) * e
        start = e
    return pairs


def hbm_bytes(T, D, F):
    """Algorithmic HBM bytes of the HBM-bound launches of one W8A8 block."""
    return {
        "adaln1": T * (2 * D + D + 4),          # bf16 x in, int8 codes + scale out
        "adaln2": T * (2 * D + D + 4),
        "qk_norm_rope": T * (3 * D * 2 + 3 * D * 2 + 64 * 8),   # qkv in; q, k, v out; cos/sin
        "quant_o": T * (2 * D + D + 4),
        "quant_g": T * (2 * F + F + 4),
    }


def gemm_traffic():
    """Counter-derived HBM bytes per int8 GEMM launch, or None if stale/absent."""
    path = os.path.join(ROOT, "profiles", "gemm_w8a8_1024px_traffic.json")
    src = os.path.join(ROOT, "diffusion_transformer_text_qwen_amd", "csrc", "gemm.hip")
    try:
        with open(path) as f:
            t = json.load(f)
        with open(src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if t.get("gemm_source_sha256") != sha:
        return None
    fetch = t["fetch_kib_per_launch"] * 1024 / t["copy_fetch_per_byte"]
    write = t["write_kib_per_launch"] * 1024 / t["copy_write_per_byte"]
    return int(fetch + write)


def hbm_kernel_traffic():
    """Counter-derived bytes (read + written) per dispatch of the adaLN and row
    quantization kernels ({site: bytes}), or {} if stale/absent."""
    path = os.path.join(ROOT, "profiles", "hbm_kernels_1024px_traffic.json")
    src = os.path.join(ROOT, "diffusion_transformer_text_qwen_amd", "csrc", "elementwise.hip")
    try:
        with open(path) as f:
            t = json.load(f)
        with open(src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return {}
    if t.get("elementwise_source_sha256") != sha:
        return {}
    k = t["kernels"]
    by = {name: v["bytes_read"] + v["bytes_written"] for name, v in k.items()}
    return {"adaln1": by["adaln"], "adaln2": by["adaln"], "quant_o": by["quant_o"], "quant_g": by["quant_g"]}


def copy_probe(mib, dq, torch):
    """dit_cast bf16 -> bf16 over mib MiB: reads and writes exactly 2n bytes."""
    n = mib * (1 << 20) // 2
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        dq.cast(x, y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe": {"dispatches": 5, "bytes_read_per_dispatch": 2 * n,
                                     "bytes_written_per_dispatch": 2 * n}}), flush=True)


def counter_summary(root):
    """Per kernel: dispatch count and the mean per dispatch of every counter in
    the rocprofv3 --pmc csv output under root (one JSON line per kernel)."""
    import csv
    import glob
    agg, ids = {}, {}
    for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                k = r["Kernel_Name"]
                agg.setdefault(k, {}).setdefault(r["Counter_Name"], 0.0)
                agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
                ids.setdefault(k, set()).add(r["Dispatch_Id"])
    for k in sorted(agg, key=lambda k: -len(ids[k])):
        n = len(ids[k])
        print(json.dumps({"kernel": k, "dispatches": n,
                          "mean": {c: v / n for c, v in sorted(agg[k].items())}}))


def site_report(prof, per_block_ops, n_blocks_timed, peak, unit):
    out = {}
    for site, ops in per_block_ops.items():
        p = prof.get(site, {"ms": 0.0, "count": 0})
        if p["count"] == 0 or p["ms"] <= 0:
            continue
        avg_ms = p["ms"] / p["count"]
        rate = ops / (avg_ms * 1e-3) / 1e12 if unit != "GB/s" else ops / (avg_ms * 1e-3) / 1e9
        out[site] = {"avg_us": round(avg_ms * 1e3, 2), "count": p["count"], unit: round(rate, 1),
                     "frac_peak": round(rate / peak, 4)}
    return out


def run_stack(args, dq, torch, ditsynth):
    w = ditsynth.workload(3)
    D, H, F, T, L = w.D, w.H, w.F, w.T, w.text
    N = w.seg_len[-1]
    dev = "cuda"
    t0 = time.time()
    blocks = []
    for b in range(w.n_blocks):
        t = {}
        for name, a in ditsynth.device_block_weights(w, b, dev):
            if name.startswith("w_"):
                q = torch.empty(a.shape, dtype=torch.int8, device=dev)
                s = torch.empty(a.shape[0], dtype=torch.float32, device=dev)
                dq.quantize_rows(a, q, s)
                t[name] = q
                t["s" + name[1:]] = s
            else:
                t[name] = a
            del a
        blocks.append(dq.BlockWeights.from_device(t, "w8a8"))
    si = ditsynth.device_step_inputs(w, dev)
    torch.cuda.synchronize()
    log(f"stack weights + inputs ready in {time.time() - t0:.1f}s")
    cfg = dq.block_config("w8a8", D, H, F)
    cos = torch.empty((T, 64), dtype=torch.float32, device=dev)
    sin = torch.empty((T, 64), dtype=torch.float32, device=dev)
    dq.rope_tables(L, w.images, 0, T, cos, sin)
    from diffusion_transformer_text_qwen_amd.loop import DenoiseLoop
    head = dq.HeadWeights({"w_txt_in": si["w_txt_in"].to(torch.bfloat16), "b_txt_in": si["b_txt_in"],
                           "w_img_in": si["w_img_in"].to(torch.bfloat16), "b_img_in": si["b_img_in"],
                           "w_proj_out": si["w_proj_out"].to(torch.bfloat16), "b_proj_out": si["b_proj_out"]})
    txt_b = si["txt_feats"].to(torch.bfloat16)
    loop = DenoiseLoop(cfg, blocks, head, w.seg_len, [0] * len(w.seg_len), L, cos, sin, n_mod=1)
    loop.mod.copy_(si["mod"][0:1])
    loop.mod_final.copy_(si["mod_final"][0])
    lat = si["latent"].clone()
    sigma, sigma_next = 1.0, 1.0 - 0.98 / 39.0

    def step(quant=False):
        loop.velocity(lat, txt_b, quant=quant)
        dq.euler_step(lat, loop.vel, sigma, sigma_next)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ok = bool(torch.isfinite(loop.vel.float()).all().item()) and bool(torch.isfinite(lat).all().item())
    # timed steps (no per-kernel events: they add ~4% per step)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    # the same steps again with HIP events around every launch (per-kernel times)
    dq.profile_begin(args.steps * w.n_blocks * 10 + 16)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    prof = dq.profile_end()
    ms_prof = ev0.elapsed_time(ev1) / args.steps
    # the same step with the int8/fp8 attention
    for _ in range(args.warmup):
        step(True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step(True)
    ev1.record()
    torch.cuda.synchronize()
    ms_q = ev0.elapsed_time(ev1) / args.steps
    dq.profile_begin(args.steps * w.n_blocks * 12 + 16)
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    prof_q = dq.profile_end()
    n_timed = args.steps * w.n_blocks
    att = prof_q["attention"]
    att_us = att["ms"] / att["count"] * 1e3
    att_tf = 4 * D * attn_pairs(w.seg_len, T) / (att_us * 1e-6) / 1e12
    quant_q = {"ms_per_step": round(ms_q, 3), "block_tokens_per_s": round(w.n_blocks * T / (ms_q * 1e-3), 1),
               "finite": bool(torch.isfinite(lat).all().item()),
               "attention_avg_us": round(att_us, 2), "attention_tflops": round(att_tf, 1),
               "attention_frac_fp8_peak": round(att_tf / PEAK_FP8_TFLOPS, 4),
               "attn_quant_avg_us": round(prof_q["attn_quant"]["ms"] / prof_q["attn_quant"]["count"] * 1e3, 2),
               "block_ms_sum_of_launches": round(sum(p["ms"] for p in prof_q.values()) / n_timed, 4)}
    log(f"int8/fp8 attention step: {quant_q}")
    res_loop = None
    if args.loop_steps:
        res_loop = run_loop(args, torch, ditsynth, w, loop, si["latent"], txt_b, None)
    return w, ms, ms_prof, prof, ok, res_loop, quant_q


def run_loop(args, torch, ditsynth, w, loop, latent0, txt, ref):
    """The whole denoise loop (args.loop_steps steps of the 40-step schedule),
    eager and with one velocity evaluation captured in a HIP graph and replayed."""
    steps = args.loop_steps
    li = ditsynth.device_loop_inputs(w, steps)
    cache = len(w.images) > 1
    res = {"steps": steps, "prefix_cached": cache}
    for label, graph, qfrom in (("eager", False, None), ("graph", True, None), ("graph_sched", True, 7)):
        lat = latent0.clone()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        loop.run(lat, txt, ref, li["mods"], li["mod_finals"], li["sigmas"], cache_prefix=cache, graph=graph,
                 quant_attn_from=qfrom)
        e1.record()
        torch.cuda.synchronize()
        res[f"{label}_ms"] = round(e0.elapsed_time(e1), 2)
        res[f"{label}_finite"] = bool(torch.isfinite(lat).all().item())
    rows = w.T + (steps - 1) * (w.seg_len[-1] if cache else w.T)
    best = min(res["graph_ms"], res["eager_ms"])
    res["block_tokens_per_s"] = round(w.n_blocks * rows / (best * 1e-3), 1)
    res["ms_per_step"] = round(best / steps, 3)
    log(f"loop: {res}")
    return res


def run_edit(args, dq, torch, ditsynth, reps):
    """One block of the 2048^2 edit workload: uncached step 1, cached step 2."""
    w = ditsynth.workload(4)
    D, H, F, T, L = w.D, w.H, w.F, w.T, w.text
    P = w.prefix_len
    dev = "cuda"
    t = {}
    for name, a in ditsynth.device_block_weights(w, 0, dev):
        if name.startswith("w_"):
            q = torch.empty(a.shape, dtype=torch.int8, device=dev)
            s = torch.empty(a.shape[0], dtype=torch.float32, device=dev)
            dq.quantize_rows(a, q, s)
            t[name], t["s" + name[1:]] = q, s
        else:
            t[name] = a
    bw = dq.BlockWeights.from_device(t, "w8a8")
    si = ditsynth.device_step_inputs(w, dev)
    cfg = dq.block_config("w8a8", D, H, F)
    cos = torch.empty((T, 64), dtype=torch.float32, device=dev)
    sin = torch.empty((T, 64), dtype=torch.float32, device=dev)
    dq.rope_tables(L, w.images, 0, T, cos, sin)
    kc = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    cfg_q = dq.block_config("w8a8", D, H, F, attn_quant=True)
    ws = torch.empty(dq.workspace_bytes(cfg_q, T, T), dtype=torch.uint8, device=dev)
    mod = si["mod"]
    x1 = torch.cat([si["x_prefix"], si["x_target"][0]]).to(torch.bfloat16)
    x2 = si["x_target"][1].to(torch.bfloat16)
    xa = torch.empty_like(x1)
    xb = torch.empty_like(x2)
    mos1 = [0, 0, 1]
    mos2 = [0, 0, 2]
    res = {}
    for label, src, dst, mos, r0, c in (("uncached", x1, xa, mos1, 0, cfg), ("cached", x2, xb, mos2, P, cfg),
                                        ("cached_attn_int8_fp8", x2, xb, mos2, P, cfg_q)):
        def call():
            dst.copy_(src)
            dq.block_forward(c, bw, dst, mod, mos, cos[r0:], sin[r0:], w.seg_len, kc, vc, ws)
        call()
        torch.cuda.synchronize()
        dq.profile_begin(reps * 10 + 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        prof = dq.profile_end()
        T_q = T - r0
        blk_ms = sum(p["ms"] for p in prof.values()) / reps
        att = prof["attention"]
        att_flops = 4 * D * attn_pairs(w.seg_len, T_q)
        att_tf = att_flops / (att["ms"] / att["count"] * 1e-3) / 1e12
        gops = sum(gemm_ops(T_q, D, F).values())
        gms = sum(prof[s]["ms"] for s in GEMM_SITES) / reps
        if label.endswith("int8_fp8"):
            res[label] = {"rows": T_q, "block_ms": round(blk_ms, 3),
                          "block_tokens_per_s": round(T_q / (blk_ms * 1e-3), 1),
                          "attention_us": round(att["ms"] / att["count"] * 1e3, 1),
                          "attention_tflops": round(att_tf, 1),
                          "attn_quant_us": round(prof["attn_quant"]["ms"] / prof["attn_quant"]["count"] * 1e3, 1)}
            continue
        res[label] = {
            "rows": T_q, "block_ms": round(blk_ms, 3),
            "block_tokens_per_s": round(T_q / (blk_ms * 1e-3), 1),
            "wall_ms_incl_copy": round(e0.elapsed_time(e1) / reps, 3),
            "attention_tflops": round(att_tf, 1), "attention_frac_bf16_peak": round(att_tf / PEAK_BF16_TFLOPS, 4),
            "int8_gemm_tops": round(gops / (gms * 1e-3) / 1e12, 1),
            "int8_gemm_frac_peak": round(gops / (gms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
        }
    return res


def run_small(args, dq, torch, ditsynth, reps):
    """One block each of the 256^2 (bf16) and 512^2 (W8A8) generations."""
    dev = "cuda"
    res = {}
    for idx in (1, 2):
        w = ditsynth.workload(idx)
        D, H, F, T, L = w.D, w.H, w.F, w.T, w.text
        t = {}
        for name, a in ditsynth.device_block_weights(w, 0, dev):
            if name.startswith("w_") and w.mode == "w8a8":
                q = torch.empty(a.shape, dtype=torch.int8, device=dev)
                s = torch.empty(a.shape[0], dtype=torch.float32, device=dev)
                dq.quantize_rows(a, q, s)
                t[name], t["s" + name[1:]] = q, s
            elif name.startswith("w_"):
                t[name] = a.to(torch.bfloat16).contiguous()
            else:
                t[name] = a
        bw = dq.BlockWeights.from_device(t, w.mode)
        cfg = dq.block_config(w.mode, D, H, F)
        g = torch.Generator(device=dev)
        g.manual_seed(idx)
        x0 = torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16)
        mod = (torch.randn((1, 6, D), generator=g, device=dev) * 0.1).contiguous()
        cos = torch.empty((T, 64), dtype=torch.float32, device=dev)
        sin = torch.empty((T, 64), dtype=torch.float32, device=dev)
        dq.rope_tables(L, w.images, 0, T, cos, sin)
        kc = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        ws = torch.empty(dq.workspace_bytes(cfg, T, T), dtype=torch.uint8, device=dev)
        x = torch.empty_like(x0)

        def call():
            x.copy_(x0)
            dq.block_forward(cfg, bw, x, mod, [0] * len(w.seg_len), cos, sin, w.seg_len, kc, vc, ws)

        call()
        torch.cuda.synchronize()
        dq.profile_begin(reps * 10 + 4)
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        prof = dq.profile_end()
        blk_ms = sum(p["ms"] for p in prof.values()) / reps
        att = prof["attention"]
        att_tf = 4 * D * attn_pairs(w.seg_len, T) / (att["ms"] / att["count"] * 1e-3) / 1e12
        gops = sum(gemm_ops(T, D, F).values())
        g_rate = gops / (sum(prof[s]["ms"] for s in GEMM_SITES) / reps * 1e-3) / 1e12
        peak = PEAK_INT8_TOPS if w.mode == "w8a8" else PEAK_BF16_TFLOPS
        res[w.name] = {"rows": T, "mode": w.mode, "block_ms": round(blk_ms, 3),
                       "block_tokens_per_s": round(T / (blk_ms * 1e-3), 1),
                       "gemm_rate": round(g_rate, 1), "gemm_unit": "TOPS" if w.mode == "w8a8" else "TFLOPS",
                       "gemm_frac_peak": round(g_rate / peak, 4),
                       "attention_tflops": round(att_tf, 1),
                       "finite": bool(torch.isfinite(x.float()).all().item())}
        del bw, t, ws, kc, vc
    return res


def run_gated(args, dq, torch, ditsynth, reps):
    """One gated-MLP block (F = 12288) over the 1024^2 token layout: all linears
    bf16, and the FlagOS page's W8A8 scope (Q/K, proj, gate int8 with asymmetric
    per-token activations; V, out, down bf16)."""
    w = ditsynth.workload(3)
    D, H, T, F = w.D, w.H, w.T, 12288
    dev = "cuda"
    arrays = ditsynth.device_gated_block_weights(w, 0, F, dev)
    si = ditsynth.device_step_inputs(w, dev)
    x0 = torch.randn((T, D), generator=ditsynth.device_generator(w, 3000), device=dev).to(torch.bfloat16)
    cos = torch.empty((T, 64), dtype=torch.float32, device=dev)
    sin = torch.empty((T, 64), dtype=torch.float32, device=dev)
    dq.rope_tables(w.text, w.images, 0, T, cos, sin)
    kc = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    x = torch.empty_like(x0)
    mod = si["mod"][0:1].contiguous()
    res = {"rows": T, "F": F}
    shapes = {"qk": (2 * D, D), "v": (D, D), "o": (D, D), "proj": (F, D), "gate": (F, D), "down": (D, F)}
    mx = {n: ditsynth.mxfp4_weights(*shp, seed=90 + i) for i, (n, shp) in enumerate(shapes.items())}
    for label, int8, aq, mxw in (("bf16", (), False, None), ("recipe_w8a8", ("qk", "proj", "gate"), False, None),
                                 ("recipe_w8a8_attn_int8_fp8", ("qk", "proj", "gate"), True, None),
                                 ("mxfp4_weights", (), False, mx)):
        cfg = dq.block_config("bf16", D, H, F, attn_quant=aq)
        gw = dq.GatedBlockWeights(arrays, int8, mx=mxw)
        ws = torch.empty(dq.gated_workspace_bytes(cfg, T, T), dtype=torch.uint8, device=dev)

        def call():
            x.copy_(x0)
            dq.block_forward_gated(cfg, gw, x, mod, [0] * len(w.seg_len), cos, sin, w.seg_len, kc, vc, ws)
        call()
        torch.cuda.synchronize()
        dq.profile_begin(reps * 16 + 4)
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        prof = dq.profile_end()
        blk_ms = sum(p["ms"] for p in prof.values()) / reps
        res[label] = {"block_ms": round(blk_ms, 3), "block_tokens_per_s": round(T / (blk_ms * 1e-3), 1),
                      "finite": bool(torch.isfinite(x.float()).all().item()),
                      "sites_us": {k: round(p["ms"] / reps * 1e3, 1) for k, p in prof.items() if p["count"]}}
        del gw, ws
    log(f"gated block: {res}")
    return res


def cpu_baseline(ditsynth):
    """The oracle, untuned, on one block of the 32-block stack (all 4352 rows) on the host."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    w = ditsynth.workload(3)
    wt = ditsynth.block_weights(w, 0)
    inp = ditsynth.block_inputs(w)
    c, s = oracle.rope_tables(oracle.rope_positions(w.text, w.images))
    t0 = time.perf_counter()
    out = oracle.block_forward(inp["x"], inp["mod"], inp["mod_of_seg"], inp["seg_len"], c, s, wt, "w8a8")
    dt = time.perf_counter() - t0
    assert np.all(np.isfinite(out["x_out"]))
    return {"value": round(w.T / dt, 1), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"one W8A8 block (block 0 of 32) over all {w.T} rows of the 1024px workload, "
                      f"fp64 NumPy oracle incl. its weight quantization; {dt:.1f}s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-edit", action="store_true")
    ap.add_argument("--edit-reps", type=int, default=5)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB")
    ap.add_argument("--counter-summary", default="", metavar="DIR",
                    help="print per-kernel means of the rocprofv3 --pmc csv files under DIR and exit")
    ap.add_argument("--loop-steps", type=int, default=40,
                    help="steps of the timed denoise loop after the step benchmark (0: skip)")
    args = ap.parse_args()
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the multi-GPU design is described, not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import ditsynth
    import diffusion_transformer_text_qwen_amd as dq

    dq.lib()
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe, dq, torch)
        return
    w, ms, ms_prof, prof, ok, loop, quant_q = run_stack(args, dq, torch, ditsynth)
    T, D, F = w.T, w.D, w.F
    n_timed = args.steps * w.n_blocks
    value = w.n_blocks * T / (ms * 1e-3)
    g_ops = gemm_ops(T, D, F)
    gemm_ms = sum(prof[s]["ms"] for s in GEMM_SITES)
    gemm_cnt = sum(prof[s]["count"] for s in GEMM_SITES)
    total_ops = sum(g_ops.values()) * n_timed
    avg_launch_ops = total_ops / gemm_cnt
    avg_launch_s = gemm_ms * 1e-3 / gemm_cnt
    achieved = avg_launch_ops / avg_launch_s / 1e12
    att_flops = 4 * D * attn_pairs(w.seg_len, T)
    kernels = {}
    kernels.update(site_report(prof, g_ops, n_timed, PEAK_INT8_TOPS, "TOPS"))
    kernels.update(site_report(prof, {"attention": att_flops}, n_timed, PEAK_BF16_TFLOPS, "TFLOPS"))
    kernels.update(site_report(prof, hbm_bytes(T, D, F), n_timed, PEAK_HBM_GBS, "GB/s"))
    # the same kernels' bytes from the FETCH_SIZE / WRITE_SIZE counters (taken
    # with the current elementwise source), at this run's launch times
    for site, nbytes in hbm_kernel_traffic().items():
        if site in kernels:
            rate = nbytes / (kernels[site]["avg_us"] * 1e-6) / 1e9
            kernels[site]["counter_bytes"] = nbytes
            kernels[site]["counter_GB/s"] = round(rate, 1)
            kernels[site]["counter_frac_peak"] = round(rate / PEAK_HBM_GBS, 4)
    block_ms = sum(p["ms"] for p in prof.values()) / n_timed
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "ms_per_step_profiled": round(ms_prof, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8/bf16",
        "data": "synthetic",
        "config": {"workload": "stack_w8a8_1024px: one denoise step = DiT head + 32 W8A8 blocks over "
                               "[256 text | 64x64 image] tokens + tail + Euler on the 4096x64 latent",
                   "blocks": w.n_blocks, "tokens": T, "image_tokens": w.seg_len[-1], "hidden": D,
                   "heads": w.H, "mlp": F, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                     "frac": round(achieved / PEAK_INT8_TOPS, 4), "traffic": gemm_traffic(),
                     "traffic_note": "FETCH_SIZE + WRITE_SIZE per launch site, calibrated by a plain copy: bytes "
                                     "that miss the XCD L2s (fabric bytes; the memory-side cache serves part of "
                                     "them), an upper bound on HBM bytes",
                     "kernel": "gemm_large_kernel<int8> (+ K-split tail and its reduce): the four W8A8 "
                               "linears of a block, one launch site each",
                     "algorithmic_ops_per_launch": int(avg_launch_ops),
                     "avg_launch_us": round(avg_launch_s * 1e6, 2)},
        "kernels": kernels,
        "block_ms_sum_of_launches": round(block_ms, 4),
        "finite": ok,
    }
    line["attn_int8_fp8_1024px"] = quant_q
    if loop is not None:
        line["denoise_loop_1024px"] = loop
    if not args.no_edit:
        line["edit_2048px"] = run_edit(args, dq, torch, ditsynth, args.edit_reps)
        line["gated_recipe_1024px"] = run_gated(args, dq, torch, ditsynth, args.edit_reps)
        line["small_blocks"] = run_small(args, dq, torch, ditsynth, args.edit_reps)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one block ...")
        line["cpu_baseline"] = cpu_baseline(ditsynth)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
