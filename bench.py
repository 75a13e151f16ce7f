#!/usr/bin/env python3
"""Throughput of one denoising step of the DiT: 50 stacked AdaLN DiT blocks at
the 864x480x56-frame latent shape (N = 14x54x30 = 22680 tokens, D = 5120,
40 heads x 128, MLP 13824, bf16), on one MI355X.

    python bench.py [--steps K] [--warmup W] [--layers L] [--no-cpu-baseline]

Prints ONE JSON line on stdout.  `value` is the whole step's algorithmic
TFLOP/s (attention 4 N^2 D, projections 2 N D (3D + D + 2F), AdaLN 12 D C per
block), with weights and activations resident in HBM before timing starts.
The timed region is bracketed by torch.cuda.synchronize(); every kernel
launch is also bracketed by hipEvents recorded by the library itself on the
launch stream (h3k_profiler), which gives the per-kernel durations used for
the roofline of the dominant kernel.  The CPU baseline times the plain numpy
oracle on the host cores on one full block of the same shape (see
`cpu_baseline.sample`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DiT step ms + TFLOP/s (MFMA util %) at 22.7k latent tokens, bf16, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 MFMA
# dense FLOP per clock per CU of v_mfma_f32_16x16x32_bf16 (16x16x32 multiply-adds per 16 cycles per
# SIMD, 4 SIMDs); int8 (16x16x64 in the same cycles) doubles it
BF16_FLOP_PER_CLK_CU = 4 * 16 * 16 * 32 * 2 // 16


def device_block():
    """The GPU this run measured on, from the library's device query, with the dense peaks its
    compute units and peak clock imply (the roofline keeps the published peaks)."""
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    d = B.h3k_get_device_info(torch.cuda.current_device())
    per_s = d["compute_units"] * d["peak_clock_khz"] * 1e3
    return {"name": torch.cuda.get_device_name(), "arch": d["arch"], "compute_units": d["compute_units"],
            "peak_clock_mhz": round(d["peak_clock_khz"] / 1e3, 1), "lds_kib_per_cu": d["lds_bytes_per_cu"] // 1024,
            "hbm_gib": round(d["hbm_bytes"] / 2**30, 1),
            "bf16_peak_from_cus_and_clock_tflops": round(per_s * BF16_FLOP_PER_CLK_CU / 1e12, 1),
            "int8_peak_from_cus_and_clock_tops": round(2 * per_s * BF16_FLOP_PER_CLK_CU / 1e12, 1)}


def bw(nbytes, ms):
    """GB/s of `nbytes` moved in `ms`, and its fraction of the 8 TB/s HBM peak."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    return round(gbs, 1), round(gbs / PEAK_HBM_GBS, 4)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def block_flops(N, D, F, C):
    return {
        "adaln": 2.0 * 6 * D * C,
        "qkv": 2.0 * N * D * 3 * D,
        "attention": 4.0 * N * N * D,
        "out_proj": 2.0 * N * D * D,
        "mlp_up": 2.0 * N * D * F,
        "mlp_down": 2.0 * N * D * F,
    }


def ln_bytes(N, D, eb=2):
    # read x row, write h row, read shift and scale (fp32)
    return 2.0 * N * D * eb + 2.0 * D * 4


COPY_BYTES = 512 * 2**20
KERNEL_SOURCES = {"attention": "attention.hip", "qkv": "gemm.hip", "out_proj": "gemm.hip", "mlp_up": "gemm.hip",
                  "mlp_down": "gemm.hip"}
TRAFFIC_KEYS = {"attention": "attention", "qkv": "qkv:bf16", "out_proj": "out_proj:bf16", "mlp_up": "mlp_up:bf16",
                "mlp_down": "mlp_down:bf16"}


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/traffic.json), or None when the kernel's source file has
    changed since the counters were taken (its sha256 no longer matches)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    src = os.path.join(ROOT, "video_diffusion_transformer_adaln_amd", "csrc", KERNEL_SOURCES.get(kernel, ""))
    if not os.path.exists(path) or not os.path.isfile(src):
        return None
    with open(path) as f:
        rec = json.load(f).get(TRAFFIC_KEYS.get(kernel, kernel))
    if not rec:
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec.get("source_sha256"):
            return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- rocprofv3 summaries
# Library kernels and what they are in a block; the gated-residual GEMM serves the
# out-projection and MLP-down, told apart by their order within each block.
def kernel_role(name):
    n = name.replace(" ", "")
    if "attention_bf16_kernel" in n:
        return "attention"
    if "gemm_ring_kernel<" in n:
        args = n.split("gemm_ring_kernel<", 1)[1].split(">", 1)[0].split(",")
        epi, i8 = args[0], args[1] == "true"
        w8 = len(args) > 2 and args[2] == "true"
        grp = len(args) > 3 and args[3] == "true"
        staged = args[4] if len(args) > 4 else "0"      # int8 weights widened into the staging buffer
        kind = "int8xint8" if i8 else ("w8a16_group" if grp else ("w8a16" if w8 else "bf16"))
        if staged in ("1", "2"):
            kind = "w8a16_staged" if staged == "1" else "w8a16_group_staged"
        return {"0": "qkv", "1": "mlp_up", "2": "gated", "3": "qkv_rope"}.get(epi, "gemm") + ":" + kind
    for key, role in (("ln_modulate_kernel", "ln_mod"), ("adaln_gemv_kernel", "adaln"),
                      ("quantize_int8_rows_kernel", "quantize_rows"), ("quantize_int8_kernel", "quantize_rows"),
                      ("quantize_int8_groups_kernel", "quantize_groups"), ("dequant_int8_kernel", "dequant"),
                      ("gemm_tail_kernel", "gemm_tail"), ("attention_combine_kernel", "attention_combine"),
                      ("copyBuffer", "copy")):
        if key in n:
            return role
    return None


def _csv_rows(path):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _per_dispatch(path):
    """dispatch id -> (kernel name, grid size, {counter: value summed over instances})"""
    out = {}
    for r in _csv_rows(path):
        d = out.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], int(r["Grid_Size"]), {}])
        d[2][r["Counter_Name"]] = d[2].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d[2]["_dur_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return dict(sorted(out.items()))


def _label(dispatches):
    """(dispatch id, role) for every library dispatch; 'gated' becomes out_proj or
    mlp_down by its order in the block (the out-projection comes first)."""
    labels, gated_seen = {}, 0
    for did, (name, grid, _) in dispatches.items():
        role = kernel_role(name)
        if role is None:
            continue
        if role.startswith("gated:"):
            role = ("out_proj:" if gated_seen % 2 == 0 else "mlp_down:") + role.split(":")[1]
            gated_seen += 1
        labels[did] = role
    return labels


def summarize_profiles(root, write_traffic=True):
    """Turn the rocprofv3 outputs under `root` (trace/, fetch/, write/, mfma/
    from the commands in profiles/*.md) into profiles/traffic.json and print the
    per-kernel tables those summaries quote."""
    import hashlib
    import statistics
    sources = {"attention": "attention.hip", "gemm": "gemm.hip", "other": "adaln_ln.hip"}

    def src_sha(role):
        key = "attention" if role.startswith("attention") else ("gemm" if ":" in role else "other")
        with open(os.path.join(ROOT, "video_diffusion_transformer_adaln_amd", "csrc", sources[key]), "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()

    fetch, write = _per_dispatch(os.path.join(root, "fetch")), _per_dispatch(os.path.join(root, "write"))
    cf = [v[2]["FETCH_SIZE"] for v in fetch.values() if kernel_role(v[0]) == "copy"]
    cw = [v[2]["WRITE_SIZE"] for v in write.values() if kernel_role(v[0]) == "copy"]
    kib = COPY_BYTES / 1024.0
    f_scale = kib / max(cf) if cf else 1.0        # the calibration copy is the largest copy dispatch
    w_scale = kib / max(cw) if cw else 1.0
    lf, lw = _label(fetch), _label(write)
    roles = {}
    for did, role in lf.items():
        roles.setdefault(role, {"fetch": [], "write": []})["fetch"].append(fetch[did][2]["FETCH_SIZE"] * 1024 * f_scale)
    for did, role in lw.items():
        roles.setdefault(role, {"fetch": [], "write": []})["write"].append(write[did][2]["WRITE_SIZE"] * 1024 * w_scale)
    traffic = {"_note": (f"bytes per launch = FETCH_SIZE x {f_scale:.4f} + WRITE_SIZE x {w_scale:.4f} (KiB x 1024), "
                         "the factors from a plain 512 MiB device copy in the same runs; written by "
                         "`bench.py --summarize-profiles`")}
    print("| Kernel | Launches | Fetch (MB) | Write (MB) | HBM bytes / launch (MB) |")
    print("|---|---:|---:|---:|---:|")
    for role, v in sorted(roles.items()):
        if role == "copy" or not v["fetch"] or not v["write"]:
            continue
        fm, wm = statistics.mean(v["fetch"]), statistics.mean(v["write"])
        traffic[role] = {"hbm_bytes_per_launch": int(fm + wm), "fetch_bytes": int(fm), "write_bytes": int(wm),
                         "launches": len(v["fetch"]), "source_sha256": src_sha(role)}
        print(f"| {role} | {len(v['fetch'])} | {fm / 1e6:.1f} | {wm / 1e6:.1f} | {(fm + wm) / 1e6:.1f} |")
    if write_traffic:
        with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
            json.dump(traffic, f, indent=1)
    mfma_dir = os.path.join(root, "mfma")
    if os.path.isdir(mfma_dir):
        m = _per_dispatch(mfma_dir)
        lm = _label(m)
        agg = {}
        for did, role in lm.items():
            agg.setdefault(role, []).append(m[did][2])
        print()
        print("| Kernel | Launches | Clock (GHz) | MFMA busy | co-exec | wait | LDS bank conflicts / launch |")
        print("|---|---:|---:|---:|---:|---:|---:|")
        for role, lst in sorted(agg.items()):
            if role == "copy":
                continue
            c = {k: statistics.mean(d.get(k, 0.0) for d in lst) for k in lst[0]}
            gui = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0            # per XCD
            busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
            dur = statistics.mean(d.get("_dur_ns", 0.0) for d in lst)
            clock = f"{gui / dur:.2f}" if dur else "-"
            util = busy / (1024 * gui) if gui else 0.0
            coex = c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / busy if busy else 0.0
            wait = c.get("SQ_WAIT_INST_ANY", 0.0) / c["SQ_WAVE_CYCLES"] if c.get("SQ_WAVE_CYCLES") else 0.0
            print(f"| {role} | {len(lst)} | {clock} | {100 * util:.1f} % | {100 * coex:.0f} % | {100 * wait:.0f} % | "
                  f"{c.get('SQ_LDS_BANK_CONFLICT', 0.0):.3g} |")


def main():
    if len(sys.argv) >= 3 and sys.argv[1] == "--summarize-profiles":
        summarize_profiles(sys.argv[2], write_traffic="--no-traffic-json" not in sys.argv[3:])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--layers", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-breadth", action="store_true",
                    help="also time the oracle on one 512-token fp32 block, one 6144-token block and one "
                         "int8-weight block")
    ap.add_argument("--no-layers45", action="store_true")
    ap.add_argument("--no-extra-blocks", action="store_true",
                    help="skip the int8-weight block and the 6144-token block timings")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 512 MiB device copy first (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the DiT step runs on a single MI355X here "
              "(multi-GPU sequence parallelism is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import seeded_inputs as si
    from video_diffusion_transformer_adaln_amd import binding as B
    from video_diffusion_transformer_adaln_amd import runtime as R

    B.lib()
    shape = si.C3
    N, D, F, C, H, d = shape.n_tokens, shape.hidden, shape.mlp_hidden, shape.cond_dim, shape.n_heads, shape.head_dim
    L = args.layers
    cfg = B.make_config(N, D, H, d, F, C, B.H3K_BF16, B.H3K_BF16, True)

    # ---- inputs, resident in HBM (drawn on the device with torch's seeded generator)
    t0 = time.time()
    blocks = []
    for l in range(L):
        t = {}
        for i, (name, shp) in enumerate(shape.weight_shapes().items()):
            if name.startswith("b_"):
                t[name] = torch.zeros(shp, dtype=torch.bfloat16, device="cuda")
            else:
                t[name] = si.torch_device_normal(shp, si.WEIGHT_STD, si.BASE_SEED, 1000 * l + i, "cuda",
                                                 torch.bfloat16)
        blocks.append(t)
    x = si.torch_device_normal((N, D), 1.0, si.BASE_SEED, 999_000, "cuda", torch.bfloat16)
    c = si.torch_device_normal((C,), 1.0, si.BASE_SEED, 999_001, "cuda", torch.bfloat16)
    stack = R.DitStack(cfg, blocks)
    out = torch.empty_like(x)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s; workspace {stack.workspace.numel() / 2**30:.2f} GiB")

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy of {COPY_BYTES} bytes done")

    # ---- warmup
    for i in range(args.warmup):
        stack.forward(x, c, out)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    # ---- timed steps, with per-kernel events recorded by the library
    prof = B.Profiler(capacity=8 * L * args.steps + 64)
    stats = prof.stats()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.steps):
        stack.forward(x, c, out, stats=stats)
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_step = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms_step:.2f} ms/step")
    kern = prof.summary()
    prof.close()
    if not torch.isfinite(out.float()).all():
        log("non-finite output")
        sys.exit(3)

    ms45 = None
    if not args.no_layers45 and L >= 45:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            stack.forward(x, c, out, n_layers=45)
        e1.record()
        torch.cuda.synchronize()
        ms45 = e0.elapsed_time(e1) / args.steps
        log(f"45-layer step: {ms45:.2f} ms")

    fl = block_flops(N, D, F, C)
    step_flops = L * sum(fl.values())
    tflops = step_flops / (ms_step * 1e-3) / 1e12

    per_kernel = {}
    for name, v in kern.items():
        if v["launches"] == 0:
            continue
        avg_ms = v["total_ms"] / v["launches"]
        e = {"avg_ms": round(avg_ms, 4), "launches": v["launches"], "share": round(v["total_ms"] / total_ms, 4)}
        if name in fl:
            e["tflops"] = round(fl[name] / (avg_ms * 1e-3) / 1e12, 1)
            e["mfma_frac"] = round(e["tflops"] / PEAK_BF16_TFLOPS, 4) if name != "adaln" else None
        if name == "ln_mod":
            e["gbs"], e["hbm_frac"] = bw(ln_bytes(N, D), avg_ms)
        if name == "adaln":
            e["gbs"], e["hbm_frac"] = bw(6 * D * C * 2 + C * 2 + 6 * D * 4, avg_ms)
        per_kernel[name] = e
    dom = max((k for k in per_kernel if k in fl and k != "adaln"), key=lambda k: kern[k]["total_ms"])
    dom_avg = per_kernel[dom]["avg_ms"]
    achieved = fl[dom] / (dom_avg * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(dom),
                "algorithmic_per_launch": f"{fl[dom] / 1e12:.3f} TFLOP"}

    extra = {}
    if not args.no_extra_blocks:
        extra = extra_blocks(blocks[0], x, c)
        if L >= 4:
            extra["token_reduction_step"] = token_reduction_step(cfg, blocks, x, c, ms_step, fl, L)
        extra["sp8_share_block"] = sp_share(blocks[0])

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(step_flops, L, breadth=args.cpu_breadth)

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights, zero biases; random init)",
        "config": {"workload": f"denoising step: {L} stacked AdaLN DiT blocks, N=22680 tokens "
                               "(14x54x30 latent of 864x480x56 frames), D=5120, 40x128 heads, F=13824, "
                               "GELU-tanh, bf16, activation aliasing on",
                   "layers": L, "tokens": N, "hidden": D, "heads": H, "head_dim": d, "mlp": F},
        "mfma_util": round(tflops / PEAK_BF16_TFLOPS, 4),
        "ms_per_step_layers45": round(ms45, 2) if ms45 is not None else None,
        "tflop_per_step": round(step_flops / 1e12, 2),
        "kernels": per_kernel,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "device": device_block(),
    }
    result.update(extra)
    print(json.dumps(result), flush=True)


def token_reduction_step(cfg, blocks, x, c, ms_full, fl, L, reps=2):
    """The same step with the middle half of the layers (L/4 .. L - L/4 - 1)
    on merged tokens: adjacent tokens of a latent row (54 per row) averaged
    before, restored after.  Reported besides the full step, not in `value`."""
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    from video_diffusion_transformer_adaln_amd import runtime as R
    first, last = L // 4, L - L // 4
    cfg_r = B.DitConfig.from_buffer_copy(cfg)
    cfg_r.token_reduction_first, cfg_r.token_reduction_last = first, last
    st = R.DitStack(cfg_r, blocks)
    out = torch.empty_like(x)
    st.forward(x, c, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        st.forward(x, c, out)
    e1.record()
    torch.cuda.synchronize()
    if not torch.isfinite(out.float()).all():
        log("non-finite output with token reduction")
        sys.exit(3)
    ms = e0.elapsed_time(e1) / reps
    N = cfg.n_tokens
    fl_half = block_flops(N // 2, cfg.hidden, cfg.mlp_hidden, cfg.cond_dim)
    work = (L - (last - first)) * sum(fl.values()) + (last - first) * sum(fl_half.values())
    del st
    log(f"token reduction step (layers {first}..{last - 1} on {N // 2} tokens): {ms:.2f} ms")
    return {
        "workload": f"the denoising step with layers {first}..{last - 1} on merged token pairs "
                    f"({N // 2} tokens), the rest on {N}",
        "ms_per_step": round(ms, 2), "speedup_vs_full_step": round(ms_full / ms, 3),
        "time_saved_frac": round(1.0 - ms / ms_full, 4),
        "tflop_per_step": round(work / 1e12, 2), "tflops": round(work / (ms * 1e-3) / 1e12, 1),
    }


def _time_block(cfg, tensors, x, c, reps=5):
    """Mean ms of one block forward, and the per-kernel event summary."""
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    from video_diffusion_transformer_adaln_amd import runtime as R
    st = R.DitStack(cfg, [tensors])
    out = torch.empty_like(x)
    st.forward(x, c, out)
    torch.cuda.synchronize()
    prof = B.Profiler(capacity=8 * reps + 16)
    stats = prof.stats()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        st.forward(x, c, out, stats=stats)
    e1.record()
    torch.cuda.synchronize()
    kern = prof.summary()
    prof.close()
    if not torch.isfinite(out.float()).all():
        log("non-finite output in an extra block")
        sys.exit(3)
    return e0.elapsed_time(e1) / reps, kern


def extra_blocks(b0, x, c):
    """More measured units besides the step: the int8-weight block (the four
    projection weights of block 0 quantised per output row by the library's
    quantiser, W8A16 GEMMs), the same with the row-quantised FC2 and with
    the group-wise int8 MLP, the bf16 block with 3D RoPE, and one bf16 block
    at 6144 tokens, D=3072 (512x512x22-frame latent).  Inputs as for the
    step."""
    import torch
    import seeded_inputs as si
    from video_diffusion_transformer_adaln_amd import binding as B
    from video_diffusion_transformer_adaln_amd import runtime as R
    res = {}
    # ---- int8 projection weights
    sh = si.C4
    N, D, F, C, H, d = sh.n_tokens, sh.hidden, sh.mlp_hidden, sh.cond_dim, sh.n_heads, sh.head_dim
    t8 = {k: v for k, v in b0.items() if k in ("w_ada", "b_ada", "b_qkv", "b_out", "b_up", "b_down")}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_el = 0
    for name in si.MATRIX_NAMES:
        q, s = R.quantize_int8(b0[name])           # allocates the outputs; the first pass also warms up
        t8[name], t8["s_" + name[2:]] = q, s
        n_el += b0[name].numel()

    def quantise_all(names, group=0):
        for name in names:
            w = b0[name]
            rows, cols = w.shape
            dst = tg if group else t8
            if group:
                B.h3k_quantize_weights_int8_groups(w, B.H3K_BF16, rows, cols, group, dst[name],
                                                   dst["s_" + name[2:]])
            else:
                B.h3k_quantize_weights_int8(w, B.H3K_BF16, rows, cols, dst[name], dst["s_" + name[2:]])

    # timed: a second pass into the same outputs, launches back to back
    torch.cuda.synchronize()
    e0.record()
    quantise_all(si.MATRIX_NAMES)
    e1.record()
    torch.cuda.synchronize()
    q_ms = e0.elapsed_time(e1)
    rows = sum(b0[n].shape[0] for n in si.MATRIX_NAMES)
    q_bytes = n_el * (2 + 1) + rows * 4
    cfg8 = B.make_config(N, D, H, d, F, C, B.H3K_BF16, B.H3K_INT8, True)
    ms8, kern8 = _time_block(cfg8, t8, x, c)
    fl = block_flops(N, D, F, C)
    k8 = {}
    for name in ("qkv", "out_proj", "mlp_up", "mlp_down"):
        v = kern8[name]
        avg = v["total_ms"] / v["launches"]
        k8[name] = {"avg_ms": round(avg, 4), "tflops": round(fl[name] / (avg * 1e-3) / 1e12, 1)}
    res["int8_block"] = {
        "workload": "one block at 22680 tokens with int8 QKV/out/up/down weights (per-row scales), "
                    "bf16 activations; each int8 weight widened to bf16 into a staging buffer, then the bf16 "
                    "GEMM with the row scale in its epilogue (W8A16 on the bf16 MFMA)",
        "ms_per_block": round(ms8, 3), "tflops": round(sum(fl.values()) / (ms8 * 1e-3) / 1e12, 1),
        "gemm_kernels": k8,
        "projection_weight_bytes": {"int8": int(n_el + rows * 4), "bf16": int(2 * n_el)},
        "quantiser": dict(zip(("ms_for_4_matrices", "gbs", "hbm_frac"), (round(q_ms, 3), *bw(q_bytes, q_ms)))),
    }
    log(f"int8-weight block: {ms8:.2f} ms; quantiser {q_ms:.3f} ms")
    # ---- the same block with the row-quantised FC2 (int8 x int8 MLP-down)
    cfgq = B.make_config(N, D, H, d, F, C, B.H3K_BF16, B.H3K_INT8, True, int8_fc2_rows=True)
    msq, kq = _time_block(cfgq, t8, x, c)
    fc2 = kq["mlp_down"]["total_ms"] / kq["mlp_down"]["launches"]
    aq = kq["act_quant"]["total_ms"] / kq["act_quant"]["launches"]
    fc2_tops = fl["mlp_down"] / (fc2 * 1e-3) / 1e12
    res["int8_fc2_block"] = {
        "workload": "the int8-weight block with the row-quantised FC2: u quantised per token row, MLP-down "
                    "as int8 x int8 on v_mfma_i32_16x16x64_i8 (int32 accumulation)",
        "ms_per_block": round(msq, 3), "tflops": round(sum(fl.values()) / (msq * 1e-3) / 1e12, 1),
        "fc2": {"avg_ms": round(fc2, 4), "tops": round(fc2_tops, 1), "peak_tops": PEAK_INT8_TOPS,
                "frac": round(fc2_tops / PEAK_INT8_TOPS, 4)},
        "u_row_quantiser": {"avg_ms": round(aq, 4),
                            "gbs": bw(N * F * 3 + N * 4, aq)[0], "hbm_frac": bw(N * F * 3 + N * 4, aq)[1]},
    }
    log(f"int8-FC2 block: {msq:.2f} ms (FC2 {fc2:.3f} ms, u quantiser {aq:.3f} ms)")
    # ---- the same block with the group-wise int8 MLP (w_up, w_down in groups of 128 input channels)
    G = 128
    tg = dict(t8)
    for name in ("w_up", "w_down"):
        tg[name], tg["s_" + name[2:]] = R.quantize_int8_groups(b0[name], G)
    torch.cuda.synchronize()
    e0.record()
    quantise_all(("w_up", "w_down"), G)
    e1.record()
    torch.cuda.synchronize()
    qg_ms = e0.elapsed_time(e1)
    g_el = b0["w_up"].numel() + b0["w_down"].numel()
    cfgg = B.make_config(N, D, H, d, F, C, B.H3K_BF16, B.H3K_INT8, True, int8_mlp_group=G)
    msg, kg = _time_block(cfgg, tg, x, c)
    kgr = {}
    for name in ("mlp_up", "mlp_down"):
        v = kg[name]
        avg = v["total_ms"] / v["launches"]
        kgr[name] = {"avg_ms": round(avg, 4), "tflops": round(fl[name] / (avg * 1e-3) / 1e12, 1)}
    res["int8_group_block"] = {
        "workload": f"the int8-weight block with group-wise int8 MLP weights (one scale per {G} input "
                    "channels, widened to bf16 times their group scales into a staging buffer before the "
                    "bf16 MFMA)",
        "ms_per_block": round(msg, 3), "tflops": round(sum(fl.values()) / (msg * 1e-3) / 1e12, 1),
        "mlp_kernels": kgr,
        "group_quantiser": {"ms_for_2_matrices": round(qg_ms, 3),
                            "gbs": bw(g_el * 3 + g_el // G * 4, qg_ms)[0],
                            "hbm_frac": bw(g_el * 3 + g_el // G * 4, qg_ms)[1]},
    }
    log(f"int8 group-MLP block: {msg:.2f} ms; group quantiser {qg_ms:.3f} ms")
    del t8, tg
    # ---- the bf16 block with 3D RoPE of q and k (14 frames x 30 rows x 54 columns), fused into the QKV epilogue
    cfgr = B.make_config(N, D, H, d, F, C, B.H3K_BF16, B.H3K_BF16, True, rope=(14, 30, 54, False))
    msr, kr = _time_block(cfgr, b0, x, c)
    cfgp = B.make_config(N, D, H, d, F, C, B.H3K_BF16, B.H3K_BF16, True)
    msp, kp = _time_block(cfgp, b0, x, c)
    qr = kr["qkv"]["total_ms"] / kr["qkv"]["launches"]
    qp = kp["qkv"]["total_ms"] / kp["qkv"]["launches"]
    res["rope_block"] = {
        "workload": "one bf16 block at 22680 tokens with 3D RoPE of q and k over the 14x30x54 latent grid, "
                    "rotated in the QKV projection's epilogue",
        "ms_per_block": round(msr, 3), "tflops": round(sum(fl.values()) / (msr * 1e-3) / 1e12, 1),
        "qkv_ms": round(qr, 4), "qkv_ms_without_rope": round(qp, 4), "block_ms_without_rope": round(msp, 3),
    }
    log(f"RoPE block: {msr:.2f} ms (QKV {qr:.3f} ms against {qp:.3f} ms without RoPE)")
    # ---- 6144-token bf16 block
    sh = si.C1
    N, D, F, C, H, d = sh.n_tokens, sh.hidden, sh.mlp_hidden, sh.cond_dim, sh.n_heads, sh.head_dim
    t1 = {}
    for i, (name, shp) in enumerate(sh.weight_shapes().items()):
        if name.startswith("b_"):
            t1[name] = torch.zeros(shp, dtype=torch.bfloat16, device="cuda")
        else:
            t1[name] = si.torch_device_normal(shp, si.WEIGHT_STD, si.BASE_SEED, 500_000 + i, "cuda", torch.bfloat16)
    x1 = si.torch_device_normal((N, D), 1.0, si.BASE_SEED, 599_000, "cuda", torch.bfloat16)
    c1 = si.torch_device_normal((C,), 1.0, si.BASE_SEED, 599_001, "cuda", torch.bfloat16)
    cfg1 = B.make_config(N, D, H, d, F, C, B.H3K_BF16, B.H3K_BF16, True)
    ms1, k1 = _time_block(cfg1, t1, x1, c1)
    flk = block_flops(N, D, F, C)
    fl1 = sum(flk.values())
    kern1 = {}
    for name, v in k1.items():
        if v["launches"]:
            avg = v["total_ms"] / v["launches"]
            kern1[name] = {"avg_ms": round(avg, 4)}
            if name in flk and name != "adaln":
                kern1[name]["tflops"] = round(flk[name] / (avg * 1e-3) / 1e12, 1)
    res["block_6144_tokens"] = {
        "workload": "one bf16 block at 6144 tokens (6x32x32 latent of 512x512x22 frames), D=3072, "
                    "24x128 heads, F=12288",
        "ms_per_block": round(ms1, 3), "tflops": round(fl1 / (ms1 * 1e-3) / 1e12, 1), "kernels": kern1}
    log(f"6144-token block: {ms1:.2f} ms")
    return res


def sp_share(b0, P=8, reps=5):
    """One GPU's share of a block under P-way sequence parallelism (the
    split the design describes; the two all-to-alls around attention are
    not built): LayerNorm + modulation and the four projection GEMMs on
    N/P tokens, attention for H/P heads over all N tokens.  Each kernel is
    timed through its own entry point on synthetic inputs of those shapes."""
    import torch
    import seeded_inputs as si
    from video_diffusion_transformer_adaln_amd import binding as B
    sh = si.C3
    N, D, F, H, d = sh.n_tokens, sh.hidden, sh.mlp_hidden, sh.n_heads, sh.head_dim
    M, Hs = N // P, H // P
    bf = torch.bfloat16
    g = lambda shp, std, sub: si.torch_device_normal(shp, std, si.BASE_SEED, 700_000 + sub, "cuda", bf)
    x = g((M, D), 1.0, 0)
    shift = si.torch_device_normal((D,), 0.1, si.BASE_SEED, 700_001, "cuda", torch.float32)
    scale = si.torch_device_normal((D,), 0.1, si.BASE_SEED, 700_002, "cuda", torch.float32)
    gate = si.torch_device_normal((D,), 0.1, si.BASE_SEED, 700_003, "cuda", torch.float32)
    h = torch.empty(M, D, dtype=bf, device="cuda")
    qk = torch.empty(M, 2 * D, dtype=bf, device="cuda")
    ldvt = (M + 7) // 8 * 8
    vt = torch.empty(D, ldvt, dtype=bf, device="cuda")
    o = g((M, D), 1.0, 4)
    y = torch.empty(M, D, dtype=bf, device="cuda")
    u = torch.empty(M, F, dtype=bf, device="cuda")
    # attention operands of H/P heads over all N tokens (after the all-to-all)
    Ds = Hs * d
    qa, ka = g((N, Ds), 0.6, 5), g((N, Ds), 0.6, 6)
    vta = g((Ds, N), 1.0, 7)
    oa = torch.empty(N, Ds, dtype=bf, device="cuda")
    E = B.H3K_BF16
    calls = {
        "ln_mod": (None, lambda: B.h3k_ln_modulate(E, M, D, 1e-6, x, D, shift, scale, h, D)),
        "qkv": (2.0 * M * D * 3 * D, lambda: B.h3k_linear(E, E, M, 3 * D, D, h, D, b0["w_qkv"], D, None, None,
                                                            B.H3K_EPI_BIAS, None, 0, None, qk, 2 * D, vt, ldvt, 2 * D)),
        "attention": (4.0 * N * N * Ds, lambda: B.h3k_attention(E, N, Hs, d, qa, Ds, ka, Ds, vta, N, oa, Ds,
                                                                           q_prescaled=True)),
        "out_proj": (2.0 * M * D * D, lambda: B.h3k_linear(E, E, M, D, D, o, D, b0["w_out"], D, None, None,
                                                            B.H3K_EPI_GATED_RESIDUAL, x, D, gate, y, D)),
        "mlp_up": (2.0 * M * D * F, lambda: B.h3k_linear(E, E, M, F, D, h, D, b0["w_up"], D, None, None,
                                                          B.H3K_EPI_GELU, None, 0, None, u, F)),
        "mlp_down": (2.0 * M * F * D, lambda: B.h3k_linear(E, E, M, D, F, u, F, b0["w_down"], F, None, None,
                                                            B.H3K_EPI_GATED_RESIDUAL, x, D, gate, y, D)),
    }
    res, total = {}, 0.0
    for name, (flops, fn) in calls.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        n_calls = 2 if name == "ln_mod" else 1
        total += n_calls * ms
        e = {"avg_ms": round(ms, 4)}
        if flops is not None:
            e["tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
        else:
            e["gbs"], e["hbm_frac"] = bw(ln_bytes(M, D), ms)
        res[name] = e
    for t in (y, u, oa):
        if not torch.isfinite(t.float()).all():
            log("non-finite output in the per-GPU share")
            sys.exit(3)
    fl = sum(v for k, v in block_flops(M, D, F, D).items() if k not in ("adaln", "attention")) + calls["attention"][0]
    log(f"one GPU's share of an {P}-way sequence-parallel block: {total:.3f} ms")
    return {
        "workload": f"one GPU's share of a block under {P}-way sequence parallelism: LayerNorm + modulation (x2) "
                    f"and the QKV / out / MLP GEMMs on {M} tokens, attention for {Hs} of {H} heads over all "
                    f"{N} tokens; all-to-alls not built",
        "ms_per_block_share": round(total, 3), "tflops": round(fl / (total * 1e-3) / 1e12, 1), "kernels": res,
    }


def _oracle_block_ms(shape, int8=False, parity=False):
    """Wall time (ms) of one oracle block forward over every token of `shape`
    (inputs drawn and, for int8 weights, quantised by the oracle beforehand,
    outside the timed call).  With `parity`, also the relative L2 distance of
    the library's block on the same host-seeded inputs from the oracle's
    output, over every token (bf16 workloads only)."""
    import oracle  # test infrastructure: CPU baseline only
    import seeded_inputs as si
    hx, hc = si.gen_activation(shape)
    hw = si.gen_block_weights(shape, 0)
    w = {k: v.values for k, v in hw.items()}
    if int8:
        for name in si.MATRIX_NAMES:
            w[name] = oracle.quantize_int8(w[name])
    t0 = time.perf_counter()
    y = oracle.block_forward(hx.values, hc.values, w, shape.n_heads)
    ms = (time.perf_counter() - t0) * 1e3
    if not parity:
        return ms, None
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    from video_diffusion_transformer_adaln_amd import runtime as R
    cfg = B.make_config(shape.n_tokens, shape.hidden, shape.n_heads, shape.head_dim, shape.mlp_hidden,
                        shape.cond_dim, B.H3K_BF16, B.H3K_BF16, True)
    stack = R.DitStack(cfg, [{k: R.upload(v.storage, v.dtype) for k, v in hw.items()}])
    x, c = R.upload(hx.storage, hx.dtype), R.upload(hc.storage, hc.dtype)
    out = torch.empty_like(x)
    stack.forward(x, c, out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = y.astype(np.float64)
    del stack, x, c, out
    torch.cuda.empty_cache()
    return ms, float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def cpu_baseline(step_flops, L, breadth=False):
    """The numpy oracle timed on this host: one full block of the step's shape
    (all 22680 tokens, every head, both projections and the MLP), measured,
    not extrapolated; the step is L such blocks.  BLAS runs on every core in
    the process's affinity mask.  With `breadth`, also one full block of the
    512-token fp32 workload, of the 6144-token workload and of the
    int8-weight workload."""
    import seeded_inputs as si
    cores = len(os.sched_getaffinity(0))
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            blas = ", ".join(f"{p.get('internal_api')} {p.get('version')} ({p.get('num_threads')} threads)" for p in libs)
    except Exception:
        limiter = None
    try:
        log(f"cpu baseline: one full 22680-token block on {cores} host cores ({blas})")
        t_block, parity = _oracle_block_ms(si.C2, parity=True)
        log(f"cpu baseline: {t_block / 1e3:.1f} s per block; the library's block on the same inputs: "
            f"rel-L2 {parity:.3e} over all {si.C2.n_tokens} tokens")
        per_block = {"n22680_d5120_bf16_inputs": round(t_block, 1)}
        if breadth:
            per_block["n512_d256_f32"] = round(_oracle_block_ms(si.C0)[0], 1)
            per_block["n6144_d3072_bf16_inputs"] = round(_oracle_block_ms(si.C1)[0], 1)
            per_block["n22680_d5120_int8_weights"] = round(_oracle_block_ms(si.C4, int8=True)[0], 1)
            log(f"cpu baseline, other workloads: {per_block}")
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    t_step = L * t_block / 1e3
    return {
        "value": round(step_flops / t_step / 1e12, 4),
        "unit": "TFLOP/s",
        "ms_per_step": round(t_step * 1e3, 1),
        "cores": cores,
        "kind": "oracle",
        "blas": blas,
        "per_block_ms": per_block,
        "block_rel_l2_vs_oracle": round(parity, 6),
        "sample": (f"one full 864x480x56-frame block (all {si.C2.n_tokens} tokens, 40 heads, D=5120, F=13824), "
                   f"the step's unit of work, measured once: {t_block / 1e3:.1f} s; the step is {L} such blocks; "
                   f"numpy fp32 oracle on bf16-valued inputs, {cores} cores ({blas})"),
    }


if __name__ == "__main__":
    main()
