#!/usr/bin/env python3
"""Benchmark of the routed MoE layer (Step-5-Preview shape) on one MI355X.

One step = one pass of the whole layer (router, grouping, routed expert
gate/up + SwiGLU and down, shared expert, combine) over one batch of
synthetic tokens already resident in HBM.  Prints one JSON line.

  python bench.py [--workload prefill_fp8|decode_fp8|decode_bf16|decode_mxfp4|prefill_mxfp4|ep8_share_fp8|
                              dense_ff_bf16|train_bf16|small_bf16]
                  [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-decode]
                  [--weight-layout tile16|rows]

The default workload is the FP8 prefill layer (T=8192 tokens, hidden 4096,
352 experts, top-8 with the Zipf-skewed router, intermediate 1536, one bf16
shared expert), scored by MFMA utilisation; the same run then times the FP8
decode layer (T=64, the same expert weights, unbiased router) in a timed
region of its own, scored by HBM bandwidth, and reports it as the nested
object "decode_fp8" (--no-decode leaves it out).  The dominant kernel's
roofline figure comes from HIP events recorded around that kernel inside the
timed steps (moe_timing.h); the CPU baseline is the fp64 oracle on a bounded
sample of the same workload, on the host's cores.

The routed experts' bf16 and fp8 weights are repacked once, before the timed
region, into the 16-row tile layout (moe_pack_weights; --weight-layout rows
keeps them row-major); MX FP4 and training workloads use row-major weights.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + HBM GB/s (decode) / MFMA TFLOP/s % peak (prefill)"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # dense MFMA, TFLOP/s (e2m1 x e4m3 runs at the fp8 rate)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_fp8")
    ap.add_argument("--no-decode", action="store_true",
                    help="prefill_fp8 only: leave out the FP8 decode layer timed in the same run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--weight-layout", choices=["tile16", "rows"], default="tile16",
                    help="storage of the routed experts' bf16/fp8 weights (packed once before timing)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run plain 1 GiB device copies only (reference dispatches for the HBM byte counters)")
    return ap.parse_args()


# HBM traffic of the dominant kernel, from two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE,
# KiB per dispatch) over this command, each scaled by what the same counter reads for a plain
# 1 GiB device copy (bench.py --copy-calibration).  Valid only for the kernel sources they were
# taken on: a different hash of the dominant kernel's sources (KERNEL_SOURCES) reports null.
TRAFFIC = {
    "prefill_fp8": {"src_hash": "34ea98c4f774e2f2", "fetch_kib": 3132184.61, "write_kib": 134275.79, "fetch_scale": 2.0, "write_scale": 1.0},
    "decode_fp8": {"src_hash": "34ea98c4f774e2f2", "fetch_kib": 1651545.47, "write_kib": 1141.0, "fetch_scale": 2.0, "write_scale": 1.0},
    "decode_bf16": {"src_hash": "34ea98c4f774e2f2", "fetch_kib": 3274900.49, "write_kib": 1730.61, "fetch_scale": 2.0, "write_scale": 1.0},
    "decode_mxfp4": {"src_hash": "34ea98c4f774e2f2", "fetch_kib": 898080.84, "write_kib": 1180.38, "fetch_scale": 2.0, "write_scale": 1.0},
    "prefill_mxfp4": {"src_hash": "34ea98c4f774e2f2", "fetch_kib": 2199479.88, "write_kib": 137705.2, "fetch_scale": 2.0, "write_scale": 1.0},
    "ep8_share_fp8": {"src_hash": "34ea98c4f774e2f2", "fetch_kib": 847462.41, "write_kib": 76832.77, "fetch_scale": 2.0, "write_scale": 1.0},
    "dense_ff_bf16": {"src_hash": "34ea98c4f774e2f2", "fetch_kib": 1360378.88, "write_kib": 221362.7, "fetch_scale": 2.0, "write_scale": 1.0},
    # per step: the four weight-gradient launches (routed dW_down, dW_gate_up; the shared expert's two)
    "train_bf16": {"src_hash": "de929ec2da51e8d2", "fetch_kib": 4392258.36, "write_kib": 26326024.52, "fetch_scale": 2.0, "write_scale": 1.0},
}


# Sources that decide what the dominant kernel of a workload does (its code,
# the structures it reads, the launch plan): the forward's grouped gate/up
# kernels, or the backward's weight-gradient kernel.
KERNEL_SOURCES = {   # relative to router_gemm_amd/csrc (build.py holds the compiler flags)
    "forward": ["expert_gemm.hip", "expert_gemm_tiled.hip", "expert_gemm_tiled_mx.hip", "layout.hip", "moe_common.h",
                "moe_kernels.h", "moe_api.cpp", "../build.py"],
    "backward": ["backward.hip", "moe_common.h", "moe_kernels.h", "moe_api.cpp", "../build.py"],
}


def _code_only(text: str, path: str) -> str:
    """C/C++/HIP source without its comments and blank-line or trailing-space
    differences (comments do not change what a kernel does); other files as is."""
    import re
    if path.endswith((".hip", ".h", ".cpp")):
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return text


def library_source_hash(family="forward"):
    """Hash of the code the family's dominant kernel is built from."""
    import hashlib
    d = os.path.join(ROOT, "router_gemm_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(KERNEL_SOURCES[family]):
        h.update(f.encode())
        h.update(_code_only(open(os.path.join(d, f)).read(), f).encode())
    return h.hexdigest()[:16]


def copy_calibration():
    """Plain device copies of a known size: 3 x copy_ and 3 x neg over 1 GiB."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(3):
        dst.copy_(src)
    ev1.record()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / 3
    print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "launches": {"copy_": 3, "neg": 3}, "copy_ms": round(ms, 4),
                      "copy_GBps": round(2 * n / (ms / 1e3) / 1e9, 1)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import numpy as np
    import torch

    from router_gemm_amd import binding as B
    from router_gemm_amd import workloads as W
    from router_gemm_amd.build import LIB

    if not os.path.exists(LIB):
        from router_gemm_amd import build as hb
        hb.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)

    cfg = W.get_config(args.workload)
    dev = torch.device("cuda:0")
    print(f"[bench] building {cfg.name} on {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    lt = W.make_layer(cfg, dev)
    x = W.make_x(cfg, dev)
    if cfg.name.startswith("train"):
        bench_train(args, cfg, lt, x, dev)
        return
    mx = cfg.expert_dtype == "mxfp4"
    layer = B.Layer.from_tensors(lt, top_k=cfg.k if not cfg.triples else 0)
    weight_layout = "rows" if (mx or args.weight_layout == "rows") else "tile16"
    if weight_layout == "tile16":
        layer = layer.packed()   # a load-time repack, outside the timed region
        torch.cuda.synchronize()
    out = measure(args, cfg, lt, layer, x, weight_layout, dev)
    if cfg.name == "prefill_fp8" and not args.no_decode:
        # the decode layer of the same model: the same expert, shared-expert and
        # router weights (same seed and shapes), no router bias, T = 64
        dcfg = W.get_config("decode_fp8")
        assert (dcfg.E, dcfg.H, dcfg.I, dcfg.Is, dcfg.expert_dtype, dcfg.seed, dcfg.router_std) == \
               (cfg.E, cfg.H, cfg.I, cfg.Is, cfg.expert_dtype, cfg.seed, cfg.router_std)
        print(f"[bench] timing {dcfg.name} (same expert weights)", file=sys.stderr, flush=True)
        dlt = dataclasses.replace(lt, cfg=dcfg, router_bias=None)
        d = measure(args, dcfg, dlt, layer.with_router_bias(None), W.make_x(dcfg, dev), weight_layout, dev)
        for key in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data", "warmup"):
            d.pop(key, None)
        out["decode_fp8"] = d
    print(json.dumps(out), flush=True)


def measure(args, cfg, lt, layer, x, weight_layout, dev):
    """Time K steps of one workload's layer (inputs resident in HBM) and return
    the JSON object of the bench line."""
    import numpy as np
    import torch

    from router_gemm_amd import binding as B
    from router_gemm_amd import workloads as W

    T, H, E, I, Is = cfg.T, cfg.H, cfg.E, cfg.I, cfg.Is
    fp8 = cfg.expert_dtype != "bf16"     # activations and h stored as e4m3 + 1x128 scales
    mx = cfg.expert_dtype == "mxfp4"
    N = cfg.N
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    if cfg.dense:
        # the dense FF layer: one expert holding every token, rows in token order
        ws = B.workspace(layer, T, T, dev)
        off = torch.tensor([0, T], dtype=torch.int32, device=dev)

        def step():
            B.moe_expert_ffn(layer, off, x, None, T, y, ws=ws)

        counts = np.array([T])
    elif cfg.triples:
        # one rank's expert-parallel share: the pre-routed triples through
        # moe_forward_routed (grouping, routed + shared expert launches, combine)
        tok, exp, gate = W.make_triples(cfg)
        tok_g, exp_g, gate_g = (torch.from_numpy(a).to(dev) for a in (tok, exp, gate))
        ws = B.workspace(layer, T, N, dev)

        def step():
            B.moe_forward_routed(layer, x, T, exp_g, tok_g, gate_g, N, y, ws=ws)

        counts = np.bincount(exp, minlength=E)
    else:
        ws = B.workspace(layer, T, N, dev)
        ids = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
        gts = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)

        def step():
            B.moe_forward(layer, x, T, y, topk_ids=ids, topk_gates=gts, ws=ws)

        step()
        torch.cuda.synchronize()
        counts = np.bincount(ids.cpu().numpy().ravel(), minlength=E)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    site = 4   # MOE_SITE_GATE_UP: grouped gate/up GEMM, which streams 2/3 of the expert weights
    B.timing_arm(site, 4 * K)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for _ in range(K):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gu_ms_total, gu_launches = B.timing_read(site)
    ms_per_step = ev0.elapsed_time(ev1) / K
    tokens_per_s = T * K / (ms_per_step * K / 1e3)

    # ---- algorithmic work (what the method must move / compute)
    active = int((counts > 0).sum())
    esz = 1 if fp8 else 2
    if mx:   # half a byte per weight plus one E8M0 byte per 32 weights
        w_gu_b = 2 * I * H // 2 + 2 * I * H // 32
        w_d_b = H * I // 2 + H * I // 32
    else:
        w_gu_b = 2 * I * H * esz + ((2 * I // 128) * (H // 128) * 4 if fp8 else 0)
        w_d_b = H * I * esz + ((H // 128) * (I // 128) * 4 if fp8 else 0)
    shared_b = 3 * Is * H * 2
    router_b = 0 if (cfg.triples or cfg.dense) else E * H * 2
    layer_bytes = active * (w_gu_b + w_d_b) + shared_b + router_b + T * H * 2 * 2
    fl_routed = 2.0 * N * 3 * I * H
    fl_bf16 = 2.0 * T * 3 * Is * H + (0 if (cfg.triples or cfg.dense) else 2.0 * T * E * H)
    if not fp8:
        fl_bf16 += fl_routed
        fl_routed_fp8 = 0.0
    else:
        fl_routed_fp8 = fl_routed
    t_s = ms_per_step / 1e3
    mfma_util = (fl_routed_fp8 / (PEAK_TFLOPS["fp8"] * 1e12) + fl_bf16 / (PEAK_TFLOPS["bf16"] * 1e12)) / t_s
    # gate/up launch of one step: the routed experts' [gate; up] weights (+ scales), their
    # input rows and h output, plus the shared expert's (same launch inside moe_forward and
    # moe_forward_routed)
    gu_bytes = active * w_gu_b + N * H * esz + N * I * esz + ((N * H // 128 + N * I // 128) * 4 if fp8 else 0)
    if Is > 0:
        gu_bytes += 2 * Is * H * 2 + T * H * 2 + T * Is * 2
    gu_f_routed = 2.0 * N * 2 * I * H
    gu_f_shared = 2.0 * T * 2 * Is * H
    gu_ms = gu_ms_total / K                      # per step (all gate/up launches of the step)
    decode_like = (N / max(active, 1)) < 64
    if decode_like:
        roof = {"bound": "hbm", "achieved": round(gu_bytes / (gu_ms / 1e3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        f8 = gu_f_routed if fp8 else 0.0
        f16 = gu_f_shared + (0.0 if fp8 else gu_f_routed)
        # mixed fp8/bf16 contraction: peak = total flops / ideal time at each dtype's dense peak
        peak = (f8 + f16) / (f8 / PEAK_TFLOPS["fp8"] + f16 / PEAK_TFLOPS["bf16"])
        roof = {"bound": "mfma", "achieved": round((f8 + f16) / (gu_ms / 1e3) / 1e12, 1), "peak": round(peak, 1),
                "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    tr = TRAFFIC.get(cfg.name)
    src_hash = library_source_hash()
    launches = max(gu_launches // K, 1)
    if tr and tr["src_hash"] == src_hash:
        roof["traffic"] = int((tr["fetch_kib"] * tr["fetch_scale"] + tr["write_kib"] * tr["write_scale"]) * 1024)
        roof["traffic_per"] = "launch"
    else:
        roof["traffic"] = None
        roof["traffic_note"] = ("no counters taken on these kernel sources" if not tr
                                else "kernel sources changed since the counters were taken")
    roof["kernel_source_hash"] = src_hash
    roof["kernel"] = ("gate/up + SwiGLU of the dense FF layer (one expert)" if cfg.dense
                      else "grouped gate/up + SwiGLU (routed and shared experts)")
    roof["kernel_ms_per_step"] = round(gu_ms, 4)
    roof["launches_per_step"] = launches
    roof["avg_launch_us"] = round(1e3 * gu_ms / launches, 2)
    roof["algorithmic_bytes_per_step"] = int(gu_bytes)
    roof["algorithmic_flops_per_step"] = gu_f_routed + gu_f_shared

    # per-step spread: a separate pass of K steps with an event between steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(K):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(K)])
    spread = {q: round(float(np.percentile(per_step, v)), 4) for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}

    # per-kernel breakdown: a separate pass of K steps with every launch site timed
    sites = {0: "router_logits", 1: "router_topk", 2: "sort", 3: "gather", 4: "gate_up", 5: "down", 8: "combine"}
    for sidx in sites:
        B.timing_arm(sidx, 4 * K)
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    breakdown = {}
    for sidx, nm in sites.items():
        ms, n = B.timing_read(sidx)
        if n:
            breakdown[nm] = round(1e3 * ms / K, 1)   # microseconds per step

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.expert_dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": T, "hidden": H, "experts": E, "top_k": cfg.k,
                   "inter": I, "shared_inter": Is, "expert_dtype": cfg.expert_dtype,
                   "assignments": N, "active_experts": active, "max_rows_per_expert": int(counts.max()),
                   "weight_layout": weight_layout, "parallelism": "1 GPU"},
        "layer": {"algorithmic_bytes": int(layer_bytes), "hbm_GBps": round(layer_bytes / t_s / 1e9, 1),
                  "hbm_frac": round(layer_bytes / t_s / 1e9 / PEAK_HBM_GBS, 4),
                  "tflops": round((fl_routed_fp8 + fl_bf16) / t_s / 1e12, 2),
                  "mfma_util_blended": round(mfma_util, 4), "wall_s": round(wall, 4)},
        "roofline": roof,
        "breakdown_us_per_step": breakdown,
        "step_ms_percentiles": spread,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, lt, x, args.cpu_seconds)
    return out


def bench_train(args, cfg, lt, x, dev):
    """Training step of the layer: moe_forward_train (the forward, keeping the
    expert pre-activations) then moe_backward (all weight, router and input
    gradients) on one batch of tokens."""
    import numpy as np
    import torch

    from router_gemm_amd import binding as B
    from router_gemm_amd import workloads as W

    T, H, E, I, Is, k = cfg.T, cfg.H, cfg.E, cfg.I, cfg.Is, cfg.k
    N = T * k
    dy = W.make_dy(cfg, dev)
    layer = B.Layer.from_tensors(lt)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    gts = torch.empty((T, k), dtype=torch.float32, device=dev)
    ws_f = B.workspace(layer, T, N, dev)
    ws_b = B.backward_workspace(layer, T, dev)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    grads = dict(dx=f32(T, H), dw_gate_up=f32(E, 2 * I, H), dw_down=f32(E, H, I),
                 dw_shared_gate_up=f32(2 * Is, H) if Is else None, dw_shared_down=f32(H, Is) if Is else None,
                 dw_router=f32(E, H), dbias=f32(E) if lt.router_bias is not None else None)

    z_saved = torch.empty(B.moe_saved_z_floats(layer, T), dtype=torch.float32, device=dev)

    def step():
        B.moe_forward_train(layer, x, T, y, ids, gts, z_saved, ws=ws_f)
        B.moe_backward(layer, x, T, ids, gts, dy, z_saved=z_saved, ws=ws_b, **grads)

    step()
    torch.cuda.synchronize()
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=E)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    gemm_sites = {9: "bwd_dgrad_gemm", 10: "bwd_wgrad_gemm"}
    for sidx in gemm_sites:
        B.timing_arm(sidx, 8 * K)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for _ in range(K):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gemm = {nm: B.timing_read(sidx) for sidx, nm in gemm_sites.items()}
    ms_per_step = ev0.elapsed_time(ev1) / K
    t_s = ms_per_step / 1e3

    # ---- algorithmic work.  Expert rows: N routed assignments + T shared-expert rows.
    ih = N * I * H + T * Is * H
    fwd_flops = 2.0 * 3 * ih + 2.0 * T * E * H
    # model flops of a training step: forward, plus twice the expert GEMM flops for the
    # data and weight gradients, plus the router's two gradient products
    model_flops = fwd_flops + 2.0 * 6 * ih + 2.0 * 2 * N * H
    # the backward's grouped GEMM launches (the forward keeps z, so no recompute): dy W_down (IH)
    # and dz W_gate_up (2IH) per row = dgrad site; dW_down (IH) and dW_gate_up (2IH) = wgrad site
    dgrad_flops, wgrad_flops = 2.0 * 3 * ih, 2.0 * 3 * ih
    g_ms = {nm: ms / K for nm, (ms, n) in gemm.items()}
    g_launch = {nm: max(n // K, 1) for nm, (ms, n) in gemm.items()}
    gemm_ms = sum(g_ms.values())
    peak = PEAK_TFLOPS["bf16"]
    # The dominant kernel is the weight-gradient GEMM (its site's launches: routed dW_down and
    # dW_gate_up, the shared expert's two).  At ~186 rows per expert it does ~90 flops per byte
    # it must move (the fp32 gradients it writes), below the MI355X ridge of 312: HBM-bound.
    # Algorithmic bytes per step: the gradients written (fp32) + each operand row read once.
    wgrad_bytes = (4 * 3 * I * H * E + 4 * 3 * Is * H) \
        + N * (H + I) * 2 + N * (2 * I + H) * 2 \
        + (T * (H + Is) * 2 + T * (2 * Is + H) * 2 if Is else 0)
    w_ms = g_ms["bwd_wgrad_gemm"]
    w_achieved = wgrad_bytes / (w_ms / 1e3) / 1e9
    roof = {"bound": "hbm", "achieved": round(w_achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(w_achieved / PEAK_HBM_GBS, 4)}
    tr = TRAFFIC.get(cfg.name)
    src_hash = library_source_hash("backward")
    if tr and tr["src_hash"] == src_hash:
        roof["traffic"] = int((tr["fetch_kib"] * tr["fetch_scale"] + tr["write_kib"] * tr["write_scale"]) * 1024)
        roof["traffic_per"] = "step (the site's launches)"
    else:
        roof["traffic"] = None
        roof["traffic_note"] = ("no counters taken on these kernel sources" if not tr
                                else "kernel sources changed since the counters were taken")
    roof.update({
        "kernel_source_hash": src_hash,
        "kernel": "weight-gradient grouped bf16 GEMM (dW_gate_up, dW_down; routed and shared)",
        "kernel_ms_per_step": round(w_ms, 4),
        "launches_per_step": g_launch["bwd_wgrad_gemm"],
        "avg_launch_us": round(1e3 * w_ms / g_launch["bwd_wgrad_gemm"], 2),
        "algorithmic_bytes_per_step": int(wgrad_bytes),
        "algorithmic_flops_per_step": wgrad_flops,
        "tflops": round(wgrad_flops / (w_ms / 1e3) / 1e12, 1)})
    gemms = {"bound": "mfma", "unit": "TFLOP/s", "peak": peak,
             "all_launches_tflops": round((dgrad_flops + wgrad_flops) / (gemm_ms / 1e3) / 1e12, 1),
             "all_launches_frac": round((dgrad_flops + wgrad_flops) / (gemm_ms / 1e3) / 1e12 / peak, 4),
             "ms_per_step": round(gemm_ms, 4),
             "per_site": {nm: {"ms_per_step": round(g_ms[nm], 4), "launches_per_step": g_launch[nm],
                               "tflops": round(f / (g_ms[nm] / 1e3) / 1e12, 1) if g_ms[nm] > 0 else None}
                          for nm, f in (("bwd_dgrad_gemm", dgrad_flops), ("bwd_wgrad_gemm", wgrad_flops))}}

    # per-kernel breakdown: a separate pass with every launch site timed
    sites = {0: "router_logits", 1: "router_topk", 2: "sort", 3: "gather", 4: "gate_up", 5: "down", 8: "combine",
             9: "bwd_dgrad_gemm", 10: "bwd_wgrad_gemm"}
    for sidx in sites:
        B.timing_arm(sidx, 8 * K)
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    breakdown = {}
    for sidx, nm in sites.items():
        ms, n = B.timing_read(sidx)
        if n:
            breakdown[nm] = round(1e3 * ms / K, 1)
    out = {
        "metric": METRIC, "value": round(T / t_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "step": "moe_forward_train + moe_backward (all gradients)", "tokens": T,
                   "hidden": H, "experts": E, "top_k": k, "inter": I, "shared_inter": Is, "expert_dtype": "bf16",
                   "assignments": N, "active_experts": int((counts > 0).sum()),
                   "min_rows_per_expert": int(counts.min()), "max_rows_per_expert": int(counts.max()),
                   "parallelism": "1 GPU"},
        "layer": {"model_tflops": round(model_flops / t_s / 1e12, 2), "mfma_util": round(model_flops / t_s / 1e12 / peak, 4),
                  "model_flops_per_step": model_flops, "wall_s": round(wall, 4)},
        "roofline": roof,
        "backward_gemms": gemms,
        "breakdown_us_per_step": breakdown,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_train(cfg, lt, x, dy, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_model() -> str:
    """The host CPU's model name (the first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline_train(cfg, lt, x, dy, target_s):
    """The fp64 oracle's forward and backward (input gradient only: its weight
    gradients would be 53 GB of fp64 at this shape) on a sample of tokens."""
    import numpy as np

    import oracle
    from router_gemm_amd import workloads as W

    print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
    h = W.host_layer_arrays(lt)
    L = oracle.Layer(cfg.H, cfg.I, cfg.E, cfg.k, "bf16", h["w_router"], h["w_gate_up"], h["w_down"],
                     router_bias=h["router_bias"], w_shared_gate_up=h["w_shared_gate_up"],
                     w_shared_down=h["w_shared_down"])
    xb, dyb = W.bf16_bits(x), W.bf16_bits(dy)
    n = 8
    sample = np.sort(np.random.default_rng(0).choice(cfg.T, n, replace=False))
    ids = np.zeros((cfg.T, cfg.k), dtype=np.int32)        # rows outside the sample are never read
    ids[sample] = oracle.route(L, xb, token_list=sample)[0]
    done, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(L, xb, token_list=sample)
        oracle.backward(L, xb, ids, dyb, token_list=sample, weights=False)
        done += n
        el = time.perf_counter() - t0
        if el >= target_s or done >= 8 * n:
            break
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": oracle.num_threads(), "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{n} of the {cfg.T} tokens of {cfg.name} (seeded choice): forward of the layer, then "
                      f"the backward's input gradient (no weight gradients), {done // n} pass(es) in {el:.1f} s; "
                      f"the sample's routing is done once beforehand, untimed"}


def cpu_baseline(cfg, lt, x, target_s):
    """The fp64 oracle on a bounded sample of tokens of the same workload."""
    import numpy as np

    import oracle
    from router_gemm_amd import workloads as W

    print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
    h = W.host_layer_arrays(lt)
    L = oracle.Layer(cfg.H, cfg.I, cfg.E, max(cfg.k, 1), cfg.expert_dtype, h["w_router"],
                     h["w_gate_up"], h["w_down"], s_gate_up=h["s_gate_up"], s_down=h["s_down"],
                     router_bias=h["router_bias"], w_shared_gate_up=h["w_shared_gate_up"],
                     w_shared_down=h["w_shared_down"])
    xb = W.bf16_bits(x)
    rng = np.random.default_rng(0)
    n = min(cfg.T, 64)
    sample = np.sort(rng.choice(cfg.T, n, replace=False))
    if cfg.triples:
        tok, exp, gate = W.make_triples(cfg)
        run = lambda: oracle.forward_triples(L, xb, tok, exp, gate, token_list=sample)
        n_assign = int(np.isin(tok, sample).sum())
        pass_flops = 2.0 * (n_assign * 3 * cfg.I * cfg.H + n * 3 * cfg.Is * cfg.H)
    else:
        run = lambda: oracle.forward(L, xb, token_list=sample)
        pass_flops = 2.0 * n * (cfg.k * 3 * cfg.I * cfg.H + 3 * cfg.Is * cfg.H + cfg.E * cfg.H)
    done, t0 = 0, time.perf_counter()
    while True:
        run()
        done += n
        el = time.perf_counter() - t0
        if el >= target_s or done >= 16 * n:
            break
    return {"value": round(done / el, 2), "unit": "tokens/s", "cores": oracle.num_threads(), "cpu": cpu_model(),
            "kind": "oracle",
            "fp64_gflops": round(pass_flops * (done // n) / el / 1e9, 2),
            "sample": f"{n} of the {cfg.T} tokens of {cfg.name} (seeded choice), full layer per token, "
                      f"{done // n} pass(es) in {el:.1f} s"}


if __name__ == "__main__":
    main()
