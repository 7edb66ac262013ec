#!/usr/bin/env python3
"""Benchmark of the fused W4A16 MoE layer on one MI355X.

A step is one call of moe_w4a16_fused (route packing, FC1 + activation, FC2 + top-k
sum) on one synthetic batch whose routing, activations and weights are already in HBM.
Every step uses a fresh routing batch, so consecutive steps touch different experts the
way consecutive decode steps do. The default workload is the decode shape: 128 experts,
hidden 4096, intermediate 1536, top-8, NVFP4 weights, SiLU-SwiGLU, m = 8 tokens.

Prints one JSON line: tokens/s of the whole layer, the effective weight bandwidth and
TFLOP/s, the dominant kernel's roofline position (HIP events around each kernel, in a
second pass of the same steps) and the CPU oracle's rate on a bounded sample.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + effective weight GB/s (m=1..8) and TFLOP/s (m=2048), 1 GPU"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=["tiny", "decode", "small", "prefill", "edge"])
    ap.add_argument("--m", type=int, default=None, help="tokens per step (default: the workload's largest m)")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "gemm"])
    ap.add_argument("--sets", type=int, default=None, help="distinct routing batches rotated through")
    ap.add_argument("--sweep", action="store_true", help="also report the workload's other token counts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--w4a8", action="store_true",
                    help="time the W4A8 variant (moe_w4a8_fused, MXFP4 workloads): whole-layer time only")
    ap.add_argument("--atomic-bf16", action="store_true",
                    help="time the opt-in packed-bf16 atomic top-k combine (moe_w4a16_fused_atomic_bf16): "
                         "whole-layer time only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle sample time")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run three device copies of MIB MiB (calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def copy_probe(mib):
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)


class HipEvents:
    """Raw HIP events (the library records them on the stream its kernels run on)."""

    def __init__(self, n):
        # the HIP runtime already in the process (torch's), never a second copy by name
        paths = sorted({ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln})
        if len(paths) != 1:
            raise RuntimeError(f"expected one HIP runtime in the process, found {paths}")
        self.hip = ctypes.CDLL(paths[0])
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            p = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(p))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.ev[i] = p

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[a]), ctypes.c_void_p(self.ev[b]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        try:
            for p in self.ev:
                self.hip.hipEventDestroy(ctypes.c_void_p(p))
        except Exception:
            pass


def expert_bytes(cfg):
    g = cfg.group
    w13 = cfg.n1 * cfg.hidden // 2 + cfg.n1 * -(-cfg.hidden // g) + (4 if cfg.fmt == "nvfp4" else 0)
    w2 = cfg.hidden * cfg.inter // 2 + cfg.hidden * -(-cfg.inter // g) + (4 if cfg.fmt == "nvfp4" else 0)
    return w13, w2


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "fp4_weight_grouped_moe_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, digest, per_launch_bytes):
    """HBM traffic of the kernel from the committed rocprofv3 counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != digest:
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported by this build "
              "(the layer has no multi-GPU path here).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_weight_grouped_moe_amd as moe
    from synth import configs as C
    from synth import draw as D

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = C.get_config(args.workload)
    m = args.m or max(cfg.ms)
    k, H = cfg.topk, cfg.hidden
    cap = moe.moe_route_pack_token_capacity(m)
    total = args.steps + args.warmup
    # rotate through distinct batches (bounded to ~256 MB of activations + routing)
    sets = args.sets or min(total, max(1, int(256e6 // (m * H * 2 + m * k * 8))))
    sets = max(1, min(sets, total))

    # weights: raw random code bytes drawn on the GPU, then prepared into the fragment layout
    codes = D.draw_random_codes_torch(cfg, seed=1000 + cfg.index, device=dev)
    layer = moe.MoeLayer(cfg.fmt, cfg.act, cfg.num_experts, H, cfg.inter, k, cap, device=dev)
    nv = cfg.fmt == "nvfp4"
    layer.prepare(codes["w13"], codes["s13"], codes["g13"] if nv else None, codes["w2"], codes["s2"],
                  codes["g2"] if nv else None)
    torch.cuda.synchronize()

    # routing batches and activations
    ids_l, w_l, x_l, touched, valid = [], [], [], [], []
    emap = None
    for s in range(sets):
        ids, w, em, rng = D.draw_routing(cfg, m, seed=cfg.index * 100003 + s)
        emap = em
        x_l.append(D.draw_activations_bf16(rng, m, H))
        ids_l.append(ids)
        w_l.append(w)
        flat = ids.reshape(-1)
        ok = (flat >= 0) & (flat < cfg.num_global_experts)
        loc = flat[ok] if em is None else em[flat[ok]]
        loc = loc[(loc >= 0) & (loc < cfg.num_experts)]
        touched.append(len(np.unique(loc)))
        valid.append(len(loc))
    d_ids = torch.from_numpy(np.stack(ids_l)).to(dev)
    d_w = torch.from_numpy(np.stack(w_l)).to(dev)
    d_x = torch.from_numpy(np.stack(x_l).view(np.int16)).to(dev).view(torch.bfloat16)
    d_map = torch.from_numpy(emap).to(dev) if emap is not None else None
    out = torch.empty((m, H), dtype=torch.bfloat16, device=dev)
    moe.moe_w4a16_set_path(args.path)

    # raw pointers resolved once so that the host launch rate does not limit small steps
    lib = moe.lib()
    dims_ref = ctypes.byref(layer.dims)
    stream = moe._stream(None)
    ptrs = [(moe._ptr(d_x[s]), moe._ptr(d_ids[s]), moe._ptr(d_w[s])) for s in range(sets)]
    fixed = (moe._ptr(layer.prepared), layer.prepared_bytes)
    tail = (k, moe._ptr(d_map), cfg.num_global_experts, cap, moe._ptr(layer.workspace), layer.workspace_bytes,
            moe._ptr(out), stream)

    fused = lib.moe_w4a8_fused if args.w4a8 else (lib.moe_w4a16_fused_atomic_bf16 if args.atomic_bf16 else lib.moe_w4a16_fused)
    whole_only = args.w4a8 or args.atomic_bf16      # the measurement twin runs the W4A16 layer

    def step(i, events=None):
        px, pi, pw = ptrs[i % sets]
        if events is None:
            rc = fused(dims_ref, fixed[0], fixed[1], px, m, pi, pw, *tail)
        else:
            arr = (ctypes.c_void_p * 5)(*events)
            rc = lib.moe_w4a16_fused_profiled(dims_ref, fixed[0], fixed[1], px, m, pi, pw, *tail, arr, 5)
        if rc != 0:
            raise moe.MoeError(rc, "moe_w4a16_fused", moe.moe_last_error())

    # ---- pass A: whole-layer throughput
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # ---- pass B: per-kernel durations from events between the launches, same steps (the
    # measurement twin runs the W4A16 layer, so the W4A8 line reports the whole layer only)
    names = ["route_pack", "fc1", "fc2", "combine"]
    per = {n: 0.0 for n in names}
    if not whole_only:
        hev = HipEvents(5 * args.steps)
        for i in range(args.steps):
            step(args.warmup + i, [hev.ev[5 * i + j] for j in range(5)])
        torch.cuda.synchronize()
        for i in range(args.steps):
            for j, n in enumerate(names):
                per[n] += hev.elapsed_ms(5 * i + j, 5 * i + j + 1)
        per = {n: v / args.steps for n, v in per.items()}
    moe.moe_w4a16_set_path("auto")

    used = [(args.warmup + i) % sets for i in range(args.steps)]
    avg_touched = float(np.mean([touched[s] for s in used]))
    avg_valid = float(np.mean([valid[s] for s in used]))
    w13b, w2b = expert_bytes(cfg)
    weight_bytes = avg_touched * (w13b + w2b)
    step_bytes = weight_bytes + 2 * m * H * 2
    flops = avg_valid * 2.0 * (H * cfg.n1 + cfg.inter * H)
    t = ms_per_step * 1e-3
    decode_path = args.path == "decode" or (args.path == "auto" and m <= moe.MOE_DECODE_MAX_M and cap <= moe.MOE_DECODE_MAX_M)
    kernel_src = "decode.hip" if decode_path else "gemm.hip"
    if whole_only:
        roof = None
    elif decode_path:
        # dominant kernel: FC1 (W13 is two thirds of the streamed weights)
        dom = "fc1"
        dom_bytes = avg_touched * w13b + m * H * 2 + avg_valid * cfg.inter * 2
        achieved = dom_bytes / (per[dom] * 1e-3) / 1e9
        traffic = load_traffic("decode_fc1", args.workload + f"_m{m}", source_digest(kernel_src, "device.hpp"), dom_bytes)
        roof = {"bound": "hbm", "kernel": "decode_fc1_kernel", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": int(dom_bytes),
                "avg_launch_us": round(per[dom] * 1e3, 2)}
    else:
        dom = "fc1" if per["fc1"] >= per["fc2"] else "fc2"
        dom_flops = avg_valid * 2.0 * (H * cfg.n1 if dom == "fc1" else cfg.inter * H)
        achieved = dom_flops / (per[dom] * 1e-3) / 1e12
        traffic = load_traffic(f"gemm_{dom}", args.workload + f"_m{m}", source_digest(kernel_src, "device.hpp"), None)
        roof = {"bound": "mfma", "kernel": f"gemm_kernel<{dom}>", "achieved": round(achieved, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": traffic, "algorithmic_flops_per_launch": int(dom_flops),
                "avg_launch_us": round(per[dom] * 1e3, 2)}

    res = {
        "metric": METRIC,
        "value": round(m / t, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: E{cfg.num_experts} H{H} I{cfg.inter} top{k} {cfg.fmt.upper()} "
                               f"{cfg.act} m={m}", "m": m, "token_capacity": cap, "routing_sets": sets,
                   "path": "decode" if decode_path else "gemm", "variant": "w4a8" if args.w4a8 else ("w4a16-atomic-bf16" if args.atomic_bf16 else "w4a16")},
        "effective_weight_GBps": round(weight_bytes / t / 1e9, 1),
        "weight_hbm_frac": round(weight_bytes / t / 1e9 / HBM_PEAK_GBPS, 4),
        "layer_bytes_per_step": int(step_bytes),
        "tflops": round(flops / t / 1e12, 3),
        "mfma_frac": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 5),
        "touched_experts_avg": round(avg_touched, 2),
        "kernel_us": None if whole_only else {n: round(v * 1e3, 2) for n, v in per.items()},
        "roofline": roof,
    }
    del codes
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline and not whole_only:
        res["cpu_baseline"] = cpu_baseline(cfg, ids_l, w_l, x_l, emap, dev, m, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def cpu_baseline(cfg, ids_l, w_l, x_l, emap, dev, m, target_s):
    """The CPU oracle on the workload's routing batches in turn (same codes, regenerated on the
    GPU) until about target_s seconds of oracle time: whole batches while one batch takes less
    than the target, else a prefix of the first batch's tokens."""
    import numpy as np
    import torch

    from oracle import formats as F
    from oracle import moe as M
    from oracle.route_pack import local_ids
    from synth import draw as D

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    codes = D.draw_random_codes_torch(cfg, seed=1000 + cfg.index, device=dev)

    def run(b, n):
        ids, w, x = ids_l[b], w_l[b], F.bf16_bits_to_f64(x_l[b])
        lid = local_ids(ids, emap, cfg.num_global_experts, cfg.num_experts).reshape(m, cfg.topk)
        toks = np.arange(n)
        need = sorted(int(e) for e in np.unique(lid[toks][lid[toks] >= 0]))
        host = {key: codes[key][need].cpu().numpy() for key in ("w13", "s13", "w2", "s2", "g13", "g2")}
        ex = M.Experts(cfg.fmt, cfg.act, cfg.hidden, cfg.inter, host, expert_ids=need)
        t0 = time.perf_counter()
        M.moe_forward(x, ids, w, emap, cfg.num_global_experts, cfg.num_experts, ex, tokens=toks)
        return time.perf_counter() - t0

    # a prefix of the first batch, grown until it takes the target time or covers the batch
    n, elapsed = 1, 0.0
    while True:
        elapsed = run(0, n)
        if elapsed >= target_s or n >= m:
            break
        n = min(m, max(n + 1, int(np.ceil(n * target_s / max(elapsed, 1e-3)))))
    tokens, batches = n, 1
    # whole batches are short: add the next routing batches up to the target
    while n == m and elapsed < target_s and batches < len(ids_l):
        elapsed += run(batches, m)
        tokens += m
        batches += 1
    del codes
    torch.cuda.empty_cache()
    sample = (f"{batches} routing batches of {m} tokens" if batches > 1 else f"first {n} of {m} tokens of one batch")
    return {"value": round(tokens / elapsed, 4), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{sample} ({cfg.topk} routes each), float64 NumPy, dequantisation of the touched "
                      f"experts included; {elapsed:.1f} s"}


if __name__ == "__main__":
    main()
