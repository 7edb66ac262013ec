#!/usr/bin/env python3
"""Benchmark of the fused W4A16 MoE layer on one MI355X.

A step is one call of moe_w4a16_fused (route packing, FC1 + activation, FC2 + top-k sum)
on one synthetic batch whose routing, activations and weights are already in HBM. Steps
rotate through distinct routing batches, so consecutive steps touch different experts the
way consecutive decode steps do.

Timings of each workload and token count m:
  cold      each call bracketed by its own HIP event pair, with a 512 MiB scratch read
            before it (outside the timed region) so that neither the L2s nor the 256 MiB
            Infinity Cache hold the previous call's weights; the median over the steps.
  warm      the same calls back to back, one event pair around all of them (mean).
  graph     the call captured once per routing batch into a HIP graph, the graphs replayed
            back to back (mean): the warm, launch-overhead-free figure.
  profiled  the measurement twin (moe_w4a16_fused_profiled) under the cold protocol: an
            event after every kernel that launched, giving each kernel's mean duration.

The JSON line's headline is the decode shape at m = 8 (128 experts, hidden 4096,
intermediate 1536, top-8, NVFP4, SiLU-SwiGLU), cold. `sweep` holds decode m = 1 and 4 and
the prefill shape at m = 2048 (256 experts, hidden 7168, intermediate 2048, top-8, NVFP4,
Zipf-skewed routing), each with its own roofline; the prefill entry also carries the CPU
oracle's rate on a bounded sample.
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
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 / f16 MFMA
SCRATCH_BYTES = 512 << 20       # cold protocol: written between calls
PASSES = ("cold", "warm", "graph", "profiled")
_T0 = time.time()


def log(msg):
    """A progress line on stderr (the JSON result is the one line on stdout)."""
    print(f"[bench {time.time() - _T0:6.1f} s] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed steps of the headline (each pass)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=["tiny", "decode", "small", "prefill", "edge"])
    ap.add_argument("--m", type=int, default=None, help="tokens per step (default: decode 8, else the workload's largest m)")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "gemm"])
    ap.add_argument("--passes", default=",".join(PASSES), help="comma-separated subset of " + ",".join(PASSES))
    ap.add_argument("--no-sweep", action="store_true", help="headline only (no decode m = 1 / 4 and prefill entries)")
    ap.add_argument("--sweep-steps", type=int, default=50, help="timed steps of each sweep entry (each pass)")
    ap.add_argument("--sweep-warmup", type=int, default=10)
    ap.add_argument("--flush", default="read", choices=["read", "write"],
                    help="cold protocol: read (default) or write 512 MiB of scratch between calls")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fmt", default=None, choices=["nvfp4", "mxfp4"],
                    help="weight format override of the workload (e.g. the prefill shape with MXFP4 weights, "
                         "to compare --w4a8 with W4A16 where FC2 is MFMA-bound)")
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
        self.ev = []
        for _ in range(n):
            p = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(p))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.ev.append(p.value)

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
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


# The arithmetic the layer's contractions run in (inputs and outputs are bf16 throughout).
DTYPE_NOTES = {
    "f16": "NVFP4 weights: f16 MFMA operands (E2M1 x E4M3 exact in f16; activations times a per-token "
           "power of two, exact above 2^-38 of the row maximum; grouped-GEMM intermediate rows f16 times a "
           "per-slot power of two), fp32 accumulation",
    "bf16": "MXFP4 weights: bf16 MFMA operands (E2M1 x E8M0 exact in bf16), fp32 accumulation",
    "bf16+fp8": "W4A8: FC1 on bf16 operands; FC2 on the block-scaled FP4 x FP8 MFMA (activation output rounded "
                "to MXFP8); fp32 accumulation",
}


def compute_dtype(cfg, args):
    if args.w4a8:
        return "bf16+fp8"
    return "f16" if cfg.fmt == "nvfp4" else "bf16"


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "fp4_weight_grouped_moe_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, digest):
    """HBM bytes per launch of the kernel from the committed rocprofv3 counter summary, if the
    kernel's sources are unchanged since the counters were taken; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != digest:
        return None
    return t.get("hbm_bytes_per_launch")


class Layer:
    """One workload's prepared weights (random canonical codes drawn on the GPU)."""

    def __init__(self, moe, cfg, dev):
        from synth import draw as D
        self.moe, self.cfg, self.dev = moe, cfg, dev
        self.codes = D.draw_random_codes_torch(cfg, seed=1000 + cfg.index, device=dev)
        self.dims = moe.make_dims(cfg.fmt, cfg.act, cfg.num_experts, cfg.hidden, cfg.inter)
        import torch
        self.prepared_bytes = moe.moe_w4a16_prepared_size(self.dims)
        self.prepared = torch.empty(self.prepared_bytes, dtype=torch.uint8, device=dev)
        nv = cfg.fmt == "nvfp4"
        c = self.codes
        moe.moe_w4a16_prepare(self.dims, c["w13"], c["s13"], c["g13"] if nv else None, c["w2"], c["s2"],
                              c["g2"] if nv else None, self.prepared, self.prepared_bytes)
        torch.cuda.synchronize()
        log(f"{cfg.name}: weights drawn and prepared")


def measure(layer, m, steps, warmup, args, passes):
    """Time one (workload, m) under each requested pass; returns the JSON fields."""
    import numpy as np
    import torch

    from synth import draw as D

    moe, cfg, dev = layer.moe, layer.cfg, layer.dev
    k, H = cfg.topk, cfg.hidden
    cap = moe.moe_route_pack_token_capacity(m)
    total = steps + warmup
    sets = min(total, max(1, int(256e6 // (m * H * 2 + m * k * 8))))

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
    ws_bytes = moe.moe_w4a16_workspace_size(layer.dims, cap, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    scratch = torch.zeros(SCRATCH_BYTES, dtype=torch.uint8, device=dev)
    scratch_words = scratch.view(torch.int32)
    flush_sink = torch.zeros((), dtype=torch.int64, device=dev)

    # raw pointers resolved once, so that the host launch rate does not limit small steps
    lib = moe.lib()
    dims_ref = ctypes.byref(layer.dims)
    ptrs = [(d_x[s].data_ptr(), d_ids[s].data_ptr(), d_w[s].data_ptr()) for s in range(sets)]
    head = (layer.prepared.data_ptr(), layer.prepared_bytes)
    tail = (k, d_map.data_ptr() if d_map is not None else None, cfg.num_global_experts, cap, ws.data_ptr(), ws_bytes,
            out.data_ptr())
    fused = lib.moe_w4a8_fused if args.w4a8 else (lib.moe_w4a16_fused_atomic_bf16 if args.atomic_bf16
                                                  else lib.moe_w4a16_fused)
    whole_only = args.w4a8 or args.atomic_bf16      # the measurement twin runs the W4A16 layer

    def call(i, stream=None):
        px, pi, pw = ptrs[i % sets]
        st = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        rc = fused(dims_ref, head[0], head[1], px, m, pi, pw, *tail, st)
        if rc != 0:
            raise moe.MoeError(rc, "fused call", moe.moe_last_error())

    def cold_fill(i):
        # Evict the previous calls' weights from the L2s and the 256 MiB Infinity Cache by
        # reading 512 MiB (reads allocate there). A write would leave up to 256 MiB of dirty
        # lines whose write-back then falls inside the next timed call.
        if args.flush == "write":
            scratch.fill_(i & 0xFF)
        else:
            torch.sum(scratch_words, dim=0, dtype=torch.int64, out=flush_sink)

    res = {"m": m, "token_capacity": cap, "routing_sets": sets}
    log(f"{cfg.name} m={m}: {sets} routing batches ready")
    stream = torch.cuda.current_stream().cuda_stream
    moe.moe_w4a16_set_path(args.path)
    try:
        for i in range(warmup):
            cold_fill(i)
            call(i, stream)
        torch.cuda.synchronize()

        if "cold" in passes:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            torch.cuda.synchronize()
            for i in range(steps):
                cold_fill(warmup + i)
                ev[i][0].record()
                call(warmup + i, stream)
                ev[i][1].record()
            torch.cuda.synchronize()
            t = np.array([a.elapsed_time(b) for a, b in ev])
            log(f"{cfg.name} m={m}: cold pass done, median {np.median(t):.4f} ms")
            res["cold"] = {"ms_median": round(float(np.median(t)), 5), "ms_p10": round(float(np.percentile(t, 10)), 5),
                           "ms_p90": round(float(np.percentile(t, 90)), 5), "samples": steps}

        if "warm" in passes:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for i in range(steps):
                call(warmup + i, stream)
            e1.record()
            torch.cuda.synchronize()
            log(f"{cfg.name} m={m}: warm pass done")
            res["warm"] = {"ms_mean": round(e0.elapsed_time(e1) / steps, 5), "samples": steps,
                           "note": "back to back, rotating routing batches"}

        if "graph" in passes:
            n_graphs = min(sets, 8)
            graphs = []
            for gi in range(n_graphs):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    call(gi)                     # the capture stream is torch's current stream here
                graphs.append(g)
            for g in graphs:
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(steps):
                graphs[i % n_graphs].replay()
            e1.record()
            torch.cuda.synchronize()
            log(f"{cfg.name} m={m}: graph pass done")
            res["graph"] = {"ms_mean": round(e0.elapsed_time(e1) / steps, 5), "samples": steps,
                            "note": f"HIP graph replay back to back, {n_graphs} routing batches"}
            del graphs

        per = {}
        if "profiled" in passes and not whole_only:
            hev = HipEvents(6 * steps)
            names = []
            for i in range(steps):
                cold_fill(warmup + i)
                px, pi, pw = ptrs[(warmup + i) % sets]
                evs = (ctypes.c_void_p * 6)(*hev.ev[6 * i:6 * i + 6])
                kid = (ctypes.c_int32 * 5)()
                n = ctypes.c_int(0)
                rc = lib.moe_w4a16_fused_profiled(dims_ref, head[0], head[1], px, m, pi, pw, *tail, stream, evs, 6,
                                                  kid, ctypes.byref(n))
                if rc != 0:
                    raise moe.MoeError(rc, "moe_w4a16_fused_profiled", moe.moe_last_error())
                names.append([moe.KERNEL_NAMES[kid[j]] for j in range(n.value)])
            torch.cuda.synchronize()
            for i in range(steps):
                for j, name in enumerate(names[i]):
                    per.setdefault(name, []).append(hev.elapsed_ms(hev.ev[6 * i + j], hev.ev[6 * i + j + 1]))
            res["kernel_us"] = {n: round(float(np.mean(v)) * 1e3, 2) for n, v in per.items()}
            log(f"{cfg.name} m={m}: profiled pass done {res['kernel_us']}")
            res["kernels_launched"] = names[0]
            del hev
    finally:
        moe.moe_w4a16_set_path("auto")

    used = [(warmup + i) % sets for i in range(steps)]
    avg_touched = float(np.mean([touched[s] for s in used]))
    avg_valid = float(np.mean([valid[s] for s in used]))
    w13b, w2b = expert_bytes(cfg)
    weight_bytes = avg_touched * (w13b + w2b)
    flops = avg_valid * 2.0 * (H * cfg.n1 + cfg.inter * H)
    res.update({"touched_experts_avg": round(avg_touched, 2), "valid_routes_avg": round(avg_valid, 2),
                "weight_bytes_per_step": int(weight_bytes), "layer_bytes_per_step": int(weight_bytes + 2 * m * H * 2),
                "useful_flops_per_step": int(flops)})
    for key in ("cold", "warm", "graph"):
        if key in res:
            t = (res[key].get("ms_median") or res[key]["ms_mean"]) * 1e-3
            res[key].update({"tokens_per_s": round(m / t, 1), "weight_GBps": round(weight_bytes / t / 1e9, 1),
                             "hbm_frac": round(weight_bytes / t / 1e9 / HBM_PEAK_GBPS, 4),
                             "tflops": round(flops / t / 1e12, 3),
                             "mfma_frac": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 5)})

    if per:
        decode_path = "combine" not in per           # the decode path has no combine pass
    else:
        decode_path = args.path == "decode" or (args.path == "auto" and m <= moe.MOE_DECODE_MAX_M
                                                and cap <= moe.MOE_DECODE_MAX_M)
    res["path"] = "decode" if decode_path else "gemm"
    kernel_src = "decode.hip" if decode_path else "gemm.hip"
    workload_tag = f"{cfg.name}_m{m}"
    if not per:
        res["roofline"] = None
    elif decode_path:
        # dominant kernel: FC1 (W13 is two thirds of the streamed weights); algorithmic bytes
        # per launch = the touched experts' W13 codes + scales + globals, the activation rows
        # read and the intermediate rows written
        dom_bytes = avg_touched * w13b + m * H * 2 + avg_valid * cfg.inter * 2
        achieved = dom_bytes / (np.mean(per["fc1"]) * 1e-3) / 1e9
        res["roofline"] = {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic("decode_fc1", workload_tag, source_digest(kernel_src, "device.hpp")),
            "kernel": "decode_fc1_kernel", "algorithmic_bytes_per_launch": int(dom_bytes),
            "avg_launch_us": round(float(np.mean(per["fc1"])) * 1e3, 2)}
    else:
        # The grouped GEMM is bound by whichever of its two algorithmic floors is higher: the
        # useful MFMA flops at the dense peak of its operand type, or the bytes it must move
        # (the touched experts' weights, the activation rows read and the rows written) at
        # the HBM peak. FC1 at m = 2048 over 256 experts (~64 routes per expert) does about 400
        # flops per byte it must move, above the chip's ~310 flop/byte ridge (2.5 PFLOP/s over
        # 8 TB/s), so the MFMA floor binds there; the few-route tiles of the edge and small
        # shapes fall below the ridge and report the HBM floor.
        dom = "fc1" if np.mean(per["fc1"]) >= np.mean(per["fc2"]) else "fc2"
        t_dom = float(np.mean(per[dom])) * 1e-3
        if dom == "fc1":
            dom_flops = avg_valid * 2.0 * H * cfg.n1
            dom_bytes = avg_touched * w13b + m * H * 2 + avg_valid * cfg.inter * 2
            peak_tf = BF16_PEAK_TFLOPS
        else:
            dom_flops = avg_valid * 2.0 * cfg.inter * H
            dom_bytes = avg_touched * w2b + avg_valid * cfg.inter * 2 + avg_valid * H * 2
            peak_tf = BF16_PEAK_TFLOPS
        mfma = {"bound": "mfma", "achieved": round(dom_flops / t_dom / 1e12, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(dom_flops / t_dom / 1e12 / peak_tf, 4)}
        hbm = {"bound": "hbm", "achieved": round(dom_bytes / t_dom / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
               "frac": round(dom_bytes / t_dom / 1e9 / HBM_PEAK_GBPS, 4)}
        first, second = (hbm, mfma) if dom_bytes / (HBM_PEAK_GBPS * 1e9) >= dom_flops / (peak_tf * 1e12) else (mfma, hbm)
        res["roofline"] = dict(first, **{
            "traffic": load_traffic(f"gemm_{dom}", workload_tag, source_digest(kernel_src, "device.hpp")),
            "kernel": f"gemm_kernel<{dom}>", "algorithmic_bytes_per_launch": int(dom_bytes),
            "algorithmic_flops_per_launch": int(dom_flops),
            "floor_us": {"hbm": round(dom_bytes / (HBM_PEAK_GBPS * 1e9) * 1e6, 1),
                         "mfma": round(dom_flops / (peak_tf * 1e12) * 1e6, 1)},
            "avg_launch_us": round(t_dom * 1e6, 2), "other_bound": second})
    res["workload"] = (f"{cfg.name}: E{cfg.num_experts} H{H} I{cfg.inter} top{k} {cfg.fmt.upper()} {cfg.act} m={m}")
    res["_batches"] = (ids_l, w_l, x_l, emap)
    del d_ids, d_w, d_x, out, ws, scratch, scratch_words, flush_sink
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer has no multi-GPU path here).", file=sys.stderr)
        sys.exit(2)

    import torch

    import fp4_weight_grouped_moe_amd as moe
    from synth import configs as C

    passes = tuple(p for p in args.passes.split(",") if p)
    bad = [p for p in passes if p not in PASSES]
    if bad:
        raise SystemExit(f"unknown passes {bad}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = C.get_config(args.workload)
    if args.fmt and args.fmt != cfg.fmt:
        import dataclasses
        cfg = dataclasses.replace(cfg, fmt=args.fmt, name=f"{cfg.name}_{args.fmt}")
    m = args.m or (8 if args.workload == "decode" else max(cfg.ms))

    layer = Layer(moe, cfg, dev)
    head = measure(layer, m, args.steps, args.warmup, args, passes)
    batches = head.pop("_batches")
    key = "cold" if "cold" in head else ("warm" if "warm" in head else "graph")
    if key not in head:
        raise SystemExit("the headline needs at least one of the cold, warm or graph passes")
    ms = head[key].get("ms_median") or head[key]["ms_mean"]
    res = {
        "metric": METRIC,
        "value": round(m / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(cfg, args),
        "dtype_note": DTYPE_NOTES[compute_dtype(cfg, args)],
        "data": "synthetic",
        "config": {"workload": head["workload"], "m": m, "token_capacity": head["token_capacity"],
                   "routing_sets": head["routing_sets"], "path": head["path"], "timing": key,
                   "variant": "w4a8" if args.w4a8 else ("w4a16-atomic-bf16" if args.atomic_bf16 else "w4a16")},
        "effective_weight_GBps": head[key]["weight_GBps"],
        "weight_hbm_frac": head[key]["hbm_frac"],
        "tflops": head[key]["tflops"],
        "mfma_frac": head[key]["mfma_frac"],
        "touched_experts_avg": head["touched_experts_avg"],
        "cold": head.get("cold"), "warm": head.get("warm"), "graph": head.get("graph"),
        "kernel_us": head.get("kernel_us"),
        "roofline": head.get("roofline"),
    }
    if not args.no_cpu_baseline and not (args.w4a8 or args.atomic_bf16):
        res["cpu_baseline"] = cpu_baseline(layer, m, batches, args.cpu_seconds)

    if not args.no_sweep and args.workload == "decode" and m == 8 and not (args.w4a8 or args.atomic_bf16):
        sweep = []
        for mm in (1, 4):
            r = measure(layer, mm, args.sweep_steps, args.sweep_warmup, args, passes)
            r.pop("_batches")
            sweep.append(r)
        del layer
        torch.cuda.empty_cache()
        pre = Layer(moe, C.get_config("prefill"), dev)
        r = measure(pre, 2048, args.sweep_steps, args.sweep_warmup, args, passes)
        b = r.pop("_batches")
        if not args.no_cpu_baseline:
            r["cpu_baseline"] = cpu_baseline(pre, 2048, b, args.cpu_seconds)
        sweep.append(r)
        res["sweep"] = sweep
    print(json.dumps(res), flush=True)


def cpu_baseline(layer, m, batches, target_s):
    """The CPU oracle on the workload's routing batches in turn (the same codes, copied back
    from the device) until about target_s seconds of oracle time: whole batches while one batch
    takes less than the target, else a prefix of the first batch's tokens."""
    import numpy as np

    from oracle import formats as F
    from oracle import moe as M
    from oracle.route_pack import local_ids

    cfg = layer.cfg
    ids_l, w_l, x_l, emap = batches
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))

    def run(b, n):
        ids, w, x = ids_l[b], w_l[b], F.bf16_bits_to_f64(x_l[b])
        lid = local_ids(ids, emap, cfg.num_global_experts, cfg.num_experts).reshape(m, cfg.topk)
        toks = np.arange(n)
        need = sorted(int(e) for e in np.unique(lid[toks][lid[toks] >= 0]))
        host = {key: layer.codes[key][need].cpu().numpy() for key in ("w13", "s13", "w2", "s2", "g13", "g2")}
        ex = M.Experts(cfg.fmt, cfg.act, cfg.hidden, cfg.inter, host, expert_ids=need, cache=False)
        t0 = time.perf_counter()
        M.moe_forward(x, ids, w, emap, cfg.num_global_experts, cfg.num_experts, ex, tokens=toks)
        dt = time.perf_counter() - t0
        log(f"{cfg.name}: oracle on {n} tokens of batch {b} took {dt:.1f} s")
        return dt

    # a prefix of the first batch, grown (at least doubling: the oracle's time grows more slowly
    # than its token count, as more tokens share the dequantised experts) until it takes about
    # the target time or covers the batch
    n, elapsed = 1, 0.0
    while True:
        elapsed = run(0, n)
        if elapsed >= 0.6 * target_s or n >= m:
            break
        n = min(m, max(2 * n, int(np.ceil(n * target_s / max(elapsed, 1e-3)))))
    tokens, nb = n, 1
    # whole batches are short: add the next routing batches up to the target
    while n == m and elapsed < target_s and nb < len(ids_l):
        elapsed += run(nb, m)
        tokens += m
        nb += 1
    sample = (f"{nb} routing batches of {m} tokens" if nb > 1 else f"first {n} of {m} tokens of one batch")
    return {"value": round(tokens / elapsed, 4), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{sample} ({cfg.topk} routes each), float64 NumPy, dequantisation of the touched "
                      f"experts included; {elapsed:.1f} s"}


if __name__ == "__main__":
    main()
