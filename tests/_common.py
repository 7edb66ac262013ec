"""Shared helpers for the GPU parity tests: seeded cases, device upload, oracle calls."""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from oracle import formats as F
from oracle import moe as M
from synth import configs as C
from synth import draw as D

# Scaled copies of the five workloads: same format, activation and routing recipe, sizes
# the oracle finishes in seconds, chosen to span several tiles and leave ragged tails.
SCALED = {
    "tiny": C.get_config("tiny"),
    "decode_s": C.scaled(C.get_config("decode"), num_experts=16, hidden=512, inter=384, name="decode_s"),
    "small_s": C.scaled(C.get_config("small"), num_experts=16, hidden=384, inter=232, name="small_s"),
    "prefill_s": C.scaled(C.get_config("prefill"), num_experts=32, hidden=512, inter=256, name="prefill_s"),
    "edge_s": C.scaled(C.get_config("edge"), num_experts=16, num_global_experts=32, hidden=384, inter=200,
                       name="edge_s"),
}


@dataclasses.dataclass
class Case:
    cfg: C.Workload
    m: int
    ids: np.ndarray
    w: np.ndarray
    emap: Optional[np.ndarray]
    xbits: np.ndarray
    codes: Optional[dict]          # canonical codes on the host (all experts), or None
    codes_dev: Optional[dict] = None
    key: Optional[tuple] = None    # full-size cases: (workload, m, routing seed, code seed), memoises the oracle


def quantised_codes(cfg: C.Workload, rng) -> dict:
    w13, w2 = D.draw_normal_weights(rng, cfg)
    if cfg.fmt == "mxfp4":
        p13, s13 = F.quantise_mxfp4(w13)
        p2, s2 = F.quantise_mxfp4(w2)
        one = np.ones(cfg.num_experts, np.float32)
        return {"w13": p13, "s13": s13, "w2": p2, "s2": s2, "g13": one, "g2": one.copy()}
    p13, s13, g13 = F.quantise_nvfp4(w13)
    p2, s2, g2 = F.quantise_nvfp4(w2)
    return {"w13": p13, "s13": s13, "w2": p2, "s2": s2, "g13": g13, "g2": g2}


def make_case(cfg: C.Workload, m: int, seed: int, weights: str = "normal") -> Case:
    ids, w, emap, rng = D.draw_routing(cfg, m, seed)
    xbits = D.draw_activations_bf16(rng, m, cfg.hidden)
    if weights == "normal":
        codes = quantised_codes(cfg, rng)
    elif weights == "random":
        codes = D.draw_random_codes(cfg, seed)
    else:
        codes = None
    return Case(cfg, m, ids, w, emap, xbits, codes)


def experts_for(case: Case, experts=None) -> M.Experts:
    cfg = case.cfg
    if case.codes is not None:
        return M.Experts(cfg.fmt, cfg.act, cfg.hidden, cfg.inter, case.codes)
    # full-size device codes: copy only the experts the oracle needs, and keep no dequantised
    # expert after its use (up to ~150 experts of 350 MB each in float64 at the prefill shape)
    ids = sorted(int(e) for e in experts)
    sub = {k: case.codes_dev[k][ids].cpu().numpy() for k in ("w13", "s13", "w2", "s2", "g13", "g2")}
    return M.Experts(cfg.fmt, cfg.act, cfg.hidden, cfg.inter, sub, expert_ids=ids, cache=False)


# Oracle outputs of full-size cases, by (case key, variant): the same prefill case is checked by
# more than one test, and its oracle run takes a minute or more.
_ORACLE_MEMO: dict = {}


def oracle_out(case: Case, tokens=None, cols=None, mxfp8: bool = False) -> np.ndarray:
    from oracle.route_pack import local_ids

    memo = case.key is not None and tokens is None and cols is None
    if memo and (case.key, mxfp8) in _ORACLE_MEMO:
        return _ORACLE_MEMO[(case.key, mxfp8)]
    cfg = case.cfg
    x = F.bf16_bits_to_f64(case.xbits)
    needed = None
    if case.codes is None:
        t = np.arange(case.m) if tokens is None else np.asarray(tokens)
        lid = local_ids(case.ids, case.emap, cfg.num_global_experts, cfg.num_experts).reshape(case.m, cfg.topk)
        needed = np.unique(lid[t][lid[t] >= 0])
    ex = experts_for(case, needed)
    out = M.moe_forward(x, case.ids, case.w, case.emap, cfg.num_global_experts, cfg.num_experts, ex,
                        tokens=tokens, cols=cols, mxfp8=mxfp8)
    if memo:
        _ORACLE_MEMO[(case.key, mxfp8)] = out
    return out


def full_case(name: str, m: int, device, codes_dev: Optional[dict] = None, fmt: Optional[str] = None) -> Case:
    """A full-size workload case: routing and activations seeded per (workload, m), random
    canonical codes drawn on the device (seed per workload) unless ``codes_dev`` is given.
    ``fmt`` overrides the workload's weight format (same shape and routing)."""
    import dataclasses
    cfg = C.get_config(name)
    if fmt is not None and fmt != cfg.fmt:
        cfg = dataclasses.replace(cfg, fmt=fmt, name=f"{name}_{fmt}")
    seed = cfg.index * 1000 + m
    case = make_case(cfg, m, seed=seed, weights="none")
    case.codes_dev = codes_dev if codes_dev is not None else D.draw_random_codes_torch(cfg, seed=1000 + cfg.index,
                                                                                         device=device)
    case.key = (cfg.name, m, seed, 1000 + cfg.index)
    return case


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return F.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def dev(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload_codes(codes: dict, device) -> dict:
    return {k: dev(v, device) for k, v in codes.items()}


def make_layer(case: Case, device, token_capacity: Optional[int] = None):
    import fp4_weight_grouped_moe_amd as moe

    cfg = case.cfg
    cap = token_capacity or moe.moe_route_pack_token_capacity(case.m)
    layer = moe.MoeLayer(cfg.fmt, cfg.act, cfg.num_experts, cfg.hidden, cfg.inter, cfg.topk, cap, device=device)
    cd = case.codes_dev if case.codes_dev is not None else upload_codes(case.codes, device)
    nv = cfg.fmt == "nvfp4"
    layer.prepare(cd["w13"], cd["s13"], cd["g13"] if nv else None, cd["w2"], cd["s2"], cd["g2"] if nv else None)
    return layer


def run_layer(layer, case: Case, device, out=None, w4a8=False, atomic_bf16=False):
    import torch

    x = dev(case.xbits.view(np.int16), device).view(torch.bfloat16)
    emap = dev(case.emap, device) if case.emap is not None else None
    out = layer(x, dev(case.ids, device), dev(case.w, device), expert_map=emap,
                num_global_experts=case.cfg.num_global_experts, out=out, w4a8=w4a8, atomic_bf16=atomic_bf16)
    torch.cuda.synchronize()
    return out
