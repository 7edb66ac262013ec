"""Seeded draws for the MoE workloads (NumPy PCG64; optional torch device draws).

Draw order for one (workload, m, seed): router logits -> invalid-route positions
-> expert_map -> activations x -> fp32 weights W13 -> fp32 weights W2.
Random FP4/FP8 code bytes (used where the fp32 weights would not fit in host
memory) come from their own generator so that they never shift the routing.
"""

from __future__ import annotations

import numpy as np

from .configs import Workload


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw_routing(cfg: Workload, m: int, seed: int):
    """Router output for m tokens: (topk_ids int32 [m,k], topk_weights f32 [m,k], expert_map or None).

    Scores: softmax (or sigmoid) of N(0,1) logits over the global experts; the
    Zipf recipe adds -s*ln(e+1) to expert e's logit. The top-k scores are
    renormalised to sum to 1 per token. Afterwards a fraction of the ids is
    overwritten with -1 (the weights stay), and an optional expert_map sends a
    random half of the global ids onto a permutation of the local ids.
    Returns also the generator so later draws continue the same stream.
    """
    rng = _rng(seed)
    eg, k = cfg.num_global_experts, cfg.topk
    logits = rng.standard_normal((m, eg))
    if cfg.routing == "zipf":
        logits = logits - cfg.zipf_s * np.log(np.arange(eg, dtype=np.float64) + 1.0)[None, :]
    if cfg.routing == "sigmoid":
        scores = 1.0 / (1.0 + np.exp(-logits))
    else:
        z = logits - logits.max(axis=1, keepdims=True)
        ez = np.exp(z)
        scores = ez / ez.sum(axis=1, keepdims=True)
    ids = np.argsort(-scores, axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(scores, ids, axis=1)
    if cfg.renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    ids = ids.astype(np.int32)
    w = w.astype(np.float32)
    if cfg.invalid_frac > 0 and m > 0:
        n_bad = int(round(cfg.invalid_frac * m * k))
        pos = rng.choice(m * k, size=n_bad, replace=False)
        flat = ids.reshape(-1)
        flat[pos] = -1
    emap = None
    if cfg.use_expert_map:
        chosen = rng.choice(eg, size=cfg.num_experts, replace=False)
        emap = np.full(eg, -1, dtype=np.int32)
        emap[chosen] = rng.permutation(cfg.num_experts).astype(np.int32)
    return ids, w, emap, rng


def draw_router_logits(cfg: Workload, m: int, seed: int) -> np.ndarray:
    """Router logits fp32 [m, Eg] for the router front end: N(0,1), plus the Zipf recipe's
    -s*ln(e+1) for expert e when the workload uses it (the same draw as draw_routing's)."""
    rng = _rng(seed)
    eg = cfg.num_global_experts
    logits = rng.standard_normal((m, eg))
    if cfg.routing == "zipf":
        logits = logits - cfg.zipf_s * np.log(np.arange(eg, dtype=np.float64) + 1.0)[None, :]
    return logits.astype(np.float32)


def draw_activations_bf16(rng: np.random.Generator, m: int, hidden: int) -> np.ndarray:
    """x = bf16(N(0,1)) as uint16 bits [m, H]."""
    return bf16_bits_from_f32(rng.standard_normal((m, hidden)).astype(np.float32))


def draw_normal_weights(rng: np.random.Generator, cfg: Workload, std: float = 0.02):
    """fp32 weights W13 [E, N1, H] and W2 [E, H, I] from N(0, std)."""
    e, h, i = cfg.num_experts, cfg.hidden, cfg.inter
    w13 = (rng.standard_normal((e, cfg.n1, h)) * std).astype(np.float32)
    w2 = (rng.standard_normal((e, h, i)) * std).astype(np.float32)
    return w13, w2


# Code bands for raw random weights. Nibbles are uniform over all 16 E2M1 codes.
# NVFP4: E4M3 block-scale bytes in [0x70, 0x7B] (128 .. 320) and a global dequant
# scale near 4e-5, so dequantised weights have an RMS close to 0.02.
# MXFP4: E8M0 bytes in [119, 121] (2^-8 .. 2^-6), again an RMS close to 0.02.
NVFP4_SCALE_BAND = (0x70, 0x7B)
NVFP4_GLOBAL_BAND = (3.5e-5, 4.5e-5)
MXFP4_SCALE_BAND = (119, 121)


def code_shapes(cfg: Workload):
    """Canonical packed shapes: nibbles [E, N, K/2] (element 2i low nibble) and scales [E, N, ceil(K/G)]."""
    e, h, i, g = cfg.num_experts, cfg.hidden, cfg.inter, cfg.group
    return {
        "w13": (e, cfg.n1, h // 2),
        "s13": (e, cfg.n1, -(-h // g)),
        "w2": (e, h, i // 2),
        "s2": (e, h, -(-i // g)),
    }


def draw_random_codes(cfg: Workload, seed: int, experts=None):
    """Random canonical code bytes (NumPy). ``experts`` limits the draw to a subset of experts.

    Every expert's codes come from its own stream (seed, expert), so a subset
    draw equals the matching slice of the full draw.
    """
    shapes = code_shapes(cfg)
    experts = list(range(cfg.num_experts)) if experts is None else list(experts)
    out = {k: np.empty((len(experts),) + v[1:], dtype=np.uint8) for k, v in shapes.items()}
    g13 = np.ones(len(experts), dtype=np.float32)
    g2 = np.ones(len(experts), dtype=np.float32)
    for j, e in enumerate(experts):
        r = _rng(seed * 100003 + 7919 * (e + 1))
        out["w13"][j] = r.integers(0, 256, size=shapes["w13"][1:], dtype=np.uint8)
        out["w2"][j] = r.integers(0, 256, size=shapes["w2"][1:], dtype=np.uint8)
        lo, hi = NVFP4_SCALE_BAND if cfg.fmt == "nvfp4" else MXFP4_SCALE_BAND
        out["s13"][j] = r.integers(lo, hi + 1, size=shapes["s13"][1:], dtype=np.uint8)
        out["s2"][j] = r.integers(lo, hi + 1, size=shapes["s2"][1:], dtype=np.uint8)
        if cfg.fmt == "nvfp4":
            g13[j] = r.uniform(*NVFP4_GLOBAL_BAND)
            g2[j] = r.uniform(*NVFP4_GLOBAL_BAND)
    out["g13"], out["g2"] = g13, g2
    return out


def draw_random_codes_torch(cfg: Workload, seed: int, device):
    """Random canonical code bytes drawn on a torch device (for workloads too large for host draws).

    Same bands as ``draw_random_codes`` but a different stream (torch's Philox).
    """
    import torch

    shapes = code_shapes(cfg)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {}
    lo, hi = NVFP4_SCALE_BAND if cfg.fmt == "nvfp4" else MXFP4_SCALE_BAND
    for key in ("w13", "w2"):
        out[key] = torch.randint(0, 256, shapes[key], generator=gen, device=device, dtype=torch.uint8)
    for key in ("s13", "s2"):
        out[key] = torch.randint(lo, hi + 1, shapes[key], generator=gen, device=device, dtype=torch.uint8)
    e = cfg.num_experts
    if cfg.fmt == "nvfp4":
        a, b = NVFP4_GLOBAL_BAND
        out["g13"] = (torch.rand(e, generator=gen, device=device) * (b - a) + a).float()
        out["g2"] = (torch.rand(e, generator=gen, device=device) * (b - a) + a).float()
    else:
        out["g13"] = torch.ones(e, device=device, dtype=torch.float32)
        out["g2"] = torch.ones(e, device=device, dtype=torch.float32)
    return out
