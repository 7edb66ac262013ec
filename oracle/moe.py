"""The MoE layer forward pass (oracle; test infrastructure).

FlashInfer PR 4255, Description: a fused FC1/FC2 mixture-of-experts kernel on
4-bit weights with bf16 activations (W4A16); Performance: relu2 and silu
activations; the top-k router-weighted sum is folded into FC2's store. For each
token t and each of its k routes (t, j) whose expert e survives remapping:

    h = W13_e x_t                      (W13_e dequantised, [N1, H])
    a = silu(h[:I]) * h[I:]            SiLU-SwiGLU (gate rows first, then up rows)
    a = max(h, 0)^2                    relu2 (W1_e has only I rows)
    y = W2_e a                         (W2_e dequantised, [H, I])
    out_t += w[t, j] * y

Dropped routes contribute nothing and the remaining weights are not
renormalised; a token with no surviving route gives a zero row. Everything is
float64 with exact exp; the result is rounded to bf16 only for comparison.
"""

from __future__ import annotations

import numpy as np

from . import formats
from .route_pack import local_ids


def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def activation(h: np.ndarray, act: str, inter: int) -> np.ndarray:
    """Apply the activation to FC1 outputs along the last axis."""
    if act == "silu_swiglu":
        return silu(h[..., :inter]) * h[..., inter:2 * inter]
    if act == "relu2":
        r = np.maximum(h, 0.0)
        return r * r
    raise ValueError(f"unknown activation {act!r}")


class Experts:
    """Dequantised expert weights, decoded on first use from the canonical packed codes.

    Canonical layout: w13 nibbles [E, N1, H/2], s13 scale bytes [E, N1, ceil(H/G)],
    w2 nibbles [E, H, I/2], s2 [E, H, ceil(I/G)], g13 / g2 fp32 [E] (NVFP4 only).
    ``expert_ids`` maps a row of these arrays to its local expert id when only a
    subset of experts is held. ``cache=False`` decodes on every use and keeps
    nothing (bounded memory for layers with many large experts; the values are
    the same either way).
    """

    def __init__(self, fmt: str, act: str, hidden: int, inter: int, codes: dict, expert_ids=None,
                 cache: bool = True):
        self.fmt, self.act, self.hidden, self.inter = fmt, act, hidden, inter
        self.codes = codes
        n = codes["w13"].shape[0]
        ids = list(range(n)) if expert_ids is None else list(expert_ids)
        self.row = {int(e): i for i, e in enumerate(ids)}
        self.cache = cache
        self._w13, self._w2 = {}, {}

    def _g(self, key, i):
        if self.fmt != "nvfp4":
            return None
        return np.asarray(self.codes[key], dtype=np.float32)[i:i + 1]

    def w13(self, e: int) -> np.ndarray:
        if e in self._w13:
            return self._w13[e]
        i = self.row[e]
        w = formats.dequant(self.fmt, self.codes["w13"][i:i + 1], self.codes["s13"][i:i + 1], self._g("g13", i))[0]
        if self.cache:
            self._w13[e] = w
        return w

    def w2(self, e: int) -> np.ndarray:
        if e in self._w2:
            return self._w2[e]
        i = self.row[e]
        w = formats.dequant(self.fmt, self.codes["w2"][i:i + 1], self.codes["s2"][i:i + 1], self._g("g2", i))[0]
        if self.cache:
            self._w2[e] = w
        return w


def fc2_input(a: np.ndarray, mxfp8: bool) -> np.ndarray:
    """The FC2 operand: the activation output itself (W4A16), or for the W4A8 variant its
    MXFP8 quantisation along I, dequantised (the router weight is applied after FC2 either
    way, so it is not quantised)."""
    if not mxfp8:
        return a
    return formats.dequant_mxfp8(*formats.quantise_mxfp8(a))


def moe_forward_loop(x: np.ndarray, topk_ids, topk_weights, expert_map, num_global_experts: int,
                     num_experts: int, experts: Experts, mxfp8: bool = False) -> np.ndarray:
    """Route-by-route forward (the definition written out). x: float64 [m, H].
    ``mxfp8``: the W4A8 variant (the activation output quantised to MXFP8 before FC2)."""
    x = np.asarray(x, dtype=np.float64)
    m, k = np.asarray(topk_ids).shape
    lid = local_ids(topk_ids, expert_map, num_global_experts, num_experts).reshape(m, k)
    w = np.asarray(topk_weights, dtype=np.float64)
    out = np.zeros((m, experts.hidden), dtype=np.float64)
    for t in range(m):
        for j in range(k):
            e = int(lid[t, j])
            if e < 0:
                continue
            h = experts.w13(e) @ x[t]
            a = fc2_input(activation(h, experts.act, experts.inter), mxfp8)
            out[t] += w[t, j] * (experts.w2(e) @ a)
    return out


def moe_forward(x: np.ndarray, topk_ids, topk_weights, expert_map, num_global_experts: int,
                num_experts: int, experts: Experts, tokens=None, cols=None, mxfp8: bool = False) -> np.ndarray:
    """Expert-grouped forward: the same per-route products, batched per expert with a matmul.

    ``tokens`` / ``cols`` restrict the result to a subset of tokens and output
    columns (sampled checks of large workloads); FC1 and the activation are
    always computed in full for the routes involved.
    """
    x = np.asarray(x, dtype=np.float64)
    m, k = np.asarray(topk_ids).shape
    tokens = np.arange(m) if tokens is None else np.asarray(tokens, dtype=np.int64)
    cols = np.arange(experts.hidden) if cols is None else np.asarray(cols, dtype=np.int64)
    lid = local_ids(topk_ids, expert_map, num_global_experts, num_experts).reshape(m, k)
    w = np.asarray(topk_weights, dtype=np.float64)
    out = np.zeros((len(tokens), len(cols)), dtype=np.float64)
    sub = lid[tokens]                                      # [T, k]
    for e in np.unique(sub[sub >= 0]):
        tt, jj = np.nonzero(sub == e)                      # rows of `out`, route index
        h = x[tokens[tt]] @ experts.w13(int(e)).T          # [R, N1]
        a = fc2_input(activation(h, experts.act, experts.inter), mxfp8)   # [R, I]
        y = a @ experts.w2(int(e))[cols].T                 # [R, len(cols)]
        np.add.at(out, tt, w[tokens[tt], jj][:, None] * y)
    return out


def within_tolerance(got_bf16_values: np.ndarray, ref: np.ndarray, rel: float = 2e-2, abs_: float = 1e-3):
    """Compare in bf16: max|got - bf16(ref)| <= rel * max|bf16(ref)| + abs_. Returns (ok, err, bound)."""
    ref_b = formats.bf16_round(ref)
    got = np.asarray(got_bf16_values, dtype=np.float64)
    if got.shape != ref_b.shape:
        raise ValueError(f"shape mismatch {got.shape} vs {ref_b.shape}")
    if not np.all(np.isfinite(got)):
        return False, float("inf"), 0.0
    err = float(np.max(np.abs(got - ref_b))) if got.size else 0.0
    bound = rel * (float(np.max(np.abs(ref_b))) if ref_b.size else 0.0) + abs_
    return err <= bound, err, bound
