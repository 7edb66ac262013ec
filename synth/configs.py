"""The five synthetic workloads of the fused W4A16 MoE layer.

Shapes, formats, activations and routing recipes follow the workload list that
accompanies the FlashInfer page (PR 4255, "Performance" section names a
Nemotron-variant MoE shape without printing it; these shapes stand in for it).
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    num_experts: int          # local experts E (after expert_map)
    num_global_experts: int   # Eg; equals E when there is no expert_map
    hidden: int               # H
    inter: int                # I
    topk: int                 # k
    ms: Tuple[int, ...]       # token counts the workload is run at
    fmt: str                  # "nvfp4" (E4M3 scale / 16 + fp32 global) or "mxfp4" (E8M0 / 32)
    act: str                  # "silu_swiglu" or "relu2"
    routing: str              # "softmax", "sigmoid" or "zipf"
    renormalize: bool = True
    invalid_frac: float = 0.0
    use_expert_map: bool = False
    zipf_s: float = 1.1
    note: str = field(default="", compare=False)

    @property
    def n1(self) -> int:
        """FC1 output rows per expert: 2I for SwiGLU (gate and up), I for relu2."""
        return 2 * self.inter if self.act == "silu_swiglu" else self.inter

    @property
    def group(self) -> int:
        return 16 if self.fmt == "nvfp4" else 32


CONFIGS = {
    "tiny": Workload(
        name="tiny", index=0, num_experts=8, num_global_experts=8, hidden=256, inter=128,
        topk=2, ms=(4,), fmt="mxfp4", act="silu_swiglu", routing="softmax",
        note="correctness only; launch bound"),
    "decode": Workload(
        name="decode", index=1, num_experts=128, num_global_experts=128, hidden=4096,
        inter=1536, topk=8, ms=(1, 4, 8), fmt="nvfp4", act="silu_swiglu", routing="softmax",
        note="weight-bandwidth bound"),
    "small": Workload(
        name="small", index=2, num_experts=128, num_global_experts=128, hidden=2688,
        inter=1856, topk=6, ms=(16, 64), fmt="nvfp4", act="relu2", routing="sigmoid",
        note="non-gated relu2; HBM bound"),
    "prefill": Workload(
        name="prefill", index=3, num_experts=256, num_global_experts=256, hidden=7168,
        inter=2048, topk=8, ms=(2048,), fmt="nvfp4", act="silu_swiglu", routing="zipf",
        note="MFMA bound; skewed expert loads"),
    "edge": Workload(
        name="edge", index=4, num_experts=64, num_global_experts=128, hidden=3072,
        inter=1400, topk=4, ms=(512, 300, 511), fmt="mxfp4", act="silu_swiglu",
        routing="softmax", invalid_frac=0.05, use_expert_map=True,
        note="E8M0 scale tail (I=1400), expert_map, invalid ids, capacity reuse"),
}


def get_config(name: str) -> Workload:
    return CONFIGS[name]


def scaled(cfg: Workload, *, num_experts: Optional[int] = None, hidden: Optional[int] = None,
           inter: Optional[int] = None, num_global_experts: Optional[int] = None,
           name: Optional[str] = None) -> Workload:
    """A smaller copy of a workload (same format, activation and routing recipe)."""
    e = num_experts if num_experts is not None else cfg.num_experts
    eg = num_global_experts if num_global_experts is not None else (
        e if not cfg.use_expert_map else max(cfg.num_global_experts * e // cfg.num_experts, e))
    return Workload(
        name=name or (cfg.name + "_scaled"), index=cfg.index, num_experts=e,
        num_global_experts=eg, hidden=hidden or cfg.hidden, inter=inter or cfg.inter,
        topk=cfg.topk, ms=cfg.ms, fmt=cfg.fmt, act=cfg.act, routing=cfg.routing,
        renormalize=cfg.renormalize, invalid_frac=cfg.invalid_frac,
        use_expert_map=cfg.use_expert_map, zipf_s=cfg.zipf_s, note=cfg.note)
