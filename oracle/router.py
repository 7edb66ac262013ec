"""Router front end (oracle; test infrastructure).

FlashInfer PR 4255, Summary (New Features: configurable routing) and Walkthrough (kernel
compilation and execution: routing modes): the pages name routing modes but print no
formula. Reading, taken from the workload definitions (softmax top-k over the router logits,
or sigmoid scores, top-k, renormalised):

* scores are softmax or sigmoid of the router logits of one token;
* the k experts with the largest scores are taken. Both maps are increasing, so these are
  the k largest logits; equal logits are taken in ascending expert id. The comparison is on
  the fp32 logits, the precision the kernel decides in;
* the weights are those scores, renormalised to sum to 1 over the k experts, or the raw
  scores without renormalisation. For softmax the renormalised weights are the softmax of
  the k selected logits alone (the full denominator cancels).

Weights are computed in float64. Logits must be finite.
"""

from __future__ import annotations

import numpy as np

SCORINGS = ("softmax", "sigmoid")


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Expert ids of the k largest fp32 logits of each row, largest first, equal values in
    ascending id: int32 [m, k]."""
    l32 = np.asarray(logits, dtype=np.float32)
    m, e = l32.shape
    if not 1 <= k <= e:
        raise ValueError("k must lie in [1, num_experts]")
    # A stable sort of the negated values keeps equal logits in ascending id.
    order = np.argsort(-l32, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def route(logits: np.ndarray, k: int, scoring: str = "softmax", renormalize: bool = True):
    """(topk_ids int32 [m, k], topk_weights float64 [m, k]) for fp32 logits [m, E]."""
    if scoring not in SCORINGS:
        raise ValueError(f"unknown scoring {scoring!r}")
    l32 = np.asarray(logits, dtype=np.float32)
    if not np.all(np.isfinite(l32)):
        raise ValueError("logits must be finite")
    ids = select_topk(l32, k)
    l = l32.astype(np.float64)
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    if scoring == "softmax":
        if renormalize:
            z = np.exp(sel - sel[:, :1])                 # the first selected logit is the row maximum
            w = z / z.sum(axis=1, keepdims=True)
        else:
            mx = l.max(axis=1, keepdims=True)
            w = np.exp(sel - mx) / np.exp(l - mx).sum(axis=1, keepdims=True)
    else:
        s = 1.0 / (1.0 + np.exp(-sel))
        w = s / s.sum(axis=1, keepdims=True) if renormalize else s
    return ids, w
