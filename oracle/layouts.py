"""Source weight layouts other than the canonical one (oracle; test infrastructure).

FlashInfer PR 4255, Summary (ModelOpt, CompressedTensors and FP4 E8M0 formats) and
Walkthrough (weight format preparation: layout normalisation, scale packing, W13
rotation), and the review of the preparation module (a single-scale branch beside the
grouped one). The pages name these variants without spelling them out. Readings:

* W13 half order: the checkpoint may store the up half of W13 before the gate half (rows
  [0, I) up, [I, 2I) gate); canonical order is gate first.
* W13 row interleave: the two halves may be stored row by row alternately instead of one
  after the other (row 2i = row i of the first half, row 2i + 1 = row i of the second);
  combined with the half order above, "first half" is the up half.
* Global scale sense: the ModelOpt convention stores the NVFP4 global dequant multiplier
  g (weights = code x block scale x g); the CompressedTensors convention stores its
  reciprocal, the encode scale 1/g. The canonical value is the fp32 quotient 1 / stored,
  correctly rounded (IEEE division), as the device computes it.
* Single scale: one scale byte per row (group size -1, or one group spanning all of K)
  instead of one per group of G along K; canonical scales repeat it for every group.

Each function returns canonical arrays (no arithmetic beyond the fp32 reciprocal).
"""

from __future__ import annotations

import numpy as np


def w13_gate_first(rows: np.ndarray, inter: int) -> np.ndarray:
    """[E, 2I, ...] with up rows first -> gate rows first (the two halves swapped)."""
    a = np.asarray(rows)
    if a.shape[1] != 2 * inter:
        raise ValueError("W13 must have 2*inter rows")
    return np.concatenate([a[:, inter:], a[:, :inter]], axis=1)


def w13_halves(rows: np.ndarray, inter: int) -> np.ndarray:
    """[E, 2I, ...] with the two halves interleaved row by row (rows 2i, 2i + 1 = row i of the
    first and the second half) -> the halves one after the other."""
    a = np.asarray(rows)
    if a.shape[1] != 2 * inter:
        raise ValueError("W13 must have 2*inter rows")
    return np.concatenate([a[:, 0::2], a[:, 1::2]], axis=1)


def global_from_encode(g_stored) -> np.ndarray:
    """Stored encode scale 1/g -> canonical dequant multiplier g, fp32 correctly rounded."""
    s = np.asarray(g_stored, dtype=np.float32)
    return (np.float32(1.0) / s).astype(np.float32)


def scales_from_per_row(per_row: np.ndarray, k: int, group: int) -> np.ndarray:
    """[E, N, 1] one scale byte per row -> [E, N, ceil(K/G)] (the byte repeated)."""
    a = np.asarray(per_row, dtype=np.uint8)
    if a.ndim != 3 or a.shape[2] != 1:
        raise ValueError("per-row scales must have shape [E, N, 1]")
    return np.repeat(a, -(-k // group), axis=2)


def canonical(fmt: str, act: str, hidden: int, inter: int, w13, s13, g13, w2, s2, g2,
              w13_up_first: bool = False, global_scale_reciprocal: bool = False, scale_per_row: bool = False,
              w13_interleaved: bool = False):
    """Canonical (w13, s13, g13, w2, s2, g2) from a source layout described by the flags."""
    group = 16 if fmt == "nvfp4" else 32
    if scale_per_row:
        s13 = scales_from_per_row(s13, hidden, group)
        s2 = scales_from_per_row(s2, inter, group)
    if w13_interleaved and act == "silu_swiglu":
        w13 = w13_halves(w13, inter)
        s13 = w13_halves(s13, inter)
    if w13_up_first and act == "silu_swiglu":
        w13 = w13_gate_first(w13, inter)
        s13 = w13_gate_first(s13, inter)
    if fmt == "nvfp4" and global_scale_reciprocal:
        g13 = global_from_encode(g13)
        g2 = global_from_encode(g2)
    return w13, s13, g13, w2, s2, g2
