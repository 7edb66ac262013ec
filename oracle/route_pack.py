"""Route packing (oracle; test infrastructure).

FlashInfer PR 4255, Description: route packing is specialised on a power-of-two
token capacity instead of the exact token count, and the W4A16 workspaces are
sized to the same capacity. Tests section: packing is checked against a host
reference covering expert_map, invalid expert ids, preallocated buffers and the
workspace capacity contract. Review round 1: the capacity helper takes the
token count (its top-k argument is unused) and the packed-route and route-block
capacities are clamped to at least one.

Readings (the page gives no formula):
* token capacity  cap = next power of two of max(m, 1);
* a route is r = t*k + j; its local expert is expert_map[g] (or g with no
  map) for the global id g = topk_ids[t, j]; it is dropped when g < 0,
  g >= Eg, or the local id is outside [0, E);
* each expert's segment holds its routes in ascending r and is padded with -1
  to a multiple of the block size B;
* cap_routes = max(round_up(cap*k + min(E, cap*k)*(B-1), B), B) bounds the
  padded total for any m <= cap; cap_blocks = cap_routes / B.
"""

from __future__ import annotations

import numpy as np


def token_capacity(m: int) -> int:
    if m < 0:
        raise ValueError("m must be >= 0")
    c = 1
    while c < max(m, 1):
        c *= 2
    return c


def capacities(cap: int, topk: int, num_experts: int, block: int):
    """(cap_routes, cap_blocks) for a token capacity."""
    routes = cap * topk
    bound = routes + min(num_experts, routes) * (block - 1)
    cap_routes = max(-(-bound // block) * block, block)
    return cap_routes, cap_routes // block


def local_ids(topk_ids: np.ndarray, expert_map, num_global_experts: int, num_experts: int) -> np.ndarray:
    """Flat local expert id per route, -1 for dropped routes."""
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    out = np.full(flat.shape, -1, dtype=np.int64)
    for r, g in enumerate(flat):
        if g < 0 or g >= num_global_experts:
            continue
        lid = int(expert_map[g]) if expert_map is not None else int(g)
        if 0 <= lid < num_experts:
            out[r] = lid
    return out


def route_pack(topk_ids: np.ndarray, expert_map, num_global_experts: int, num_experts: int,
               block: int, cap: int):
    """Group routes by local expert.

    Returns a dict of int32 arrays:
      expert_counts [E]          valid routes per expert
      expert_offsets [E+1]       padded segment starts (multiples of B)
      sorted_route_ids [cap_routes]  route id per packed slot, -1 for padding
      block_expert [cap_blocks]  expert of each B-row block, -1 after the live blocks
      live [4]                   (valid routes, padded routes, live blocks, m)
      route_slot [cap*k]         packed slot of each route, -1 if dropped or r >= m*k
    """
    topk_ids = np.asarray(topk_ids)
    m, k = topk_ids.shape
    if m > cap:
        raise ValueError("m exceeds the token capacity")
    E = num_experts
    cap_routes, cap_blocks = capacities(cap, k, E, block)
    lid = local_ids(topk_ids, expert_map, num_global_experts, E)

    counts = np.zeros(E, dtype=np.int64)
    for le in lid:
        if le >= 0:
            counts[le] += 1
    padded = -(-counts // block) * block
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + padded[e]

    sorted_ids = np.full(cap_routes, -1, dtype=np.int64)
    route_slot = np.full(cap * k, -1, dtype=np.int64)
    fill = offsets[:-1].copy()
    for r, le in enumerate(lid):                          # ascending r => stable within a segment
        if le < 0:
            continue
        slot = fill[le]
        fill[le] += 1
        sorted_ids[slot] = r
        route_slot[r] = slot

    block_expert = np.full(cap_blocks, -1, dtype=np.int64)
    for e in range(E):
        for b in range(offsets[e] // block, offsets[e + 1] // block):
            block_expert[b] = e

    live = np.array([counts.sum(), offsets[E], offsets[E] // block, m], dtype=np.int64)
    return {
        "expert_counts": counts.astype(np.int32),
        "expert_offsets": offsets.astype(np.int32),
        "sorted_route_ids": sorted_ids.astype(np.int32),
        "block_expert": block_expert.astype(np.int32),
        "live": live.astype(np.int32),
        "route_slot": route_slot.astype(np.int32),
    }
