"""Pins for the oracle's route packing (CPU only): hand-computed cases, brute force
against NumPy's stable argsort, invariants and the power-of-two capacity."""

import json
import os

import numpy as np
import pytest

from oracle import route_pack as RP

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "route_pack_worked.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    ids = np.array(case["topk_ids"], dtype=np.int32)
    emap = None if case["expert_map"] is None else np.array(case["expert_map"], dtype=np.int32)
    cap = RP.token_capacity(ids.shape[0])
    got = RP.route_pack(ids, emap, case["num_global_experts"], case["num_experts"], case["block"], cap)
    for key, want in case["expect"].items():
        assert got[key].tolist() == want, key


@pytest.mark.parametrize("m,cap", [(0, 1), (1, 1), (2, 2), (3, 4), (4, 4), (5, 8), (300, 512), (511, 512),
                                   (512, 512), (513, 1024), (2048, 2048)])
def test_token_capacity(m, cap):
    assert RP.token_capacity(m) == cap


def test_token_capacity_rejects_negative():
    with pytest.raises(ValueError):
        RP.token_capacity(-1)


def test_capacity_shared_across_a_pow2_bucket():
    sizes = {RP.capacities(RP.token_capacity(m), 4, 64, 16) for m in (300, 511, 512)}
    assert len(sizes) == 1


def _brute(ids, emap, eg, E, B, cap):
    """Independent formulation: stable argsort of the local ids of the valid routes."""
    m, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    lid = np.full(flat.shape, -1)
    ok = (flat >= 0) & (flat < eg)
    lid[ok] = flat[ok] if emap is None else emap[flat[ok]]
    lid[(lid < 0) | (lid >= E)] = -1
    valid = np.nonzero(lid >= 0)[0]
    order = valid[np.argsort(lid[valid], kind="stable")]
    counts = np.bincount(lid[valid], minlength=E)
    padded = (counts + B - 1) // B * B
    off = np.concatenate([[0], np.cumsum(padded)])
    cap_routes, cap_blocks = RP.capacities(cap, k, E, B)
    sorted_ids = -np.ones(cap_routes, dtype=np.int64)
    pos = 0
    for e in range(E):
        seg = order[pos:pos + counts[e]]
        sorted_ids[off[e]:off[e] + counts[e]] = seg
        pos += counts[e]
    return counts, off, sorted_ids


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_against_stable_argsort(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(0, 60))
    k = int(rng.integers(1, 9))
    E = int(rng.integers(1, 20))
    use_map = bool(rng.integers(0, 2))
    eg = E + int(rng.integers(0, 10)) if use_map else E
    B = int(rng.choice([1, 2, 4, 16, 32, 64, 128]))
    ids = rng.integers(-2, eg + 2, size=(m, k)).astype(np.int32)
    emap = None
    if use_map:
        emap = rng.integers(-1, E + 1, size=eg).astype(np.int32)   # includes -1 and one out-of-range id
    cap = RP.token_capacity(m)
    got = RP.route_pack(ids, emap, eg, E, B, cap)
    counts, off, sorted_ids = _brute(ids, emap, eg, E, B, cap)
    assert got["expert_counts"].tolist() == counts.tolist()
    assert got["expert_offsets"].tolist() == off.tolist()
    assert got["sorted_route_ids"].tolist() == sorted_ids.tolist()
    # invariants
    s = got["sorted_route_ids"]
    valid_routes = s[s >= 0]
    assert len(set(valid_routes.tolist())) == len(valid_routes) == counts.sum()
    assert np.all(got["expert_offsets"] % B == 0)
    live = got["live"].tolist()
    assert live == [counts.sum(), off[-1], off[-1] // B, m]
    slot = got["route_slot"]
    for r in range(m * k):
        if slot[r] >= 0:
            assert s[slot[r]] == r
    assert np.count_nonzero(slot >= 0) == counts.sum()
    be = got["block_expert"]
    assert np.all(be[live[2]:] == -1)
    for b in range(live[2]):
        e = be[b]
        assert off[e] <= b * B < off[e + 1]


def test_every_dropped_kind_is_dropped():
    ids = np.array([[-1, -5, 3, 100]], dtype=np.int32)      # -1, below -1, valid, >= Eg
    got = RP.route_pack(ids, None, 4, 4, 16, 1)
    assert got["live"][0] == 1 and got["sorted_route_ids"][0] == 2
