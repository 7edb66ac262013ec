"""Pins for the oracle's MoE forward (CPU only): hand cases, reduction to a dense
MLP, linearity, drop semantics, duplicate routes and bug-detecting checks."""

import json
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as M
from synth import configs as C
from synth import draw as D

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "moe_hand_cases.json")


def _hand_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def build_hand_case(case):
    """Canonical codes and inputs of a hand case (shared with the GPU parity tests)."""
    h, i = case["hidden"], case["inter"]
    x = np.zeros((1, h))
    for t, col, v in case["x_nonzero"]:
        x[t, col] = v
    w13 = np.zeros(case["w13_bytes"]["shape"], dtype=np.uint8)
    for e, r, c, v in case["w13_bytes"]["nonzero"]:
        w13[e, r, c] = v
    s13 = np.array(case["s13"]["values"], dtype=np.uint8).reshape(case["s13"]["shape"])
    g = 16 if case["fmt"] == "nvfp4" else 32
    w2 = np.full((1, h, i // 2), case["w2_fill_byte"], dtype=np.uint8)
    s2 = np.full((1, h, -(-i // g)), case["s2_fill"], dtype=np.uint8)
    codes = {"w13": w13, "s13": s13, "w2": w2, "s2": s2,
             "g13": np.array(case.get("g13", [1.0]), dtype=np.float32),
             "g2": np.array(case.get("g2", [1.0]), dtype=np.float32)}
    return x, codes


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_hand_cases(case):
    x, codes = build_hand_case(case)
    ex = M.Experts(case["fmt"], case["act"], case["hidden"], case["inter"], codes)
    ids = np.array(case["topk_ids"], dtype=np.int32)
    w = np.array(case["topk_weights"], dtype=np.float32)
    for fn in (M.moe_forward, M.moe_forward_loop):
        out = fn(x, ids, w, None, 1, 1, ex)
        assert np.allclose(out, case["expect_out_all"], rtol=1e-15, atol=0)
        assert np.all(F.bf16_round(out) == case["expect_bf16"])


def _small_setup(act="silu_swiglu", fmt="mxfp4", E=4, H=64, I=32, k=2, m=6, seed=0):
    cfg = C.Workload(name="t", index=0, num_experts=E, num_global_experts=E, hidden=H, inter=I, topk=k,
                     ms=(m,), fmt=fmt, act=act, routing="softmax")
    ids, w, emap, rng = D.draw_routing(cfg, m, seed)
    x = F.bf16_bits_to_f64(D.draw_activations_bf16(rng, m, H))
    w13, w2 = D.draw_normal_weights(rng, cfg)
    if fmt == "mxfp4":
        p13, s13 = F.quantise_mxfp4(w13)
        p2, s2 = F.quantise_mxfp4(w2)
        g13 = g2 = np.ones(E, dtype=np.float32)
    else:
        p13, s13, g13 = F.quantise_nvfp4(w13)
        p2, s2, g2 = F.quantise_nvfp4(w2)
    codes = {"w13": p13, "s13": s13, "w2": p2, "s2": s2, "g13": g13, "g2": g2}
    return cfg, x, ids, w, M.Experts(fmt, act, H, I, codes)


@pytest.mark.parametrize("act", ["silu_swiglu", "relu2"])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_single_expert_reduces_to_dense_mlp(act, fmt):
    cfg, x, _, _, ex = _small_setup(act=act, fmt=fmt, E=1, k=1)
    m = x.shape[0]
    ids = np.zeros((m, 1), dtype=np.int32)
    w = np.ones((m, 1), dtype=np.float32)
    out = M.moe_forward(x, ids, w, None, 1, 1, ex)
    W13, W2 = ex.w13(0), ex.w2(0)
    hh = x @ W13.T
    if act == "silu_swiglu":
        g, u = hh[:, :cfg.inter], hh[:, cfg.inter:]
        a = g / (1 + np.exp(-g)) * u
    else:
        a = np.where(hh > 0, hh * hh, 0.0)
    assert np.allclose(out, a @ W2.T, rtol=1e-12, atol=1e-14)


def test_grouped_equals_route_loop_and_samples():
    cfg, x, ids, w, ex = _small_setup(E=5, k=3, m=9, seed=3)
    a = M.moe_forward(x, ids, w, None, 5, 5, ex)
    b = M.moe_forward_loop(x, ids, w, None, 5, 5, ex)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-15)
    toks, cols = np.array([8, 0, 3]), np.array([5, 63, 0, 17])
    s = M.moe_forward(x, ids, w, None, 5, 5, ex, tokens=toks, cols=cols)
    assert np.allclose(s, a[np.ix_(toks, cols)], rtol=1e-12, atol=1e-15)


def test_router_weight_linearity():
    cfg, x, ids, w, ex = _small_setup(seed=4)
    a = M.moe_forward(x, ids, w, None, 4, 4, ex)
    b = M.moe_forward(x, ids, w.astype(np.float64) * 3.0, None, 4, 4, ex)
    assert np.allclose(b, 3.0 * a, rtol=1e-12, atol=1e-15)


def test_dropped_route_equals_zero_weight_and_no_renormalisation():
    cfg, x, ids, w, ex = _small_setup(seed=5)
    ids2, w2 = ids.copy(), w.copy()
    ids2[1, 0] = -1
    w2[1, 0] = 0.0
    a = M.moe_forward(x, ids2, w, None, 4, 4, ex)
    b = M.moe_forward(x, ids, w2, None, 4, 4, ex)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-15)
    ids3 = ids.copy()
    ids3[2, :] = -1
    c = M.moe_forward(x, ids3, w, None, 4, 4, ex)
    assert np.all(c[2] == 0)


def test_duplicate_expert_counts_twice():
    cfg, x, ids, w, ex = _small_setup(seed=6)
    dup = ids.copy()
    dup[:, 1] = dup[:, 0]
    a = M.moe_forward(x, dup, w, None, 4, 4, ex)
    single = np.stack([ids[:, 0], -np.ones_like(ids[:, 0])], axis=1).astype(np.int32)
    w64 = w.astype(np.float64)
    b = M.moe_forward(x, single, np.stack([w64.sum(axis=1), w64[:, 1]], axis=1), None, 4, 4, ex)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-15)


def test_expert_map_routes_to_local_ids():
    cfg, x, ids, w, ex = _small_setup(seed=7)
    emap = np.array([3, 2, 1, 0, -1, -1, -1, -1], dtype=np.int32)   # 8 global ids onto 4 local
    gids = 3 - ids                                                  # global id whose map gives ids
    a = M.moe_forward(x, gids.astype(np.int32), w, emap, 8, 4, ex)
    b = M.moe_forward(x, ids, w, None, 4, 4, ex)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-15)
    c = M.moe_forward(x, (ids + 4).astype(np.int32), w, emap, 8, 4, ex)   # all unmapped
    assert np.all(c == 0)


def test_swapping_gate_and_up_changes_the_result():
    cfg, x, ids, w, ex = _small_setup(seed=8)
    a = M.moe_forward(x, ids, w, None, 4, 4, ex)
    I = cfg.inter
    codes = dict(ex.codes)
    codes["w13"] = np.concatenate([ex.codes["w13"][:, I:], ex.codes["w13"][:, :I]], axis=1)
    codes["s13"] = np.concatenate([ex.codes["s13"][:, I:], ex.codes["s13"][:, :I]], axis=1)
    ex2 = M.Experts(cfg.fmt, cfg.act, cfg.hidden, I, codes)
    b = M.moe_forward(x, ids, w, None, 4, 4, ex2)
    assert not np.allclose(a, b, rtol=1e-3)


def test_tolerance_helper():
    ref = np.array([1.0, -2.0, 0.5])
    ok, err, bound = M.within_tolerance(F.bf16_round(ref), ref)
    assert ok and err == 0 and bound == pytest.approx(2e-2 * 2 + 1e-3)
    bad = F.bf16_round(ref) + np.array([0, 0.05, 0])
    assert not M.within_tolerance(bad, ref)[0]
    assert not M.within_tolerance(np.array([np.nan, 0, 0]), ref)[0]
