"""GPU parity of the W4A8 variant (moe_w4a8_fused) against the oracle's W4A8 forward.

The activation output is rounded to MXFP8 (E4M3, one E8M0 scale per 32 along the
intermediate axis) before FC2 and the router weight is applied after FC2 (FlashInfer
PR 4255, review: grouped MXFP8 quantisation of the SiLU-mul output). MXFP4 weights only.
Tolerance as for the W4A16 layer: max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3 in bf16.
"""

from __future__ import annotations

import numpy as np
import pytest

from _common import SCALED, bf16_tensor_to_f64, dev, full_case, make_case, make_layer, oracle_out, run_layer
from oracle import formats as F
from oracle import moe as M
from oracle import route_pack as RP
from synth import configs as C
from synth import draw as D

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    return d


@pytest.fixture(scope="module")
def moe():
    import fp4_weight_grouped_moe_amd as m
    yield m
    m.moe_w4a16_set_path("auto")


def _say(msg):
    print(msg, flush=True)


def _check(case, got, tokens=None, cols=None, label=""):
    ref = oracle_out(case, tokens=tokens, cols=cols, mxfp8=True)
    if tokens is not None or cols is not None:
        t = np.arange(case.m) if tokens is None else np.asarray(tokens)
        c = np.arange(case.cfg.hidden) if cols is None else np.asarray(cols)
        got = got[np.ix_(t, c)]
    ok, err, bound = M.within_tolerance(got, ref)
    _say(f"  {label}: max|err| = {err:.3e}, bound = {bound:.3e}, max|ref| = {np.max(np.abs(ref)):.3e}")
    assert ok, f"{label}: {err} > {bound}"


def _mx_weights(rows, cols, entries):
    codes = np.zeros((1, rows, cols), np.uint8)
    for (r, c), v in entries.items():
        codes[0, r, c] = v
    return F.pack_nibbles(codes), np.full((1, rows, -(-cols // 32)), 127, np.uint8)


@pytest.mark.parametrize("path", ["decode", "gemm"])
def test_hand_layer_exact(moe, device, path):
    """E = 1, H = 32, I = 32, relu2, x = [1, 0.25, 0...]: h = [3, 1.25], a = [9, 1.5625]; MXFP8
    rounds 1.5625 * 2^5 = 50 (a tie) to 48, so a = [9, 1.5] and every output is 9 + 2 * 1.5 = 12
    (W4A16: 12.125). The oracle's hand case, through the GPU bit for bit."""
    w1, s1 = _mx_weights(32, 32, {(0, 0): 0x5, (1, 0): 0x2, (1, 1): 0x2})
    w2, s2 = _mx_weights(32, 32, {**{(r, 0): 0x2 for r in range(32)}, **{(r, 1): 0x4 for r in range(32)}})
    layer = moe.MoeLayer("mxfp4", "relu2", 1, 32, 32, 1, 1, device=device)
    layer.prepare(dev(w1, device), dev(s1, device), None, dev(w2, device), dev(s2, device), None)
    x = torch.zeros((1, 32), dtype=torch.bfloat16, device=device)
    x[0, 0], x[0, 1] = 1.0, 0.25
    ids = torch.zeros((1, 1), dtype=torch.int32, device=device)
    w = torch.ones((1, 1), dtype=torch.float32, device=device)
    moe.moe_w4a16_set_path(path)
    try:
        o8 = bf16_tensor_to_f64(layer(x, ids, w, w4a8=True))
        o16 = bf16_tensor_to_f64(layer(x, ids, w))
    finally:
        moe.moe_w4a16_set_path("auto")
    _say(f"hand W4A8 {path}: {o8[0, :4]} / W4A16 {o16[0, :4]}")
    assert np.all(o8 == 12.0) and np.all(o16 == 12.125)


W4A8_CASES = [("tiny", 4), ("edge_s", 1), ("edge_s", 3), ("edge_s", 8), ("edge_s", 100)]


@pytest.mark.parametrize("name,m", W4A8_CASES)
@pytest.mark.parametrize("path", ["auto", "decode", "gemm"])
def test_w4a8_matches_oracle_scaled(moe, device, name, m, path):
    if path == "decode" and m > moe.MOE_DECODE_MAX_M:
        pytest.skip("decode path serves m <= 16")
    cfg = SCALED[name]
    _say(f"w4a8 {name} m={m} path={path}")
    case = make_case(cfg, m, seed=cfg.index * 11 + m, weights="normal")
    if m > 2:
        case.ids[1, 0] = -1
        case.ids[2, :] = -1                      # a token with no surviving route
    layer = make_layer(case, device)
    moe.moe_w4a16_set_path(path)
    try:
        got8 = bf16_tensor_to_f64(run_layer(layer, case, device, w4a8=True))
        again = bf16_tensor_to_f64(run_layer(layer, case, device, w4a8=True))
        got16 = bf16_tensor_to_f64(run_layer(layer, case, device))
    finally:
        moe.moe_w4a16_set_path("auto")
    assert np.array_equal(got8, again)
    assert not np.array_equal(got8, got16)       # the rounding to MXFP8 is applied
    if m > 2:
        assert np.all(got8[2] == 0)
    _check(case, got8, label=f"w4a8 {name} m={m} {path}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("m", [512, 16, 8])
def test_w4a8_full_size_edge_every_output(moe, device, m):
    """Full-size edge shape: m = 512 on the grouped GEMM, m = 16 and 8 on the decode path (FC2 on
    the block-scaled FP4 x FP8 MFMA on both). Every token x every column against the W4A8
    oracle."""
    case = full_case("edge", m, device)
    layer = make_layer(case, device, token_capacity=RP.token_capacity(m))
    _say(f"w4a8 full edge m={m}")
    got = bf16_tensor_to_f64(run_layer(layer, case, device, w4a8=True))
    assert np.all(np.isfinite(got))
    ref = oracle_out(case, mxfp8=True)
    ok, err, bound = M.within_tolerance(got, ref)
    _say(f"  w4a8 edge m={m}: max|err| = {err:.3e}, bound = {bound:.3e}")
    assert ok, f"w4a8 edge m={m}: {err} > {bound}"
    del layer, case
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_w4a8_full_size_prefill_mxfp4_every_output(moe, device):
    """The prefill shape (256 experts, hidden 7168, inter 2048, top-8, Zipf routing, m = 2048)
    with MXFP4 weights: the grouped GEMM's MXFP8-rounding FC1 epilogue and block-scaled FC2 over
    full 8-block tiles, 16 / 28 N tiles per M tile and the per-XCD queues. Every token x every
    column against the W4A8 oracle; W4A16 on the same layer differs (the rounding is applied)."""
    case = full_case("prefill", 2048, device, fmt="mxfp4")
    layer = make_layer(case, device)
    _say("w4a8 full prefill mxfp4 m=2048")
    got = bf16_tensor_to_f64(run_layer(layer, case, device, w4a8=True))
    assert np.all(np.isfinite(got))
    ref = oracle_out(case, mxfp8=True)
    ok, err, bound = M.within_tolerance(got, ref)
    _say(f"  w4a8 prefill mxfp4: max|err| = {err:.3e}, bound = {bound:.3e}")
    assert ok, f"w4a8 prefill mxfp4: {err} > {bound}"
    del layer, case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("act", ["relu2", "silu_swiglu"])
@pytest.mark.parametrize("path,m", [("decode", 5), ("decode", 16), ("gemm", 40), ("gemm", 512)])
def test_w4a8_both_activations(moe, device, act, path, m):
    """Both activations on both paths: with relu2 a grouped-GEMM wave holds whole MX groups in
    its FC1 epilogue, with SiLU-SwiGLU two waves exchange their halves' maxima; m = 512 puts
    ~150 routes on each of the 8 local experts (full 8-block tiles). Every output against the
    oracle's W4A8 forward, and a second call equal to the first."""
    import dataclasses
    cfg = dataclasses.replace(C.get_config("edge"), num_experts=8, num_global_experts=16, hidden=512, inter=384,
                              act=act, name=f"edge_w4a8_{act}")
    _say(f"w4a8 {act} m={m} path={path}")
    case = make_case(cfg, m, seed=m * 3 + len(act), weights="normal")
    layer = make_layer(case, device)
    moe.moe_w4a16_set_path(path)
    try:
        got = bf16_tensor_to_f64(run_layer(layer, case, device, w4a8=True))
        again = bf16_tensor_to_f64(run_layer(layer, case, device, w4a8=True))
    finally:
        moe.moe_w4a16_set_path("auto")
    assert np.array_equal(got, again)
    ok, err, bound = M.within_tolerance(got, oracle_out(case, mxfp8=True))
    _say(f"  max|err| = {err:.3e}, bound = {bound:.3e}")
    assert ok, f"w4a8 {act} m={m} {path}: {err} > {bound}"


@pytest.mark.parametrize("topk", [8, 16])
def test_w4a8_decode_fallback_many_routes(moe, device, topk):
    """More than 128 routes on the decode path (m = 12 at top-16): the K-split FC2 cannot stage
    every route's slice, so the rounding pass writes the exact MXFP8 values as bf16 rows for the
    one-pass FC2; at top-8 (96 routes) the block-scaled FC2 runs. Against the W4A8 oracle."""
    import dataclasses
    cfg = dataclasses.replace(C.get_config("edge"), num_experts=32, num_global_experts=64, hidden=512, inter=256,
                              topk=topk, name=f"edge_w4a8_top{topk}")
    m = 12
    _say(f"w4a8 decode top{topk} m={m}")
    case = make_case(cfg, m, seed=700 + topk, weights="normal")
    layer = make_layer(case, device)
    moe.moe_w4a16_set_path("decode")
    try:
        got = bf16_tensor_to_f64(run_layer(layer, case, device, w4a8=True))
    finally:
        moe.moe_w4a16_set_path("auto")
    ok, err, bound = M.within_tolerance(got, oracle_out(case, mxfp8=True))
    _say(f"  max|err| = {err:.3e}, bound = {bound:.3e}")
    assert ok, f"w4a8 top{topk} m={m}: {err} > {bound}"


def test_w4a8_rejects_nvfp4(moe, device):
    cfg = SCALED["decode_s"]
    case = make_case(cfg, 2, seed=1, weights="normal")
    layer = make_layer(case, device)
    with pytest.raises(moe.MoeError) as ei:
        run_layer(layer, case, device, w4a8=True)
    assert ei.value.code == moe.MOE_ERR_UNSUPPORTED
