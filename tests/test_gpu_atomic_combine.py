"""GPU parity of the opt-in approximate top-k combine (moe_w4a16_fused_atomic_bf16).

On the grouped-GEMM path FC2 rounds each route's weighted row to bf16 and adds it into its
token's output row with packed-bf16 atomics (the FlashInfer fused-MoE source's opt-in bf16
scatter-add beside its f32 reduction); FC1 zeroes the output first. Same tolerance as the
W4A16 layer against the float64 oracle: max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3 in bf16
(each route row is rounded once and every add rounds to bf16: at most about k bf16 ulps of
the row's magnitude). On the decode path the entry point is moe_w4a16_fused bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest

from _common import SCALED, bf16_tensor_to_f64, full_case, make_case, make_layer, oracle_out, run_layer
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
    ref = oracle_out(case, tokens=tokens, cols=cols)
    if tokens is not None or cols is not None:
        t = np.arange(case.m) if tokens is None else np.asarray(tokens)
        c = np.arange(case.cfg.hidden) if cols is None else np.asarray(cols)
        got = got[np.ix_(t, c)]
    ok, err, bound = M.within_tolerance(got, ref)
    _say(f"  {label}: max|err| = {err:.3e}, bound = {bound:.3e}, max|ref| = {np.max(np.abs(ref)):.3e}")
    assert ok, f"{label}: {err} > {bound}"


def _nan_out(m, hidden, device):
    # a dirty output buffer: quiet-NaN bf16 everywhere, so a missed zero fill shows
    return torch.full((m, hidden), 0x7FC0, dtype=torch.int16, device=device).view(torch.bfloat16)


ATOMIC_CASES = [("tiny", 4), ("prefill_s", 300), ("prefill_s", 40), ("edge_s", 100), ("small_s", 64), ("decode_s", 24)]


@pytest.mark.parametrize("name,m", ATOMIC_CASES)
def test_atomic_combine_matches_oracle_scaled(moe, device, name, m):
    cfg = SCALED[name]
    _say(f"atomic bf16 {name} m={m}")
    case = make_case(cfg, m, seed=cfg.index * 17 + m, weights="normal")
    if m > 2:
        case.ids[1, 0] = -1
        case.ids[2, :] = -1                      # a token with no surviving route
    layer = make_layer(case, device)
    moe.moe_w4a16_set_path("gemm")
    try:
        got = bf16_tensor_to_f64(run_layer(layer, case, device, out=_nan_out(m, cfg.hidden, device), atomic_bf16=True))
        ref16 = bf16_tensor_to_f64(run_layer(layer, case, device))
    finally:
        moe.moe_w4a16_set_path("auto")
    assert np.all(np.isfinite(got))
    if m > 2:
        assert np.all(got[2] == 0)
    _check(case, got, label=f"atomic {name} m={m}")
    # against the deterministic combine: within a few bf16 ulps of each row's magnitude
    scale = np.max(np.abs(ref16), axis=1, keepdims=True)
    assert np.all(np.abs(got - ref16) <= cfg.topk * 2.0 ** -7 * scale + 1e-6)


@pytest.mark.parametrize("m", [1, 8, 16])
def test_atomic_combine_is_the_fused_layer_on_the_decode_path(moe, device, m):
    cfg = SCALED["decode_s"]
    case = make_case(cfg, m, seed=300 + m, weights="normal")
    layer = make_layer(case, device)
    moe.moe_w4a16_set_path("decode")
    try:
        a = bf16_tensor_to_f64(run_layer(layer, case, device, atomic_bf16=True))
        b = bf16_tensor_to_f64(run_layer(layer, case, device))
    finally:
        moe.moe_w4a16_set_path("auto")
    assert np.array_equal(a, b)


@pytest.mark.timeout(900)
def test_atomic_combine_full_size_prefill_every_output(moe, device):
    """Full-size prefill shape (E256 H7168 I2048 top-8 NVFP4, Zipf routing, m = 2048) on a NaN-filled
    output buffer: every token x every column against the oracle."""
    m = 2048
    case = full_case("prefill", m, device)
    layer = make_layer(case, device, token_capacity=RP.token_capacity(m))
    _say("atomic bf16 full prefill m=2048")
    got = bf16_tensor_to_f64(run_layer(layer, case, device, out=_nan_out(m, case.cfg.hidden, device), atomic_bf16=True))
    assert np.all(np.isfinite(got))
    _check(case, got, label="atomic prefill m=2048, every token x every column")
    del layer, case
    torch.cuda.empty_cache()
