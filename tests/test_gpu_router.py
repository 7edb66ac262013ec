"""Router front end on the GPU against the oracle: expert ids bit-exact, weights within
float32 rounding of the float64 oracle, on every workload's router recipe and edge cases."""

from __future__ import annotations

import numpy as np
import pytest

from oracle import router as RT
from synth import configs as C
from synth import draw as D

pytestmark = pytest.mark.gpu

W_RTOL, W_ATOL = 2e-6, 1e-7     # fp32 exp / division against the float64 oracle


@pytest.fixture(scope="module")
def device():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    return d


@pytest.fixture(scope="module")
def moe():
    import fp4_weight_grouped_moe_amd as m

    return m


def _run(moe, device, logits, k, scoring, renormalize):
    import torch

    m, e = logits.shape
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(device)
    ids = torch.full((m, k), -7, dtype=torch.int32, device=device)
    w = torch.full((m, k), float("nan"), dtype=torch.float32, device=device)
    moe.moe_router_topk(lg, m, e, k, scoring, renormalize, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _check(moe, device, logits, k, scoring, renormalize, label):
    print(label, flush=True)
    got_ids, got_w = _run(moe, device, logits, k, scoring, renormalize)
    ref_ids, ref_w = RT.route(logits, k, scoring, renormalize)
    assert np.array_equal(got_ids, ref_ids), f"{label}: ids differ in {int((got_ids != ref_ids).any(axis=1).sum())} rows"
    np.testing.assert_allclose(got_w, ref_w, rtol=W_RTOL, atol=W_ATOL, err_msg=label)


@pytest.mark.parametrize("name", ["tiny", "decode", "small", "prefill", "edge"])
@pytest.mark.parametrize("m", [1, 100, 2048])
def test_router_matches_oracle_on_workload_recipes(moe, device, name, m):
    cfg = C.get_config(name)
    logits = D.draw_router_logits(cfg, m, seed=300 + cfg.index * 10 + m)
    scoring = "sigmoid" if cfg.routing == "sigmoid" else "softmax"
    _check(moe, device, logits, cfg.topk, scoring, cfg.renormalize, f"router {name} m={m} {scoring}")


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
@pytest.mark.parametrize("renormalize", [True, False])
def test_router_ties_and_signed_zero(moe, device, scoring, renormalize):
    rng = np.random.default_rng(17)
    logits = (rng.integers(-3, 4, size=(257, 40)) * 0.5).astype(np.float32)   # many equal values
    logits[:, 5] = -0.0
    logits[:, 6] = 0.0
    _check(moe, device, logits, 7, scoring, renormalize, f"router ties {scoring} renorm={renormalize}")


@pytest.mark.parametrize("e,k", [(1, 1), (8, 8), (64, 64), (65, 3), (1000, 64), (1024, 9)])
def test_router_sizes(moe, device, e, k):
    rng = np.random.default_rng(e * 100 + k)
    logits = (rng.standard_normal((33, e)) * 3).astype(np.float32)
    _check(moe, device, logits, k, "softmax", True, f"router E={e} k={k}")


def test_router_empty_and_rejects(moe, device):
    import torch

    ids = torch.empty((0, 4), dtype=torch.int32, device=device)
    w = torch.empty((0, 4), dtype=torch.float32, device=device)
    lg = torch.empty((0, 16), dtype=torch.float32, device=device)
    moe.moe_router_topk(lg, 0, 16, 4, "softmax", True, ids, w)
    for e, k in ((16, 17), (16, 0), (1025, 4), (128, 65)):
        with pytest.raises(moe.MoeError):
            moe.moe_router_topk(lg, 0, e, k, "softmax", True, ids, w)
    with pytest.raises(moe.MoeError):
        moe.moe_router_topk(lg, 0, 16, 4, 7, True, ids, w)


def test_router_timing_prefill_shape(moe, device):
    """Timing at the prefill shape (2048 tokens x 256 experts, top 8): reads 2 MiB of logits."""
    import torch

    cfg = C.get_config("prefill")
    m, e, k = 2048, cfg.num_global_experts, cfg.topk
    lg = torch.from_numpy(D.draw_router_logits(cfg, m, seed=5)).to(device)
    ids = torch.empty((m, k), dtype=torch.int32, device=device)
    w = torch.empty((m, k), dtype=torch.float32, device=device)
    for _ in range(5):
        moe.moe_router_topk(lg, m, e, k, "softmax", True, ids, w)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(50):
        moe.moe_router_topk(lg, m, e, k, "softmax", True, ids, w)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / 50 * 1e3
    print(f"router m={m} E={e} k={k}: {us:.2f} us per call, {(m * e * 4 + m * k * 8) / (us * 1e-6) / 1e9:.1f} GB/s",
          flush=True)
    assert us > 0
