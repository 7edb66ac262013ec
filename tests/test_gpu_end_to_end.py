"""End to end on the GPU: router front end (moe_router_topk) feeding the fused layer.

The GPU router's top-k ids and weights go straight into moe_w4a16_fused (or the W4A8
variant); the oracle chains its own router (top-k of the fp32 logits, softmax or sigmoid
weights, renormalised) with its own layer. The ids must agree exactly, the layer outputs
within the usual bf16 tolerance: max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3.
"""

from __future__ import annotations

import numpy as np
import pytest

from _common import SCALED, Case, bf16_tensor_to_f64, dev, make_case, make_layer, oracle_out
from oracle import moe as M
from oracle import router as RT
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


@pytest.mark.parametrize("name,m,w4a8", [("decode_s", 1, False), ("decode_s", 8, False), ("small_s", 16, False),
                                         ("small_s", 64, False), ("prefill_s", 300, False), ("tiny", 4, True)])
def test_router_then_fused_matches_oracle(moe, device, name, m, w4a8):
    cfg = SCALED[name]
    assert not cfg.use_expert_map                        # the router scores the local experts
    scoring = "sigmoid" if cfg.routing == "sigmoid" else "softmax"
    print(f"router -> fused {name} m={m} {scoring} w4a8={w4a8}", flush=True)
    base = make_case(cfg, m, seed=cfg.index * 13 + m, weights="normal")
    logits = D.draw_router_logits(cfg, m, seed=700 + m)
    layer = make_layer(base, device)

    d_logits = dev(logits, device)
    ids = torch.empty((m, cfg.topk), dtype=torch.int32, device=device)
    wts = torch.empty((m, cfg.topk), dtype=torch.float32, device=device)
    moe.moe_router_topk(d_logits, m, cfg.num_experts, cfg.topk, scoring, cfg.renormalize, ids, wts)
    x = dev(base.xbits.view(np.int16), device).view(torch.bfloat16)
    out = layer(x, ids, wts, w4a8=w4a8)
    torch.cuda.synchronize()

    ref_ids, ref_w = RT.route(logits, cfg.topk, scoring, cfg.renormalize)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    case = Case(cfg, m, ref_ids, ref_w, None, base.xbits, base.codes)
    ref = oracle_out(case, mxfp8=w4a8)
    ok, err, bound = M.within_tolerance(bf16_tensor_to_f64(out), ref)
    print(f"  max|err| = {err:.3e}, bound = {bound:.3e}", flush=True)
    assert ok, f"{name} m={m}: {err} > {bound}"
