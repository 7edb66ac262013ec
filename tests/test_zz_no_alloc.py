"""GPU: moe_w4a16_fused_static_workspace, the allocation-free entry point, against moe_w4a16_fused.

The entry point runs the fused layer's kernels with the library's own device array as the
workspace. Two calls in a row (the second with a smaller m, over the contents the first left
in the array) must equal moe_w4a16_fused with a caller workspace bit for bit -- both paths are
deterministic -- and stay within the oracle's tolerance; a layer whose workspace need exceeds
the array is refused before any device work.
"""

from __future__ import annotations

import numpy as np
import pytest

from _common import SCALED, bf16_tensor_to_f64, dev, make_case, make_layer, oracle_out
from oracle import moe as M
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


def _inputs(case, device):
    x = dev(case.xbits.view(np.int16), device).view(torch.bfloat16)
    emap = dev(case.emap, device) if case.emap is not None else None
    return x, dev(case.ids, device), dev(case.w, device), emap


@pytest.mark.parametrize("name,ms,path", [("decode_s", (8, 3), "auto"), ("edge_s", (100, 40), "auto"),
                                          ("small_s", (16, 5), "decode"), ("prefill_s", (300, 17), "gemm")])
def test_static_workspace_matches_caller_workspace(moe, device, name, ms, path):
    cfg = SCALED[name]
    cap = moe.moe_route_pack_token_capacity(ms[0])
    case0 = make_case(cfg, ms[0], seed=cfg.index * 19 + ms[0], weights="normal")
    layer = make_layer(case0, device, token_capacity=cap)
    moe.moe_w4a16_set_path(path)
    try:
        for i, m in enumerate(ms):
            if i == 0:
                case = case0
            else:
                ids, w, emap, rng = D.draw_routing(cfg, m, seed=cfg.index * 23 + m)
                case = type(case0)(cfg, m, ids, w, emap, D.draw_activations_bf16(rng, m, cfg.hidden), case0.codes)
            print(f"static workspace {name} m={m} cap={cap} path={path}", flush=True)
            x, ids, w, emap = _inputs(case, device)
            ref_out = layer(x, ids, w, expert_map=emap, num_global_experts=cfg.num_global_experts)
            out = torch.full((m, cfg.hidden), float("nan"), dtype=torch.bfloat16, device=device)
            moe.moe_w4a16_fused_static_workspace(layer.dims, layer.prepared, layer.prepared_bytes, x, m, ids, w,
                                                 cfg.topk, emap, cfg.num_global_experts, cap, out)
            torch.cuda.synchronize()
            a, b = bf16_tensor_to_f64(ref_out), bf16_tensor_to_f64(out)
            assert np.array_equal(a, b), f"{name} m={m}: static workspace differs from the caller workspace"
            ok, err, bound = M.within_tolerance(b, oracle_out(case))
            assert ok, f"{name} m={m}: {err} > {bound}"
    finally:
        moe.moe_w4a16_set_path("auto")


def test_static_workspace_refuses_layers_beyond_its_size(moe, device):
    cfg = C.get_config("prefill")
    d = moe.make_dims(cfg.fmt, cfg.act, cfg.num_experts, cfg.hidden, cfg.inter)
    assert moe.moe_w4a16_workspace_size(d, 2048, cfg.topk) > moe.MOE_STATIC_WORKSPACE_BYTES
    fake = 1 << 20          # never dereferenced: the size check comes first
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_w4a16_fused_static_workspace(d, fake, 1 << 40, fake, 2048, fake, fake, cfg.topk, None,
                                             cfg.num_experts, 2048, fake, stream=0)
    assert ei.value.code == moe.MOE_ERR_WORKSPACE
    assert "static workspace" in moe.moe_last_error()
