"""GPU: the fused layer on streams other than torch's current one.

* Stream ordering (FlashInfer PR 4255, Review round 1: a packing entry point had dropped its
  `stream` argument and ran on the default stream): every launch of a call must go on the
  caller's stream. The test writes the call's inputs on a side stream behind a long-running
  kernel and calls the layer on that stream at once; a launch on any other stream would read
  the stale inputs (large finite garbage) and miss the oracle.
* No co-residency assumption (PR 4255, Performance: the m = 2048 stall of grid-wide barriers
  without a cooperative launch): the persistent grouped GEMM and the decode path's FC1 run with
  their grids cut down to a few workgroups. Nothing in either path waits for another workgroup,
  so the call completes and matches the unrestricted call bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest

from _common import SCALED, bf16_tensor_to_f64, dev, make_case, make_layer, oracle_out
from oracle import moe as M

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


def _inputs(case, device):
    x = dev(case.xbits.view(np.int16), device).view(torch.bfloat16)
    emap = dev(case.emap, device) if case.emap is not None else None
    return x, dev(case.ids, device), dev(case.w, device), emap


@pytest.mark.parametrize("name,m,path", [("prefill_s", 300, "gemm"), ("decode_s", 8, "decode"),
                                         ("small_s", 16, "decode"), ("edge_s", 100, "gemm")])
def test_inputs_written_on_the_call_stream_behind_a_long_kernel(moe, device, name, m, path):
    cfg = SCALED[name]
    case = make_case(cfg, m, seed=cfg.index * 13 + m, weights="normal")
    layer = make_layer(case, device)
    x, ids, w, emap = _inputs(case, device)
    # the call's buffers hold stale values (finite garbage, valid ids) until the side stream rewrites them
    bx = torch.full_like(x, 1000.0)
    bids = torch.zeros_like(ids)
    bw = torch.full_like(w, 7.0)
    out = torch.full((m, cfg.hidden), float("nan"), dtype=torch.bfloat16, device=device)
    layer.workspace.fill_(0x7F)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=device)          # default priority
    moe.moe_w4a16_set_path(path)
    try:
        _say(f"stream order {name} m={m} path={path}")
        with torch.cuda.stream(side):
            torch.cuda._sleep(20_000_000)                # ~10 ms of spinning on the side stream
            bx.copy_(x)
            bids.copy_(ids)
            bw.copy_(w)
            layer(bx, bids, bw, expert_map=emap, num_global_experts=cfg.num_global_experts, out=out, stream=side)
        side.synchronize()
    finally:
        moe.moe_w4a16_set_path("auto")
    torch.cuda.synchronize()
    got = bf16_tensor_to_f64(out)
    ok, err, bound = M.within_tolerance(got, oracle_out(case))
    _say(f"  max|err| = {err:.3e}, bound = {bound:.3e}")
    assert ok, f"{name} m={m} {path}: {err} > {bound}"


@pytest.mark.parametrize("name,m,path", [("prefill_s", 300, "gemm"), ("edge_s", 100, "gemm"),
                                         ("decode_s", 8, "decode"), ("small_s", 16, "decode")])
def test_few_workgroups_no_co_residency(moe, device, name, m, path):
    """The same call with its persistent and grid-stride launches cut to 1, 3 and 7 workgroups'
    worth of CUs (moe_w4a16_set_grid_limit): one workgroup then works through every grouped-GEMM
    item, and the decode FC1's items are dealt to a few. No workgroup waits for another, so every
    result equals the unrestricted call bit for bit and matches the oracle. (Streams with a CU
    mask, the other way to run a launch on a few CUs, are refused on the MI355X systems used
    here: hipExtStreamCreateWithCUMask returns hipErrorOutOfMemory.)"""
    cfg = SCALED[name]
    case = make_case(cfg, m, seed=cfg.index * 17 + m, weights="normal")
    layer = make_layer(case, device)
    x, ids, w, emap = _inputs(case, device)
    moe.moe_w4a16_set_path(path)
    try:
        full = bf16_tensor_to_f64(layer(x, ids, w, expert_map=emap, num_global_experts=cfg.num_global_experts))
        for limit in (1, 3, 7):
            _say(f"few workgroups {name} m={m} path={path} limit={limit}")
            prev = moe.moe_w4a16_set_grid_limit(limit)
            try:
                out = torch.full((m, cfg.hidden), float("nan"), dtype=torch.bfloat16, device=device)
                layer(x, ids, w, expert_map=emap, num_global_experts=cfg.num_global_experts, out=out)
                torch.cuda.synchronize()
            finally:
                moe.moe_w4a16_set_grid_limit(prev)
            got = bf16_tensor_to_f64(out)
            assert np.array_equal(got, full), f"limit {limit}: differs from the unrestricted call"
    finally:
        moe.moe_w4a16_set_path("auto")
    ok, err, bound = M.within_tolerance(full, oracle_out(case))
    assert ok, f"{name} m={m} {path}: {err} > {bound}"
