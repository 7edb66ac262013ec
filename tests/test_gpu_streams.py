"""GPU: the fused layer on streams other than torch's current one.

* Stream ordering (FlashInfer PR 4255, Review round 1: a packing entry point had dropped its
  `stream` argument and ran on the default stream): every launch of a call must go on the
  caller's stream. The test writes the call's inputs on a side stream behind a long-running
  kernel and calls the layer on that stream at once; a launch on any other stream would read
  the stale inputs (large finite garbage) and miss the oracle.
* No co-residency assumption (PR 4255, Performance: the m = 2048 stall of grid-wide barriers
  without a cooperative launch): the persistent grouped GEMM and the decode path's split-K FC2
  run on a stream whose work may use only a few CUs, so most workgroups of each launch wait for
  others to finish before they start. Nothing in either path waits for another workgroup, so
  the call completes and matches the oracle and the unrestricted call bit for bit.
"""

from __future__ import annotations

import ctypes

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


def _hip():
    # the HIP runtime already in the process (torch's), never a second copy by name
    paths = sorted({ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln})
    assert len(paths) == 1, paths
    return ctypes.CDLL(paths[0])


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


@pytest.mark.parametrize("name,m,path,cus", [("prefill_s", 300, "gemm", 4), ("edge_s", 100, "gemm", 1),
                                             ("decode_s", 8, "decode", 4), ("small_s", 16, "decode", 2)])
def test_few_cus_no_co_residency(moe, device, name, m, path, cus):
    hip = _hip()
    cfg = SCALED[name]
    case = make_case(cfg, m, seed=cfg.index * 17 + m, weights="normal")
    layer = make_layer(case, device)
    x, ids, w, emap = _inputs(case, device)
    out_full = torch.empty((m, cfg.hidden), dtype=torch.bfloat16, device=device)
    out_few = torch.full((m, cfg.hidden), float("nan"), dtype=torch.bfloat16, device=device)
    moe.moe_w4a16_set_path(path)
    stream = ctypes.c_void_p()
    try:
        layer(x, ids, w, expert_map=emap, num_global_experts=cfg.num_global_experts, out=out_full)
        torch.cuda.synchronize()
        # the first `cus` CUs of the mask (one 32-bit word per 32 CUs)
        mask = (ctypes.c_uint32 * 8)(*([(1 << cus) - 1] + [0] * 7))
        rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(stream), ctypes.c_uint32(8), mask)
        assert rc == 0, f"hipExtStreamCreateWithCUMask failed ({rc})"
        _say(f"few CUs {name} m={m} path={path} cus={cus}")
        layer(x, ids, w, expert_map=emap, num_global_experts=cfg.num_global_experts, out=out_few,
              stream=int(stream.value))
        rc = hip.hipStreamSynchronize(stream)
        assert rc == 0, f"hipStreamSynchronize failed ({rc})"
    finally:
        moe.moe_w4a16_set_path("auto")
        if stream.value:
            hip.hipStreamDestroy(stream)
    a, b = bf16_tensor_to_f64(out_full), bf16_tensor_to_f64(out_few)
    assert np.array_equal(a, b), "the call on a few CUs differs from the unrestricted call"
    ok, err, bound = M.within_tolerance(b, oracle_out(case))
    _say(f"  max|err| = {err:.3e}, bound = {bound:.3e}")
    assert ok, f"{name} m={m} {path}: {err} > {bound}"
