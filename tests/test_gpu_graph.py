"""Capture of the fused layer into a HIP graph and replay over new data (GPU).

The fused call allocates nothing, never synchronises with the host and reads no device data
on the host, so a graph captured once replays correctly for new activations, routing and
expert maps written into the same device buffers (same m, same workspace). Every replay is
checked bit for bit against an eager call on the same data, with eager work and host
synchronisations between the replays, and one replay against the oracle.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import moe as M
from synth import draw as D

from _common import SCALED, Case, bf16_tensor_to_f64, make_case, make_layer, oracle_out

pytestmark = pytest.mark.gpu


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

    yield m
    m.moe_w4a16_set_path("auto")


@pytest.mark.parametrize("name,m,path,w4a8", [("decode_s", 8, "decode", False), ("small_s", 16, "decode", False),
                                              ("edge_s", 100, "gemm", False), ("prefill_s", 300, "gemm", False),
                                              ("edge_s", 8, "decode", True), ("edge_s", 100, "gemm", True)])
def test_graph_replay_matches_eager(moe, device, name, m, path, w4a8):
    """w4a8: the W4A8 entry point (moe_w4a8_fused), whose MXFP8 rounding pass is one more launch
    in the captured graph."""
    import torch

    print(f"graph {name} m={m} path={path} w4a8={w4a8}", flush=True)
    cfg = SCALED[name]
    case0 = make_case(cfg, m, seed=cfg.index * 7 + m + 3, weights="normal")
    cases = [case0]
    for i in (1, 2):
        ids, w, emap, rng = D.draw_routing(cfg, m, seed=900 + 10 * i + m)
        cases.append(Case(cfg, m, ids, w, emap, D.draw_activations_bf16(rng, m, cfg.hidden), case0.codes))
    layer = make_layer(case0, device)

    # Static device buffers the graph reads and writes.
    x = torch.empty((m, cfg.hidden), dtype=torch.bfloat16, device=device)
    ids = torch.empty((m, cfg.topk), dtype=torch.int32, device=device)
    wts = torch.empty((m, cfg.topk), dtype=torch.float32, device=device)
    emap = (torch.empty(cfg.num_global_experts, dtype=torch.int32, device=device)
            if case0.emap is not None else None)
    out = torch.empty((m, cfg.hidden), dtype=torch.bfloat16, device=device)

    def load(c):
        x.copy_(torch.from_numpy(c.xbits.view(np.int16)).view(torch.bfloat16))
        ids.copy_(torch.from_numpy(c.ids))
        wts.copy_(torch.from_numpy(c.w))
        if emap is not None:
            emap.copy_(torch.from_numpy(c.emap))

    def call():
        layer(x, ids, wts, expert_map=emap, num_global_experts=cfg.num_global_experts, out=out, w4a8=w4a8)

    moe.moe_w4a16_set_path(path)
    try:
        eager = []
        for c in cases:
            load(c)
            call()
            torch.cuda.synchronize()
            eager.append(out.clone())

        load(cases[0])
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()                                   # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        torch.cuda.synchronize()

        for rep in range(6):
            c = rep % len(cases)
            load(cases[c])
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager[c].view(torch.int16)), f"{name} replay {rep}: differs from eager"
            # eager work on the same stream between replays
            assert float((x.float() * 0.5).sum().item()) == pytest.approx(float(x.float().sum().item()) * 0.5, rel=1e-3)

        ok, err, bound = M.within_tolerance(bf16_tensor_to_f64(out), oracle_out(cases[(6 - 1) % len(cases)], mxfp8=w4a8))
        assert ok, f"{name}: {err} > {bound}"
        del graph
    finally:
        moe.moe_w4a16_set_path("auto")
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,m", [("prefill_s", 300), ("edge_s", 100)])
def test_graph_replay_atomic_bf16_combine(moe, device, name, m):
    """The opt-in atomic combine captured once and replayed over new batches into a NaN-filled
    output: the zero fill is inside the captured FC1 launch. Its sums are order-dependent, so
    each replay is checked against the oracle and against the eager call within k bf16 ulps of
    each row's magnitude instead of bit for bit."""
    import torch

    print(f"graph atomic {name} m={m}", flush=True)
    cfg = SCALED[name]
    case0 = make_case(cfg, m, seed=cfg.index * 7 + m + 5, weights="normal")
    cases = [case0]
    for i in (1, 2):
        ids, w, emap, rng = D.draw_routing(cfg, m, seed=950 + 10 * i + m)
        cases.append(Case(cfg, m, ids, w, emap, D.draw_activations_bf16(rng, m, cfg.hidden), case0.codes))
    layer = make_layer(case0, device)
    x = torch.empty((m, cfg.hidden), dtype=torch.bfloat16, device=device)
    ids = torch.empty((m, cfg.topk), dtype=torch.int32, device=device)
    wts = torch.empty((m, cfg.topk), dtype=torch.float32, device=device)
    emap = (torch.empty(cfg.num_global_experts, dtype=torch.int32, device=device)
            if case0.emap is not None else None)
    out = torch.empty((m, cfg.hidden), dtype=torch.bfloat16, device=device)

    def load(c):
        x.copy_(torch.from_numpy(c.xbits.view(np.int16)).view(torch.bfloat16))
        ids.copy_(torch.from_numpy(c.ids))
        wts.copy_(torch.from_numpy(c.w))
        if emap is not None:
            emap.copy_(torch.from_numpy(c.emap))

    def call():
        layer(x, ids, wts, expert_map=emap, num_global_experts=cfg.num_global_experts, out=out, atomic_bf16=True)

    moe.moe_w4a16_set_path("gemm")
    try:
        eager = []
        for c in cases:
            load(c)
            call()
            torch.cuda.synchronize()
            eager.append(bf16_tensor_to_f64(out))
        load(cases[0])
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        torch.cuda.synchronize()
        for rep in range(6):
            c = rep % len(cases)
            load(cases[c])
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = bf16_tensor_to_f64(out)
            assert np.all(np.isfinite(got)), f"{name} replay {rep}: output not fully written"
            scale = np.max(np.abs(eager[c]), axis=1, keepdims=True)
            assert np.all(np.abs(got - eager[c]) <= cfg.topk * 2.0 ** -7 * scale + 1e-6), f"{name} replay {rep}"
            ok, err, bound = M.within_tolerance(got, oracle_out(cases[c]))
            assert ok, f"{name} replay {rep}: {err} > {bound}"
        del graph
    finally:
        moe.moe_w4a16_set_path("auto")
    del layer
    torch.cuda.empty_cache()
