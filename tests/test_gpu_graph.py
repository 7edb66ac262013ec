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


def _full_or_scaled(name):
    from synth import configs as C
    return SCALED[name] if name in SCALED else C.get_config(name)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,cap,ms", [("edge_s", 512, (300, 511, 512, 1, 0)), ("prefill_s", 512, (257, 512, 40)),
                                         ("decode_s", 16, (1, 9, 16, 4)), ("small_s", 16, (16, 3)),
                                         ("edge", 512, (300, 511, 512))])
def test_graph_replay_across_m_on_one_capacity(moe, device, name, cap, ms):
    """moe_w4a16_fused_device_m captured once at a power-of-two capacity and replayed for several
    token counts m <= capacity written into a device int32 between replays (the page's reason for
    the power-of-two route capacity: batch-size changes need no new launch shapes). Input rows at
    or past m hold junk routed to a valid expert, which must not reach the result; output rows
    past m must be zero. Each replay equals the eager moe_w4a16_fused call at that m -- bit for bit
    on the grouped-GEMM path -- and matches the oracle on every output. `edge` is the full-size
    edge workload (expert map, -1 ids, I = 1400) at capacity 512, rerun at m = 300, 511 and 512."""
    import torch

    from _common import full_case

    cfg = _full_or_scaled(name)
    full = name not in SCALED
    print(f"graph across m {name} capacity {cap} m={ms}", flush=True)
    base = full_case(name, ms[0], device) if full else make_case(cfg, ms[0], seed=cfg.index * 29 + 1, weights="normal")
    layer = make_layer(base, device, token_capacity=cap)
    H, k = cfg.hidden, cfg.topk
    x = torch.empty((cap, H), dtype=torch.bfloat16, device=device)
    ids = torch.empty((cap, k), dtype=torch.int32, device=device)
    wts = torch.empty((cap, k), dtype=torch.float32, device=device)
    emap = torch.empty(cfg.num_global_experts, dtype=torch.int32, device=device) if base.emap is not None else None
    m_dev = torch.zeros(1, dtype=torch.int32, device=device)
    out = torch.empty((cap, H), dtype=torch.bfloat16, device=device)

    def device_m_call():
        moe.moe_w4a16_fused_device_m(layer.dims, layer.prepared, layer.prepared_bytes, x, m_dev, ids, wts, k, emap,
                                     cfg.num_global_experts, cap, layer.workspace, layer.workspace_bytes, out)

    def case_at(m):
        if m == ms[0]:
            return base
        if full:
            return full_case(name, m, device, base.codes_dev)
        i, w, em, rng = D.draw_routing(cfg, m, seed=cfg.index * 29 + 2 + m)
        return Case(cfg, m, i, w, em, D.draw_activations_bf16(rng, m, H), base.codes)

    def load(c):
        m = c.m
        x.fill_(1000.0)                       # junk past m: large, finite, routed to expert 0 with weight 5
        ids.zero_()
        wts.fill_(5.0)
        if m:
            x[:m].copy_(torch.from_numpy(c.xbits.view(np.int16)).view(torch.bfloat16))
            ids[:m].copy_(torch.from_numpy(c.ids))
            wts[:m].copy_(torch.from_numpy(c.w))
        if emap is not None:
            emap.copy_(torch.from_numpy(c.emap))
        m_dev.fill_(m)

    load(case_at(ms[0]))
    device_m_call()                           # first call outside capture (one-time kernel attributes)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        device_m_call()
    torch.cuda.synchronize()
    for m in ms:
        c = case_at(m)
        load(c)
        g.replay()
        torch.cuda.synchronize()
        got = bf16_tensor_to_f64(out)
        assert np.all(got[m:] == 0), f"m={m}: rows past m not zero"
        got = got[:m]
        # eager reference at this m: the plain entry point on buffers of exactly m rows
        ex = torch.from_numpy(c.xbits.view(np.int16)).view(torch.bfloat16).to(device)
        ref_out = layer(ex, torch.from_numpy(c.ids).to(device), torch.from_numpy(c.w).to(device), expert_map=emap,
                        num_global_experts=cfg.num_global_experts) if m else torch.empty((0, H), dtype=torch.bfloat16, device=device)
        torch.cuda.synchronize()
        eager = bf16_tensor_to_f64(ref_out)
        decode_path = cap <= moe.MOE_DECODE_MAX_M
        same = np.array_equal(got, eager)
        print(f"  m={m}: replay == eager bit for bit: {same}", flush=True)
        if not decode_path:
            assert same, f"m={m}: graph replay differs from the eager call"
        if m:
            ok, err, bound = M.within_tolerance(got, oracle_out(c))
            print(f"  m={m}: max|err| = {err:.3e}, bound = {bound:.3e}", flush=True)
            assert ok, f"m={m}: {err} > {bound}"
            ok, err, bound = M.within_tolerance(eager, oracle_out(c))
            assert ok
    del g, layer
    torch.cuda.empty_cache()
