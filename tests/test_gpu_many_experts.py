"""Route packing and the fused layer with more than 256 local experts or more than 16 384
routes (GPU).

Above 256 experts the segmented pack ranks each 64-route chunk with one ballot pass per
distinct expert instead of per-wave lane masks, and the slot-ordered tables are written from
an LDS slot -> route map only while that map fits (else by the route-order scatter). The
route pack must match the oracle bit for bit (FlashInfer PR 4255, Description and Tests:
shape-stable packing, expert_map, invalid ids); the fused layer within the usual bf16
tolerance, max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3.
"""

from __future__ import annotations

import numpy as np
import pytest

from _common import bf16_tensor_to_f64, dev, make_case, make_layer, oracle_out, run_layer
from oracle import moe as M
from oracle import route_pack as RP
from synth import configs as C

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


# (local experts, global experts, expert_map?, m, k, block_m): 1 025 - 16 384 routes (the
# segmented pack); B = 64 with 1 024 experts overflows the LDS slot map (route-order scatter);
# above 16 384 routes the pack runs 1 024-route chunks with running per-expert slots.
MANY = [(300, 300, False, 512, 8, 16), (1024, 2048, True, 2048, 8, 16), (1024, 1024, False, 2048, 8, 64),
        (600, 600, False, 1000, 6, 32), (257, 257, False, 171, 6, 128),
        (256, 256, False, 4096, 8, 16), (64, 128, True, 3001, 6, 128), (2048, 2048, False, 2100, 8, 32),
        (2048, 2048, False, 100, 8, 16), (1500, 1500, False, 700, 7, 64),   # above 1 024 experts: chunked
        # route counts at the mode boundaries: one chunk (1 024), segmented (1 025, 16 384),
        # chunked (16 392, 16 385)
        (64, 64, False, 128, 8, 16), (64, 64, False, 1025, 1, 32), (200, 200, False, 2048, 8, 128),
        (200, 200, False, 2049, 8, 16), (96, 96, False, 16385, 1, 64), (1024, 1024, False, 0, 4, 16)]


@pytest.mark.parametrize("E,Eg,use_map,m,k,B", MANY)
def test_route_pack_many_experts_bit_exact(moe, device, E, Eg, use_map, m, k, B):
    rng = np.random.default_rng(E * 7 + m + B)
    ids = rng.integers(-2, Eg + 3, size=(m, k)).astype(np.int32)        # -1, -2 and out-of-range ids too
    ids[rng.random((m, k)) < 0.3] = int(rng.integers(0, 4))             # a few heavy experts
    emap = None
    if use_map:
        emap = np.full(Eg, -1, np.int32)
        keep = rng.permutation(Eg)[:E]
        emap[keep] = np.arange(E, dtype=np.int32)
    cap = RP.token_capacity(m)
    _say(f"route_pack E={E} Eg={Eg} map={use_map} m={m} k={k} B={B}")
    nbytes = moe.moe_route_pack_workspace_size(cap, k, E, B)
    ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device=device)
    d_ids = dev(ids, device)
    d_map = dev(emap, device) if emap is not None else None
    view = moe.moe_route_pack(d_ids, m, k, d_map, Eg, E, B, cap, ws, nbytes)
    torch.cuda.synchronize()
    base = ws.data_ptr()

    def read(ptr, n):
        off = ptr - base
        return ws[off:off + 4 * n].view(torch.int32).cpu().numpy().copy()

    got = {
        "expert_counts": read(view.expert_counts, E),
        "expert_offsets": read(view.expert_offsets, E + 1),
        "sorted_route_ids": read(view.sorted_route_ids, view.cap_routes),
        "block_expert": read(view.block_expert, view.cap_blocks),
        "live": read(view.live, 4),
        "route_slot": read(view.route_slot, cap * k),
    }
    want = RP.route_pack(ids, emap, Eg, E, B, cap)
    for key in want:
        assert np.array_equal(got[key], want[key]), key


FUSED_MANY = [
    (C.scaled(C.get_config("prefill"), num_experts=512, hidden=256, inter=128, name="prefill_e512"), 1024, "normal"),
    (C.scaled(C.get_config("prefill"), num_experts=64, hidden=256, inter=128, name="prefill_m4096"), 4096, "normal"),
    (C.scaled(C.get_config("edge"), num_experts=1024, num_global_experts=2048, hidden=256, inter=200,
              name="edge_e1024"), 512, "random"),
]


@pytest.mark.parametrize("cfg,m,weights", FUSED_MANY, ids=lambda v: getattr(v, "name", str(v)))
def test_fused_many_experts_matches_oracle(moe, device, cfg, m, weights):
    _say(f"fused {cfg.name} m={m}")
    case = make_case(cfg, m, seed=cfg.index * 31 + m, weights=weights)
    layer = make_layer(case, device)
    got = bf16_tensor_to_f64(run_layer(layer, case, device))
    ref = oracle_out(case)
    ok, err, bound = M.within_tolerance(got, ref)
    _say(f"  max|err| = {err:.3e}, bound = {bound:.3e}")
    assert ok, f"{cfg.name} m={m}: {err} > {bound}"
    del layer
    torch.cuda.empty_cache()


def _decode_cfg(base, **kw):
    import dataclasses
    return dataclasses.replace(base, **kw)


DECODE_MANY = [
    (_decode_cfg(C.get_config("decode"), num_experts=2048, num_global_experts=2048, hidden=256, inter=128,
                 name="decode_e2048"), (1, 8, 16)),
    (_decode_cfg(C.get_config("edge"), num_experts=1500, num_global_experts=3000, hidden=256, inter=200,
                 name="edge_e1500_map"), (8,)),
    (_decode_cfg(C.get_config("decode"), num_experts=128, num_global_experts=128, hidden=256, inter=128, topk=64,
                 name="decode_top64"), (1, 4, 8, 16)),
]


@pytest.mark.parametrize("cfg,ms", DECODE_MANY, ids=lambda v: getattr(v, "name", str(v)))
def test_decode_path_many_experts_and_large_topk(moe, device, cfg, ms):
    """Decode path (m <= 16): FC1's own route pack up to 2 048 experts and 256 routes (one per
    thread), the separate pack launch and the one-pass FC2 beyond 128 routes (top-64 at
    m = 4 .. 16); an expert_map over 3 000 global ids with 5 % invalid ids."""
    moe.moe_w4a16_set_path("decode")
    try:
        for m in ms:
            _say(f"decode {cfg.name} m={m}")
            case = make_case(cfg, m, seed=cfg.index * 37 + m, weights="random")
            layer = make_layer(case, device)
            got = bf16_tensor_to_f64(run_layer(layer, case, device))
            ok, err, bound = M.within_tolerance(got, oracle_out(case))
            _say(f"  max|err| = {err:.3e}, bound = {bound:.3e}")
            assert ok, f"{cfg.name} m={m}: {err} > {bound}"
            del layer
    finally:
        moe.moe_w4a16_set_path("auto")
    torch.cuda.empty_cache()


ODD_DIMS = [
    # (base workload, hidden, inter): hidden not a multiple of 128 (FC1 K tail, FC2's last row
    # group partial; NVFP4 hidden 200 also ends in an 8-wide scale group), inter tails too
    ("decode", 200, 136), ("decode", 1000, 232), ("small", 264, 100), ("edge", 200, 72), ("edge", 1000, 1400),
]


@pytest.mark.parametrize("base,H,I", ODD_DIMS)
@pytest.mark.parametrize("path,m", [("decode", 3), ("decode", 16), ("gemm", 40)])
def test_fused_hidden_not_a_multiple_of_128(moe, device, base, H, I, path, m):
    import dataclasses
    ref_cfg = C.get_config(base)
    cfg = dataclasses.replace(ref_cfg, num_experts=8, num_global_experts=16 if ref_cfg.use_expert_map else 8,
                              hidden=H, inter=I, name=f"{base}_h{H}_i{I}")
    _say(f"{cfg.name} {cfg.fmt} {cfg.act} m={m} path={path}")
    case = make_case(cfg, m, seed=H * 7 + I + m, weights="normal")
    layer = make_layer(case, device)
    moe.moe_w4a16_set_path(path)
    try:
        got = bf16_tensor_to_f64(run_layer(layer, case, device))
    finally:
        moe.moe_w4a16_set_path("auto")
    ok, err, bound = M.within_tolerance(got, oracle_out(case))
    _say(f"  max|err| = {err:.3e}, bound = {bound:.3e}")
    assert ok, f"{cfg.name} m={m} {path}: {err} > {bound}"
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("H,I", [(200, 72), (1000, 1400), (264, 136)])
@pytest.mark.parametrize("path,m", [("decode", 3), ("decode", 16), ("gemm", 40)])
def test_w4a8_hidden_not_a_multiple_of_128(moe, device, H, I, path, m):
    """The W4A8 variant (MXFP8 activation output, block-scaled FC2 on the decode path) at the
    same odd shapes, against the oracle's W4A8 forward."""
    import dataclasses
    cfg = dataclasses.replace(C.get_config("edge"), num_experts=8, num_global_experts=16, hidden=H, inter=I,
                              name=f"edge_w4a8_h{H}_i{I}")
    _say(f"{cfg.name} m={m} path={path}")
    case = make_case(cfg, m, seed=H * 11 + I + m, weights="normal")
    layer = make_layer(case, device)
    moe.moe_w4a16_set_path(path)
    try:
        got = bf16_tensor_to_f64(run_layer(layer, case, device, w4a8=True))
    finally:
        moe.moe_w4a16_set_path("auto")
    ok, err, bound = M.within_tolerance(got, oracle_out(case, mxfp8=True))
    _say(f"  max|err| = {err:.3e}, bound = {bound:.3e}")
    assert ok, f"{cfg.name} m={m} {path}: {err} > {bound}"
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,m,cap", [("decode_s", 1, 16), ("decode_s", 5, 16), ("prefill_s", 17, 8192),
                                        ("edge_s", 3, 1024), ("small_s", 64, 4096)])
def test_fused_capacity_far_above_m(moe, device, name, m, cap):
    """A workspace sized for far more tokens than the call has: the auto path takes the decode
    kernels only while the capacity is at most 16, otherwise the grouped GEMM over a mostly
    empty route space (padding slots, -1 block ids, empty tile queues)."""
    from _common import SCALED
    cfg = SCALED[name]
    _say(f"capacity {name} m={m} cap={cap}")
    case = make_case(cfg, m, seed=cfg.index * 41 + m, weights="normal")
    layer = make_layer(case, device, token_capacity=cap)
    got = bf16_tensor_to_f64(run_layer(layer, case, device))
    ok, err, bound = M.within_tolerance(got, oracle_out(case))
    _say(f"  max|err| = {err:.3e}, bound = {bound:.3e}")
    assert ok, f"{name} m={m} cap={cap}: {err} > {bound}"
    del layer
    torch.cuda.empty_cache()
