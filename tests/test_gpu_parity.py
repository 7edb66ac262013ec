"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Route packing must be bit-exact; the prepared weights must invert byte-exactly to the
canonical codes; the fused layer must satisfy max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3
in bf16 on every workload shape, on the default dispatch and with each path forced.
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


# ----------------------------------------------------------------------------- route packing

def _gpu_route_pack(moe, device, ids, emap, eg, E, B, cap, ws=None):
    k = ids.shape[1]
    nbytes = moe.moe_route_pack_workspace_size(cap, k, E, B)
    if ws is None:
        ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device=device)   # garbage: result must not depend on it
    d_ids = dev(ids.astype(np.int32), device)
    d_map = dev(emap.astype(np.int32), device) if emap is not None else None
    view = moe.moe_route_pack(d_ids, ids.shape[0], k, d_map, eg, E, B, cap, ws, nbytes)
    torch.cuda.synchronize()
    base = ws.data_ptr()

    def read(ptr, n):
        off = ptr - base
        return ws[off:off + 4 * n].view(torch.int32).cpu().numpy().copy()

    return {
        "expert_counts": read(view.expert_counts, E),
        "expert_offsets": read(view.expert_offsets, E + 1),
        "sorted_route_ids": read(view.sorted_route_ids, view.cap_routes),
        "block_expert": read(view.block_expert, view.cap_blocks),
        "live": read(view.live, 4),
        "route_slot": read(view.route_slot, cap * k),
    }, ws


@pytest.mark.parametrize("name", ["tiny", "decode", "small", "prefill", "edge"])
@pytest.mark.parametrize("block_m", [16, 32, 64, 128])
def test_route_pack_bit_exact_full_configs(moe, device, name, block_m):
    cfg = C.get_config(name)
    for m in cfg.ms:
        _say(f"route_pack {name} m={m} B={block_m}")
        ids, _, emap, _ = D.draw_routing(cfg, m, seed=cfg.index)
        cap = RP.token_capacity(m)
        got, _ = _gpu_route_pack(moe, device, ids, emap, cfg.num_global_experts, cfg.num_experts, block_m, cap)
        want = RP.route_pack(ids, emap, cfg.num_global_experts, cfg.num_experts, block_m, cap)
        for key in want:
            assert np.array_equal(got[key], want[key]), (name, m, block_m, key)


def test_route_pack_capacity_reuse_one_workspace(moe, device):
    cfg = C.get_config("edge")
    ws = None
    for m in (512, 300, 511):
        _say(f"route_pack edge reuse m={m}")
        ids, _, emap, _ = D.draw_routing(cfg, m, seed=10 + m)
        got, ws = _gpu_route_pack(moe, device, ids, emap, cfg.num_global_experts, cfg.num_experts, 16, 512, ws)
        want = RP.route_pack(ids, emap, cfg.num_global_experts, cfg.num_experts, 16, 512)
        for key in want:
            assert np.array_equal(got[key], want[key]), (m, key)


@pytest.mark.parametrize("seed", range(6))
def test_route_pack_edge_cases(moe, device, seed):
    rng = np.random.default_rng(100 + seed)
    cases = [
        (np.zeros((0, 4), np.int32), None, 8, 8),                         # m = 0
        (np.full((5, 3), -1, np.int32), None, 8, 8),                      # everything dropped
        (np.full((7, 4), 2, np.int32), None, 8, 8),                       # one expert, duplicates
        (rng.integers(-3, 40, (33, 6)).astype(np.int32), rng.integers(-1, 20, 36).astype(np.int32), 36, 17),
        (rng.integers(0, 3, (1000, 8)).astype(np.int32), None, 3, 3),     # heavy skew, several chunks
    ]
    ids, emap, eg, E = cases[seed % len(cases)]
    B = [16, 32, 64, 128][seed % 4]
    cap = RP.token_capacity(ids.shape[0])
    _say(f"route_pack edge case {seed} m={ids.shape[0]} B={B}")
    got, _ = _gpu_route_pack(moe, device, ids, emap, eg, E, B, cap)
    want = RP.route_pack(ids, emap, eg, E, B, cap)
    for key in want:
        assert np.array_equal(got[key], want[key]), key


# ----------------------------------------------------------------------------- prepare inverse

def _invert_prepared(buf: np.ndarray, cfg: C.Workload):
    """Canonical codes back from the prepared bytes, written from the documented layout."""
    E, H, I = cfg.num_experts, cfg.hidden, cfg.inter
    hp, ip = -(-H // 128) * 128, -(-I // 128) * 128
    swiglu = cfg.act == "silu_swiglu"
    n1g = (2 if swiglu else 1) * ip // 16
    n2g = hp // 16
    kb1, kb2 = hp // 128, ip // 128
    nv = cfg.fmt == "nvfp4"
    chunk = 512 if nv else 256

    def a256(v):
        return (v + 255) // 256 * 256

    sc1pg = -(-kb1 // 4) * chunk
    sc2pg = -(-kb2 // 4) * chunk
    o_n1 = 0
    o_s1 = a256(o_n1 + E * n1g * kb1 * 1024)
    o_n2 = a256(o_s1 + E * n1g * sc1pg)
    o_s2 = a256(o_n2 + E * n2g * kb2 * 1024)
    o_g13 = a256(o_s2 + E * n2g * sc2pg)
    o_g2 = a256(o_g13 + 4 * E)

    def nibbles(off, groups, kbs):
        a = buf[off:off + E * groups * kbs * 1024].reshape(E, groups, kbs, 4, 16, 4, 4)   # kb, q, r, s, byte
        a = a.transpose(0, 1, 4, 2, 5, 3, 6)                                               # E, g, r, kb, s, q, b
        return a.reshape(E, groups * 16, kbs * 64)                                         # row, byte along K

    def scales(off, groups, per_group):
        nch = per_group // chunk
        a = buf[off:off + E * groups * per_group]
        if nv:
            a = a.reshape(E, groups, nch, 2, 16, 4, 4).transpose(0, 1, 4, 2, 5, 6, 3)     # r, ch, kbm, s, h
            return a.reshape(E, groups * 16, nch * 32)
        a = a.reshape(E, groups, nch, 16, 4, 4).transpose(0, 1, 3, 2, 4, 5)               # r, ch, kbm, s
        return a.reshape(E, groups * 16, nch * 16)

    def fc1_rows(a):
        if not swiglu:
            return a[:, :I]
        a = a.reshape(E, ip // 16, 2, 16, a.shape[-1]).transpose(0, 2, 1, 3, 4).reshape(E, 2, ip, a.shape[-1])
        return a[:, :, :I].reshape(E, 2 * I, a.shape[-1])

    G = 16 if nv else 32
    n13 = fc1_rows(nibbles(o_n1, n1g, kb1))
    s13 = fc1_rows(scales(o_s1, n1g, sc1pg))
    n2 = nibbles(o_n2, n2g, kb2)[:, :H]
    s2 = scales(o_s2, n2g, sc2pg)[:, :H]
    out = {
        "w13": n13[..., :H // 2], "s13": s13[..., :-(-H // G)],
        "w2": n2[..., :I // 2], "s2": s2[..., :-(-I // G)],
        "g13": buf[o_g13:o_g13 + 4 * E].view(np.float32), "g2": buf[o_g2:o_g2 + 4 * E].view(np.float32),
        "pad_nib13": n13[..., H // 2:], "pad_nib2": n2[..., I // 2:],
    }
    return out


@pytest.mark.parametrize("name", list(SCALED))
def test_prepare_inverts_byte_exact(moe, device, name):
    cfg = SCALED[name]
    _say(f"prepare inverse {name}")
    case = make_case(cfg, 1, seed=3, weights="random")
    layer = make_layer(case, device)
    torch.cuda.synchronize()
    buf = layer.prepared.cpu().numpy()
    inv = _invert_prepared(buf, cfg)
    for key in ("w13", "s13", "w2", "s2"):
        assert np.array_equal(inv[key], case.codes[key]), key
    if cfg.fmt == "nvfp4":
        assert np.array_equal(inv["g13"], case.codes["g13"]) and np.array_equal(inv["g2"], case.codes["g2"])
    else:
        assert np.all(inv["g13"] == 1.0) and np.all(inv["g2"] == 1.0)
    assert not inv["pad_nib13"].any() and not inv["pad_nib2"].any()


# ----------------------------------------------------------------------------- fused layer

def _check(case, got, tokens=None, cols=None, label=""):
    ref = oracle_out(case, tokens=tokens, cols=cols)
    if tokens is not None or cols is not None:
        t = np.arange(case.m) if tokens is None else np.asarray(tokens)
        c = np.arange(case.cfg.hidden) if cols is None else np.asarray(cols)
        got = got[np.ix_(t, c)]
    ok, err, bound = M.within_tolerance(got, ref)
    _say(f"  {label}: max|err| = {err:.3e}, bound = {bound:.3e}, max|ref| = {np.max(np.abs(ref)):.3e}")
    assert ok, f"{label}: {err} > {bound}"


FUSED_CASES = [("tiny", 4), ("decode_s", 1), ("decode_s", 4), ("decode_s", 8), ("decode_s", 16),
               ("small_s", 16), ("small_s", 64), ("prefill_s", 300), ("edge_s", 100)]


@pytest.mark.parametrize("name,m", FUSED_CASES)
@pytest.mark.parametrize("path", ["auto", "decode", "gemm"])
def test_fused_matches_oracle_scaled(moe, device, name, m, path):
    if path == "decode" and m > moe.MOE_DECODE_MAX_M:
        pytest.skip("decode path serves m <= 16")
    cfg = SCALED[name]
    _say(f"fused {name} m={m} path={path}")
    case = make_case(cfg, m, seed=cfg.index * 7 + m, weights="normal")
    layer = make_layer(case, device)
    moe.moe_w4a16_set_path(path)
    try:
        out = run_layer(layer, case, device)
    finally:
        moe.moe_w4a16_set_path("auto")
    _check(case, bf16_tensor_to_f64(out), label=f"{name} m={m} {path}")


@pytest.mark.parametrize("name,m", [("edge_s", 100), ("prefill_s", 300)])
def test_gemm_repeat_runs_over_a_dirty_workspace(moe, device, name, m):
    """The grouped-GEMM pipeline reads every activation stage only after it has landed: repeated
    runs over a workspace holding large finite garbage all match the oracle (a stage read too
    early shows up as a wrong intermediate row in some of the runs)."""
    cfg = SCALED[name]
    _say(f"gemm repeat {name} m={m}")
    case = make_case(cfg, m, seed=cfg.index * 7 + m, weights="normal")
    layer = make_layer(case, device)
    ref = oracle_out(case)
    moe.moe_w4a16_set_path("gemm")
    try:
        for rep in range(6):
            layer.workspace.fill_(0x7F)
            got = bf16_tensor_to_f64(run_layer(layer, case, device))
            ok, err, bound = M.within_tolerance(got, ref)
            assert ok, f"{name} m={m} run {rep}: {err} > {bound}"
    finally:
        moe.moe_w4a16_set_path("auto")


@pytest.mark.parametrize("name,m", [("decode_s", 8), ("decode_s", 16), ("small_s", 16)])
def test_decode_repeat_runs_over_a_dirty_workspace(moe, device, name, m):
    """The decode path reads nothing it did not write in the same call: the FC2 K-split arrival
    counts are zeroed by FC1 and every partial is written before its count goes up, so runs over
    a workspace holding garbage, and back-to-back runs with no refill, all match the oracle."""
    cfg = SCALED[name]
    _say(f"decode repeat {name} m={m}")
    case = make_case(cfg, m, seed=cfg.index * 7 + m, weights="normal")
    layer = make_layer(case, device)
    ref = oracle_out(case)
    moe.moe_w4a16_set_path("decode")
    try:
        for rep in range(6):
            if rep % 2 == 0:
                layer.workspace.fill_(0x7F if rep % 4 == 0 else 0xFF)
            got = bf16_tensor_to_f64(run_layer(layer, case, device))
            ok, err, bound = M.within_tolerance(got, ref)
            assert ok, f"{name} m={m} run {rep}: {err} > {bound}"
    finally:
        moe.moe_w4a16_set_path("auto")


def test_fused_capacity_reuse_one_workspace(moe, device):
    cfg = SCALED["edge_s"]
    case0 = make_case(cfg, 128, seed=41, weights="normal")
    layer = make_layer(case0, device, token_capacity=128)
    for m in (128, 100, 63, 64, 1):
        _say(f"fused edge_s reuse cap=128 m={m}")
        ids, w, emap, rng = D.draw_routing(cfg, m, seed=50 + m)
        xbits = D.draw_activations_bf16(rng, m, cfg.hidden)
        case = type(case0)(cfg, m, ids, w, emap, xbits, case0.codes)
        out = run_layer(layer, case, device)
        _check(case, bf16_tensor_to_f64(out), label=f"reuse m={m}")


def test_fused_hand_cases(moe, device):
    import json
    import os

    from test_oracle_moe import build_hand_case

    with open(os.path.join(os.path.dirname(__file__), "golden", "moe_hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    import fp4_weight_grouped_moe_amd as m_

    for hc in cases:
        x, codes = build_hand_case(hc)
        from oracle import formats as F
        xbits = np.zeros(x.shape, np.uint16)
        xbits[x == 1.0] = 0x3F80
        cfg = C.Workload(name=hc["name"], index=0, num_experts=1, num_global_experts=1, hidden=hc["hidden"],
                         inter=hc["inter"], topk=1, ms=(1,), fmt=hc["fmt"], act=hc["act"], routing="softmax")
        if cfg.hidden % 8:
            continue
        for path in ("decode", "gemm"):
            _say(f"hand case {hc['name']} path={path}")
            from _common import Case
            case = Case(cfg, 1, np.array(hc["topk_ids"], np.int32), np.array(hc["topk_weights"], np.float32), None,
                        xbits, codes)
            layer = make_layer(case, device)
            m_.moe_w4a16_set_path(path)
            try:
                out = run_layer(layer, case, device)
            finally:
                m_.moe_w4a16_set_path("auto")
            got = bf16_tensor_to_f64(out)
            assert np.all(got == hc["expect_bf16"]), (hc["name"], path, got)


def test_fused_dropped_tokens_are_zero_and_m0(moe, device):
    cfg = SCALED["prefill_s"]
    case = make_case(cfg, 40, seed=5, weights="normal")
    case.ids[3, :] = -1
    case.ids[17, :] = 1000
    layer = make_layer(case, device)
    for path in ("decode", "gemm"):
        if path == "decode" and case.m > 16:
            continue
        moe.moe_w4a16_set_path(path)
        try:
            out = run_layer(layer, case, device)
        finally:
            moe.moe_w4a16_set_path("auto")
        got = bf16_tensor_to_f64(out)
        assert np.all(got[3] == 0) and np.all(got[17] == 0)
        _check(case, got, label=f"dropped rows {path}")
    # m = 0 is a no-op that succeeds
    x = torch.empty((0, cfg.hidden), dtype=torch.bfloat16, device=device)
    e = torch.empty((0, cfg.topk), dtype=torch.int32, device=device)
    w = torch.empty((0, cfg.topk), dtype=torch.float32, device=device)
    out = layer(x, e, w)
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.hidden)


@pytest.mark.parametrize("name,m", [("edge_s", 1), ("edge_s", 3), ("edge_s", 8), ("edge_s", 12), ("decode_s", 8)])
def test_decode_path_map_and_dropped_routes(moe, device, name, m):
    """The decode path with an expert map, -1 and out-of-range ids, an expert repeated inside one
    token's top-k and a token whose routes are all dropped, run twice over the same workspace.
    At these small shapes the FC1 launch packs the routes itself."""
    cfg = SCALED[name]
    case = make_case(cfg, m, seed=900 + m, weights="normal")
    case.ids[0, 0] = -1
    case.ids[0, 1] = cfg.num_global_experts + 3
    if m > 1:
        case.ids[1, 1] = case.ids[1, 0]
        case.ids[m - 1, :] = -1
    _say(f"decode path {name} m={m} map={case.emap is not None}: dropped and repeated routes")
    layer = make_layer(case, device)
    moe.moe_w4a16_set_path("decode")
    try:
        got = bf16_tensor_to_f64(run_layer(layer, case, device))
        again = bf16_tensor_to_f64(run_layer(layer, case, device))
    finally:
        moe.moe_w4a16_set_path("auto")
    if m > 1:
        assert np.all(got[m - 1] == 0)
    assert np.array_equal(got, again)
    _check(case, got, label=f"decode path {name} m={m} dropped routes")


# ----------------------------------------------------------------------------- full-size, every output

@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,m", [("decode", 12), ("decode", 16), ("small", 16), ("edge", 16), ("prefill", 4),
                                    ("prefill", 12), ("prefill", 16)])
def test_decode_path_full_size_above_eight_tokens(moe, device, name, m):
    """The decode path at 9..16 tokens stages more than 64 KiB of activation rows (one FC1
    workgroup per CU, routes packed by the route-pack launch; the edge shape adds an expert
    map and -1 ids); on the prefill shape (hidden 7168) beyond 9 tokens the rows exceed the
    128 KiB of LDS and FC1 reads them from memory, NVFP4 on the bf16 route, and at 4 tokens
    the FC1 launch packs the routes itself over 256 experts: every output of the full-size
    layer against the oracle."""
    case = full_case(name, m, device)
    layer = make_layer(case, device, token_capacity=RP.token_capacity(m))
    _say(f"full {name} m={m} path=decode")
    moe.moe_w4a16_set_path("decode")
    try:
        out = run_layer(layer, case, device)
    finally:
        moe.moe_w4a16_set_path("auto")
    got = bf16_tensor_to_f64(out)
    assert np.all(np.isfinite(got))
    _check(case, got, label=f"{name} m={m} decode, every token x every column")
    del layer, case
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,ms", [("decode", (1, 4, 8)), ("small", (16, 64)), ("prefill", (2048,)),
                                     ("edge", (512, 300, 511))])
def test_fused_full_size_every_output(moe, device, name, ms):
    """The full-size workloads on the default dispatch (decode m = 1/4/8 and small m = 16 on the
    decode path; small m = 64, prefill m = 2048 and edge m = 512/300/511 on the grouped GEMM, the
    edge ones on one workspace of capacity 512): every token x every column against the oracle."""
    cap = max(RP.token_capacity(m) for m in ms)
    case0 = full_case(name, ms[0], device)
    layer = make_layer(case0, device, token_capacity=cap)
    for m in ms:
        case = full_case(name, m, device, case0.codes_dev) if m != ms[0] else case0
        _say(f"full {name} m={m} (capacity {cap})")
        out = run_layer(layer, case, device)
        got = bf16_tensor_to_f64(out)
        assert np.all(np.isfinite(got))
        _check(case, got, label=f"{name} m={m}, every token x every column")
    del layer, case0
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_fused_full_size_prefill_mxfp4_every_output(moe, device):
    """The prefill shape (256 experts, hidden 7168, inter 2048, top-8, Zipf routing, m = 2048)
    with MXFP4 weights on the W4A16 layer: the bf16-operand grouped GEMM (E8M0 scales folded into
    the FP4 convert) over full 8-block tiles, 56 FC1 and 16 FC2 K blocks, 16 / 28 N tiles per M
    tile and the per-XCD queues. Every token x every column against the oracle."""
    case = full_case("prefill", 2048, device, fmt="mxfp4")
    layer = make_layer(case, device)
    _say("full prefill mxfp4 m=2048")
    got = bf16_tensor_to_f64(run_layer(layer, case, device))
    assert np.all(np.isfinite(got))
    _check(case, got, label="prefill mxfp4 m=2048, every token x every column")
    del layer, case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("act", ["relu2", "silu_swiglu"])
@pytest.mark.parametrize("path,m", [("decode", 5), ("decode", 16), ("gemm", 40), ("gemm", 512)])
def test_fused_every_format_and_activation(moe, device, fmt, act, path, m):
    """Both weight formats with both activations on both paths (the workloads pair MXFP4 only
    with SiLU-SwiGLU and relu2 only with NVFP4, whose intermediate rows the two formats store
    differently: bf16 for MXFP4, f16 times a per-slot power of two for NVFP4 on the grouped
    GEMM). Intermediate 400 (a partial 32-group for MXFP4, a 128-block tail for both), an
    expert map with dropped ids; m = 512 puts ~100 routes on each of the 8 local experts (full
    8-block tiles). Every output against the oracle, and a second call equal to the first."""
    import dataclasses
    cfg = dataclasses.replace(C.get_config("edge"), num_experts=8, num_global_experts=16, hidden=512, inter=400,
                              act=act, fmt=fmt, name=f"edge_{fmt}_{act}")
    _say(f"{fmt} {act} m={m} path={path}")
    case = make_case(cfg, m, seed=m * 7 + len(act) + len(fmt), weights="normal")
    layer = make_layer(case, device)
    moe.moe_w4a16_set_path(path)
    try:
        got = bf16_tensor_to_f64(run_layer(layer, case, device))
        again = bf16_tensor_to_f64(run_layer(layer, case, device))
    finally:
        moe.moe_w4a16_set_path("auto")
    assert np.array_equal(got, again)
    assert np.all(np.isfinite(got))
    _check(case, got, label=f"{fmt} {act} m={m} {path}")


@pytest.mark.parametrize("path", ["decode", "gemm"])
def test_tiny_and_zero_activation_rows(moe, device, path):
    """A token row scaled by 1e-36 (its maximum below 2^-113, where the f16 conversion's power-of-two
    factor 2^-p alone would overflow) and an all-zero row, with NVFP4 weights, on the decode path
    (m = 12 at hidden 3072: the activation rows are converted by the route-pack launch) and the
    grouped GEMM: every output finite, the zero row exactly zero, and all within the oracle's
    tolerance."""
    cfg = C.scaled(C.get_config("decode"), num_experts=16, hidden=3072, inter=256, name="decode_wide")
    case = make_case(cfg, 12, seed=77, weights="normal")
    x = F.bf16_bits_to_f64(case.xbits)
    x[2] *= 1e-36
    x[5] = 0.0
    case.xbits = D.bf16_bits_from_f32(x.astype(np.float32))
    assert np.abs(F.bf16_bits_to_f64(case.xbits[2])).max() < 2.0 ** -113
    layer = make_layer(case, device)
    _say(f"tiny / zero rows path={path}")
    moe.moe_w4a16_set_path(path)
    try:
        got = bf16_tensor_to_f64(run_layer(layer, case, device))
    finally:
        moe.moe_w4a16_set_path("auto")
    assert np.all(np.isfinite(got))
    assert np.all(got[5] == 0)
    _check(case, got, label=f"tiny / zero rows {path}")


@pytest.mark.parametrize("pattern", ["smallest_expert_heavy", "middle_expert_heavy"])
def test_decode_in_launch_pack_with_repeated_ids(moe, device, pattern):
    """The decode FC1 launch that packs its own routes issues each wave's first unit before the
    pack whenever the experts up to that unit's block hold at most 16 routes each. Top-k lists
    that repeat one expert (more than 16 routes on it: two route blocks) exercise both the early
    issue (blocks before the heavy expert) and the fallback (blocks at or after it): m = 8, every
    output against the oracle."""
    cfg = SCALED["decode_s"]
    case = make_case(cfg, 8, seed=23, weights="normal")
    ids = case.ids.copy()
    heavy = 0 if pattern == "smallest_expert_heavy" else 9
    ids[:3, :] = heavy                                   # 24 routes on one expert
    if pattern == "middle_expert_heavy":
        ids[3:, :] = np.where(ids[3:, :] == heavy, 1, ids[3:, :])
    case.ids = ids.astype(np.int32)
    assert (case.ids == heavy).sum() > 16
    layer = make_layer(case, device)
    _say(f"decode in-launch pack, {pattern}")
    moe.moe_w4a16_set_path("decode")
    try:
        got = bf16_tensor_to_f64(run_layer(layer, case, device))
    finally:
        moe.moe_w4a16_set_path("auto")
    _check(case, got, label=f"decode pack {pattern}")


@pytest.mark.parametrize("name,E,hidden,inter,m", [("edge", 4, 384, 1400, 176), ("small", 8, 384, 256, 120)])
def test_gemm_six_block_tiles(moe, device, name, E, hidden, inter, m):
    """Experts with 81-96 routes, whose tail M tiles run as six-block tiles on the grouped GEMM:
    MXFP4 SwiGLU with the intermediate's K tail (I = 1400) and an expert map, and NVFP4 relu2.
    Every output against the oracle."""
    cfg = C.scaled(C.get_config(name), num_experts=E, hidden=hidden, inter=inter, name=f"{name}_six")
    case = make_case(cfg, m, seed=5, weights="normal")
    ids = case.ids[case.ids >= 0]
    loc = case.emap[ids] if case.emap is not None else ids
    counts = np.bincount(loc[loc >= 0], minlength=E)
    tails = ((counts + 15) // 16) % 8
    assert np.any((tails == 5) | (tails == 6)), counts
    layer = make_layer(case, device)
    _say(f"six-block tiles {name} m={m} expert loads {counts.tolist()}")
    moe.moe_w4a16_set_path("gemm")
    try:
        got = bf16_tensor_to_f64(run_layer(layer, case, device))
    finally:
        moe.moe_w4a16_set_path("auto")
    _check(case, got, label=f"six-block tiles {name}")


@pytest.mark.parametrize("name", ["decode_s", "small_s"])
def test_gemm_f16_intermediate_rows_across_magnitudes(moe, device, name):
    """The NVFP4 grouped GEMM stores each route's intermediate row as f16 times a power of two
    chosen from a bound on the row (activation-row norm, the expert's largest FC1 row norms, the
    global scales and the router weight). Token rows scaled by 1e-8 and 1e8, a token with router
    weights scaled by 1e-12, and one expert's global scales moved by 2^30 (FC1) and 2^-40 (FC2):
    every token's output row within the relative tolerance of its own largest value (SwiGLU and
    relu2), and none of it non-finite."""
    cfg = SCALED[name]
    assert cfg.fmt == "nvfp4"
    case = make_case(cfg, 24, seed=91, weights="normal")
    x = F.bf16_bits_to_f64(case.xbits)
    x[1] *= 1e-8
    x[4] *= 1e8
    case.xbits = D.bf16_bits_from_f32(x.astype(np.float32))
    case.w = case.w.copy()
    case.w[7] *= 1e-12
    e0 = int(case.ids[10, 0])
    case.codes = dict(case.codes)
    case.codes["g13"] = case.codes["g13"].copy()
    case.codes["g2"] = case.codes["g2"].copy()
    case.codes["g13"][e0] *= np.float32(2.0 ** 30)
    case.codes["g2"][e0] *= np.float32(2.0 ** -40)
    layer = make_layer(case, device)
    _say(f"f16 intermediate magnitudes {name} (expert {e0} rescaled)")
    moe.moe_w4a16_set_path("gemm")
    try:
        got = bf16_tensor_to_f64(run_layer(layer, case, device))
    finally:
        moe.moe_w4a16_set_path("auto")
    assert np.all(np.isfinite(got))
    ref = oracle_out(case)
    for t in range(case.m):
        ok, err, bound = M.within_tolerance(got[t], ref[t], abs_=0.0)
        assert ok, f"{name} token {t}: max|err| {err:.3e} > {bound:.3e} (max|ref| {np.abs(ref[t]).max():.3e})"
    _say(f"  every row within 2e-2 of its own maximum (row maxima {np.abs(ref).max(axis=1).min():.2e} .. "
         f"{np.abs(ref).max(axis=1).max():.2e})")
