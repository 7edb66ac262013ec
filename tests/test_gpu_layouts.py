"""Preparation from the source-layout variants (GPU): the prepared buffer equals, byte for
byte, the one prepared from the canonical arrays that the oracle maps the variant to."""

from __future__ import annotations

import itertools

import numpy as np
import pytest

from oracle import layouts as L
from synth import draw as D

from _common import SCALED

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

    return m


def _interleave(a, inter):
    """The two W13 halves stored row by row alternately (rows 2i, 2i + 1 = row i of each)."""
    return np.stack([a[:, :inter], a[:, inter:]], axis=2).reshape(a.shape)


def _variant(cfg, seed, up_first, reciprocal, per_row, interleaved=0):
    """A source-layout variant drawn at random: (w13, s13, g13, w2, s2, g2) as stored."""
    codes = D.draw_random_codes(cfg, seed)
    w13, s13, g13, w2, s2, g2 = (codes[k] for k in ("w13", "s13", "g13", "w2", "s2", "g2"))
    if per_row:
        s13 = np.ascontiguousarray(s13[:, :, :1])
        s2 = np.ascontiguousarray(s2[:, :, :1])
    if up_first and cfg.act == "silu_swiglu":
        w13 = L.w13_gate_first(w13, cfg.inter)          # the swap is its own inverse
        s13 = L.w13_gate_first(s13, cfg.inter)
    if interleaved and cfg.act == "silu_swiglu":
        w13 = _interleave(w13, cfg.inter)
        s13 = _interleave(s13, cfg.inter)
    if reciprocal and cfg.fmt == "nvfp4":
        g13 = (np.float32(1) / np.asarray(g13, np.float32)).astype(np.float32)
        g2 = (np.float32(1) / np.asarray(g2, np.float32)).astype(np.float32)
    return w13, s13, g13, w2, s2, g2


def _prepare(moe, device, cfg, arrays, layout):
    import torch

    dims = moe.make_dims(cfg.fmt, cfg.act, cfg.num_experts, cfg.hidden, cfg.inter)
    size = moe.moe_w4a16_prepared_size(dims)
    out = torch.full((size,), 0xA5, dtype=torch.uint8, device=device)
    t = [torch.from_numpy(np.ascontiguousarray(a)).to(device) if a is not None else None for a in arrays]
    if cfg.fmt != "nvfp4":
        t[2] = t[5] = None
    if layout is None:
        moe.moe_w4a16_prepare(dims, t[0], t[1], t[2], t[3], t[4], t[5], out, size)
    else:
        moe.moe_w4a16_prepare_layout(dims, layout, t[0], t[1], t[2], t[3], t[4], t[5], out, size)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", ["decode_s", "small_s", "edge_s"])
@pytest.mark.parametrize("up_first,reciprocal,per_row", list(itertools.product([0, 1], repeat=3))[1:])
def test_prepare_layout_equals_canonical(moe, device, name, up_first, reciprocal, per_row):
    cfg = SCALED[name]
    print(f"layout {name} up_first={up_first} reciprocal={reciprocal} per_row={per_row}", flush=True)
    var = _variant(cfg, 77 + 8 * up_first + 4 * reciprocal + 2 * per_row, up_first, reciprocal, per_row)
    canon = L.canonical(cfg.fmt, cfg.act, cfg.hidden, cfg.inter, *var, w13_up_first=bool(up_first),
                        global_scale_reciprocal=bool(reciprocal), scale_per_row=bool(per_row))
    layout = moe.moe_w4a16_source_layout(up_first, reciprocal, per_row)
    got = _prepare(moe, device, cfg, var, layout)
    want = _prepare(moe, device, cfg, canon, None)
    assert got.shape == want.shape
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} prepared bytes differ, first at {bad[:8]}"


def test_prepare_layout_rejects_bad_flags(moe, device):
    import torch

    cfg = SCALED["decode_s"]
    dims = moe.make_dims(cfg.fmt, cfg.act, cfg.num_experts, cfg.hidden, cfg.inter)
    size = moe.moe_w4a16_prepared_size(dims)
    buf = torch.empty(size, dtype=torch.uint8, device=device)
    with pytest.raises(moe.MoeError):
        moe.moe_w4a16_prepare_layout(dims, moe.moe_w4a16_source_layout(2, 0, 0), buf, buf, buf, buf, buf, buf, buf, size)
    with pytest.raises(moe.MoeError):
        moe.moe_w4a16_prepare_layout(dims, moe.moe_w4a16_source_layout(0, 0, 0, 3), buf, buf, buf, buf, buf, buf, buf, size)


def _odd(base, H, I):
    import dataclasses

    from synth import configs as C
    return dataclasses.replace(C.get_config(base), num_experts=4, num_global_experts=8 if base == "edge" else 4,
                               hidden=H, inter=I, name=f"{base}_h{H}_i{I}")


ODD = [_odd("decode", 200, 136), _odd("small", 264, 100), _odd("edge", 1000, 72)]


@pytest.mark.parametrize("cfg", ODD, ids=lambda c: c.name)
@pytest.mark.parametrize("up_first,reciprocal,per_row", [(1, 0, 0), (0, 1, 1), (1, 1, 1)])
def test_prepare_layout_equals_canonical_odd_shapes(moe, device, cfg, up_first, reciprocal, per_row):
    """The same at hidden sizes that are not a multiple of 128 (K tails and, for NVFP4 at
    hidden 200, an 8-wide last scale group) and intermediate tails."""
    print(f"layout {cfg.name} up_first={up_first} reciprocal={reciprocal} per_row={per_row}", flush=True)
    var = _variant(cfg, 91 + 8 * up_first + 4 * reciprocal + 2 * per_row, up_first, reciprocal, per_row)
    canon = L.canonical(cfg.fmt, cfg.act, cfg.hidden, cfg.inter, *var, w13_up_first=bool(up_first),
                        global_scale_reciprocal=bool(reciprocal), scale_per_row=bool(per_row))
    layout = moe.moe_w4a16_source_layout(up_first, reciprocal, per_row)
    got = _prepare(moe, device, cfg, var, layout)
    want = _prepare(moe, device, cfg, canon, None)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} prepared bytes differ, first at {bad[:8]}"


@pytest.mark.parametrize("cfg", [SCALED["decode_s"], SCALED["edge_s"], SCALED["small_s"]] + ODD, ids=lambda c: c.name)
@pytest.mark.parametrize("up_first,per_row", [(0, 0), (1, 0), (1, 1)])
def test_prepare_layout_row_interleaved_w13(moe, device, cfg, up_first, per_row):
    """W13 (and its scales) stored with the gate and up rows alternating, alone and with the
    up half first: prepared byte for byte as the canonical arrays (relu2 ignores the flag)."""
    print(f"layout {cfg.name} interleaved up_first={up_first} per_row={per_row}", flush=True)
    var = _variant(cfg, 131 + 8 * up_first + 2 * per_row, up_first, 0, per_row, interleaved=1)
    canon = L.canonical(cfg.fmt, cfg.act, cfg.hidden, cfg.inter, *var, w13_up_first=bool(up_first),
                        scale_per_row=bool(per_row), w13_interleaved=True)
    layout = moe.moe_w4a16_source_layout(up_first, 0, per_row, 1)
    got = _prepare(moe, device, cfg, var, layout)
    want = _prepare(moe, device, cfg, canon, None)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} prepared bytes differ, first at {bad[:8]}"
