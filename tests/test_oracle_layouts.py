"""Pins for the source-layout readings of the oracle (CPU only): hand cases, involution,
the IEEE reciprocal, and dequantised weights that do not depend on the layout."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import layouts as L


def test_half_swap_hand_case():
    rows = np.arange(2 * 2 * 3, dtype=np.uint8).reshape(1, 4, 3)      # I = 2: rows r0 r1 (up), r2 r3 (gate)
    got = L.w13_gate_first(rows, 2)
    assert got[0].tolist() == [[6, 7, 8], [9, 10, 11], [0, 1, 2], [3, 4, 5]]
    np.testing.assert_array_equal(L.w13_gate_first(got, 2), rows)     # swapping twice is the identity


def test_interleave_hand_case():
    # I = 2, rows stored alternately: g0 u0 g1 u1 (gate first) -> g0 g1 u0 u1
    rows = np.array([[[10], [20], [11], [21]]], np.uint8)
    assert L.w13_halves(rows, 2)[0, :, 0].tolist() == [10, 11, 20, 21]
    with pytest.raises(ValueError):
        L.w13_halves(np.zeros((1, 3, 1), np.uint8), 2)
    # with the up half first: u0 g0 u1 g1 -> canonical g0 g1 u0 u1
    up_first = np.array([[[20, 20], [10, 10], [21, 21], [11, 11]]], np.uint8)
    c = L.canonical("mxfp4", "silu_swiglu", 64, 2, up_first, up_first, None, None, None, None,
                    w13_up_first=True, w13_interleaved=True)
    assert c[0][0, :, 0].tolist() == [10, 11, 20, 21] and c[1][0, :, 1].tolist() == [10, 11, 20, 21]


def test_half_swap_rejects_wrong_rows():
    with pytest.raises(ValueError):
        L.w13_gate_first(np.zeros((1, 3, 2), np.uint8), 2)


@pytest.mark.parametrize("g", [0.5, 3.0, 1e-3, 4.0e-5, 7.0])
def test_reciprocal_is_the_ieee_quotient(g):
    stored = np.float32(1.0) / np.float32(g)
    got = L.global_from_encode(np.array([stored], np.float32))[0]
    assert got == np.float32(1.0) / stored                            # fp32 division, correctly rounded
    assert abs(float(got) - g) <= 2 * np.spacing(np.float32(g))       # within two ulp of the original


def test_powers_of_two_are_exact():
    stored = np.array([0.25, 8.0, 2.0 ** -20], np.float32)
    np.testing.assert_array_equal(L.global_from_encode(stored), np.array([4.0, 0.125, 2.0 ** 20], np.float32))


def test_per_row_scales_repeat_hand_case():
    per_row = np.array([[[7], [9]]], np.uint8)                         # E = 1, N = 2
    got = L.scales_from_per_row(per_row, k=40, group=16)              # ceil(40 / 16) = 3 groups
    assert got.tolist() == [[[7, 7, 7], [9, 9, 9]]]
    with pytest.raises(ValueError):
        L.scales_from_per_row(np.zeros((1, 2, 2), np.uint8), 40, 16)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_dequantised_weights_do_not_depend_on_layout(fmt):
    rng = np.random.default_rng(4)
    e, h, i = 2, 64, 32
    group = 16 if fmt == "nvfp4" else 32
    w13 = rng.integers(0, 256, size=(e, 2 * i, h // 2), dtype=np.uint8)
    w2 = rng.integers(0, 256, size=(e, h, i // 2), dtype=np.uint8)
    band = (0x70, 0x7B) if fmt == "nvfp4" else (119, 122)
    r13 = rng.integers(*band, size=(e, 2 * i, 1), dtype=np.uint8)    # one scale per row
    r2 = rng.integers(*band, size=(e, h, 1), dtype=np.uint8)
    g13 = np.array([2.0, 0.5], np.float32)
    g2 = np.array([0.25, 4.0], np.float32)
    # the variant: up half first, rows interleaved, encode-sense globals, per-row scales
    def stored(a):
        a = np.concatenate([a[:, i:], a[:, :i]], axis=1)                # up half first
        return np.stack([a[:, :i], a[:, i:]], axis=2).reshape(a.shape)  # then row by row
    v13, vr13 = stored(w13), stored(r13)
    c = L.canonical(fmt, "silu_swiglu", h, i, v13, vr13, np.float32(1) / g13, w2, r2, np.float32(1) / g2,
                    w13_up_first=True, global_scale_reciprocal=True, scale_per_row=True, w13_interleaved=True)
    want13 = F.dequant(fmt, w13, np.repeat(r13, h // group, axis=2), g13 if fmt == "nvfp4" else None)
    got13 = F.dequant(fmt, c[0], c[1], c[2] if fmt == "nvfp4" else None)
    np.testing.assert_array_equal(got13, want13)
    want2 = F.dequant(fmt, w2, np.repeat(r2, i // group, axis=2), g2 if fmt == "nvfp4" else None)
    got2 = F.dequant(fmt, c[3], c[4], c[5] if fmt == "nvfp4" else None)
    np.testing.assert_array_equal(got2, want2)


def test_relu2_ignores_the_half_order():
    w1 = np.arange(12, dtype=np.uint8).reshape(1, 4, 3)
    c = L.canonical("mxfp4", "relu2", 6, 4, w1, np.zeros((1, 4, 1), np.uint8), None, w1, np.zeros((1, 6, 1), np.uint8),
                    None, w13_up_first=True)
    np.testing.assert_array_equal(c[0], w1)
