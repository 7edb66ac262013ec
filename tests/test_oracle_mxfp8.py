"""Pins for the oracle's MXFP8 quantiser and the W4A8 forward (CPU only).

MXFP8 here: E4M3FN elements (OCP FP8) with one E8M0 scale per 32 along K, scale
2^ceil(log2(amax/448)); the W4A8 variant quantises the activation output this way
before FC2 (FlashInfer PR 4255, review: the grouped MXFP8 quantisation of the
SiLU-mul output). Pinned by hand-worked scales and ties, torch's independent
float8_e4m3fn converter, grid round trips, an accuracy bound, and a hand-computed
layer whose intermediate needs a tie-breaking rounding.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as M

torch = pytest.importorskip("torch")


def _q(row):
    a = np.zeros((1, 32))
    a[0, :len(row)] = row
    c, s = F.quantise_mxfp8(a)
    return c[0], int(s[0, 0]), F.dequant_mxfp8(c, s)[0]


@pytest.mark.parametrize("amax,byte", [(448.0, 127), (449.0, 128), (1.0, 119), (224.0, 126), (224.5, 127),
                                       (2.0 ** -140, 0), (3.0 * 2.0 ** 100, 220)])
def test_scale_byte_hand_cases(amax, byte):
    # 2^ceil(log2(amax / 448)): 1/448 -> 2^-8.81 -> e = -8; 224/448 = 2^-1 exactly; 224.5 just above;
    # a tiny group clamps to e = -127; 3 * 2^100 / 448 = 2^(100 - 7.22) -> e = 93, byte 220
    _, s, _ = _q([amax])
    assert s == byte


def test_zero_group_stores_zero_scale_and_codes():
    c, s, d = _q([0.0, -0.0])
    assert s == 0 and not np.any(c & 0x7F) and np.all(d == 0)


@pytest.mark.parametrize("v,want", [
    (17.0, 16.0),              # tie between 16 (mantissa 000) and 18 (001): even
    (19.0, 20.0),              # tie between 18 (001) and 20 (010): even
    (232.0, 224.0),            # tie between 224 (110) and 240 (111): even
    (1.5 * 2.0 ** -9, 2.0 ** -8),   # subnormal tie between codes 1 and 2: even code 2
    (0.5 * 2.0 ** -9, 0.0),    # tie between 0 and the smallest subnormal: code 0
    (-17.0, -16.0),
])
def test_e4m3_ties_at_unit_scale(v, want):
    # 448 in the group fixes the scale at 2^0 (byte 127)
    _, s, d = _q([448.0, v])
    assert s == 127
    assert d[1] == want


def test_hand_pair_needs_a_tie():
    # amax 9 -> e = ceil(log2(9/448)) = -5; 9 * 32 = 288 is on the grid; 1.5625 * 32 = 50 lies
    # halfway between 48 and 52 and goes to 48 (even mantissa): 1.5
    c, s, d = _q([9.0, 1.5625])
    assert s == 122 and c[0] == 0x79 and c[1] == 0x64
    assert d[0] == 9.0 and d[1] == 1.5


@pytest.mark.parametrize("k", [32, 40, 96, 200])
def test_random_groups_match_torch_and_invariants(k):
    rng = np.random.default_rng(k)
    rows = []
    for mag in range(-24, 25, 4):
        rows.append(rng.standard_normal(k) * 2.0 ** mag)
    rows.append(np.where(rng.random(k) < 0.5, 0.0, rng.standard_normal(k)))     # sparse groups
    a = np.array(rows, dtype=np.float32).astype(np.float64)                    # float32-exact inputs
    codes, scales = F.quantise_mxfp8(a)
    d = F.dequant_mxfp8(codes, scales)
    assert not np.any((codes & 0x7F) == 0x7F)                                   # never NaN
    for g in range(scales.shape[1]):
        blk = a[:, g * 32:(g + 1) * 32]
        amax = np.max(np.abs(blk), axis=1)
        sc = np.ldexp(1.0, scales[:, g].astype(np.int64) - 127)
        nz = amax > 0
        ratio = amax[nz] / sc[nz]
        assert np.all(ratio > 224.0) and np.all(ratio <= 448.0)
        # torch's converter on the scaled values (exact in float32): the same codes
        scaled = torch.from_numpy((blk * (1.0 / sc)[:, None]).astype(np.float32))
        tcode = scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        mine = codes[:, g * 32:(g + 1) * 32]
        assert np.array_equal(tcode[nz], mine[nz])
    # accuracy: half an E4M3 spacing (relative 2^-4 for normals, 2^-10 of the scale below)
    sc_el = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)[:, :k]
    assert np.all(np.abs(d - a) <= np.maximum(2.0 ** -4 * np.abs(a), 2.0 ** -10 * sc_el) + 0.0)


def test_round_trip_on_grid():
    rng = np.random.default_rng(7)
    k = 96
    codes = rng.integers(0, 256, size=(50, k)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E                                         # no NaN
    for g in range(k // 32):                                                     # one +-448 per group
        codes[:, g * 32 + rng.integers(0, 32)] = np.where(rng.random(50) < 0.5, 0x7E, 0xFE)
    scales = rng.integers(100, 150, size=(50, k // 32)).astype(np.uint8)
    a = F.dequant_mxfp8(codes, scales)
    c2, s2 = F.quantise_mxfp8(a)
    assert np.array_equal(s2, scales) and np.array_equal(c2, codes)


def test_tail_group_uses_its_own_elements():
    a = np.zeros((1, 40))
    a[0, 0] = 448.0
    a[0, 35] = 3.0                                   # tail of 8: amax 3 -> e = ceil(log2(3/448)) = -7
    c, s = F.quantise_mxfp8(a)
    assert s.shape == (1, 2) and s[0, 0] == 127 and s[0, 1] == 120
    assert F.dequant_mxfp8(c, s)[0, 35] == 3.0


def _mx_weights(rows, cols, entries):
    """MXFP4 codes for a [rows, cols] matrix with the given {(r, c): code} and scale 2^0."""
    codes = np.zeros((1, rows, cols), np.uint8)
    for (r, c), v in entries.items():
        codes[0, r, c] = v
    return F.pack_nibbles(codes), np.full((1, rows, -(-cols // 32)), 127, np.uint8)


def test_w4a8_hand_layer():
    """E = 1, H = 32, I = 32, relu2, one token, weight 1. x = [1, 0.25, 0, ...].
    W1 row 0 = 3 at h = 0 (code 0x5); row 1 = 1 at h = 0 and h = 1 (code 0x2): h = [3, 1.25, 0...].
    relu2: a = [9, 1.5625, 0, ...]; MXFP8 makes it [9, 1.5] (the tie above).
    Every W2 row = [1, 2, 0, ...]: y = 9 + 3 = 12 (W4A8) against 9 + 3.125 = 12.125 (W4A16)."""
    w1, s1 = _mx_weights(32, 32, {(0, 0): 0x5, (1, 0): 0x2, (1, 1): 0x2})
    w2, s2 = _mx_weights(32, 32, {**{(r, 0): 0x2 for r in range(32)}, **{(r, 1): 0x4 for r in range(32)}})
    ex = M.Experts("mxfp4", "relu2", 32, 32, {"w13": w1, "s13": s1, "w2": w2, "s2": s2})
    x = np.zeros((1, 32))
    x[0, 0], x[0, 1] = 1.0, 0.25
    ids, w = np.zeros((1, 1), np.int32), np.ones((1, 1))
    out8 = M.moe_forward(x, ids, w, None, 1, 1, ex, mxfp8=True)
    out16 = M.moe_forward(x, ids, w, None, 1, 1, ex)
    assert np.all(out8 == 12.0) and np.all(out16 == 12.125)
    assert np.array_equal(M.moe_forward_loop(x, ids, w, None, 1, 1, ex, mxfp8=True), out8)


def test_w4a8_equals_w4a16_when_the_intermediate_is_on_the_grid():
    # relu2 of integers in [0, 4] gives {0, 1, 4, 9, 16}: exact in MXFP8 for every group maximum
    rng = np.random.default_rng(3)
    E, H, I, m, k = 3, 64, 64, 5, 2
    w1c = rng.choice(np.array([0x0, 0x2, 0x4, 0xA], np.uint8), size=(E, I, H))   # 0, 1, 2, -1
    w1c[:, :, 2:] = 0                                                              # only h = 0, 1 used
    w2c = rng.integers(0, 16, size=(E, H, I)).astype(np.uint8)
    codes = {"w13": F.pack_nibbles(w1c), "s13": np.full((E, I, H // 32), 127, np.uint8),
             "w2": F.pack_nibbles(w2c), "s2": rng.integers(120, 130, size=(E, H, I // 32)).astype(np.uint8)}
    ex = M.Experts("mxfp4", "relu2", H, I, codes)
    x = np.zeros((m, H))
    x[:, :2] = rng.integers(0, 2, size=(m, 2))
    ids = rng.integers(0, E, size=(m, k)).astype(np.int32)
    w = rng.random((m, k))
    assert np.array_equal(M.moe_forward(x, ids, w, None, E, E, ex, mxfp8=True), M.moe_forward(x, ids, w, None, E, E, ex))


def test_w4a8_router_weight_is_outside_the_quantisation():
    rng = np.random.default_rng(5)
    E, H, I, m, k = 4, 64, 96, 6, 3
    w13 = rng.standard_normal((E, 2 * I, H)) * 0.3
    w2 = rng.standard_normal((E, H, I)) * 0.3
    p13, s13 = F.quantise_mxfp4(w13)
    p2, s2 = F.quantise_mxfp4(w2)
    ex = M.Experts("mxfp4", "silu_swiglu", H, I, {"w13": p13, "s13": s13, "w2": p2, "s2": s2})
    x = rng.standard_normal((m, H))
    ids = rng.integers(0, E, size=(m, k)).astype(np.int32)
    w = rng.random((m, k))
    o1 = M.moe_forward(x, ids, w, None, E, E, ex, mxfp8=True)
    o2 = M.moe_forward(x, ids, 4.0 * w, None, E, E, ex, mxfp8=True)
    assert np.array_equal(o2, 4.0 * o1)
    # the quantisation moves the result, but only by the MXFP8 rounding of the intermediate
    o16 = M.moe_forward(x, ids, w, None, E, E, ex)
    assert not np.array_equal(o1, o16)
    assert np.max(np.abs(o1 - o16)) <= 2.0 ** -3 * np.max(np.abs(o16))
    assert np.allclose(M.moe_forward_loop(x, ids, w, None, E, E, ex, mxfp8=True), o1, rtol=1e-12, atol=1e-12)
