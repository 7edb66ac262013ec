"""Pins for the oracle's code tables, quantisers and bf16 rounding (CPU only).

Each check ties the oracle to something other than itself: the OCP MX v1.0 E2M1
value list typed from the specification, torch's float8 / bfloat16 decoders and
converters (library routines), exact rational arithmetic, and hand tie tables.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

# OCP MX v1.0, E2M1 code points 0000 .. 1111 (positive half, then the negated half).
SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_table_matches_spec_list():
    assert F.E2M1_TABLE.tolist() == SPEC_E2M1
    assert np.signbit(F.E2M1_TABLE[8])                     # 0x8 is -0


def test_e4m3_table_matches_torch_decoder():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(F.E4M3_TABLE), nan)
    assert nan.sum() == 2                                  # 0x7F and 0xFF only
    assert np.array_equal(F.E4M3_TABLE[~nan], ref[~nan])
    assert F.E4M3_TABLE[0x7E] == 448.0 and F.E4M3_TABLE[0x01] == 2.0 ** -9


def test_e8m0_table_matches_torch_decoder():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(F.E8M0_TABLE[255]) and np.isnan(ref[255])
    assert np.array_equal(F.E8M0_TABLE[:255], ref[:255])
    assert F.E8M0_TABLE[127] == 1.0 and F.E8M0_TABLE[0] == 2.0 ** -127


@pytest.mark.parametrize("v,code", [
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),   # ties -> even mantissa
    (0.26, 1), (0.74, 1), (2.49, 4), (2.51, 5), (4.99, 6), (5.01, 7),
    (6.0, 7), (7.0, 7), (1e9, 7),                                                # saturation at 6
    (-0.75, 10), (-5.0, 14), (-100.0, 15), (0.0, 0),
])
def test_e2m1_rounding_ties_and_saturation(v, code):
    assert int(F.e2m1_encode(v)) == code


def test_e2m1_encode_matches_exhaustive_distance_search():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.uniform(-8, 8, 4000), np.array(SPEC_E2M1) * 1.0,
                        (np.array(SPEC_E2M1[:8])[1:] + np.array(SPEC_E2M1[:8])[:-1]) / 2])
    codes = F.e2m1_encode(v)
    for x, c in zip(v, codes):
        d = [abs(abs(x) - abs(SPEC_E2M1[i])) for i in range(8)]
        best = min(d)
        cands = [i for i in range(8) if d[i] == best]
        want = [i for i in cands if i % 2 == 0][0] if len(cands) > 1 else cands[0]
        assert (int(c) & 7) == want
        assert (int(c) >> 3) == (1 if np.signbit(x) else 0)


def test_e4m3_encode_matches_torch_conversion_in_range():
    rng = np.random.default_rng(6)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000))
    v = mags * rng.choice([-1.0, 1.0], mags.size)
    v = np.concatenate([v, F.E4M3_TABLE[:127], (F.E4M3_TABLE[1:127] + F.E4M3_TABLE[:126]) / 2])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(v.astype(np.float32).astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    assert int(F.e4m3_encode(1e6)) == 0x7E and int(F.e4m3_encode(-1e6)) == 0xFE
    assert int(F.e4m3_encode(470.0)) == 0x7E


def test_ceil_log2_exact_against_rationals():
    rng = np.random.default_rng(7)
    xs = list(np.exp(rng.uniform(-80, 80, 3000))) + [2.0 ** e for e in range(-130, 130)] + \
        [np.nextafter(2.0 ** e, 0) for e in range(-60, 60)] + [np.nextafter(2.0 ** e, 10 ** 40) for e in range(-60, 60)]
    got = F.ceil_log2(np.array(xs))
    for x, g in zip(xs, got):
        fx = Fraction(float(x))
        assert Fraction(2) ** int(g) >= fx and Fraction(2) ** (int(g) - 1) < fx


def test_pack_nibble_order():
    assert F.pack_nibbles(np.array([1, 2], dtype=np.uint8)).tolist() == [0x21]
    codes = np.random.default_rng(1).integers(0, 16, (3, 5, 18)).astype(np.uint8)
    assert np.array_equal(F.unpack_nibbles(F.pack_nibbles(codes)), codes)
    with pytest.raises(ValueError):
        F.pack_nibbles(np.zeros(3, dtype=np.uint8))


def test_mxfp4_scale_rule_invariant_and_tail():
    rng = np.random.default_rng(8)
    w = rng.standard_normal((7, 40)) * 0.02                # K = 40 -> groups of 32 and a tail of 8
    packed, scales = F.quantise_mxfp4(w)
    assert packed.shape == (7, 20) and scales.shape == (7, 2)
    for gi, (a, b) in enumerate([(0, 32), (32, 40)]):
        amax = np.max(np.abs(w[:, a:b]), axis=1)
        scale = 2.0 ** (scales[:, gi].astype(np.int64) - 127)
        ratio = amax / scale
        assert np.all(ratio > 3.0) and np.all(ratio <= 6.0)
    wh = F.dequant_mxfp4(packed, scales)
    scale_full = np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)[:, :40]
    assert np.all(np.abs(wh - w) <= scale_full * 1.0 + 1e-30)   # half the widest E2M1 gap (2) times scale


def test_mxfp4_grid_values_round_trip_exactly():
    rng = np.random.default_rng(9)
    e = rng.integers(-20, 10, size=(5, 3))
    codes = rng.integers(0, 16, size=(5, 96))
    codes[:, ::32] = 7                                     # each group's amax is exactly 6 * 2^e
    vals = np.array(SPEC_E2M1)[codes] * np.repeat(2.0 ** e, 32, axis=1)
    packed, scales = F.quantise_mxfp4(vals)
    assert np.array_equal(scales.astype(np.int64), e + 127)
    assert np.array_equal(F.dequant_mxfp4(packed, scales), vals)


def test_mxfp4_zero_group_is_byte_zero_and_zero_codes():
    w = np.zeros((2, 64))
    w[1, 40] = 0.3
    packed, scales = F.quantise_mxfp4(w)
    assert scales[0].tolist() == [0, 0] and scales[1, 0] == 0 and scales[1, 1] != 0
    assert np.all(F.unpack_nibbles(packed)[0] == 0)
    assert np.all(F.dequant_mxfp4(packed, scales)[0] == 0)


def test_nvfp4_two_level_scales():
    rng = np.random.default_rng(10)
    w = rng.standard_normal((3, 6, 48)) * 0.02
    w[2] = 0.0                                             # an all-zero expert
    packed, scales, g = F.quantise_nvfp4(w)
    assert scales.shape == (3, 6, 3) and g.dtype == np.float32
    for e in range(2):
        assert g[e] == np.float32(np.max(np.abs(w[e])) / 2688.0)
        sv = F.E4M3_TABLE[scales[e]]
        amax_b = np.max(np.abs(w[e].reshape(6, 3, 16)), axis=2)
        # the E4M3 scale is amax/6/g rounded to 4 significant bits (relative error <= 1/16)
        assert np.all(np.abs(sv * 6 * float(g[e]) - amax_b) <= amax_b / 16 + 1e-12)
    assert g[2] == 1.0 and np.all(scales[2] == 0) and np.all(packed[2] == 0)
    wh = F.dequant_nvfp4(packed, scales, g)
    assert np.all(wh[2] == 0)
    sv_full = np.repeat(F.E4M3_TABLE[scales[:2]], 16, axis=2) * g[:2, None, None]
    assert np.all(np.abs(wh[:2] - w[:2]) <= sv_full * 1.0 + 1e-12)


def test_nvfp4_dequant_hand_values():
    packed = F.pack_nibbles(np.array([[[3, 15] + [0] * 14]], dtype=np.uint8))
    scales = np.array([[[0x3C]]], dtype=np.uint8)          # 1.5
    wh = F.dequant_nvfp4(packed, scales, np.array([0.5], dtype=np.float32))
    assert wh[0, 0, 0] == 1.5 * 1.5 * 0.5 and wh[0, 0, 1] == -6 * 1.5 * 0.5


def test_bf16_round_matches_torch_including_ties_and_subnormals():
    rng = np.random.default_rng(11)
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32),
        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32),       # exact ties
        (rng.integers(0, 1 << 23, 4000, dtype=np.uint32)).view(np.float32),           # subnormals
        np.array([3.3961e38, 3.4e38, -3.4e38, 1e-45], dtype=np.float32),
    ])
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    got = F.bf16_round(f.astype(np.float64))
    same = (got == ref) | (np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref)))
    assert np.all(same)


def test_bf16_bits_decoder_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = F.bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
