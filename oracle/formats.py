"""FP4 / FP8 / E8M0 codes, quantisers and dequantisers (oracle; test infrastructure).

The page (FlashInfer PR 4255, Description) names NVFP4 weights (E2M1 values, one
E4M3 scale per 16 along K, an fp32 global scale) and the fp4_e8m0_k32 source
(E2M1 values, one E8M0 scale per 32 along K, with a scale tail when K is not a
multiple of the group). It does not define the encodings; they are taken from
the OCP Microscaling (MX) v1.0 and OCP 8-bit floating point specifications:

* E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no inf/NaN; max 6.
* E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; S.1111.111 is NaN;
  no infinity; max 448; exponent field 0 is subnormal.
* E8M0: an unsigned biased exponent, value 2^(b-127); 0xFF is NaN.

All arithmetic is float64. Readings where the page is silent (rounding, scale
rules, packing order) are listed in the design notes and pinned by tests.
"""

from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0


# ----------------------------------------------------------------------------- code tables

def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code (bit 3 sign, bits 2..1 exponent, bit 0 mantissa)."""
    code = int(code) & 0xF
    s = code >> 3
    e = (code >> 1) & 3
    mt = code & 1
    mag = 0.5 * mt if e == 0 else (2.0 ** (e - 1)) * (1.0 + mt / 2.0)
    return -mag if s else mag


def e4m3_value(byte: int) -> float:
    """Value of an E4M3FN byte; NaN for 0x7F / 0xFF."""
    byte = int(byte) & 0xFF
    s = byte >> 7
    e = (byte >> 3) & 0xF
    mt = byte & 7
    if e == 0xF and mt == 7:
        return float("nan")
    if e == 0:
        mag = (mt / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + mt / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def e8m0_value(byte: int) -> float:
    """Value of an E8M0 scale byte: 2^(b-127); NaN for 0xFF."""
    byte = int(byte) & 0xFF
    if byte == 0xFF:
        return float("nan")
    return 2.0 ** (byte - 127)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


# ----------------------------------------------------------------------------- rounding

def _rne_to_grid(mag: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest value of an ascending non-negative grid; ties go to the even index.

    Magnitudes above the last grid value saturate to it. For E2M1 and E4M3 the
    code index equals the code, and an even code has mantissa LSB 0, so ties to
    the even index are IEEE round-half-to-even.
    """
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(grid, mag, side="left")          # grid[hi-1] < mag <= grid[hi]
    hi = np.clip(hi, 1, len(grid) - 1)
    lo = hi - 1
    d_lo = mag - grid[lo]
    d_hi = grid[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag >= grid[-1], len(grid) - 1, idx)
    idx = np.where(mag <= 0.0, 0, idx)
    return idx.astype(np.int64)


_E2M1_POS_GRID = E2M1_TABLE[:8].copy()                    # 0, .5, 1, 1.5, 2, 3, 4, 6
_E4M3_POS_GRID = E4M3_TABLE[:127].copy()                  # codes 0x00 .. 0x7E, ascending


def e2m1_encode(v) -> np.ndarray:
    """Round to the nearest E2M1 value (ties to even), saturating at +-6. Returns uint8 codes 0..15."""
    v = np.asarray(v, dtype=np.float64)
    idx = _rne_to_grid(np.abs(v), _E2M1_POS_GRID)
    sign = np.signbit(v).astype(np.int64) << 3
    return (idx | sign).astype(np.uint8)


def e4m3_encode(v) -> np.ndarray:
    """Round to the nearest E4M3FN value (ties to even), saturating at +-448. Returns uint8 bytes."""
    v = np.asarray(v, dtype=np.float64)
    idx = _rne_to_grid(np.abs(v), _E4M3_POS_GRID)
    sign = np.signbit(v).astype(np.int64) << 7
    return (idx | sign).astype(np.uint8)


def ceil_log2(x) -> np.ndarray:
    """Exact ceil(log2(x)) for finite x > 0, from the binary exponent (no log2 rounding)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                                     # x = m * 2^e, m in [0.5, 1)
    return np.where(m == 0.5, e - 1, e).astype(np.int64)


# ----------------------------------------------------------------------------- nibble packing

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., K] codes -> [..., K/2] bytes; element 2i in the low nibble, 2i+1 in the high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("K must be even to pack two E2M1 codes per byte")
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes (inverse of pack_nibbles)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# ----------------------------------------------------------------------------- quantisers

def quantise_mxfp4(w: np.ndarray):
    """MXFP4 with one E8M0 scale per 32 along the last axis K.

    Per group (the last group holds K mod 32 elements when K is not a multiple
    of 32): amax over the present elements; the scale is the power-of-two
    ceiling 2^ceil(log2(amax/6)), exponent clamped to [-127, 127], stored as
    byte e+127; codes are E2M1 round-to-nearest-even of w / scale. A group whose
    amax is 0 stores byte 0 and all-zero codes (no division by zero).
    Returns (packed nibbles [..., K/2], scale bytes [..., ceil(K/32)]).
    """
    w = np.asarray(w, dtype=np.float64)
    k = w.shape[-1]
    ng = -(-k // 32)
    codes = np.zeros(w.shape, dtype=np.uint8)
    scales = np.zeros(w.shape[:-1] + (ng,), dtype=np.uint8)
    for gi in range(ng):
        blk = w[..., gi * 32:(gi + 1) * 32]
        amax = np.max(np.abs(blk), axis=-1)
        nz = amax > 0
        e = np.zeros(amax.shape, dtype=np.int64)
        e[nz] = np.clip(ceil_log2(amax[nz] / E2M1_MAX), -127, 127)
        scales[..., gi] = np.where(nz, e + 127, 0).astype(np.uint8)
        q = e2m1_encode(blk * np.ldexp(1.0, -e)[..., None])
        codes[..., gi * 32:(gi + 1) * 32] = np.where(nz[..., None], q, 0)
    return pack_nibbles(codes), scales


def quantise_mxfp8(a: np.ndarray):
    """MXFP8 (E4M3 elements, one E8M0 scale per 32 along the last axis K).

    The W4A8 variant quantises the activation output between FC1 and FC2 this way
    (PR 4255 review: the grouped MXFP8 quantisation of the SiLU-mul output). Per
    group (the last one holds K mod 32 elements when K is not a multiple of 32):
    amax over the present elements; scale 2^ceil(log2(amax/448)) (the power-of-two
    ceiling used for the MX weight scales), exponent clamped to [-127, 127], stored
    as byte e+127; codes are E4M3 round-to-nearest-even of a / scale, so the largest
    element lands in (224, 448] and nothing saturates. A group whose amax is 0
    stores byte 0 and zero codes. Returns (codes uint8 [..., K], scales uint8
    [..., ceil(K/32)]).
    """
    a = np.asarray(a, dtype=np.float64)
    k = a.shape[-1]
    ng = -(-k // 32)
    codes = np.zeros(a.shape, dtype=np.uint8)
    scales = np.zeros(a.shape[:-1] + (ng,), dtype=np.uint8)
    for gi in range(ng):
        blk = a[..., gi * 32:(gi + 1) * 32]
        amax = np.max(np.abs(blk), axis=-1)
        nz = amax > 0
        e = np.zeros(amax.shape, dtype=np.int64)
        e[nz] = np.clip(ceil_log2(amax[nz] / E4M3_MAX), -127, 127)
        scales[..., gi] = np.where(nz, e + 127, 0).astype(np.uint8)
        q = e4m3_encode(blk * np.ldexp(1.0, -e)[..., None])
        codes[..., gi * 32:(gi + 1) * 32] = np.where(nz[..., None], q, 0)
    return codes, scales


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """a_hat[..., k] = e4m3(code) * 2^(scale[k // 32] - 127), float64."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    k = codes.shape[-1]
    s = np.repeat(E8M0_TABLE[scales], 32, axis=-1)[..., :k]
    return E4M3_TABLE[codes] * s


def quantise_nvfp4(w: np.ndarray):
    """NVFP4 for [E, N, K] weights: E4M3 scale per 16 along K and one fp32 global scale per expert.

    Two-level recipe: g = fp32(amax_e / (448*6)) is the stored dequant multiplier
    of expert e (g = 1 and all codes 0 when the expert's weights are all zero);
    each 16-group's scale byte is E4M3-RNE(amax_group / 6 / g); codes are
    E2M1-RNE(w / (decode(scale) * g)), and 0 when the decoded scale is 0.
    Returns (packed [E, N, K/2], scales [E, N, ceil(K/16)], g float32 [E]).
    """
    w = np.asarray(w, dtype=np.float64)
    ne, n, k = w.shape
    ng = -(-k // 16)
    codes = np.zeros(w.shape, dtype=np.uint8)
    scales = np.zeros((ne, n, ng), dtype=np.uint8)
    gvec = np.ones(ne, dtype=np.float32)
    for e in range(ne):
        amax_t = float(np.max(np.abs(w[e]))) if w[e].size else 0.0
        if amax_t == 0.0:
            continue
        g = np.float32(amax_t / (E4M3_MAX * E2M1_MAX))
        gvec[e] = g
        g = float(g)
        for gi in range(ng):
            blk = w[e, :, gi * 16:(gi + 1) * 16]
            amax_b = np.max(np.abs(blk), axis=-1)
            sb = e4m3_encode(amax_b / E2M1_MAX / g)
            scales[e, :, gi] = sb
            sv = E4M3_TABLE[sb]
            safe = np.where(sv > 0, sv * g, 1.0)
            q = e2m1_encode(blk / safe[:, None])
            codes[e, :, gi * 16:(gi + 1) * 16] = np.where((sv > 0)[:, None], q, 0)
    return pack_nibbles(codes), scales, gvec


# ----------------------------------------------------------------------------- dequantisers

def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """w_hat[..., k] = e2m1(code) * 2^(scale[k // 32] - 127), float64."""
    codes = unpack_nibbles(packed)
    k = codes.shape[-1]
    s = E8M0_TABLE[np.asarray(scales, dtype=np.uint8)]
    s_full = np.repeat(s, 32, axis=-1)[..., :k]
    return E2M1_TABLE[codes] * s_full


def dequant_nvfp4(packed: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """w_hat[e, n, k] = e2m1(code) * e4m3(scale[e, n, k // 16]) * g[e], float64."""
    codes = unpack_nibbles(packed)
    k = codes.shape[-1]
    s = E4M3_TABLE[np.asarray(scales, dtype=np.uint8)]
    s_full = np.repeat(s, 16, axis=-1)[..., :k]
    g = np.asarray(g, dtype=np.float64).reshape((-1,) + (1,) * (codes.ndim - 1))
    return E2M1_TABLE[codes] * s_full * g


def dequant(fmt: str, packed, scales, g=None) -> np.ndarray:
    if fmt == "mxfp4":
        return dequant_mxfp4(packed, scales)
    if fmt == "nvfp4":
        return dequant_nvfp4(packed, scales, g)
    raise ValueError(f"unknown format {fmt!r}")


# ----------------------------------------------------------------------------- bfloat16

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(x) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits, nearest, ties to even).

    Subnormals use the fixed quantum 2^-133; results above the largest finite
    bfloat16 become +-inf. Returned as float64.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(xf, -q)), q)
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64 by their sign / exponent / mantissa fields."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    mt = (b & 0x7F).astype(np.float64)
    val = np.where(e == 0, mt / 128.0 * 2.0 ** -126, (1.0 + mt / 128.0) * np.ldexp(1.0, (e - 127).clip(-200, 200)))
    val = np.where((e == 0xFF) & (mt == 0), np.inf, val)
    val = np.where((e == 0xFF) & (mt != 0), np.nan, val)
    return s * val
