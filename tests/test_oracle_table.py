"""Pins for the oracle's NF4 table, 8-bit float codec and bf16 rounding.

Nothing here re-uses the oracle's own routine for the value it checks: the
levels are checked through the normal CDF (math.erfc) and a second quantile
routine (scipy), the E4M3 encoder against a bit-manipulation encoder written
here, and bf16 rounding against torch's cast.
"""

import math
import struct

import numpy as np
import pytest
import torch
from scipy.special import ndtri

from oracle import qlora_oracle as O


def phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


# ---------------- NF4 levels: QLoRA: Efficient Fine-Tuning, Step 1, Eq. 2 ----

def test_levels_sit_at_bucket_midpoints_of_probability():
    q = O.nf4_levels(4)
    assert len(q) == 16
    for i, qi in enumerate(q, start=1):
        assert abs(phi(qi) - (i - 0.5) / 16) < 1e-15


def test_each_level_inside_its_equal_probability_bucket():
    q = O.nf4_levels(4)
    for i, qi in enumerate(q, start=1):
        lo = -math.inf if i == 1 else ndtri((i - 1) / 16)
        hi = math.inf if i == 16 else ndtri(i / 16)
        assert lo < qi < hi
        # every bucket carries the same probability mass 1/16
        assert abs((phi(hi) if hi != math.inf else 1.0) - (phi(lo) if lo != -math.inf else 0.0) - 1 / 16) < 1e-14


def test_levels_agree_with_second_quantile_routine():
    q = O.nf4_levels(4)
    q2 = ndtri((np.arange(1, 17) - 0.5) / 16)
    assert np.max(np.abs(q - q2)) < 1e-13
    Q2 = (q2 / q2[-1]).astype(np.float32)
    assert np.array_equal(Q2.view(np.uint32), O.NF4_Q.view(np.uint32))


def test_normalized_table_shape():
    Q, T = O.NF4_Q, O.NF4_T
    assert Q.dtype == np.float32 and T.dtype == np.float32
    assert Q[0] == -1.0 and Q[15] == 1.0          # normalized weight range [-1, 1] (Eq. 1 text)
    assert np.all(np.diff(Q.astype(np.float64)) > 0)
    for j in range(16):                            # symmetric, bit for bit
        assert f32_bits(Q[15 - j]) == f32_bits(-Q[j])
    assert 0.0 not in Q.tolist()                   # Eq. 2 has no zero level
    for j in range(15):
        assert Q[j] < T[j] < Q[j + 1]
        exact_mid = (float(Q[j]) + float(Q[j + 1])) / 2
        assert abs(float(T[j]) - exact_mid) <= np.spacing(np.float32(abs(exact_mid))) / 2
    assert T[7] == 0.0
    for j in range(15):
        assert f32_bits(T[14 - j]) == f32_bits(-T[j]) or (T[j] == 0 and T[14 - j] == 0)


def test_levels_match_probit_scaled_by_largest_level():
    # independent closed form for the ratio: Phi(Q_j * q16) = (j + 1/2) / 16
    q16 = ndtri(31 / 32)
    for j, Qj in enumerate(O.NF4_Q):
        assert abs(phi(float(Qj) * q16) - (j + 0.5) / 16) < 1e-7


# ---------------- E4M3FN codec --------------------------------------------------

def e4m3_encode_bits(v: float) -> int:
    """Round-to-nearest-even E4M3FN encoder by mantissa rounding (v in [0, 448])."""
    if v == 0.0:
        return 0
    b = f32_bits(v)
    e = ((b >> 23) & 0xFF) - 127
    mant = b & 0x7FFFFF
    if e < -6:                                    # subnormal range: multiples of 2^-9
        scaled = v * 512.0                          # exact (power of two)
        k = math.floor(scaled)
        frac = scaled - k
        if frac > 0.5 or (frac == 0.5 and (k & 1)):
            k += 1
        return k                                    # k == 8 is the smallest normal, 0x08
    top = mant >> 20
    rest = mant & 0xFFFFF
    if rest > 0x80000 or (rest == 0x80000 and (top & 1)):
        top += 1
        if top == 8:
            top = 0
            e += 1
    return ((e + 7) << 3) | top


def test_e4m3_decode_known_values():
    assert O.e4m3_decode(0x38) == 1.0
    assert O.e4m3_decode(0x7E) == 448.0
    assert O.e4m3_decode(0x08) == 2.0 ** -6
    assert O.e4m3_decode(0x01) == 2.0 ** -9
    assert O.e4m3_decode(0x00) == 0.0
    assert np.isnan(O.e4m3_decode(0x7F))
    vals = O.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0)


def test_e4m3_roundtrip_every_finite_code():
    codes = np.arange(0x7F)
    assert np.array_equal(O.e4m3_encode_rne(O.e4m3_decode(codes)), codes.astype(np.uint8))


def test_e4m3_encoder_against_bit_encoder():
    rng = np.random.default_rng(7)
    vals = list(rng.random(20000, dtype=np.float32).astype(np.float64))
    vals += list((rng.random(5000, dtype=np.float32) * 2.0 ** -8).astype(np.float64))
    # every midpoint between adjacent codes, and one fp32 ulp either side
    grid = O.e4m3_decode(np.arange(0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    for mid in mids[mids <= 1.0]:
        m32 = np.float32(mid)
        assert float(m32) == mid                  # midpoints are exact in fp32
        vals += [mid, float(np.nextafter(m32, np.float32(0))), float(np.nextafter(m32, np.float32(2)))]
    vals = np.array(vals, dtype=np.float64)
    got = O.e4m3_encode_rne(vals)
    want = np.array([e4m3_encode_bits(v) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_error_bound_and_monotone():
    rng = np.random.default_rng(3)
    v = np.sort(rng.random(100000, dtype=np.float32).astype(np.float64))
    c = O.e4m3_encode_rne(v)
    assert np.all(np.diff(c.astype(np.int64)) >= 0)
    d = O.e4m3_decode(c)
    # half the code spacing at v: 2^(e-4) for normals, 2^-10 for subnormals
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    assert np.all(np.abs(d - v) <= 2.0 ** (e - 4) + 1e-300)


# ---------------- bf16 rounding -------------------------------------------------

def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=400000, dtype=np.uint64).astype(np.uint32)
    bits[::4] = (bits[::4] & 0xFFFF0000) | 0x8000        # exact ties
    bits[1::8] = bits[1::8] & 0x807FFFFF                  # subnormals
    bits = bits[(bits & 0x7F800000) != 0x7F800000]        # finite only
    bits = bits[(bits & 0x7FFFFFFF) < 0x7F7F8000]         # below the bf16 overflow point
    x = bits.view(np.float32)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits_rne(x), want)


def test_bf16_rne_sign_of_zero():
    z = np.array([0.0, -0.0], dtype=np.float32)
    assert O.bf16_bits_rne(z).tolist() == [0x0000, 0x8000]
