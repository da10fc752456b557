"""Pins for the oracle's adapter merge, W_merged = bf16(W' + s B A).

The pages give the merge as a formula only (W_merged = W0 + B A, with the
dequantize-to-BF16-then-add recipe), so the oracle is pinned by:
  * its rounding step against an independent exact-rational brute force;
  * the B = 0 and s = 0 cases, where the merged weight is W' bit for bit;
  * the merge identity: a plain layer with the merged weight gives the
    adapted forward h = x W'^T + s (x A^T) B^T up to the bf16 rounding of
    the weight.
"""

from fractions import Fraction

import numpy as np

from oracle import qlora_oracle as O
import qlora_inputs as QI


def exact_bf16_value(bits: int) -> Fraction:
    """Value of a bf16 pattern as an exact rational (finite, any exponent)."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    mant = bits & 0x7F
    if e == 0:
        mag = Fraction(mant, 1 << 7) * Fraction(1, 1 << 126)
    else:
        mag = (1 + Fraction(mant, 1 << 7)) * (Fraction(2) ** (e - 127))
    return sign * mag


def brute_round_bf16(v: Fraction) -> int:
    """Nearest bf16 pattern to the rational v, ties to the even pattern,
    found by comparing exact distances to the patterns around float(v)."""
    approx = np.float32(float(v)).view(np.uint32) >> 16
    best = None
    for cand in range(int(approx) - 2, int(approx) + 3):
        if cand < 0 or cand > 0xFFFF or ((cand >> 7) & 0xFF) == 0xFF:
            continue
        d = abs(exact_bf16_value(cand) - v)
        key = (d, cand & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    if v == 0:
        return 0
    return best[1]


def test_f64_rounding_matches_fp32_rounding_on_fp32_values():
    x = np.random.default_rng(5).standard_normal(50000).astype(np.float32)
    assert np.array_equal(O.bf16_bits_rne_f64(x.astype(np.float64)), O.bf16_bits_rne(x))


def test_f64_rounding_ties_and_single_rounding():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even pattern 0x3f80;
    # 1 + 3 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even 0x3f82
    assert O.bf16_bits_rne_f64(1 + 2.0 ** -8) == 0x3F80
    assert O.bf16_bits_rne_f64(1 + 3 * 2.0 ** -8) == 0x3F82
    assert O.bf16_bits_rne_f64(-(1 + 3 * 2.0 ** -8)) == 0xBF82
    # just above a tie: one rounding goes up; rounding to fp32 first would
    # land on the tie and go down to even
    assert O.bf16_bits_rne_f64(1 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert O.bf16_bits_rne_f64(-0.0) == 0x8000


def test_merge_matches_exact_rational_brute_force():
    rng = np.random.default_rng(11)
    m, n, r, s = 3, 64, 2, 1.5
    Wd_bits = O.bf16_bits_rne(rng.standard_normal(m * n).astype(np.float32) * 0.02)
    A_bits = O.bf16_bits_rne(rng.standard_normal((r, n)).astype(np.float32) * 0.1)
    B_bits = O.bf16_bits_rne(rng.standard_normal((m, r)).astype(np.float32) * 0.1)
    got = O.merge_adapter(Wd_bits, A_bits, B_bits, s, m, n)
    for f in range(m):
        for k in range(n):
            v = exact_bf16_value(int(Wd_bits[f * n + k]))
            for q in range(r):
                v += Fraction(s) * exact_bf16_value(int(B_bits[f, q])) * exact_bf16_value(int(A_bits[q, k]))
            assert int(got[f, k]) == brute_round_bf16(v), (f, k)


def test_merge_with_zero_adapter_is_the_dequantized_weight():
    inp = QI.custom_inputs(seed=21, M=4, n=128, m=40, r=8)
    qw = O.quantize_nf4_dq(inp["W"])
    Wd_bits = O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], 40 * 128)
    zeros_B = np.zeros_like(inp["B"])
    assert np.array_equal(O.merge_adapter(Wd_bits, inp["A"], zeros_B, 2.0, 40, 128).reshape(-1), Wd_bits)
    assert np.array_equal(O.merge_adapter(Wd_bits, inp["A"], inp["B"], 0.0, 40, 128).reshape(-1), Wd_bits)


def test_merge_identity_against_the_adapted_forward():
    # a plain layer with the merged weight reproduces the adapted forward up
    # to the weight's bf16 rounding (relative 2^-9 per element)
    M, n, m, r, s = 16, 256, 96, 16, 2.0
    inp = QI.custom_inputs(seed=33, M=M, n=n, m=m, r=r)
    qw = O.quantize_nf4_dq(inp["W"])
    Wd_bits = O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], m * n)
    Wd = O.bf16_bits_to_float64(Wd_bits).reshape(m, n)
    x = O.bf16_bits_to_float64(inp["x"])
    A = O.bf16_bits_to_float64(inp["A"])
    B = O.bf16_bits_to_float64(inp["B"])
    h, _ = O.linear_fwd(x, Wd, A, B, s)
    Wm = O.bf16_bits_to_float64(O.merge_adapter(Wd_bits, inp["A"], inp["B"], s, m, n))
    hm = x @ Wm.T
    rel = np.linalg.norm(hm - h) / np.linalg.norm(h)
    assert rel < 2.0 ** -8, rel
    # a merge that dropped s, or used A B^T's transpose pattern, misses by far more
    adapter = s * (B @ A)
    assert np.linalg.norm(x @ (Wd + adapter / s).T - h) / np.linalg.norm(h) > 10 * rel
