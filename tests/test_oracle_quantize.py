"""Pins for the oracle's quantizer and dequantizer.

Checked against: brute-force nearest-level search, constructed inputs that
land exactly on and one ulp around every threshold, invariants the method
fixes (the absmax element maps to +-1, the largest block of a group decodes
to c2 exactly), the storage arithmetic printed on the pages, and the pages'
claim that NF4 beats uniform INT4 on normal weights.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import qlora_oracle as O
import qlora_inputs as QI


def brute_nearest_codes(w, Q=None):
    """argmin_j |w/c1 - Q_j| in float64 per element, ties to the lower code."""
    wb = np.asarray(w, dtype=np.float32).reshape(-1, 64)
    c1 = np.max(np.abs(wb), axis=1)
    out = np.empty(wb.shape, dtype=np.int64)
    Q = (O.NF4_Q if Q is None else Q).astype(np.float64)
    for b in range(wb.shape[0]):
        for e in range(64):
            what = 0.0 if c1[b] == 0 else float(np.float32(wb[b, e]) / np.float32(c1[b]))
            d = np.abs(what - Q)
            out[b, e] = int(np.argmin(d))          # argmin returns the first (lower) on ties
    return out.reshape(-1)


def test_threshold_rule_equals_nearest_level():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    qw = O.quantize_nf4_dq(W)
    got = O.unpack_codes(qw["codes"], W.size).astype(np.int64)
    want = brute_nearest_codes(W)
    diff = np.nonzero(got != want)[0]
    # a disagreement is only possible within one fp32 ulp of a threshold
    wb = W.reshape(-1)
    c1 = np.repeat(qw["c1"], 64)
    for i in diff:
        what = np.float32(wb[i]) / np.float32(c1[i])
        assert np.min(np.abs(O.NF4_T.astype(np.float64) - float(what))) <= float(np.spacing(np.float32(what)))
    assert len(diff) <= 2


def test_threshold_boundaries_exact():
    # c1 = 1 (one element of the block is 1.0), so w_hat = w exactly.
    T = O.NF4_T
    vals = []
    for t in T:
        vals += [t, np.nextafter(t, np.float32(-2)), np.nextafter(t, np.float32(2))]
    vals = np.array(vals, dtype=np.float32)
    blocks = []
    for i in range(0, len(vals), 63):
        chunk = list(vals[i:i + 63])
        chunk += [0.5] * (63 - len(chunk))
        blocks.append(np.array([1.0] + chunk, dtype=np.float32))
    W = np.concatenate(blocks)
    qw = O.quantize_nf4_dq(W)
    codes = O.unpack_codes(qw["codes"], W.size).reshape(-1, 64)[:, 1:].reshape(-1)[:len(vals)]
    for j in range(15):
        at, below, above = codes[3 * j], codes[3 * j + 1], codes[3 * j + 2]
        assert at == j            # equal to the threshold: not above it, lower code
        assert below == j
        assert above == j + 1


def test_zero_weights_and_zero_blocks():
    W = np.zeros(128, dtype=np.float32)
    W[64:] = np.linspace(-1, 1, 64, dtype=np.float32)
    W[70] = 0.0
    qw = O.quantize_nf4_dq(W)
    codes = O.unpack_codes(qw["codes"], 128)
    assert np.all(codes[:64] == 7)                 # all-zero block: normalized weight 0 -> code 7
    assert codes[70] == 7                          # exact zero weight: T_7 = 0 is not exceeded
    assert qw["absmax8"][0] == 0                   # c1 = 0 encodes to 0
    deq = O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], 128)
    assert np.all(deq[:64] == 0x8000)              # bf16(-0.042 * 0) = -0.0


def test_all_zero_weight_matrix():
    qw = O.quantize_nf4_dq(np.zeros((4, 64 * 8), dtype=np.float32))
    assert np.all(qw["c2"] == 0) and np.all(qw["absmax8"] == 0)
    assert np.all(O.unpack_codes(qw["codes"], 4 * 512) == 7)


def test_absmax_element_maps_to_extreme_code():
    rng = np.random.default_rng(9)
    W = (rng.standard_normal(64 * 300) * 0.02).astype(np.float32)
    qw = O.quantize_nf4_dq(W)
    codes = O.unpack_codes(qw["codes"], W.size).reshape(-1, 64)
    wb = W.reshape(-1, 64)
    for b in range(wb.shape[0]):
        k = int(np.argmax(np.abs(wb[b])))
        assert codes[b, k] == (15 if wb[b, k] > 0 else 0)


def test_group_max_block_decodes_to_c2_exactly():
    rng = np.random.default_rng(10)
    W = (rng.standard_normal(16384 * 3 + 64 * 5) * 0.02).astype(np.float32)   # partial last group
    qw = O.quantize_nf4_dq(W)
    nblk = W.size // 64
    assert len(qw["c2"]) == 4 and len(qw["absmax8"]) == nblk
    for g in range(4):
        a = qw["absmax8"][g * 256:(g + 1) * 256]
        c1 = qw["c1"][g * 256:(g + 1) * 256]
        assert qw["c2"][g] == np.max(c1)
        assert 0x38 in a.tolist()                        # fl(c1/c1) = 1 -> 0x38
        k = int(np.argmax(c1))
        s = O.block_scales(qw["absmax8"], qw["c2"], nblk)[g * 256 + k]
        assert s == qw["c2"][g]                          # 1.0 * c2 exactly


def test_reconstruction_is_code_times_scale():
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((8, 2048)) * 0.02).astype(np.float32)
    qw = O.quantize_nf4_dq(W)
    deq = O.bf16_bits_to_float64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], W.size))
    codes = O.unpack_codes(qw["codes"], W.size)
    s = np.repeat(O.block_scales(qw["absmax8"], qw["c2"], W.size // 64), 64).astype(np.float64)
    exact = O.NF4_Q[codes].astype(np.float64) * s
    # bf16 keeps 8 significant bits; two roundings (fp32 product, then bf16)
    assert np.all(np.abs(deq - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-30)
    # the dequantized absmax element of every block is +-s_b to bf16 precision
    db = deq.reshape(-1, 64)
    sb = O.block_scales(qw["absmax8"], qw["c2"], W.size // 64).astype(np.float64)
    assert np.allclose(np.max(np.abs(db), axis=1), sb, rtol=2.0 ** -8)


def test_dequant_of_row_slices_matches_whole():
    rng = np.random.default_rng(13)
    m, n = 6, 16384 // 2 + 64 * 3      # rows straddle c2 groups
    W = (rng.standard_normal((m, n)) * 0.02).astype(np.float32)
    qw = O.quantize_nf4_dq(W)
    full = O.bf16_bits_to_float64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], W.size)).reshape(m, n)
    rows = [5, 0, 3]
    assert np.array_equal(O.dequant_rows(qw, m, n, rows), full[rows])


def test_quantization_error_nf4_below_int4():
    # NF4 targets normally distributed weights and beats uniform INT4 there
    rng = np.random.default_rng(14)
    W = (rng.standard_normal((256, 1024)) * 0.02).astype(np.float32)
    qw = O.quantize_nf4_dq(W)
    deq = O.bf16_bits_to_float64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], W.size))
    w64 = W.reshape(-1).astype(np.float64)
    rel = lambda a: np.linalg.norm(a - w64) / np.linalg.norm(w64)
    e_nf4 = rel(deq)
    e_int4 = rel(O.int4_absmax_roundtrip(W))
    assert e_nf4 < e_int4
    assert 0.07 < e_nf4 < 0.12 and 0.09 < e_int4 < 0.13


def test_sliced_quantization_equals_whole():
    # groups are independent: quantizing one 16384-element group alone gives its slice
    rng = np.random.default_rng(15)
    W = (rng.standard_normal(16384 * 3) * 0.02).astype(np.float32)
    qw = O.quantize_nf4_dq(W)
    part = O.quantize_nf4_dq(W[16384:32768])
    assert np.array_equal(part["codes"], qw["codes"][8192:16384])
    assert np.array_equal(part["absmax8"], qw["absmax8"][256:512])
    assert part["c2"][0] == qw["c2"][1]


# ---------------- storage arithmetic against the pages' printed numbers -------

@pytest.fixture(scope="module")
def pages(golden_dir):
    with open(os.path.join(golden_dir, "pages_worked_examples.json")) as f:
        return json.load(f)


def test_constant_overhead(pages):
    no_dq = O.constant_overhead_bits(False)
    dq = O.constant_overhead_bits(True)
    assert no_dq == pages["scale_overhead_bits_without_dq"]["value"]
    assert round(dq, 3) == pages["scale_overhead_bits_with_dq"]["value"]
    assert round(no_dq - dq, 2) == pages["scale_overhead_saving_bits"]["value"]
    assert abs((no_dq - dq) - pages["scale_overhead_saving_fraction_of_bit"]["value"]) < 0.05
    saving_gb = pages["saving_65b_gb"]["params"] * (no_dq - dq) / 8 / 1e9
    assert round(saving_gb) == pages["saving_65b_gb"]["value"]


def test_storage_bytes_exact():
    for m, n in [(256, 256), (14336, 4096), (4096, 14336), (1024, 4096), (28672, 8192)]:
        numel = m * n
        b = O.storage_bytes(numel)
        assert b == numel // 2 + numel // 64 + 4 * math.ceil(numel / 16384)
        assert b * 8 / numel == 4.0 + O.constant_overhead_bits(True) == 4.126953125


def test_worked_example_8b_and_70b(pages):
    bits = 4.0 + O.constant_overhead_bits(True)
    assert round(bits, 3) == pages["nf4_dq_bits_per_param"]["value"]
    p8 = pages["llama31_8b_params"]["value"]
    assert round(p8 * bits / 8 / 1e9, 2) == pages["llama31_8b_base_gb"]["value"]
    assert round(p8 * 2 / 1e9, 2) == pages["llama31_8b_bf16_gb"]["value"]
    assert round(p8 * 16 / 1e9, 1) == pages["llama31_8b_full_ft_gb"]["value"]
    p70 = pages["llama_70b_params"]["value"]
    assert round(p70 * bits / 8 / 1e9, 1) == pages["llama_70b_base_gb"]["value"]
    assert round(pages["bf16_7b_weights_gb"]["params"] * 2 / 1e9) == pages["bf16_7b_weights_gb"]["value"]


def test_adapter_counts_pin_the_8b_block_shapes(pages):
    layers = QI.WORKLOADS[4]["layers"]
    per_block = sum(O.adapter_params(L.m, L.n, 16) for L in layers)
    assert per_block == pages["llama31_8b_adapter_params_per_block_r16"]["value"]
    total = per_block * pages["llama31_8b_adapter_params_total_r16"]["layers"]
    assert round(total / 1e6, 1) == pages["llama31_8b_adapter_params_total_r16"]["value"] / 1e6
    assert round(total * 16 / 1e9, 2) == pages["llama31_8b_adapter_state_gb"]["value"]
    ex = pages["lora_4096_r8_params"]
    assert O.adapter_params(ex["m"], ex["n"], ex["r"]) == ex["value"]


def test_eq4_ratio(pages):
    ex = pages["eq4_ratio_r16_4096"]
    exact = O.adapter_params(ex["m"], ex["n"], ex["r"]) / (ex["m"] * ex["n"])
    approx = ex["r"] / min(ex["m"], ex["n"])
    assert approx * 100 < ex["printed_bound_percent"]      # the printed approximation
    assert abs(exact - 2 * approx) < 1e-15                 # square layers: exactly twice that


def test_dequant_cols_matches_whole():
    rng = np.random.default_rng(16)
    m, n = 40, 16384 // 4 + 64
    W = (rng.standard_normal((m, n)) * 0.02).astype(np.float32)
    qw = O.quantize_nf4_dq(W)
    full = O.bf16_bits_to_float64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], W.size)).reshape(m, n)
    cols = [0, 1, 63, 64, 4095, n - 1, 777]
    assert np.array_equal(O.dequant_cols(qw, m, n, cols), full[:, cols])


def test_code_encoding_is_sign_and_magnitude():
    # every stored code denotes its level: sign in bit 3, magnitude rank in bits 0-2
    L = np.arange(16)
    c = O.level_to_code(L)
    assert sorted(c.tolist()) == list(range(16))                 # a bijection
    assert np.array_equal(O.code_to_level(c), L)
    for lev, code in zip(L, c):
        mag = O.NF4_Q[8 + (code & 7)]
        val = O.NF4_Q[lev]
        assert (code >> 3) == (1 if val < 0 else 0)
        assert float(abs(val)) == float(mag)


def test_packing_order_and_roundtrip():
    rng = np.random.default_rng(17)
    lev = rng.integers(0, 16, size=64 * 5).astype(np.uint8)
    packed = O.pack_levels(lev)
    assert packed.size == lev.size // 2
    assert np.array_equal(O.unpack_codes(packed, lev.size), lev)
    # byte j of each 8-weight group: weight j low nibble, weight j + 4 high nibble
    codes = O.level_to_code(lev)
    for g in range(lev.size // 8):
        for j in range(4):
            b = int(packed[4 * g + j])
            assert b & 0xF == codes[8 * g + j] and b >> 4 == codes[8 * g + j + 4]


# ------------------------------------------------------------ uniform 4-bit grid

def test_uniform4_table_closed_form():
    Q, T = O.uniform4_table()
    for j in range(16):
        assert Q[j] == np.float32((2 * j - 15) / 15.0)
        assert Q[15 - j] == -Q[j]
    assert np.all(np.diff(Q.astype(np.float64)) > 0)
    assert T[7] == 0.0
    for j in range(15):
        assert T[j] == np.float32((float(Q[j]) + float(Q[j + 1])) / 2.0)
    # the spacing is uniform to fp32 rounding
    assert np.allclose(np.diff(Q.astype(np.float64)), 2.0 / 15.0, rtol=0, atol=1e-7)


def test_uniform4_threshold_rule_equals_nearest_level():
    rng = np.random.default_rng(6)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    qw = O.quantize_nf4_dq(W, table=O.uniform4_table())
    got = O.unpack_codes(qw["codes"], W.size).astype(np.int64)
    want = brute_nearest_codes(W, O.UNIFORM4_Q)
    diff = np.nonzero(got != want)[0]
    wb = W.reshape(-1)
    c1 = np.repeat(qw["c1"], 64)
    for i in diff:
        what = np.float32(wb[i]) / np.float32(c1[i])
        assert np.min(np.abs(O.UNIFORM4_T.astype(np.float64) - float(what))) <= float(np.spacing(np.float32(what)))
    assert len(diff) <= 2


def test_uniform4_error_above_nf4_and_near_int4():
    # the uniform grid through the same pipeline (double quant, bf16) loses to
    # NF4 on normal weights, and lands near the 15-level INT4 absmax round trip
    rng = np.random.default_rng(15)
    W = (rng.standard_normal((256, 1024)) * 0.02).astype(np.float32)
    w64 = W.reshape(-1).astype(np.float64)
    rel = lambda a: np.linalg.norm(a - w64) / np.linalg.norm(w64)  # noqa: E731
    errs = {}
    for name, table in (("nf4", None), ("uniform4", O.uniform4_table())):
        qw = O.quantize_nf4_dq(W, table=table)
        deq = O.bf16_bits_to_float64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], W.size, table=table))
        errs[name] = rel(deq)
    assert errs["nf4"] < errs["uniform4"]
    e_int4 = rel(O.int4_absmax_roundtrip(W))
    assert abs(errs["uniform4"] - e_int4) < 0.25 * e_int4


# ------------------------------------------------------ INT4 absmax as a level table

def test_int4_table_closed_form():
    Q, T = O.int4_table()
    for k in range(8):
        assert Q[8 + k] == np.float32(k / 7.0)
        assert Q[7 - k].view(np.uint32) == (-Q[8 + k]).view(np.uint32)   # bitwise, -0.0 included
    assert Q[7] == 0.0 and np.signbit(Q[7]) and not np.signbit(Q[8])
    assert np.all(np.diff(Q.astype(np.float64)) >= 0) and np.count_nonzero(np.diff(Q.astype(np.float64)) == 0) == 1
    assert T[7] == 0.0
    for j in range(15):
        assert T[j] == np.float32((float(Q[j]) + float(Q[j + 1])) / 2.0)
    for k in range(7):   # thresholds (2k + 1)/14 up to the two roundings (levels, then midpoint)
        assert abs(float(T[8 + k]) - (2 * k + 1) / 14.0) <= 2.0 * float(np.spacing(T[8 + k]))


def _int4_values(qw, n):
    lev = O.unpack_codes(qw["codes"], n).astype(np.int64)   # level index 0..15
    return O.INT4_Q.astype(np.float64)[lev]


def test_int4_table_is_the_integer_absmax_quantizer():
    # the threshold rule on the INT4 table picks k/7 with k = rint(7 w_hat),
    # the textbook integer quantizer, except within one ulp of a threshold
    rng = np.random.default_rng(21)
    W = (rng.standard_normal((96, 512)) * 0.02).astype(np.float32)
    W[3, :64] = 0.0                                    # an all-zero block: w_hat = 0 -> the zero level
    qw = O.quantize_nf4_dq(W, table=O.int4_table())
    got = np.rint(_int4_values(qw, W.size) * 7.0)          # fl32(k/7) * 7 rounds back to k
    wb = W.reshape(-1, 64)
    c1 = np.max(np.abs(wb), axis=1)
    what = np.where(c1[:, None] > 0, wb / np.where(c1 > 0, c1, 1)[:, None], 0).astype(np.float32).reshape(-1)
    k = np.rint(what.astype(np.float64) * 7.0)
    diff = np.nonzero(got != k)[0]
    for i in diff:
        assert np.min(np.abs(O.INT4_T.astype(np.float64) - float(what[i]))) <= float(np.spacing(what[i]))
    assert len(diff) <= 4
    assert np.all(got[3 * 512:3 * 512 + 64] == 0.0)


def test_int4_threshold_rule_equals_nearest_value():
    # nearest level by brute force: the two zeros are one value, so compare
    # values, not indices
    rng = np.random.default_rng(22)
    W = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    qw = O.quantize_nf4_dq(W, table=O.int4_table())
    got = _int4_values(qw, W.size)
    want = O.INT4_Q.astype(np.float64)[brute_nearest_codes(W, O.INT4_Q)]
    diff = np.nonzero(got != want)[0]
    wb = W.reshape(-1)
    c1 = np.repeat(qw["c1"], 64)
    for i in diff:
        what = np.float32(wb[i]) / np.float32(c1[i])
        assert np.min(np.abs(O.INT4_T.astype(np.float64) - float(what))) <= float(np.spacing(np.float32(what)))
    assert len(diff) <= 2


def test_int4_table_error_above_nf4_and_at_int4_roundtrip():
    # through the same pipeline (double quant, bf16) INT4 loses to NF4 on
    # normal weights, and sits at the exact-scale INT4 round trip
    rng = np.random.default_rng(23)
    W = (rng.standard_normal((256, 1024)) * 0.02).astype(np.float32)
    w64 = W.reshape(-1).astype(np.float64)
    rel = lambda a: np.linalg.norm(a - w64) / np.linalg.norm(w64)  # noqa: E731
    errs = {}
    for name, table in (("nf4", None), ("int4", O.int4_table())):
        qw = O.quantize_nf4_dq(W, table=table)
        deq = O.bf16_bits_to_float64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], W.size, table=table))
        errs[name] = rel(deq)
    assert errs["nf4"] < errs["int4"]
    e_exact = rel(O.int4_absmax_roundtrip(W))
    assert abs(errs["int4"] - e_exact) < 0.05 * e_exact


# ------------------------------------------------- edge-mean (quantile-average) table

def _phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def test_edge_mean_table_shape():
    Q, T = O.edge_mean_table()
    assert Q[15] == 1.0 and Q[0] == -1.0
    for j in range(16):
        assert Q[15 - j] == -Q[j]
    assert np.all(np.diff(Q.astype(np.float64)) > 0)
    assert T[7] == 0.0
    for j in range(15):
        assert T[j] == np.float32((float(Q[j]) + float(Q[j + 1])) / 2.0)


def test_edge_mean_levels_sit_in_their_buckets():
    # level i lies strictly inside its equal-probability bucket (the outer
    # buckets cut at their midpoints), checked through the normal CDF itself
    q = O.edge_mean_levels(4)
    edges = [i / 16 for i in range(17)]
    edges[0], edges[16] = 1 / 32, 31 / 32
    for i in range(16):
        assert edges[i] < _phi(float(q[i])) < edges[i + 1], i


def test_edge_mean_levels_exceed_bucket_midpoint_quantiles():
    # the mean of the two edge quantiles of an inner bucket above 1/2 exceeds
    # the quantile of the bucket's mid probability (the quantile function is
    # strictly convex there), and mirrors below 1/2; an implementation that
    # took the midpoint's quantile (the Eq. 2 level) would tie
    q = O.edge_mean_levels(4)
    p1 = O.nf4_levels(4)
    for i in range(8, 15):
        assert q[i] > p1[i] + 1e-6, i
        assert q[15 - i] < p1[15 - i] - 1e-6, i


def test_edge_mean_threshold_rule_equals_nearest_level():
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    table = O.edge_mean_table()
    qw = O.quantize_nf4_dq(W, table=table)
    got = O.unpack_codes(qw["codes"], W.size).astype(np.int64)
    want = brute_nearest_codes(W, O.EDGE_MEAN_Q)
    diff = np.nonzero(got != want)[0]
    wb = W.reshape(-1)
    c1 = np.repeat(qw["c1"], 64)
    for i in diff:
        what = np.float32(wb[i]) / np.float32(c1[i])
        assert np.min(np.abs(O.EDGE_MEAN_T.astype(np.float64) - float(what))) <= float(np.spacing(np.float32(what)))
    assert len(diff) <= 2


def test_edge_mean_error_close_to_nf4_below_uniform():
    rng = np.random.default_rng(15)
    W = (rng.standard_normal((256, 1024)) * 0.02).astype(np.float32)
    w64 = W.reshape(-1).astype(np.float64)
    rel = lambda a: np.linalg.norm(a - w64) / np.linalg.norm(w64)  # noqa: E731
    errs = {}
    for name, table in (("nf4", None), ("uniform4", O.uniform4_table()), ("edge", O.edge_mean_table())):
        qw = O.quantize_nf4_dq(W, table=table)
        deq = O.bf16_bits_to_float64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], W.size, table=table))
        errs[name] = rel(deq)
    assert errs["edge"] < errs["uniform4"]
    assert abs(errs["edge"] - errs["nf4"]) < 0.05 * errs["nf4"]
