"""Plain CPU oracle for the QLoRA adapted-linear hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py`` and nowhere else.  It shares
no code, table or constant with the HIP library; the NF4 levels, the
thresholds and the 8-bit-float codebook are re-derived here from the pages'
definitions every time the module is imported.

Sources (the text of five web pages on QLoRA):
  [P1] "QLoRA: Efficient Fine-Tuning" (beta.fermi.ai wiki)
  [P2] "How QLoRA Fine-Tunes Large Models on Small GPUs: 4-bit Basics"
  [P3] "What is QLoRA?" (aquanode GPU glossary)
  [P4] "QLoRA & 4-bit Fine-Tuning" (prepfeed)
  [P5] "quantized low-rank adaptation (QLoRA)" (Real Python glossary)

What is computed, step by step (numpy; float64 unless a step fixes fp32):
  nf4_levels / nf4_table   [P1] Step 1, Eq. 2 (levels), Eq. 1 (range [-1, 1])
  block absmax c1          [P1] Step 1, Eq. 1 with alpha = 1; block of 64
                           weights from [P3] "The three pieces" and [P4]
                           Innovation 2
  encode                   [P1] Step 1, text under Eq. 1 ("snapped to the
                           nearest NF4 quantile level")
  double quantization      [P1] Step 2; [P4] Innovation 2 (c1 -> 8-bit float
                           with a second scale c2, blocks of 256)
  dequantization           [P1] Step 3 symbols (W0 dequantized to BF16 at
                           run time); [P3] "The three pieces"
  forward                  [P1] Step 3, Eq. 3 with the alpha/r scale of the
                           code snippet's LoraConfig comment
  backward                 [P1] Step 4, Eq. 5 (adapter gradients), and the
                           chain rule of the forward for grad_x
  adapter merge            [P1] Real-World Impact; [P4] Followups to expect
                           (W' + s B A rounded once to bf16)
  LoRA dropout             [P1] LoraConfig snippet (lora_dropout) on the
                           adapter input; mask from Philox4x32-10 (counter-
                           based, published definition)
  adapter optimizer step   [P1] memory-layout figure (Adam moments for the
                           adapters only); [P3] Worked example (fp32 state,
                           16 bytes per trainable parameter); Adam with
                           decoupled weight decay

Readings taken where the pages are silent or garbled (each is listed, with
its reason, in the design notes of the repository):
  * levels are divided by q_16 so the table spans exactly [-1, 1]
  * thresholds are fp32 midpoints of adjacent levels; ties go to the lower
    code (strict ">" count)
  * blocks are 64 consecutive elements of the row-major (out x in) weight
  * the 8-bit float is OCP E4M3FN, round to nearest, ties to even
  * c2 is the plain fp32 max of the 256 c1 values of its group
  * an all-zero block has c1 = 0, every normalized weight is 0 (level 7)
  * a level L (0..15, ascending) is stored as a 4-bit code with the sign in
    bit 3 and the magnitude rank in bits 0-2: code = L - 8 for L >= 8 and
    15 - L for L < 8; in every group of 8 consecutive weights, byte j of the
    group's 4 bytes holds weight j in its low nibble and weight j + 4 in its
    high nibble
  * s = alpha / r multiplies every adapter term, gradients included

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
closed forms, worked examples printed on the pages, brute force on small
inputs and automatic differentiation.  The values of h and of the gradients
for a given input are fixed by no printed example on the pages; they are
pinned by the identities (B = 0, W0 = 0, merge, autograd, finite
differences) only.
"""

from __future__ import annotations

import math
import statistics

import numpy as np

BLOCK = 64            # weights per first-level absmax block  ([P3], [P4])
DQ_BLOCKS = 256       # first-level constants per second-level group ([P1] Step 2)
GROUP = BLOCK * DQ_BLOCKS


# --------------------------------------------------------------------------
# NF4 code table  ([P1] Step 1, Eq. 2; range from the text under Eq. 1)
# --------------------------------------------------------------------------

def nf4_levels(k: int = 4) -> np.ndarray:
    """Unnormalized levels q_i = Phi^-1((i - 1/2) / 2^k), i = 1..2^k, float64.

    [P1] Step 1, Eq. 2.  Phi^-1 is the standard normal quantile function,
    evaluated with ``statistics.NormalDist.inv_cdf``.
    """
    nd = statistics.NormalDist(0.0, 1.0)
    n = 2 ** k
    return np.array([nd.inv_cdf((i - 0.5) / n) for i in range(1, n + 1)], dtype=np.float64)


def nf4_table():
    """Return (Q, T): 16 fp32 levels spanning [-1, 1] and 15 fp32 thresholds.

    Q_j = fl32(q_{j+1} / q_16): the normalized weight of Eq. 1 lies in
    [-1, 1] ([P1] Step 1), so the Eq. 2 levels are scaled by their largest
    value to span exactly that range.
    T_j = fl32((Q_j + Q_{j+1}) / 2): the midpoint between adjacent levels,
    formed exactly in float64 and rounded once; a weight is "snapped to the
    nearest" level ([P1] Step 1) by counting the thresholds below it.
    """
    q = nf4_levels(4)
    Q = (q / q[-1]).astype(np.float32)
    T = ((Q[:-1].astype(np.float64) + Q[1:].astype(np.float64)) / 2.0).astype(np.float32)
    return Q, T


NF4_Q, NF4_T = nf4_table()


def uniform4_table():
    """Return (Q, T) of the uniform 4-bit comparison grid: 16 evenly spaced
    levels spanning [-1, 1] with no zero level, Q_j = fl32((2j - 15) / 15),
    and the fp32 midpoints T_j as for NF4.

    [P1] Step 1 and [P4] Innovation 1 set NF4 against plain (uniform) 4-bit
    quantization; this grid is that baseline on the same block absmax
    normalization, symmetric like the NF4 table so that the same code layout
    and dequantization apply.
    """
    Q = np.array([(2 * j - 15) / 15.0 for j in range(16)], dtype=np.float64).astype(np.float32)
    T = ((Q[:-1].astype(np.float64) + Q[1:].astype(np.float64)) / 2.0).astype(np.float32)
    return Q, T


UNIFORM4_Q, UNIFORM4_T = uniform4_table()


def edge_mean_levels(k: int = 4) -> np.ndarray:
    """Unnormalized levels of the [P4] Innovation 1 construction, float64:
    level i (i = 0 .. 2^k - 1) is the mean of the normal quantiles at its
    bucket's edges i / 2^k and (i + 1) / 2^k.

    As printed the two outermost edges, probabilities 0 and 1, have infinite
    quantiles.  Reading taken here: those two edges move to the outer
    buckets' midpoints 1 / 2^(k+1) and 1 - 1 / 2^(k+1) (where [P1] Eq. 2
    puts its end levels); every inner edge stays.  The construction is
    symmetric about probability 1/2, so the upper half is computed and the
    lower half mirrored.
    """
    nd = statistics.NormalDist(0.0, 1.0)
    n = 2 ** k
    def edge(i):
        if i == n:
            return 1.0 - 0.5 / n
        return i / n
    upper = [0.5 * (nd.inv_cdf(edge(i)) + nd.inv_cdf(edge(i + 1))) for i in range(n // 2, n)]
    return np.array([-v for v in reversed(upper)] + upper, dtype=np.float64)


def edge_mean_table():
    """Return (Q, T) for edge_mean_levels: levels normalized by the largest
    to span [-1, 1], fp32 midpoints as for NF4."""
    q = edge_mean_levels(4)
    Q = (q / q[-1]).astype(np.float32)
    T = ((Q[:-1].astype(np.float64) + Q[1:].astype(np.float64)) / 2.0).astype(np.float32)
    return Q, T


EDGE_MEAN_Q, EDGE_MEAN_T = edge_mean_table()


# --------------------------------------------------------------------------
# The 8-bit float used for the double-quantized constants
# ([P1] Step 2 "8-bit floats"; [P1] figure "scales stored in FP8";
#  [P4] Innovation 2 "from FP32 down to FP8").  Reading: OCP E4M3FN.
# --------------------------------------------------------------------------

def e4m3_decode(code) -> np.ndarray:
    """Exact value of E4M3FN codes (bias 7, 3 mantissa bits, no infinities).

    Exponent field 0 is subnormal: m * 2^-9.  Otherwise 2^(e-7) * (1 + m/8).
    Codes 0x7F and 0xFF are NaN.
    """
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, 2.0 ** (e.astype(np.float64) - 7.0) * (1.0 + m / 8.0))
    mag = np.where((code & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


_E4M3_POS_CODES = np.arange(0, 0x7F, dtype=np.int64)        # 0x00 .. 0x7E, all finite
_E4M3_POS_VALUES = e4m3_decode(_E4M3_POS_CODES)              # strictly increasing


def e4m3_encode_rne(v) -> np.ndarray:
    """Nearest E4M3FN code to each non-negative finite v, ties to even code.

    Written as a plain search over the 127 finite non-negative codes: take
    the code whose exact value is nearest to v (in float64, which holds the
    fp32 input and every code value exactly); at an exact tie take the code
    with an even mantissa.  Values above 448 saturate to 448 (never reached
    on this path, where v <= 1).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode_rne expects finite non-negative values")
    vals = _E4M3_POS_VALUES
    hi = np.searchsorted(vals, v, side="left")             # vals[hi-1] < v <= vals[hi]
    hi = np.clip(hi, 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = np.abs(v - vals[lo])
    d_hi = np.abs(vals[hi] - v)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_E4M3_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _E4M3_POS_CODES[hi], _E4M3_POS_CODES[lo])
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# bfloat16 rounding (round to nearest, ties to even), written out
# --------------------------------------------------------------------------

def bf16_bits_rne(x) -> np.ndarray:
    """bf16 bit patterns of fp32 values, round to nearest with ties to even.

    The two bf16 neighbours of x are its truncation toward zero and the next
    bf16 away from zero; pick the nearer in exact float64 arithmetic, and on
    an exact tie the one whose last kept bit is 0.  Zeros keep their sign.
    Finite inputs only (overflow past the largest bf16 rounds to infinity).
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lo_bits = bits & 0xFFFF0000
    hi_bits = lo_bits + 0x10000
    lo = lo_bits.astype(np.uint32).view(np.float32).astype(np.float64)
    hi = hi_bits.astype(np.uint32).view(np.float32).astype(np.float64)
    xd = x.astype(np.float64)
    d_lo = np.abs(xd - lo)
    d_hi = np.abs(hi - xd)
    lo_even = ((lo_bits >> 16) & 1) == 0
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    out = np.where(take_hi, hi_bits, lo_bits) >> 16
    return out.astype(np.uint16)


def bf16_bits_rne_f64(x) -> np.ndarray:
    """bf16 bit patterns of float64 values, rounded once to nearest, ties even.

    bf16 keeps 8 significant bits: with x = f 2^e (0.5 <= |f| < 1), the
    result is rint(f 2^8) 2^(e - 8) (numpy's rint rounds ties to even), with
    the exponent held at bf16's subnormal quantum 2^-133 for tiny values.
    The rounded value is exact in fp32, whose top 16 bits are the pattern.
    Finite inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    e = np.maximum(e, -125)
    r = np.rint(np.ldexp(x, 8 - e))
    y = np.ldexp(r, e - 8)
    return (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_float64(b) -> np.ndarray:
    """Exact value of bf16 bit patterns."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Quantizer: blockwise NF4 with double quantization
# --------------------------------------------------------------------------

def quantize_nf4_dq(W, table=None) -> dict:
    """Quantize a weight matrix (any shape, fp32) in row-major order.

    Steps, in the pages' order:
      1. c1_b = max |w| over block b (64 consecutive weights)      [P1] Eq. 1
      2. w_hat = fl32(w / c1_b) (alpha = 1); an all-zero block gives 0
      3. level = number of thresholds T_j strictly below w_hat     [P1] Step 1
      4. levels written as sign-magnitude 4-bit codes, packed per group of 8
         weights (see pack_levels)
      5. c2_g = max c1 over group g of 256 blocks                   [P1] Step 2
      6. a_b = E4M3(fl32(c1_b / c2_g)); a zero group gives a_b = 0  [P4] Innov. 2
    The element count must be a multiple of 64; the last group may hold
    fewer than 256 blocks.
    Returns dict(codes=uint8[numel/2], absmax8=uint8[numel/64],
                 c2=float32[ceil(numel/16384)], c1=float32[numel/64]).
    ``table`` = (Q, T) replaces the NF4 levels and thresholds (for example
    uniform4_table()); everything else is the same.
    """
    Tt = NF4_T if table is None else table[1]
    w = np.ascontiguousarray(W, dtype=np.float32).reshape(-1)
    if w.size % BLOCK:
        raise ValueError("element count must be a multiple of 64")
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    nblk = w.size // BLOCK
    wb = w.reshape(nblk, BLOCK)
    c1 = np.max(np.abs(wb), axis=1).astype(np.float32)                      # step 1
    safe = np.where(c1 > 0, c1, np.float32(1.0)).astype(np.float32)
    w_hat = (wb / safe[:, None]).astype(np.float32)                         # step 2
    w_hat = np.where(c1[:, None] > 0, w_hat, np.float32(0.0))
    level = np.zeros(wb.shape, dtype=np.uint8)
    for t in Tt:                                                            # step 3
        level += (w_hat > t).astype(np.uint8)
    packed = pack_levels(level.reshape(-1))                                 # step 4
    ngrp = (nblk + DQ_BLOCKS - 1) // DQ_BLOCKS
    c2 = np.zeros(ngrp, dtype=np.float32)
    for g in range(ngrp):                                                   # step 5
        c2[g] = np.max(c1[g * DQ_BLOCKS:(g + 1) * DQ_BLOCKS])
    c2_of_block = np.repeat(c2, DQ_BLOCKS)[:nblk]
    ratio = np.where(c2_of_block > 0,
                     (c1 / np.where(c2_of_block > 0, c2_of_block, np.float32(1.0))).astype(np.float32),
                     np.float32(0.0))
    absmax8 = e4m3_encode_rne(ratio)                                        # step 6
    return dict(codes=packed, absmax8=absmax8, c2=c2, c1=c1)


def level_to_code(level) -> np.ndarray:
    """4-bit code of an NF4 level: sign in bit 3, magnitude rank in bits 0-2.

    The 16 levels are symmetric (level 15 - L is minus level L), so a level is
    written as its sign (bit 3 set for the 8 negative levels) and the rank of
    its magnitude among the 8 positive levels: code = L - 8 for L >= 8 and
    15 - L for L < 8.  The pages fix the levels, not their bit patterns.
    """
    L = np.asarray(level, dtype=np.int64)
    return np.where(L >= 8, L - 8, 15 - L).astype(np.uint8)


def code_to_level(code) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    return np.where(c < 8, c + 8, 15 - c).astype(np.uint8)


def pack_levels(level) -> np.ndarray:
    """Pack levels (numel a multiple of 8) into bytes.

    In each group of 8 consecutive weights, byte j (j = 0..3) of the group's
    4 bytes holds the code of weight j in its low nibble and of weight j + 4
    in its high nibble.
    """
    c = level_to_code(level).reshape(-1, 8)
    return (c[:, 0:4] | (c[:, 4:8] << 4)).astype(np.uint8).reshape(-1)


def unpack_codes(codes, numel: int) -> np.ndarray:
    """NF4 level (0..15) of each element; inverse of pack_levels."""
    b = np.asarray(codes, dtype=np.uint8)[: numel // 2].reshape(-1, 4)
    c = np.concatenate([b & 0xF, b >> 4], axis=1).reshape(-1)
    return code_to_level(c)


def block_scales(absmax8, c2, nblk: int) -> np.ndarray:
    """s_b = fl32(dec(a_b) * c2_g): the reconstructed first-level constants."""
    dec = e4m3_decode(np.asarray(absmax8)[:nblk]).astype(np.float32)
    c2_of_block = np.repeat(np.asarray(c2, dtype=np.float32), DQ_BLOCKS)[:nblk]
    return (dec * c2_of_block).astype(np.float32)


def dequant_nf4_dq(codes, absmax8, c2, numel: int, first_element: int = 0, table=None) -> np.ndarray:
    """bf16 bit patterns of W' = bf16(fl32(Q[code] * s_b)).

    [P1] Step 3 symbols: W0 is dequantized to BF16 at run time.
    ``codes``/``absmax8`` may describe a contiguous slice of a larger weight:
    ``first_element`` is that slice's offset in the full weight (a multiple
    of 64) so the right c2 group is used; ``c2`` is the full c2 array.
    """
    if first_element % BLOCK or numel % BLOCK:
        raise ValueError("slices must be whole 64-element blocks")
    nblk = numel // BLOCK
    b0 = first_element // BLOCK
    grp = (b0 + np.arange(nblk)) // DQ_BLOCKS
    dec = e4m3_decode(np.asarray(absmax8)[:nblk]).astype(np.float32)
    s = (dec * np.asarray(c2, dtype=np.float32)[grp]).astype(np.float32)
    Qt = NF4_Q if table is None else table[0]
    q = Qt[unpack_codes(codes, numel)].reshape(nblk, BLOCK)
    vals = (q * s[:, None]).astype(np.float32)
    return bf16_bits_rne(vals.reshape(-1))


def dequant_cols(qw: dict, m: int, n: int, cols) -> np.ndarray:
    """float64 values of W'[:, cols] for an m x n weight (same definition)."""
    cols = np.asarray(cols, dtype=np.int64)
    e = (np.arange(m, dtype=np.int64)[:, None] * n + cols[None, :]).reshape(-1)
    byte = np.asarray(qw["codes"], dtype=np.uint8)[(e // 8) * 4 + (e % 4)]
    code = code_to_level(np.where((e % 8) < 4, byte & 0xF, byte >> 4))
    blk = e // BLOCK
    dec = e4m3_decode(np.asarray(qw["absmax8"])[blk]).astype(np.float32)
    s = (dec * np.asarray(qw["c2"], dtype=np.float32)[blk // DQ_BLOCKS]).astype(np.float32)
    vals = (NF4_Q[code] * s).astype(np.float32)
    return bf16_bits_to_float64(bf16_bits_rne(vals)).reshape(m, len(cols))


def dequant_rows(qw: dict, m: int, n: int, rows) -> np.ndarray:
    """float64 values of W' for the given output rows of an m x n weight."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), n), dtype=np.float64)
    for i, r in enumerate(rows):
        e0 = int(r) * n
        out[i] = bf16_bits_to_float64(dequant_nf4_dq(
            qw["codes"][e0 // 2:(e0 + n) // 2], qw["absmax8"][e0 // BLOCK:(e0 + n) // BLOCK],
            qw["c2"], n, first_element=e0))
    return out


# --------------------------------------------------------------------------
# Adapted linear layer, forward and backward, float64
# --------------------------------------------------------------------------

def linear_fwd(x, Wd, A, B, s: float):
    """h = x W'^T + s (x A^T) B^T, and u = x A^T.   [P1] Step 3, Eq. 3.

    x: M x n, Wd (= W', dequantized): m x n, A: r x n, B: m x r, all float64.
    Eq. 3 writes the layer as h = W0 x + B A x for one column x; with the
    tokens as the rows of x that is h = x W0^T + x A^T B^T.  The adapter term
    carries s = alpha / r (the code snippet's LoraConfig comment).
    """
    x = np.asarray(x, dtype=np.float64)
    u = x @ np.asarray(A, dtype=np.float64).T
    h = x @ np.asarray(Wd, dtype=np.float64).T + s * (u @ np.asarray(B, dtype=np.float64).T)
    return h, u


def linear_bwd(x, g, Wd, A, B, s: float, u=None):
    """Gradients of <g, h> for the forward above, float64.

    [P1] Step 4, Eq. 5: dL/dA = B^T (dL/dh) x^T and dL/dB = (dL/dh)(A x)^T,
    here with tokens as rows and the s factor: grad_A = s v^T x,
    grad_B = s g^T u, with v = g B and u = x A^T.  The input gradient follows
    the chain rule through the frozen W': grad_x = g W' + s v A (W0 itself
    gets no gradient).
    """
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    if u is None:
        u = x @ A.T
    v = g @ B
    grad_x = g @ np.asarray(Wd, dtype=np.float64) + s * (v @ A)
    grad_A = s * (v.T @ x)
    grad_B = s * (g.T @ u)
    return dict(grad_x=grad_x, grad_A=grad_A, grad_B=grad_B, v=v)


def merge_adapter(Wd_bits, A_bits, B_bits, s: float, m: int, n: int) -> np.ndarray:
    """bf16 bit patterns of W' + s B A, summed exactly and rounded once.

    [P1] Real-World Impact: after training, the adapter is merged into the
    base weight, W_merged = W0 + B A, so inference runs a plain layer.
    [P4] Followups to expect: the 4-bit weight is dequantized to BF16 first,
    the adapter added, and a 16-bit weight kept.  The adapter term carries
    s = alpha / r as in the forward.  Wd_bits: m*n bf16 patterns of W'
    (dequant_nf4_dq), A_bits: r x n, B_bits: m x r bf16 patterns.
    """
    Wd = bf16_bits_to_float64(np.asarray(Wd_bits)).reshape(m, n)
    A = bf16_bits_to_float64(np.asarray(A_bits))
    B = bf16_bits_to_float64(np.asarray(B_bits))
    return bf16_bits_rne_f64(Wd + s * (B @ A)).reshape(m, n)


def adam_step(p, g, m, v, t: int, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float):
    """One Adam step with decoupled weight decay on an adapter tensor, float64.

    [P1] memory-layout figure: Adam moments m, v kept for the adapters only;
    [P3] "Worked example": fp32 parameter, gradient and the two Adam moments,
    16 bytes per trainable parameter.  The step is the textbook one:
      p <- p (1 - lr wd)
      m <- b1 m + (1 - b1) g            v <- b2 v + (1 - b2) g^2
      p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
    with t >= 1 the step number.  Returns (p, m, v); inputs are not modified.
    """
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    p = p - lr * mhat / (np.sqrt(vhat) + eps)
    return p, m, v


# --------------------------------------------------------------------------
# LoRA dropout on the adapter input (the snippet's lora_dropout)
# --------------------------------------------------------------------------

PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57   # round multipliers
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85   # key schedule increments


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw: "Parallel random
    numbers: as easy as 1, 2, 3", SC 2011), in Python integers.

    ctr: four 32-bit words, key: two.  A round multiplies counter words 0 and
    2 by the two constants (64-bit products split into high and low halves),
    then permutes and mixes: (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3
    ^ k1, lo(M0 c0)); the key gets the Weyl increments between rounds.
    """
    c = [int(v) & 0xFFFFFFFF for v in ctr]
    k = [int(v) & 0xFFFFFFFF for v in key]
    for r in range(10):
        if r:
            k = [(k[0] + PHILOX_W0) & 0xFFFFFFFF, (k[1] + PHILOX_W1) & 0xFFFFFFFF]
        p0 = PHILOX_M0 * c[0]
        p1 = PHILOX_M1 * c[2]
        c = [((p1 >> 32) ^ c[1] ^ k[0]) & 0xFFFFFFFF, p1 & 0xFFFFFFFF,
             ((p0 >> 32) ^ c[3] ^ k[1]) & 0xFFFFFFFF, p0 & 0xFFFFFFFF]
    return c


def dropout_keep_threshold(p: float) -> int:
    """32-bit threshold: an element is dropped when its random word is below it."""
    return min(int(round(p * 2.0 ** 32)), 0xFFFFFFFF)


def dropout_mask(M: int, n: int, p: float, seed: int, offset: int = 0) -> np.ndarray:
    """Keep-mask (bool, M x n) of the adapter input.

    Element e = t n + k takes word e % 4 of Philox4x32-10 at the 64-bit
    counter e // 4 + offset (low word first, upper two words zero) under the
    key (seed low 32 bits, seed high 32 bits); it is kept when that word is
    at least round(p 2^32).  [P1] LoraConfig snippet (lora_dropout), applied
    to the input of the adapter branch only.
    """
    thr = dropout_keep_threshold(p)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    total = M * n
    words = np.empty(((total + 3) // 4) * 4, dtype=np.uint64)
    for c in range((total + 3) // 4):
        ctr = c + offset
        words[4 * c:4 * c + 4] = philox4x32_10((ctr & 0xFFFFFFFF, (ctr >> 32) & 0xFFFFFFFF, 0, 0), key)
    return (words[:total] >= thr).reshape(M, n)


def philox4x32_10_np(ctr_lo, ctr_hi, key):
    """philox4x32_10 over arrays of counters (words 2 and 3 zero), the same
    rounds in numpy uint64 arithmetic (each 32 x 32-bit product fits).
    Returns the four output words as uint64 arrays."""
    m32 = np.uint64(0xFFFFFFFF)
    c0 = np.asarray(ctr_lo, dtype=np.uint64) & m32
    c1 = np.asarray(ctr_hi, dtype=np.uint64) & m32
    c2 = np.zeros_like(c0)
    c3 = np.zeros_like(c0)
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for r in range(10):
        if r:
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
        p0 = np.uint64(PHILOX_M0) * c0
        p1 = np.uint64(PHILOX_M1) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0), p1 & m32,
                          (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1), p0 & m32)
    return c0, c1, c2, c3


def dropout_mask_np(M: int, n: int, p: float, seed: int, offset: int = 0) -> np.ndarray:
    """dropout_mask vectorized over the counters (for large tensors)."""
    total = M * n
    nctr = (total + 3) // 4
    ctr = np.arange(nctr, dtype=np.uint64) + np.uint64(offset)   # wraps like the 64-bit counter
    words = philox4x32_10_np(ctr & np.uint64(0xFFFFFFFF), ctr >> np.uint64(32),
                             (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    w = np.stack(words, axis=1).reshape(-1)[:total]
    return (w >= np.uint64(dropout_keep_threshold(p))).reshape(M, n)


def dropout_mask_at(rows, cols, n: int, p: float, seed: int, offset: int = 0) -> np.ndarray:
    """dropout_mask restricted to the elements (rows x cols) of an (any) x n
    tensor, vectorized: for sampled outputs of large tensors."""
    rows = np.asarray(rows, dtype=np.uint64)
    cols = np.asarray(cols, dtype=np.uint64)
    e = rows[:, None] * np.uint64(n) + cols[None, :]
    ctr = (e >> np.uint64(2)) + np.uint64(offset)   # offsets near 2^64 wrap like the 64-bit counter
    words = philox4x32_10_np(ctr & np.uint64(0xFFFFFFFF), ctr >> np.uint64(32),
                             (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    w = np.select([(e & np.uint64(3)) == np.uint64(j) for j in range(4)], list(words))
    return w >= np.uint64(dropout_keep_threshold(p))


def linear_fwd_dropout(x, Wd, A, B, s: float, keep, p: float):
    """Forward with dropout on the adapter input: u = (x * keep / (1 - p)) A^T,
    h = x W'^T + s u B^T.  [P1] Step 3, Eq. 3 and the snippet's lora_dropout."""
    x = np.asarray(x, dtype=np.float64)
    xd = x * np.asarray(keep, dtype=np.float64) / (1.0 - p)
    u = xd @ np.asarray(A, dtype=np.float64).T
    h = x @ np.asarray(Wd, dtype=np.float64).T + s * (u @ np.asarray(B, dtype=np.float64).T)
    return h, u


def linear_bwd_dropout(x, g, Wd, A, B, s: float, keep, p: float):
    """Gradients of <g, h> for linear_fwd_dropout (chain rule; the mask is fixed):
    v = g B, grad_x = g W' + s (v A) * keep / (1 - p),
    grad_A = s v^T (x * keep / (1 - p)), grad_B = s g^T u."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    kf = np.asarray(keep, dtype=np.float64) / (1.0 - p)
    xd = x * kf
    u = xd @ A.T
    v = g @ B
    grad_x = g @ np.asarray(Wd, dtype=np.float64) + s * (v @ A) * kf
    grad_A = s * (v.T @ xd)
    grad_B = s * (g.T @ u)
    return dict(grad_x=grad_x, grad_A=grad_A, grad_B=grad_B, v=v, u=u)


def linear_fwd_loops(x, Wd, A, B, s: float):
    """Same as linear_fwd with explicit Python loops (small inputs only)."""
    M, n = len(x), len(x[0])
    m, r = len(Wd), len(A)
    u = [[math.fsum(float(x[t][k]) * float(A[q][k]) for k in range(n)) for q in range(r)] for t in range(M)]
    h = [[math.fsum(float(x[t][k]) * float(Wd[j][k]) for k in range(n))
          + s * math.fsum(u[t][q] * float(B[j][q]) for q in range(r)) for j in range(m)] for t in range(M)]
    return np.array(h), np.array(u)


def linear_bwd_loops(x, g, Wd, A, B, s: float):
    """Same as linear_bwd with explicit Python loops (small inputs only)."""
    M, n = len(x), len(x[0])
    m, r = len(Wd), len(A)
    u = [[math.fsum(float(x[t][k]) * float(A[q][k]) for k in range(n)) for q in range(r)] for t in range(M)]
    v = [[math.fsum(float(g[t][j]) * float(B[j][q]) for j in range(m)) for q in range(r)] for t in range(M)]
    gx = [[math.fsum(float(g[t][j]) * float(Wd[j][k]) for j in range(m))
           + s * math.fsum(v[t][q] * float(A[q][k]) for q in range(r)) for k in range(n)] for t in range(M)]
    gA = [[s * math.fsum(v[t][q] * float(x[t][k]) for t in range(M)) for k in range(n)] for q in range(r)]
    gB = [[s * math.fsum(float(g[t][j]) * u[t][q] for t in range(M)) for q in range(r)] for j in range(m)]
    return dict(grad_x=np.array(gx), grad_A=np.array(gA), grad_B=np.array(gB))


# --------------------------------------------------------------------------
# Storage arithmetic  ([P3] "The three pieces", worked example; [P4] Innov. 2)
# --------------------------------------------------------------------------

def storage_bytes(numel: int) -> int:
    """Bytes of codes + 8-bit constants + fp32 c2 for one quantized weight."""
    nblk = numel // BLOCK
    return numel // 2 + nblk + 4 * ((nblk + DQ_BLOCKS - 1) // DQ_BLOCKS)


def constant_overhead_bits(double_quant: bool) -> float:
    """Bits per parameter spent on scale constants.

    Without double quantization: one fp32 per 64 weights.  With it: one
    8-bit float per 64 weights plus one fp32 per 64 * 256 weights.
    """
    if not double_quant:
        return 32.0 / BLOCK
    return 8.0 / BLOCK + 32.0 / (BLOCK * DQ_BLOCKS)


def adapter_params(m: int, n: int, r: int) -> int:
    """r (m + n): trainable parameters of one adapted m x n layer ([P1] Eq. 4)."""
    return r * (m + n)


# --------------------------------------------------------------------------
# Comparison point: plain 4-bit integer absmax quantization ([P1] Step 1 and
# [P4] Innovation 1 contrast NF4 with uniformly spaced INT4 levels)
# --------------------------------------------------------------------------

def int4_table():
    """Return (Q, T) of symmetric INT4 absmax quantization as a 16-entry
    table for the same pipeline: the 15 levels k/7, k = -7..7, with the zero
    level written twice, as -0 (index 7) and +0 (index 8), so that the table
    keeps the sign-magnitude symmetry Q_{15-j} = -Q_j bit for bit.
    Q_{8+k} = fl32(k/7); T_j = fl32((Q_j + Q_{j+1}) / 2) as for NF4, which
    makes T_7 = 0: a normalized weight w_hat > 0 takes +0 or above, w_hat <= 0
    takes -0 or below, and both zeros dequantize to the value 0.  Apart from
    fp32 rounding of the thresholds (and ties, which the threshold rule sends
    to the lower level) the level of w_hat is rint(7 w_hat) / 7: the integer
    absmax quantizer of int4_absmax_roundtrip, with double-quantized scales.
    """
    pos = np.array([k / 7.0 for k in range(8)], dtype=np.float64).astype(np.float32)
    Q = np.concatenate([-pos[::-1], pos]).astype(np.float32)   # index 7 is -0.0
    T = ((Q[:-1].astype(np.float64) + Q[1:].astype(np.float64)) / 2.0).astype(np.float32)
    return Q, T


INT4_Q, INT4_T = int4_table()


def int4_absmax_roundtrip(W) -> np.ndarray:
    """Round trip through symmetric INT4 absmax quantization, blocks of 64.

    Levels k/7 * c1, k = -7..7 (uniform spacing), nearest level, fp32 c1.
    """
    w = np.asarray(W, dtype=np.float64).reshape(-1, BLOCK)
    c1 = np.max(np.abs(w), axis=1, keepdims=True)
    safe = np.where(c1 > 0, c1, 1.0)
    k = np.clip(np.rint(w / safe * 7.0), -7, 7)
    return (k / 7.0 * c1).reshape(-1)
