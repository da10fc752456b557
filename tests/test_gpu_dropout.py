"""GPU parity of LoRA dropout on the adapter input (qlora_linear_fwd_ex and
qlora_linear_bwd_ex) against the oracle's linear_fwd_dropout /
linear_bwd_dropout with the oracle's own Philox mask.

Bit-exact: the keep-mask, read off outputs on which it shows alone (W = 0,
A = B = identity: u and grad_x are the masked x and g, and with one-hot g
grad_A is the masked x), on the weight-streaming and the tiled paths; p = 0
gives the plain layer's bits.  Within the float tolerance of the other
parity tests (relative L2 <= 1e-2, max-abs <= 2e-2 max|ref|): h, u, grad_x,
grad_A, grad_B on small and ragged shapes and, on sampled outputs, on a
full-size layer.  p is passed to the oracle as the fp32 value the library
receives, so both draw the same threshold.
"""

import numpy as np
import pytest
import torch

import qlora_inputs as QI
from oracle import qlora_oracle as O
from parity_utils import assert_close, dev_bf16, f64, host_bits, sample_indices

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import bit_quantized_fine_qlora_amd as lib
    lib._lib.load()
    return lib


def say(msg):
    print(f"[case] {msg}", flush=True)


def f32(v):
    return float(np.float32(v))


def gpu_case(Q, inp, s, drop, u_from_fwd=True):
    q = Q.quantize_nf4_dq(torch.from_numpy(inp["W"]).cuda())
    x, A, B, g = (dev_bf16(inp[k]) for k in ("x", "A", "B", "g"))
    h, u = Q.linear_fwd(x, q, A, B, s, dropout=drop)
    gx, gA, gB = Q.linear_bwd(x, g, q, A, B, s, u=u if u_from_fwd else None, dropout=drop)
    torch.cuda.synchronize()
    return dict(q=q, x=x, A=A, B=B, g=g, h=h, u=u, grad_x=gx, grad_A=gA, grad_B=gB)


def oracle_case(inp, s, p, seed, offset):
    W = inp["W"]
    m, n = W.shape
    M = inp["x"].shape[0]
    qw = O.quantize_nf4_dq(W)
    Wd = f64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], m * n)).reshape(m, n)
    x, A, B, g = (f64(inp[k]) for k in ("x", "A", "B", "g"))
    keep = O.dropout_mask(M, n, p, seed, offset)
    h, u = O.linear_fwd_dropout(x, Wd, A, B, s, keep, p)
    bw = O.linear_bwd_dropout(x, g, Wd, A, B, s, keep, p)
    out = dict(bw)
    out.update(h=h, u=u, keep=keep)
    return out


def check_against_oracle(got, ref, label):
    assert_close(f64(host_bits(got["h"])), ref["h"], f"{label} h")
    assert_close(got["u"].cpu().numpy(), ref["u"], f"{label} u")
    assert_close(f64(host_bits(got["grad_x"])), ref["grad_x"], f"{label} grad_x")
    assert_close(f64(host_bits(got["grad_A"])), ref["grad_A"], f"{label} grad_A")
    assert_close(f64(host_bits(got["grad_B"])), ref["grad_B"], f"{label} grad_B")


CASES = [
    # (M, n, m, r, s, p, seed, offset)
    (16, 512, 384, 16, 2.0, 0.1, 1234, 0),                  # weight-streaming forward
    (5, 256, 200, 8, 1.0, 0.3, 2 ** 33 + 7, 11),           # ragged M, m % 8 != 0 (padded g)
    (300, 512, 320, 8, 2.0, 0.05, 99, 2 ** 32 - 100),      # tiled; counters carry into the high word
    (128, 384, 256, 32, 1.0, 0.2, 77, 3),                  # rank 32 (v and grad_B in one pass over g)
    (256, 256, 512, 64, 0.5, 0.5, 5, 0),                   # rank 64 (separate v and grad_B kernels)
    (64, 512, 2048, 16, 2.0, 0.1, 4321, 5),                # grad_x GEMM in 4 K pieces, masked term added after
]


@pytest.mark.parametrize("M,n,m,r,s,p,seed,offset", CASES)
def test_dropout_matches_oracle(Q, M, n, m, r, s, p, seed, offset):
    p = f32(p)
    inp = QI.custom_inputs(seed=500 + M + r, M=M, n=n, m=m, r=r)
    say(f"dropout M={M} n={n} m={m} r={r} p={p} seed={seed} offset={offset}")
    got = gpu_case(Q, inp, s, (p, seed, offset))
    ref = oracle_case(inp, s, p, seed, offset)
    check_against_oracle(got, ref, f"dropout M={M}")
    # u recomputed inside the backward (with the mask) instead of the forward's
    say(f"dropout M={M}: backward with u recomputed")
    gx2, gA2, gB2 = Q.linear_bwd(got["x"], got["g"], got["q"], got["A"], got["B"], s, u=None,
                                 dropout=(p, seed, offset))
    torch.cuda.synchronize()
    assert torch.equal(gx2, got["grad_x"]) and torch.equal(gA2, got["grad_A"])
    if M > 32:
        # the tiled forward and the backward form u by the same kernels and splits
        assert torch.equal(gB2, got["grad_B"])
    else:
        assert_close(f64(host_bits(gB2)), ref["grad_B"], f"dropout M={M} grad_B (u recomputed)")


def _random_cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        M = int(rng.integers(1, 33)) if i % 2 == 0 else int(rng.integers(33, 400))
        out.append((M, 64 * int(rng.integers(1, 17)), int(rng.integers(1, 900)), int(rng.integers(1, 129)),
                    float(rng.choice([0.5, 1.0, 2.0])), float(rng.choice([0.1, 0.3, 0.5])),
                    int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 40))))
    return out


@pytest.mark.parametrize("M,n,m,r,s,p,seed,offset", _random_cases(6, 77))
def test_dropout_random_shapes(Q, M, n, m, r, s, p, seed, offset):
    p = f32(p)
    inp = QI.custom_inputs(seed=900 + M + n + r, M=M, n=n, m=m, r=r)
    say(f"dropout random M={M} n={n} m={m} r={r} p={p}")
    got = gpu_case(Q, inp, s, (p, seed, offset))
    ref = oracle_case(inp, s, p, seed, offset)
    check_against_oracle(got, ref, f"dropout random M={M} n={n} m={m} r={r}")


@pytest.mark.parametrize("M", [16, 300])
def test_p_zero_is_the_plain_layer(Q, M):
    inp = QI.custom_inputs(seed=61, M=M, n=256, m=192, r=16)
    s = 1.5
    say(f"dropout p=0 against the plain layer, M={M}")
    got = gpu_case(Q, inp, s, (0.0, 1, 2))
    q, x, A, B, g = got["q"], got["x"], got["A"], got["B"], got["g"]
    h, u = Q.linear_fwd(x, q, A, B, s)
    gx, gA, gB = Q.linear_bwd(x, g, q, A, B, s, u=u)
    torch.cuda.synchronize()
    for k, t in (("h", h), ("u", u), ("grad_x", gx), ("grad_A", gA), ("grad_B", gB)):
        assert torch.equal(got[k], t), k


def identity_bits(k):
    return O.bf16_bits_rne(np.eye(k, dtype=np.float32))


def nonzero_bf16(seed, shape):
    bits = QI.to_bf16_bits(QI.normal_f32(seed, shape, 1.0))
    assert np.all(bits & 0x7FFF), "draw has a zero"
    return bits


@pytest.mark.parametrize("M", [16, 27, 100])
def test_mask_exact_on_u_and_grad_x(Q, M):
    # W = 0, A = B = I (n = m = r = 64): u = x_d and grad_x = bf16(s g keep / (1 - p)),
    # so their zero pattern is the mask itself
    n = 64
    p, seed, offset, s = f32(0.37), 0xDEADBEEF12345678, 2 ** 32 - 9, 1.25
    inp = dict(W=np.zeros((n, n), dtype=np.float32), x=nonzero_bf16(71 + M, (M, n)),
               g=nonzero_bf16(72 + M, (M, n)), A=identity_bits(n), B=identity_bits(n))
    say(f"dropout mask exact, u and grad_x, M={M}")
    got = gpu_case(Q, inp, s, (p, seed, offset))
    keep = O.dropout_mask(M, n, p, seed, offset)
    assert 0 < keep.sum() < keep.size
    u = got["u"].cpu().numpy()
    assert np.array_equal(u != 0, keep), "u: mask differs"
    x = f64(inp["x"])
    assert np.allclose(u, x * keep / (1 - p), rtol=2.0 ** -22, atol=0)
    gx = f64(host_bits(got["grad_x"]))
    assert np.array_equal(gx != 0, keep), "grad_x: mask differs"
    assert_close(gx, s * f64(inp["g"]) * keep / (1 - p), f"mask M={M} grad_x")


def test_mask_exact_on_grad_A(Q):
    # one-hot g (token t -> rank t) with B = I: grad_A row q is s x_d[q]
    M = n = 64
    p, seed, offset, s = f32(0.25), 31337, 1000, 2.0
    inp = dict(W=np.zeros((n, n), dtype=np.float32), x=nonzero_bf16(81, (M, n)), g=identity_bits(n),
               A=identity_bits(n), B=identity_bits(n))
    say("dropout mask exact, grad_A")
    got = gpu_case(Q, inp, s, (p, seed, offset))
    keep = O.dropout_mask(M, n, p, seed, offset)
    gA = f64(host_bits(got["grad_A"]))
    assert np.array_equal(gA != 0, keep), "grad_A: mask differs"
    assert_close(gA, s * f64(inp["x"]) * keep / (1 - p), "mask grad_A")


def test_full_size_layer_sampled(Q):
    # the 14336 x 4096 gate projection, 4096 tokens, rank 16, p = 0.05
    L = QI.WORKLOADS[2]["layers"][0]
    p, seed, offset = f32(0.05), 2024, 77
    say(f"dropout full size {L.name} {L.m}x{L.n} M={L.M} r={L.r}: drawing inputs")
    inp = QI.layer_inputs(2, L)
    got = gpu_case(Q, inp, L.s, (p, seed, offset))
    say("dropout full size: oracle on samples")
    qw = O.quantize_nf4_dq(inp["W"])
    rows = sample_indices(L.m, 96, 11)
    toks = sample_indices(L.M, 48, 12)
    cols = sample_indices(L.n, 96, 13)
    Wr = O.dequant_rows(qw, L.m, L.n, rows)
    Wc = O.dequant_cols(qw, L.m, L.n, cols)
    x, A, B, g = (f64(inp[k]) for k in ("x", "A", "B", "g"))
    keep = O.dropout_mask_np(L.M, L.n, p, seed, offset)
    xd = x * keep / (1 - p)
    u = xd @ A.T
    v = g @ B
    h_ref = x[toks] @ Wr.T + L.s * (u[toks] @ B[rows].T)
    gx_ref = g[toks] @ Wc + L.s * (v[toks] @ A[:, cols]) * keep[np.ix_(toks, cols)] / (1 - p)
    gA_ref = L.s * (v.T @ xd[:, cols])
    gB_ref = L.s * (g[:, rows].T @ u)
    tc, cc, rc = (torch.from_numpy(a).cuda() for a in (toks, cols, rows))
    assert_close(f64(host_bits(got["h"][tc][:, rc])), h_ref, "dropout full h (sampled)")
    assert_close(got["u"][tc].cpu().numpy(), u[toks], "dropout full u (sampled)")
    assert_close(f64(host_bits(got["grad_x"][tc][:, cc])), gx_ref, "dropout full grad_x (sampled)")
    assert_close(f64(host_bits(got["grad_A"][:, cc])), gA_ref, "dropout full grad_A (sampled)")
    assert_close(f64(host_bits(got["grad_B"][rc])), gB_ref, "dropout full grad_B (sampled)")
    del got
    torch.cuda.empty_cache()


def test_many_tokens_sampled(Q):
    # 2.2 M tokens of a narrow layer: more 32-token tiles than a grid's y
    # dimension allows (65535), so the dropout term and the g pass must
    # launch 1D grids; checked on sampled tokens
    M, n, m, r, s = 2_200_000, 64, 64, 8, 2.0
    p, seed, offset = f32(0.2), 4242, 17
    say(f"dropout many tokens M={M} n={n} m={m} r={r}")
    rng = np.random.default_rng(5)
    x_bits = QI.to_bf16_bits(rng.standard_normal((M, n), dtype=np.float32))
    g_bits = QI.to_bf16_bits(rng.standard_normal((M, m), dtype=np.float32))
    inp = QI.custom_inputs(seed=3, M=1, n=n, m=m, r=r)
    inp["x"], inp["g"] = x_bits, g_bits
    got = gpu_case(Q, inp, s, (p, seed, offset))
    qw = O.quantize_nf4_dq(inp["W"])
    Wd = f64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], m * n)).reshape(m, n)
    toks = sample_indices(M, 64, 21)
    keep = O.dropout_mask_at(toks, np.arange(n), n, p, seed, offset)
    x, g = f64(x_bits[toks]), f64(g_bits[toks])
    A, B = f64(inp["A"]), f64(inp["B"])
    u = (x * keep / (1 - p)) @ A.T
    v = g @ B
    tc = torch.from_numpy(toks).cuda()
    assert_close(f64(host_bits(got["h"][tc])), x @ Wd.T + s * (u @ B.T), "many tokens h (sampled)")
    assert_close(got["u"][tc].cpu().numpy(), u, "many tokens u (sampled)")
    assert_close(f64(host_bits(got["grad_x"][tc])), g @ Wd + s * (v @ A) * keep / (1 - p),
                 "many tokens grad_x (sampled)")
    del got
    torch.cuda.empty_cache()
