"""Pins for the oracle's forward and backward of the adapted linear layer.

The pages print no worked example of h or of a gradient, so these values are
pinned by identities: automatic differentiation of the forward, central
finite differences, Eq. 3 evaluated one token (column) at a time, the B = 0
and W0 = 0 special cases, the merged-weight identity, and a loop-based
evaluation of the same definitions.
"""

import numpy as np
import pytest
import torch

from oracle import qlora_oracle as O
import qlora_inputs as QI


def small_case(seed=1, M=5, n=128, m=24, r=3, s=1.75):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, n))
    Wd = rng.standard_normal((m, n)) * 0.05
    A = rng.standard_normal((r, n)) * 0.2
    B = rng.standard_normal((m, r)) * 0.3
    g = rng.standard_normal((M, m))
    return x, Wd, A, B, g, s


def test_forward_matches_eq3_per_token():
    x, Wd, A, B, g, s = small_case()
    h, u = O.linear_fwd(x, Wd, A, B, s)
    for t in range(x.shape[0]):
        col = x[t][:, None]                                  # Eq. 3 acts on a column vector
        ht = Wd @ col + s * (B @ (A @ col))
        assert np.allclose(h[t], ht[:, 0], rtol=1e-13, atol=1e-13)
        assert np.allclose(u[t], (A @ col)[:, 0], rtol=1e-13, atol=1e-13)


def test_forward_b_zero_is_plain_matmul():
    x, Wd, A, B, g, s = small_case()
    h, _ = O.linear_fwd(x, Wd, A, np.zeros_like(B), s)
    assert np.array_equal(h, x @ Wd.T)


def test_forward_w_zero_is_pure_adapter():
    x, Wd, A, B, g, s = small_case()
    h, _ = O.linear_fwd(x, np.zeros_like(Wd), A, B, s)
    assert np.allclose(h, s * np.einsum("tk,qk,jq->tj", x, A, B), rtol=1e-12, atol=1e-13)


def test_merge_identity():
    # merging the adapter into the dequantized weight gives the same layer
    x, Wd, A, B, g, s = small_case()
    h, _ = O.linear_fwd(x, Wd, A, B, s)
    merged = Wd + s * (B @ A)
    assert np.max(np.abs(x @ merged.T - h)) <= 1e-12 * np.max(np.abs(h))


def test_backward_matches_autograd():
    x, Wd, A, B, g, s = small_case(seed=2)
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tA = torch.tensor(A, dtype=torch.float64, requires_grad=True)
    tB = torch.tensor(B, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(Wd, dtype=torch.float64)
    h = torch.nn.functional.linear(tx, tW) + s * torch.nn.functional.linear(torch.nn.functional.linear(tx, tA), tB)
    loss = (h * torch.tensor(g, dtype=torch.float64)).sum()
    loss.backward()
    got = O.linear_bwd(x, g, Wd, A, B, s)
    for k, t in (("grad_x", tx), ("grad_A", tA), ("grad_B", tB)):
        ref = t.grad.numpy()
        assert np.max(np.abs(got[k] - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref))), k


def test_backward_matches_eq5_per_token():
    # Eq. 5 (one token, column vectors): dA = B^T dh x^T, dB = dh (A x)^T, times s
    x, Wd, A, B, g, s = small_case(seed=3, M=1)
    got = O.linear_bwd(x, g, Wd, A, B, s)
    dh = g[0][:, None]
    col = x[0][:, None]
    assert np.allclose(got["grad_A"], s * (B.T @ dh @ col.T), rtol=1e-13, atol=1e-14)
    assert np.allclose(got["grad_B"], s * (dh @ (A @ col).T), rtol=1e-13, atol=1e-14)


def test_backward_finite_differences():
    x, Wd, A, B, g, s = small_case(seed=4, M=3, n=64, m=8, r=2)
    got = O.linear_bwd(x, g, Wd, A, B, s)

    def loss(x_, A_, B_):
        h, _ = O.linear_fwd(x_, Wd, A_, B_, s)
        return float(np.sum(h * g))

    eps = 1e-6
    rng = np.random.default_rng(0)
    for name, arr in (("grad_x", x), ("grad_A", A), ("grad_B", B)):
        for _ in range(4):
            idx = tuple(int(rng.integers(0, d)) for d in arr.shape)
            p, mns = arr.copy(), arr.copy()
            p[idx] += eps
            mns[idx] -= eps
            args_p = dict(x_=x, A_=A, B_=B)
            args_m = dict(x_=x, A_=A, B_=B)
            key = {"grad_x": "x_", "grad_A": "A_", "grad_B": "B_"}[name]
            args_p[key], args_m[key] = p, mns
            fd = (loss(**args_p) - loss(**args_m)) / (2 * eps)
            assert abs(fd - got[name][idx]) <= 1e-6 * max(1.0, abs(fd)), name


def test_b_zero_gives_zero_grad_a():
    x, Wd, A, B, g, s = small_case(seed=5)
    got = O.linear_bwd(x, g, Wd, A, np.zeros_like(B), s)
    assert np.all(got["grad_A"] == 0)
    assert np.array_equal(got["grad_x"], g @ Wd)


def test_loops_match_vectorized_on_config1_shapes():
    # the real config-1 inputs, a slice of tokens to keep the loops short
    L = QI.WORKLOADS[1]["layers"][0]
    inp = QI.layer_inputs(1, L, M=4)
    qw = O.quantize_nf4_dq(inp["W"])
    Wd = O.bf16_bits_to_float64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], L.m * L.n)).reshape(L.m, L.n)
    x = O.bf16_bits_to_float64(inp["x"])
    g = O.bf16_bits_to_float64(inp["g"])
    A = O.bf16_bits_to_float64(inp["A"])
    B = O.bf16_bits_to_float64(inp["B"])
    m_sub = 16                                   # a few output features keep it fast
    h, u = O.linear_fwd(x, Wd[:m_sub], A, B[:m_sub], L.s)
    hl, ul = O.linear_fwd_loops(x.tolist(), Wd[:m_sub].tolist(), A.tolist(), B[:m_sub].tolist(), L.s)
    assert np.max(np.abs(h - hl)) <= 1e-12 * np.max(np.abs(h))
    assert np.max(np.abs(u - ul)) <= 1e-12 * np.max(np.abs(u))
    bw = O.linear_bwd(x, g[:, :m_sub], Wd[:m_sub], A, B[:m_sub], L.s)
    bl = O.linear_bwd_loops(x.tolist(), g[:, :m_sub].tolist(), Wd[:m_sub].tolist(), A.tolist(), B[:m_sub].tolist(), L.s)
    for k in ("grad_x", "grad_A", "grad_B"):
        assert np.max(np.abs(bw[k] - bl[k])) <= 1e-12 * max(1e-30, np.max(np.abs(bw[k]))), k
