"""Pins for the oracle's LoRA dropout (mask generator, forward and backward).

  * Philox4x32-10 against the generator's published known-answer vectors
    (Salmon et al., SC 2011: the Random123 distribution's tests for
    philox4x32 with 10 rounds);
  * the mask: p = 0 keeps everything, the dropped fraction matches p within
    binomial error, the same (seed, offset) gives the same mask, another
    offset a different one;
  * forward and backward: p = 0 reduces to the plain layer, and the backward
    equals float64 autograd of the forward with the mask held fixed.
"""

import numpy as np
import torch

from oracle import qlora_oracle as O


def test_philox_known_answers():
    cases = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, want in cases:
        assert tuple(O.philox4x32_10(ctr, key)) == want


def test_mask_statistics_and_determinism():
    assert O.dropout_mask(8, 64, 0.0, seed=5).all()
    p = 0.3
    m = O.dropout_mask(64, 256, p, seed=123456789)
    frac = 1.0 - m.mean()
    sd = np.sqrt(p * (1 - p) / m.size)
    assert abs(frac - p) < 5 * sd
    assert np.array_equal(m, O.dropout_mask(64, 256, p, seed=123456789))
    assert not np.array_equal(m, O.dropout_mask(64, 256, p, seed=123456789, offset=7))
    # element e uses word e % 4 of counter e // 4: the 4 elements of a counter
    # come from one Philox call
    seed = 0x0123456789ABCDEF
    words = O.philox4x32_10((2, 0, 0, 0), (seed & 0xFFFFFFFF, seed >> 32))
    thr = O.dropout_keep_threshold(0.5)
    row = O.dropout_mask(1, 64, 0.5, seed=seed)[0]
    assert [bool(w >= thr) for w in words] == list(row[8:12])


def small():
    rng = np.random.default_rng(2)
    M, n, m, r = 6, 64, 24, 3
    return (rng.standard_normal((M, n)), rng.standard_normal((m, n)) * 0.05, rng.standard_normal((r, n)) * 0.2,
            rng.standard_normal((m, r)) * 0.3, rng.standard_normal((M, m)))


def test_p_zero_is_the_plain_layer():
    x, Wd, A, B, g = small()
    keep = np.ones(x.shape, dtype=bool)
    h, u = O.linear_fwd_dropout(x, Wd, A, B, 1.5, keep, 0.0)
    h0, u0 = O.linear_fwd(x, Wd, A, B, 1.5)
    assert np.allclose(h, h0, rtol=1e-14, atol=1e-14) and np.allclose(u, u0, rtol=1e-14, atol=1e-14)
    bw = O.linear_bwd_dropout(x, g, Wd, A, B, 1.5, keep, 0.0)
    bw0 = O.linear_bwd(x, g, Wd, A, B, 1.5)
    for k in ("grad_x", "grad_A", "grad_B"):
        assert np.allclose(bw[k], bw0[k], rtol=1e-13, atol=1e-13), k


def test_backward_matches_autograd_with_fixed_mask():
    x, Wd, A, B, g = small()
    p, s = 0.25, 0.75
    keep = O.dropout_mask(*x.shape, p, seed=42)
    bw = O.linear_bwd_dropout(x, g, Wd, A, B, s, keep, p)
    tx = torch.tensor(x, requires_grad=True)
    tA = torch.tensor(A, requires_grad=True)
    tB = torch.tensor(B, requires_grad=True)
    km = torch.tensor(keep, dtype=torch.float64) / (1 - p)
    h = tx @ torch.tensor(Wd).T + s * ((tx * km) @ tA.T) @ tB.T
    h.backward(torch.tensor(g))
    assert np.allclose(bw["grad_x"], tx.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(bw["grad_A"], tA.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(bw["grad_B"], tB.grad.numpy(), rtol=1e-12, atol=1e-12)
    hf, _ = O.linear_fwd_dropout(x, Wd, A, B, s, keep, p)
    assert np.allclose(hf, h.detach().numpy(), rtol=1e-13, atol=1e-13)


def test_vectorized_mask_matches_the_scalar_generator():
    # the array form of the generator against the scalar one (itself pinned by
    # the known answers): every word of random counters, and whole masks,
    # including a counter offset that carries into the high word
    rng = np.random.default_rng(9)
    ctrs = [int(c) for c in rng.integers(0, 2 ** 63, 40)] + [0xFFFFFFFF, 0x100000000, 2 ** 64 - 1]
    key = (0x9ABCDEF0, 0x12345678)
    lo = np.array([c & 0xFFFFFFFF for c in ctrs], dtype=np.uint64)
    hi = np.array([c >> 32 for c in ctrs], dtype=np.uint64)
    got = O.philox4x32_10_np(lo, hi, key)
    for i, c in enumerate(ctrs):
        want = O.philox4x32_10((c & 0xFFFFFFFF, c >> 32, 0, 0), key)
        assert [int(w[i]) for w in got] == want, hex(c)
    for (M, n, p, seed, off) in ((5, 64, 0.3, 77, 0), (3, 128, 0.05, 2 ** 40 + 3, 2 ** 32 - 20)):
        full = O.dropout_mask(M, n, p, seed, off)
        sub = O.dropout_mask_at(np.arange(M), np.arange(n), n, p, seed, off)
        assert np.array_equal(full, sub)
        assert np.array_equal(full, O.dropout_mask_np(M, n, p, seed, off))
        rows, cols = np.array([4 % M, 0]), np.array([63, 1, 8])
        assert np.array_equal(O.dropout_mask_at(rows, cols, n, p, seed, off), full[np.ix_(rows, cols)])
