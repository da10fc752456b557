"""GPU parity of the adapter optimizer step (qlora_adam_step) against the oracle.

Inputs: the oracle and the GPU start from the same host arrays (seeded
generators); the oracle applies the same number of steps in float64 with the
hyperparameters as the kernel receives them (fp32).  Bar, derived from fp32
arithmetic over a few steps: first and second moments within 1e-6 relative to
the size of their terms, weights within 2^-21 relative plus 1e-5 of the
learning rate per step; the bf16 copy equals the rounding of the kernel's own
fp32 weight; state in pinned host memory gives the same bits as state in HBM.
"""

import numpy as np
import pytest
import torch

import qlora_inputs as QI
from oracle import qlora_oracle as O
from parity_utils import dev_bf16, host_bits

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


f32 = lambda x: float(np.float32(x))  # noqa: E731


def run_case(Q, counts, steps, lr, b1, b2, eps, wd, seed, host_state=False, with_copy=True):
    rng_p = [QI.normal_f32(seed * 100 + i, (c,), 0.05) for i, c in enumerate(counts)]
    grads = [[QI.to_bf16_bits(QI.normal_f32(seed * 1000 + 10 * t + i, (c,), 10.0 ** (-1 - (i % 3)))) for i, c
              in enumerate(counts)] for t in range(steps)]
    kw = dict(pin_memory=True) if host_state else dict(device="cuda")
    P = [torch.from_numpy(p.copy()).to(**({"device": "cuda"} if not host_state else {})) for p in rng_p]
    if host_state:
        P = [torch.empty(c, dtype=torch.float32, pin_memory=True) for c in counts]
        for t, p in zip(P, rng_p):
            t.copy_(torch.from_numpy(p))
    Mm = [torch.zeros(c, dtype=torch.float32, **kw) for c in counts]
    Vv = [torch.zeros(c, dtype=torch.float32, **kw) for c in counts]
    P16 = [torch.empty(c, dtype=torch.bfloat16, device="cuda") if with_copy and i % 2 == 0 else None
           for i, c in enumerate(counts)]
    for t in range(steps):
        G = [dev_bf16(g) for g in grads[t]]
        Q.adam_step(list(zip(P, P16, G, Mm, Vv)), lr, b1, b2, eps, wd, step=t + 1)
        torch.cuda.synchronize()
    # oracle from the same host arrays, float64, the fp32 hyperparameters
    hp = [f32(v) for v in (lr, b1, b2, eps, wd)]
    out = []
    for i, c in enumerate(counts):
        p, m, v = rng_p[i].astype(np.float64), np.zeros(c), np.zeros(c)
        gsum, g2sum = np.zeros(c), np.zeros(c)
        for t in range(steps):
            g = O.bf16_bits_to_float64(grads[t][i])
            gsum += np.abs(g)
            g2sum += g * g
            p, m, v = O.adam_step(p, g, m, v, t + 1, *hp)
        out.append((p, m, v, gsum, g2sum))
    return P, P16, Mm, Vv, out


def check(P, P16, Mm, Vv, ref, lr, steps, what):
    for i, (p_ref, m_ref, v_ref, gsum, g2sum) in enumerate(ref):
        p = P[i].cpu().numpy().astype(np.float64)
        m = Mm[i].cpu().numpy().astype(np.float64)
        v = Vv[i].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(m - m_ref) <= 1e-6 * (np.abs(m_ref) + gsum) + 1e-30), f"{what} tensor {i}: exp_avg"
        assert np.all(np.abs(v - v_ref) <= 1e-6 * (np.abs(v_ref) + g2sum) + 1e-30), f"{what} tensor {i}: exp_avg_sq"
        assert np.all(np.abs(p - p_ref) <= 2.0 ** -21 * np.abs(p_ref) + 1e-5 * lr * steps), f"{what} tensor {i}: param"
        if P16[i] is not None:
            want = O.bf16_bits_rne(P[i].cpu().numpy())
            assert np.array_equal(host_bits(P16[i]), want), f"{what} tensor {i}: bf16 copy"


def test_adam_steps_match_oracle(Q):
    # A (r x n) and B (m x r) of two layers, one ragged tensor (tail of 5), one tiny
    counts = [16 * 4096, 14336 * 16, 5 * 192 + 5, 7]
    lr, b1, b2, eps, wd, steps = 2e-4, 0.9, 0.999, 1e-8, 0.01, 3
    say("adam 3 steps, 4 tensors")
    P, P16, Mm, Vv, ref = run_case(Q, counts, steps, lr, b1, b2, eps, wd, seed=3)
    check(P, P16, Mm, Vv, ref, lr, steps, "adam")


def test_adam_many_tensors_and_no_decay(Q):
    # 70 tensors: two launches of at most 64
    counts = [64 * (i + 1) + (i % 3) for i in range(70)]
    lr, b1, b2, eps, wd, steps = 1e-3, 0.8, 0.99, 1e-6, 0.0, 2
    say("adam 2 steps, 70 tensors")
    P, P16, Mm, Vv, ref = run_case(Q, counts, steps, lr, b1, b2, eps, wd, seed=5)
    check(P, P16, Mm, Vv, ref, lr, steps, "adam-70")


def test_adam_state_in_pinned_host_memory(Q):
    # the paged case: weights and moments in host memory, gradient in HBM;
    # same arithmetic as with the state in HBM, so the same bits
    counts = [16 * 1024, 4096 * 16 + 3]
    args = (counts, 2, 5e-4, 0.9, 0.999, 1e-8, 0.05)
    say("adam with state in pinned host memory")
    Ph, P16h, Mh, Vh, ref = run_case(Q, *args, seed=9, host_state=True)
    Pd, P16d, Md, Vd, _ = run_case(Q, *args, seed=9, host_state=False)
    for a, b in zip(Ph + Mh + Vh, Pd + Md + Vd):
        assert torch.equal(a.cpu(), b.cpu())
    check(Ph, P16h, Mh, Vh, ref, 5e-4, 2, "adam-host")
