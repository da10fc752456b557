"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
oracle references (full or on sampled outputs) and the tolerance check.

Tolerance for bf16 outputs of the forward and backward: relative L2 error
<= 1e-2 and max-abs error <= 2e-2 * max|reference|, against the float64
oracle.  Quantizer outputs and the dequantized weight are compared bit for
bit.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import qlora_oracle as O

REL_L2 = 1e-2
MAX_ABS = 2e-2


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits) -> np.ndarray:
    return O.bf16_bits_to_float64(bits)


def assert_close(got, ref, what: str):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    mref = np.max(np.abs(ref)) if ref.size else 0.0
    mx = np.max(np.abs(err)) if err.size else 0.0
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS * mref + 1e-30, f"{what}: max abs error {mx:.3e} > {MAX_ABS} * {mref:.3e}"
    return rel, mx / mref if mref > 0 else 0.0


def oracle_full(W, x_bits, g_bits, A_bits, B_bits, s):
    """Quantize + forward + backward of one small layer, all in the oracle."""
    m, n = W.shape
    qw = O.quantize_nf4_dq(W)
    Wd = f64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], m * n)).reshape(m, n)
    x, A, B = f64(x_bits), f64(A_bits), f64(B_bits)
    h, u = O.linear_fwd(x, Wd, A, B, s)
    out = dict(qw=qw, Wd=Wd, h=h, u=u)
    if g_bits is not None:
        bw = O.linear_bwd(x, f64(g_bits), Wd, A, B, s, u=u)
        out.update(bw)
    return out


def sample_indices(count: int, k: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    idx = set([0, count - 1])
    idx.update(rng.integers(0, count, size=min(k, count)).tolist())
    return np.array(sorted(idx), dtype=np.int64)
