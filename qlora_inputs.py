"""Seeded synthetic inputs for the QLoRA adapted-linear path.

This module only draws random numbers and rounds them to the storage types
the path takes (fp32 weights, bf16 activations, gradients and adapters).  It
holds none of the method's arithmetic, and both the oracle-based tests and
the GPU path take their inputs from here.

Recipe: numpy PCG64 with seed = 1000 * config + 10 * layer + tensor, where
tensor is W 1, x 2, g 3, A 4, B 5 and layer 0..6 runs q, k, v, o, gate, up,
down.  Values are drawn as fp32 standard normals times sigma; x, g, A and B
are then rounded to bf16 (round to nearest even).  The weights stand in for
a trained checkpoint: pretrained weights are roughly normal (QLoRA pages,
NF4 sections), so Gaussian weights at the layer shapes of the 8B and 70B
models are the synthetic workload.
"""

from __future__ import annotations

import dataclasses

import numpy as np

try:  # bf16 rounding of the drawn values; torch's CPU cast is round-to-nearest-even
    import torch
except ImportError:  # pragma: no cover
    torch = None


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    m: int           # out features
    n: int           # in features
    M: int           # tokens
    r: int           # LoRA rank
    alpha: float
    w_sigma: float
    index: int = 0   # position in the transformer block (seed component)

    @property
    def s(self) -> float:
        return self.alpha / self.r


def _block(hidden, kv, ffn, M, r, alpha, sigma):
    shapes = [("q", hidden, hidden), ("k", kv, hidden), ("v", kv, hidden), ("o", hidden, hidden),
              ("gate", ffn, hidden), ("up", ffn, hidden), ("down", hidden, ffn)]
    return [Layer(nm, m, n, M, r, alpha, sigma, i) for i, (nm, m, n) in enumerate(shapes)]


# The five workloads: 1 small single layer, 2 the 8B gate projection at 4096
# tokens, 3 the 8B down projection at 4096 tokens with r = 64, 4 the seven
# layers of an 8B block at 16 tokens (forward only), 5 the seven layers of a
# 70B block at 8192 tokens.
WORKLOADS = {
    1: dict(name="single 256x256 layer, 32 tokens, r=8",
            layers=[Layer("single", 256, 256, 32, 8, 16.0, 0.02, 0)], backward=True),
    2: dict(name="8B gate projection 14336x4096, 4096 tokens, r=16",
            layers=[Layer("gate", 14336, 4096, 4096, 16, 32.0, 0.02, 4)], backward=True),
    3: dict(name="8B down projection 4096x14336, 4096 tokens, r=64",
            layers=[Layer("down", 4096, 14336, 4096, 64, 16.0, 0.02, 6)], backward=True),
    4: dict(name="8B block, seven layers, 16 tokens, r=16, forward",
            layers=_block(4096, 1024, 14336, 16, 16, 32.0, 0.02), backward=False),
    5: dict(name="70B block, seven layers, 8192 tokens, r=64",
            layers=_block(8192, 1024, 28672, 8192, 64, 16.0, 0.015), backward=True),
}

TENSOR_ID = dict(W=1, x=2, g=3, A=4, B=5)
A_SIGMA = 1.0 / 16.0      # A ~ N(0, 1/256)
B_SIGMA = 0.01            # B ~ N(0, 0.01^2)


def seed_of(cfg: int, layer_index: int, tensor: str) -> int:
    return 1000 * cfg + 10 * layer_index + TENSOR_ID[tensor]


def normal_f32(seed: int, shape, sigma: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    out = rng.standard_normal(size=int(np.prod(shape)), dtype=np.float32)
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out.reshape(shape)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_as_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def layer_inputs(cfg: int, layer: Layer, tensors=("W", "x", "g", "A", "B"), M: int | None = None):
    """Draw the named tensors of one layer.

    W: fp32 m x n.  x: bf16 bits M x n.  g: bf16 bits M x m.  A: bf16 bits
    r x n.  B: bf16 bits m x r.  ``M`` overrides the token count (rows are
    drawn from the same stream, so a smaller M gives the leading rows).
    """
    M = layer.M if M is None else M
    out = {}
    for t in tensors:
        sd = seed_of(cfg, layer.index, t)
        if t == "W":
            out[t] = normal_f32(sd, (layer.m, layer.n), layer.w_sigma)
        elif t == "x":
            out[t] = to_bf16_bits(normal_f32(sd, (M, layer.n), 1.0))
        elif t == "g":
            out[t] = to_bf16_bits(normal_f32(sd, (M, layer.m), 1.0))
        elif t == "A":
            out[t] = to_bf16_bits(normal_f32(sd, (layer.r, layer.n), A_SIGMA))
        elif t == "B":
            out[t] = to_bf16_bits(normal_f32(sd, (layer.m, layer.r), B_SIGMA))
        else:
            raise KeyError(t)
    return out


def custom_inputs(seed: int, M: int, n: int, m: int, r: int, w_sigma: float = 0.02):
    """Inputs of arbitrary shape for edge cases (ragged sizes, tiny layers)."""
    return dict(
        W=normal_f32(seed * 10 + 1, (m, n), w_sigma),
        x=to_bf16_bits(normal_f32(seed * 10 + 2, (M, n), 1.0)),
        g=to_bf16_bits(normal_f32(seed * 10 + 3, (M, m), 1.0)),
        A=to_bf16_bits(normal_f32(seed * 10 + 4, (r, n), A_SIGMA)),
        B=to_bf16_bits(normal_f32(seed * 10 + 5, (m, r), B_SIGMA)),
    )
